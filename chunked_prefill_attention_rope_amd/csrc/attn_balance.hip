// attn_balance.hip -- balanced key splits for batches of unequal past lengths.
//
// [SKaiNET] "Change (additive)": the chunk's rows attend their sequence's whole live past;
// in a batch whose past lengths differ (a Llama-8B-like batch of 16 sequences with pasts
// uniform in [0, 4095]), the workgroups of the longest sequence set the attention's time
// while the CUs that ran the short ones idle.  The lengths are only known on the device
// (seen), so a one-workgroup plan kernel, launched ahead of the attention:
//  - counts each (sequence, query tile)'s key tiles with the attention's own tile lists;
//  - picks a piece length T >= total tiles / the workgroups the GPU holds at once, and cuts
//    each sequence's keys into ceil(tiles / T) near-equal pieces (the same cut for all its
//    KV heads and query tiles);
//  - ranks the pieces longest first and lays them out so that block i, which the hardware
//    deals to XCD i mod 8, gets a longest-first share on every XCD, and the query tiles of
//    one (sequence, KV head, piece) share an XCD and its L2;
//  - writes one 8-int item per block (sequence, KV head, query tile, piece, pieces,
//    partial slot, seen, n_valid), so the attention reads its work and the lengths in one
//    scalar load, and one 8-int entry per split (sequence, KV head, query tile).
// Unsplit items write their output directly; the split ones write normalized bf16
// partials (and fp32 m, l) in the matrix-core fragment order to their slots, and
// k_attn_merge_plan combines them.
#include "attn_common.h"

namespace cp {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kMergeRound = 4;  // pieces the plan merge fetches per memory round trip

// The plan's three exclusive prefix sums in one pass (out[n] = the total; every thread
// of the block calls it): units per rank k (pieces of the k-th longest sequence times
// the KV heads), split entries per sequence and partial slots per sequence, formed from
// pc (pieces per sequence) and order (sequences by rank) as they are summed.  Each
// thread sums a run of consecutive elements, the runs' sums are scanned within each wave
// by lane shuffles, and the waves' totals are added through LDS: two barriers for all
// three (a log-step scan through LDS costs two per step).  wsum: 3 x (threads / 64).
__device__ void plan_scans(const int *pc, const int *order, int n, int nKV, int qtiles,
                           int *upre, int *gpre, int *spre, int *wsum) {
  const int t = threadIdx.x, nt = blockDim.x, nw = nt / 64;
  const int per = (n + nt - 1) / nt;
  const int lo = imin(n, t * per), hi = imin(n, lo + per);
  auto vals = [&](int k, int &u, int &gq, int &sq) {
    const int P = pc[k];
    u = pc[order[k]] * nKV;
    gq = P > 1 ? nKV * qtiles : 0;
    sq = P > 1 ? nKV * qtiles * P : 0;
  };
  int s0 = 0, s1 = 0, s2 = 0;
  for (int k = lo; k < hi; ++k) {
    int u, gq, sq;
    vals(k, u, gq, sq);
    s0 += u;
    s1 += gq;
    s2 += sq;
  }
  const int lane = t & 63, w = t >> 6;
  int x0 = s0, x1 = s1, x2 = s2;  // inclusive scans over the wave
  for (int o = 1; o < 64; o <<= 1) {
    const int y0 = __shfl_up(x0, o, 64), y1 = __shfl_up(x1, o, 64), y2 = __shfl_up(x2, o, 64);
    if (lane >= o) {
      x0 += y0;
      x1 += y1;
      x2 += y2;
    }
  }
  if (lane == 63) {
    wsum[w] = x0;
    wsum[nw + w] = x1;
    wsum[2 * nw + w] = x2;
  }
  __syncthreads();
  int r0 = x0 - s0, r1 = x1 - s1, r2 = x2 - s2;
  for (int v = 0; v < w; ++v) {
    r0 += wsum[v];
    r1 += wsum[nw + v];
    r2 += wsum[2 * nw + v];
  }
  for (int k = lo; k < hi; ++k) {
    int u, gq, sq;
    vals(k, u, gq, sq);
    upre[k] = r0;
    gpre[k] = r1;
    spre[k] = r2;
    r0 += u;
    r1 += gq;
    r2 += sq;
  }
  if (t == nt - 1) {  // the last thread's runs end at the totals
    upre[n] = r0;
    gpre[n] = r1;
    spre[n] = r2;
  }
  __syncthreads();
}

// Sum of v over the block, added into *acc (which the caller zeroed and publishes with a
// barrier): a shuffle reduction per wave, one LDS atomic per wave.
__device__ void block_add(int v, int *acc) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if ((threadIdx.x & 63) == 0) atomicAdd(acc, v);
}

__global__ void __launch_bounds__(kPlanThreads) k_attn_plan(AttnParams p, int32_t *plan) {
  __shared__ int nb_s[kPlanMaxB];     // tiles of the longest query tile of sequence b
  __shared__ int pc_s[kPlanMaxB];     // pieces of b
  __shared__ int len_s[kPlanMaxB];    // tiles per piece of b (ranking key)
  __shared__ int order_s[kPlanMaxB];  // sequences by rank
  __shared__ int upre_s[kPlanMaxB + 1], gpre_s[kPlanMaxB + 1], spre_s[kPlanMaxB + 1];
  __shared__ int seen_s[kPlanMaxB], nvr_s[kPlanMaxB];  // seen and raw n_valid, read once
  __shared__ int wsum_s[3 * (kPlanThreads / 64)];
  __shared__ int tot_s, sum_s, T_s;
  const int t = threadIdx.x, nt = static_cast<int>(blockDim.x);
  const int B = p.B;
  const bool explicit_mask = p.mask != nullptr;
  if (t == 0) tot_s = 0;
  __syncthreads();
  // 1. tile counts per sequence (bad sequences count nothing; the attention flags them)
  int tot = 0;
  for (int b = t; b < B; b += nt) {
    const int seen = p.seen[b];
    int nv = p.n_valid ? p.n_valid[b] : p.C;
    seen_s[b] = seen;
    nvr_s[b] = nv;
    nv = nv < 0 ? 0 : (nv > p.C ? p.C : nv);
    bool bad = seen < 0 || (!p.ring && seen > p.cap);
    const Live gl = live_geometry(bad ? 0 : seen, p.cap, p.ring, p.sink);
    if (explicit_mask && static_cast<int64_t>(gl.L) + p.C > p.mld) bad = true;
    int nmax = 0, sum = 0;
    for (int q = 0; q < p.qtiles && !bad; ++q) {
      const int i_min = q * p.qpos;
      const int i_last = imin(imin(i_min + p.qpos, p.C), nv) - 1;
      if (i_last < i_min) continue;
      const TileSeq ts = make_tiles(gl, seen, p.C, p.plan_kt, i_min, i_last,
                                    explicit_mask ? 0 : p.window, p.sink,
                                    explicit_mask || p.full_tiles);
      nmax = imax(nmax, ts.count());
      sum += ts.count();
    }
    nb_s[b] = nmax;
    tot += sum;
  }
  block_add(tot, &tot_s);
  __syncthreads();
  // 2. piece length: at least plan_tmin tiles and the total over the resident slots;
  // longer while the items would not fit the launch's grid (its last group of 8 padded)
  const int total = tot_s * p.nKV;
  if (t == 0) T_s = imax(p.plan_tmin, (total + p.plan_slots - 1) / p.plan_slots);
  __syncthreads();
  // a sequence is cut only when its longest query tile exceeds the piece length by more
  // than an eighth (equal lengths -- whose query tiles differ by their few chunk tiles --
  // stay whole)
  for (;;) {
    const int T = T_s + T_s / 8;
    if (t == 0) sum_s = 0;
    __syncthreads();
    int part = 0;
    for (int b = t; b < B; b += nt) part += imax(1, (nb_s[b] + T - 1) / T);
    block_add(part, &sum_s);
    __syncthreads();
    const int units = sum_s * p.nKV;
    const bool fits = ((units + 7) / 8) * 8 * p.qtiles <= p.plan_grid;
    __syncthreads();
    if (fits) break;
    if (t == 0) T_s = T_s + imax(1, T_s / 8);
    __syncthreads();
  }
  const int T = T_s + T_s / 8;
  for (int b = t; b < B; b += nt) {
    const int P = imax(1, (nb_s[b] + T - 1) / T);
    pc_s[b] = P;
    len_s[b] = (nb_s[b] + P - 1) / P;
  }
  __syncthreads();
  // 3. rank: longest piece first, ties by sequence
  for (int b = t; b < B; b += nt) {
    const int lb = len_s[b];
    int r = 0;
#pragma unroll 8
    for (int o = 0; o < B; ++o) {  // (unrolled: eight LDS reads in flight, not one)
      const int lo_ = len_s[o];
      r += (lo_ > lb) || (lo_ == lb && o < b);
    }
    order_s[r] = b;
  }
  __syncthreads();
  // 4. units (sequence, piece, KV head) in rank order; split entries and partial slots in
  // sequence order
  plan_scans(pc_s, order_s, B, p.nKV, p.qtiles, upre_s, gpre_s, spre_s, wsum_s);
  const int U = upre_s[B];
  // 5. one item per block: unit r's query tile q at block (r / 8) * 8 * qtiles + 8 q + r % 8
  int32_t *items = plan + kPlanHeaderInts;
  const int per_group = 8 * p.qtiles;
  for (int blk = t; blk < p.plan_grid; blk += nt) {
    const int grp = blk / per_group, rem = blk - grp * per_group;
    const int q = rem >> 3, r = grp * 8 + (rem & 7);
    int32_t *it = items + static_cast<size_t>(blk) * kPlanItemInts;
    if (r >= U) {
      it[0] = -1;
      continue;
    }
    int lo = 0, hi = B;  // the rank k with upre[k] <= r < upre[k + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (upre_s[mid] <= r) lo = mid; else hi = mid;
    }
    const int b = order_s[lo];
    const int off = r - upre_s[lo];
    const int piece = off / p.nKV, g = off - piece * p.nKV;
    const int P = pc_s[b];
    it[0] = b;
    it[1] = g;
    it[2] = q;
    it[3] = piece;
    it[4] = P;
    it[5] = P > 1 ? spre_s[b] + (g * p.qtiles + q) * P + piece : -1;
    it[6] = seen_s[b];  // (from LDS: a global read here would cost every item a round trip)
    it[7] = nvr_s[b];
  }
  // 6. the split entries, for the merge: one thread per (sequence, KV head, query tile)
  int32_t *groups = items + static_cast<size_t>(p.plan_grid) * kPlanItemInts;
  const int per_b = p.nKV * p.qtiles;
  for (int x = t; x < B * per_b; x += nt) {
    const int b = x / per_b, j = x - b * per_b;
    const int P = pc_s[b];
    if (P <= 1) continue;
    int32_t *e = groups + static_cast<size_t>(gpre_s[b] + j) * kPlanItemInts;
    e[0] = b;
    e[1] = j / p.qtiles;
    e[2] = j % p.qtiles;
    e[3] = P;
    e[4] = spre_s[b] + j * P;
    e[5] = imin(imax(nvr_s[b], 0), p.C);
  }
  if (t == 0) {
    plan[0] = gpre_s[B];  // split entries
    plan[1] = T;
    plan[2] = total;
    plan[3] = U;
  }
}

// Combine the pieces of every split (sequence, KV head, query tile) of a plan: one thread
// per 4 floats of a partial block (fragment order, as the partials were stored), reading
// the P pieces' (m, l, O) and writing the bf16 output row (pad rows as zeros) and the
// selection.  Also advances seen for an early-appended chunk (every attention workgroup
// has read it before this kernel starts).
__global__ void __launch_bounds__(256) k_attn_merge_plan(AttnParams p, int D) {
  const int32_t *groups = p.plan + kPlanHeaderInts + static_cast<size_t>(p.plan_grid) * kPlanItemInts;
  const unsigned ngrp = static_cast<unsigned>(p.plan[0]);
  const int rw = p.frag_rows >> 5;        // 32-row groups per query tile
  const int lgb = __builtin_ctz(static_cast<unsigned>(D)) - 5;  // log2(D / 32)
  const unsigned per_grp = static_cast<unsigned>(rw) << (lgb + 8);  // float4s per split entry
  const unsigned total = ngrp * per_grp;
  uint16_t *O = static_cast<uint16_t *>(p.out);
  for (unsigned t = blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += gridDim.x * blockDim.x) {
    const unsigned gi = t / per_grp, e = t - gi * per_grp;
    const int32_t *G = groups + static_cast<size_t>(gi) * kPlanItemInts;
    const int b = G[0], g = G[1], q = G[2], P = G[3], base = G[4], nv = G[5];
    const int n = static_cast<int>(e & 31);
    const int rg = static_cast<int>((e >> 8) >> lgb);
    const int k = static_cast<int>((e >> 8) & ((1u << lgb) - 1));
    const int r = rg * 32 + n;
    const int hl = r / p.qpos, i = q * p.qpos + (r - hl * p.qpos);
    if (hl >= p.G || i >= p.C) continue;  // a spare row of the tile: no output row
    const int d0 = 32 * k + 8 * static_cast<int>((e >> 6) & 3) + 4 * static_cast<int>((e >> 5) & 1);
    float res[4] = {0.f, 0.f, 0.f, 0.f};
    if (i < nv) {
      // the pieces' (m, l) and O in rounds of kMergeRound, every load of a round issued
      // before any is used (one memory round trip per round), with a running maximum;
      // the bf16 pairs stay packed until they are used
      const uint16_t *WO = reinterpret_cast<const uint16_t *>(p.wo) +
                           static_cast<size_t>(k) * 1024 + (e & 255) * 4;
      float M = -INFINITY, l = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
      for (int s0 = 0; s0 < P; s0 += kMergeRound) {
        // (unconditional loads: the pieces past P read piece P - 1 again and are masked
        // afterwards; loads under a per-piece branch waited one by one)
        float2 mlv[kMergeRound];
        uint2 pk[kMergeRound];
#pragma unroll
        for (int j = 0; j < kMergeRound; ++j) {
          const size_t grp = static_cast<size_t>(base + imin(s0 + j, P - 1)) * rw + rg;
          mlv[j] = *reinterpret_cast<const float2 *>(p.wml + (grp * 32 + n) * 2);
          pk[j] = *reinterpret_cast<const uint2 *>(WO + (grp << lgb) * 1024);  // O / l, bf16
        }
        float mv[kMergeRound], lv[kMergeRound];
#pragma unroll
        for (int j = 0; j < kMergeRound; ++j) {
          mv[j] = s0 + j < P ? mlv[j].x : -INFINITY;
          lv[j] = s0 + j < P ? mlv[j].y : 0.f;
        }
        float Mn = M;
#pragma unroll
        for (int j = 0; j < kMergeRound; ++j) Mn = fmaxf(Mn, mv[j]);
        // no branch on an empty maximum (the compiler would sink the l and O loads below
        // it, a second round trip): with nothing attended so far every weight is 0
        const float Ms = Mn == -INFINITY ? 0.f : Mn;
        const float a = __builtin_amdgcn_exp2f(M - Ms);  // 0 while M = -inf
        l *= a;
#pragma unroll
        for (int x = 0; x < 4; ++x) o[x] *= a;
#pragma unroll
        for (int j = 0; j < kMergeRound; ++j) {
          const float w = __builtin_amdgcn_exp2f(mv[j] - Ms);  // 0 for an empty piece
          const float wl = w * lv[j];
          l += wl;
          o[0] = fmaf(wl, __uint_as_float(pk[j].x << 16), o[0]);
          o[1] = fmaf(wl, __uint_as_float(pk[j].x & 0xffff0000u), o[1]);
          o[2] = fmaf(wl, __uint_as_float(pk[j].y << 16), o[2]);
          o[3] = fmaf(wl, __uint_as_float(pk[j].y & 0xffff0000u), o[3]);
        }
        M = Mn;
      }
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) res[x] = o[x] * inv;
    }
    uint32_t w0 = f32_to_bf16_rne(res[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(res[1])) << 16);
    uint32_t w1 = f32_to_bf16_rne(res[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(res[3])) << 16);
    const size_t bh = static_cast<size_t>(b) * p.H + g * p.G + hl;
    uint2 *dst = reinterpret_cast<uint2 *>(O + (bh * p.C + i) * D + d0);
    *dst = make_uint2(w0, w1);
    if (p.sel && i == selected_row(nv))
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(p.sel) + bh * D + d0) = make_uint2(w0, w1);
  }
  if (p.advance && blockIdx.x == 0)
    for (int b = threadIdx.x; b < p.B; b += blockDim.x) {
      const AppendPlan a = append_plan(p.cache, p.n_valid, b, p.C, false);
      if (!a.skip) p.cache.seen[b] = a.s0 + a.n;
    }
}

}  // namespace

hipError_t launch_attn_plan(const AttnParams &p, hipStream_t s) {
  hipLaunchKernelGGL(k_attn_plan, dim3(1), dim3(kPlanThreads), 0, s, p,
                     const_cast<int32_t *>(p.plan));
  return hipGetLastError();
}

hipError_t launch_attn_merge_plan(const AttnParams &p, int D, hipStream_t s) {
  // at most plan_grid split entries; a grid-stride loop over the ones the plan made
  const size_t most = static_cast<size_t>(p.plan_grid) * p.frag_rows * D / 4;
  size_t blocks = (most + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_attn_merge_plan, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p,
                     D);
  return hipGetLastError();
}

}  // namespace cp
