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

constexpr int kPlanThreads = 1024;

// exclusive prefix sums of in[0..n) into out[0..n] (out[n] = total); n <= blockDim.x;
// every thread of the block calls it
__device__ void block_scan(const int *in, int *out, int n, int *buf) {
  const int t = threadIdx.x;
  buf[t] = t < n ? in[t] : 0;
  __syncthreads();
  for (int off = 1; off < static_cast<int>(blockDim.x); off <<= 1) {
    const int add = t >= off ? buf[t - off] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  if (t < n) out[t + 1] = buf[t];
  if (t == 0) out[0] = 0;
  __syncthreads();
}

__global__ void __launch_bounds__(kPlanThreads) k_attn_plan(AttnParams p, int32_t *plan) {
  __shared__ int nb_s[kPlanMaxB];     // tiles of the longest query tile of sequence b
  __shared__ int pc_s[kPlanMaxB];     // pieces of b
  __shared__ int len_s[kPlanMaxB];    // tiles per piece of b (ranking key)
  __shared__ int order_s[kPlanMaxB];  // sequences by rank
  __shared__ int tmp_s[kPlanMaxB];
  __shared__ int upre_s[kPlanMaxB + 1], gpre_s[kPlanMaxB + 1], spre_s[kPlanMaxB + 1];
  __shared__ int buf_s[kPlanThreads];
  __shared__ int tot_s, sum_s, T_s;
  const int t = threadIdx.x, nt = static_cast<int>(blockDim.x);  // nt >= B (one per sequence)
  const int B = p.B;
  const bool explicit_mask = p.mask != nullptr;
  if (t == 0) tot_s = 0;
  __syncthreads();
  // 1. tile counts per sequence (bad sequences count nothing; the attention flags them)
  for (int b = t; b < B; b += nt) {
    const int seen = p.seen[b];
    int nv = p.n_valid ? p.n_valid[b] : p.C;
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
    atomicAdd(&tot_s, sum);
  }
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
    atomicAdd(&sum_s, part);
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
    int r = 0;
    for (int o = 0; o < B; ++o)
      r += (len_s[o] > len_s[b]) || (len_s[o] == len_s[b] && o < b);
    order_s[r] = b;
  }
  __syncthreads();
  // 4. units (sequence, piece, KV head) in rank order; split entries and partial slots in
  // sequence order
  for (int k = t; k < B; k += nt) tmp_s[k] = pc_s[order_s[k]] * p.nKV;
  __syncthreads();
  block_scan(tmp_s, upre_s, B, buf_s);
  for (int b = t; b < B; b += nt) tmp_s[b] = pc_s[b] > 1 ? p.nKV * p.qtiles : 0;
  __syncthreads();
  block_scan(tmp_s, gpre_s, B, buf_s);
  for (int b = t; b < B; b += nt) tmp_s[b] = pc_s[b] > 1 ? p.nKV * p.qtiles * pc_s[b] : 0;
  __syncthreads();
  block_scan(tmp_s, spre_s, B, buf_s);
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
    it[6] = p.seen[b];
    it[7] = p.n_valid ? p.n_valid[b] : p.C;
  }
  // 6. the split entries, for the merge
  int32_t *groups = items + static_cast<size_t>(p.plan_grid) * kPlanItemInts;
  for (int b = t; b < B; b += nt) {
    const int P = pc_s[b];
    if (P <= 1) continue;
    int nv = p.n_valid ? p.n_valid[b] : p.C;
    nv = nv < 0 ? 0 : (nv > p.C ? p.C : nv);
    for (int g = 0; g < p.nKV; ++g)
      for (int q = 0; q < p.qtiles; ++q) {
        const int j = g * p.qtiles + q;
        int32_t *e = groups + static_cast<size_t>(gpre_s[b] + j) * kPlanItemInts;
        e[0] = b;
        e[1] = g;
        e[2] = q;
        e[3] = P;
        e[4] = spre_s[b] + j * P;
        e[5] = nv;
      }
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
      float M = -INFINITY;
      for (int s = 0; s < P; ++s) {
        const size_t grp = static_cast<size_t>(base + s) * rw + rg;
        M = fmaxf(M, p.wml[(grp * 32 + n) * 2]);
      }
      if (M != -INFINITY) {
        float l = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < P; ++s) {
          const size_t grp = static_cast<size_t>(base + s) * rw + rg;
          const float2 ml = *reinterpret_cast<const float2 *>(p.wml + (grp * 32 + n) * 2);
          const uint2 v = *reinterpret_cast<const uint2 *>(
              reinterpret_cast<const uint16_t *>(p.wo) + (grp << lgb) * 1024 +
              static_cast<size_t>(k) * 1024 + (e & 255) * 4);  // normalized, bf16
          const float w = __builtin_amdgcn_exp2f(ml.x - M);  // 0 for an empty piece
          const float wl = w * ml.y;
          l = fmaf(w, ml.y, l);
          o[0] = fmaf(wl, __uint_as_float(v.x << 16), o[0]);
          o[1] = fmaf(wl, __uint_as_float(v.x & 0xffff0000u), o[1]);
          o[2] = fmaf(wl, __uint_as_float(v.y << 16), o[2]);
          o[3] = fmaf(wl, __uint_as_float(v.y & 0xffff0000u), o[3]);
        }
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) res[x] = o[x] * inv;
      }
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
  // one wave for up to 64 sequences (its barriers cost next to nothing), else as many
  // threads as sequences, rounded up to whole waves
  const unsigned nt = p.B <= 64 ? 64u : static_cast<unsigned>((p.B + 63) / 64 * 64);
  hipLaunchKernelGGL(k_attn_plan, dim3(1), dim3(nt), 0, s, p, const_cast<int32_t *>(p.plan));
  return hipGetLastError();
}

hipError_t launch_attn_merge_plan(const AttnParams &p, int D, hipStream_t s) {
  // at most plan_grid split entries; a grid-stride loop over the ones the plan made
  const size_t most = static_cast<size_t>(p.plan_grid) * p.frag_rows * D / 4;
  size_t blocks = (most + 255) / 256;
  if (blocks > 512) blocks = 512;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(k_attn_merge_plan, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p,
                     D);
  return hipGetLastError();
}

}  // namespace cp
