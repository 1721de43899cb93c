// attn_valu.hip -- chunk attention on the vector ALUs (fp32 path, and the
// fallback for shapes the matrix-core kernel does not take), plus the merge
// of key-split partials.
//
// [SKaiNET] "Change (additive)": attention over past + C keys with the
// additive per-head mask.  One workgroup = 16 query rows (hb heads of one KV
// group x qpos chunk rows) x 16 lanes per row; a lane owns D/16 output
// columns.  K/V tiles of 16 keys are staged in LDS as fp32 and shared by the
// rows; scores are reduced across the 16 lanes of a row with DPP moves; the softmax is the online (running max / running sum) form in
// base 2 with scale*log2(e) folded into one FMA.  fp32 accumulation.
#include "attn_common.h"

namespace cp {
namespace {

constexpr int KTG = 16;  // keys per tile

template <typename T>
__device__ __forceinline__ float ld(const T *p, size_t i);
template <>
__device__ __forceinline__ float ld<float>(const float *p, size_t i) {
  return p[i];
}
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, size_t i) {
  return bf16_to_f32(p[i]);
}
// the value an fp32 result has once stored in T (bf16: round to nearest even)
template <typename T>
__device__ __forceinline__ float round_to(float v);
template <>
__device__ __forceinline__ float round_to<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ float round_to<uint16_t>(float v) {
  return bf16_to_f32(f32_to_bf16_rne(v));
}
__device__ __forceinline__ void st(float *p, size_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(uint16_t *p, size_t i, float v) { p[i] = f32_to_bf16_rne(v); }

// One DPP move within rows of 16 lanes (a VALU operand modifier: no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
// Sum over the 16 lanes of a row, left in every lane (bitwise the same in each: every
// step adds a lane's value to its partner's, and the partner does the same in the
// other order).  quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);
  v += dpp<0x4E>(v);
  v += dpp<0x141>(v);
  v += dpp<0x140>(v);
  return v;
}

template <typename T, int DPT, bool EXPLICIT>
__global__ void __launch_bounds__(256) k_attn_valu(AttnParams p, int D) {
  request_args(p);
  constexpr int NF = KTG * DPT / 16;  // >= KTG * D / 256 tile elements per thread
  extern __shared__ float lds[];
  float *Ks = lds;             // [KTG][D]
  float *Vs = lds + KTG * D;   // [KTG][D]

  const int tid = threadIdx.x;
  const int r = tid / 16;      // row in the workgroup
  const int ql = tid % 16;     // lane within the row

  int w = blockIdx.x;
  const int qtile = w % p.qtiles;
  w /= p.qtiles;
  const int hgrp = w % p.hgroups;
  w /= p.hgroups;
  const int split = w % p.splits;
  const int bg = w / p.splits;
  const int b = bg / p.nKV;
  const int g = bg % p.nKV;

  const int i_min = qtile * p.qpos;
  const int hl = hgrp * p.hb + r / p.qpos;
  const int i = i_min + r % p.qpos;
  const bool row_ok = r < p.hb * p.qpos && hl < p.G && i < p.C;
  const int head = g * p.G + (hl < p.G ? hl : 0);

  // the query row does not depend on the cache state: requested first, so that its
  // latency overlaps that of seen
  float q[DPT], acc[DPT];
  const T *Q = static_cast<const T *>(p.q);
  const size_t qoff = ((static_cast<size_t>(b) * p.H + head) * p.C + (i < p.C ? i : 0)) * D;
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    const int d = ql + 16 * e;
    q[e] = (row_ok && d < D) ? ld<T>(Q, qoff + d) : 0.f;
    acc[e] = 0.f;
  }
  // RoPE folded into the load (q given before rotation): each element is rotated with
  // its half-split partner, read again from memory, by the RoPE launch's arithmetic and
  // rounding to the storage dtype.
  if (p.q_cos) {
    const int h2 = D / 2;
    const size_t trow = (static_cast<size_t>(p.q_tables == 1 ? 0 : b) * p.C +
                         (i < p.C ? i : 0)) * D;
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      const int d = ql + 16 * e;
      if (row_ok && d < D) {
        const bool low = d < h2;
        const float other = ld<T>(Q, qoff + (low ? d + h2 : d - h2));
        const float c = p.q_cos[trow + d], sn = p.q_sin[trow + d];
        const float r = low ? rot_lo(q[e], other, c, sn) : rot_hi(other, q[e], c, sn);
        q[e] = round_to<T>(r);
      }
    }
  }
  // seen and n_valid are both requested before either is used (scalar loads complete
  // out of order, so the first use waits for every one in flight: one round trip)
  const int seen = p.seen[b];
  int nv = p.n_valid ? p.n_valid[b] : p.C;
  const bool lead = tid == 0 && qtile == 0 && hgrp == 0 && split == 0 && g == 0;
  if (nv < 0 || nv > p.C) {
    if (lead) flag(p.status, CP_DEV_NVALID);
    nv = nv < 0 ? 0 : p.C;
  }
  bool bad = seen < 0 || (!p.ring && seen > p.cap);
  if (bad && lead) flag(p.status, CP_DEV_SEEN);
  const Live gl = live_geometry(bad ? 0 : seen, p.cap, p.ring, p.sink);
  if (EXPLICIT && !bad && static_cast<int64_t>(gl.L) + p.C > p.mld) {
    bad = true;
    if (lead) flag(p.status, CP_DEV_MASK_LD);
  }
  const int i_end = imin(i_min + p.qpos, p.C);
  const int i_last = imin(i_end, nv) - 1;
  const bool any_real = !bad && i_last >= i_min;

  float m_run = -INFINITY, l_run = 0.f;

  TileSeq ts{};
  int u0 = 0, u1 = 0;
  if (any_real) {
    ts = make_tiles(gl, seen, p.C, KTG, i_min, i_last, EXPLICIT ? 0 : p.window, p.sink,
                    EXPLICIT || p.full_tiles);
    // near-equal split ranges, the first cnt % splits one tile longer (one 32-bit
    // division: a 64-bit one is a long software sequence ahead of the first load)
    const unsigned cnt = static_cast<unsigned>(ts.count()), ns = static_cast<unsigned>(p.splits);
    const unsigned qn = cnt / ns, rm = cnt - qn * ns, us = static_cast<unsigned>(split);
    u0 = static_cast<int>(us * qn + (us < rm ? us : rm));
    u1 = u0 + static_cast<int>(qn + (us < rm ? 1u : 0u));
  }
  const T *KC = static_cast<const T *>(p.kc);
  const T *VC = static_cast<const T *>(p.vc);
  const T *KN = static_cast<const T *>(p.kn);
  const T *VN = static_cast<const T *>(p.vn);
  const size_t cbase = (static_cast<size_t>(b) * p.nKV + g) * p.cap;
  const size_t nbase = (static_cast<size_t>(b) * p.nKV + g) * p.C;
  const int qabs = seen + i;

  // K/V tile u into registers: thread tid holds elements tid + 256 j of the KTG x D
  // tile (KTG * D / 256 <= NF of them), all loads in flight together
  float kreg[NF], vreg[NF];
  auto fetch = [&](int u) __attribute__((always_inline)) {
    int first;
    const bool chunk = ts.at(u, KTG, &first);
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int e = tid + 256 * j;
      const int kk = e / D, d = e - kk * D;
      const int col = first + kk;
      float kv = 0.f, vv = 0.f;
      if (e < KTG * D) {
        if (chunk) {
          if (col < p.C) {
            kv = ld<T>(KN, (nbase + col) * D + d);
            vv = ld<T>(VN, (nbase + col) * D + d);
          }
        } else if (col < gl.L) {
          const int sl = slot_of(column_position(gl, col), p.cap, p.ring, p.sink);
          kv = ld<T>(KC, (cbase + sl) * D + d);
          vv = ld<T>(VC, (cbase + sl) * D + d);
        }
      }
      kreg[j] = kv;
      vreg[j] = vv;
    }
  };
  // explicit mask row of this lane's query row (a valid row for the rows past the
  // tile's end, whose results are discarded)
  const float *mrow = nullptr;
  if (EXPLICIT)
    mrow = p.mask + b * p.mbs + head * p.mhs + static_cast<int64_t>(i < p.C ? i : 0) * p.mld;
  // this lane's columns, clamped into the row: the tile loops run without a branch per
  // element (a guarded LDS read waited for its own round trip, element by element);
  // columns past D carry q = 0 into the scores, and their sums are never stored
  int dcl[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) dcl[e] = imin(ql + 16 * e, D - 1);
  if (u0 < u1) fetch(u0);
  for (int u = u0; u < u1; ++u) {
    int first;
    const bool chunk = ts.at(u, KTG, &first);
    // the tile's KTG mask values: unconditional loads of clamped columns, all in flight
    // at once (columns past the valid range become -inf below)
    float madd[KTG];
    if (EXPLICIT) {
      const int lim = chunk ? p.C : gl.L;
      const int64_t mb = chunk ? static_cast<int64_t>(gl.L) : 0;
#pragma unroll
      for (int kk = 0; kk < KTG; ++kk) madd[kk] = mrow[mb + imin(first + kk, lim - 1)];
    }
    __syncthreads();  // every row is done with the previous tile
#pragma unroll
    for (int j = 0; j < NF; ++j) {
      const int e = tid + 256 * j;
      if (e < KTG * D) {
        Ks[e] = kreg[j];
        Vs[e] = vreg[j];
      }
    }
    __syncthreads();
    if (u + 1 < u1) fetch(u + 1);  // next tile's loads fly while this one computes
    const bool visible =
        !EXPLICIT && tile_all_visible(chunk, first, KTG, gl, seen, p.C, i_min, i_last, p.window);
    float t[KTG];
    float m_tile = -INFINITY;
#pragma unroll
    for (int kk = 0; kk < KTG; ++kk) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < DPT; ++e) part = fmaf(q[e], Ks[kk * D + dcl[e]], part);
      part = row16_sum(part);
      const int col = first + kk;
      float add;
      if (EXPLICIT) {
        const bool in = chunk ? col < p.C : col < gl.L;
        add = in ? madd[kk] : -INFINITY;
      } else if (visible) {
        add = 0.f;
      } else {
        add = inkernel_add(chunk, col, gl, seen, p.C, nv, qabs, p.window, p.sink);
      }
      const float tv = add == -INFINITY ? -INFINITY : fmaf(part, p.sl2e, add * kLog2e);
      t[kk] = tv;
      m_tile = fmaxf(m_tile, tv);
    }
    const float m_new = fmaxf(m_run, m_tile);
    // a row whose keys so far are all -inf keeps nothing: use 0 as reference
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < DPT; ++e) acc[e] *= alpha;
#pragma unroll
    for (int kk = 0; kk < KTG; ++kk) {
      const float pk = __builtin_amdgcn_exp2f(t[kk] - m_use);
      l_run += pk;
#pragma unroll
      for (int e = 0; e < DPT; ++e) acc[e] = fmaf(pk, Vs[kk * D + dcl[e]], acc[e]);
    }
  }

  if (!row_ok) return;
  const size_t orow = (static_cast<size_t>(b) * p.H + head) * p.C + i;
  const bool real = any_real && i < nv;
  if (p.splits == 1) {
    T *O = static_cast<T *>(p.out);
    T *S = p.sel && i == selected_row(nv)
               ? static_cast<T *>(p.sel) + (static_cast<size_t>(b) * p.H + head) * D
               : nullptr;
    const float inv = real ? 1.f / l_run : 0.f;
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      const int d = ql + 16 * e;
      if (d < D) {
        st(O, orow * D + d, real ? acc[e] * inv : 0.f);
        if (S) st(S, d, real ? acc[e] * inv : 0.f);
      }
    }
  } else if (i < nv) {  // partials of real rows only: the merge writes pad rows as zeros
    const size_t rows = static_cast<size_t>(p.B) * p.H * p.C;
    float *WO = p.wo + (split * rows + orow) * D;
#pragma unroll
    for (int e = 0; e < DPT; ++e) {
      const int d = ql + 16 * e;
      if (d < D) WO[d] = real ? acc[e] : 0.f;
    }
    if (ql == 0) {
      float *ML = p.wml + (split * rows + orow) * 2;
      ML[0] = real ? m_run : -INFINITY;
      ML[1] = real ? l_run : 0.f;
    }
  }
}

// Merge key-split partials: out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, for
// VEC consecutive output columns per thread; pad rows are written as zeros.  The
// partials are fetched SB splits at a time (independent loads in flight together)
// and folded into a running maximum, so a row costs ceil(splits / SB) memory round
// trips instead of one per split.
// I: index type (32-bit when every partial's offset allows; see the RoPE kernel).
// SB: splits fetched per round -- 32 when there are more than 16 splits (one round
// for up to 32), else 16 (the narrower kernel keeps more waves resident for merges of
// many rows).
// FRAG: the partials are in the matrix-core kernel's fragment order (AttnParams::wo),
// D a power of two, normalized (O / l) in bf16: out = sum_s 2^(m_s - M) l_s O_s /
// sum_s 2^(m_s - M) l_s.  Thread t takes the 4 values at 4 t of each split, so that a
// wave's partial reads are 512 consecutive bytes (the reads are SB times the writes;
// the bf16 output rows are written 8 bytes per row and instruction).
template <typename T, int VEC, typename I, int SB, bool FRAG>
__global__ void __launch_bounds__(256) k_attn_combine(AttnParams p, int D) {
  static_assert(!FRAG || (VEC == 4 && sizeof(T) == 2), "fragment order: 4 bf16 per thread");
  const size_t rows = static_cast<size_t>(p.B) * p.H * p.C;
  // rows of one split's partials (fragment order: every row of every query tile)
  const size_t prow = FRAG ? static_cast<size_t>(p.B) * p.nKV * p.qtiles * p.frag_rows : rows;
  const I per_row = D / VEC;
  const I total = static_cast<I>(prow) * per_row;
  // one split's partials apart (element offsets: with a 32-bit I, every offset in the
  // workspace fits 32 bits, so a load is one scalar base plus a 32-bit vector offset
  // instead of a 64-bit address per split kept live across the loop)
  const I o_str = static_cast<I>(prow) * D, m_str = static_cast<I>(prow) * 2;
  const int lg_blk = FRAG ? __builtin_ctz(static_cast<unsigned>(D)) - 5 : 0;  // log2(D / 32)
  T *O = static_cast<T *>(p.out);
  I t0 = blockIdx.x * static_cast<I>(blockDim.x) + threadIdx.x;
  I tstep = static_cast<I>(gridDim.x) * blockDim.x;
  if (FRAG && p.xmerge > 0) {
    // XCD placement (AttnParams::xmerge): block k is slot k / 8 of XCD k % 8; a unit of
    // xmerge 32-row groups is 8 D threads per group, one pass
    const unsigned bpu = static_cast<unsigned>(p.xmerge) * 8u * D / blockDim.x;
    const unsigned j = blockIdx.x / 8, unit = blockIdx.x % 8 + 8 * (j / bpu);
    t0 = (static_cast<I>(unit) * bpu + j % bpu) * blockDim.x + threadIdx.x;
    tstep = total;
  }
  for (I t = t0; t < total; t += tstep) {
    // The split count and strides pass through an empty asm each iteration: loop
    // invariants to the compiler, which would otherwise compute the SB per-split
    // conditions and offsets once ahead of the loop and keep them (spilled) across it
    // -- several hundred instructions ahead of the first load, for a loop that
    // normally runs once.
    int nsp = p.splits;
    I os = o_str, ms = m_str;
    asm volatile("" : "+s"(nsp), "+s"(os), "+s"(ms));
    // partial offsets first (shifts only), so that the loads go out before the
    // divisions that place the row
    I u = 0;      // fragment order: 32-row group
    int n = 0;    // fragment order: row within the group
    I o_at, ml_at;  // offsets of this thread's values in one split's O and (m, l)
    I row_i = 0;  // row-major: output row
    if constexpr (FRAG) {
      // float4 j * 64 + 32 h + n of a block: row n, columns 8 j + 4 h .. + 3
      n = static_cast<int>(t & 31);
      u = (t >> 8) >> lg_blk;
      o_at = t * 4;
      ml_at = (u * 32 + static_cast<I>(n)) * 2;
    } else {
      row_i = t / per_row;
      o_at = row_i * D + (t - row_i * per_row) * VEC;
      ml_at = row_i * 2;
    }
    // partials of splits s0 .. s0 + SB - 1 (pad rows, and the spare rows of a query
    // tile, have none written: their values are read but not used)
    // (fragment order: the packed bf16 pairs as loaded, widened only where they are
    // used -- widening them here would make each split's load wait before the next
    // split's goes out)
    float mv[SB], lv[SB], ov[SB][FRAG ? 1 : VEC];
    uint32_t pk[SB][2];
    auto fetch = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < SB; ++j) {
        mv[j] = -INFINITY;
        lv[j] = 0.f;
        if constexpr (FRAG) {
          pk[j][0] = pk[j][1] = 0u;
        } else {
#pragma unroll
          for (int e = 0; e < VEC; ++e) ov[j][e] = 0.f;
        }
        if (s0 + j < nsp) {
          const I sj = static_cast<I>(s0 + j);
          const float2 ml = *reinterpret_cast<const float2 *>(p.wml + (sj * ms + ml_at));
          mv[j] = ml.x;
          lv[j] = ml.y;
          const float *src = p.wo + (sj * os + o_at);
          if constexpr (FRAG) {
            const uint2 v = *reinterpret_cast<const uint2 *>(
                reinterpret_cast<const uint16_t *>(p.wo) + (sj * os + o_at));
            pk[j][0] = v.x;
            pk[j][1] = v.y;
          } else if constexpr (VEC == 4) {
            const float4 v = *reinterpret_cast<const float4 *>(src);
            ov[j][0] = v.x;
            ov[j][1] = v.y;
            ov[j][2] = v.z;
            ov[j][3] = v.w;
          } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) ov[j][e] = src[e];
          }
        }
      }
    };
    // the first round goes out together with the n_valid read, not after it
    fetch(0);
    size_t row;  // output row (b * H + head) * C + i
    int d0, i, b;
    I bh;        // b * H + head
    if constexpr (FRAG) {
      const int rw = p.frag_rows >> 5;
      const I tq = u / static_cast<I>(rw);  // query tile, over (b, kv head)
      const int r = static_cast<int>(u - tq * rw) * 32 + n;
      const I bg = tq / static_cast<I>(p.qtiles);
      const int qt = static_cast<int>(tq - bg * p.qtiles);
      b = static_cast<int>(bg / static_cast<I>(p.nKV));
      const int g = static_cast<int>(bg - static_cast<I>(b) * p.nKV);
      const int hl = r / p.qpos;
      i = qt * p.qpos + (r - hl * p.qpos);
      if (hl >= p.G || i >= p.C) continue;  // a spare row of the tile: no output row
      bh = static_cast<I>(b) * p.H + g * p.G + hl;
      row = static_cast<size_t>(bh) * p.C + i;
      d0 = 32 * static_cast<int>((t >> 8) & ((1u << lg_blk) - 1)) +
           8 * static_cast<int>((t >> 6) & 3) + 4 * static_cast<int>((t >> 5) & 1);
    } else {
      row = row_i;
      d0 = static_cast<int>(t - row_i * per_row) * VEC;
      bh = row_i / static_cast<I>(p.C);
      i = static_cast<int>(row_i - bh * p.C);
      b = static_cast<int>(bh / static_cast<I>(p.H));
    }
    const int nv = read_nvalid(p.n_valid, b, p.C, nullptr);
    float res[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) res[e] = 0.f;
    if (i < nv) {
      float M = -INFINITY, l = 0.f, o[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = 0.f;
      for (int s0 = 0; s0 < nsp; s0 += SB) {
        if (s0 > 0) fetch(s0);
        float Mn = M;
#pragma unroll
        for (int j = 0; j < SB; ++j) Mn = fmaxf(Mn, mv[j]);
        if (Mn == -INFINITY) continue;  // nothing attended so far
        const float a = __builtin_amdgcn_exp2f(M - Mn);  // 0 while M = -inf
        l *= a;
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] *= a;
#pragma unroll
        for (int j = 0; j < SB; ++j) {
          const float wgt = __builtin_amdgcn_exp2f(mv[j] - Mn);
          l = fmaf(wgt, lv[j], l);
          if constexpr (FRAG) {
            const float wo = wgt * lv[j];  // normalized partials carry l apart
            o[0] = fmaf(wo, __uint_as_float(pk[j][0] << 16), o[0]);
            o[1] = fmaf(wo, __uint_as_float(pk[j][0] & 0xffff0000u), o[1]);
            o[2] = fmaf(wo, __uint_as_float(pk[j][1] << 16), o[2]);
            o[3] = fmaf(wo, __uint_as_float(pk[j][1] & 0xffff0000u), o[3]);
          } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = fmaf(wgt, ov[j][e], o[e]);
          }
        }
        M = Mn;
      }
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) res[e] = o[e] * inv;
    }
    if constexpr (FRAG) {
      // one 8-byte store per lane (the matrix-core path's out is 16-byte aligned and
      // d0 a multiple of 4); four 2-byte stores made partial-line writes
      const uint2 w = make_uint2(
          f32_to_bf16_rne(res[0]) | (static_cast<uint32_t>(f32_to_bf16_rne(res[1])) << 16),
          f32_to_bf16_rne(res[2]) | (static_cast<uint32_t>(f32_to_bf16_rne(res[3])) << 16));
      *reinterpret_cast<uint2 *>(O + (row * D + d0)) = w;
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) st(O, row * D + d0 + e, res[e]);
    }
    if (p.sel && i == selected_row(nv)) {
      T *S = static_cast<T *>(p.sel) + static_cast<size_t>(bh) * D + d0;  // bh = b * H + h
#pragma unroll
      for (int e = 0; e < VEC; ++e) st(S, e, res[e]);
    }
  }
  // Early-appended chunk: advance seen.  Every attention workgroup read seen before this
  // kernel started, and the merge itself never reads it.
  if (p.advance && blockIdx.x == 0)
    for (int b = threadIdx.x; b < p.B; b += blockDim.x) {
      const AppendPlan a = append_plan(p.cache, p.n_valid, b, p.C, false);
      if (!a.skip) p.cache.seen[b] = a.s0 + a.n;
    }
}

template <typename T, bool EXPLICIT>
hipError_t launch_valu_t(const AttnParams &p, int D, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>(p.qtiles) * p.hgroups * p.splits * p.B * p.nKV;
  if (blocks == 0) return hipSuccess;
  const size_t shm = 2 * KTG * static_cast<size_t>(D) * sizeof(float);
  const int dpt = (D + 15) / 16;
  if (dpt <= 1)
    hipLaunchKernelGGL((k_attn_valu<T, 1, EXPLICIT>), dim3(blocks), dim3(256), shm, s, p, D);
  else if (dpt <= 2)
    hipLaunchKernelGGL((k_attn_valu<T, 2, EXPLICIT>), dim3(blocks), dim3(256), shm, s, p, D);
  else if (dpt <= 4)
    hipLaunchKernelGGL((k_attn_valu<T, 4, EXPLICIT>), dim3(blocks), dim3(256), shm, s, p, D);
  else if (dpt <= 8)
    hipLaunchKernelGGL((k_attn_valu<T, 8, EXPLICIT>), dim3(blocks), dim3(256), shm, s, p, D);
  else
    hipLaunchKernelGGL((k_attn_valu<T, 16, EXPLICIT>), dim3(blocks), dim3(256), shm, s, p, D);
  return hipGetLastError();
}

}  // namespace

int valu_keys(int) { return KTG; }

hipError_t launch_attn_valu(const AttnParams &p, int D, int dtype, hipStream_t s) {
  const bool ex = p.mask != nullptr;
  if (dtype == CP_BF16)
    return ex ? launch_valu_t<uint16_t, true>(p, D, s) : launch_valu_t<uint16_t, false>(p, D, s);
  return ex ? launch_valu_t<float, true>(p, D, s) : launch_valu_t<float, false>(p, D, s);
}

hipError_t launch_attn_combine(const AttnParams &p, int D, int dtype, hipStream_t s) {
  if (static_cast<size_t>(p.B) * p.H * p.C * D == 0) return hipSuccess;
  // fragment order: the bf16 matrix-core kernel's partials (D a power of two >= 32)
  const bool frag = p.frag_rows > 0;
  if (frag && (dtype != CP_BF16 || D < 32 || (D & (D - 1)) != 0 || p.frag_rows % 32 != 0))
    return hipErrorInvalidValue;
  const size_t prow = frag ? static_cast<size_t>(p.B) * p.nKV * p.qtiles * p.frag_rows
                           : static_cast<size_t>(p.B) * p.H * p.C;
  const size_t total = prow * D;  // partial elements of one split
  const bool v4 = D % 4 == 0;
  const unsigned bs = 64;  // threads per workgroup: the rows spread over more CUs
  size_t blocks = (total / (v4 ? 4 : 1) + bs - 1) / bs;
  if (blocks > 16384) blocks = 16384;
  if (frag && p.xmerge > 0) {
    // XCD placement: 8 XCDs x the units of one XCD, every partial in one pass
    const size_t groups = prow / 32;
    const size_t units = (groups + p.xmerge - 1) / p.xmerge;
    if ((8 * static_cast<size_t>(D)) % bs != 0) return hipErrorInvalidValue;
    blocks = 8 * ((units + 7) / 8) * p.xmerge * (8 * static_cast<size_t>(D) / bs);
  }
  // 32-bit offsets when the whole workspace's byte offsets fit 32 bits
  const bool i32 = total * static_cast<size_t>(p.splits) < (size_t(1) << 30);
  const bool wide = p.splits > 16;
#define CP_COMBINE_SB(T, V, SB, F)                                                           \
  do {                                                                                       \
    if (i32)                                                                                 \
      hipLaunchKernelGGL((k_attn_combine<T, V, uint32_t, SB, F>), dim3(blocks), dim3(bs), 0, \
                         s, p, D);                                                           \
    else                                                                                     \
      hipLaunchKernelGGL((k_attn_combine<T, V, size_t, SB, F>), dim3(blocks), dim3(bs), 0,    \
                         s, p, D);                                                           \
  } while (0)
#define CP_COMBINE(T, V, F)          \
  do {                               \
    if (wide)                        \
      CP_COMBINE_SB(T, V, 32, F);    \
    else                             \
      CP_COMBINE_SB(T, V, 16, F);    \
  } while (0)
  if (frag) {
    CP_COMBINE(uint16_t, 4, true);
  } else if (dtype == CP_BF16) {
    if (v4)
      CP_COMBINE(uint16_t, 4, false);
    else
      CP_COMBINE(uint16_t, 1, false);
  } else {
    if (v4)
      CP_COMBINE(float, 4, false);
    else
      CP_COMBINE(float, 1, false);
  }
#undef CP_COMBINE
#undef CP_COMBINE_SB
  return hipGetLastError();
}

}  // namespace cp
