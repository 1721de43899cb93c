// attn_mfma.hip -- bf16 chunk attention on the CDNA4 matrix cores (gfx950).
//
// [SKaiNET] "Change (additive)": attention of C chunk rows over past + C keys
// under an additive mask per head.  Both products are dense contractions, so
// they run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Work split.  A workgroup is 4 waves x 32 query rows; the 128 rows are the G
// query heads of one KV head times qpos = 128 / G chunk rows, so every K/V
// tile staged in LDS serves the whole GQA group (read from HBM once per query
// tile).  Workgroups are mapped so that consecutive query tiles of one
// (sequence, KV head) land on the same XCD and share its L2.
//
// Orientation.  Each wave computes S^T = K Q^T (32 keys x 32 queries per
// MFMA): lane l then holds, for query l % 32, 16 keys of each 32-key block, so
// the row max and row sum are lane-local plus one exchange with lane l ^ 32.
// The probabilities are already in the B-operand layout of O^T += V^T P^T,
// so P never leaves registers.  V is staged in LDS row-major and its
// transposed A operand is gathered with ds_read_b64_tr_b16 (a 16-lane
// transpose read of 4 x 16-bit elements per lane).
//
// LDS.  K and V tiles are stored row-major without padding; 16-byte chunks of
// a row are XOR-swizzled by the row index so that the K operand reads (16
// rows, one chunk each) and the V transpose reads (4 rows, two chunks each)
// hit distinct banks.
//
// Softmax.  Base 2 with scale*log2(e) folded into one FMA.  With the in-kernel
// rule each wave decides per tile whether every real row attends every key
// (then no mask work at all) or not (then the additive mask is applied per
// element).  The explicit mask is applied to every tile, and so is the rule
// under CP_ATTN_FULL_TILES: the two modes then evaluate identical expressions
// on an identical key partition.  The running max is only raised when a tile
// exceeds it by more than 2^8 (exact: numerator and denominator share it), so
// the O accumulator is rarely rescaled.
//
// Pipeline.  K/V tile t+1 is loaded from HBM into registers while tile t is
// computed from LDS; chunk rows come from the caller's k_new / v_new, past
// rows from the cache slots.  Tiles outside the window or past the last real
// row are skipped.
#include "attn_common.h"

namespace cp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kRescaleSlack = 8.f;  // log2 units

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  const bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Swizzle of the 16-byte chunks of LDS row r.
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 64 ? ((r >> 1) & 7) : (r & 15);
}
__device__ __forceinline__ int vswz(int r) { return (r & 3) << 1; }

template <int D>
struct WavesPerEU {
  static constexpr int value = D >= 256 ? 1 : 2;
};

template <int D, int KT, bool EXPLICIT>
__global__ void __launch_bounds__(256)
    __attribute__((amdgpu_waves_per_eu(WavesPerEU<D>::value, WavesPerEU<D>::value)))
    k_attn_mfma(AttnParams p) {
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int NK = KT * CPR;       // chunks per tile (K or V)
  constexpr int NL = NK / 256;       // chunk loads per thread per tile
  constexpr int NS = D / 16;         // k-steps of QK^T
  constexpr int NKB = KT / 32;       // 32-key blocks per tile
  constexpr int NDB = D / 32;        // 32-dim blocks of the output
  constexpr int NPT = KT / 16;       // k-steps of PV
  static_assert(NK % 256 == 0, "tile must split evenly over 256 threads");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[KT * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;

  // XCD-aware order: the hardware deals workgroups round-robin over 8 XCDs;
  // give each XCD a contiguous range of work items.
  const unsigned nblk = gridDim.x;
  unsigned wk = blockIdx.x;
  if (nblk % 8 == 0) wk = (wk % 8) * (nblk / 8) + wk / 8;
  const int qtile = wk % p.qtiles;
  wk /= p.qtiles;
  const int split = wk % p.splits;
  const int bg = wk / p.splits;
  const int b = bg / p.nKV;
  const int g = bg % p.nKV;

  const int r = wave * 32 + n;
  const int hl = r / p.qpos;
  const int i_min = qtile * p.qpos;
  const int i = i_min + r % p.qpos;
  const bool row_ok = hl < p.G && i < p.C;
  const int head = g * p.G + (row_ok ? hl : 0);
  const int irow = row_ok ? i : 0;

  const int seen = p.seen[b];
  const bool lead = tid == 0 && qtile == 0 && split == 0 && g == 0;
  const int nv = read_nvalid(p.n_valid, b, p.C, lead ? p.status : nullptr);
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
  const bool real_row = row_ok && i < nv;
  // this wave's real rows (for its own tile visibility test)
  const int wi_lo = wave_min_i(real_row ? i : 0x7fffffff);
  const int wi_hi = wave_max_i(real_row ? i : -1);

  // Q^T fragments: lane holds q[row n][16 s + 8 hh .. + 7] for every k-step s.
  bf16x8 qf[NS];
  {
    const uint16_t *Q = static_cast<const uint16_t *>(p.q) +
                        ((static_cast<size_t>(b) * p.H + head) * p.C + irow) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4 *>(Q + 16 * s);
      qf[s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  TileSeq ts{};
  int u0 = 0, u1 = 0;
  if (any_real) {
    ts = make_tiles(gl, seen, p.C, KT, i_min, i_last, EXPLICIT ? 0 : p.window, p.sink,
                    EXPLICIT || p.full_tiles);
    const int cnt = ts.count();
    u0 = static_cast<int>((static_cast<long>(cnt) * split) / p.splits);
    u1 = static_cast<int>((static_cast<long>(cnt) * (split + 1)) / p.splits);
  }

  const uint16_t *KC = static_cast<const uint16_t *>(p.kc) +
                       (static_cast<size_t>(b) * p.nKV + g) * p.cap * static_cast<size_t>(D);
  const uint16_t *VC = static_cast<const uint16_t *>(p.vc) +
                       (static_cast<size_t>(b) * p.nKV + g) * p.cap * static_cast<size_t>(D);
  const uint16_t *KN = static_cast<const uint16_t *>(p.kn) +
                       (static_cast<size_t>(b) * p.nKV + g) * p.C * static_cast<size_t>(D);
  const uint16_t *VN = static_cast<const uint16_t *>(p.vn) +
                       (static_cast<size_t>(b) * p.nKV + g) * p.C * static_cast<size_t>(D);
  const int R = p.cap - p.sink;
  const bool small_ring = p.ring && R < KT;

  // ---- global -> registers -> LDS staging (thread owns chunks tid + 256 e)
  u32x4 kreg[NL], vreg[NL];
  auto load_tile = [&](int u) {
    int first;
    const bool chunk = ts.at(u, KT, &first);
    // slot of the tile's first non-sink column (past tiles of a ring)
    int c_ns = imax(first, gl.ns), s_ns = 0;
    if (!chunk && p.ring && c_ns < gl.L) s_ns = slot_of(gl.lo + (c_ns - gl.ns), p.cap, 1, p.sink);
#pragma unroll
    for (int e = 0; e < NL; ++e) {
      const int idx = tid + 256 * e;
      const int row = idx / CPR, ch = idx % CPR;
      const int col = first + row;
      const uint16_t *ks = nullptr, *vs = nullptr;
      if (chunk) {
        if (col < p.C) {
          ks = KN + static_cast<size_t>(col) * D;
          vs = VN + static_cast<size_t>(col) * D;
        }
      } else if (col < gl.L) {
        int sl;
        if (!p.ring) {
          sl = col;
        } else if (col < gl.ns) {
          sl = col;
        } else if (!small_ring) {
          sl = s_ns + (col - c_ns);
          if (sl >= p.cap) sl -= R;
        } else {
          sl = slot_of(gl.lo + (col - gl.ns), p.cap, 1, p.sink);
        }
        ks = KC + static_cast<size_t>(sl) * D;
        vs = VC + static_cast<size_t>(sl) * D;
      }
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (ks) {
        kv = *reinterpret_cast<const u32x4 *>(ks + ch * 8);
        vv = *reinterpret_cast<const u32x4 *>(vs + ch * 8);
      }
      kreg[e] = kv;
      vreg[e] = vv;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int e = 0; e < NL; ++e) {
      const int idx = tid + 256 * e;
      const int row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<u32x4 *>(&Ks[row * D + ((ch ^ kswz<D>(row)) << 3)]) = kreg[e];
      *reinterpret_cast<u32x4 *>(&Vs[row * D + ((ch ^ vswz(row)) << 3)]) = vreg[e];
    }
  };

  // per-lane LDS read geometry
  const int k_sw = kswz<D>(n);  // rows 32 kb + n share n's swizzle
  const int s16 = lane & 15;
  const int v_key = 4 * hh + (s16 >> 2);           // + 16 t (+ 8)
  const int v_sw = vswz(v_key);                   // (16 t + 8 keeps it)
  const int v_cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within a 32-dim block
  const int v_el = 4 * (lane & 1);

  const float *mrow = nullptr;
  if (EXPLICIT && row_ok)
    mrow = p.mask + b * p.mbs + head * p.mhs + static_cast<int64_t>(irow) * p.mld;
  const int qabs = seen + i;

  if (u0 < u1) load_tile(u0);
  for (int u = u0; u < u1; ++u) {
    int first;
    const bool chunk = ts.at(u, KT, &first);
    __syncthreads();
    store_tile();
    __syncthreads();
    if (u + 1 < u1) load_tile(u + 1);

    // ---- S^T = K Q^T
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int off = ((2 * s + hh) ^ k_sw) << 3;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(&Ks[(32 * kb + n) * D + off]);
        sacc[kb] = mfma(__builtin_bit_cast(bf16x8, a), qf[s], sacc[kb]);
      }
    }

    // ---- tile classification (wave-uniform): does every real row of this wave
    // attend every key of the tile?  Then no mask work at all.
    const int lim = chunk ? p.C : gl.L;
    const int64_t mbase = chunk ? static_cast<int64_t>(gl.L) + first : first;
    // additive bias of key kk of this lane's row (explicit mask or rule), -inf out of range
    auto bias4 = [&](int kk, float *a4) {
      if (EXPLICIT) {
        if (mrow && p.mask_vec4 && first + kk + 3 < lim && ((mbase + kk) & 3) == 0) {
          const float4 mv = *reinterpret_cast<const float4 *>(mrow + mbase + kk);
          a4[0] = mv.x;
          a4[1] = mv.y;
          a4[2] = mv.z;
          a4[3] = mv.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            a4[e] = first + kk + e < lim ? (mrow ? mrow[mbase + kk + e] : 0.f) : -INFINITY;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          a4[e] = inkernel_add(chunk, first + kk + e, gl, seen, p.C, nv, qabs, p.window, p.sink);
      }
    };
    bool visible;
    if (EXPLICIT || p.full_tiles) {
      visible = false;  // the mask is applied to every tile (same expressions in both modes)
    } else if (wi_hi < wi_lo) {
      visible = true;  // no real row in this wave: its results are discarded
    } else if (chunk) {
      visible = first + KT <= p.C && first + KT - 1 <= wi_lo &&
                (p.window == 0 || wi_hi - first < p.window);
    } else {
      visible = first + KT <= gl.L;
      if (visible && p.window > 0) {
        const int cn = imax(first, gl.ns);  // oldest non-sink column of the tile
        if (cn < first + KT) visible = (seen + wi_hi) - column_position(gl, cn) < p.window;
      }
    }

    // ---- online softmax in base 2.  Visible tiles keep raw scores s and use
    // p = 2^(s*scale*log2e - m); masked tiles first form t = s*scale*log2e +
    // bias*log2e and use p = 2^(t - m).  (scale > 0, so max(s)*c = max(s*c).)
    float mt = -INFINITY;
    if (visible) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kb][e]);
      mt *= p.sl2e;
    } else {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          float a4[4];
          bias4(32 * kb + 8 * rq + 4 * hh, a4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float tv = fmaf(sacc[kb][4 * rq + e], p.sl2e, a4[e] * kLog2e);
            sacc[kb][4 * rq + e] = tv;
            mt = fmaxf(mt, tv);
          }
        }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const bool raise = mt > m_run + kRescaleSlack;
    if (__any(raise)) {
      const float m_new = raise ? mt : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    }
    // p = 2^(x * k - m): x = s with k = scale*log2e on visible tiles, x = t with
    // k = 1 on masked ones (fma(t, 1, -m) rounds exactly as t - m)
    const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
    const float kx = visible ? p.sl2e : 1.f;

    bf16x8 pb[NPT];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = sacc[kb][8 * half + 2 * e], x1 = sacc[kb][8 * half + 2 * e + 1];
          const float p0 = __builtin_amdgcn_exp2f(fmaf(x0, kx, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(x1, kx, neg_m));
          l_run += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pb[2 * kb + half] = __builtin_bit_cast(bf16x8, w);
      }
    }

    // ---- O^T += V^T P^T, V^T gathered by transpose reads
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int voff = (((4 * db + v_cl) ^ v_sw) << 3) + v_el;
#pragma unroll
      for (int t = 0; t < NPT; ++t) {
        const uint16_t *v0 = &Vs[(16 * t + v_key) * D + voff];
        const uint16_t *v1 = &Vs[(16 * t + 8 + v_key) * D + voff];
        const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(v0));
        const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(v1));
        const u32x2 w0 = __builtin_bit_cast(u32x2, a0), w1 = __builtin_bit_cast(u32x2, a1);
        const u32x4 a = {w0[0], w0[1], w1[0], w1[1]};
        oacc[db] = mfma(__builtin_bit_cast(bf16x8, a), pb[t], oacc[db]);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const bool real = any_real && i < nv;
  const size_t orow = (static_cast<size_t>(b) * p.H + head) * p.C + i;
  if (p.splits == 1) {
    uint16_t *O = static_cast<uint16_t *>(p.out) + orow * D;
    const float inv = real ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = 32 * db + 8 * rq + 4 * hh;
        const float o0 = oacc[db][4 * rq + 0] * inv, o1 = oacc[db][4 * rq + 1] * inv;
        const float o2 = oacc[db][4 * rq + 2] * inv, o3 = oacc[db][4 * rq + 3] * inv;
        const u32x2 w = {pack_bf16x2(real ? o0 : 0.f, real ? o1 : 0.f),
                         pack_bf16x2(real ? o2 : 0.f, real ? o3 : 0.f)};
        *reinterpret_cast<u32x2 *>(O + d) = w;
      }
    }
  } else if (i < nv) {  // partials of real rows only: the merge writes pad rows as zeros
    const size_t rows = static_cast<size_t>(p.B) * p.H * p.C;
    float *WO = p.wo + (split * rows + orow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = 32 * db + 8 * rq + 4 * hh;
        float4 w;
        w.x = real ? oacc[db][4 * rq + 0] : 0.f;
        w.y = real ? oacc[db][4 * rq + 1] : 0.f;
        w.z = real ? oacc[db][4 * rq + 2] : 0.f;
        w.w = real ? oacc[db][4 * rq + 3] : 0.f;
        *reinterpret_cast<float4 *>(WO + d) = w;
      }
    }
    if (hh == 0) {
      float *ML = p.wml + (split * rows + orow) * 2;
      ML[0] = real ? m_run : -INFINITY;
      ML[1] = real ? l_tot : 0.f;
    }
  }
}

template <int D, int KT>
hipError_t launch_d(const AttnParams &p, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>(p.qtiles) * p.splits * p.B * p.nKV;
  if (blocks == 0) return hipSuccess;
  if (p.mask)
    hipLaunchKernelGGL((k_attn_mfma<D, KT, true>), dim3(blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_attn_mfma<D, KT, false>), dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams &p, int D, hipStream_t s) {
  switch (D) {
    case 64:
      return launch_d<64, 64>(p, s);
    case 128:
      return launch_d<128, 64>(p, s);
    case 256:
      return launch_d<256, 32>(p, s);
    default:
      return hipErrorInvalidValue;
  }
}

int mfma_keys_per_tile(int D) { return D == 256 ? 32 : 64; }

}  // namespace cp
