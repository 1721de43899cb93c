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
// MFMA): lane l then holds, for query l % 32, 16 keys per 32-key block, so the
// row max and row sum are lane-local plus one exchange with lane l ^ 32.  The
// probabilities are already in the B-operand layout of O^T += V^T P^T, so P
// never leaves registers; V is staged in LDS as key-quads ([key/4][d][4]) so
// the A operand is two 8-byte LDS reads per lane.  The online softmax runs in
// base 2 with scale*log2(e) folded into one FMA per score.
//
// Pipeline.  K/V tile t+1 is loaded from HBM into registers while tile t is
// computed from LDS; the chunk's own K/V rows are read straight from the
// caller's k_new / v_new tensors, the past rows from the cache slots (ring
// slot arithmetic per row).  Tiles entirely outside the window or beyond the
// last real row are skipped; the per-element mask is evaluated only on tiles
// that straddle a boundary.
#include "attn_common.h"

namespace cp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  const bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ f32x16 mfma(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, int KT, bool EXPLICIT>
__global__ void __launch_bounds__(256) k_attn_mfma(AttnParams p) {
  constexpr int KP = D + 8;          // K row stride in bf16 elements (16-byte pad)
  constexpr int NK = KT * D / 8;     // 16-byte K chunks per tile
  constexpr int NKL = (NK + 255) / 256;
  constexpr int NV = (KT / 4) * (D / 8);  // V quad-chunks (4 keys x 8 dims) per tile
  constexpr int NVL = (NV + 255) / 256;
  constexpr int NS = D / 16;         // k-steps of QK^T
  constexpr int NKB = KT / 32;       // 32-key blocks per tile
  constexpr int NDB = D / 32;        // 32-dim blocks of the output
  constexpr int NPT = KT / 16;       // k-steps of PV

  __shared__ __attribute__((aligned(16))) uint16_t Ks[KT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[(KT / 4) * D * 4];

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

  const uint16_t *KC = static_cast<const uint16_t *>(p.kc);
  const uint16_t *VC = static_cast<const uint16_t *>(p.vc);
  const uint16_t *KN = static_cast<const uint16_t *>(p.kn);
  const uint16_t *VN = static_cast<const uint16_t *>(p.vn);
  const size_t cbase = (static_cast<size_t>(b) * p.nKV + g) * p.cap;
  const size_t nbase = (static_cast<size_t>(b) * p.nKV + g) * p.C;

  // Row pointer of key column `col` of a tile (nullptr outside the valid range).
  auto krow = [&](bool chunk, int col, const uint16_t *cache, const uint16_t *fresh) {
    const uint16_t *ptr = nullptr;
    if (chunk) {
      if (col < p.C) ptr = fresh + (nbase + col) * D;
    } else if (col < gl.L) {
      ptr = cache + (cbase + slot_of(column_position(gl, col), p.cap, p.ring, p.sink)) * D;
    }
    return ptr;
  };

  u32x4 kreg[NKL];
  u32x4 vreg[NVL][4];
  auto load_tile = [&](int u) {
    int first;
    const bool chunk = ts.at(u, KT, &first);
#pragma unroll
    for (int e = 0; e < NKL; ++e) {
      const int idx = tid + 256 * e;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (idx < NK) {
        const int kk = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
        const uint16_t *src = krow(chunk, first + kk, KC, KN);
        if (src) v = *reinterpret_cast<const u32x4 *>(src + d0);
      }
      kreg[e] = v;
    }
#pragma unroll
    for (int e = 0; e < NVL; ++e) {
      const int idx = tid + 256 * e;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (idx < NV) {
          const int kq = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
          const uint16_t *src = krow(chunk, first + 4 * kq + k4, VC, VN);
          if (src) v = *reinterpret_cast<const u32x4 *>(src + d0);
        }
        vreg[e][k4] = v;
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int e = 0; e < NKL; ++e) {
      const int idx = tid + 256 * e;
      if (idx < NK) {
        const int kk = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
        *reinterpret_cast<u32x4 *>(&Ks[kk * KP + d0]) = kreg[e];
      }
    }
#pragma unroll
    for (int e = 0; e < NVL; ++e) {
      const int idx = tid + 256 * e;
      if (idx < NV) {
        const int kq = idx / (D / 8), d0 = (idx % (D / 8)) * 8;
        uint16_t *dst = &Vs[(kq * D + d0) * 4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t a0 = vreg[e][0][m], a1 = vreg[e][1][m];
          const uint32_t a2 = vreg[e][2][m], a3 = vreg[e][3][m];
          // element d0 + 2m: low halves; d0 + 2m + 1: high halves
          const u32x2 lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
          const u32x2 hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
          *reinterpret_cast<u32x2 *>(dst + (2 * m) * 4) = lo;
          *reinterpret_cast<u32x2 *>(dst + (2 * m + 1) * 4) = hi;
        }
      }
    }
  };

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

    // S^T = K Q^T for the tile's 32-key blocks
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(&Ks[(32 * kb + n) * KP + 16 * s + 8 * hh]);
        sacc[kb] = mfma(__builtin_bit_cast(bf16x8, a), qf[s], sacc[kb]);
      }
    }

    // scores in base 2: t = s * scale * log2e + mask * log2e
    const bool visible =
        !EXPLICIT && tile_all_visible(chunk, first, KT, gl, seen, p.C, i_min, i_last, p.window);
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int c0 = first + 32 * kb + 8 * rq + 4 * hh;  // 4 consecutive key columns
        float add[4];
        if (EXPLICIT) {
          const int lim = chunk ? p.C : gl.L;
          const int64_t mc0 = chunk ? static_cast<int64_t>(gl.L) + c0 : c0;
          if (mrow && p.mask_vec4 && c0 + 3 < lim && (mc0 & 3) == 0) {
            const float4 mv = *reinterpret_cast<const float4 *>(mrow + mc0);
            add[0] = mv.x;
            add[1] = mv.y;
            add[2] = mv.z;
            add[3] = mv.w;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              add[e] = c0 + e < lim ? (mrow ? mrow[mc0 + e] : 0.f) : -INFINITY;
          }
        } else if (visible) {
#pragma unroll
          for (int e = 0; e < 4; ++e) add[e] = 0.f;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            add[e] = inkernel_add(chunk, c0 + e, gl, seen, p.C, nv, qabs, p.window, p.sink);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float tv =
              add[e] == -INFINITY ? -INFINITY : fmaf(sacc[kb][4 * rq + e], p.sl2e, add[e] * kLog2e);
          sacc[kb][4 * rq + e] = tv;
          mt = fmaxf(mt, tv);
        }
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;

    // P^T in the B-operand layout: k-step t = 2 kb + half covers regs 8 half .. + 7
    bf16x8 pb[NPT];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(sacc[kb][8 * half + 2 * e] - m_use);
          const float p1 = __builtin_amdgcn_exp2f(sacc[kb][8 * half + 2 * e + 1] - m_use);
          l_run += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pb[2 * kb + half] = __builtin_bit_cast(bf16x8, w);
      }
    }

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * db + n;
#pragma unroll
      for (int t = 0; t < NPT; ++t) {
        const u32x2 v0 = *reinterpret_cast<const u32x2 *>(&Vs[((4 * t + hh) * D + d) * 4]);
        const u32x2 v1 = *reinterpret_cast<const u32x2 *>(&Vs[((4 * t + 2 + hh) * D + d) * 4]);
        const u32x4 a = {v0[0], v0[1], v1[0], v1[1]};
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
  } else {
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
