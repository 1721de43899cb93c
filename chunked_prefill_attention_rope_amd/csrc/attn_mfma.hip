// attn_mfma.hip -- bf16 chunk attention on the CDNA4 matrix cores (gfx950).
//
// [SKaiNET] "Change (additive)": attention of C chunk rows over past + C keys
// under an additive mask per head.  Both products are dense contractions, so
// they run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Work split.  A workgroup holds 4 x 32 query rows (one wave per 32 rows, or two
// waves sharing them for D = 256, see Cfg); the 128 rows are the G
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
// Loads.  K/V tiles stream into a ring of LDS stages with direct-to-LDS loads
// (global_load_lds_dwordx4, 1 KB per wave instruction), STAGES - 1 tiles ahead
// of the one being computed, without passing through registers; the waits on
// them are explicit (vmcnt) followed by a plain s_barrier.  Chunk rows come from
// the caller's k_new / v_new, past rows from the cache slots.  Tiles outside
// the window or past the last real row are skipped.
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
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kRescaleSlack = 8.f;  // log2 units

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2 v = {a, b};
  const bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

// One wave-wide direct-to-LDS load: each lane's 16 bytes at src land at
// lds_base + 16 * lane.  The builtin only exists for the gfx950 device pass; the
// host pass of a HIP kernel never runs device code, and would otherwise drop the
// kernel's launch stub, so it gets an empty body.
__device__ __forceinline__ void dma16(const uint16_t *src, uint16_t *lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_base, 16, 0, 0);
#else
  (void)src;
  (void)lds_base;
#endif
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *ptr) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)ptr));
}

// ds_read_b64_tr_b16 issued as inline asm: the builtin makes the compiler drain all
// in-flight direct-to-LDS loads before it, which would serialise the K/V ring.  The
// result registers are only valid after lds_wait() below has been passed through them.
__device__ __forceinline__ u32x2 tr_read(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr));
  return r;
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

// Per head size: keys per tile, LDS ring stages, waves per SIMD, and the number of
// wave groups the output dims are split over (DSPLIT).  A stage holds one K and one V
// tile (KT x D bf16 each).  With DSPLIT = 2 a workgroup has 8 waves: waves w and
// w + 4 own the same 32 query rows, both form the full scores and probabilities, and
// each accumulates half of the output dims -- a 256-dim accumulator per wave would
// leave room for only one wave per SIMD and nothing to hide LDS and MFMA latency.
template <int D>
struct Cfg;
template <>
struct Cfg<64> {
  static constexpr int KT = 64, STAGES = 4, WAVES = 2, DSPLIT = 1;
};
template <>
struct Cfg<128> {
  static constexpr int KT = 64, STAGES = 2, WAVES = 2, DSPLIT = 1;
};
template <>
struct Cfg<256> {
  static constexpr int KT = 32, STAGES = 4, WAVES = 2, DSPLIT = 2;
};

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most n * PER vector-memory loads of this wave are outstanding
// (n = tiles issued after the one about to be consumed).
template <int PER, int STAGES>
__device__ __forceinline__ void wait_tiles_after(int n) {
  if (STAGES > 3 && n >= 2) {
    wait_vm<(STAGES > 3 ? 2 : 0) * PER>();
  } else if (STAGES > 2 && n >= 1) {
    wait_vm<(STAGES > 2 ? 1 : 0) * PER>();
  } else {
    wait_vm<0>();
  }
}

template <int D, bool EXPLICIT>
__global__ void __launch_bounds__(256 * Cfg<D>::DSPLIT)
    __attribute__((amdgpu_waves_per_eu(Cfg<D>::WAVES, Cfg<D>::WAVES)))
    k_attn_mfma(AttnParams p) {
  constexpr int KT = Cfg<D>::KT;
  constexpr int STAGES = Cfg<D>::STAGES;
  constexpr int DSPLIT = Cfg<D>::DSPLIT;
  constexpr int NW = 4 * DSPLIT;     // waves per workgroup
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int NK = KT * CPR;       // chunks per tile (K or V)
  constexpr int NL = NK / (64 * NW); // direct-to-LDS loads per wave per tile per tensor
  constexpr int RPI = 64 / CPR;      // rows covered by one wave-wide 1 KB load
  constexpr int NS = D / 16;         // k-steps of QK^T
  constexpr int NKB = KT / 32;       // 32-key blocks per tile
  constexpr int NDB = D / 32;        // 32-dim blocks of the output
  constexpr int NDW = NDB / DSPLIT;  // ... accumulated by one wave
  constexpr int NPT = KT / 16;       // k-steps of PV
  constexpr int TILE = KT * D;       // bf16 elements of one K (or V) tile
  static_assert(NK % (64 * NW) == 0, "tile must split evenly over the waves");
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");

  // ring of STAGES x (K tile, V tile)
  __shared__ __attribute__((aligned(1024))) uint16_t ring[STAGES * 2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int dgrp = wave / 4;         // which NDW dim blocks this wave accumulates

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

  const int r = (wave & 3) * 32 + n;
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

  f32x16 oacc[NDW];
#pragma unroll
  for (int db = 0; db < NDW; ++db)
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

  // ---- direct-to-LDS staging.  Wave-wide load q (= wave * NL + e) fills 1 KB of
  // the tile: rows q * RPI + lane / CPR, physical chunk lane % CPR, which holds the
  // row's logical chunk (physical ^ swizzle).  Rows outside the tile's valid range
  // read a valid row instead; their scores are masked to -inf.
  auto issue = [&](int u, uint16_t *kdst, uint16_t *vdst) __attribute__((always_inline)) {
    int first;
    const bool chunk = ts.at(u, KT, &first);
    const int lim = chunk ? p.C : gl.L;
    int c_ns = imax(first, gl.ns), s_ns = 0;
    if (!chunk && p.ring && !small_ring && c_ns < gl.L)
      s_ns = slot_of(gl.lo + (c_ns - gl.ns), p.cap, 1, p.sink);
#pragma unroll
    for (int e = 0; e < NL; ++e) {
      const int q = wave * NL + e;
      const int row = q * RPI + lane / CPR, phys = lane % CPR;
      int col = first + row;
      if (col >= lim) col = lim - 1;
      const uint16_t *kr, *vr;
      if (chunk) {
        kr = KN + static_cast<size_t>(col) * D;
        vr = VN + static_cast<size_t>(col) * D;
      } else {
        int sl;
        if (!p.ring || col < gl.ns) {
          sl = col;
        } else if (!small_ring) {
          sl = s_ns + (col - c_ns);
          if (sl >= p.cap) sl -= R;
        } else {
          sl = slot_of(gl.lo + (col - gl.ns), p.cap, 1, p.sink);
        }
        kr = KC + static_cast<size_t>(sl) * D;
        vr = VC + static_cast<size_t>(sl) * D;
      }
      if (kdst) dma16(kr + ((phys ^ kswz<D>(row)) << 3), kdst + q * 512);
      if (vdst) dma16(vr + ((phys ^ vswz(row)) << 3), vdst + q * 512);
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

  // S^T = K Q^T for the tile whose K sits at Ks
  auto qk = [&](const uint16_t *Ks, f32x16 (&sacc)[NKB]) __attribute__((always_inline)) {
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
  };

  // mask, online softmax and O^T += V^T P^T for tile u (scores in sacc, V at Vs)
  auto softmax_pv = [&](int u, f32x16 (&sacc)[NKB], const uint16_t *Vs)
                            __attribute__((always_inline)) {
    int first;
    const bool chunk = ts.at(u, KT, &first);
    // ---- tile classification (wave-uniform): does every real row of this wave
    // attend every key of the tile?  Then no mask work at all.
    const int lim = chunk ? p.C : gl.L;
    const int64_t mbase = chunk ? static_cast<int64_t>(gl.L) + first : first;
    // additive bias of key kk of this lane's row (explicit mask or rule), -inf out of range
    auto bias4 = [&](int kk, float *a4) __attribute__((always_inline)) {
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
      for (int db = 0; db < NDW; ++db)
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

    // ---- O^T += V^T P^T, V^T gathered by transpose reads (one batch per 32 dims)
    const uint32_t vbase = lds_addr(Vs) + 2 * (v_key * D);
#pragma unroll
    for (int db = 0; db < NDW; ++db) {
      const uint32_t va = vbase + 2 * ((((4 * (dgrp * NDW + db) + v_cl) ^ v_sw) << 3) + v_el);
      u32x2 w[2 * NPT];
#pragma unroll
      for (int t = 0; t < NPT; ++t) {
        w[2 * t] = tr_read(va + 2 * (16 * t * D));
        w[2 * t + 1] = tr_read(va + 2 * ((16 * t + 8) * D));
      }
      if constexpr (NPT == 4) {
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]),
                       "+v"(w[6]), "+v"(w[7]));
      } else {
        static_assert(NPT == 2, "PV k-steps per tile");
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
      }
#pragma unroll
      for (int t = 0; t < NPT; ++t) {
        const u32x4 a = {w[2 * t][0], w[2 * t][1], w[2 * t + 1][0], w[2 * t + 1][1]};
        oacc[db] = mfma(__builtin_bit_cast(bf16x8, a), pb[t], oacc[db]);
      }
    }
  };

  // tile u lives in stage u % STAGES of a ring of (K, V) tiles (a key split starts
  // at u0 > 0)
  for (int j = 0; j < STAGES - 1; ++j)
    if (u0 + j < u1) {
      uint16_t *st = ring + ((u0 + j) % STAGES) * 2 * TILE;
      issue(u0 + j, st, st + TILE);
    }
  for (int u = u0; u < u1; ++u) {
    // tile u has landed in this wave's share of the ring once at most the loads of
    // the tiles issued after it are outstanding; the barrier makes that true for all
    // waves and also guarantees every wave has finished reading the stage refilled
    wait_tiles_after<2 * NL, STAGES>(imin(u1 - 1, u + STAGES - 2) - u);
    __builtin_amdgcn_s_barrier();
    if (u + STAGES - 1 < u1) {
      uint16_t *st = ring + ((u + STAGES - 1) % STAGES) * 2 * TILE;
      issue(u + STAGES - 1, st, st + TILE);
    }
    const uint16_t *Ks = ring + (u % STAGES) * 2 * TILE;
    f32x16 sacc[NKB];
    qk(Ks, sacc);
    softmax_pv(u, sacc, Ks + TILE);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!row_ok) return;
  const bool real = any_real && i < nv;
  const size_t orow = (static_cast<size_t>(b) * p.H + head) * p.C + i;
  if (p.splits == 1) {
    uint16_t *O = static_cast<uint16_t *>(p.out) + orow * D;
    const float inv = real ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < NDW; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = 32 * (dgrp * NDW + db) + 8 * rq + 4 * hh;
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
    for (int db = 0; db < NDW; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = 32 * (dgrp * NDW + db) + 8 * rq + 4 * hh;
        float4 w;
        w.x = real ? oacc[db][4 * rq + 0] : 0.f;
        w.y = real ? oacc[db][4 * rq + 1] : 0.f;
        w.z = real ? oacc[db][4 * rq + 2] : 0.f;
        w.w = real ? oacc[db][4 * rq + 3] : 0.f;
        *reinterpret_cast<float4 *>(WO + d) = w;
      }
    }
    if (hh == 0 && dgrp == 0) {
      float *ML = p.wml + (split * rows + orow) * 2;
      ML[0] = real ? m_run : -INFINITY;
      ML[1] = real ? l_tot : 0.f;
    }
  }
}

template <int D>
hipError_t launch_d(const AttnParams &p, hipStream_t s) {
  const unsigned blocks = static_cast<unsigned>(p.qtiles) * p.splits * p.B * p.nKV;
  if (blocks == 0) return hipSuccess;
  const dim3 threads(256 * Cfg<D>::DSPLIT);
  if (p.mask)
    hipLaunchKernelGGL((k_attn_mfma<D, true>), dim3(blocks), threads, 0, s, p);
  else
    hipLaunchKernelGGL((k_attn_mfma<D, false>), dim3(blocks), threads, 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const AttnParams &p, int D, hipStream_t s) {
  switch (D) {
    case 64:
      return launch_d<64>(p, s);
    case 128:
      return launch_d<128>(p, s);
    case 256:
      return launch_d<256>(p, s);
    default:
      return hipErrorInvalidValue;
  }
}

int mfma_keys_per_tile(int D) {
  return D == 256 ? Cfg<256>::KT : (D == 128 ? Cfg<128>::KT : Cfg<64>::KT);
}

}  // namespace cp
