// attn_mfma.hip -- bf16 chunk attention on the CDNA4 matrix cores (gfx950).
//
// [SKaiNET] "Change (additive)": attention of C chunk rows over past + C keys
// under an additive mask per head.  Both products are dense contractions, so
// they run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//
// Work split.  A workgroup holds ROWS = 128 or 256 query rows in groups of 32 (one
// wave per group, or two waves sharing it for D = 256, see Cfg); the rows are the G
// query heads of one KV head times qpos = ROWS / G chunk rows, so every K/V tile
// staged in LDS serves the whole GQA group (read from HBM once per query tile).  Workgroups are mapped so that consecutive query tiles of one
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
// Loads.  K/V tiles -- and, with an explicit mask, the tile's ROWS x KT block of
// mask values -- stream into a ring of LDS stages with direct-to-LDS loads
// (global_load_lds, 1 KB per wave instruction for K/V, 256 bytes for the mask),
// STAGES - 1 tiles ahead of the one being computed, without passing through
// registers.  The loads of the next tile are spread between the MFMAs of this
// tile's QK^T, so the issuing wave does not stall on the memory pipeline; the
// waits on them are explicit (vmcnt) followed by a plain s_barrier.  Mask values
// never wait in registers behind in-flight tile loads (loads complete in order).
// Chunk rows come from the caller's k_new / v_new, past rows from the cache
// slots.  Tiles outside the window or past the last real row are skipped.
//
// Pipelining inside a tile: K fragments are read one k-step ahead of the MFMAs,
// and the V^T transpose reads of dim block db + 1 are in flight while block db
// multiplies (the reads of block 0 overlap the softmax arithmetic).
#include <type_traits>

#include "attn_mfma_ops.h"

namespace cp {
namespace {

// Per head size and mask mode: keys per tile, LDS ring stages, waves per SIMD, the
// number of 32-row groups of a workgroup (ROWW) and of wave groups the output dims
// are split over (DSPLIT).  A stage holds one K and one V tile (KT x D bf16 each)
// and, with an explicit mask, the tile's 32 ROWW x KT fp32 mask block.
//  - D = 128: one 256-row workgroup of 8 waves per CU (2 per SIMD) rather than two
//    of 128 rows: each K/V tile serves twice the rows, and the LDS left over holds a
//    4-stage ring, so a tile is requested three tiles before it is needed.
//  - D = 256: DSPLIT = 2, a workgroup of 8 waves where waves w and w + 4 own the same
//    32 query rows, both form the full scores and probabilities, and each accumulates
//    half of the output dims -- a 256-dim accumulator per wave would leave room for
//    only one wave per SIMD and nothing to hide LDS and MFMA latency.
template <int D, bool EX>
struct Cfg;
template <>
struct Cfg<64, false> {
  static constexpr int KT = 64, STAGES = 4, WAVES = 2, DSPLIT = 1;
  static constexpr int ROWW = 4;
};
template <>
struct Cfg<64, true> {
  static constexpr int KT = 32, STAGES = 3, WAVES = 2, DSPLIT = 1;
  static constexpr int ROWW = 4;
};
template <>
struct Cfg<128, false> {
  static constexpr int KT = 64, STAGES = 4, WAVES = 2, DSPLIT = 1;
  static constexpr int ROWW = 8;
};
template <>
struct Cfg<128, true> {
  static constexpr int KT = 32, STAGES = 2, WAVES = 2, DSPLIT = 1;
  static constexpr int ROWW = 4;
};
template <>
struct Cfg<256, false> {
  static constexpr int KT = 32, STAGES = 4, WAVES = 2, DSPLIT = 2;
  static constexpr int ROWW = 4;
};
template <>
struct Cfg<256, true> {
  static constexpr int KT = 32, STAGES = 3, WAVES = 2, DSPLIT = 2;
  static constexpr int ROWW = 4;
};

// Small-rows configuration, for chunks whose rows of one KV head fit 64 (C * G <= 64,
// decode steps included): 64-row workgroups of 32-key tiles in a 2-stage ring, so that
// several workgroups share a CU and stream independent K/V (the regime is HBM-bound:
// a standard workgroup would leave most of its rows empty and stream one tile at a
// time per CU).
//  SM = 1: a 2-stage ring, four workgroups per CU.
//  SM = 2 (in-kernel mask): a 3-stage ring, three per CU, for splits that stream many
//  tiles (long decode contexts), where the steady state needs more bytes in flight per
//  CU than four shallow workgroups keep; short splits prefer more workgroups.
template <int D, bool EX, int SM>
struct Sel : Cfg<D, EX> {};
//  At D = 256 the explicit-mask and deep-ring forms need more than the 256 registers
//  of two waves per SIMD (about 310-340), so they are declared one wave per SIMD: the
//  split planner then counts one workgroup per CU for them, as the hardware runs them.
template <int D, bool EX>
struct Sel<D, EX, 1> {
  static constexpr int KT = 32, STAGES = 2, WAVES = D == 256 && EX ? 1 : 2,
                       DSPLIT = Cfg<D, EX>::DSPLIT;
  static constexpr int ROWW = 2;
};
template <int D, bool EX>
struct Sel<D, EX, 2> : Sel<D, EX, 1> {
  static constexpr int STAGES = EX ? 2 : 3;
  static constexpr int WAVES = D == 256 ? 1 : 2;
};
//  SM = 3 (D = 128, in-kernel rule, 64 < C * G <= 128 rows per KV head): 128-row
//  workgroups of 4 waves with 32-key tiles in a 4-stage ring (64 KB), two per CU.  The
//  standard 256-row workgroup would leave half its rows empty and stream one tile at a
//  time per CU in a regime (C = 32, G = 4) where the keys' bytes, not the products, set
//  the time.
template <int D, bool EX>
struct Sel<D, EX, 3> {
  static constexpr int KT = 32, STAGES = 4, WAVES = 2, DSPLIT = 1;
  static constexpr int ROWW = 4;
};

// EXPLICIT: the additive mask comes from memory.  EXT: use the explicit-mask tiling
// (set with EXPLICIT, and for the in-kernel rule under CP_ATTN_FULL_TILES so that both
// modes see the same key partition).
template <int D, bool EXPLICIT, bool EXT, int SM>
__global__ void __launch_bounds__((64 * Sel<D, EXT, SM>::ROWW * Sel<D, EXT, SM>::DSPLIT))
    __attribute__((amdgpu_waves_per_eu(Sel<D, EXT, SM>::WAVES, Sel<D, EXT, SM>::WAVES)))
    k_attn_mfma(AttnParams p) {
  static_assert(EXT || !EXPLICIT, "explicit masks use the explicit tiling");
  using CF = Sel<D, EXT, SM>;
  constexpr int KT = CF::KT;
  constexpr int STAGES = CF::STAGES;
  constexpr int DSPLIT = CF::DSPLIT;
  constexpr int ROWW = CF::ROWW;    // 32-row groups per workgroup
  constexpr int ROWS = 32 * ROWW;    // query rows per workgroup
  constexpr int NW = ROWW * DSPLIT;  // waves per workgroup
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int NK = KT * CPR;       // chunks per tile (K or V)
  constexpr int NL = NK / (64 * NW); // direct-to-LDS loads per wave per tile per tensor
  constexpr int RPI = 64 / CPR;      // rows covered by one wave-wide 1 KB load
  constexpr int NS = D / 16;         // k-steps of QK^T
  constexpr bool PRESCALE = D == 128;  // Q scaled by scale * log2 e, products from C = -m
  constexpr int NKB = KT / 32;       // 32-key blocks per tile
  constexpr int NDB = D / 32;        // 32-dim blocks of the output
  constexpr int NDW = NDB / DSPLIT;  // ... accumulated by one wave
  constexpr int NPT = KT / 16;       // k-steps of PV
  constexpr int TILE = KT * D;       // bf16 elements of one K (or V) tile
  constexpr int MT = EXPLICIT ? ROWS * KT * 2 : 0;    // mask block (in 16-bit units)
  constexpr int STAGE = 2 * TILE + MT;
  constexpr int NMK = EXPLICIT ? ROWS * KT / (64 * NW) : 0;  // mask loads per wave per tile
  constexpr int ND = 2 * NL + NMK;   // direct-to-LDS loads per wave per tile
  static_assert(!EXPLICIT || (KT == 32 && (ROWS * KT) % (64 * NW) == 0), "mask block split");
  static_assert(NK % (64 * NW) == 0, "tile must split evenly over the waves");
  static_assert(STAGES >= 2 && STAGES <= 4, "ring depth");

  // ring of STAGES x (K tile, V tile[, mask block])
  __shared__ __attribute__((aligned(1024))) uint16_t ring[STAGES * STAGE];
  // explicit mask: element offset of the mask row of each of the ROWS query rows
  __shared__ int64_t mtab[EXPLICIT ? ROWS : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int dgrp = wave / ROWW;      // which NDW dim blocks this wave accumulates

  // Block order.  The hardware dispatches blocks in order and deals them round-robin
  // over 8 XCDs.  The query tiles of one (split, sequence, KV head) group read the same
  // K/V, so they go to one XCD and share its L2; the groups are dealt round-robin over
  // the XCDs, so that sequences of different lengths spread evenly (each XCD drains
  // only its own blocks); and the split index varies slowest, so that the first part
  // of every sequence starts at once and the later parts of long sequences fill the
  // CUs that short sequences free.  When the groups are not a multiple of 8 the blocks
  // go in tile-minor order (a multiple of 8 query tiles: each tile's splits on one XCD),
  // or the group count is padded to the next multiple of 8 (AttnParams::xpad).
  // With a balancing plan, block i takes item i of the plan: its sequence, KV head,
  // query tile, key piece and partial slot, and the sequence's seen and n_valid (one
  // scalar load; the plan kernel read them).
  int qtile, split, nsplit, b, g, slot = -1, seen_in = 0, nv_in = 0;
  if (p.plan) {
    const int32_t *it = p.plan + kPlanHeaderInts + static_cast<size_t>(blockIdx.x) * kPlanItemInts;
    b = it[0];
    g = it[1];
    qtile = it[2];
    split = it[3];
    nsplit = it[4];
    slot = it[5];
    seen_in = it[6];
    nv_in = it[7];
    if (b < 0) return;  // no work in this entry (uniform over the workgroup)
  } else {
    const unsigned nbg = static_cast<unsigned>(p.B) * p.nKV;
    const unsigned groups = static_cast<unsigned>(p.splits) * nbg;
    unsigned gi, qt;
    if (groups % 8 == 0 || p.xpad) {
      const unsigned rest = blockIdx.x / 8;
      qt = rest % p.qtiles;
      gi = (rest / p.qtiles) * 8 + blockIdx.x % 8;
      if (gi >= groups) return;  // padding of the last 8 groups (uniform)
    } else {
      qt = blockIdx.x % p.qtiles;
      gi = blockIdx.x / p.qtiles;
    }
    qtile = static_cast<int>(qt);
    split = static_cast<int>(gi / nbg);
    nsplit = p.splits;
    const int bg0 = static_cast<int>(gi % nbg);
    b = bg0 / p.nKV;
    g = bg0 % p.nKV;
  }
  const int bg = b * p.nKV + g;

  const int r = (wave % ROWW) * 32 + n;
  const int hl = r / p.qpos;
  const int i_min = qtile * p.qpos;
  const int i = i_min + r % p.qpos;
  const bool row_ok = hl < p.G && i < p.C;
  const int head = g * p.G + (row_ok ? hl : 0);
  const int irow = row_ok ? i : 0;

  // Q^T fragments: lane holds q[row n][16 s + 8 hh .. + 7] for every k-step s.  They do
  // not depend on the cache state, so they are requested first and their latency
  // overlaps that of `seen` (and they do not queue behind the first tiles' loads).
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
    // RoPE folded into the load (q given before rotation): dims 16 s + 8 hh + e of the
    // lower half pair with the same lane's dims 16 (s + NS/2) + 8 hh + e, so the
    // rotation is lane-local; the arithmetic and rounding are the RoPE launch's.
    if (p.q_cos) {
      const size_t trow = (static_cast<size_t>(p.q_tables == 1 ? 0 : b) * p.C + irow) * D + 8 * hh;
      const float *tc = p.q_cos + trow, *ts = p.q_sin + trow;
#pragma unroll
      for (int s = 0; s < NS / 2; ++s) {
        const int sh = s + NS / 2;
        const float4 cl0 = *reinterpret_cast<const float4 *>(tc + 16 * s);
        const float4 cl1 = *reinterpret_cast<const float4 *>(tc + 16 * s + 4);
        const float4 sl0 = *reinterpret_cast<const float4 *>(ts + 16 * s);
        const float4 sl1 = *reinterpret_cast<const float4 *>(ts + 16 * s + 4);
        const float4 ch0 = *reinterpret_cast<const float4 *>(tc + 16 * sh);
        const float4 ch1 = *reinterpret_cast<const float4 *>(tc + 16 * sh + 4);
        const float4 sh0 = *reinterpret_cast<const float4 *>(ts + 16 * sh);
        const float4 sh1 = *reinterpret_cast<const float4 *>(ts + 16 * sh + 4);
        const float cl[8] = {cl0.x, cl0.y, cl0.z, cl0.w, cl1.x, cl1.y, cl1.z, cl1.w};
        const float sl[8] = {sl0.x, sl0.y, sl0.z, sl0.w, sl1.x, sl1.y, sl1.z, sl1.w};
        const float chv[8] = {ch0.x, ch0.y, ch0.z, ch0.w, ch1.x, ch1.y, ch1.z, ch1.w};
        const float shv[8] = {sh0.x, sh0.y, sh0.z, sh0.w, sh1.x, sh1.y, sh1.z, sh1.w};
        const u32x4 lo = __builtin_bit_cast(u32x4, qf[s]), hi = __builtin_bit_cast(u32x4, qf[sh]);
        u32x4 ylo, yhi;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t rl = 0, rh = 0;
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const int e = 2 * w + e2;
            const float xl = __uint_as_float(e2 ? lo[w] & 0xffff0000u : lo[w] << 16);
            const float xh = __uint_as_float(e2 ? hi[w] & 0xffff0000u : hi[w] << 16);
            const uint32_t bl = f32_to_bf16_rne(rot_lo(xl, xh, cl[e], sl[e]));
            const uint32_t bh = f32_to_bf16_rne(rot_hi(xl, xh, chv[e], shv[e]));
            rl |= bl << (16 * e2);
            rh |= bh << (16 * e2);
          }
          ylo[w] = rl;
          yhi[w] = rh;
        }
        qf[s] = __builtin_bit_cast(bf16x8, ylo);
        qf[sh] = __builtin_bit_cast(bf16x8, yhi);
      }
    }
    // D = 128 (the long tile loops): scaled by scale * log2 e and rounded to bf16 (RNE),
    // so that the products give the scores in the base-2 units of the softmax with no
    // multiply per score.  (At D = 256 the scaling costs a latency-bound call more
    // than it saves: its scores are scaled in the softmax.)
#pragma unroll
    for (int s = 0; s < (PRESCALE ? NS : 0); ++s) {
      const u32x4 v = __builtin_bit_cast(u32x4, qf[s]);
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack_bf16x2(__uint_as_float(v[e] << 16) * p.sl2e,
                           __uint_as_float(v[e] & 0xffff0000u) * p.sl2e);
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // seen and n_valid are both requested before either is used (scalar loads complete
  // out of order, so the first use waits for every one in flight: one round trip)
  const int seen = p.plan ? seen_in : p.seen[b];
  int nv = p.plan ? nv_in : (p.n_valid ? p.n_valid[b] : p.C);
  const bool lead = tid == 0 && qtile == 0 && split == 0 && g == 0;
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
  const bool real_row = row_ok && i < nv;
  // this wave's real rows (for its own tile visibility test)
  const int wi_lo = wave_min_i(real_row ? i : 0x7fffffff);
  const int wi_hi = wave_max_i(real_row ? i : -1);

  if constexpr (EXPLICIT) {
    // mask row of query row t (rows past the tile's end read a valid row; their
    // results are discarded), then make the table visible to every wave.
    if (tid < ROWS) {
      const int hl_t = imin(tid / p.qpos, p.G - 1);
      const int i_t = imin(i_min + tid % p.qpos, p.C - 1);
      mtab[tid] = b * p.mbs + static_cast<int64_t>(g * p.G + hl_t) * p.mhs +
                  static_cast<int64_t>(i_t) * p.mld;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
  }
  // Mask loads: load j of every tile reads the same rows and chunk positions, so each
  // lane's row offset and column within the tile are formed once (float P = q * 64 +
  // lane of the block: row P / 32, physical chunk (P % 32) / 4 holding the row's logical
  // chunk physical ^ mswz(row)).
  int64_t mrow[EXPLICIT ? NMK : 1];
  int mcol[EXPLICIT ? NMK : 1];
  if constexpr (EXPLICIT) {
#pragma unroll
    for (int j = 0; j < NMK; ++j) {
      const int P = (wave * NMK + j) * 64 + lane;
      const int row = P >> 5, pp = P & 31;
      mrow[j] = mtab[row];
      mcol[j] = 4 * ((pp >> 2) ^ mswz(row)) + (pp & 3);
    }
  }

  f32x16 oacc[NDW];
#pragma unroll
  for (int db = 0; db < NDW; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[db][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  // With the scaled Q the score products start from C = -msub (nmb), so that they give
  // s' = s * scale * log2 e - msub, the exponent of the probability: msub is the
  // running maximum once a row has seen an attended key (0 before).  Otherwise the
  // products give the raw scores s and the softmax scales them (kq = scale * log2 e).
  const float kq = PRESCALE ? 1.f : p.sl2e;
  float msub = 0.f;
  f32x16 nmb;
#pragma unroll
  for (int e = 0; e < 16; ++e) nmb[e] = 0.f;

  TileSeq ts{};
  int u0 = 0, u1 = 0;
  if (any_real) {
    ts = make_tiles(gl, seen, p.C, KT, i_min, i_last, EXPLICIT ? 0 : p.window, p.sink,
                    EXPLICIT || p.full_tiles);
    // near-equal split ranges, the first cnt % splits one tile longer (one 32-bit
    // division: a 64-bit one is a long software sequence ahead of the first load)
    const unsigned cnt = static_cast<unsigned>(ts.count()), ns = static_cast<unsigned>(nsplit);
    const unsigned q = cnt / ns, rm = cnt - q * ns, us = static_cast<unsigned>(split);
    u0 = static_cast<int>(us * q + (us < rm ? us : rm));
    u1 = u0 + static_cast<int>(q + (us < rm ? 1u : 0u));
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
  // read a valid row instead; their scores are masked to -inf.  The source of load e
  // is a scalar base plus a 32-bit per-lane byte offset: lk[e] / lv[e] (the tile row
  // lrow[e] and its swizzled chunk, fixed for the loop) plus, on a tile whose rows are
  // not consecutive slots from `first` (ring wrap, a partial last tile), the lane's
  // own row shift d[e].
  uint32_t lk[NL], lv[NL];
  int lrow[NL];
#pragma unroll
  for (int e = 0; e < NL; ++e) {
    const int row = (wave * NL + e) * RPI + lane / CPR, phys = lane % CPR;
    lrow[e] = row;
    lk[e] = static_cast<uint32_t>(row * (2 * D) + ((phys ^ kswz<D>(row)) << 4));
    lv[e] = static_cast<uint32_t>(row * (2 * D) + ((phys ^ vswz<D>(row)) << 4));
  }
  const char *KCb = reinterpret_cast<const char *>(KC), *VCb = reinterpret_cast<const char *>(VC);
  const char *KNb = reinterpret_cast<const char *>(KN), *VNb = reinterpret_cast<const char *>(VN);
  // Tile u's sources.  At D = 128 (long tile loops) the loads ahead of the final tiles
  // are issued too, reading the last tile again into the stage a real load would
  // refill: every tile issues the same loads, with no branch.  At D = 64 and 256 (short
  // calls, few tiles per split) they are skipped: there they only added latency.
  struct Src {
    const char *k, *v;
    uint32_t d[NL];
    int first, lim;
    bool chunk;
  };
  auto plan = [&](int u) __attribute__((always_inline)) {
    Src sr;
    sr.chunk = ts.at(imin(u, u1 - 1), KT, &sr.first);
    sr.lim = sr.chunk ? p.C : gl.L;
    sr.k = sr.chunk ? KNb : KCb;
    sr.v = sr.chunk ? VNb : VCb;
    const bool ringp = !sr.chunk && p.ring && sr.first + KT > gl.ns;
#pragma unroll
    for (int e = 0; e < NL; ++e) sr.d[e] = 0;
    // a tile of KT consecutive slots from base_row, or -1.  A ring tile past the sinks
    // that does not wrap qualifies at D = 256 only: same box, the ring path was faster
    // per lane at D = 128 (sliding layers 132.4-132.9 against 136.0-137.4 us) and as a
    // base at D = 256 (16.6 against 16.9 us).
    int base_row = -1;
    if (!ringp) {
      if (sr.first + KT <= sr.lim) base_row = sr.first;
    } else if (D != 128 && !small_ring && sr.first >= gl.ns && sr.first + KT <= sr.lim) {
      const int s0 = slot_of(gl.lo + (sr.first - gl.ns), p.cap, 1, p.sink);
      if (s0 + KT <= p.cap) base_row = s0;
    }
    if (base_row >= 0) {
      // the shift is the base's
      const size_t off = static_cast<size_t>(base_row) * (2 * D);
      sr.k += off;
      sr.v += off;
    } else {
      const int c_ns = imax(sr.first, gl.ns);
      int s_ns = 0;
      if (ringp && !small_ring && c_ns < gl.L) s_ns = slot_of(gl.lo + (c_ns - gl.ns), p.cap, 1, p.sink);
#pragma unroll
      for (int e = 0; e < NL; ++e) {
        const int col = imin(sr.first + lrow[e], sr.lim - 1);
        int sl = col;
        if (ringp && col >= gl.ns) {
          if (!small_ring) {
            sl = s_ns + (col - c_ns);
            if (sl >= p.cap) sl -= R;
          } else {
            sl = slot_of(gl.lo + (col - gl.ns), p.cap, 1, p.sink);
          }
        }
        sr.d[e] = static_cast<uint32_t>(sl - lrow[e]) * (2 * D);
      }
    }
    return sr;
  };
  // load j of a tile into ring stage st: j < NL K rows, j < 2 NL V rows, else 256
  // bytes of the mask block (positions from mrow / mcol above; columns clamped into the
  // valid range -- those past it are masked to -inf)
  auto dma = [&](int j, const Src &sr, uint16_t *st) __attribute__((always_inline)) {
    if (j < 2 * NL) {
      const int e = j < NL ? j : j - NL;
      const int q = wave * NL + e;
      if (j < NL)
        dma16(reinterpret_cast<const uint16_t *>(sr.k + (lk[e] + sr.d[e])), st + q * 512);
      else
        dma16(reinterpret_cast<const uint16_t *>(sr.v + (lv[e] + sr.d[e])), st + TILE + q * 512);
    } else if constexpr (EXPLICIT) {
      const int jm = j - 2 * NL;
      const int q = wave * NMK + jm;
      const int col = imin(sr.first + mcol[jm], sr.lim - 1);
      dma4(p.mask + mrow[jm] + (sr.chunk ? static_cast<int64_t>(gl.L) : 0) + col,
           reinterpret_cast<float *>(st + 2 * TILE) + q * 64);
    }
  };

  // per-lane LDS read geometry
  const int k_sw = kswz<D>(n);  // rows 32 kb + n share n's swizzle
  const int s16 = lane & 15;
  const int v_key = 4 * hh + (s16 >> 2);           // + 16 t (+ 8)
  const int v_sw = vswz<D>(v_key);                // (16 t + 8 keeps it)
  const int v_cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within a 32-dim block
  const int v_el = 4 * (lane & 1);

  const int qabs = seen + i;

  // In-kernel rule for this lane's row as column ranges.  A past column c attends
  // iff c < pa1 (sink rows; for a global cache the first `sink` positions) or
  // c >= pb0 (inside the window); a chunk row j iff j < cb1 (causal, real) and
  // (j < ca1 (a sink position) or j >= cb0 (inside the window)).
  int pa1 = 0x7fffffff, pb0 = 0, ca1 = 0x7fffffff, cb0 = 0;
  const int cb1 = imin(i, nv - 1) + 1;
  if (!EXPLICIT && p.window > 0) {
    pa1 = p.ring ? gl.ns : p.sink;
    pb0 = qabs - p.window + 1 - gl.lo + gl.ns;
    ca1 = p.sink - seen;
    cb0 = i - p.window + 1;
  }

  // V^T operand reads of one 32-dim block (2 * NPT transpose reads)
  auto v_reads = [&](uint32_t vbase, int db, u32x2 *w) __attribute__((always_inline)) {
    const uint32_t va = vbase + 2 * ((((4 * (dgrp * NDW + db) + v_cl) ^ v_sw) << 3) + v_el);
    tr_read_rows<D, 0, NPT>(va, w);
  };

  // ---- the pieces of one tile
  // S^T = K Q^T for the tile in Ks, K fragments read one k-step ahead; hook(s) runs
  // after k-step s (the caller's direct-to-LDS loads, spread over the steps)
  auto qk_tile = [&](const uint16_t *Ks, f32x16 *sacc, auto &&hook) __attribute__((always_inline)) {
    // K fragments of KP k-steps in flight; lane: key row 32 kb + n, 16-byte chunk
    // 2 s + hh of the row, stored at chunk (2 s + hh) ^ k_sw = 2 s ^ (hh ^ k_sw)
    constexpr int KP = NS < 3 ? NS : 3;
    const uint32_t kbase = lds_addr(Ks) + 2 * (n * D);
    const int kx = hh ^ k_sw;
    u32x4 kf[KP][NKB];
    __builtin_amdgcn_s_setprio(1);  // the products go first when both waves of a SIMD are ready
#pragma unroll
    for (int s = 0; s + 1 < KP; ++s) k_read_blocks<D, 0, NKB>(kbase + 16 * ((2 * s) ^ kx), kf[s]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + KP - 1 < NS)
        k_read_blocks<D, 0, NKB>(kbase + 16 * ((2 * (s + KP - 1)) ^ kx), kf[(s + KP - 1) % KP]);
      // reads issued after step s's: those of the steps still ahead
      const int later = (NS - 1 - s < KP - 1 ? NS - 1 - s : KP - 1) * NKB;
      u32x4 *cur = kf[s % KP];
      if (later >= 2 * NKB)
        k_wait<2 * NKB, NKB>(cur);
      else if (later >= NKB)
        k_wait<NKB, NKB>(cur);
      else
        k_wait<0, NKB>(cur);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        sacc[kb] = mfma(__builtin_bit_cast(bf16x8, cur[kb]), qf[s],
                        s == 0 ? (PRESCALE ? nmb : f32x16{}) : sacc[kb]);
      hook(s);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Masking and online softmax of tile u: turns the scores in sacc into the bf16
  // probabilities pb, rescaling the running output when the row maximum rises.
  // (Mask blocks, for an explicit mask, are read from the tile's ring stage Ms.)
  auto softmax_tile = [&](int u, f32x16 *sacc, const float *Mst, bf16x8 *pb)
                          __attribute__((always_inline)) {
    int first;
    const bool chunk = ts.at(u, KT, &first);
    // ---- tile classification (wave-uniform): does every real row of this wave
    // attend every key of the tile?  Then no mask work at all.
    const int lim = chunk ? p.C : gl.L;
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

    // ---- online softmax in base 2 on s' = kq * (products) - msub (kq = 1, or the scale
    // for the raw scores of the unscaled Q): visible tiles use p = 2^s' directly;
    // masked tiles first add bias * log2 e.  (scale > 0, so max(s) * c = max(s * c).)
    float mt = -INFINITY;
    if (visible) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[kb][e]);
      if (!PRESCALE) {
        mt *= kq;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) sacc[kb][e] = fmaf(sacc[kb][e], kq, -msub);
        mt -= msub;
      }
    } else if constexpr (EXPLICIT) {
      // mask block of this stage, row r of this lane; keys past the valid range -inf
      const float *Ms = Mst + r * KT;
      const int xl = lim - first - 4 * hh;
      const int msw = mswz(r);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const float4 mv =
              *reinterpret_cast<const float4 *>(Ms + 4 * ((8 * kb + 2 * rq + hh) ^ msw));
          const float m4[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = 32 * kb + 8 * rq + e;
            const float a = k < xl ? m4[e] : -INFINITY;
            const float tv = PRESCALE ? sacc[kb][4 * rq + e] + a * kLog2e
                                      : fmaf(sacc[kb][4 * rq + e], kq, a * kLog2e - msub);
            sacc[kb][4 * rq + e] = tv;
            mt = fmaxf(mt, tv);
          }
        }
    } else {
      // column c of key k of this lane is base + k; compare against range bounds
      // shifted by base once per tile
      const int base = first + 4 * hh;
      const int xl = lim - base;
      int xa, xb, xc = 0x7fffffff;
      if (chunk) {
        xa = ca1 == 0x7fffffff ? 0x7fffffff : ca1 - base;
        xb = cb0 - base;
        xc = cb1 - base;
      } else {
        xa = pa1 == 0x7fffffff ? 0x7fffffff : pa1 - base;
        xb = pb0 - base;
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = 32 * kb + 8 * rq + e;
            const bool att = (k < xc) & ((k < xa) | (k >= xb));
            const float a = k < xl ? (att ? 0.f : kMasked) : -INFINITY;
            const float tv = PRESCALE ? sacc[kb][4 * rq + e] + a * kLog2e
                                      : fmaf(sacc[kb][4 * rq + e], kq, a * kLog2e - msub);
            sacc[kb][4 * rq + e] = tv;
            mt = fmaxf(mt, tv);
          }
    }
    // The maximum over the lane pair; a rise by more than 2^8 over the running maximum
    // (or the row's first attended key) moves msub there: the tile's scores shift by
    // the rise, C = -msub for the next tiles, and l and O are rescaled.  A row with no
    // attended key in the tile (its maximum near -1e30 log2 e, or -inf) never moves
    // msub: C must stay near the real scores, or fp32 would lose them.
    mt = pair_max(mt);
    const float mabs = mt + msub;
    const bool raise = mabs > m_run + kRescaleSlack && mabs > kNoKeyFloor;
    if (__any(raise)) {
      const float m_new = raise ? mabs : m_run;
      const float delta = raise ? mt : 0.f;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;  // 0 from -inf
      m_run = m_new;
      msub = raise ? m_new : msub;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDW; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[kb][e] -= delta;
      if (PRESCALE) {
#pragma unroll
        for (int e = 0; e < 16; ++e) nmb[e] = -msub;
      }
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = sacc[kb][8 * half + 2 * e], x1 = sacc[kb][8 * half + 2 * e + 1];
          const float p0 = __builtin_amdgcn_exp2f(x0);
          const float p1 = __builtin_amdgcn_exp2f(x1);
          l_run += p0 + p1;
          w[e] = pack_bf16x2(p0, p1);
        }
        pb[2 * kb + half] = __builtin_bit_cast(bf16x8, w);
      }
    }
  };

  // O^T += V^T P^T for the V tile at LDS byte address vbase; the reads of dim block 0
  // are already in wv[0], those of block db + 1 are in flight while block db multiplies
  auto pv_tile = [&](uint32_t vbase, const bf16x8 *pb, u32x2 (*wv)[2 * NPT])
                     __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < NDW; ++db) {
      u32x2 *cur = wv[db & 1];
      if (db + 1 < NDW) {
        v_reads(vbase, db + 1, wv[(db + 1) & 1]);
        lds_wait_keep<2 * NPT, 2 * NPT>(cur);
      } else {
        lds_wait_keep<0, 2 * NPT>(cur);
      }
#pragma unroll
      for (int t = 0; t < NPT; ++t) {
        const u32x4 a = {cur[2 * t][0], cur[2 * t][1], cur[2 * t + 1][0], cur[2 * t + 1][1]};
        oacc[db] = mfma(__builtin_bit_cast(bf16x8, a), pb[t], oacc[db]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Staggered stages (in-kernel rule, 8 waves as two per SIMD): waves 4..7 run a tile's
  // stages as [O update of the previous tile, S, softmax] and waves 0..3 as [S, softmax,
  // O update], so after each barrier one wave's softmax meets the other's matrix
  // products on every SIMD.  V of tile u - 1 is then still read after the barrier of
  // tile u, so the ring loads STAGES - 2 tiles ahead instead of STAGES - 1.
  constexpr bool STAG = !EXPLICIT && NW == 8 && CF::WAVES == 2 && SM == 0 && STAGES >= 3;
  constexpr int PD = STAG ? STAGES - 2 : STAGES - 1;  // tiles loaded ahead
  constexpr bool ALL_LOADS = D == 128;                // loads past the last tile too
  const bool lagging = STAG && __builtin_amdgcn_readfirstlane(wave) >= 4;

  // tile u lives in stage u % STAGES of a ring of (K, V) tiles (a key split starts
  // at u0 > 0); tiles u0 .. u0 + PD - 1 are loaded ahead (repeats of the last tile past
  // it)
  if (u1 > u0)
    for (int j = 0; j < PD; ++j) {
      if (!ALL_LOADS && u0 + j >= u1) break;
      const Src sr = plan(u0 + j);
      uint16_t *st = ring + ((u0 + j) % STAGES) * STAGE;
#pragma unroll
      for (int l = 0; l < ND; ++l) dma(l, sr, st);
    }

  // the tile loop, specialized for the leading and the lagging order (one copy each, so
  // neither carries the other's registers)
  auto tile_loop = [&](auto lag_tag) __attribute__((always_inline)) {
    constexpr bool LAG = decltype(lag_tag)::value;
    bf16x8 pb_lag[NPT];  // LAG waves: probabilities of the tile before
  #pragma unroll
    for (int t = 0; t < NPT; ++t) pb_lag[t] = bf16x8{};
    for (int u = u0; u < u1; ++u) {
      // tile u has landed in this wave's share of the ring once at most the loads of
      // the tiles issued after it are outstanding; the barrier makes that true for all
      // waves and also guarantees every wave has finished reading the stage refilled
      wait_tiles_after<ND, STAGES>(ALL_LOADS ? PD - 1 : imin(u1 - 1, u + PD - 1) - u);
      __builtin_amdgcn_s_barrier();
      const uint16_t *Ks = ring + (u % STAGES) * STAGE;
      const uint16_t *Vs = Ks + TILE;

      if (LAG && u > u0) {  // the previous tile's O update (its V still in the ring)
        const uint32_t vb = lds_addr(ring + ((u - 1) % STAGES) * STAGE + TILE) + 2 * (v_key * D);
        u32x2 wv[2][2 * NPT];
        v_reads(vb, 0, wv[0]);
        pv_tile(vb, pb_lag, wv);
      }

      // the tile PD ahead is loaded while this one's QK^T runs
      const int w_pf = u + PD;
      const bool pf = ALL_LOADS || w_pf < u1;
      const Src psr = plan(w_pf);
      uint16_t *pst = ring + (w_pf % STAGES) * STAGE;

      f32x16 sacc[NKB];
      qk_tile(Ks, sacc, [&](int s) __attribute__((always_inline)) {
  #pragma unroll
        for (int j = s * ND / NS; j < (s + 1) * ND / NS; ++j)
          if (pf) dma(j, psr, pst);
      });

      if (LAG) {
        softmax_tile(u, sacc, reinterpret_cast<const float *>(Ks + 2 * TILE), pb_lag);
      } else {
        // V^T reads of the first dim block go out before the softmax needs the ALUs
        const uint32_t vbase = lds_addr(Vs) + 2 * (v_key * D);
        u32x2 wv[2][2 * NPT];
        v_reads(vbase, 0, wv[0]);
        bf16x8 pb[NPT];
        softmax_tile(u, sacc, reinterpret_cast<const float *>(Ks + 2 * TILE), pb);
        pv_tile(vbase, pb, wv);
      }
    }
    if (LAG && u1 > u0) {  // the last tile's O update (no load refills the ring now)
      const uint32_t vb = lds_addr(ring + ((u1 - 1) % STAGES) * STAGE + TILE) + 2 * (v_key * D);
      u32x2 wv[2][2 * NPT];
      v_reads(vb, 0, wv[0]);
      pv_tile(vb, pb_lag, wv);
    }
  };
  if (lagging)
    tile_loop(std::integral_constant<bool, true>{});
  else
    tile_loop(std::integral_constant<bool, false>{});
  // the repeated loads of the last tiles land before the workgroup's LDS is released
  if (ALL_LOADS) wait_vm<0>();

  const float l_tot = pair_sum(l_run);
  if (!row_ok) return;
  const bool real = any_real && i < nv;
  const size_t orow = (static_cast<size_t>(b) * p.H + head) * p.C + i;
  if (nsplit == 1) {
    uint16_t *O = static_cast<uint16_t *>(p.out) + orow * D;
    uint16_t *S = p.sel && i == selected_row(nv)
                      ? static_cast<uint16_t *>(p.sel) + (static_cast<size_t>(b) * p.H + head) * D
                      : nullptr;
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
        if (S) *reinterpret_cast<u32x2 *>(S + d) = w;
      }
    }
  } else if (i < nv) {  // partials of real rows only: the merge writes pad rows as zeros
    // fragment order (p.frag_rows == ROWS): the accumulators leave as they sit in the
    // lanes, each store instruction 512 bytes of consecutive bytes (in row order every
    // one would touch 32 rows)
    const size_t nu = static_cast<size_t>(p.B) * p.nKV * p.qtiles * ROWW;
    const size_t u = (static_cast<size_t>(bg) * p.qtiles + qtile) * ROWW + wave % ROWW;
    const size_t grp = slot >= 0 ? static_cast<size_t>(slot) * ROWW + wave % ROWW
                                 : static_cast<size_t>(split) * nu + u;
    // normalized (O / l) in bf16, half the bytes of fp32 sums; the merge weighs each
    // split by 2^(m - M) l (an empty split: l = 0, zeros here)
    uint16_t *WO = reinterpret_cast<uint16_t *>(p.wo) + grp * (D / 32) * 1024 + 4 * lane;
    const float inv = real && l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < NDW; ++db) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const u32x2 w = {pack_bf16x2(oacc[db][4 * rq + 0] * inv, oacc[db][4 * rq + 1] * inv),
                         pack_bf16x2(oacc[db][4 * rq + 2] * inv, oacc[db][4 * rq + 3] * inv)};
        *reinterpret_cast<u32x2 *>(WO + (dgrp * NDW + db) * 1024 + rq * 256) = w;
      }
    }
    if (hh == 0 && dgrp == 0) {
      float *ML = p.wml + (grp * 32 + n) * 2;
      ML[0] = real ? m_run : -INFINITY;
      ML[1] = real ? l_tot : 0.f;
    }
  }
}

template <int D, bool EXPLICIT, bool EXT, int SM>
hipError_t launch_one(const AttnParams &p, unsigned blocks, hipStream_t s) {
  using CF = Sel<D, EXT, SM>;
  // split partials go out in the fragment order of this configuration's query tile
  if ((p.splits > 1 || p.plan) && p.frag_rows != 32 * CF::ROWW) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_attn_mfma<D, EXPLICIT, EXT, SM>), dim3(blocks),
                     dim3(64 * CF::ROWW * CF::DSPLIT), 0, s, p);
  return hipSuccess;
}

template <int D, int SM>
hipError_t launch_mode(const AttnParams &p, unsigned blocks, hipStream_t s) {
  if (p.mask) return launch_one<D, true, true, SM>(p, blocks, s);
  if (p.full_tiles) return launch_one<D, false, true, SM>(p, blocks, s);
  return launch_one<D, false, false, SM>(p, blocks, s);
}

template <int D>
hipError_t launch_d(const AttnParams &p, hipStream_t s) {
  const unsigned nu = static_cast<unsigned>(p.qtiles) * p.B * p.nKV;
  unsigned blocks = nu * p.splits;
  if (p.plan) {
    blocks = static_cast<unsigned>(p.plan_grid);
  } else if (p.xpad) {
    // the (split, sequence, KV head) groups padded to a multiple of 8
    const unsigned groups = static_cast<unsigned>(p.splits) * p.B * p.nKV;
    blocks = (groups + 7) / 8 * 8 * p.qtiles;
  }
  if (blocks == 0) return hipSuccess;
  hipError_t e;
  if (p.small_rows == 3) {
    // medium rows: D = 128 and the in-kernel rule only
    if constexpr (D == 128) {
      if (p.mask || p.full_tiles) return hipErrorInvalidValue;
      e = launch_one<D, false, false, 3>(p, blocks, s);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (p.small_rows == 2) {
    if (p.mask || p.full_tiles) return hipErrorInvalidValue;  // deep ring: in-kernel rule only
    e = launch_one<D, false, false, 2>(p, blocks, s);
  } else if (p.small_rows == 1) {
    e = launch_mode<D, 1>(p, blocks, s);
  } else {
    e = launch_mode<D, 0>(p, blocks, s);
  }
  return e != hipSuccess ? e : hipGetLastError();
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

template <bool EX, int SM>
int rows_of(int D) {
  return 32 * (D == 256 ? Sel<256, EX, SM>::ROWW
                        : (D == 128 ? Sel<128, EX, SM>::ROWW : Sel<64, EX, SM>::ROWW));
}
template <bool EX, int SM>
int keys_of(int D) {
  return D == 256 ? Sel<256, EX, SM>::KT
                  : (D == 128 ? Sel<128, EX, SM>::KT : Sel<64, EX, SM>::KT);
}

// small_rows: 0 standard, 1 small rows, 2 small rows with the deep ring (same tiling)
int mfma_rows_per_tile(int D, bool explicit_tiling, int small_rows) {
  if (small_rows == 3) return 32 * Sel<128, false, 3>::ROWW;
  if (small_rows) return explicit_tiling ? rows_of<true, 1>(D) : rows_of<false, 1>(D);
  return explicit_tiling ? rows_of<true, 0>(D) : rows_of<false, 0>(D);
}

// Workgroups of one configuration resident per CU: waves (the kernels ask for two per
// SIMD) and LDS (ring, plus the explicit mask's row table) both bound it.
template <int D, bool EX, int SM>
int wgs_of() {
  using CF = Sel<D, EX, SM>;
  constexpr int STAGE = 2 * CF::KT * D + (EX ? 32 * CF::ROWW * CF::KT * 2 : 0);
  constexpr int lds = CF::STAGES * STAGE * 2 + (EX ? 32 * CF::ROWW * 8 : 0);
  constexpr int by_waves = 4 * CF::WAVES / (CF::ROWW * CF::DSPLIT);
  constexpr int by_lds = 160 * 1024 / lds;
  return by_waves < by_lds ? by_waves : by_lds;
}
template <bool EX, int SM>
int wgs_d(int D) {
  return D == 256 ? wgs_of<256, EX, SM>() : (D == 128 ? wgs_of<128, EX, SM>() : wgs_of<64, EX, SM>());
}

int mfma_wgs_per_cu(int D, bool explicit_tiling, int small_rows) {
  if (small_rows == 3) return wgs_of<128, false, 3>();
  if (small_rows == 2) return wgs_d<false, 2>(D);
  if (small_rows == 1) return explicit_tiling ? wgs_d<true, 1>(D) : wgs_d<false, 1>(D);
  return explicit_tiling ? wgs_d<true, 0>(D) : wgs_d<false, 0>(D);
}

int mfma_keys_per_tile(int D, bool explicit_tiling, int small_rows) {
  if (small_rows == 3) return Sel<128, false, 3>::KT;
  if (small_rows) return explicit_tiling ? keys_of<true, 1>(D) : keys_of<false, 1>(D);
  return explicit_tiling ? keys_of<true, 0>(D) : keys_of<false, 0>(D);
}

}  // namespace cp
