// attn_common.h -- pieces shared by the two attention kernels of libcp.
//
// [SKaiNET] "Change (additive)": attention of C chunk rows over past + C keys
// with an additive mask (0 attends, -1e30 masks) that carries the causal band,
// the zero padding and the sliding window.  The keys are the live past rows in
// chronological order followed by the chunk's own rows; the past is read as
// it stands before the chunk is appended.
#pragma once

#include "cp_common.h"

namespace cp {

// Kernel parameters (passed by value).
struct AttnParams {
  const void *q, *kn, *vn, *kc, *vc;
  void *out;
  void *sel;   // optional [B][H][D]: copy of the row max(n_valid, 1) - 1 of out
  const int32_t *seen, *n_valid;
  int32_t *status;
  const float *mask;
  int64_t mld, mhs, mbs;
  // Split partials.  Row-major (frag_rows == 0, vector-ALU kernel): fp32 sums O
  // [S][B][H][C][D], m and l [S][B][H][C][2].  Fragment order (frag_rows = R, the rows
  // of one query tile, a multiple of 32; matrix-core kernel): bf16 normalized O / l; a
  // query tile's rows form R / 32 groups of 32, numbered
  // u = ((b * nKV + g) * qtiles + qtile) * (R / 32) + group, NU groups in all; O of
  // split s, group u, dims 32 k .. 32 k + 31 is a block of 1024 elements at
  // ((s * NU + u) * (D / 32) + k) * 1024, holding row n of the group, dims
  // 32 k + 8 j + 4 h + e (n, j, e < 4, h < 2) at (j * 64 + 32 h + n) * 4 + e -- the
  // order in which a 32 x 32 matrix-core accumulator sits in a wave's lanes, so that
  // each store instruction writes 512 consecutive bytes; fp32 m and l of the row at
  // ((s * NU + u) * 32 + n) * 2.  Row r of a query tile is head g * G + r / qpos,
  // chunk row qtile * qpos + r % qpos.
  float *wo;
  float *wml;
  int frag_rows;
  int B, H, nKV, C, cap, ring, sink, window;
  int G;       // query heads per KV head
  int qpos;    // chunk rows per query tile
  int hb;      // heads per tile (vector-ALU kernel)
  int hgroups; // head groups per KV head (vector-ALU kernel)
  int qtiles;  // query tiles per (b, kv head, head group)
  int splits;
  int full_tiles;
  int small_rows; // matrix-core kernel: 0, the 64-row configuration (1), its deep ring (2),
                  // or the 128-row medium configuration (3)
  float sl2e;     // scale * log2(e)
  int advance;    // the split merge also advances cache.seen by n_valid (early append)
  cp_cache cache; // the cache the call reads (for advance)
  // RoPE of q at load time: fp32 [q_tables][C][D] tables, or nullptr (q already rotated)
  const float *q_cos, *q_sin;
  int q_tables;
  // Block order of the matrix-core kernel when its (split, sequence, KV head) groups are
  // not a multiple of 8: 1 pads their count to one (the query tiles of each group share
  // an XCD, its K/V fetched once), 0 deals the query tiles in order.  (This and xmerge
  // are 16-bit and sit in the padding after q_tables: the block stays 320 bytes, five
  // 64-byte lines that the kernels request at once.)
  int16_t xpad;
  // Merge of fragment-order partials: 0 deals its blocks in order; M > 0 puts the blocks
  // of M consecutive 32-row groups (numbered as in AttnParams::wo) on one XCD, unit j
  // on XCD j % 8, so that the output lines a unit writes are whole in one L2.
  int16_t xmerge;
  // Balanced key splits (matrix-core kernel): the plan written by the plan kernel, or
  // nullptr.  Block i of the attention takes item i; split items write their partials to
  // their slot (AttnParams::wo in fragment order, slot * (frag_rows / 32) groups).
  const int32_t *plan;
  int plan_grid;   // blocks of the attention launch = item entries
  int plan_slots;  // workgroups the GPU holds at once
  int plan_kt;     // keys per tile
  int plan_tmin;   // fewest tiles per piece
};
// the kernels request their argument block as five 64-byte lines; a sixth line measured
// 0.2 us more per short step
static_assert(sizeof(AttnParams) <= 320, "AttnParams outgrew five 64-byte lines");

// Plan layout (int32): a header (split entries, piece length, total tiles, units), then
// plan_grid items of kPlanItemInts (sequence, KV head, query tile, piece, pieces, partial
// slot or -1, seen, n_valid; sequence -1: no work), then the split entries (sequence, KV
// head, query tile, pieces, first partial slot, n_valid clamped).
constexpr int kPlanHeaderInts = 64;
constexpr int kPlanItemInts = 8;
constexpr int kPlanMaxB = 1024;  // sequences a plan can balance

// Requests every 64-byte line of a kernel's argument block in one batch, so that the
// later reads of its fields hit the scalar cache.  Left to itself the compiler reads
// the fields lazily, a line or two at a time, and waits for each batch before the
// next: several memory round trips in a row ahead of the first dependent load.
template <typename P>
__device__ __forceinline__ void request_args(const P &p) {
  constexpr int kLines = static_cast<int>((sizeof(P) + 63) / 64);
  static_assert(kLines >= 1 && kLines <= 6, "argument block of at most six lines");
  const int32_t *w = reinterpret_cast<const int32_t *>(&p);
  int32_t v[6];
#pragma unroll
  for (int k = 0; k < 6; ++k) v[k] = w[16 * (k < kLines ? k : kLines - 1)];
  asm volatile("" ::"s"(v[0]), "s"(v[1]), "s"(v[2]), "s"(v[3]), "s"(v[4]), "s"(v[5]));
}

// Ordered list of the key tiles one query tile needs.  Past tiles cover
// columns [t*kt, t*kt + kt) of the live past, chunk tiles rows [t*kt, ...).
// With the in-kernel mask, tiles no real row of the query tile attends
// (older than the window, later than the last real row) are left out; part A
// is the tiles holding pinned sink rows.
struct TileSeq {
  int nA, tB0, nB, tC0, nC;
  __device__ int count() const { return nA + nB + nC; }
  // returns true for a chunk tile; *first = first column (past) or row (chunk)
  __device__ bool at(int u, int kt, int *first) const {
    if (u < nA) {
      *first = u * kt;
      return false;
    }
    u -= nA;
    if (u < nB) {
      *first = (tB0 + u) * kt;
      return false;
    }
    *first = (tC0 + u - nB) * kt;
    return true;
  }
};

__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }
__device__ __forceinline__ int imin(int a, int b) { return a < b ? a : b; }

// Chunk row whose output is also written to the selection (the last real row; row 0,
// all zeros, when a sequence has no real row).
__device__ __forceinline__ int selected_row(int nv) { return nv > 0 ? nv - 1 : 0; }

__device__ __forceinline__ TileSeq make_tiles(const Live &g, int seen, int C, int kt, int i_min,
                                              int i_last, int window, int sink, bool full) {
  TileSeq s;
  const int nPT = (g.L + kt - 1) / kt;
  if (full) {
    s.nA = 0;
    s.tB0 = 0;
    s.nB = nPT;
    s.tC0 = 0;
    s.nC = (C + kt - 1) / kt;
    return s;
  }
  s.nA = (g.ns + kt - 1) / kt;
  int cfirst = g.ns;
  if (window > 0) {
    const long pfirst = static_cast<long>(seen) + i_min - window + 1;
    long d = pfirst - g.lo;
    if (d < 0) d = 0;
    if (d > g.L - g.ns) d = g.L - g.ns;
    cfirst = g.ns + static_cast<int>(d);
  }
  s.tB0 = imax(s.nA, cfirst / kt);
  s.nB = imax(0, nPT - s.tB0);
  int jlo = 0;
  if (window > 0 && seen >= sink) jlo = imax(0, i_min - window + 1);
  const int jhi = i_last + 1;
  s.tC0 = jlo / kt;
  s.nC = imax(0, (jhi + kt - 1) / kt - s.tC0);
  return s;
}

// True when every real row of the query tile attends every key of the tile,
// so the in-kernel mask can be skipped for it.
__device__ __forceinline__ bool tile_all_visible(bool chunk, int first, int kt, const Live &g,
                                                 int seen, int C, int i_min, int i_last,
                                                 int window) {
  if (chunk) {
    if (first + kt > C || first + kt - 1 > i_min) return false;
    return window == 0 || i_last - first < window;
  }
  if (first + kt > g.L) return false;
  if (window == 0) return true;
  const int cn = imax(first, g.ns);  // first non-sink column: the oldest position
  if (cn >= first + kt) return true;  // sink rows only
  return (seen + i_last) - column_position(g, cn) < window;
}

// Additive mask value (log2 units applied later) of one (row, key) pair with
// the in-kernel rule; -inf for keys outside the tile's valid range.
__device__ __forceinline__ float inkernel_add(bool chunk, int col, const Live &g, int seen, int C,
                                              int nv, int qpos_abs, int window, int sink) {
  if (chunk) {
    if (col >= C) return -INFINITY;
    return attend(qpos_abs, seen + col, col < nv, window, sink) ? 0.f : kMasked;
  }
  if (col >= g.L) return -INFINITY;
  return attend(qpos_abs, column_position(g, col), true, window, sink) ? 0.f : kMasked;
}

hipError_t launch_attn_valu(const AttnParams &p, int D, int dtype, hipStream_t s);
hipError_t launch_attn_mfma(const AttnParams &p, int D, hipStream_t s);
hipError_t launch_attn_combine(const AttnParams &p, int D, int dtype, hipStream_t s);
hipError_t launch_attn_plan(const AttnParams &p, hipStream_t s);
hipError_t launch_attn_merge_plan(const AttnParams &p, int D, hipStream_t s);

}  // namespace cp
