// cp_common.h -- internal helpers shared by the libcp HIP sources (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cp.h"

namespace cp {

constexpr float kMasked = -1e30f;  // additive value of a masked score
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 bits

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// ------------------------------------------------------------------ RoPE

// Half-split rotation of the pair (lo = x[j], hi = x[j + D/2]) with the position's
// table values: each fp32 x fp32 product is exact in fp64, so the difference (or sum)
// is rounded once, then to fp32 -- independent of FMA contraction, the same bits in
// every kernel that rotates (RoPE launch, attention prologue).
__device__ __forceinline__ float rot_lo(float lo, float hi, float c, float s) {
  const double a = static_cast<double>(lo) * static_cast<double>(c);
  const double b = static_cast<double>(hi) * static_cast<double>(s);
  return static_cast<float>(a - b);
}
__device__ __forceinline__ float rot_hi(float lo, float hi, float c, float s) {
  const double a = static_cast<double>(hi) * static_cast<double>(c);
  const double b = static_cast<double>(lo) * static_cast<double>(s);
  return static_cast<float>(a + b);
}

// ------------------------------------------------------------- cache layout

// Geometry of one sequence's cache after `seen` positions were absorbed.
struct Live {
  int L;    // live rows
  int ns;   // live sink rows (columns [0, ns) are positions [0, ns))
  int lo;   // first live non-sink position; column c >= ns is position lo + (c - ns)
};

__device__ __forceinline__ Live live_geometry(int seen, int cap, int ring, int sink) {
  Live g;
  if (!ring) {
    // every position is live in its own slot; the first `sink` of them are the sink
    // rows (attended regardless of the window), so the tile lists visit them even when
    // the window starts far later.  Column c is still position c (lo == ns).
    g.L = seen;
    g.ns = seen < sink ? seen : sink;
    g.lo = g.ns;
    return g;
  }
  const int R = cap - sink;
  g.ns = seen < sink ? seen : sink;
  g.lo = seen - R > sink ? seen - R : sink;
  g.L = g.ns + (seen > g.lo ? seen - g.lo : 0);
  return g;
}

// Absolute position of past column c (chronological order of live rows).
__device__ __forceinline__ int column_position(const Live &g, int c) {
  return c < g.ns ? c : g.lo + (c - g.ns);
}

// Physical slot of absolute position p.
__device__ __forceinline__ int slot_of(int p, int cap, int ring, int sink) {
  if (!ring || p < cap) return p;
  return sink + (p - sink) % (cap - sink);
}

// In-kernel attend rule: causal, real key, inside the window or a sink row.
__device__ __forceinline__ bool attend(int qpos, int kpos, bool key_real, int window, int sink) {
  if (!key_real || kpos > qpos) return false;
  return window == 0 || qpos - kpos < window || kpos < sink;
}

__device__ __forceinline__ void flag(int32_t *status, int bits) {
  if (status) atomicOr(status, bits);
}

// Reads n_valid[b] (or C when absent), clamped to [0, C].
__device__ __forceinline__ int read_nvalid(const int32_t *n_valid, int b, int C, int32_t *status) {
  if (!n_valid) return C;
  int nv = n_valid[b];
  if (nv < 0 || nv > C) {
    flag(status, CP_DEV_NVALID);
    nv = nv < 0 ? 0 : C;
  }
  return nv;
}

// Where a C-row append lands (device-side checks): rows [0, n) at positions s0..;
// a sequence with a bad seen, or a global sequence that would overflow, is skipped.
struct AppendPlan {
  int s0;     // seen before
  int n;      // rows appended
  bool skip;  // sequence not appended (overflow / bad seen)
};

__device__ __forceinline__ AppendPlan append_plan(const cp_cache &c, const int32_t *n_rows, int b,
                                                  int C, bool report) {
  AppendPlan a;
  // both counters are requested before either is checked (one round trip)
  a.s0 = c.seen[b];
  int n = n_rows ? n_rows[b] : C;
  if (n < 0 || n > C) {
    if (report) flag(c.status, CP_DEV_NVALID);
    n = n < 0 ? 0 : C;
  }
  a.n = n;
  a.skip = false;
  if (a.s0 < 0 || (!c.ring && a.s0 > c.cap)) {
    a.skip = true;
    if (report) flag(c.status, CP_DEV_SEEN);
  } else if (!c.ring && a.s0 + a.n > c.cap) {
    a.skip = true;
    if (report) flag(c.status, CP_DEV_OVERFLOW);
  }
  return a;
}

// --------------------------------------------------------- host launchers

size_t gdn_workspace_bytes(int B, int H, int P, int dk, int dv);
bool gdn_dims_supported(int dk, int dv);
bool gdn_grid_fits(int B, int H, int P);
hipError_t launch_gdn(const float *q, const float *k, const float *v, const float *beta,
                      const float *alpha, float *state, float *out, int B, int H, int P, int dk,
                      int dv, void *ws, hipStream_t s);
hipError_t launch_rope(const void *x, void *y, const float *cos, const float *sin, int B, int Hx,
                       int C, int D, int Bt, int dtype, hipStream_t s);
// Two tensors (Q and K of a chunk) rotated by one launch from the same tables.
hipError_t launch_rope2(const void *x0, void *y0, int H0, const void *x1, void *y1, int H1,
                        const float *cos, const float *sin, int B, int C, int D, int Bt, int dtype,
                        hipStream_t s);
hipError_t launch_rope_qk_append(const cp_cache &c, const void *q, void *q_out, int H,
                                 const void *k, void *k_out, const void *v, const float *cos,
                                 const float *sin, int C, int Bt, const int32_t *n_valid,
                                 hipStream_t s);
// cp_rope_qk_chunk plus the padded-append snapshot, in one launch (H = 0: keys only).
hipError_t launch_rope_qk_snapshot(const cp_cache &c, const void *q, void *q_out, int H,
                                   const void *k, void *k_out, const float *cos, const float *sin,
                                   int C, int Bt, const int32_t *n_valid, void *buf,
                                   hipStream_t s);
// A padded append of all C rows and its rollback, in one launch.
hipError_t launch_append_rollback(const cp_cache &c, const void *k_new, const void *v_new, int C,
                                  const void *buf, hipStream_t s);
hipError_t launch_advance_seen(const cp_cache &c, int C, const int32_t *n_rows, hipStream_t s);
hipError_t launch_kv_append(const cp_cache &c, const void *k_new, const void *v_new, int C,
                            const int32_t *n_rows, hipStream_t s);
hipError_t launch_snapshot(const cp_cache &c, int C, const int32_t *n_valid, void *buf,
                           hipStream_t s);
hipError_t launch_rollback(const cp_cache &c, int C, const void *buf, hipStream_t s);
hipError_t launch_build_mask(float *mask, int64_t ld, const cp_cache &c, const int32_t *n_valid,
                             int H, int C, int window, hipStream_t s);
hipError_t launch_select(const void *x, void *y, const int32_t *idx, int off, int B, int H, int C,
                         int D, int dtype, hipStream_t s);

// Snapshot buffer layout: header of 2*B int32 (seen_before, n_valid) padded to
// 256 bytes, then K rows [B][nKV][C][D], then V rows of the same shape.
inline size_t snapshot_header_bytes(int B) {
  size_t h = sizeof(int32_t) * 2 * static_cast<size_t>(B);
  return (h + 255) & ~static_cast<size_t>(255);
}

// Attention plan chosen on the host.
struct AttnPlan {
  bool mfma;      // bf16 matrix-core kernel, else the vector-ALU kernel
  int splits;     // key splits (1 = direct output)
  int qtiles;     // query tiles per (b, kv head)
  int qpos;       // chunk rows per query tile
  int kt;         // keys per tile
  int small_rows;   // matrix-core kernel: 0, or its 64-row configuration (1; 2 = deep ring),
                    // or the 128-row medium configuration (3)
  int rows;         // matrix-core kernel: query rows per query tile (its split partials
                    // are stored in that tile's fragment order)
  bool planned;     // balanced key splits from a device-side plan (CP_ATTN_BALANCE)
  int plan_grid;    // ... its attention blocks (item entries)
  int plan_slots;   // ... workgroups the GPU holds at once
  int xpad;         // block order of the split groups (AttnParams::xpad)
  int xmerge;       // XCD placement of the merge (AttnParams::xmerge)
};

AttnPlan plan_attention(const cp_cache &c, const cp_attn_args &a, bool for_workspace);
size_t attn_workspace_bytes(const cp_cache &c, const cp_attn_args &a, const AttnPlan &p);
hipError_t launch_attention(const cp_cache &c, const cp_attn_args &a, hipStream_t s);

}  // namespace cp
