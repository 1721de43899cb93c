// attn_mfma_ops.h -- device helpers of the bf16 matrix-core attention kernels (gfx950):
// operand types, direct-to-LDS loads, LDS operand reads issued as inline asm with
// explicit waits, lane-pair reductions, LDS swizzles and memory-counter waits.
#pragma once

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
// scaled maxima at or below this carry no attended key (masked scores: -1e30 log2 e)
constexpr float kNoKeyFloor = -1e29f;

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
// The constant byte offset OFF rides in the instruction's 16-bit offset field instead
// of costing an address add.
template <int OFF>
__device__ __forceinline__ u32x2 tr_read_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field is 16 bits");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}

// Transpose reads of rows 16t and 16t + 8 (t = T .. NPT-1) of a V tile with D
// columns, as consecutive operand pairs.
template <int D, int T, int NPT>
__device__ __forceinline__ void tr_read_rows(uint32_t va, u32x2 *w) {
  if constexpr (T < NPT) {
    w[2 * T] = tr_read_at<2 * (16 * T * D)>(va);
    w[2 * T + 1] = tr_read_at<2 * ((16 * T + 8) * D)>(va);
    tr_read_rows<D, T + 1, NPT>(va, w);
  }
}

// K operand read: 16 bytes at a constant byte offset OFF from addr, issued as inline
// asm for the same reason as the transpose reads (the compiler would otherwise wait for
// every LDS read before the MFMA right after it, exposing the full LDS latency on each
// k-step); its results are valid only after k_wait() has been passed through them.
template <int OFF>
__device__ __forceinline__ u32x4 k_read_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field is 16 bits");
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// the K fragments of key blocks KB .. NKB-1 (32 rows of D bf16 apart) at one k-step
template <int D, int KB, int NKB>
__device__ __forceinline__ void k_read_blocks(uint32_t addr, u32x4 *f) {
  if constexpr (KB < NKB) {
    f[KB] = k_read_at<2 * 32 * KB * D>(addr);
    k_read_blocks<D, KB + 1, NKB>(addr, f);
  }
}
// s_waitcnt lgkmcnt(N) that marks the NKB fragments f[] as written by it; the N LDS
// reads issued after them may stay in flight
template <int N, int NKB>
__device__ __forceinline__ void k_wait(u32x4 *f) {
  static_assert(N >= 0 && N < 16 && (NKB == 1 || NKB == 2), "lgkmcnt range");
  if constexpr (NKB == 1)
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(f[0]) : "i"(N));
  else
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(f[0]), "+v"(f[1]) : "i"(N));
}

// Lanes l and l ^ 32 hold the two halves of one query row's keys: combine them with
// one v_permlane32_swap (no LDS round trip).  Both lanes get the same value.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return fmaxf(__builtin_bit_cast(float, static_cast<unsigned>(r[0])),
               __builtin_bit_cast(float, static_cast<unsigned>(r[1])));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, v),
                                                  __builtin_bit_cast(unsigned, v), false, false);
  return __builtin_bit_cast(float, static_cast<unsigned>(r[0])) +
         __builtin_bit_cast(float, static_cast<unsigned>(r[1]));
}

// s_waitcnt lgkmcnt(N) that also marks the CNT transpose-read results w[] as written
// by it, so no use of them is scheduled before the wait.  LDS operations complete in
// order: the N reads issued after w[] may stay in flight.
template <int N, int CNT>
__device__ __forceinline__ void lds_wait_keep(u32x2 *w) {
  static_assert(CNT == 4 || CNT == 8, "transpose reads per dim block");
  static_assert(N == 0 || N == CNT, "reads left in flight");
  if constexpr (CNT == 8) {
    if constexpr (N == 0)
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]),
                     "+v"(w[6]), "+v"(w[7]));
    else
      asm volatile("s_waitcnt lgkmcnt(8)"
                   : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]),
                     "+v"(w[6]), "+v"(w[7]));
  } else {
    if constexpr (N == 0)
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
    else
      asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
  }
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

// Swizzle of the 16-byte chunks of LDS row r.  K: the 16 rows one ds_read_b128 pass
// reads (one chunk each) land on distinct banks.  V: a 32-lane pass of the transpose
// read touches 4 rows x 8 chunks; with rows of 256 bytes or more every row starts at
// bank 0, so the 4 rows' chunk groups are spread by 4 chunks (D = 64 rows alternate
// bank halves, so 2 chunks suffice there).
template <int D>
__device__ __forceinline__ int kswz(int r) {
  return D == 64 ? ((r >> 1) & 7) : (r & 15);
}
template <int D>
__device__ __forceinline__ int vswz(int r) {
  return D == 64 ? (r & 3) << 1 : (r & 3) << 2;
}

// One wave-wide 4-byte direct-to-LDS load (mask blocks: no alignment beyond 4 bytes).
__device__ __forceinline__ void dma4(const float *src, float *lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(src, (lds_void *)lds_base, 4, 0, 0);
#else
  (void)src;
  (void)lds_base;
#endif
}

// Swizzle of the 16-byte chunks of row r of a ROWS x 32 fp32 mask block (rows of
// 128 bytes: rows r and r + 1 share a 256-byte bank line).
__device__ __forceinline__ int mswz(int r) { return (r >> 1) & 7; }

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

}  // namespace
}  // namespace cp
