// rope.hip -- rotary embedding of a chunk from per-position cos/sin tables.
//
// [SKaiNET] "Change (additive)": RoPE from per-position [C, headDim] cos/sin
// tables, one pair per RoPE base; [TICO] "Runtime behavior": (cos_t, sin_t)
// for the absolute position.  Half-split pairing (j with j + D/2).
//
// HBM-bound elementwise kernel: each thread rotates VEC consecutive pairs of
// one row, reading the lower and upper halves with vector loads.  The math
// runs in fp64: an fp32 x fp32 product is exact in fp64, so the difference
// (or sum) of the two products is rounded exactly once, independent of FMA
// contraction; the result is then rounded to fp32 and, for bf16 storage, to
// bf16 by round-to-nearest-even.  The cache rows built from it are therefore
// reproducible bit for bit.
#include "cp_common.h"

namespace cp {
namespace {

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float load(const float *p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float *p, size_t i, float v) { p[i] = v; }
};
template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t *p, size_t i) {
    return bf16_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(uint16_t *p, size_t i, float v) {
    p[i] = f32_to_bf16_rne(v);
  }
};

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

// One thread: VEC consecutive pairs (j .. j+VEC-1, j+h2 .. j+h2+VEC-1) of a row.
// x and y may alias: every element is read and written by the same thread.
template <typename T, int VEC>
__global__ void __launch_bounds__(256) k_rope(const T *x, T *y,
                                              const float *__restrict__ cosb,
                                              const float *__restrict__ sinb, int B, int Hx, int C,
                                              int D, int Bt) {
  const int h2 = D / 2;
  const int per_row = h2 / VEC;
  const size_t rows = static_cast<size_t>(B) * Hx * C;
  const size_t total = rows * per_row;
  for (size_t t = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; t < total;
       t += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const size_t row = t / per_row;
    const int j0 = static_cast<int>(t % per_row) * VEC;
    const int i = static_cast<int>(row % C);
    const int b = static_cast<int>(row / (static_cast<size_t>(Hx) * C));
    const size_t xo = row * D;
    const size_t to = (static_cast<size_t>(Bt == 1 ? 0 : b) * C + i) * D;
    float lo[VEC], hi[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      lo[e] = Elem<T>::load(x, xo + j0 + e);
      hi[e] = Elem<T>::load(x, xo + j0 + h2 + e);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int j = j0 + e;
      const float ylo = rot_lo(lo[e], hi[e], cosb[to + j], sinb[to + j]);
      const float yhi = rot_hi(lo[e], hi[e], cosb[to + j + h2], sinb[to + j + h2]);
      Elem<T>::store(y, xo + j, ylo);
      Elem<T>::store(y, xo + j + h2, yhi);
    }
  }
}

template <typename T>
hipError_t launch_t(const void *x, void *y, const float *cos, const float *sin, int B, int Hx,
                    int C, int D, int Bt, hipStream_t s) {
  const int h2 = D / 2;
  const size_t rows = static_cast<size_t>(B) * Hx * C;
  if (rows == 0) return hipSuccess;
  auto grid_for = [&](int vec) {
    size_t total = rows * (h2 / vec);
    size_t blocks = (total + 255) / 256;
    if (blocks > 65535 * 4) blocks = 65535 * 4;
    return static_cast<unsigned>(blocks);
  };
  const T *xi = static_cast<const T *>(x);
  T *yo = static_cast<T *>(y);
  if (h2 % 8 == 0) {
    hipLaunchKernelGGL((k_rope<T, 8>), dim3(grid_for(8)), dim3(256), 0, s, xi, yo, cos, sin, B,
                       Hx, C, D, Bt);
  } else if (h2 % 4 == 0) {
    hipLaunchKernelGGL((k_rope<T, 4>), dim3(grid_for(4)), dim3(256), 0, s, xi, yo, cos, sin, B,
                       Hx, C, D, Bt);
  } else {
    hipLaunchKernelGGL((k_rope<T, 1>), dim3(grid_for(1)), dim3(256), 0, s, xi, yo, cos, sin, B,
                       Hx, C, D, Bt);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const void *x, void *y, const float *cos, const float *sin, int B, int Hx,
                       int C, int D, int Bt, int dtype, hipStream_t s) {
  if (dtype == CP_BF16) return launch_t<uint16_t>(x, y, cos, sin, B, Hx, C, D, Bt, s);
  return launch_t<float>(x, y, cos, sin, B, Hx, C, D, Bt, s);
}

}  // namespace cp
