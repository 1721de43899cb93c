// mask_select.hip -- explicit mask materialisation and last-real-row selection.
//
// [SKaiNET] "Change (additive)": a caller-supplied additive mask per head
// [1, nHeads, C, past+C] (0 attends, -1e30 masks) carrying the causal band,
// the zero padding and the sliding window; the LM head runs on the one-hot
// selected row ("Validation": row 51, the last real row of a 52-token chunk).
#include "cp_common.h"

namespace cp {
namespace {

// mask[b, h, i, col]: col < L -> past column (chronological), col < L + C ->
// chunk row col - L, else masked.  One thread per element, grid-stride.
__global__ void __launch_bounds__(256) k_build_mask(float *__restrict__ mask, int64_t ld,
                                                    cp_cache c, const int32_t *__restrict__ n_valid,
                                                    int H, int C, int window) {
  const size_t total = static_cast<size_t>(c.B) * H * C * ld;
  for (size_t t = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; t < total;
       t += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int64_t col = static_cast<int64_t>(t % ld);
    const size_t row = t / ld;
    const int i = static_cast<int>(row % C);
    const int b = static_cast<int>(row / (static_cast<size_t>(H) * C));
    const int seen = c.seen[b];
    const bool lead = col == 0 && row % (static_cast<size_t>(H) * C) == 0;
    const int nv = read_nvalid(n_valid, b, C, lead ? c.status : nullptr);
    float val = kMasked;
    if (seen >= 0 && (c.ring || seen <= c.cap)) {
      const Live g = live_geometry(seen, c.cap, c.ring, c.sink);
      const int qpos = seen + i;
      if (col < g.L) {
        val = attend(qpos, column_position(g, static_cast<int>(col)), true, window, c.sink) ? 0.f
                                                                                            : kMasked;
      } else if (col < static_cast<int64_t>(g.L) + C) {
        const int j = static_cast<int>(col - g.L);
        val = attend(qpos, seen + j, j < nv, window, c.sink) ? 0.f : kMasked;
      }
      if (lead && static_cast<int64_t>(g.L) + C > ld) flag(c.status, CP_DEV_MASK_LD);
    } else if (lead) {
      flag(c.status, CP_DEV_SEEN);
    }
    mask[t] = val;
  }
}

// y[b, h, :] = x[b, h, idx[b] + off, :]; zeros outside [0, C).  W is the
// copy word (16 bytes when the row allows it).
template <typename W>
__global__ void __launch_bounds__(256) k_select(const W *__restrict__ x, W *__restrict__ y,
                                                const int32_t *__restrict__ idx, int off, int B,
                                                int H, int C, int wpr) {
  const size_t total = static_cast<size_t>(B) * H * wpr;
  for (size_t t = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; t < total;
       t += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int w = static_cast<int>(t % wpr);
    const size_t bh = t / wpr;
    const int b = static_cast<int>(bh / H);
    const long r = static_cast<long>(idx[b]) + off;
    W v{};
    if (r >= 0 && r < C) v = x[(bh * C + static_cast<size_t>(r)) * wpr + w];
    y[t] = v;
  }
}

struct alignas(16) W16 {
  uint32_t w[4];
};

unsigned grid_for(size_t total) {
  size_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  return static_cast<unsigned>(blocks);
}

}  // namespace

hipError_t launch_build_mask(float *mask, int64_t ld, const cp_cache &c, const int32_t *n_valid,
                             int H, int C, int window, hipStream_t s) {
  const size_t total = static_cast<size_t>(c.B) * H * C * ld;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_build_mask, dim3(grid_for(total)), dim3(256), 0, s, mask, ld, c, n_valid, H,
                     C, window);
  return hipGetLastError();
}

hipError_t launch_select(const void *x, void *y, const int32_t *idx, int off, int B, int H, int C,
                         int D, int dtype, hipStream_t s) {
  const size_t rb = static_cast<size_t>(D) * (dtype == CP_BF16 ? 2 : 4);
  if (static_cast<size_t>(B) * H == 0) return hipSuccess;
  if (rb % 16 == 0) {
    const int wpr = static_cast<int>(rb / 16);
    hipLaunchKernelGGL(k_select<W16>, dim3(grid_for((size_t)B * H * wpr)), dim3(256), 0, s,
                       static_cast<const W16 *>(x), static_cast<W16 *>(y), idx, off, B, H, C, wpr);
  } else {
    const int wpr = static_cast<int>(rb / 2);
    hipLaunchKernelGGL(k_select<uint16_t>, dim3(grid_for((size_t)B * H * wpr)), dim3(256), 0, s,
                       static_cast<const uint16_t *>(x), static_cast<uint16_t *>(y), idx, off, B,
                       H, C, wpr);
  }
  return hipGetLastError();
}

}  // namespace cp
