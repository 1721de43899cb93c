// kv_cache.hip -- external KV cache: append, padded-append snapshot/rollback.
//
// [SKaiNET] "Change (additive)": K/V extended by the chunk.  [TICO] "Runtime
// behavior" / "Mask/cache layout": the cache lives outside the graph, past
// tokens packed in the first past_len slots, the runtime writes the delta K/V.
// [cactus] "Fix": sliding caches evict chronologically; a padded append
// over-evicts up to pad_count of the oldest window rows, so the rows are
// saved before and reinserted after, leaving the cache byte-identical to an
// unpadded prefill; the region past the live length is dead.
//
// All kernels are HBM-bound row copies: a thread moves one 16-byte chunk
// (4-byte chunk when a row is not a multiple of 16 bytes), consecutive
// threads cover consecutive bytes of a row.  The ring is a modular ring, so
// an append writes O(n) rows rather than compacting the window.  Every copy
// thread must read the pre-append seen, so the bookkeeping update comes after
// all of them: for a small append (up to kOneBlockChunks 16-byte chunks per
// tensor) one 1024-thread workgroup copies and then, past a workgroup barrier,
// updates seen itself -- one launch instead of two; a larger append runs the
// copy kernel over the whole GPU followed by a one-block seen kernel.
#include "cp_common.h"

namespace cp {
namespace {

struct alignas(16) Chunk16 {
  uint32_t w[4];
};

// Which rows of a C-row append survive in the cache (device-side checks).
struct AppendPlan {
  int s0;     // seen before
  int n;      // rows appended
  bool skip;  // sequence not appended (overflow / bad seen)
};

__device__ __forceinline__ AppendPlan append_plan(const cp_cache &c, const int32_t *n_rows, int b,
                                                  int C, bool report) {
  AppendPlan a;
  a.s0 = c.seen[b];
  a.n = read_nvalid(n_rows, b, C, report ? c.status : nullptr);
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

// Copy kernel of an append.  Row r of sequence b goes to position s0 + r; in
// a ring only rows that are still live after the whole append are written
// (an append longer than the window would otherwise write one slot twice).
template <typename W>
__global__ void __launch_bounds__(256) k_append(cp_cache c, const void *__restrict__ kn,
                                                const void *__restrict__ vn, int C,
                                                const int32_t *__restrict__ n_rows, int cpr,
                                                size_t row_bytes) {
  const size_t total = static_cast<size_t>(c.B) * c.nKV * C * cpr;
  for (size_t t = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; t < total;
       t += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int ch = static_cast<int>(t % cpr);
    size_t rest = t / cpr;
    const int r = static_cast<int>(rest % C);
    rest /= C;
    const int g = static_cast<int>(rest % c.nKV);
    const int b = static_cast<int>(rest / c.nKV);
    const AppendPlan a = append_plan(c, n_rows, b, C, g == 0 && r == 0 && ch == 0);
    if (a.skip || r >= a.n) continue;
    const int p = a.s0 + r;
    if (c.ring && p >= c.sink && p < a.s0 + a.n - (c.cap - c.sink)) continue;
    const int sl = slot_of(p, c.cap, c.ring, c.sink);
    const size_t src = (static_cast<size_t>(b) * c.nKV + g) * C + r;
    const size_t dst = (static_cast<size_t>(b) * c.nKV + g) * c.cap + sl;
    const size_t w = row_bytes / sizeof(W);
    static_cast<W *>(c.k)[dst * w + ch] = static_cast<const W *>(kn)[src * w + ch];
    static_cast<W *>(c.v)[dst * w + ch] = static_cast<const W *>(vn)[src * w + ch];
  }
}

// Single-workgroup append: the copy, then (after every thread has read seen) the
// seen update.  Each thread keeps kUnroll rows' chunks in flight at once.
constexpr int kOneBlock = 1024, kUnroll = 8;
constexpr size_t kOneBlockChunks = static_cast<size_t>(kOneBlock) * kUnroll;

template <typename W>
__global__ void __launch_bounds__(kOneBlock) k_append_one(cp_cache c, const void *__restrict__ kn,
                                                         const void *__restrict__ vn, int C,
                                                         const int32_t *__restrict__ n_rows,
                                                         int cpr, size_t row_bytes) {
  const size_t total = static_cast<size_t>(c.B) * c.nKV * C * cpr;
  const size_t w = row_bytes / sizeof(W);
  for (size_t t0 = threadIdx.x; t0 < total; t0 += static_cast<size_t>(kOneBlock) * kUnroll) {
    W kv[kUnroll], vv[kUnroll];
    size_t dst[kUnroll];
    bool go[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t t = t0 + static_cast<size_t>(u) * kOneBlock;
      go[u] = false;
      dst[u] = 0;
      if (t >= total) continue;
      const int ch = static_cast<int>(t % cpr);
      size_t rest = t / cpr;
      const int r = static_cast<int>(rest % C);
      rest /= C;
      const int g = static_cast<int>(rest % c.nKV);
      const int b = static_cast<int>(rest / c.nKV);
      const AppendPlan a = append_plan(c, n_rows, b, C, g == 0 && r == 0 && ch == 0);
      if (a.skip || r >= a.n) continue;
      const int p = a.s0 + r;
      if (c.ring && p >= c.sink && p < a.s0 + a.n - (c.cap - c.sink)) continue;
      const int sl = slot_of(p, c.cap, c.ring, c.sink);
      const size_t src = ((static_cast<size_t>(b) * c.nKV + g) * C + r) * w + ch;
      dst[u] = ((static_cast<size_t>(b) * c.nKV + g) * c.cap + sl) * w + ch;
      kv[u] = static_cast<const W *>(kn)[src];
      vv[u] = static_cast<const W *>(vn)[src];
      go[u] = true;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (go[u]) {
        static_cast<W *>(c.k)[dst[u]] = kv[u];
        static_cast<W *>(c.v)[dst[u]] = vv[u];
      }
  }
  __syncthreads();  // every read of seen above happens before it changes
  for (int b = threadIdx.x; b < c.B; b += kOneBlock) {
    const AppendPlan a = append_plan(c, n_rows, b, C, false);
    if (!a.skip) c.seen[b] = a.s0 + a.n;
  }
}

__global__ void k_append_seen(cp_cache c, const int32_t *__restrict__ n_rows, int C) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= c.B) return;
  const AppendPlan a = append_plan(c, n_rows, b, C, false);
  if (!a.skip) c.seen[b] = a.s0 + a.n;
}

// Over-evicted range of a padded append: [lo, hi), a subset of the rows live
// before the append when cap > C + sink (checked on the host).
__device__ __forceinline__ void overevicted(const cp_cache &c, int s0, int nv, int C, int *lo,
                                            int *hi) {
  if (!c.ring) {
    *lo = *hi = 0;
    return;
  }
  const int R = c.cap - c.sink;
  const int a = s0 + nv - R, e = s0 + C - R;
  *lo = a > c.sink ? a : c.sink;
  *hi = e > c.sink ? e : c.sink;
  if (*hi < *lo) *hi = *lo;
}

template <typename W>
__global__ void __launch_bounds__(256) k_snapshot(cp_cache c, int C, const int32_t *__restrict__ n_valid,
                                                  unsigned char *__restrict__ buf, size_t hdr,
                                                  int cpr, size_t row_bytes) {
  int32_t *h = reinterpret_cast<int32_t *>(buf);
  const size_t half = static_cast<size_t>(c.B) * c.nKV * C * row_bytes;
  W *sk = reinterpret_cast<W *>(buf + hdr);
  W *sv = reinterpret_cast<W *>(buf + hdr + half);
  const size_t w = row_bytes / sizeof(W);
  const size_t gid = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  if (gid < static_cast<size_t>(c.B)) {
    const int b = static_cast<int>(gid);
    const int s0 = c.seen[b];
    h[b] = s0;
    h[c.B + b] = read_nvalid(n_valid, b, C, c.status);
    if (s0 < 0) flag(c.status, CP_DEV_SEEN);
    if (!c.ring && s0 + C > c.cap) flag(c.status, CP_DEV_OVERFLOW);
  }
  const size_t total = static_cast<size_t>(c.B) * c.nKV * C * cpr;
  for (size_t t = gid; t < total; t += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int ch = static_cast<int>(t % cpr);
    size_t rest = t / cpr;
    const int r = static_cast<int>(rest % C);
    rest /= C;
    const int g = static_cast<int>(rest % c.nKV);
    const int b = static_cast<int>(rest / c.nKV);
    const int s0 = c.seen[b];
    const int nv = read_nvalid(n_valid, b, C, nullptr);
    if (s0 < 0) continue;
    int lo, hi;
    overevicted(c, s0, nv, C, &lo, &hi);
    if (r >= hi - lo) continue;
    const int sl = slot_of(lo + r, c.cap, c.ring, c.sink);
    const size_t src = (static_cast<size_t>(b) * c.nKV + g) * c.cap + sl;
    const size_t dst = (static_cast<size_t>(b) * c.nKV + g) * C + r;
    sk[dst * w + ch] = static_cast<const W *>(c.k)[src * w + ch];
    sv[dst * w + ch] = static_cast<const W *>(c.v)[src * w + ch];
  }
}

template <typename W>
__global__ void __launch_bounds__(256) k_restore(cp_cache c, int C, const unsigned char *__restrict__ buf,
                                                 size_t hdr, int cpr, size_t row_bytes) {
  const int32_t *h = reinterpret_cast<const int32_t *>(buf);
  const size_t half = static_cast<size_t>(c.B) * c.nKV * C * row_bytes;
  const W *sk = reinterpret_cast<const W *>(buf + hdr);
  const W *sv = reinterpret_cast<const W *>(buf + hdr + half);
  const size_t w = row_bytes / sizeof(W);
  const size_t total = static_cast<size_t>(c.B) * c.nKV * C * cpr;
  for (size_t t = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x; t < total;
       t += static_cast<size_t>(gridDim.x) * blockDim.x) {
    const int ch = static_cast<int>(t % cpr);
    size_t rest = t / cpr;
    const int r = static_cast<int>(rest % C);
    rest /= C;
    const int g = static_cast<int>(rest % c.nKV);
    const int b = static_cast<int>(rest / c.nKV);
    const int s0 = h[b], nv = h[c.B + b];
    if (s0 < 0 || c.seen[b] != s0 + C) continue;  // flagged by k_rollback_seen
    int lo, hi;
    overevicted(c, s0, nv, C, &lo, &hi);
    if (r >= hi - lo) continue;
    const int sl = slot_of(lo + r, c.cap, c.ring, c.sink);
    const size_t dst = (static_cast<size_t>(b) * c.nKV + g) * c.cap + sl;
    const size_t src = (static_cast<size_t>(b) * c.nKV + g) * C + r;
    static_cast<W *>(c.k)[dst * w + ch] = sk[src * w + ch];
    static_cast<W *>(c.v)[dst * w + ch] = sv[src * w + ch];
  }
}

// Single-workgroup rollback: restore the saved rows, then (after every thread has
// compared seen) set seen.
template <typename W>
__global__ void __launch_bounds__(kOneBlock) k_restore_one(cp_cache c, int C,
                                                          const unsigned char *__restrict__ buf,
                                                          size_t hdr, int cpr, size_t row_bytes) {
  const int32_t *h = reinterpret_cast<const int32_t *>(buf);
  const size_t half = static_cast<size_t>(c.B) * c.nKV * C * row_bytes;
  const W *sk = reinterpret_cast<const W *>(buf + hdr);
  const W *sv = reinterpret_cast<const W *>(buf + hdr + half);
  const size_t w = row_bytes / sizeof(W);
  const size_t total = static_cast<size_t>(c.B) * c.nKV * C * cpr;
  for (size_t t0 = threadIdx.x; t0 < total; t0 += static_cast<size_t>(kOneBlock) * kUnroll) {
    W kv[kUnroll], vv[kUnroll];
    size_t dst[kUnroll];
    bool go[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const size_t t = t0 + static_cast<size_t>(u) * kOneBlock;
      go[u] = false;
      dst[u] = 0;
      if (t >= total) continue;
      const int ch = static_cast<int>(t % cpr);
      size_t rest = t / cpr;
      const int r = static_cast<int>(rest % C);
      rest /= C;
      const int g = static_cast<int>(rest % c.nKV);
      const int b = static_cast<int>(rest / c.nKV);
      const int s0 = h[b], nv = h[c.B + b];
      if (s0 < 0 || c.seen[b] != s0 + C) continue;
      int lo, hi;
      overevicted(c, s0, nv, C, &lo, &hi);
      if (r >= hi - lo) continue;
      const int sl = slot_of(lo + r, c.cap, c.ring, c.sink);
      dst[u] = ((static_cast<size_t>(b) * c.nKV + g) * c.cap + sl) * w + ch;
      const size_t src = ((static_cast<size_t>(b) * c.nKV + g) * C + r) * w + ch;
      kv[u] = sk[src];
      vv[u] = sv[src];
      go[u] = true;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (go[u]) {
        static_cast<W *>(c.k)[dst[u]] = kv[u];
        static_cast<W *>(c.v)[dst[u]] = vv[u];
      }
  }
  __syncthreads();  // every comparison with seen above happens before it changes
  for (int b = threadIdx.x; b < c.B; b += kOneBlock) {
    const int s0 = h[b], nv = h[c.B + b];
    if (s0 < 0 || c.seen[b] != s0 + C) {
      flag(c.status, CP_DEV_ROLLBACK);
      continue;
    }
    c.seen[b] = s0 + nv;
  }
}

__global__ void k_rollback_seen(cp_cache c, int C, const unsigned char *__restrict__ buf) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= c.B) return;
  const int32_t *h = reinterpret_cast<const int32_t *>(buf);
  const int s0 = h[b], nv = h[c.B + b];
  if (s0 < 0 || c.seen[b] != s0 + C) {
    flag(c.status, CP_DEV_ROLLBACK);
    return;
  }
  c.seen[b] = s0 + nv;
}

unsigned grid_for(size_t total) {
  size_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks == 0) blocks = 1;
  return static_cast<unsigned>(blocks);
}

size_t row_bytes_of(const cp_cache &c) {
  return static_cast<size_t>(c.D) * (c.dtype == CP_BF16 ? 2 : 4);
}

}  // namespace

hipError_t launch_kv_append(const cp_cache &c, const void *k_new, const void *v_new, int C,
                            const int32_t *n_rows, hipStream_t s) {
  if (c.B == 0) return hipSuccess;
  const size_t rb = row_bytes_of(c);
  {
    const bool c16 = rb % 16 == 0;
    const int cpr = static_cast<int>(c16 ? rb / 16 : rb / 4);
    if (static_cast<size_t>(c.B) * c.nKV * C * cpr <= kOneBlockChunks) {
      if (c16)
        hipLaunchKernelGGL(k_append_one<Chunk16>, dim3(1), dim3(kOneBlock), 0, s, c, k_new,
                           v_new, C, n_rows, cpr, rb);
      else
        hipLaunchKernelGGL(k_append_one<uint32_t>, dim3(1), dim3(kOneBlock), 0, s, c, k_new,
                           v_new, C, n_rows, cpr, rb);
      return hipGetLastError();
    }
  }
  if (C > 0) {
    if (rb % 16 == 0) {
      const int cpr = static_cast<int>(rb / 16);
      hipLaunchKernelGGL(k_append<Chunk16>, dim3(grid_for((size_t)c.B * c.nKV * C * cpr)),
                         dim3(256), 0, s, c, k_new, v_new, C, n_rows, cpr, rb);
    } else {
      const int cpr = static_cast<int>(rb / 4);
      hipLaunchKernelGGL(k_append<uint32_t>, dim3(grid_for((size_t)c.B * c.nKV * C * cpr)),
                         dim3(256), 0, s, c, k_new, v_new, C, n_rows, cpr, rb);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_append_seen, dim3((c.B + 255) / 256), dim3(256), 0, s, c, n_rows, C);
  return hipGetLastError();
}

hipError_t launch_snapshot(const cp_cache &c, int C, const int32_t *n_valid, void *buf,
                           hipStream_t s) {
  if (c.B == 0) return hipSuccess;
  const size_t rb = row_bytes_of(c);
  const size_t hdr = snapshot_header_bytes(c.B);
  unsigned char *b = static_cast<unsigned char *>(buf);
  // the grid always covers B threads: they write the header, even for C == 0
  if (rb % 16 == 0) {
    const int cpr = static_cast<int>(rb / 16);
    const size_t total = (size_t)c.B * c.nKV * C * cpr;
    hipLaunchKernelGGL(k_snapshot<Chunk16>, dim3(grid_for(total > (size_t)c.B ? total : c.B)),
                       dim3(256), 0, s, c, C, n_valid, b, hdr, cpr, rb);
  } else {
    const int cpr = static_cast<int>(rb / 4);
    const size_t total = (size_t)c.B * c.nKV * C * cpr;
    hipLaunchKernelGGL(k_snapshot<uint32_t>, dim3(grid_for(total > (size_t)c.B ? total : c.B)),
                       dim3(256), 0, s, c, C, n_valid, b, hdr, cpr, rb);
  }
  return hipGetLastError();
}

hipError_t launch_rollback(const cp_cache &c, int C, const void *buf, hipStream_t s) {
  if (c.B == 0) return hipSuccess;
  const size_t rb = row_bytes_of(c);
  const size_t hdr = snapshot_header_bytes(c.B);
  const unsigned char *b = static_cast<const unsigned char *>(buf);
  {
    const bool c16 = rb % 16 == 0;
    const int cpr = static_cast<int>(c16 ? rb / 16 : rb / 4);
    if (static_cast<size_t>(c.B) * c.nKV * C * cpr <= kOneBlockChunks) {
      if (c16)
        hipLaunchKernelGGL(k_restore_one<Chunk16>, dim3(1), dim3(kOneBlock), 0, s, c, C, b, hdr,
                           cpr, rb);
      else
        hipLaunchKernelGGL(k_restore_one<uint32_t>, dim3(1), dim3(kOneBlock), 0, s, c, C, b, hdr,
                           cpr, rb);
      return hipGetLastError();
    }
  }
  if (C > 0) {
    if (rb % 16 == 0) {
      const int cpr = static_cast<int>(rb / 16);
      hipLaunchKernelGGL(k_restore<Chunk16>, dim3(grid_for((size_t)c.B * c.nKV * C * cpr)),
                         dim3(256), 0, s, c, C, b, hdr, cpr, rb);
    } else {
      const int cpr = static_cast<int>(rb / 4);
      hipLaunchKernelGGL(k_restore<uint32_t>, dim3(grid_for((size_t)c.B * c.nKV * C * cpr)),
                         dim3(256), 0, s, c, C, b, hdr, cpr, rb);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_rollback_seen, dim3((c.B + 255) / 256), dim3(256), 0, s, c, C, b);
  return hipGetLastError();
}

}  // namespace cp
