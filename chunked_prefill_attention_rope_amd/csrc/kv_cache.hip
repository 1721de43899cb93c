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
// all of them: for a tiny append (up to kOneBlockChunks 16-byte chunks per
// tensor) one 1024-thread workgroup copies and then, past a workgroup barrier,
// updates seen itself -- one launch instead of two; a larger append runs the
// copy kernel over the whole GPU followed by a one-block seen kernel.
#include "cp_common.h"

namespace cp {
namespace {

struct alignas(16) Chunk16 {
  uint32_t w[4];
};

// Copy kernel of an append.  Row r of sequence b goes to position s0 + r; in
// a ring only rows that are still live after the whole append are written
// (an append longer than the window would otherwise write one slot twice).
// I: index type, 32-bit when the chunk count allows (integer division is a software
// sequence, a 64-bit one several times longer).
template <typename W, typename I>
__global__ void __launch_bounds__(256) k_append(cp_cache c, const void *__restrict__ kn,
                                                const void *__restrict__ vn, int C,
                                                const int32_t *__restrict__ n_rows, int cpr,
                                                size_t row_bytes) {
  const I total = static_cast<I>(c.B) * c.nKV * C * cpr;
  for (I t = blockIdx.x * static_cast<I>(blockDim.x) + threadIdx.x; t < total;
       t += static_cast<I>(gridDim.x) * blockDim.x) {
    const I row = t / static_cast<I>(cpr);
    const int ch = static_cast<int>(t - row * cpr);
    const I bg = row / static_cast<I>(C);
    const int r = static_cast<int>(row - bg * C);
    const int g = static_cast<int>(bg % static_cast<I>(c.nKV));
    const int b = static_cast<int>(bg / static_cast<I>(c.nKV));
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
// seen update.  The per-sequence plans are formed once into LDS; a thread owns one
// 16-byte column (cpr divides the block) of rows row0, row0 + rstep, ... and keeps
// kUnroll of them in flight at once.
constexpr int kOneBlock = 1024, kUnroll = 8, kOneBlockMaxB = 1024;
// One CU moves only ~45 GB/s, so one workgroup pays off (it saves a launch, ~1.5 us)
// only for copies of up to 16 KB per tensor.
constexpr size_t kOneBlockChunks = 1024;

// The single-workgroup kernels apply: small copy, cpr a power of two, B plans fit LDS.
bool one_block_ok(const cp_cache &c, int C, int cpr) {
  return static_cast<size_t>(c.B) * c.nKV * C * cpr <= kOneBlockChunks && c.B <= kOneBlockMaxB &&
         (cpr & (cpr - 1)) == 0 && cpr <= kOneBlock;
}

template <typename W>
__global__ void __launch_bounds__(kOneBlock) k_append_one(cp_cache c, const void *__restrict__ kn,
                                                         const void *__restrict__ vn, int C,
                                                         const int32_t *__restrict__ n_rows,
                                                         int cpr, size_t row_bytes) {
  __shared__ int plan_s0[kOneBlockMaxB], plan_n[kOneBlockMaxB];  // n < 0: skipped
  for (int b = threadIdx.x; b < c.B; b += kOneBlock) {
    const AppendPlan a = append_plan(c, n_rows, b, C, true);
    plan_s0[b] = a.s0;
    plan_n[b] = a.skip ? -1 : a.n;
  }
  __syncthreads();  // also: every read of seen happens before the update below
  const int ch = threadIdx.x & (cpr - 1);
  const int rstep = kOneBlock / cpr;
  const int rows = c.B * c.nKV * C;
  const size_t w = row_bytes / sizeof(W);
  const W *K = static_cast<const W *>(kn);
  const W *V = static_cast<const W *>(vn);
  for (int row0 = threadIdx.x / cpr; row0 < rows; row0 += rstep * kUnroll) {
    W kv[kUnroll], vv[kUnroll];
    size_t dst[kUnroll];
    bool go[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int row = row0 + u * rstep;
      go[u] = false;
      dst[u] = 0;
      if (row >= rows) continue;
      const int bg = row / C, r = row - bg * C;
      const int b = bg / c.nKV;
      const int s0 = plan_s0[b], n = plan_n[b];
      if (r >= n) continue;
      const int p = s0 + r;
      if (c.ring && p >= c.sink && p < s0 + n - (c.cap - c.sink)) continue;
      const int sl = slot_of(p, c.cap, c.ring, c.sink);
      dst[u] = (static_cast<size_t>(bg) * c.cap + sl) * w + ch;
      const size_t src = static_cast<size_t>(row) * w + ch;
      kv[u] = K[src];
      vv[u] = V[src];
      go[u] = true;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (go[u]) {
        static_cast<W *>(c.k)[dst[u]] = kv[u];
        static_cast<W *>(c.v)[dst[u]] = vv[u];
      }
  }
  for (int b = threadIdx.x; b < c.B; b += kOneBlock)
    if (plan_n[b] >= 0) c.seen[b] = plan_s0[b] + plan_n[b];
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

template <typename W, typename I>
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
  const I total = static_cast<I>(c.B) * c.nKV * C * cpr;
  for (I t = static_cast<I>(gid); t < total; t += static_cast<I>(gridDim.x) * blockDim.x) {
    const I row = t / static_cast<I>(cpr);
    const int ch = static_cast<int>(t - row * cpr);
    const I bg = row / static_cast<I>(C);
    const int r = static_cast<int>(row - bg * C);
    const int g = static_cast<int>(bg % static_cast<I>(c.nKV));
    const int b = static_cast<int>(bg / static_cast<I>(c.nKV));
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

template <typename W, typename I>
__global__ void __launch_bounds__(256) k_restore(cp_cache c, int C, const unsigned char *__restrict__ buf,
                                                 size_t hdr, int cpr, size_t row_bytes) {
  const int32_t *h = reinterpret_cast<const int32_t *>(buf);
  const size_t half = static_cast<size_t>(c.B) * c.nKV * C * row_bytes;
  const W *sk = reinterpret_cast<const W *>(buf + hdr);
  const W *sv = reinterpret_cast<const W *>(buf + hdr + half);
  const size_t w = row_bytes / sizeof(W);
  const I total = static_cast<I>(c.B) * c.nKV * C * cpr;
  for (I t = blockIdx.x * static_cast<I>(blockDim.x) + threadIdx.x; t < total;
       t += static_cast<I>(gridDim.x) * blockDim.x) {
    const I row = t / static_cast<I>(cpr);
    const int ch = static_cast<int>(t - row * cpr);
    const I bg = row / static_cast<I>(C);
    const int r = static_cast<int>(row - bg * C);
    const int g = static_cast<int>(bg % static_cast<I>(c.nKV));
    const int b = static_cast<int>(bg / static_cast<I>(c.nKV));
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

// Single-workgroup rollback: restore the saved rows, then set seen.  As the append:
// per-sequence state formed once into LDS (every comparison with seen happens
// before the barrier), one 16-byte column of rows per thread.
template <typename W>
__global__ void __launch_bounds__(kOneBlock) k_restore_one(cp_cache c, int C,
                                                          const unsigned char *__restrict__ buf,
                                                          size_t hdr, int cpr, size_t row_bytes) {
  __shared__ int st_lo[kOneBlockMaxB], st_cnt[kOneBlockMaxB];  // cnt < 0: sequence left alone
  const int32_t *h = reinterpret_cast<const int32_t *>(buf);
  for (int b = threadIdx.x; b < c.B; b += kOneBlock) {
    const int s0 = h[b], nv = h[c.B + b];
    int lo = 0, hi = 0;
    if (s0 >= 0 && c.seen[b] == s0 + C) {
      overevicted(c, s0, nv, C, &lo, &hi);
      st_cnt[b] = hi - lo;
    } else {
      st_cnt[b] = -1;
    }
    st_lo[b] = lo;
  }
  __syncthreads();
  const size_t half = static_cast<size_t>(c.B) * c.nKV * C * row_bytes;
  const W *sk = reinterpret_cast<const W *>(buf + hdr);
  const W *sv = reinterpret_cast<const W *>(buf + hdr + half);
  const size_t w = row_bytes / sizeof(W);
  const int ch = threadIdx.x & (cpr - 1);
  const int rstep = kOneBlock / cpr;
  const int rows = c.B * c.nKV * C;
  for (int row0 = threadIdx.x / cpr; row0 < rows; row0 += rstep * kUnroll) {
    W kv[kUnroll], vv[kUnroll];
    size_t dst[kUnroll];
    bool go[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int row = row0 + u * rstep;
      go[u] = false;
      dst[u] = 0;
      if (row >= rows) continue;
      const int bg = row / C, r = row - bg * C;
      const int b = bg / c.nKV;
      if (r >= st_cnt[b]) continue;
      const int sl = slot_of(st_lo[b] + r, c.cap, c.ring, c.sink);
      dst[u] = (static_cast<size_t>(bg) * c.cap + sl) * w + ch;
      const size_t src = static_cast<size_t>(row) * w + ch;
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
  for (int b = threadIdx.x; b < c.B; b += kOneBlock) {
    if (st_cnt[b] < 0) {
      flag(c.status, CP_DEV_ROLLBACK);
      continue;
    }
    c.seen[b] = h[b] + h[c.B + b];
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

// A padded append of all C rows followed by its rollback, in one launch and with the
// same bytes in every slot (live or dead) and the same seen and status bits as the two
// calls (cp_kv_append with n_rows NULL, then cp_kv_rollback_padded_append), on a cache
// left unchanged since the snapshot:
//  - row r < nv: the chunk row, at slot(s0 + r), as the append writes it;
//  - pad row r >= nv at position p = s0 + r: in a ring with p >= cap its slot held the
//    over-evicted position p - R, which the rollback writes back from the snapshot;
//    otherwise (a global cache, or p < cap) it is the chunk's pad row, which the append
//    writes and the rollback leaves in the dead region.
// The pre-append seen comes from the snapshot header (s0), never from cache.seen, so
// one thread per sequence can check that cache.seen still equals s0 and advance it to
// s0 + nv in this launch without racing the copies.  A sequence the append would skip
// (bad seen, global overflow) is skipped with the append's and the rollback's status
// bits.  If cache.seen moved since the snapshot the rows are still written for s0, but
// seen is left alone and CP_DEV_ROLLBACK is set (the two separate calls would append at
// the moved seen instead: the cache state is then the caller's error either way).
__device__ __forceinline__ bool padded_skip(const cp_cache &c, int s0, int C) {
  return s0 < 0 || (!c.ring && (s0 > c.cap || s0 + C > c.cap));
}

template <typename W, typename I>
__global__ void __launch_bounds__(256) k_append_rollback(cp_cache c, const void *__restrict__ kn,
                                                         const void *__restrict__ vn, int C,
                                                         const unsigned char *__restrict__ buf,
                                                         size_t hdr, int cpr, size_t row_bytes) {
  const int32_t *h = reinterpret_cast<const int32_t *>(buf);
  const size_t half = static_cast<size_t>(c.B) * c.nKV * C * row_bytes;
  const W *sk = reinterpret_cast<const W *>(buf + hdr);
  const W *sv = reinterpret_cast<const W *>(buf + hdr + half);
  const size_t w = row_bytes / sizeof(W);
  const size_t gid = blockIdx.x * static_cast<size_t>(blockDim.x) + threadIdx.x;
  if (gid < static_cast<size_t>(c.B)) {  // bookkeeping of sequence gid
    const int b = static_cast<int>(gid);
    const int s0 = h[b], nv = h[c.B + b];
    if (s0 < 0 || (!c.ring && s0 > c.cap)) {
      flag(c.status, CP_DEV_SEEN | CP_DEV_ROLLBACK);
    } else if (!c.ring && s0 + C > c.cap) {
      flag(c.status, CP_DEV_OVERFLOW | CP_DEV_ROLLBACK);
    } else if (c.seen[b] != s0) {
      flag(c.status, CP_DEV_ROLLBACK);
    } else {
      c.seen[b] = s0 + nv;
    }
  }
  const I total = static_cast<I>(c.B) * c.nKV * C * cpr;
  for (I t = static_cast<I>(gid); t < total; t += static_cast<I>(gridDim.x) * blockDim.x) {
    const I row = t / static_cast<I>(cpr);
    const int ch = static_cast<int>(t - row * cpr);
    const I bg = row / static_cast<I>(C);
    const int r = static_cast<int>(row - bg * C);
    const int b = static_cast<int>(bg / static_cast<I>(c.nKV));
    const int s0 = h[b], nv = h[c.B + b];
    if (padded_skip(c, s0, C)) continue;
    const int p = s0 + r;
    // an append longer than the window writes only the rows still live after it (the
    // window guard of the snapshot makes this empty, kept for equality with the append)
    if (c.ring && p >= c.sink && p < s0 + C - (c.cap - c.sink)) continue;
    const int sl = slot_of(p, c.cap, c.ring, c.sink);
    const size_t dst = (static_cast<size_t>(bg) * c.cap + sl) * w + ch;
    if (r >= nv && c.ring && p >= c.cap) {
      int lo, hi;
      overevicted(c, s0, nv, C, &lo, &hi);
      const int q = p - (c.cap - c.sink);  // the position the pad row displaced
      if (q >= lo && q < hi) {
        const size_t src = ((static_cast<size_t>(bg) * C) + (q - lo)) * w + ch;
        static_cast<W *>(c.k)[dst] = sk[src];
        static_cast<W *>(c.v)[dst] = sv[src];
        continue;
      }
    }
    const size_t src = static_cast<size_t>(row) * w + ch;
    static_cast<W *>(c.k)[dst] = static_cast<const W *>(kn)[src];
    static_cast<W *>(c.v)[dst] = static_cast<const W *>(vn)[src];
  }
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

// 32-bit indices when every chunk index of a launch over B * nKV * C rows fits.
static bool fits32(const cp_cache &c, int C, size_t row_bytes) {
  return static_cast<size_t>(c.B) * c.nKV * C * (row_bytes / 4) < (size_t(1) << 31);
}

#define CP_LAUNCH_IDX(K, W, grid, ...)                                               \
  do {                                                                              \
    if (f32)                                                                        \
      hipLaunchKernelGGL((K<W, uint32_t>), dim3(grid), dim3(256), 0, s, __VA_ARGS__); \
    else                                                                            \
      hipLaunchKernelGGL((K<W, size_t>), dim3(grid), dim3(256), 0, s, __VA_ARGS__);   \
  } while (0)

hipError_t launch_advance_seen(const cp_cache &c, int C, const int32_t *n_rows, hipStream_t s) {
  if (c.B == 0) return hipSuccess;
  hipLaunchKernelGGL(k_append_seen, dim3((c.B + 255) / 256), dim3(256), 0, s, c, n_rows, C);
  return hipGetLastError();
}

hipError_t launch_kv_append(const cp_cache &c, const void *k_new, const void *v_new, int C,
                            const int32_t *n_rows, hipStream_t s) {
  if (c.B == 0) return hipSuccess;
  const size_t rb = row_bytes_of(c);
  const bool c16 = rb % 16 == 0;
  const int cpr = static_cast<int>(c16 ? rb / 16 : rb / 4);
  const size_t total = static_cast<size_t>(c.B) * c.nKV * C * cpr;
  if (one_block_ok(c, C, cpr)) {
    if (c16)
      hipLaunchKernelGGL(k_append_one<Chunk16>, dim3(1), dim3(kOneBlock), 0, s, c, k_new, v_new,
                         C, n_rows, cpr, rb);
    else
      hipLaunchKernelGGL(k_append_one<uint32_t>, dim3(1), dim3(kOneBlock), 0, s, c, k_new, v_new,
                         C, n_rows, cpr, rb);
    return hipGetLastError();
  }
  const bool f32 = fits32(c, C, rb);
  if (c16)
    CP_LAUNCH_IDX(k_append, Chunk16, grid_for(total), c, k_new, v_new, C, n_rows, cpr, rb);
  else
    CP_LAUNCH_IDX(k_append, uint32_t, grid_for(total), c, k_new, v_new, C, n_rows, cpr, rb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_append_seen, dim3((c.B + 255) / 256), dim3(256), 0, s, c, n_rows, C);
  return hipGetLastError();
}

hipError_t launch_snapshot(const cp_cache &c, int C, const int32_t *n_valid, void *buf,
                           hipStream_t s) {
  if (c.B == 0) return hipSuccess;
  const size_t rb = row_bytes_of(c);
  const size_t hdr = snapshot_header_bytes(c.B);
  unsigned char *b = static_cast<unsigned char *>(buf);
  const bool c16 = rb % 16 == 0;
  const int cpr = static_cast<int>(c16 ? rb / 16 : rb / 4);
  const size_t total = static_cast<size_t>(c.B) * c.nKV * C * cpr;
  // the grid always covers B threads: they write the header, even for C == 0
  const unsigned grid = grid_for(total > static_cast<size_t>(c.B) ? total : c.B);
  const bool f32 = fits32(c, C, rb);
  if (c16)
    CP_LAUNCH_IDX(k_snapshot, Chunk16, grid, c, C, n_valid, b, hdr, cpr, rb);
  else
    CP_LAUNCH_IDX(k_snapshot, uint32_t, grid, c, C, n_valid, b, hdr, cpr, rb);
  return hipGetLastError();
}

hipError_t launch_rollback(const cp_cache &c, int C, const void *buf, hipStream_t s) {
  if (c.B == 0) return hipSuccess;
  const size_t rb = row_bytes_of(c);
  const size_t hdr = snapshot_header_bytes(c.B);
  const unsigned char *b = static_cast<const unsigned char *>(buf);
  const bool c16 = rb % 16 == 0;
  const int cpr = static_cast<int>(c16 ? rb / 16 : rb / 4);
  const size_t total = static_cast<size_t>(c.B) * c.nKV * C * cpr;
  if (one_block_ok(c, C, cpr)) {
    if (c16)
      hipLaunchKernelGGL(k_restore_one<Chunk16>, dim3(1), dim3(kOneBlock), 0, s, c, C, b, hdr, cpr,
                         rb);
    else
      hipLaunchKernelGGL(k_restore_one<uint32_t>, dim3(1), dim3(kOneBlock), 0, s, c, C, b, hdr,
                         cpr, rb);
    return hipGetLastError();
  }
  const bool f32 = fits32(c, C, rb);
  if (c16)
    CP_LAUNCH_IDX(k_restore, Chunk16, grid_for(total), c, C, b, hdr, cpr, rb);
  else
    CP_LAUNCH_IDX(k_restore, uint32_t, grid_for(total), c, C, b, hdr, cpr, rb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_rollback_seen, dim3((c.B + 255) / 256), dim3(256), 0, s, c, C, b);
  return hipGetLastError();
}

hipError_t launch_append_rollback(const cp_cache &c, const void *k_new, const void *v_new, int C,
                                  const void *buf, hipStream_t s) {
  if (c.B == 0) return hipSuccess;
  const size_t rb = row_bytes_of(c);
  const size_t hdr = snapshot_header_bytes(c.B);
  const unsigned char *b = static_cast<const unsigned char *>(buf);
  const bool c16 = rb % 16 == 0 && ((reinterpret_cast<uintptr_t>(k_new) |
                                     reinterpret_cast<uintptr_t>(v_new) |
                                     reinterpret_cast<uintptr_t>(c.k) |
                                     reinterpret_cast<uintptr_t>(c.v)) & 15) == 0;
  const int cpr = static_cast<int>(c16 ? rb / 16 : rb / 4);
  const size_t total = static_cast<size_t>(c.B) * c.nKV * C * cpr;
  // the grid always covers B threads: they do the bookkeeping, even for C == 0
  const unsigned grid = grid_for(total > static_cast<size_t>(c.B) ? total : c.B);
  const bool f32 = fits32(c, C, rb);
  if (c16)
    CP_LAUNCH_IDX(k_append_rollback, Chunk16, grid, c, k_new, v_new, C, b, hdr, cpr, rb);
  else
    CP_LAUNCH_IDX(k_append_rollback, uint32_t, grid, c, k_new, v_new, C, b, hdr, cpr, rb);
  return hipGetLastError();
}

#undef CP_LAUNCH_IDX

}  // namespace cp
