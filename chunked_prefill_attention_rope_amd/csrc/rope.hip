// rope.hip -- rotary embedding of a chunk from per-position cos/sin tables.
//
// [SKaiNET] "Change (additive)": RoPE from per-position [C, headDim] cos/sin
// tables, one pair per RoPE base; [TICO] "Runtime behavior": (cos_t, sin_t)
// for the absolute position.  Half-split pairing (j with j + D/2).
//
// HBM-bound elementwise kernel: each thread rotates the pairs of one 16-byte
// slice of a row's lower half (and the matching upper-half slice), with
// 16-byte loads and stores.  The math
// runs in fp64: an fp32 x fp32 product is exact in fp64, so the difference
// (or sum) of the two products is rounded exactly once, independent of FMA
// contraction; the result is then rounded to fp32 and, for bf16 storage, to
// bf16 by round-to-nearest-even.  The cache rows built from it are therefore
// reproducible bit for bit.
#include <type_traits>

#include "cp_common.h"

namespace cp {
namespace {

struct alignas(16) Chunk16 {
  uint32_t w[4];
};

__device__ __forceinline__ int imax_(int a, int b) { return a > b ? a : b; }

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float get(float v) { return v; }
  static __device__ __forceinline__ float put(float v) { return v; }
};
template <>
struct Elem<uint16_t> {
  static __device__ __forceinline__ float get(uint16_t v) { return bf16_to_f32(v); }
  static __device__ __forceinline__ uint16_t put(float v) { return f32_to_bf16_rne(v); }
};

// Threads per workgroup: 64 while that keeps the grid within one workgroup per CU
// (a chunk's rows spread over more CUs), else 128.
constexpr int kRopeThreads = 128;

template <typename T, int N>
struct alignas(sizeof(T) * N) Pack {
  T v[N];
};

// A plain register type of B bytes, for rows that are only copied (an aggregate held
// across other work is kept in memory by the compiler).
template <int B>
struct RawOf;
template <>
struct RawOf<16> {
  typedef unsigned type __attribute__((ext_vector_type(4)));
};
template <>
struct RawOf<4> {
  typedef unsigned type;
};
template <>
struct RawOf<2> {
  typedef unsigned short type;
};

// One rotated tensor of a launch: x, y [B, Hx, C, D].
template <typename T>
struct RopeOp {
  const T *x;
  T *y;
  int Hx;
};

// Early append of the second tensor (the keys) into a global cache: the rotated rows,
// and the same slices of the chunk's value rows, go to slots seen[b] + i for the real
// rows i < n_valid[b] -- slots the attention of this chunk never reads, since it reads
// the past below seen and the chunk's own rows from the chunk tensors.  seen is not
// advanced here.  kc == nullptr: no append.
template <typename T>
struct EarlyAppend {
  cp_cache c;
  T *kc, *vc;
  const T *v;
  const int32_t *n_valid;
};

// Snapshot of a padded ring append taken by the same launch ([cactus] "Fix": the rows
// the padded append would over-evict are saved before it): the header (seen, n_valid per
// sequence) and the over-evicted rows of every KV head, into a buffer laid out as
// cp_kv_snapshot_padded_append's.  Safe in the RoPE launch: nothing writes the cache
// before the append that follows the attention.  buf == nullptr: no snapshot.
struct SnapOp {
  cp_cache c;
  unsigned char *buf;
  size_t hdr;            // header bytes
  const int32_t *n_valid;
  int cpr;               // chunks (W) per row
};

// One snapshot work item: t < B writes sequence t's header, t >= B copies chunk
// (t - B) % cpr of row (t - B) / cpr of the [B][nKV][C] snapshot rows (rows past the
// sequence's over-evicted count are skipped).  The same header and rows as k_snapshot.
template <typename W, typename I>
__device__ __forceinline__ void snapshot_item(const SnapOp &sn, int C, I t) {
  const cp_cache &c = sn.c;
  int32_t *h = reinterpret_cast<int32_t *>(sn.buf);
  if (t < static_cast<I>(c.B)) {
    const int b = static_cast<int>(t);
    const int s0 = c.seen[b];
    h[b] = s0;
    h[c.B + b] = read_nvalid(sn.n_valid, b, C, c.status);
    if (s0 < 0) flag(c.status, CP_DEV_SEEN);
    if (!c.ring && s0 + C > c.cap) flag(c.status, CP_DEV_OVERFLOW);
    return;
  }
  t -= static_cast<I>(c.B);
  const I row = t / static_cast<I>(sn.cpr);
  const int ch = static_cast<int>(t - row * sn.cpr);
  const I bg = row / static_cast<I>(C);
  const int r = static_cast<int>(row - bg * C);
  const int b = static_cast<int>(bg / static_cast<I>(c.nKV));
  const int s0 = c.seen[b];
  const int nv = read_nvalid(sn.n_valid, b, C, nullptr);
  if (s0 < 0 || !c.ring) return;
  const int R = c.cap - c.sink;
  const int lo = imax_(c.sink, s0 + nv - R), hi = imax_(lo, imax_(c.sink, s0 + C - R));
  if (r >= hi - lo) return;
  const int sl = slot_of(lo + r, c.cap, c.ring, c.sink);
  const size_t w = static_cast<size_t>(sn.cpr);
  const size_t half = static_cast<size_t>(c.B) * c.nKV * C * w;
  const size_t src = (static_cast<size_t>(bg) * c.cap + sl) * w + ch;
  const size_t dst = static_cast<size_t>(row) * w + ch;
  W *sk = reinterpret_cast<W *>(sn.buf + sn.hdr);
  sk[dst] = static_cast<const W *>(c.k)[src];
  sk[half + dst] = static_cast<const W *>(c.v)[src];
}

// One thread: VEC consecutive pairs (j .. j+VEC-1, j+h2 .. j+h2+VEC-1) of a row,
// moved with vector loads/stores (VEC > 1 needs 16-byte aligned rows and tables).
// x and y may alias: every element is read and written by the same thread.  The grid
// covers the rows of a, then those of b (b.Hx = 0 for a single tensor), so Q and K of
// a chunk are rotated by one launch.
// I: index type -- 32-bit whenever the launch's element count allows (integer division
// is a software sequence, and a 64-bit one several times longer).
// The grid covers the rotation work items, then (with a snapshot) the snapshot's.
template <typename T, int VEC, typename I>
__global__ void __launch_bounds__(kRopeThreads) k_rope(RopeOp<T> a, RopeOp<T> bop, EarlyAppend<T> app,
                                              SnapOp sn, const float *__restrict__ cosb,
                                              const float *__restrict__ sinb, int B, int C, int D,
                                              int Bt) {
  using W = typename std::conditional<(VEC > 1), Chunk16, uint32_t>::type;
  const int h2 = D / 2;
  const I per_row = h2 / VEC;
  const I rows_a = static_cast<I>(B) * a.Hx * C;
  const I rows = rows_a + static_cast<I>(B) * bop.Hx * C;
  const I total = rows * per_row;
  const I total_sn =
      sn.buf ? static_cast<I>(B) + static_cast<I>(B) * sn.c.nKV * C * sn.cpr : static_cast<I>(0);
  for (I t = blockIdx.x * static_cast<I>(blockDim.x) + threadIdx.x; t < total + total_sn;
       t += static_cast<I>(gridDim.x) * blockDim.x) {
    if (t >= total) {
      snapshot_item<W, I>(sn, C, t - total);
      continue;
    }
    I row = t / per_row;
    const int j0 = static_cast<int>(t - row * per_row) * VEC;
    const bool second = row >= rows_a;
    // the tensor's fields selected by value (a reference to one of the two argument
    // structs would make the compiler load the struct through a pointer first)
    const T *opx = second ? bop.x : a.x;
    T *opy = second ? bop.y : a.y;
    const int opH = second ? bop.Hx : a.Hx;
    if (second) row -= rows_a;
    const I bh = row / static_cast<I>(C);
    const int i = static_cast<int>(row - bh * C);
    const int b = static_cast<int>(bh / static_cast<I>(opH));
    const size_t xo = static_cast<size_t>(row) * D;
    const size_t to = (static_cast<size_t>(Bt == 1 ? 0 : b) * C + i) * D;
    const Pack<T, VEC> lo = *reinterpret_cast<const Pack<T, VEC> *>(opx + xo + j0);
    const Pack<T, VEC> hi = *reinterpret_cast<const Pack<T, VEC> *>(opx + xo + j0 + h2);
    const Pack<float, VEC> cl = *reinterpret_cast<const Pack<float, VEC> *>(cosb + to + j0);
    const Pack<float, VEC> sl = *reinterpret_cast<const Pack<float, VEC> *>(sinb + to + j0);
    const Pack<float, VEC> ch = *reinterpret_cast<const Pack<float, VEC> *>(cosb + to + j0 + h2);
    const Pack<float, VEC> sh = *reinterpret_cast<const Pack<float, VEC> *>(sinb + to + j0 + h2);
    // early append of a K row: the append plan (seen, n_valid) and the V row are read
    // along with the row itself, not after the rotation (one round trip, not three)
    // (other rows read their own row again instead: no conditionally filled aggregate)
    const bool app_row = second && app.kc;
    using Raw = typename RawOf<sizeof(T) * VEC>::type;
    const T *vsrc = (app_row ? app.v : opx) + xo;
    const Raw vlo = *reinterpret_cast<const Raw *>(vsrc + j0);
    const Raw vhi = *reinterpret_cast<const Raw *>(vsrc + j0 + h2);
    AppendPlan pl{0, 0, true};
    if (app_row) {
      const int g = static_cast<int>(bh - static_cast<I>(b) * opH);
      pl = append_plan(app.c, app.n_valid, b, C, g == 0 && i == 0 && j0 == 0);
    }
    Pack<T, VEC> ylo, yhi;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float xa = Elem<T>::get(lo.v[e]), xc = Elem<T>::get(hi.v[e]);
      ylo.v[e] = Elem<T>::put(rot_lo(xa, xc, cl.v[e], sl.v[e]));
      yhi.v[e] = Elem<T>::put(rot_hi(xa, xc, ch.v[e], sh.v[e]));
    }
    *reinterpret_cast<Pack<T, VEC> *>(opy + xo + j0) = ylo;
    *reinterpret_cast<Pack<T, VEC> *>(opy + xo + j0 + h2) = yhi;
    if (app_row && !pl.skip && i < pl.n) {
      const int g = static_cast<int>(bh - static_cast<I>(b) * opH);
      const size_t dst = ((static_cast<size_t>(b) * opH + g) * app.c.cap + pl.s0 + i) * D;
      *reinterpret_cast<Pack<T, VEC> *>(app.kc + dst + j0) = ylo;
      *reinterpret_cast<Pack<T, VEC> *>(app.kc + dst + j0 + h2) = yhi;
      *reinterpret_cast<Raw *>(app.vc + dst + j0) = vlo;
      *reinterpret_cast<Raw *>(app.vc + dst + j0 + h2) = vhi;
    }
  }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename T>
hipError_t launch_t(const void *x0, void *y0, int H0, const void *x1, void *y1, int H1,
                    const float *cos, const float *sin, int B, int C, int D, int Bt,
                    hipStream_t s, const EarlyAppend<T> &app = EarlyAppend<T>{},
                    SnapOp sn = SnapOp{}) {
  const int h2 = D / 2;
  const size_t rows = static_cast<size_t>(B) * (H0 + H1) * C;
  if (rows == 0 && !sn.buf) return hipSuccess;
  const RopeOp<T> a{static_cast<const T *>(x0), static_cast<T *>(y0), H0};
  const RopeOp<T> b{static_cast<const T *>(x1), static_cast<T *>(y1), H1};
  constexpr int V16 = 16 / sizeof(T);  // elements per 16 bytes
  bool al = aligned16(cos) && aligned16(sin);
  if (H0 > 0) al = al && aligned16(x0) && aligned16(y0);
  if (H1 > 0) al = al && aligned16(x1) && aligned16(y1);
  if (app.kc) al = al && aligned16(app.kc) && aligned16(app.vc) && aligned16(app.v);
  if (sn.buf) al = al && aligned16(sn.c.k) && aligned16(sn.c.v) && aligned16(sn.buf);
  const bool vec = al && h2 % V16 == 0;
  const size_t row_bytes = static_cast<size_t>(D) * sizeof(T);
  sn.cpr = static_cast<int>(row_bytes / (vec ? 16 : 4));  // the snapshot's copy chunks per row
  const size_t total_sn =
      sn.buf ? static_cast<size_t>(B) + static_cast<size_t>(B) * sn.c.nKV * C * sn.cpr : 0;
  const size_t total = rows * (h2 / (vec ? V16 : 1)) + total_sn;  // threads
  const unsigned bs = total <= 64 * 256 ? 64 : kRopeThreads;
  size_t nb = (total + bs - 1) / bs;
  if (nb > 65535 * 4) nb = 65535 * 4;
  const dim3 grid(static_cast<unsigned>(nb)), block(bs);
  const bool i32 = rows * h2 + total_sn < (size_t(1) << 31);
  if (vec) {
    if (i32)
      hipLaunchKernelGGL((k_rope<T, V16, uint32_t>), grid, block, 0, s, a, b, app, sn, cos, sin,
                         B, C, D, Bt);
    else
      hipLaunchKernelGGL((k_rope<T, V16, size_t>), grid, block, 0, s, a, b, app, sn, cos, sin, B,
                         C, D, Bt);
  } else {
    if (i32)
      hipLaunchKernelGGL((k_rope<T, 1, uint32_t>), grid, block, 0, s, a, b, app, sn, cos, sin, B,
                         C, D, Bt);
    else
      hipLaunchKernelGGL((k_rope<T, 1, size_t>), grid, block, 0, s, a, b, app, sn, cos, sin, B, C,
                         D, Bt);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope(const void *x, void *y, const float *cos, const float *sin, int B, int Hx,
                       int C, int D, int Bt, int dtype, hipStream_t s) {
  return launch_rope2(x, y, Hx, nullptr, nullptr, 0, cos, sin, B, C, D, Bt, dtype, s);
}

hipError_t launch_rope_qk_append(const cp_cache &c, const void *q, void *q_out, int H,
                                 const void *k, void *k_out, const void *v, const float *cos,
                                 const float *sin, int C, int Bt, const int32_t *n_valid,
                                 hipStream_t s) {
  if (c.dtype == CP_BF16) {
    const EarlyAppend<uint16_t> app{c, static_cast<uint16_t *>(c.k), static_cast<uint16_t *>(c.v),
                                    static_cast<const uint16_t *>(v), n_valid};
    return launch_t<uint16_t>(q, q_out, H, k, k_out, c.nKV, cos, sin, c.B, C, c.D, Bt, s, app);
  }
  const EarlyAppend<float> app{c, static_cast<float *>(c.k), static_cast<float *>(c.v),
                               static_cast<const float *>(v), n_valid};
  return launch_t<float>(q, q_out, H, k, k_out, c.nKV, cos, sin, c.B, C, c.D, Bt, s, app);
}

hipError_t launch_rope_qk_snapshot(const cp_cache &c, const void *q, void *q_out, int H,
                                   const void *k, void *k_out, const float *cos, const float *sin,
                                   int C, int Bt, const int32_t *n_valid, void *buf,
                                   hipStream_t s) {
  const SnapOp sn{c, static_cast<unsigned char *>(buf), snapshot_header_bytes(c.B), n_valid, 0};
  if (c.dtype == CP_BF16)
    return launch_t<uint16_t>(q, q_out, H, k, k_out, c.nKV, cos, sin, c.B, C, c.D, Bt, s,
                              EarlyAppend<uint16_t>{}, sn);
  return launch_t<float>(q, q_out, H, k, k_out, c.nKV, cos, sin, c.B, C, c.D, Bt, s,
                         EarlyAppend<float>{}, sn);
}

hipError_t launch_rope2(const void *x0, void *y0, int H0, const void *x1, void *y1, int H1,
                        const float *cos, const float *sin, int B, int C, int D, int Bt, int dtype,
                        hipStream_t s) {
  if (dtype == CP_BF16)
    return launch_t<uint16_t>(x0, y0, H0, x1, y1, H1, cos, sin, B, C, D, Bt, s);
  return launch_t<float>(x0, y0, H0, x1, y1, H1, cos, sin, B, C, D, Bt, s);
}

}  // namespace cp
