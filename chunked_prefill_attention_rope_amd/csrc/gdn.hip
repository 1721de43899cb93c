// gdn.hip -- gated delta rule prefill in chunks (the linear-attention layer of a
// hybrid model), fp32 on the matrix cores.
//
// [Kazeia] "Chantier 4 -- GDN chunkwise prefill", sections "Le kernel actuel" and
// "P1 -- chunk f32": per (sequence, head) a state S of dk x dv; per token the state
// decays by the gate g_t = exp(alpha_t), delta = (v_t - S^T k_t) beta_t, S += k_t
// delta^T, out_t = S^T q_t.  Token by token that is a serial chain of rank-1
// updates; the section "Chunkwise (delta rule)" turns a chunk of 64 tokens into
// dense products.  With lg_t = alpha_1 + ... + alpha_t inside the chunk, R[t,s] =
// exp(lg_t - lg_s) (s <= t) and entry state S0:
//   A[t,s] = beta_t R[t,s] k_t.k_s (s < t)          T = (I + A)^-1
//   U = T diag(beta) V       W = T diag(beta e^lg) K       D = U - W S0
//   O = diag(e^lg) Q S0 + (tril(R) * Q K^T) D
//   S = e^{lg_last} S0 + K^T diag(R[last, :]) D
// A, T, U and W never see the state, and O of a chunk needs only the chunk's entry
// state and D: only D and the state update form the serial chain across chunks.
//
// Two kernels, both on v_mfma_f32_16x16x4f32 (fp32 products, fp32 sums):
//  - k_gdn_prep, two workgroups per (chunk, head, sequence): one forms the Gram
//    product K K^T, T by inverting the four 16x16 diagonal blocks of I + A
//    (one lane per column) and filling the blocks below them in three rounds
//    (T_ij = -T_ii sum_k A_ik T_kj); then [U | W] = T [diag(beta) V | diag(beta e^lg) K],
//    and writes W, U and lg; the other forms P = tril(R) * Q K^T and writes it with K^T.
//  - k_gdn_scan, one workgroup per (16 state columns, head, sequence): the state's
//    columns evolve independently.  Four waves walk the chunks: each computes 16 rows
//    of D = U - W S, then updates its own row blocks of S (kept in MFMA accumulators,
//    mirrored to LDS transposed for the next chunk's D).  Four more waves form the
//    chunk's output O = diag(e^lg) Q S_c + P D_c for the same 16 columns from the entry
//    state and D in LDS, so neither goes back to memory.
// Pad rows of a last partial chunk are zero with beta = 0 and a zero log-gate: their
// rows of A, U, W and D are zero, they leave the state untouched and are not stored.
//
// MFMA 16x16x4 fp32 operand layout (lane l, m = l % 16, g = l / 16): A supplies
// A[m][g], B supplies B[g][m], and accumulator register r holds C[4g + r][m].  A
// product's register r is therefore a valid B operand for the k-step whose four
// contraction indices are {4g + r}, which chains products without a trip through LDS.
#include <algorithm>
#include <type_traits>

#include "cp_common.h"

namespace cp {
namespace {

constexpr int CH = 64;      // tokens per chunk
constexpr int VB = 16;      // state columns per scan workgroup
constexpr int AP = CH + 4;  // LDS row stride of the 64 x 64 tiles

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Workgroup L runs on XCD L % 8.  All workgroups of one (sequence, head) -- which read
// the same chunk products -- go to one XCD, so those reads share its L2: (sequence,
// head) G takes XCD G % 8, and its `per` workgroups the successive slots there.  The
// grid has 8 * ceil(BH / 8) * per workgroups; the surplus ones (G >= BH) exit at once.
__device__ __forceinline__ bool head_slot(int per, int BH, int &G, int &k) {
  const int L = blockIdx.x, x = L % 8, slot = L / 8;
  G = x + 8 * (slot / per);
  k = slot % per;
  return G < BH;
}

__device__ __forceinline__ f4 ld4(const float *p) { return *reinterpret_cast<const f4 *>(p); }
__device__ __forceinline__ void st4(float *p, f4 v) { *reinterpret_cast<f4 *>(p) = v; }

// Block orders of the chunk products.  A matrix with ncb column blocks of 16 is stored
// as 16 x 16 blocks, block (rb, cb) the 256 consecutive floats at (rb * ncb + cb) * 256,
// in which lane l = 16 g + m of a wave owns the four floats at 4 l:
//  - operand order: row m, columns 4 g .. 4 g + 3 of the block (an A operand's four
//    k-steps);
//  - accumulator order: rows 4 g .. 4 g + 3, column m (a 16x16x4 product's registers).
// A wave moves a block with one 16-byte access per lane, 1 KB of consecutive memory.
// Row-major, a wave's 16 lanes of one column group would touch 16 different rows, and
// an accumulator would leave in four 4-byte stores.  A product computed transposed
// (operands swapped) leaves its accumulator in operand order.
__device__ __forceinline__ size_t blk(int rb, int cb, int ncb, int lane) {
  return ((static_cast<size_t>(rb) * ncb + cb) * 64 + lane) * 4;
}

// Workspace of one (sequence, head, chunk), in floats.
template <int DK, int DV>
struct Chunk {
  static constexpr size_t W = 0;               // [CH][DK]  T diag(beta e^lg) K, operand order
  static constexpr size_t U = W + CH * DK;     // [CH][DV]  T diag(beta) V, accumulator order
  static constexpr size_t P = U + CH * DV;     // [CH][CH]  tril(R) * Q K^T (lower blocks), operand order
  static constexpr size_t LG = P + CH * CH;    // [CH]      cumulated log-gates
  static constexpr size_t KT = LG + CH;        // [DK][CH]  K^T, operand order
  static constexpr size_t SIZE = KT + DK * CH;
};

__host__ __device__ constexpr size_t gdn_chunk_floats(int dk, int dv) {
  return 2 * static_cast<size_t>(CH) * dk + static_cast<size_t>(CH) * dv + CH * CH + CH;
}
static_assert(Chunk<128, 64>::SIZE == gdn_chunk_floats(128, 64), "workspace layout");

constexpr int PREP_THREADS = 512;  // 8 waves: two per SIMD to overlap LDS and MFMA latency

template <int DK, int DV>
__global__ void __launch_bounds__(PREP_THREADS) k_gdn_prep(const float *__restrict__ q,
                                                  const float *__restrict__ k,
                                                  const float *__restrict__ v,
                                                  const float *__restrict__ beta,
                                                  const float *__restrict__ alpha,
                                                  float *__restrict__ ws, int BH, int P, int nch) {
  using L = Chunk<DK, DV>;
  constexpr int KP = DK + 4, VP = DV + 4;
  __shared__ __align__(16) float Ks[CH * KP];
  __shared__ __align__(16) float Qs[CH * KP];
  __shared__ __align__(16) float Vs[CH * VP];
  __shared__ __align__(16) float As[CH * AP];
  __shared__ __align__(16) float Ts[CH * AP];
  __shared__ float lg[CH], bt[CH], fk[CH];  // lg, beta, beta e^lg
  // Two workgroups per chunk: role 0 forms A = K K^T, T and [U | W]; role 1 the output's
  // P = tril(R) * Q K^T and K^T.  They write disjoint parts of the chunk's workspace.
  int G, cr;
  if (!head_slot(2 * nch, BH, G, cr)) return;  // whole workgroup, before any barrier
  const int role = cr >= nch ? 1 : 0;
  const int c = cr - role * nch;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, m = lane & 15, g = lane >> 4;
  const size_t bh = G;
  const int t0 = c * CH;
  const int n = min(CH, P - t0);
  float *ck = ws + (bh * nch + c) * L::SIZE;

  const f4 zero = {0.f, 0.f, 0.f, 0.f};
  {  // the chunk's K and V (role 0) or K and Q (role 1): every load in flight before the
     // first LDS store
    constexpr int NK = CH * DK / (4 * PREP_THREADS), NV = CH * DV / (4 * PREP_THREADS);
    f4 kr[NK], qr[NK], vr[NV];
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int e = tid + PREP_THREADS * u, t = e / (DK / 4), i = (e % (DK / 4)) * 4;
      const size_t src = (bh * P + t0 + t) * DK + i;
      kr[u] = t < n ? ld4(k + src) : zero;
      qr[u] = t < n && role == 1 ? ld4(q + src) : zero;
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int e = tid + PREP_THREADS * u, t = e / (DV / 4), j = (e % (DV / 4)) * 4;
      vr[u] = t < n && role == 0 ? ld4(v + (bh * P + t0 + t) * DV + j) : zero;
    }
#pragma unroll
    for (int u = 0; u < NK; ++u) {
      const int e = tid + PREP_THREADS * u, t = e / (DK / 4), i = (e % (DK / 4)) * 4;
      st4(&Ks[t * KP + i], kr[u]);
      if (role == 1) st4(&Qs[t * KP + i], qr[u]);
    }
    if (role == 0) {
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int e = tid + PREP_THREADS * u, t = e / (DV / 4), j = (e % (DV / 4)) * 4;
        st4(&Vs[t * VP + j], vr[u]);
      }
    }
  }
  if (w == 0) {  // inclusive prefix sum of the log-gates over the chunk
    const bool in = lane < n;
    float a = in ? alpha[bh * P + t0 + lane] : 0.f;
    for (int off = 1; off < CH; off <<= 1) {
      const float y = __shfl_up(a, off, 64);
      if (lane >= off) a += y;
    }
    const float be = in ? beta[bh * P + t0 + lane] : 0.f;
    lg[lane] = a;
    bt[lane] = be;
    fk[lane] = be * __expf(a);
    if (role == 0) ck[L::LG + lane] = a;
  }
  __syncthreads();

  // Gram tiles on and below the diagonal: the 10 tiles of K K^T (-> A, role 0) or of
  // Q K^T (-> P, role 1), dealt over the waves, computed transposed so that lane (m, g)
  // holds row tt 16 + m, columns st 16 + 4 g .. + 3.  Contraction index of k-step (kk, j):
  // g * DK/4 + 4 kk + j.
  for (int p = w + 10 * role; p < 10 + 10 * role; p += PREP_THREADS / 64) {
    const int tl = p % 10;
    const int tt = (tl >= 1) + (tl >= 3) + (tl >= 6);
    const int st = tl - tt * (tt + 1) / 2;
    const float *X = p >= 10 ? Qs : Ks;
    f4 acc0 = zero, acc1 = zero;
#pragma unroll
    for (int kk = 0; kk < DK / 16; kk += 2) {
      const int i0 = g * (DK / 4) + kk * 4;
      const f4 a0 = ld4(&X[(tt * 16 + m) * KP + i0]);
      const f4 b0 = ld4(&Ks[(st * 16 + m) * KP + i0]);
      const f4 a1 = ld4(&X[(tt * 16 + m) * KP + i0 + 4]);
      const f4 b1 = ld4(&Ks[(st * 16 + m) * KP + i0 + 4]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc0 = mma(b0[j], a0[j], acc0);
        acc1 = mma(b1[j], a1[j], acc1);
      }
    }
    const int t = tt * 16 + m;
    const float lgt = lg[t], bq = bt[t];
    f4 o;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = st * 16 + 4 * g + r;
      const float gram = acc0[r] + acc1[r];
      const float rr = s <= t ? __expf(lgt - lg[s]) : 0.f;
      o[r] = p < 10 ? (s < t ? bq * rr * gram : 0.f) : rr * gram;
    }
    if (p < 10)
      st4(&As[t * AP + st * 16 + 4 * g], o);
    else
      st4(&ck[L::P + blk(tt, st, CH / 16, lane)], o);
  }
  if (role == 1) {
    // K^T for the scan's state update, one lane's four operand floats per thread
    for (int e = tid; e < DK * CH / 4; e += PREP_THREADS) {
      const int b = e / 64, l = e % 64;
      const int i = (b / (CH / 16)) * 16 + l % 16, t = (b % (CH / 16)) * 16 + 4 * (l / 16);
      const f4 x = {Ks[t * KP + i], Ks[(t + 1) * KP + i], Ks[(t + 2) * KP + i],
                    Ks[(t + 3) * KP + i]};
      st4(&ck[L::KT + 4 * static_cast<size_t>(e)], x);
    }
    return;  // (the whole workgroup: role 1 passes no further barrier)
  }
  __syncthreads();

  // T = (I + A)^-1.  Diagonal blocks: wave w < 4 inverts block w, lane m < 16 one
  // column (unit lower triangular: forward substitution on e_m).
  if (w < 4 && g == 0) {
    const int o = w * 16;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float acc = t == m ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < t; ++s) acc = fmaf(-As[(o + t) * AP + o + s], x[s], acc);
      x[t] = acc;
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) Ts[(o + t) * AP + o + m] = x[t];
  }
  __syncthreads();
  // Blocks below the diagonal, by distance from it: T_ij = -T_ii sum_{k=j}^{i-1} A_ik T_kj.
  auto below = [&](int i, int j) {
    f4 acc = zero;
    for (int kb = j; kb < i; ++kb) {
      const f4 a = ld4(&As[(i * 16 + m) * AP + kb * 16 + 4 * g]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = mma(a[kk], Ts[(kb * 16 + 4 * g + kk) * AP + j * 16 + m], acc);
    }
    const f4 a2 = ld4(&Ts[(i * 16 + m) * AP + i * 16 + 4 * g]);
    f4 t = zero;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t = mma(a2[kk], acc[kk], t);
#pragma unroll
    for (int r = 0; r < 4; ++r) Ts[(i * 16 + 4 * g + r) * AP + j * 16 + m] = -t[r];
  };
  if (w < 3) below(w + 1, w);
  __syncthreads();
  if (w < 2) below(w + 2, w);
  __syncthreads();
  if (w == 0) below(3, 0);
  __syncthreads();

  // [U | W] = T [diag(beta) V | diag(beta e^lg) K]: column tiles dealt over the waves.
  // U leaves in accumulator order (the scan's D rows take it so); W is computed
  // transposed and leaves in operand order (the scan's A operand).
  auto tile = [&](auto transposed, int ct) {
    constexpr bool TR = decltype(transposed)::value;
    const float *Y = TR ? Ks + ct * 16 : Vs + ct * 16;
    const int yp = TR ? KP : VP;
    const float *f = TR ? fk : bt;
    f4 acc[4] = {zero, zero, zero, zero};
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      float bv[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int s = sb * 16 + 4 * g + kk;
        bv[kk] = f[s] * Y[s * yp + m];
      }
#pragma unroll
      for (int tt = sb; tt < 4; ++tt) {
        const f4 a = ld4(&Ts[(tt * 16 + m) * AP + sb * 16 + 4 * g]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc[tt] = TR ? mma(bv[kk], a[kk], acc[tt]) : mma(a[kk], bv[kk], acc[tt]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
      st4(&ck[TR ? L::W + blk(tt, ct, DK / 16, lane) : L::U + blk(tt, ct, DV / 16, lane)], acc[tt]);
  };
  for (int ct = w; ct < DV / 16; ct += PREP_THREADS / 64) tile(std::false_type{}, ct);
  for (int ct = w; ct < DK / 16; ct += PREP_THREADS / 64) tile(std::true_type{}, ct);
}

constexpr int SCAN_THREADS = 512;  // four waves walk the state, four form the output

template <int DK, int DV>
__global__ void __launch_bounds__(SCAN_THREADS) k_gdn_scan(const float *__restrict__ q,
                                                           float *__restrict__ ws,
                                                           float *__restrict__ state,
                                                           float *__restrict__ out, int BH, int P,
                                                           int nch) {
  using L = Chunk<DK, DV>;
  constexpr int NIB = DK / 16;  // row blocks of the state
  constexpr int OWN = NIB / 4;  // row blocks each state wave updates
  constexpr int SP = DK + 4;
  constexpr int QP = DK + 4;    // LDS row stride of an output wave's staged rows of Q
  __shared__ __align__(16) float St[VB * SP];     // S^T of this column block: St[j][i]
  __shared__ __align__(16) float Dt[VB * AP];     // (diag(R[last, :]) D)^T: Dt[j][t]
  __shared__ __align__(16) float Dc[CH * VB];     // D, row blocks in accumulator order
  __shared__ __align__(16) float Qs[4 * 16 * QP];  // output wave ow's 16 rows of Q
  int G, jb;
  if (!head_slot(DV / VB, BH, G, jb)) return;  // whole workgroup, before any barrier
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, m = lane & 15, g = lane >> 4;
  const bool walker = w < 4;  // waves 0..3 walk the state, 4..7 form the output
  const size_t bh = G;
  const int j0 = jb * VB;
  float *S = state + bh * DK * DV;
  const f4 zero = {0.f, 0.f, 0.f, 0.f};

  // The state walk (waves 0..3) is the serial chain; the output waves fill the matrix
  // cores' idle cycles, so the walkers take issue priority on their SIMDs.
  if (walker) __builtin_amdgcn_s_setprio(1);

  f4 sacc[OWN];
  if (walker) {
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int ib = w * OWN + o;
#pragma unroll
      for (int r = 0; r < 4; ++r) sacc[o][r] = S[(ib * 16 + 4 * g + r) * DV + j0 + m];
      st4(&St[m * SP + ib * 16 + 4 * g], sacc[o]);
    }
  }

  // Walker operands: rows of W, U and the log-gates of a chunk, loaded one chunk ahead;
  // the K^T rows of the state update during the same chunk's D products.  Each
  // workgroup pulls 64 KB of W and K^T per chunk through its CU: issued in one burst
  // those loads fill the vector-memory queue and stall the wave's MFMAs behind them,
  // so they are spread over the D products below (four loads per eight MFMAs).
  struct Ops {
    f4 w[NIB], lg, u;
    float lglast;
  };
  auto fetch_small = [&](const float *ck, Ops &x) {
    x.u = ld4(&ck[L::U + blk(w, jb, DV / 16, lane)]);
    x.lg = ld4(&ck[L::LG + w * 16 + 4 * g]);
    x.lglast = ck[L::LG + CH - 1];
  };
  auto fetch = [&](int c, Ops &x) {
    const float *ck = ws + (bh * nch + c) * L::SIZE;
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) x.w[ib] = ld4(&ck[L::W + blk(w, ib, NIB, lane)]);
    fetch_small(ck, x);
  };

  // Output waves: O = diag(e^lg) Q S_c + P D_c for rows 16 ow .. 16 ow + 15 of chunk c and
  // this workgroup's 16 columns.  Q S_c runs while the walkers form D_c (S_c is in St
  // until the state update); P D_c while they update the state (D_c in Dc).  Chunk
  // c + 1's rows of Q (loaded row-major into registers, then through the wave's LDS
  // stage into operand order), its P blocks and log-gates are loaded one chunk ahead.
  const int ow = w - 4;
  constexpr int NQ = 16 * DK / 4 / 64;  // float4s per lane of 16 rows of Q
  f4 qreg[NQ], pa[4], lgo = zero, oacc = zero;
  auto out_fetch = [&](int c) {
    const int t0 = c * CH;
    const float *ck = ws + (bh * nch + c) * L::SIZE;
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int e = lane + 64 * u, row = e / (DK / 4), t = t0 + 16 * ow + row;
      qreg[u] = t < P ? ld4(q + (bh * P + t) * DK + (e % (DK / 4)) * 4) : zero;
    }
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) pa[sb] = sb <= ow ? ld4(&ck[L::P + blk(ow, sb, CH / 16, lane)]) : zero;
    lgo = ld4(&ck[L::LG + 16 * ow + 4 * g]);
  };
  float *qs = Qs + ow * 16 * QP;
  // Q S_c is split over both intervals, so that the output waves' share of the matrix
  // cores in each is about half the walkers' and the barriers do not wait for them: the
  // first half of the contraction while the walkers form D_c, the second half (its S_c
  // operands kept in registers, since the state update overwrites St) with P D_c.
  constexpr int NH = NIB / 2;
  f4 svh[NH];  // S_c operands of the second half
  auto out_qs = [&]() {  // first half of Q S_c
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int e = lane + 64 * u;
      st4(&qs[(e / (DK / 4)) * QP + (e % (DK / 4)) * 4], qreg[u]);
    }
    f4 qa[NH], sv[NH];
#pragma unroll
    for (int ib = 0; ib < NH; ++ib) {
      qa[ib] = ld4(&qs[m * QP + ib * 16 + 4 * g]);
      sv[ib] = ld4(&St[m * SP + ib * 16 + 4 * g]);
      svh[ib] = ld4(&St[m * SP + (NH + ib) * 16 + 4 * g]);
    }
    f4 o0 = zero, o1 = zero;
#pragma unroll
    for (int ib = 0; ib < NH; ib += 2) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        o0 = mma(qa[ib][kk], sv[ib][kk], o0);
        o1 = mma(qa[ib + 1][kk], sv[ib + 1][kk], o1);
      }
    }
    oacc = o0 + o1;
  };
  auto out_pd = [&](int c) {  // second half of Q S_c, e^lg, + P D_c, then store
    const int t0 = c * CH;
    {
      f4 qa[NH];
#pragma unroll
      for (int ib = 0; ib < NH; ++ib) qa[ib] = ld4(&qs[m * QP + (NH + ib) * 16 + 4 * g]);
      f4 o1 = zero;
#pragma unroll
      for (int ib = 0; ib < NH; ib += 2) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          oacc = mma(qa[ib][kk], svh[ib][kk], oacc);
          o1 = mma(qa[ib + 1][kk], svh[ib + 1][kk], o1);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[r] = (oacc[r] + o1[r]) * __expf(lgo[r]);
    }
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      if (sb > ow) break;
      const f4 db = ld4(&Dc[sb * 256 + 4 * lane]);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) oacc = mma(pa[sb][kk], db[kk], oacc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = t0 + 16 * ow + 4 * g + r;
      if (t < P) out[(bh * P + t) * DV + j0 + m] = oacc[r];
    }
  };

  // One chunk: the walkers consume the operands in cu and load chunk c + 1's into nx.
  // Two operand sets alternate roles (the loop below is unrolled by two), so the
  // prefetched registers are never copied -- a copy would wait for the loads it is
  // meant to hide.
  auto step = [&](int c, const Ops &cu, Ops &nx) {
    const float *ck = ws + (bh * nch + c) * L::SIZE;
    const float *cn = ws + (bh * nch + min(c + 1, nch - 1)) * L::SIZE;
    float glast = 0.f;
    f4 kt[OWN * 4];  // this chunk's K^T operands, for the state update
    if (walker) {
      // rows 16w..16w+15 of D = U - W S (contraction over the state's rows)
      f4 d0 = zero, d1 = zero;
#pragma unroll
      for (int ib = 0; ib < NIB; ib += 2) {
        const f4 b0 = ld4(&St[m * SP + ib * 16 + 4 * g]);
        const f4 b1 = ld4(&St[m * SP + ib * 16 + 16 + 4 * g]);
        nx.w[ib] = ld4(&cn[L::W + blk(w, ib, NIB, lane)]);
        nx.w[ib + 1] = ld4(&cn[L::W + blk(w, ib + 1, NIB, lane)]);
#pragma unroll
        for (int u = ib; u < ib + 2; ++u)
          kt[u] = ld4(&ck[L::KT + blk(w * OWN + u / 4, u % 4, CH / 16, lane)]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          d0 = mma(cu.w[ib][kk], b0[kk], d0);
          d1 = mma(cu.w[ib + 1][kk], b1[kk], d1);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the next loads behind these MFMAs
      }
      fetch_small(cn, nx);
      const f4 dd = cu.u - (d0 + d1);
      st4(&Dc[w * 256 + 4 * lane], dd);
      f4 dw;
#pragma unroll
      for (int r = 0; r < 4; ++r) dw[r] = __expf(cu.lglast - cu.lg[r]) * dd[r];
      st4(&Dt[m * AP + w * 16 + 4 * g], dw);
      glast = __expf(cu.lglast);
    } else {
      out_qs();
    }
    __syncthreads();  // Dt and Dc complete; every wave is done reading St
    if (walker) {
      // S = e^{lg_last} S + K^T diag(R[last, :]) D for this wave's row blocks
#pragma unroll
      for (int o = 0; o < OWN; ++o) {
        const int ib = w * OWN + o;
        f4 acc = sacc[o] * glast;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
          const f4 a = kt[o * 4 + tb];
          const f4 bb = ld4(&Dt[m * AP + tb * 16 + 4 * g]);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) acc = mma(a[kk], bb[kk], acc);
        }
        sacc[o] = acc;
        st4(&St[m * SP + ib * 16 + 4 * g], acc);
      }
    } else {
      out_pd(c);
      if (c + 1 < nch) out_fetch(c + 1);
    }
    __syncthreads();  // St holds the next entry state; Dt and Dc are free
  };
  Ops xa, xb;
  if (walker)
    fetch(0, xa);
  else
    out_fetch(0);
  __syncthreads();  // St holds the entry state
  for (int c = 0; c < nch; c += 2) {
    step(c, xa, xb);
    if (c + 1 < nch) step(c + 1, xb, xa);
  }
  if (walker) {
#pragma unroll
    for (int o = 0; o < OWN; ++o) {
      const int ib = w * OWN + o;
#pragma unroll
      for (int r = 0; r < 4; ++r) S[(ib * 16 + 4 * g + r) * DV + j0 + m] = sacc[o][r];
    }
  }
}

template <int DK, int DV>
hipError_t launch_dims(const float *q, const float *k, const float *v, const float *beta,
                       const float *alpha, float *state, float *out, int B, int H, int P,
                       float *ws, hipStream_t s) {
  const int nch = (P + CH - 1) / CH;
  const int BH = B * H, slots = 8 * ((BH + 7) / 8);  // grid sizes checked by gdn_grid_fits
  hipLaunchKernelGGL((k_gdn_prep<DK, DV>), dim3(slots * 2 * nch), dim3(PREP_THREADS), 0, s, q,
                     k, v, beta, alpha, ws, BH, P, nch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gdn_scan<DK, DV>), dim3(slots * (DV / VB)), dim3(SCAN_THREADS), 0, s, q,
                     ws, state, out, BH, P, nch);
  return hipGetLastError();
}

}  // namespace

size_t gdn_workspace_bytes(int B, int H, int P, int dk, int dv) {
  const size_t nch = (static_cast<size_t>(P) + CH - 1) / CH;
  return static_cast<size_t>(B) * H * nch * gdn_chunk_floats(dk, dv) * sizeof(float);
}

bool gdn_grid_fits(int B, int H, int P) {
  const size_t slots = 8 * ((static_cast<size_t>(B) * H + 7) / 8);
  const size_t nch = (static_cast<size_t>(P) + CH - 1) / CH;
  const size_t per = std::max<size_t>(2 * nch, 128 / VB);  // the larger of the two grids
  return slots * per <= 0x7fffffff;
}

bool gdn_dims_supported(int dk, int dv) {
  return (dk == 64 || dk == 128) && (dv == 64 || dv == 128);
}

hipError_t launch_gdn(const float *q, const float *k, const float *v, const float *beta,
                      const float *alpha, float *state, float *out, int B, int H, int P, int dk,
                      int dv, void *ws, hipStream_t s) {
  float *w = static_cast<float *>(ws);
  if (dk == 64 && dv == 64) return launch_dims<64, 64>(q, k, v, beta, alpha, state, out, B, H, P, w, s);
  if (dk == 64 && dv == 128)
    return launch_dims<64, 128>(q, k, v, beta, alpha, state, out, B, H, P, w, s);
  if (dk == 128 && dv == 64)
    return launch_dims<128, 64>(q, k, v, beta, alpha, state, out, B, H, P, w, s);
  return launch_dims<128, 128>(q, k, v, beta, alpha, state, out, B, H, P, w, s);
}

}  // namespace cp
