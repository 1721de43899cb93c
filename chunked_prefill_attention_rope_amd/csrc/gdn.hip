// gdn.hip -- gated delta rule prefill in chunks (the linear-attention layer of a
// hybrid model), fp32.
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
// (A, U and W never see the state: they are computed for every chunk at once.)
//
// Two kernels:
//  - k_gdn_prep: one workgroup per (sequence, head, chunk).  K and Q of the chunk
//    in LDS; the gated, masked products A and P = tril(R) * Q K^T; U and W by forward
//    substitution, one thread per column (rows of a column depend only on earlier
//    rows of the same column, so the columns need no barriers).  Writes W, U, P and lg
//    to the workspace.
//  - k_gdn_scan: one workgroup per (sequence, head, 16 columns of the state): the
//    columns of S evolve independently, so the state's dv columns are split over
//    workgroups.  Walks the chunks in order: D, O and the next state, all from LDS.
// Pad rows of a last partial chunk are zero with beta = 0 and a zero log-gate: their
// rows of U, W and D are zero and they leave the state untouched.
#include "cp_common.h"

namespace cp {
namespace {

constexpr int CH = 64;   // tokens per chunk
constexpr int VB = 16;   // state columns per scan workgroup

__host__ __device__ constexpr size_t gdn_chunk_floats(int dk, int dv) {
  return static_cast<size_t>(CH) * dk + static_cast<size_t>(CH) * dv + CH * CH + CH;
}

template <int DK, int DV>
__global__ void __launch_bounds__(256) k_gdn_prep(const float *__restrict__ q,
                                                  const float *__restrict__ k,
                                                  const float *__restrict__ v,
                                                  const float *__restrict__ beta,
                                                  const float *__restrict__ alpha,
                                                  float *__restrict__ ws, int H, int P, int nch) {
  constexpr int NX = DV + DK;  // columns of the substitution: U's, then W's
  __shared__ float Ks[CH][DK + 1];
  __shared__ float Qs[CH][DK + 1];
  __shared__ float As[CH][CH + 1];
  __shared__ float Xs[CH][NX];
  __shared__ float lg[CH], bt[CH];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const int t0 = c * CH;
  const int n = min(CH, P - t0);
  for (int e = tid; e < CH * DK; e += 256) {
    const int t = e / DK, i = e % DK;
    const bool in = t < n;
    Ks[t][i] = in ? k[(bh * P + t0 + t) * DK + i] : 0.f;
    Qs[t][i] = in ? q[(bh * P + t0 + t) * DK + i] : 0.f;
  }
  if (tid < CH) {
    const bool in = tid < n;
    lg[tid] = in ? alpha[bh * P + t0 + tid] : 0.f;
    bt[tid] = in ? beta[bh * P + t0 + tid] : 0.f;
  }
  __syncthreads();
  if (tid == 0) {  // inclusive prefix sum of the log-gates (64 terms, fp32)
    float acc = 0.f;
    for (int t = 0; t < CH; ++t) {
      acc += lg[t];
      lg[t] = acc;
    }
  }
  __syncthreads();

  float *W = ws + (bh * nch + c) * gdn_chunk_floats(DK, DV);
  float *U = W + CH * DK;
  float *Pm = U + CH * DV;
  float *LG = Pm + CH * CH;
  // A (strictly lower) into LDS, P = tril(R) * Q K^T into the workspace
  for (int e = tid; e < CH * CH; e += 256) {
    const int t = e / CH, s = e % CH;
    float a = 0.f, pv = 0.f;
    if (s <= t) {
      float kk = 0.f, qk = 0.f;
#pragma unroll 8
      for (int i = 0; i < DK; ++i) {
        kk = fmaf(Ks[t][i], Ks[s][i], kk);
        qk = fmaf(Qs[t][i], Ks[s][i], qk);
      }
      const float r = __expf(lg[t] - lg[s]);
      pv = r * qk;
      if (s < t) a = bt[t] * r * kk;
    }
    As[t][s] = a;
    Pm[e] = pv;
  }
  if (tid < CH) LG[tid] = lg[tid];
  __syncthreads();

  // right-hand sides: beta V (U's columns), beta e^lg K (W's columns)
  for (int e = tid; e < CH * NX; e += 256) {
    const int t = e / NX, col = e % NX;
    float rhs = 0.f;
    if (col < DV) {
      if (t < n) rhs = bt[t] * v[(bh * P + t0 + t) * DV + col];
    } else {
      rhs = bt[t] * __expf(lg[t]) * Ks[t][col - DV];
    }
    Xs[t][col] = rhs;
  }
  __syncthreads();
  // forward substitution (I + A) X = rhs in place, one column per thread: row t of a
  // column needs only the earlier rows of the same column
  for (int col = tid; col < NX; col += 256) {
    for (int t = 1; t < CH; ++t) {
      float acc = Xs[t][col];
      for (int s = 0; s < t; ++s) acc = fmaf(-As[t][s], Xs[s][col], acc);
      Xs[t][col] = acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < CH * NX; e += 256) {
    const int t = e / NX, col = e % NX;
    if (col < DV)
      U[t * DV + col] = Xs[t][col];
    else
      W[t * DK + col - DV] = Xs[t][col];
  }
}

template <int DK, int DV>
__global__ void __launch_bounds__(256) k_gdn_scan(const float *__restrict__ q,
                                                  const float *__restrict__ k,
                                                  const float *__restrict__ ws,
                                                  float *__restrict__ state,
                                                  float *__restrict__ out, int H, int P, int nch) {
  __shared__ float Ws[CH][DK + 1];
  __shared__ float Qs[CH][DK + 1];
  __shared__ float Ks[CH][DK + 1];
  __shared__ float Pm[CH][CH + 1];
  __shared__ float Ss[DK][VB + 1];
  __shared__ float Us[CH][VB + 1];
  __shared__ float Dl[CH][VB + 1];
  __shared__ float lg[CH], eg[CH], wl[CH];  // lg, e^lg, e^(lg_last - lg)
  const int jb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const size_t bh = static_cast<size_t>(b) * H + h;
  const int j0 = jb * VB;
  float *S = state + bh * DK * DV;
  for (int e = tid; e < DK * VB; e += 256) Ss[e / VB][e % VB] = S[(e / VB) * DV + j0 + e % VB];

  for (int c = 0; c < nch; ++c) {
    const int t0 = c * CH;
    const int n = min(CH, P - t0);
    const float *W = ws + (bh * nch + c) * gdn_chunk_floats(DK, DV);
    const float *U = W + CH * DK;
    const float *Pg = U + CH * DV;
    const float *LG = Pg + CH * CH;
    __syncthreads();  // the previous chunk is done with the LDS tiles
    for (int e = tid; e < CH * DK; e += 256) {
      const int t = e / DK, i = e % DK;
      const bool in = t < n;
      Ws[t][i] = W[e];
      Qs[t][i] = in ? q[(bh * P + t0 + t) * DK + i] : 0.f;
      Ks[t][i] = in ? k[(bh * P + t0 + t) * DK + i] : 0.f;
    }
    for (int e = tid; e < CH * CH; e += 256) Pm[e / CH][e % CH] = Pg[e];
    for (int e = tid; e < CH * VB; e += 256) Us[e / VB][e % VB] = U[(e / VB) * DV + j0 + e % VB];
    if (tid < CH) {
      const float l = LG[tid];
      lg[tid] = l;
      eg[tid] = __expf(l);
      wl[tid] = __expf(LG[CH - 1] - l);
    }
    __syncthreads();
    // D = U - W S
    for (int e = tid; e < CH * VB; e += 256) {
      const int t = e / VB, j = e % VB;
      float acc = Us[t][j];
#pragma unroll 8
      for (int i = 0; i < DK; ++i) acc = fmaf(-Ws[t][i], Ss[i][j], acc);
      Dl[t][j] = acc;
    }
    __syncthreads();
    // O = diag(e^lg) Q S + P D
    for (int e = tid; e < CH * VB; e += 256) {
      const int t = e / VB, j = e % VB;
      if (t >= n) continue;
      float qs = 0.f, pd = 0.f;
#pragma unroll 8
      for (int i = 0; i < DK; ++i) qs = fmaf(Qs[t][i], Ss[i][j], qs);
      for (int s = 0; s <= t; ++s) pd = fmaf(Pm[t][s], Dl[s][j], pd);
      out[(bh * P + t0 + t) * DV + j0 + j] = fmaf(eg[t], qs, pd);
    }
    __syncthreads();  // the old state is no longer read
    // S = e^{lg_last} S + K^T diag(R[last, :]) D
    const float glast = eg[CH - 1];
    for (int e = tid; e < DK * VB; e += 256) {
      const int i = e / VB, j = e % VB;
      float acc = glast * Ss[i][j];
      for (int s = 0; s < n; ++s) acc = fmaf(Ks[s][i] * wl[s], Dl[s][j], acc);
      Ss[i][j] = acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < DK * VB; e += 256) S[(e / VB) * DV + j0 + e % VB] = Ss[e / VB][e % VB];
}

template <int DK, int DV>
hipError_t launch_dims(const float *q, const float *k, const float *v, const float *beta,
                       const float *alpha, float *state, float *out, int B, int H, int P,
                       float *ws, hipStream_t s) {
  const int nch = (P + CH - 1) / CH;
  hipLaunchKernelGGL((k_gdn_prep<DK, DV>), dim3(nch, H, B), dim3(256), 0, s, q, k, v, beta,
                     alpha, ws, H, P, nch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gdn_scan<DK, DV>), dim3(DV / VB, H, B), dim3(256), 0, s, q, k, ws, state,
                     out, H, P, nch);
  return hipGetLastError();
}

}  // namespace

size_t gdn_workspace_bytes(int B, int H, int P, int dk, int dv) {
  const size_t nch = (static_cast<size_t>(P) + CH - 1) / CH;
  return static_cast<size_t>(B) * H * nch * gdn_chunk_floats(dk, dv) * sizeof(float);
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
