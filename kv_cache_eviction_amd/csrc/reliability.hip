// Trajectory reliability weights, LORE-KV page, Method, "Reliability
// weights" (Eqs. 2-4 and 10): R_m = beta cbar_m - gamma Hbar_m - lambda_D
// Dhat_m and omega = softmax over the M lookahead trajectories.
//
// Dhat_m is the disagreement of trajectory m's lookahead queries with the
// other trajectories' queries: the mean of 1 - cos over every query head and
// every cross-trajectory pair of queries at that head (a zero query has cosine
// 0), standardized over the trajectories (population std; Dhat = 0 when the
// spread is below 1e-6).  cbar_m and Hbar_m are the means over the
// trajectory's T tokens of c_u = log q(y_u) + H_u and of H_u, from the caller's
// per-token log-probability and entropy.
//
// The work is tiny (at most 63 queries per head), so it is written for
// exactness, not speed: queries are staged as fp32 (exact for bf16 and fp16),
// dot products, norms and every sum after them run in fp64, and all sums have
// a fixed order, so results do not depend on scheduling.
#include <float.h>

#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace kvs {

constexpr int kRelThreads = 256;
constexpr double kStdFloor = 1e-6;

__host__ __device__ inline int traj_pair_index(int a, int c, int m) {
  // (a, c) with a < c, row-major over the upper triangle
  return a * m - a * (a + 1) / 2 + (c - a - 1);
}

// Grid (h_q, batch).  Cosine sums per trajectory pair at one query head:
// pair_sum[(b*h_q + h)*npairs + traj_pair_index(a, c)] = sum over the t x t
// query pairs (a's, c's) of cos.  The head's m*t lookahead rows are staged with
// 16-byte loads issued together; four lanes share a row's norm; each wave takes
// trajectory pairs in turn, its lanes the query pairs (a dot product per lane,
// four interleaved partial sums), and a fixed-order wave reduction sums them.
template <typename T>
__global__ void __launch_bounds__(kRelThreads)
traj_cosine_kernel(const T *__restrict__ Q, int h_q, int nq, int d, int w, int m, int t,
                   double *__restrict__ pair_sum) {
  constexpr int kMaxRows = 64, kMaxD = 128, kStride = kMaxD + 4;  // 16-byte aligned rows
  constexpr int kEpc = 16 / sizeof(T);                             // elements per 16 bytes
  constexpr int kMaxChunks = kMaxRows * kMaxD / kEpc;
  constexpr int kPerThread = (kMaxChunks + kRelThreads - 1) / kRelThreads;
  __shared__ __align__(16) float rows[kMaxRows * kStride];
  __shared__ double inv_norm[kMaxRows];
  const int h = blockIdx.x, b = blockIdx.y;
  const int mt = m * t;
  const int cpr = d / kEpc, nchunks = mt * cpr;
  const T *q0 = Q + (((long)b * h_q + h) * nq + w) * d;
  U128 v[kPerThread];
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int i = threadIdx.x + u * kRelThreads;
    if (i < nchunks) v[u] = *reinterpret_cast<const U128 *>(q0 + (long)(i / cpr) * d + (i % cpr) * kEpc);
  }
#pragma unroll
  for (int u = 0; u < kPerThread; ++u) {
    const int i = threadIdx.x + u * kRelThreads;
    if (i < nchunks) {
      const Elems16<T> e = elems16<T>(v[u]);
      float *dst = &rows[(i / cpr) * kStride + (i % cpr) * kEpc];
#pragma unroll
      for (int k = 0; k < kEpc; ++k) dst[k] = to_f32(e.e[k]);
    }
  }
  __syncthreads();
  {
    // four lanes per row, each a quarter of the row, added in a fixed order
    const int r = threadIdx.x / 4, qtr = threadIdx.x % 4, len = d / 4;
    double ss = 0.0;
    if (r < mt) {
      const float *x = &rows[r * kStride + qtr * len];
      for (int k = 0; k < len; ++k) ss = fma((double)x[k], (double)x[k], ss);
    }
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if (r < mt && qtr == 0) inv_norm[r] = ss > 0.0 ? 1.0 / sqrt(ss) : 0.0;
  }
  __syncthreads();
  const int lane = threadIdx.x % 64, wv = threadIdx.x / 64;
  const int npairs = m * (m - 1) / 2;
  double *out = pair_sum + ((long)b * h_q + h) * npairs;
  for (int a = 0; a < m; ++a) {
    for (int c = a + 1; c < m; ++c) {
      const int pidx = traj_pair_index(a, c, m);
      if (pidx % (kRelThreads / 64) != wv) continue;
      double acc = 0.0;
      for (int p = lane; p < t * t; p += 64) {
        const int ra = a * t + p / t, rc = c * t + p % t;
        const float4 *xa = reinterpret_cast<const float4 *>(&rows[ra * kStride]);
        const float4 *xc = reinterpret_cast<const float4 *>(&rows[rc * kStride]);
        double d0 = 0.0, d1 = 0.0, d2 = 0.0, d3 = 0.0;
        for (int k = 0; k < d / 4; ++k) {
          const float4 ua = xa[k], uc = xc[k];
          d0 = fma((double)ua.x, (double)uc.x, d0);
          d1 = fma((double)ua.y, (double)uc.y, d1);
          d2 = fma((double)ua.z, (double)uc.z, d2);
          d3 = fma((double)ua.w, (double)uc.w, d3);
        }
        acc += ((d0 + d1) + (d2 + d3)) * inv_norm[ra] * inv_norm[rc];
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (lane == 0) out[pidx] = acc;
    }
  }
}

// Grid (batch), one wave.  D, Dhat, R and the softmax of one sequence; lane j
// handles trajectory j (a loop covers m > 64).  Sums over heads and pairs run
// in a fixed order.
__global__ void __launch_bounds__(64)
reliability_finish_kernel(const double *__restrict__ pair_sum, int h_q, int m, int t,
                          const float *__restrict__ logp, const float *__restrict__ entropy,
                          double beta, double gamma, double lambda_d, float *__restrict__ omega,
                          float *__restrict__ dhat_out) {
  constexpr int kMaxM = 64;
  __shared__ double Dm[kMaxM], Rm[kMaxM];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int npairs = m * (m - 1) / 2;
  const double count = (double)h_q * t * t * (m - 1);
  for (int j = lane; j < m; j += 64) {
    double cs = 0.0;
    for (int h = 0; h < h_q; ++h) {
      const double *ps = pair_sum + ((long)b * h_q + h) * npairs;
      for (int c = 0; c < m; ++c) {
        if (c == j) continue;
        cs += ps[c < j ? traj_pair_index(c, j, m) : traj_pair_index(j, c, m)];
      }
    }
    Dm[j] = m > 1 ? 1.0 - cs / count : 0.0;
  }
  __syncthreads();
  double mu = 0.0;
  for (int j = 0; j < m; ++j) mu += Dm[j];
  mu /= m;
  double var = 0.0;
  for (int j = 0; j < m; ++j) var += (Dm[j] - mu) * (Dm[j] - mu);
  const double sd = sqrt(var / m);
  for (int j = lane; j < m; j += 64) {
    const double dh = sd < kStdFloor ? 0.0 : (Dm[j] - mu) / sd;
    double cbar = 0.0, hbar = 0.0;
    const long base = ((long)b * m + j) * t;
    for (int u = 0; u < t; ++u) {
      const double lp = logp[base + u], en = entropy[base + u];
      cbar += lp + en;
      hbar += en;
    }
    cbar /= t;
    hbar /= t;
    Rm[j] = beta * cbar - gamma * hbar - lambda_d * dh;
    if (dhat_out) dhat_out[(long)b * m + j] = (float)dh;
  }
  __syncthreads();
  double rmax = -DBL_MAX;
  for (int j = 0; j < m; ++j) rmax = fmax(rmax, Rm[j]);
  double z = 0.0;
  for (int j = 0; j < m; ++j) z += exp(Rm[j] - rmax);
  for (int j = lane; j < m; j += 64) omega[(long)b * m + j] = (float)(exp(Rm[j] - rmax) / z);
}

size_t reliability_ws_bytes(int batch, int h_q, int m) {
  return (size_t)batch * h_q * (size_t)(m * (m - 1) / 2) * sizeof(double);
}

hipError_t launch_reliability(int etype, const void *Q, int batch, int h_q, int nq, int d, int w,
                              int m, int t, const float *logp, const float *entropy, float beta,
                              float gamma, float lambda_d, float *omega, float *dhat,
                              double *pair_sum, hipStream_t st) {
  if (m < 1 || m > 64 || t < 1 || w + m * t > nq || nq > 64 || d < 1 || d > 128)
    return hipErrorInvalidValue;
  if (m > 1) {
    TimedLaunch tl_("traj_cosine", st);
    const dim3 grid(h_q, batch);
    if (etype == E_F32)
      hipLaunchKernelGGL(traj_cosine_kernel<float>, grid, dim3(kRelThreads), 0, st,
                         (const float *)Q, h_q, nq, d, w, m, t, pair_sum);
    else if (etype == E_BF16)
      hipLaunchKernelGGL(traj_cosine_kernel<bf16>, grid, dim3(kRelThreads), 0, st,
                         (const bf16 *)Q, h_q, nq, d, w, m, t, pair_sum);
    else
      hipLaunchKernelGGL(traj_cosine_kernel<f16>, grid, dim3(kRelThreads), 0, st,
                         (const f16 *)Q, h_q, nq, d, w, m, t, pair_sum);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    TimedLaunch tl_("reliability_finish", st);
    hipLaunchKernelGGL(reliability_finish_kernel, dim3(batch), dim3(64), 0, st, pair_sum, h_q, m,
                       t, logp, entropy, (double)beta, (double)gamma, (double)lambda_d, omega,
                       dhat);
  }
  return hipGetLastError();
}

}  // namespace kvs
