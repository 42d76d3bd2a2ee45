// Attention-output fidelity of a retained cache (LORE-KV page, "Why it
// works", "Output fidelity"): the cosine between each held-out query's
// attention output over the full cache and over the kept tokens, per query
// head, and its mean per sequence.  The two outputs come from the attention
// pass (attn.hip) run once on each cache; this file holds the cosine step.
#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace kvs {

constexpr int kCosWaves = 4;

// Grid (batch), kCosWaves waves.  Wave v takes rows v, v + kCosWaves, ... of
// the sequence's h_q * n_f rows; a row's three sums (o_f.o_k, |o_f|^2,
// |o_k|^2) are butterfly-reduced across the wave, so every lane holds the
// same totals and the result does not depend on scheduling.  Two zero outputs
// agree (cosine 1); one zero output gives 0.  The mean adds each wave's rows
// in order, then the waves in order.
template <int D>
__global__ void __launch_bounds__(64 * kCosWaves)
output_cosine_kernel(const float *__restrict__ Of, const float *__restrict__ Ok, int rows,
                     float *__restrict__ cos_out, float *__restrict__ fidelity) {
  constexpr int EPL = D / 64;  // elements per lane
  __shared__ float wsum[kCosWaves];
  const int b = blockIdx.x, lane = threadIdx.x % 64, wv = threadIdx.x / 64;
  const long base = (long)b * rows;
  float acc = 0.f;
  for (int r = wv; r < rows; r += kCosWaves) {
    const float *f = Of + (base + r) * D + lane * EPL;
    const float *k = Ok + (base + r) * D + lane * EPL;
    float dot = 0.f, ff = 0.f, kk = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      dot = fmaf(f[e], k[e], dot);
      ff = fmaf(f[e], f[e], ff);
      kk = fmaf(k[e], k[e], kk);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      dot += __shfl_xor(dot, o, 64);
      ff += __shfl_xor(ff, o, 64);
      kk += __shfl_xor(kk, o, 64);
    }
    float c;
    if (ff == 0.f && kk == 0.f) c = 1.f;
    else if (ff == 0.f || kk == 0.f) c = 0.f;
    else c = dot / sqrtf(ff * kk);
    if (lane == 0) cos_out[base + r] = c;
    acc += c;
  }
  if (lane == 0) wsum[wv] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float s = 0.f;
    for (int v = 0; v < kCosWaves; ++v) s += wsum[v];
    fidelity[b] = s / (float)rows;
  }
}

hipError_t launch_output_cosine(int d, const float *Of, const float *Ok, int batch, int rows,
                                float *cos_out, float *fidelity, hipStream_t st) {
  if (batch < 1 || rows < 1) return hipErrorInvalidValue;
  TimedLaunch tl_("output_cosine", st);
  if (d == 64)
    hipLaunchKernelGGL(output_cosine_kernel<64>, dim3(batch), dim3(64 * kCosWaves), 0, st, Of, Ok,
                       rows, cos_out, fidelity);
  else if (d == 128)
    hipLaunchKernelGGL(output_cosine_kernel<128>, dim3(batch), dim3(64 * kCosWaves), 0, st, Of,
                       Ok, rows, cos_out, fidelity);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvs
