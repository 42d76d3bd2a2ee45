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

// Grid (ceil(rows / kCosWaves), batch), kCosWaves waves, one row per wave.
// The row's three sums (o_f.o_k, |o_f|^2, |o_k|^2) are butterfly-reduced
// across the wave, so every lane holds the same totals and the result does
// not depend on scheduling.  Two zero outputs agree (cosine 1); one zero
// output gives 0.
template <int D>
__global__ void __launch_bounds__(64 * kCosWaves)
output_cosine_kernel(const float *__restrict__ Of, const float *__restrict__ Ok, int rows,
                     float *__restrict__ cos_out) {
  constexpr int EPL = D / 64;  // elements per lane
  const int lane = threadIdx.x % 64;
  const int r = blockIdx.x * kCosWaves + threadIdx.x / 64;
  if (r >= rows) return;  // whole waves leave together
  const long row = (long)blockIdx.y * rows + r;
  const float *f = Of + row * D + lane * EPL;
  const float *k = Ok + row * D + lane * EPL;
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
  if (lane == 0) cos_out[row] = c;
}

// Grid (batch), 256 threads: the mean of a sequence's cosines.  Thread i adds
// rows i, i + 256, ... in order, then a fixed tree over the threads.
__global__ void __launch_bounds__(256)
cosine_mean_kernel(const float *__restrict__ cos_in, int rows, float *__restrict__ fidelity) {
  __shared__ float part[256];
  const float *c = cos_in + (long)blockIdx.x * rows;
  float s = 0.f;
  for (int r = threadIdx.x; r < rows; r += 256) s += c[r];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) fidelity[blockIdx.x] = part[0] / (float)rows;
}

hipError_t launch_output_cosine(int d, const float *Of, const float *Ok, int batch, int rows,
                                float *cos_out, float *fidelity, hipStream_t st) {
  if (batch < 1 || rows < 1 || (d != 64 && d != 128)) return hipErrorInvalidValue;
  {
    TimedLaunch tl_("output_cosine", st);
    const dim3 grid((rows + kCosWaves - 1) / kCosWaves, batch);
    if (d == 64)
      hipLaunchKernelGGL(output_cosine_kernel<64>, grid, dim3(64 * kCosWaves), 0, st, Of, Ok, rows,
                         cos_out);
    else
      hipLaunchKernelGGL(output_cosine_kernel<128>, grid, dim3(64 * kCosWaves), 0, st, Of, Ok,
                         rows, cos_out);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    TimedLaunch tl_("cosine_mean", st);
    hipLaunchKernelGGL(cosine_mean_kernel, dim3(batch), dim3(256), 0, st, cos_out, rows,
                       fidelity);
  }
  return hipGetLastError();
}

}  // namespace kvs
