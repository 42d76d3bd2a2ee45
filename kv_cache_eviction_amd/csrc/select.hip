// Per-KV-head top-B selection and cache compaction.
//
// LORE-KV ("Monte Carlo Estimation for KV-Cache Eviction", "Evict and decode",
// Eq. 8): each KV head keeps the protected set (attention sink + last w tokens)
// and its top-B tokens by score.  Adjacent-token grouping (chunk = 4 in the
// Hyperparameters table) is read as pooling: a candidate ranks by the mean
// score of the candidates in its aligned chunk, ties going to the lower index.
//
// Because every candidate of a chunk shares the pooled score, ranking tokens is
// ranking chunks weighted by their candidate count: one workgroup per row
// turns each chunk's mean into an order-preserving 32-bit key, runs a 4-pass
// 8-bit radix select with token-count weights to find the threshold key tau
// and how many tokens of the tau-chunks are still needed, then writes the
// selection in ascending index order with two block-wide scans.
#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace kvs {

// Larger float -> larger key; NaN above everything.
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0xFFFFFFFFu;
  const uint32_t u = __float_as_uint(x + 0.0f);  // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the block (blockDim.x a multiple of 64, <= 1024).
__device__ int block_exclusive_scan(int v, int *sh, int *total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wid] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int t = sh[w];
      sh[w] = run;
      run += t;
    }
    sh[nw] = run;
  }
  __syncthreads();
  const int excl = sh[wid] + x - v;
  *total = sh[nw];
  __syncthreads();
  return excl;
}

__global__ void __launch_bounds__(1024)
topb_kernel(const float *__restrict__ S, int n, int n_sink, int w, int chunk, int budget,
            int n_keep, uint32_t *__restrict__ keys_ws, int32_t *__restrict__ kept,
            float *__restrict__ pooled) {
  __shared__ int hist[256];
  __shared__ int scan_sh[17];
  __shared__ uint32_t s_prefix;
  __shared__ int s_rem;
  const int tid = threadIdx.x, bs = blockDim.x;
  const long row = blockIdx.x;
  const float *Sr = S + row * n;
  const int lo = n_sink, hi = n - w;
  const int n_cand = hi - lo;
  const int B = min(budget, n_cand);
  const int nchunks = (n + chunk - 1) / chunk;
  uint32_t *keys = keys_ws + row * nchunks;
  int32_t *kr = kept + row * n_keep;
  float *pr = pooled ? pooled + row * n : nullptr;

  for (int i = tid; i < n_sink; i += bs) kr[i] = i;
  for (int i = tid; i < w; i += bs) kr[n_sink + B + i] = n - w + i;
  if (pr) {
    for (int i = tid; i < lo; i += bs) pr[i] = __int_as_float(0x7FC00000);
    for (int i = hi + tid; i < n; i += bs) pr[i] = __int_as_float(0x7FC00000);
  }
  for (int cj = tid; cj < nchunks; cj += bs) {
    const int a = max(cj * chunk, lo), e = min(cj * chunk + chunk, hi);
    uint32_t key = 0;
    if (e > a) {
      float s = 0.f;
      for (int i = a; i < e; ++i) s += Sr[i];
      const float P = s / (float)(e - a);
      key = order_key(P);
      if (pr)
        for (int i = a; i < e; ++i) pr[i] = P;
    }
    keys[cj] = key;
  }
  if (B <= 0) return;
  __syncthreads();

  uint32_t prefix = 0, mask = 0;
  int rem = B;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += bs) hist[i] = 0;
    __syncthreads();
    for (int cj = tid; cj < nchunks; cj += bs) {
      const int cnt = min(cj * chunk + chunk, hi) - max(cj * chunk, lo);
      if (cnt <= 0) continue;
      const uint32_t key = keys[cj];
      if ((key & mask) != prefix) continue;
      atomicAdd(&hist[(key >> shift) & 255u], cnt);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, sel = 0;
      for (int dg = 255; dg >= 0; --dg) {
        if (cum + hist[dg] >= rem) {
          sel = dg;
          break;
        }
        cum += hist[dg];
      }
      s_prefix = prefix | ((uint32_t)sel << shift);
      s_rem = rem - cum;
    }
    __syncthreads();
    prefix = s_prefix;
    rem = s_rem;
    mask |= 255u << shift;
  }
  const uint32_t tau = prefix;

  const int per = (nchunks + bs - 1) / bs;
  const int c_lo = min(nchunks, tid * per), c_hi = min(nchunks, c_lo + per);
  int ties = 0;
  for (int cj = c_lo; cj < c_hi; ++cj) {
    const int cnt = min(cj * chunk + chunk, hi) - max(cj * chunk, lo);
    if (cnt > 0 && keys[cj] == tau) ties += cnt;
  }
  int total;
  const int tie_before = block_exclusive_scan(ties, scan_sh, &total);
  int sel = 0, tb = tie_before;
  for (int cj = c_lo; cj < c_hi; ++cj) {
    const int cnt = min(cj * chunk + chunk, hi) - max(cj * chunk, lo);
    if (cnt <= 0) continue;
    const uint32_t key = keys[cj];
    if (key > tau) {
      sel += cnt;
    } else if (key == tau) {
      sel += min(max(rem - tb, 0), cnt);
      tb += cnt;
    }
  }
  int out = n_sink + block_exclusive_scan(sel, scan_sh, &total);
  tb = tie_before;
  for (int cj = c_lo; cj < c_hi; ++cj) {
    const int a = max(cj * chunk, lo), e = min(cj * chunk + chunk, hi);
    const int cnt = e - a;
    if (cnt <= 0) continue;
    const uint32_t key = keys[cj];
    int take = 0;
    if (key > tau) {
      take = cnt;
    } else if (key == tau) {
      take = min(max(rem - tb, 0), cnt);
      tb += cnt;
    }
    for (int i = a; i < a + take; ++i, ++out)
      if (out < n_sink + B) kr[out] = i;
  }
}

hipError_t launch_topb(const float *S, int rows, int n, int n_sink, int w, int chunk, int budget,
                       int n_keep, uint32_t *keys_ws, int32_t *kept, float *pooled,
                       hipStream_t st) {
  {
    TimedLaunch tl_("topb_select", st);
    hipLaunchKernelGGL(topb_kernel, dim3(rows), dim3(1024), 0, st, S, n, n_sink, w, chunk, budget,
                       n_keep, keys_ws, kept, pooled);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Compaction: K'[row][r] = K[row][kept[r]] (and V), 16 bytes per thread.
__global__ void __launch_bounds__(256)
compact_kernel(const uint8_t *__restrict__ K, const uint8_t *__restrict__ V,
               const int32_t *__restrict__ kept, int n_src, int n_keep, int cap, int cpr,
               uint8_t *__restrict__ Ko, uint8_t *__restrict__ Vo, int32_t *__restrict__ pos_out,
               const float *__restrict__ sin, float *__restrict__ sout) {
  const long row = blockIdx.y;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int r = (int)(idx / cpr), c = (int)(idx % cpr);
  if (r >= cap) return;
  const long rb = (long)cpr * 16;
  const int src = r < n_keep ? kept[row * n_keep + r] : -1;
  if (src >= 0 && src < n_src) {
    const long so = (row * n_src + src) * rb + c * 16;
    const long dof = (row * cap + r) * rb + c * 16;
    *reinterpret_cast<U128 *>(Ko + dof) = *reinterpret_cast<const U128 *>(K + so);
    *reinterpret_cast<U128 *>(Vo + dof) = *reinterpret_cast<const U128 *>(V + so);
    if (c == 0) {
      if (pos_out) pos_out[row * cap + r] = src;
      if (sout) sout[row * cap + r] = sin[row * n_src + src];
    }
  } else if (c == 0) {  // beyond n_keep, or an index outside [0, n_src): nothing copied
    if (pos_out) pos_out[row * cap + r] = -1;
    if (sout) sout[row * cap + r] = 0.f;
  }
}

hipError_t launch_compact(int rows, int n_src, int n_keep, int cap_dst, int row_bytes,
                          const void *K, const void *V, const int32_t *kept, void *K_out,
                          void *V_out, int32_t *pos_out, const float *score_in,
                          float *score_out, hipStream_t st) {
  const int cpr = row_bytes / 16;
  const long threads = (long)cap_dst * cpr;
  const int blocks = (int)((threads + 255) / 256);
  if (blocks == 0 || rows == 0) return hipSuccess;
  {
    TimedLaunch tl_("compact", st);
    hipLaunchKernelGGL(compact_kernel, dim3(blocks, rows), dim3(256), 0, st, (const uint8_t *)K,
                       (const uint8_t *)V, kept, n_src, n_keep, cap_dst, cpr, (uint8_t *)K_out,
                       (uint8_t *)V_out, pos_out, score_in, score_out);
  }
  return hipGetLastError();
}

}  // namespace kvs
