// Per-KV-head top-B selection and cache compaction.
//
// LORE-KV ("Monte Carlo Estimation for KV-Cache Eviction", "Evict and decode",
// Eq. 8): each KV head keeps the protected set (attention sink + last w tokens)
// and its top-B tokens by score.  Adjacent-token grouping (chunk = 4 in the
// Hyperparameters table) is read as pooling: a candidate ranks by the mean
// score of the candidates in its aligned chunk, ties going to the lower index.
//
// Because every candidate of a chunk shares the pooled score, ranking tokens is
// ranking chunks weighted by their candidate count.  Each chunk's mean becomes
// an order-preserving 32-bit key.  Selection runs in two levels so a row is
// spread over many workgroups: every segment of kSeg chunks keeps the chunks
// whose key reaches the 16-bit bin of its own top-B threshold (a superset of the row's
// selection within that segment), then one workgroup per row runs a 4-pass
// 8-bit radix select with token-count weights over the surviving candidates
// to find the threshold key tau and how many tokens of the tau-chunks are
// still needed, and writes the selection in ascending index order with
// block-wide scans.
#include <atomic>
#include <mutex>

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
  const int x = wave_incl_scan(v);
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

// ---------------------------------------------------------------------------
// Weighted radix select over a list of items (item i: key(i), tokens cnt(i)):
// the largest key tau such that the items with key >= tau hold at least rem
// tokens, and how many tokens of the tau-items are still needed (*rem_out).
// The caller guarantees the list holds at least rem tokens.  hist holds
// nw * 256 ints (one histogram per wave: the high digits of nearby scores
// collide, and one shared histogram would serialise every atomic on one bin).
// With last_shift > 0 the select stops after the digit at last_shift: the
// result is the threshold's high bits, and keys >= it form a superset.
template <class KeyF, class CntF>
__device__ uint32_t radix_threshold(int n_items, KeyF key, CntF cnt, int rem, int *hist,
                                    uint32_t *s_prefix, int *s_rem, int *rem_out,
                                    int last_shift = 0) {
  const int tid = threadIdx.x, bs = blockDim.x;
  const int wv = tid >> 6, nw = bs >> 6;
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= last_shift; shift -= 8) {
    for (int i = tid; i < nw * 256; i += bs) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n_items; i += bs) {
      const int c = cnt(i);
      const uint32_t k = key(i);
      if (c > 0 && (k & mask) == prefix) atomicAdd(&hist[wv * 256 + ((k >> shift) & 255u)], c);
    }
    __syncthreads();
    for (int dg = tid; dg < 256; dg += bs) {
      int t = 0;
      for (int w2 = 0; w2 < nw; ++w2) t += hist[w2 * 256 + dg];
      hist[dg] = t;  // wave 0's bins now hold the totals
    }
    __syncthreads();
    if (tid < 64) {
      // wave 0 walks the 256 bins from the top: lane l owns bins 255-4l-j
      int hb[4], ltot = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hb[j] = hist[255 - 4 * tid - j];
        ltot += hb[j];
      }
      const int incl = wave_incl_scan(ltot);
      const int before = incl - ltot;  // tokens in bins above this lane's
      if (before < rem && incl >= rem) {
        int cum = before, sel = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (cum + hb[j] >= rem) {
            sel = 255 - 4 * tid - j;
            break;
          }
          cum += hb[j];
        }
        *s_prefix = prefix | ((uint32_t)sel << shift);
        *s_rem = rem - cum;
      }
    }
    __syncthreads();
    prefix = *s_prefix;
    rem = *s_rem;
    mask |= 255u << shift;
    __syncthreads();
  }
  *rem_out = rem;
  return prefix;
}

__device__ __forceinline__ int chunk_tokens(int cj, int chunk, int lo, int hi) {
  return min(cj * chunk + chunk, hi) - max(cj * chunk, lo);
}

// Level 1: one workgroup of 256 threads per (segment of kSeg chunks, row);
// thread t owns chunks 4t..4t+3 of the segment.  The workgroup pools its
// chunks from S (keys for the final pass, pooled scores when asked for), then
// keeps, in index order, the chunks whose key reaches the 16-bit bin of the
// segment's own top-B threshold (all of them when the segment holds at most
// B tokens).  A row of one segment (kept != nullptr) is selected here in
// full: the 4-digit threshold, then the kept list, as the final level would.
constexpr int kSeg = 1024;

__global__ void __launch_bounds__(256)
topb_local_kernel(const float *__restrict__ S, int n, int n_sink, int w, int chunk, int nchunks,
                  int B, int nseg, uint32_t *__restrict__ keys_ws, float *__restrict__ pooled,
                  int32_t *__restrict__ cand, int32_t *__restrict__ cand_n,
                  int32_t *__restrict__ kept, int n_keep) {
  __shared__ int hist[4 * 256];
  __shared__ int scan_sh[5];
  __shared__ uint32_t s_prefix;
  __shared__ int s_rem;
  __shared__ uint32_t seg_keys[kSeg];
  const int seg = blockIdx.x;
  const long row = blockIdx.y;
  const int lo = n_sink, hi = n - w;
  const int c0 = seg * kSeg;
  const int items = min(kSeg, nchunks - c0);
  const float *Sr = S + row * n;
  // pooling: chunk c holds tokens [c*chunk, c*chunk + chunk); its key is the
  // order key of the mean over its candidates (0 when it has none)
  int toks = 0;
  // Chunks of 4 tokens wholly inside the candidate range (all but the ones
  // at the sink and the window) are read as one 16-byte load each, the
  // thread's four loads issued together; the sum keeps the token order, so
  // the pooled value is the same as the general loop's.
  const int tt0 = (c0 + 4 * (int)threadIdx.x) * chunk;
  const bool whole4 = chunk == 4 && 4 * (int)threadIdx.x + 3 < items && tt0 >= lo &&
                      tt0 + 16 <= hi && ((reinterpret_cast<uintptr_t>(Sr + tt0) & 15) == 0) &&
                      (!pooled || (reinterpret_cast<uintptr_t>(pooled + row * n + tt0) & 15) == 0);
  if (whole4) {
    float4 sv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) sv[k] = reinterpret_cast<const float4 *>(Sr + tt0)[k];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * threadIdx.x + k;
      const float P = (((sv[k].x + sv[k].y) + sv[k].z) + sv[k].w) / 4.f;
      const uint32_t key = order_key(P);
      keys_ws[row * nchunks + c0 + i] = key;
      if (pooled)
        reinterpret_cast<float4 *>(pooled + row * n + tt0)[k] = make_float4(P, P, P, P);
      seg_keys[i] = key;
    }
    toks = 16;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (whole4) break;
    const int i = 4 * threadIdx.x + k;
    uint32_t key = 0;
    if (i < items) {
      const int cj = c0 + i;
      const int t0 = cj * chunk, t1 = min(t0 + chunk, n);
      const int a = max(t0, lo), e = min(t1, hi);
      float P = 0.f;
      if (e > a) {
        float sum = 0.f;
        for (int t = a; t < e; ++t) sum += Sr[t];
        P = sum / (float)(e - a);
        key = order_key(P);
        toks += e - a;
      }
      keys_ws[row * nchunks + cj] = key;
      if (pooled) {
        float *pr = pooled + row * n;
        for (int t = t0; t < t1; ++t) pr[t] = (t >= lo && t < hi) ? P : __int_as_float(0x7FC00000);
      }
    }
    seg_keys[i] = key;
  }
  if (kept) {
    // one segment holds the whole row: the protected entries, then the top B
    int32_t *kr = kept + row * n_keep;
    for (int i = threadIdx.x; i < n_sink; i += blockDim.x) kr[i] = i;
    for (int i = threadIdx.x; i < w; i += blockDim.x) kr[n_sink + max(B, 0) + i] = n - w + i;
    if (B <= 0) return;
    int total;
    block_exclusive_scan(toks, scan_sh, &total);  // (also orders the seg_keys writes)
    uint32_t tau = 0;
    int rem = 0;
    if (total > B)
      tau = radix_threshold(
          items, [&](int i) { return seg_keys[i]; },
          [&](int i) { return chunk_tokens(c0 + i, chunk, lo, hi); }, B, hist, &s_prefix, &s_rem,
          &rem);
    // in index order: chunks above tau whole, tau chunks until rem tokens
    // (ties to the lower index), as the final level emits them
    int cnt[4], tcnt = 0;
    uint32_t key[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * threadIdx.x + k;
      cnt[k] = i < items ? max(chunk_tokens(c0 + i, chunk, lo, hi), 0) : 0;
      key[k] = i < items ? seg_keys[i] : 0u;
      if (cnt[k] > 0 && key[k] == tau) tcnt += cnt[k];
    }
    int dummy;
    int tb = block_exclusive_scan(tcnt, scan_sh, &dummy);  // tau tokens before this thread
    int take[4], ntake = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      take[k] = 0;
      if (cnt[k] > 0) {
        if (key[k] > tau) {
          take[k] = cnt[k];
        } else if (key[k] == tau) {
          take[k] = min(max(rem - tb, 0), cnt[k]);
          tb += cnt[k];
        }
      }
      ntake += take[k];
    }
    int out = n_sink + block_exclusive_scan(ntake, scan_sh, &dummy);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int a = max((c0 + 4 * (int)threadIdx.x + k) * chunk, lo);
      for (int t = 0; t < take[k]; ++t, ++out)
        if (out < n_sink + B) kr[out] = a + t;
    }
    return;
  }
  if (B <= 0) return;  // nothing to select: the pooled output was the only work
  int total;
  block_exclusive_scan(toks, scan_sh, &total);  // (also orders the seg_keys writes)
  uint32_t tau = 0;
  if (total > B) {
    int rem_unused;
    // two 8-bit digits suffice here: every chunk at or above the 16-bit
    // threshold bin is kept, a superset the final select narrows exactly
    tau = radix_threshold(
        items, [&](int i) { return seg_keys[i]; },
        [&](int i) { return chunk_tokens(c0 + i, chunk, lo, hi); }, B, hist, &s_prefix, &s_rem,
        &rem_unused, 16);
  }
  int keep[4], nk = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * threadIdx.x + k;
    keep[k] = i < items && chunk_tokens(c0 + i, chunk, lo, hi) > 0 && seg_keys[i] >= tau;
    nk += keep[k];
  }
  int kept_total;
  int pos = block_exclusive_scan(nk, scan_sh, &kept_total);
  int32_t *out = cand + row * (long)nchunks + c0;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (keep[k]) out[pos++] = c0 + 4 * threadIdx.x + k;
  if (threadIdx.x == 0) cand_n[row * nseg + seg] = kept_total;
}

// Level 2: one workgroup per row over the candidates of all segments (staged
// in LDS when they fit, else the row's chunks are scanned directly).
constexpr int kCandLds = 12288;

__global__ void __launch_bounds__(1024)
topb_final_kernel(int n, int n_sink, int w, int chunk, int budget, int n_keep, int nchunks,
                  int nseg, const uint32_t *__restrict__ keys_ws,
                  const int32_t *__restrict__ cand, const int32_t *__restrict__ cand_n,
                  int32_t *__restrict__ kept) {
  __shared__ uint32_t c_key[kCandLds];
  __shared__ int32_t c_idx[kCandLds];
  __shared__ int hist[16 * 256];
  __shared__ int scan_sh[17];
  __shared__ int seg_at[1024], seg_cn[1024];
  __shared__ uint32_t s_prefix;
  __shared__ int s_rem;
  const int tid = threadIdx.x, bs = blockDim.x;
  const long row = blockIdx.x;
  const int lo = n_sink, hi = n - w;
  const int n_cand = hi - lo;
  const int B = min(budget, n_cand);
  int32_t *kr = kept + row * n_keep;

  for (int i = tid; i < n_sink; i += bs) kr[i] = i;
  for (int i = tid; i < w; i += bs) kr[n_sink + B + i] = n - w + i;
  if (B <= 0) return;

  const uint32_t *rk = keys_ws + row * nchunks;
  const int32_t *rc = cand + row * (long)nchunks;
  // gather the segments' candidate lists in order: a scan over the list
  // lengths gives each segment's offset, then 32 threads per segment copy
  // its list, so every load is one of a few independent rounds
  int total = 0;
  for (int base = 0; base < nseg; base += bs) {
    const int sg = base + tid;
    const int cn = sg < nseg ? cand_n[row * nseg + sg] : 0;
    int part;
    const int at = total + block_exclusive_scan(cn, scan_sh, &part);
    seg_at[tid] = at;
    seg_cn[tid] = cn;
    __syncthreads();
    const int nsg = min(bs, nseg - base);
    for (int k = tid >> 5; k < nsg; k += bs >> 5) {
      const int a0 = seg_at[k], c = seg_cn[k];
      if (a0 + c > kCandLds) continue;
      const int32_t *src = rc + (long)(base + k) * kSeg;
      for (int j = tid & 31; j < c; j += 32) {
        const int ci = src[j];
        c_idx[a0 + j] = ci;
        c_key[a0 + j] = rk[ci];
      }
    }
    __syncthreads();
    total += part;
  }
  const bool in_lds = total <= kCandLds;
  const int n_items = in_lds ? total : nchunks;
  auto idx_of = [&](int i) { return in_lds ? (int)c_idx[i] : i; };
  auto key_of = [&](int i) { return in_lds ? c_key[i] : rk[i]; };
  auto cnt_of = [&](int i) { return chunk_tokens(idx_of(i), chunk, lo, hi); };

  int rem;
  const uint32_t tau = radix_threshold(n_items, key_of, cnt_of, B, hist, &s_prefix, &s_rem, &rem);

  // Emit in ascending order.  Wave v owns the contiguous item range
  // [v*per, (v+1)*per), walked 64 items at a time (one per lane);
  // tau-items are taken in index order until rem tokens, using in-wave prefix
  // sums and block scans over the wave totals.
  const int lane = tid & 63, wv = tid >> 6, nw = bs >> 6;
  const int per = ((n_items + nw - 1) / nw + 63) / 64 * 64;
  const int c_lo = min(n_items, wv * per), c_hi = min(n_items, c_lo + per);
  auto wave_incl = [&](int x) { return wave_incl_scan(x); };
  auto last_lane = [&](int x) { return __builtin_amdgcn_readlane(x, 63); };
  // pass 1: tau-tokens per wave
  int ties = 0;
  for (int base = c_lo; base < c_hi; base += 64) {
    const int it = base + lane;
    if (it < c_hi) {
      const int cnt = cnt_of(it);
      if (cnt > 0 && key_of(it) == tau) ties += cnt;
    }
  }
  ties = last_lane(wave_incl(ties));
  int tot;
  const int tie_before_wave = block_exclusive_scan(lane == 0 ? ties : 0, scan_sh, &tot);
  const int tie_wave0 = __builtin_amdgcn_readlane(tie_before_wave, 0);
  // pass 2: selected tokens per wave
  int sel = 0, tie_run = tie_wave0;
  for (int base = c_lo; base < c_hi; base += 64) {
    const int it = base + lane;
    int cnt = 0, tcnt = 0;
    uint32_t key = 0;
    if (it < c_hi) {
      cnt = max(cnt_of(it), 0);
      key = key_of(it);
      tcnt = (cnt > 0 && key == tau) ? cnt : 0;
    }
    const int tincl = wave_incl(tcnt);
    const int tb = tie_run + tincl - tcnt;  // tau-tokens before this item
    if (cnt > 0) {
      if (key > tau) sel += cnt;
      else if (key == tau) sel += min(max(rem - tb, 0), cnt);
    }
    tie_run += last_lane(tincl);
  }
  sel = last_lane(wave_incl(sel));
  const int out_before_wave = block_exclusive_scan(lane == 0 ? sel : 0, scan_sh, &tot);
  int out_run = n_sink + __builtin_amdgcn_readlane(out_before_wave, 0);
  // pass 3: write
  tie_run = tie_wave0;
  for (int base = c_lo; base < c_hi; base += 64) {
    const int it = base + lane;
    int cnt = 0, tcnt = 0, a = 0;
    uint32_t key = 0;
    if (it < c_hi) {
      const int cj = idx_of(it);
      cnt = max(chunk_tokens(cj, chunk, lo, hi), 0);
      a = max(cj * chunk, lo);
      key = key_of(it);
      tcnt = (cnt > 0 && key == tau) ? cnt : 0;
    }
    const int tincl = wave_incl(tcnt);
    const int tb = tie_run + tincl - tcnt;
    int take = 0;
    if (cnt > 0) {
      if (key > tau) take = cnt;
      else if (key == tau) take = min(max(rem - tb, 0), cnt);
    }
    const int oincl = wave_incl(take);
    int out = out_run + oincl - take;
    for (int i = a; i < a + take; ++i, ++out)
      if (out < n_sink + B) kr[out] = i;
    out_run += last_lane(oincl);
    tie_run += last_lane(tincl);
  }
}

size_t topb_workspace_bytes(int rows, int n, int chunk) {
  const size_t nchunks = ((size_t)n + chunk - 1) / chunk;
  const size_t nseg = (nchunks + kSeg - 1) / kSeg;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return al((size_t)rows * nchunks * 4) + al((size_t)rows * nchunks * 4) + al((size_t)rows * nseg * 4);
}

hipError_t launch_topb(const float *S, int rows, int n, int n_sink, int w, int chunk, int budget,
                       int n_keep, void *ws, int32_t *kept, float *pooled, hipStream_t st) {
  const int nchunks = (n + chunk - 1) / chunk;
  const int nseg = (nchunks + kSeg - 1) / kSeg;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  uint32_t *keys_ws = static_cast<uint32_t *>(ws);
  int32_t *cand = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + al((size_t)rows * nchunks * 4));
  int32_t *cand_n = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + 2 * al((size_t)rows * nchunks * 4));
  const int n_cand = n - n_sink - w;
  const int B = budget < n_cand ? budget : n_cand;
  // a row of one segment is selected in full by the first level
  const bool one = nseg == 1;
  {
    TimedLaunch tl_("topb_local", st);
    hipLaunchKernelGGL(topb_local_kernel, dim3(nseg, rows), dim3(256), 0, st, S, n, n_sink, w,
                       chunk, nchunks, B, nseg, keys_ws, pooled, cand, cand_n,
                       one ? kept : nullptr, n_keep);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || one) return e;
  {
    TimedLaunch tl_("topb_select", st);
    hipLaunchKernelGGL(topb_final_kernel, dim3(rows), dim3(1024), 0, st, n, n_sink, w, chunk,
                       budget, n_keep, nchunks, nseg, keys_ws, cand, cand_n, kept);
  }
  return hipGetLastError();
}

// Retention-order shift (LORE-KV page, "More analyses"): per row, the
// candidates [n_sink, n - w) that kept list A holds and kept list B does
// not, as a fraction of A's candidates (0 when A has none).  One workgroup
// per row; B is ascending (as kvscore_topb_select writes it), so each of A's
// candidates is looked up by a binary search over B (bounded by n_keep
// steps whatever B holds).
__global__ void __launch_bounds__(256)
retention_shift_kernel(const int32_t *__restrict__ ka, const int32_t *__restrict__ kb,
                       int n_keep, int n_sink, int w, int n, float *__restrict__ shift) {
  __shared__ int scan_sh[5];
  const long row = blockIdx.x;
  const int32_t *a = ka + row * n_keep;
  const int32_t *b = kb + row * n_keep;
  int miss = 0, cnt = 0;
  for (int i = threadIdx.x; i < n_keep; i += blockDim.x) {
    const int x = a[i];
    if (x < n_sink || x >= n - w) continue;
    ++cnt;
    int lo = 0, hi = n_keep;  // first position of B holding a value >= x
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (b[mid] < x) lo = mid + 1;
      else hi = mid;
    }
    miss += (lo < n_keep && b[lo] == x) ? 0 : 1;
  }
  int miss_total, cnt_total;
  block_exclusive_scan(miss, scan_sh, &miss_total);
  block_exclusive_scan(cnt, scan_sh, &cnt_total);
  if (threadIdx.x == 0) shift[row] = cnt_total > 0 ? (float)miss_total / (float)cnt_total : 0.f;
}

hipError_t launch_retention_shift(int rows, int n_keep, int n_sink, int w, int n,
                                  const int32_t *kept_a, const int32_t *kept_b, float *shift,
                                  hipStream_t st) {
  {
    TimedLaunch tl_("retention_shift", st);
    hipLaunchKernelGGL(retention_shift_kernel, dim3(rows), dim3(256), 0, st, kept_a, kept_b,
                       n_keep, n_sink, w, n, shift);
  }
  return hipGetLastError();
}

// Scratch of the allocation-free selection (kvscore_topb_select_noalloc): the
// level-1 chunk keys, candidate lists and counts that kvscore_topb_select
// otherwise takes from the caller's workspace.  A file-scope device array, so
// every GPU the library runs on holds its own copy from the code object's
// load until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is taken once per device
// with hipGetSymbolAddress (that device current) and only that address is
// ever passed to a kernel.  Every launch writes each scratch entry it reads
// earlier in the same call (keys of every chunk, the lists up to their
// counts, the counts of every segment), so nothing needs clearing between
// calls; calls that overlap on one GPU share the array and race.
static __device__ __align__(256) uint8_t scratch[kTopbScratchBytes];

hipError_t topb_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void *> addr[kMaxDevices];
  static std::mutex mu;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

// Compaction: K'[row][r] = K[row][kept[r]] (and V), 16 bytes per thread.
// Rows share kept lists in groups of kept_div (1: one list per row; the head
// count: one token-level list per sequence).  pos_out and the 32-bit payload
// (scores, or token ids) follow the kept list: one entry per list, written by
// the first row of its group.
__global__ void __launch_bounds__(256)
compact_kernel(const uint8_t *__restrict__ K, const uint8_t *__restrict__ V,
               const int32_t *__restrict__ kept, int kept_div, int n_src, int n_keep, int cap,
               int cpr, uint8_t *__restrict__ Ko, uint8_t *__restrict__ Vo,
               int32_t *__restrict__ pos_out, const uint32_t *__restrict__ pin,
               uint32_t *__restrict__ pout) {
  const long row = blockIdx.y;
  const long krow = row / kept_div;
  const bool lead = row % kept_div == 0;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int r = (int)(idx / cpr), c = (int)(idx % cpr);
  if (r >= cap) return;
  const long rb = (long)cpr * 16;
  const int src = r < n_keep ? kept[krow * n_keep + r] : -1;
  if (src >= 0 && src < n_src) {
    const long so = (row * n_src + src) * rb + c * 16;
    const long dof = (row * cap + r) * rb + c * 16;
    *reinterpret_cast<U128 *>(Ko + dof) = *reinterpret_cast<const U128 *>(K + so);
    *reinterpret_cast<U128 *>(Vo + dof) = *reinterpret_cast<const U128 *>(V + so);
    if (c == 0 && lead) {
      if (pos_out) pos_out[krow * cap + r] = src;
      if (pout) pout[krow * cap + r] = pin[krow * n_src + src];
    }
  } else if (c == 0 && lead) {  // beyond n_keep, or an index outside [0, n_src): nothing copied
    if (pos_out) pos_out[krow * cap + r] = -1;
    if (pout) pout[krow * cap + r] = 0u;
  }
}

hipError_t launch_compact(int rows, int n_src, int n_keep, int cap_dst, int row_bytes,
                          const void *K, const void *V, const int32_t *kept, void *K_out,
                          void *V_out, int32_t *pos_out, const void *payload_in,
                          void *payload_out, hipStream_t st, int kept_div) {
  const int cpr = row_bytes / 16;
  const long threads = (long)cap_dst * cpr;
  const int blocks = (int)((threads + 255) / 256);
  if (blocks == 0 || rows == 0) return hipSuccess;
  if (kept_div < 1 || rows % kept_div != 0) return hipErrorInvalidValue;
  {
    TimedLaunch tl_("compact", st);
    hipLaunchKernelGGL(compact_kernel, dim3(blocks, rows), dim3(256), 0, st, (const uint8_t *)K,
                       (const uint8_t *)V, kept, kept_div, n_src, n_keep, cap_dst, cpr,
                       (uint8_t *)K_out, (uint8_t *)V_out, pos_out, (const uint32_t *)payload_in,
                       (uint32_t *)payload_out);
  }
  return hipGetLastError();
}

}  // namespace kvs
