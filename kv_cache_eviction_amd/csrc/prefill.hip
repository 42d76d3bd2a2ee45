// H2O prefill accumulate for 16-bit prompts (H2O page, 3.4 "Handling the
// prefill phase": every prompt token's accumulated score is the attention the
// causal prompt rows give it).  Two passes over the causal triangle of each
// (sequence, head), c = log2(e) / sqrt(d):
//   rows:   beta2_r = m_r + log2 sum_{j <= r} 2^(s_rj c - m_r), m_r = max_{j <= r} s_rj c,
//           stored as the row constants (beta2, 0, 1, last = r);
//   colsum: acc_i = sum_{r >= i} 2^(s_ri c - beta2_r).
// The triangle has nb = ceil(P/64) blocks of 64 rows; row block v meets key
// tiles 0..v.  A workgroup takes the pair of blocks (p, nb-1-p), which holds
// nb + 1 block-tile products for every p, and each of its four waves takes 16
// rows (rows pass) or 16 keys (colsum pass) of both blocks, so waves and
// workgroups carry equal work.  The pairs of one (sequence, head) are placed
// on one XCD (workgroups go to the eight XCDs in turn), so the K tiles (rows
// pass) or Q blocks (colsum pass) they share are read from that XCD's L2.
// Tiles are staged in LDS, double-buffered: the next tile's loads are in
// flight while the current one is computed.
#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

#include <type_traits>

namespace kvs {

namespace {

// Logical block of this workgroup when consecutive logical blocks should share
// an XCD: hardware block L runs on XCD L % 8, so XCD x takes the contiguous
// logical range x * (nblk_pad / 8) + [0, nblk_pad / 8).
__device__ __forceinline__ int xcd_block(int nblk_pad) {
  const int L = blockIdx.x;
  return (L & 7) * (nblk_pad >> 3) + (L >> 3);
}

constexpr float kNegBig = -1e30f;  // finite start of a running maximum


template <bool B> using Bool = std::integral_constant<bool, B>;

// 64 rows of one (sequence, head) staged as 16-bit LDS rows padded by 32
// bytes (conflict-free 16-byte fragment reads of 16 consecutive rows).
template <typename Tin, int D>
struct Tile {
  static constexpr int TN = 64;
  static constexpr int EPC = 8;  // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;
  static constexpr int ROW = D + 16;
  static constexpr int PF = TN * CPR / 256;  // chunks per thread (256 threads)
  U128 r[PF];
  // rows 64 blk .. 64 blk + 63; rows past the resource's range read zeros
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int blk) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int idx = threadIdx.x + u * 256;
      const int row = idx / CPR, ch = idx % CPR;
      r[u] = buf_load16(rs, (uint32_t)((blk * TN + row) * D + ch * EPC) * (uint32_t)sizeof(Tin));
    }
  }
  __device__ __forceinline__ void store(Tin *lds) const {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int idx = threadIdx.x + u * 256;
      const int row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<U128 *>(&lds[row * ROW + ch * EPC]) = r[u];
    }
  }
};

}  // namespace

// Rows pass.  Logits are formed transposed (S^T = K Q^T, keys across the
// MFMA rows): a lane owns one query row and four keys of each 16-key block,
// so its running maximum and sum stay in registers; the four lanes of a row
// are merged once at the end.
template <typename Tin, int D>
__global__ void __launch_bounds__(256)
prefill_rows_kernel(const Tin *__restrict__ Q, const Tin *__restrict__ K, int P, int bh_count,
                    int npairs, int nblk_pad, float4 *__restrict__ consts) {
  typedef typename FragOf<Tin>::type FQ;
  typedef Tile<Tin, D> T;
  constexpr int KS = D / 32;
  __shared__ __align__(16) Tin Ks[2][T::TN * T::ROW];

  const int blk = xcd_block(nblk_pad);
  if (blk >= bh_count * npairs) return;  // (workgroup-uniform)
  const int bh = blk / npairs, p = blk % npairs;
  const int nb = (P + 63) / 64;
  const int vb[2] = {p, nb - 1 - p};
  const bool two = vb[1] != vb[0];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const Tin *Qh = Q + (long)bh * P * D;
  const Tin *Kh = K + (long)bh * P * D;
  const float c = kLog2e * rsqrtf((float)D);

  // B fragments: query row 64 vb[qb] + 16 wv + col
  FQ qf[2][KS];
  int row[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    row[qb] = 64 * vb[qb] + 16 * wv + col;
    const bool valid = row[qb] < P && (qb == 0 || two);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[qb][ks] = valid ? load8<Tin>(Qh + (long)row[qb] * D + ks * 32 + 8 * grp) : zero8<Tin>();
  }
  float m[2] = {kNegBig, kNegBig}, l[2] = {0.f, 0.f};

  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh, (uint32_t)P * D * (uint32_t)sizeof(Tin));
  T pk;
  wait_vmem_all();
  pk.load(rk, 0);
  pk.store(Ks[0]);
  __syncthreads();
  const int nt = vb[1] + 1;
  for (int t = 0; t < nt; ++t) {
    const int cur = t & 1;
    if (t + 1 < nt) pk.load(rk, t + 1);
    const Tin *kt = Ks[cur];
    // Row block vb[0] meets tiles 0..vb[0], block vb[1] every tile of the
    // loop; a block's own tile (the diagonal) hides the keys past each row.
    // Each combination is its own compiled body (wave-uniform dispatch).
    auto body = [&](auto use0, auto use1, auto diag0, auto diag1) {
      constexpr bool U[2] = {decltype(use0)::value, decltype(use1)::value};
      constexpr bool DG[2] = {decltype(diag0)::value, decltype(diag1)::value};
      // each 16-key block's K fragments are read from LDS once for both row
      // blocks, one block ahead of the products that use them
      f32x4 sc[2][4];
      FQ kb[2][KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[0][ks] = load8<Tin>(&kt[col * T::ROW + ks * 32 + 8 * grp]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        if (tb + 1 < 4) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            kb[(tb + 1) & 1][ks] = load8<Tin>(&kt[((tb + 1) * 16 + col) * T::ROW + ks * 32 + 8 * grp]);
        }
        sched_fence();
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (!U[qb]) continue;
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) a = mma(kb[tb & 1][ks], qf[qb][ks], a);
          sc[qb][tb] = a;
        }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (!U[qb]) continue;
        if (DG[qb]) {
#pragma unroll
          for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (t * 64 + tb * 16 + 4 * grp + j > row[qb]) sc[qb][tb][j] = -INFINITY;
        }
        // c > 0, so the maximum is taken on the raw logits
        float mx = max2(sc[qb][0][0], sc[qb][0][1]);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int j = (tb == 0 ? 2 : 0); j < 4; ++j) mx = max2(mx, sc[qb][tb][j]);
        const float mn = max2(m[qb], mx * c);
        float sum = hw_exp2(fmaf(sc[qb][0][0], c, -mn));
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
          for (int j = (tb == 0 ? 1 : 0); j < 4; ++j) sum += hw_exp2(fmaf(sc[qb][tb][j], c, -mn));
        l[qb] = fmaf(l[qb], hw_exp2(m[qb] - mn), sum);
        m[qb] = mn;
      }
    };
    if (t < vb[0]) {
      if (two) body(Bool<true>{}, Bool<true>{}, Bool<false>{}, Bool<false>{});
      else body(Bool<true>{}, Bool<false>{}, Bool<false>{}, Bool<false>{});
    } else if (t == vb[0]) {
      if (two) body(Bool<true>{}, Bool<true>{}, Bool<true>{}, Bool<false>{});
      else body(Bool<true>{}, Bool<false>{}, Bool<true>{}, Bool<false>{});
    } else if (t < vb[1]) {
      body(Bool<false>{}, Bool<true>{}, Bool<false>{}, Bool<false>{});
    } else {
      body(Bool<false>{}, Bool<true>{}, Bool<false>{}, Bool<true>{});
    }
    if (t + 1 < nt) pk.store(Ks[cur ^ 1]);
    __syncthreads();
  }
  // merge the four lanes (grp) of each row; rows past the prompt keep no keys
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float M = group4_max(m[qb]);
    const float L = group4_sum(l[qb] * hw_exp2(m[qb] - M));
    if (grp == 0 && (qb == 0 || two)) {
      const bool ok = row[qb] < P;
      consts[((long)bh * nb + vb[qb]) * 64 + 16 * wv + col] =
          make_float4(ok ? M + log2f(L) : 0.f, 0.f, 1.f, __int_as_float(ok ? row[qb] : -1));
    }
  }
}

// Column-sum pass.  S = Q K^T with the keys across the MFMA columns: a lane
// owns one key (its K fragments stay in registers for the whole pass) and
// four rows of each 16-row block, so the sum over rows is in-lane; row blocks
// of Q and their constants are staged in LDS.  Rows are added in a fixed
// order (deterministic).
template <typename Tin, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4)))
prefill_colsum_kernel(const Tin *__restrict__ Q, const Tin *__restrict__ K,
                      const float4 *__restrict__ consts, int P, int bh_count, int npairs,
                      int nblk_pad, float *__restrict__ acc) {
  typedef typename FragOf<Tin>::type FQ;
  typedef Tile<Tin, D> T;
  constexpr int KS = D / 32;
  __shared__ __align__(16) Tin Qs[2][T::TN * T::ROW];
  __shared__ __align__(16) float bs[2][64];
  __shared__ __align__(16) int ls[2][64];

  const int blk = xcd_block(nblk_pad);
  if (blk >= bh_count * npairs) return;  // (workgroup-uniform)
  const int bh = blk / npairs, p = blk % npairs;
  const int nb = (P + 63) / 64;
  const int tt[2] = {p, nb - 1 - p};
  const bool two = tt[1] != tt[0];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const Tin *Qh = Q + (long)bh * P * D;
  const Tin *Kh = K + (long)bh * P * D;
  const float4 *ch = consts + (long)bh * nb * 64;
  const float c = kLog2e * rsqrtf((float)D);

  // B fragments: key 64 tt[tb] + 16 wv + col
  FQ kf[2][KS];
  int tok[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    tok[tb] = 64 * tt[tb] + 16 * wv + col;
    const bool valid = tok[tb] < P && (tb == 0 || two);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[tb][ks] = valid ? load8<Tin>(Kh + (long)tok[tb] * D + ks * 32 + 8 * grp) : zero8<Tin>();
  }
  float cs[2] = {0.f, 0.f};

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qh, (uint32_t)P * D * (uint32_t)sizeof(Tin));
  T pq;
  float4 pc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto prefetch = [&](int v) {
    pq.load(rq, v);
    if (threadIdx.x < 64) pc = ch[v * 64 + threadIdx.x];
  };
  auto stash = [&](int buf) {
    pq.store(Qs[buf]);
    if (threadIdx.x < 64) {
      bs[buf][threadIdx.x] = pc.x;
      ls[buf][threadIdx.x] = __float_as_int(pc.w);
    }
  };
  wait_vmem_all();
  prefetch(tt[0]);
  stash(0);
  __syncthreads();
  for (int v = tt[0]; v < nb; ++v) {
    const int cur = (v - tt[0]) & 1;
    if (v + 1 < nb) prefetch(v + 1);
    const Tin *qt = Qs[cur];
    // Key tile tt[0] meets row blocks tt[0]..nb-1, tile tt[1] blocks
    // tt[1]..nb-1; a tile's diagonal block and the last (possibly ragged)
    // block are masked.  Each combination is its own compiled body.
    auto body = [&](auto use1, auto mask0, auto mask1) {
      constexpr bool U1 = decltype(use1)::value;
      constexpr bool MK[2] = {decltype(mask0)::value, decltype(mask1)::value};
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        FQ qa[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[ks] = load8<Tin>(&qt[(qb * 16 + col) * T::ROW + ks * 32 + 8 * grp]);
        const float4 be = *reinterpret_cast<const float4 *>(&bs[cur][qb * 16 + 4 * grp]);
        const float bt[4] = {be.x, be.y, be.z, be.w};
        int lt[4] = {0, 0, 0, 0};
        if (MK[0] || MK[1]) {
          const int4 la = *reinterpret_cast<const int4 *>(&ls[cur][qb * 16 + 4 * grp]);
          lt[0] = la.x; lt[1] = la.y; lt[2] = la.z; lt[3] = la.w;
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          if (tb == 1 && !U1) continue;
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) a = mma(qa[ks], kf[tb][ks], a);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float e = fmaf(a[j], c, -bt[j]);
            if (MK[tb] && tok[tb] > lt[j]) e = -INFINITY;
            cs[tb] += hw_exp2(e);
          }
        }
      }
    };
    const bool use1 = two && v >= tt[1];
    const bool m0 = v == tt[0] || v == nb - 1;
    const bool m1 = v == tt[1] || v == nb - 1;
    if (!use1) {
      if (m0) body(Bool<false>{}, Bool<true>{}, Bool<false>{});
      else body(Bool<false>{}, Bool<false>{}, Bool<false>{});
    } else if (!m0 && !m1) {
      body(Bool<true>{}, Bool<false>{}, Bool<false>{});
    } else if (!m0) {
      body(Bool<true>{}, Bool<false>{}, Bool<true>{});
    } else {
      body(Bool<true>{}, Bool<true>{}, Bool<true>{});
    }
    if (v + 1 < nb) stash(cur ^ 1);
    __syncthreads();
  }
  float *ah = acc + (long)bh * P;
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const float sum = group4_sum(cs[tb]);
    if (grp == 0 && (tb == 0 || two) && tok[tb] < P) ah[tok[tb]] = sum;
  }
}

template <typename Tin, int D>
static hipError_t run_prefill(const void *Q, const void *K, int batch, int heads, int P,
                              float4 *consts, float *acc, hipStream_t st) {
  const int nb = (P + 63) / 64;
  const int npairs = (nb + 1) / 2;
  const int bh = batch * heads;
  const long nblk = (long)bh * npairs;
  const long nblk_pad = (nblk + 7) / 8 * 8;
  if (nblk_pad > 0x7FFFFFFFL) return hipErrorInvalidValue;
  {
    TimedLaunch tl_("prefill_rows", st);
    hipLaunchKernelGGL((prefill_rows_kernel<Tin, D>), dim3((unsigned)nblk_pad), dim3(256), 0, st,
                       (const Tin *)Q, (const Tin *)K, P, bh, npairs, (int)nblk_pad, consts);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedLaunch tl_("prefill_colsum", st);
    hipLaunchKernelGGL((prefill_colsum_kernel<Tin, D>), dim3((unsigned)nblk_pad), dim3(256), 0, st,
                       (const Tin *)Q, (const Tin *)K, (const float4 *)consts, P, bh, npairs,
                       (int)nblk_pad, acc);
  }
  return hipGetLastError();
}

hipError_t launch_prefill(int etype, int d, const void *Q, const void *K, int batch, int heads,
                          int P, float4 *consts, float *acc, hipStream_t st) {
  if (etype == E_BF16) return d == 64 ? run_prefill<bf16, 64>(Q, K, batch, heads, P, consts, acc, st)
                                      : run_prefill<bf16, 128>(Q, K, batch, heads, P, consts, acc, st);
  if (etype == E_F16) return d == 64 ? run_prefill<f16, 64>(Q, K, batch, heads, P, consts, acc, st)
                                     : run_prefill<f16, 128>(Q, K, batch, heads, P, consts, acc, st);
  return hipErrorInvalidValue;
}

}  // namespace kvs
