// Pass 1 of the scoring path: softmax statistics (and attention outputs) of
// the scoring rows over the cache, split over token ranges.
//
// LORE-KV ("Monte Carlo Estimation for KV-Cache Eviction", Method): the
// w + M*T scoring queries of a query head attend over the n cached tokens;
// a_{q,i} = softmax(q.k_i / sqrt(d)) and o_q = sum_i a_{q,i} v_i feed the
// projected deletion score (Eq. 5).  Window row r < w sits at position
// n - w + r and sees tokens 0..n-w+r; lookahead rows see all n.
// H2O ("H2O: Heavy-Hitter Oracle", 3.4): a causal prompt row r attends to keys
// 0..r; only its max and normaliser are needed here.
//
// One workgroup per (token split, KV head, sequence) holds one wavefront per
// query head of the group, so a K/V tile staged in LDS is read once for the
// whole group.  The logits are formed transposed, S^T = K Q^T (tokens down the
// rows, query rows across the 16 columns): every lane then owns one query
// column, keeps that row's running max/sum in registers, and its eight
// accumulator values are eight tokens of that row.  Loading the K rows in the
// permuted order token(tb, rho) = 8*(rho/4) + 4*tb + rho%4 makes those eight
// tokens consecutive (8*(lane/16) + 0..7), which is exactly the k-slot order
// of a B fragment, so P^T enters the P.V product straight from registers.
// V is staged transposed (and converted to fp16 for 16-bit inputs) so the A
// fragment of O^T = V^T P^T is one 16-byte LDS read.
#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace kvs {

__device__ __forceinline__ int row_last(const RowGeom &g, int hv, int r) {
  if (g.mode == 0) {
    if (r >= g.nq) return -1;
    return r < g.w ? g.n - g.w + r : g.n - 1;
  }
  const int R = hv * 64 + r;
  return R < g.n ? R : -1;
}

// Index of scoring row r of query head hv (within KV head kvh's group) in Q.
__device__ __forceinline__ long q_row(const RowGeom &g, int b, int h_kv, int kvh, int hv, int r) {
  if (g.mode == 0) return (((long)b * h_kv + kvh) * g.group + hv) * g.nq + r;
  return ((long)b * h_kv + kvh) * g.n + (long)hv * 64 + r;
}

// QBW = 16-row query blocks per wave: a query head's 64 rows are spread over
// 4/QBW waves (QBW = 2 keeps the per-wave register set small).  Tiles of 64
// tokens are double-buffered in LDS: the next tile's global loads go to
// registers before the current tile is computed and into the other buffer
// after, so one barrier per tile separates the two.
template <typename Tin, int D, bool WITH_O, int MAXW, int QBW>
__global__ void __launch_bounds__(64 * MAXW)
attn_partial_kernel(const Tin *__restrict__ Q, const Tin *__restrict__ K, const Tin *__restrict__ V,
                    RowGeom geo, int h_kv, int tps, int splits, float *__restrict__ pm,
                    float *__restrict__ pl, float *__restrict__ pO) {
  typedef typename ValueType<Tin>::type TV;
  typedef typename FragOf<Tin>::type FQ;
  typedef typename FragOf<TV>::type FV;
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  constexpr int TN = 64;
  constexpr int WPH = 4 / QBW;                // waves per query head
  constexpr int EPC = 16 / (int)sizeof(Tin);  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                // chunks per row
  constexpr int KROW = D + EPC;               // padded LDS row (elements)
  constexpr int VROW = TN + 16 / (int)sizeof(TV);
  constexpr bool V16 = sizeof(TV) == 2;
  // K items: one 16-byte chunk; V items: a row pair (16-bit) or one row (fp32)
  constexpr int KITEMS = TN * CPR;
  constexpr int VITEMS = V16 ? (TN / 2) * CPR : TN * CPR;
  constexpr int PFK = (KITEMS + 32 * MAXW - 1) / (32 * MAXW);
  constexpr int PFV = (VITEMS + 32 * MAXW - 1) / (32 * MAXW);
  __shared__ __align__(16) Tin Ks[2][TN * KROW];
  __shared__ __align__(16) TV Vt[WITH_O ? 2 : 1][WITH_O ? D * VROW : 8];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int hv = wv / WPH, qb0 = (wv % WPH) * QBW;
  const int col = lane & 15, grp = lane >> 4;
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int n = geo.n;
  const long kv_base = ((long)b * h_kv + kvh) * (long)n * D;
  const int t_begin = s * tps;
  const int t_end = min(n, t_begin + tps);
  const int nt = (t_end - t_begin + TN - 1) / TN;
  const float c = kLog2e * rsqrtf((float)D);

  FQ qf[QBW][KS];
  int lim[QBW];
  int wave_last = -1;
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int r = (qb0 + qb) * 16 + col;
    lim[qb] = row_last(geo, hv, r);
    wave_last = max(wave_last, lim[qb]);
    if (lim[qb] >= 0) {
      const Tin *qp = Q + q_row(geo, b, h_kv, kvh, hv, r) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = load8<Tin>(qp + ks * 32 + 8 * grp);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = zero8<Tin>();
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) wave_last = max(wave_last, __shfl_xor(wave_last, o, 64));

  float m2[QBW], lsum[QBW];
  f32x4 oacc[WITH_O ? DB : 1][QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    m2[qb] = -INFINITY;
    lsum[qb] = 0.f;
  }
  if (WITH_O) {
#pragma unroll
    for (int db = 0; db < (WITH_O ? DB : 1); ++db)
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  U128 pk[PFK];
  U128 pv[WITH_O ? PFV : 1][V16 ? 2 : 1];
  auto prefetch = [&](int t0) {
#pragma unroll
    for (int u = 0; u < PFK; ++u) {
      const int idx = threadIdx.x + u * blockDim.x;
      const int row = idx / CPR, ch = idx % CPR;
      pk[u] = U128{0, 0, 0, 0};
      if (idx < KITEMS && t0 + row < n)
        pk[u] = *reinterpret_cast<const U128 *>(K + kv_base + (long)(t0 + row) * D + ch * EPC);
    }
    if (WITH_O) {
#pragma unroll
      for (int u = 0; u < PFV; ++u) {
        const int idx = threadIdx.x + u * blockDim.x;
        if constexpr (V16) {
          const int kp = idx % (TN / 2), ch = idx / (TN / 2);
          const int r0 = t0 + 2 * kp;
          pv[u][0] = U128{0, 0, 0, 0};
          pv[u][V16 ? 1 : 0] = U128{0, 0, 0, 0};
          if (idx < VITEMS && r0 < n)
            pv[u][0] = *reinterpret_cast<const U128 *>(V + kv_base + (long)r0 * D + ch * EPC);
          if (idx < VITEMS && r0 + 1 < n)
            pv[u][V16 ? 1 : 0] =
                *reinterpret_cast<const U128 *>(V + kv_base + (long)(r0 + 1) * D + ch * EPC);
        } else {
          const int r = idx % TN, ch = idx / TN;
          pv[u][0] = U128{0, 0, 0, 0};
          if (idx < VITEMS && t0 + r < n)
            pv[u][0] = *reinterpret_cast<const U128 *>(V + kv_base + (long)(t0 + r) * D + ch * EPC);
        }
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PFK; ++u) {
      const int idx = threadIdx.x + u * blockDim.x;
      if (idx < KITEMS) {
        const int row = idx / CPR, ch = idx % CPR;
        *reinterpret_cast<U128 *>(&Ks[buf][row * KROW + ch * EPC]) = pk[u];
      }
    }
    if (WITH_O) {
#pragma unroll
      for (int u = 0; u < PFV; ++u) {
        const int idx = threadIdx.x + u * blockDim.x;
        if (idx >= VITEMS) continue;
        if constexpr (V16) {
          const int kp = idx % (TN / 2), ch = idx / (TN / 2);
          const Tin *ae = reinterpret_cast<const Tin *>(&pv[u][0]);
          const Tin *be = reinterpret_cast<const Tin *>(&pv[u][V16 ? 1 : 0]);
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            const uint32_t packed = bits16(from_f32<TV>(to_f32(ae[e]))) |
                                    (bits16(from_f32<TV>(to_f32(be[e]))) << 16);
            *reinterpret_cast<uint32_t *>(&Vt[buf][(ch * EPC + e) * VROW + 2 * kp]) = packed;
          }
        } else {
          const int r = idx % TN, ch = idx / TN;
          const Tin *ae = reinterpret_cast<const Tin *>(&pv[u][0]);
#pragma unroll
          for (int e = 0; e < EPC; ++e) Vt[buf][(ch * EPC + e) * VROW + r] = from_f32<TV>(to_f32(ae[e]));
        }
      }
    }
  };

  if (nt > 0) {
    prefetch(t_begin);
    stash(0);
  }
  __syncthreads();
  for (int it = 0; it < nt; ++it) {
    const int t0 = t_begin + it * TN;
    const int cur = it & 1;
    if (it + 1 < nt) prefetch(t0 + TN);
#pragma unroll
    for (int sub = 0; sub < TN / 32; ++sub) {
      const int ts = t0 + sub * 32;
      if (ts > wave_last) continue;  // this wave's rows see none of these tokens

      f32x4 sacc[2][QBW];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int trow = sub * 32 + 8 * (col >> 2) + 4 * tb + (col & 3);
        FQ kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = load8<Tin>(&Ks[cur][trow * KROW + ks * 32 + 8 * grp]);
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mma(kf[ks], qf[qb][ks], acc);
          sacc[tb][qb] = acc;
        }
      }

      typename FragOf<TV>::type pf[QBW];
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        float sv[8];
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int tok = ts + 8 * grp + 4 * tb + j;
            float x = sacc[tb][qb][j] * c;
            x = (tok <= lim[qb]) ? x : -INFINITY;
            sv[4 * tb + j] = x;
            mx = fmaxf(mx, x);
          }
        mx = wave_max_xor(mx, 16);
        mx = wave_max_xor(mx, 32);
        const float mnew = fmaxf(m2[qb], mx);
        const float muse = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = hw_exp2(m2[qb] - muse);
        float p[8];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = hw_exp2(sv[e] - muse);
          psum += p[e];
        }
        lsum[qb] = lsum[qb] * alpha + psum;
        m2[qb] = mnew;
        if (WITH_O) {
#pragma unroll
          for (int db = 0; db < (WITH_O ? DB : 1); ++db) oacc[db][qb] *= alpha;
          pf[qb] = pack8<TV>(p);
        }
      }
      if (WITH_O) {
#pragma unroll
        for (int db = 0; db < (WITH_O ? DB : 1); ++db) {
          const FV vf = load8<TV>(&Vt[cur][(db * 16 + col) * VROW + sub * 32 + 8 * grp]);
#pragma unroll
          for (int qb = 0; qb < QBW; ++qb) oacc[db][qb] = mma(vf, pf[qb], oacc[db][qb]);
        }
      }
    }
    if (it + 1 < nt) stash(cur ^ 1);
    __syncthreads();
  }

  const long head = ((long)b * h_kv + kvh) * geo.group + hv;
  const long pbase = (head * splits + s) * 64;
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    float l = lsum[qb];
    l = wave_sum_xor(l, 16);
    l = wave_sum_xor(l, 32);
    const int r = (qb0 + qb) * 16 + col;
    if (grp == 0) {
      pm[pbase + r] = m2[qb];
      pl[pbase + r] = l;
    }
  }
  if (WITH_O) {
    float *po = pO + (head * splits + s) * (long)D * 64;
#pragma unroll
    for (int db = 0; db < (WITH_O ? DB : 1); ++db)
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          po[(db * 16 + 4 * grp + j) * 64 + (qb0 + qb) * 16 + col] = oacc[db][qb][j];
  }
}

// LORE: merge the splits of every scoring row into row_max (natural units of
// q.k/sqrt(d)), row_sum and the normalised O.  One block per (query head,
// 16-wide slice of d): thread (q = tid % 64, d-lane = tid / 64); the split
// weights are computed once per block into LDS.
template <int D>
__global__ void __launch_bounds__(256)
attn_combine_lore_kernel(const float *__restrict__ pm, const float *__restrict__ pl,
                         const float *__restrict__ pO, int splits, int nq,
                         float *__restrict__ row_max, float *__restrict__ row_sum,
                         float *__restrict__ O) {
  extern __shared__ float wsh[];  // [splits][64] split weights, then [64] 1/L
  const long head = blockIdx.x;
  const int d0 = blockIdx.y * 16;
  const int q = threadIdx.x & 63, part = threadIdx.x >> 6;
  const float *hm = pm + head * splits * 64;
  const float *hl = pl + head * splits * 64;
  if (part == 0) {
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, hm[s * 64 + q]);
    const float muse = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float wgt = exp2f(hm[s * 64 + q] - muse);
      wsh[s * 64 + q] = wgt;
      L += hl[s * 64 + q] * wgt;
    }
    wsh[splits * 64 + q] = 1.f / L;
    if (q < nq && blockIdx.y == 0) {
      row_max[head * nq + q] = M * kLn2;
      row_sum[head * nq + q] = L;
    }
  }
  __syncthreads();
  const float inv = wsh[splits * 64 + q];
  const float *ho = pO + head * splits * (long)D * 64;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int d = d0 + part * 4 + u;
    float o = 0.f;
    for (int s = 0; s < splits; ++s) o += ho[((long)s * D + d) * 64 + q] * wsh[s * 64 + q];
    if (q < nq) O[(head * nq + q) * D + d] = o * inv;
  }
}

// H2O prefill: merge the splits into per-row constants for the column-sum
// pass: x = beta2 = max2 + log2(sum), w = bits of the last visible key.
__global__ void __launch_bounds__(64)
attn_combine_rows_kernel(const float *__restrict__ pm, const float *__restrict__ pl, int splits,
                         int group, int P, float4 *__restrict__ consts) {
  const long head = blockIdx.x;  // virtual head
  const int q = threadIdx.x;
  const float *hm = pm + head * splits * 64;
  const float *hl = pl + head * splits * 64;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, hm[s * 64 + q]);
  const float muse = (M == -INFINITY) ? 0.f : M;
  float L = 0.f;
  for (int s = 0; s < splits; ++s) L += hl[s * 64 + q] * exp2f(hm[s * 64 + q] - muse);
  const int R = (int)(head % group) * 64 + q;
  const int last = R < P ? R : -1;
  const float beta2 = (last >= 0) ? muse + log2f(L) : 0.f;
  consts[head * 64 + q] = make_float4(beta2, 0.f, 1.f, __int_as_float(last));
}

SplitPlan attn_split_plan(int units, int n) {
  const int target = 256;  // one workgroup per CU: splits share nothing, and fewer splits mean less partial-O traffic
  int splits = (target + units - 1) / units;
  const int max_splits = (n + 511) / 512;
  if (splits > max_splits) splits = max_splits;
  if (splits > 128) splits = 128;
  if (splits < 1) splits = 1;
  int tps = (n + splits - 1) / splits;
  tps = (tps + 63) / 64 * 64;
  splits = (n + tps - 1) / tps;
  return SplitPlan{splits, tps};
}

template <typename Tin, int D, bool WITH_O, int MAXW, int QBW>
static hipError_t run_partial(const void *Q, const void *K, const void *V, RowGeom geo, int batch,
                              int h_kv, SplitPlan plan, float *pm, float *pl, float *pO,
                              hipStream_t st) {
  dim3 grid(plan.splits, h_kv, batch), block(64 * geo.group * (4 / QBW));
  if ((int)block.x < 32 * MAXW || (int)block.x > 64 * MAXW) return hipErrorInvalidConfiguration;
  {
    TimedLaunch tl_("attn_partial", st);
    hipLaunchKernelGGL((attn_partial_kernel<Tin, D, WITH_O, MAXW, QBW>), grid, block, 0, st,
                       (const Tin *)Q, (const Tin *)K, (const Tin *)V, geo, h_kv, plan.tps,
                       plan.splits, pm, pl, pO);
  }
  return hipGetLastError();
}

// Waves per workgroup = group * 4 / QBW <= 16; MAXW is the next power of two
// (at least 2), so a block has between 32*MAXW and 64*MAXW threads.
template <typename Tin, int D>
static hipError_t run_partial_d(bool with_o, const void *Q, const void *K, const void *V,
                                RowGeom geo, int batch, int h_kv, SplitPlan plan, float *pm,
                                float *pl, float *pO, hipStream_t st) {
#define KVS_RP(O, MAXW, QBW) \
  return run_partial<Tin, D, O, MAXW, QBW>(Q, K, V, geo, batch, h_kv, plan, pm, pl, pO, st)
  if (!with_o) {
    if (geo.group <= 2) KVS_RP(false, 2, 4);
    if (geo.group <= 4) KVS_RP(false, 4, 4);
    if (geo.group <= 8) KVS_RP(false, 8, 4);
    KVS_RP(false, 16, 4);
  }
  if (geo.group <= 2) KVS_RP(true, 4, 2);
  if (geo.group <= 4) KVS_RP(true, 8, 2);
  if (geo.group <= 8) KVS_RP(true, 16, 2);
  KVS_RP(true, 16, 4);
#undef KVS_RP
}

hipError_t launch_attn_partial(int etype, int d, bool with_o, const void *Q, const void *K,
                               const void *V, RowGeom geo, int batch, int h_kv, SplitPlan plan,
                               float *part_m, float *part_l, float *part_O, hipStream_t st) {
#define KVS_PARTIAL(T, DD) \
  return run_partial_d<T, DD>(with_o, Q, K, V, geo, batch, h_kv, plan, part_m, part_l, part_O, st)
  if (etype == E_F32) { if (d == 64) KVS_PARTIAL(float, 64); KVS_PARTIAL(float, 128); }
  if (etype == E_BF16) { if (d == 64) KVS_PARTIAL(bf16, 64); KVS_PARTIAL(bf16, 128); }
  if (d == 64) KVS_PARTIAL(f16, 64);
  KVS_PARTIAL(f16, 128);
#undef KVS_PARTIAL
}

hipError_t launch_attn_combine_lore(int d, const float *part_m, const float *part_l,
                                    const float *part_O, int heads, int splits, int nq,
                                    float *row_max, float *row_sum, float *O, hipStream_t st) {
  const size_t shm = sizeof(float) * 64 * ((size_t)splits + 1);
  {
    TimedLaunch tl_("attn_combine", st);
    if (d == 64)
      hipLaunchKernelGGL(attn_combine_lore_kernel<64>, dim3(heads, 64 / 16), dim3(256), shm, st,
                         part_m, part_l, part_O, splits, nq, row_max, row_sum, O);
    else
      hipLaunchKernelGGL(attn_combine_lore_kernel<128>, dim3(heads, 128 / 16), dim3(256), shm, st,
                         part_m, part_l, part_O, splits, nq, row_max, row_sum, O);
  }
  return hipGetLastError();
}

hipError_t launch_attn_combine_rows(const float *part_m, const float *part_l, int heads,
                                    int splits, int group, int P, float4 *consts, hipStream_t st) {
  {
    TimedLaunch tl_("attn_combine_rows", st);
    hipLaunchKernelGGL(attn_combine_rows_kernel, dim3(heads), dim3(64), 0, st, part_m, part_l,
                       splits, group, P, consts);
  }
  return hipGetLastError();
}

}  // namespace kvs
