// Pass 2 of the scoring path: LORE-KV's projected deletion score, and the
// causal column sums H2O's prefill needs.
//
// LORE-KV ("Monte Carlo Estimation for KV-Cache Eviction", Method,
// "Projected deletion score", Eqs. 5-7):
//   e_{q,i} = a_{q,i} / (1 - a_{q,i} + eps) * ||W_h (v_i - o_q)||,
//   S_i     = psi(E_{i,W}) + lambda_L sum_m omega_m psi(E_{i,m}),  psi = mean,
// and the KV head's score is the mean over its query-head group.  The norm is
// expanded in the Gram form  ||W_h(v - o)||^2 = N_i - 2 x_{q,i} + pi_q  with
//   G_h = W_h^T W_h (d x d),  N_i = v_i^T G_h v_i,  y_q = G_h o_q,
//   x_{q,i} = v_i . y_q,  pi_q = o_q^T G_h o_q,
// so the per-token work is three dense contractions on the matrix cores
// (S = Q K^T recomputing the logits, X = Y V^T, and G_h V^T for N) plus a
// short elementwise epilogue, and W_O (d_model wide) is touched once per call.
//
// Kernels, in call order:
//   gram_kernel        G_h partial sums over d_model ranges, upper blocks (MFMA)
//   gram_reduce_kernel G~_h = G_h rounded to the value type, mirrored (symmetric)
//   prep_kernel        y_q = G~_h o_q (fp16 hi + lo; lo as scaled fp8 for 16-bit
//                      inputs), pi_q, per-row constants
//   vnorm_kernel       N_i for every token and query head (MFMA)
//   score_kernel<0>    recompute a, form e, aggregate rows and group heads -> S
//   score_kernel<1>    H2O: column sums of the causal prompt probabilities
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace kvs {

// ---------------------------------------------------------------------------
// G_h = W_h^T W_h, one range of d_model rows per block.  W_h is the column
// slice h*D .. h*D+D-1 of W_O [d_model][h_q*D].  Stages of SR rows (128 for
// 16-bit inputs: four MFMA k-steps) are staged transposed in LDS so both MFMA
// operands are 16-byte reads.  A split holds at most kGramStages stages,
// whose loads are all issued before the first is multiplied.
template <typename Tin> struct GramStage { static constexpr int rows = sizeof(Tin) == 2 ? 128 : 32; };
constexpr int kGramStages = 4;  // stages per split, all in flight at once

template <typename Tin, int D>
__global__ void __launch_bounds__(256)
gram_kernel(const Tin *__restrict__ W, int dm, int h_q, int rows_per_split,
            float *__restrict__ Gpart) {
  typedef typename FragOf<Tin>::type FW;
  constexpr int SR = GramStage<Tin>::rows;
  constexpr int KSTEP = SR / 32;
  constexpr int EPC = 16 / (int)sizeof(Tin);
  constexpr int CPR = D / EPC;
  constexpr int WROW = SR + EPC;
  constexpr int DB = D / 16;
  constexpr int RPW = (DB + 3) / 4;  // row blocks per wave
  constexpr bool P16 = sizeof(Tin) == 2;
  // staging items: 16-bit -> (row pair, chunk), fp32 -> (row, chunk)
  constexpr int RI = P16 ? SR / 2 : SR;
  constexpr int ITEMS = RI * CPR;
  constexpr int PFG = (ITEMS + 255) / 256;
  __shared__ __align__(16) Tin Wt[2][D * WROW];
  // wave-uniform in a scalar register, so the per-wave block-triangle tests
  // below are scalar branches, not exec masks
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int s = blockIdx.x, h = blockIdx.y;
  const long ld = (long)h_q * D;
  const int k_begin = s * rows_per_split;
  const int k_end = min(dm, k_begin + rows_per_split);
  const int nslab = (k_end - k_begin + SR - 1) / SR;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(
      W + (long)k_begin * ld + (long)h * D,
      (uint32_t)max(k_end - k_begin, 0) * (uint32_t)(ld * sizeof(Tin)));

  constexpr int NR = kGramStages;
  U128 pw[NR][PFG][P16 ? 2 : 1];
  auto prefetch = [&](int slab, U128 (&pw)[PFG][P16 ? 2 : 1]) {
#pragma unroll
    for (int u = 0; u < PFG; ++u) {
      const int idx = threadIdx.x + u * 256;
      if (ITEMS % 256 != 0 && idx >= ITEMS) continue;
      // 16-bit: chunks of a row pair are adjacent lanes, so a wave reads whole
      // 256-byte row slices; fp32: rows are adjacent lanes
      const int kr = P16 ? idx / CPR : idx % RI, ch = P16 ? idx % CPR : idx / RI;
      if constexpr (P16) {
        const uint32_t r0 = (uint32_t)(slab * SR + 2 * kr);
        pw[u][0] = buf_load16(rw, (uint32_t)((r0 * ld + ch * EPC) * sizeof(Tin)));
        pw[u][P16 ? 1 : 0] = buf_load16(rw, (uint32_t)(((r0 + 1) * ld + ch * EPC) * sizeof(Tin)));
      } else {
        pw[u][0] = buf_load16(rw, (uint32_t)(((uint32_t)(slab * SR + kr) * ld + ch * EPC) * sizeof(Tin)));
      }
    }
  };
  auto stash = [&](int buf, const U128 (&pw)[PFG][P16 ? 2 : 1]) {
#pragma unroll
    for (int u = 0; u < PFG; ++u) {
      const int idx = threadIdx.x + u * 256;
      if (ITEMS % 256 != 0 && idx >= ITEMS) continue;
      const int kr = P16 ? idx / CPR : idx % RI, ch = P16 ? idx % CPR : idx / RI;
      if constexpr (P16) {
        const Elems16<Tin> ae = elems16<Tin>(pw[u][0]);
        const Elems16<Tin> be = elems16<Tin>(pw[u][P16 ? 1 : 0]);
        // row pair kr lands at dword kr ^ 4*((row >> 3) & 7) of LDS row
        // ch*8 + e: the 16 lanes of a row pair then hit distinct banks
        const int kd = kr ^ (4 * (ch & 7));
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          *reinterpret_cast<uint32_t *>(&Wt[buf][(ch * EPC + e) * WROW + 2 * kd]) =
              bits16(ae.e[e]) | (bits16(be.e[e]) << 16);
      } else {
        const Elems16<Tin> ae = elems16<Tin>(pw[u][0]);
#pragma unroll
        for (int e = 0; e < EPC; ++e) Wt[buf][(ch * EPC + e) * WROW + kr] = ae.e[e];
      }
    }
  };

  f32x4 acc[RPW][DB];
#pragma unroll
  for (int ri = 0; ri < RPW; ++ri)
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) acc[ri][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the blocks a wave forms depend on its index; each wave runs a copy of the
  // loop specialised for it, so the block-triangle tests are resolved at
  // compile time
  auto compute_w = [&](auto wvc, int cur) {
    constexpr int WV = decltype(wvc)::value;
#pragma unroll
    for (int ks = 0; ks < KSTEP; ++ks) {
      // k offset of the 8-element group, undoing the staging swizzle of row r
      auto koff = [&](int r) { return P16 ? (ks * 32 + 8 * grp) ^ (8 * ((r >> 3) & 7)) : ks * 32 + 8 * grp; };
      FW af[RPW];
#pragma unroll
      for (int ri = 0; ri < RPW; ++ri) {
        const int rb = WV + 4 * ri;
        const int r = rb * 16 + col;
        af[ri] = rb < DB ? load8<Tin>(&Wt[cur][r * WROW + koff(r)]) : zero8<Tin>();
      }
#pragma unroll
      for (int cb = WV; cb < DB; ++cb) {
        const int r = cb * 16 + col;
        const FW bfr = load8<Tin>(&Wt[cur][r * WROW + koff(r)]);
#pragma unroll
        for (int ri = 0; ri < RPW; ++ri)
          if (cb >= WV + 4 * ri) acc[ri][cb] = mma(af[ri], bfr, acc[ri][cb]);
      }
    }
  };
  auto compute = [&](int cur) {
    switch (wv) {
      case 0: compute_w(std::integral_constant<int, 0>{}, cur); break;
      case 1: compute_w(std::integral_constant<int, 1>{}, cur); break;
      case 2: compute_w(std::integral_constant<int, 2>{}, cur); break;
      default: compute_w(std::integral_constant<int, 3>{}, cur); break;
    }
  };

  // a split holds at most NR stages (gram_splits), all requested up front
  // stages past the split read zeros; the fences keep the loads in stage
  // order, so each stage waits only for its own
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    prefetch(r, pw[r]);
    sched_fence();
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if (r >= nslab) break;
    // LDS buffer r % 2 was last read by stage r - 2, which every wave
    // finished before the previous barrier
    stash(r & 1, pw[r]);
    __syncthreads();
    compute(r & 1);
  }
  // G is symmetric: only the 16x16 blocks on and above the diagonal are
  // formed and written (the reduction mirrors them).
  float *G = Gpart + ((long)s * h_q + h) * D * D;
#pragma unroll
  for (int ri = 0; ri < RPW; ++ri) {
    const int rb = wv + 4 * ri;
    if (rb >= DB) continue;
#pragma unroll
    for (int cb = 0; cb < DB; ++cb) {
      if (cb < rb) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) G[(rb * 16 + 4 * grp + j) * D + cb * 16 + col] = acc[ri][cb][j];
    }
  }
}

int gram_splits(int h_q, int d_model, int elem_bytes) {
  const int sr = elem_bytes == 2 ? GramStage<bf16>::rows : GramStage<float>::rows;
  const int stages = (d_model + sr - 1) / sr;
  int splits = (256 + h_q - 1) / h_q;
  const int need = (stages + kGramStages - 1) / kGramStages;  // at most kGramStages per split
  if (splits < need) splits = need;
  if (splits > stages) splits = stages;
  if (splits < 1) splits = 1;
  return splits;
}

// ---------------------------------------------------------------------------
// Sum the G_h partials (fixed order) and round G_h to the value type once:
// Gv = G~ (value type, for the MFMA in vnorm_kernel) and Gr = float(G~),
// exactly symmetric (mirrored from the upper triangle).  Every
// term of the norm expansion is then formed from that same G~: y_q = G~ o_q
// and pi_q = o_q . y_q in prep_kernel, N_i = v_i^T G~ v_i in vnorm_kernel.  So
// N - 2x + pi equals (v - o)^T G~ (v - o) up to fp32 accumulation: no term
// carries a rounding the others do not share, and tokens whose value is close
// to the attention output (where the three terms nearly cancel) keep their
// relative accuracy.
template <int D, typename TV>
__global__ void __launch_bounds__(256)
gram_reduce_kernel(const float *__restrict__ Gpart, int gsplits, int h_q, TV *__restrict__ Gv,
                   float *__restrict__ Gr) {
  // block (32 x 32 tile (I, J) with I <= J, head h).  Thread (row ti, 4
  // columns) sums the entries with j >= i over the splits in a fixed order;
  // the tile is written in place and, through LDS, transposed to (J, I), so
  // G~ is exactly symmetric and every global access is a 16-byte row chunk.
  constexpr int NT = D / 32;
  __shared__ float T[32][33];
  int I = 0, rem = blockIdx.x;
  while (rem >= NT - I) { rem -= NT - I; ++I; }
  const int J = I + rem;
  const int h = blockIdx.y;
  const int ti = threadIdx.x >> 3, tj = (threadIdx.x & 7) * 4;
  const long total = (long)h_q * D * D;
  const int i = 32 * I + ti, j0 = 32 * J + tj;
  const long idx = ((long)h * D + i) * D + j0;
  float4 g = make_float4(0.f, 0.f, 0.f, 0.f);
  if (j0 + 3 >= i) {  // some entry of the chunk is on or above the diagonal
    int s = 0;
    for (; s + 4 <= gsplits; s += 4) {
      const float4 a0 = *reinterpret_cast<const float4 *>(Gpart + (long)s * total + idx);
      const float4 a1 = *reinterpret_cast<const float4 *>(Gpart + (long)(s + 1) * total + idx);
      const float4 a2 = *reinterpret_cast<const float4 *>(Gpart + (long)(s + 2) * total + idx);
      const float4 a3 = *reinterpret_cast<const float4 *>(Gpart + (long)(s + 3) * total + idx);
      g.x += a0.x; g.y += a0.y; g.z += a0.z; g.w += a0.w;
      g.x += a1.x; g.y += a1.y; g.z += a1.z; g.w += a1.w;
      g.x += a2.x; g.y += a2.y; g.z += a2.z; g.w += a2.w;
      g.x += a3.x; g.y += a3.y; g.z += a3.z; g.w += a3.w;
    }
    for (; s < gsplits; ++s) {
      const float4 a = *reinterpret_cast<const float4 *>(Gpart + (long)s * total + idx);
      g.x += a.x; g.y += a.y; g.z += a.z; g.w += a.w;
    }
  }
  float gv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    gv[e] = to_f32(from_f32<TV>(gv[e]));
    T[ti][tj + e] = gv[e];
  }
  // direct write: entries with j >= i (all of them off the diagonal tile)
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (j0 + e >= i) {
      Gv[idx + e] = from_f32<TV>(gv[e]);
      Gr[idx + e] = gv[e];
    }
  __syncthreads();
  // transposed write: entry (32J + ti, 32I + tj + e) = tile (tj + e, ti),
  // taken where that tile entry is above the diagonal (the rest is written
  // directly on a diagonal tile)
  const int r = 32 * J + ti;
  const long tdx = ((long)h * D + r) * D + 32 * I + tj;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int c = 32 * I + tj + e;
    if (r > c) {
      const float v = T[tj + e][ti];
      Gv[tdx + e] = from_f32<TV>(v);
      Gr[tdx + e] = v;
    }
  }
}

// Per (query head, sequence, 16-row group): y_q = G~ o_q (stored as a hi + lo
// pair of the value type, y = hi + lo to ~22 bits, for the MFMA product V.y),
// pi_q = o_q . y_q, and the per-row constants of the score pass:
//   x = beta2 = row_max*log2(e) + log2(row_sum)   (a = exp2(s*log2e/sqrt(d) - beta2))
//   y = pi_q,  z = row weight (1/w for window rows, lambda_L omega_m / T for
//   lookahead rows, 0 for padding rows),  w = bits of the last visible token.
template <int D, typename TV>
__global__ void __launch_bounds__(256)
prep_kernel(const float *__restrict__ Gr, const float *__restrict__ O,
            const float *__restrict__ row_max, const float *__restrict__ row_sum,
            const float *__restrict__ omega, int h_q, int n, int nq, int w, int m, int t,
            float lambda_l, TV *__restrict__ Yhi, TV *__restrict__ Ylo,
            float4 *__restrict__ consts) {
  constexpr int SLAB = 32;
  constexpr int RG = 16;  // rows per block
  __shared__ float Os[RG * D];
  __shared__ float Gs[SLAB * (D + 1)];
  const int h = blockIdx.x, b = blockIdx.y, r0 = blockIdx.z * RG;
  const long hb = (long)b * h_q + h;
  for (int idx = threadIdx.x; idx < RG * D; idx += blockDim.x) {
    const int r = r0 + idx / D;
    Os[idx] = r < nq ? O[(hb * nq + r) * D + idx % D] : 0.f;
  }
  // thread -> (row rl = tid/16, 2 consecutive outputs of every 32-row slab)
  const int rl = threadIdx.x >> 4, sub = threadIdx.x & 15;
  const int r = r0 + rl;
  float pi = 0.f;
  for (int dd0 = 0; dd0 < D; dd0 += SLAB) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < SLAB * D; idx += blockDim.x) {
      const int row = idx / D, k = idx % D;
      Gs[row * (D + 1) + k] = Gr[((long)h * D + dd0 + row) * D + k];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int row = sub * 2 + u;
      float y = 0.f;
      for (int k = 0; k < D; ++k) y += Gs[row * (D + 1) + k] * Os[rl * D + k];
      if (r >= nq) y = 0.f;
      pi += Os[rl * D + dd0 + row] * y;
      const TV hi = from_f32<TV>(y);
      Yhi[(hb * 64 + r) * D + dd0 + row] = hi;
      Ylo[(hb * 64 + r) * D + dd0 + row] = from_f32<TV>(y - to_f32(hi));
    }
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) pi += __shfl_xor(pi, o, 64);
  if (sub == 0) {
    float beta2 = 0.f, wr = 0.f;
    int last = -1;
    if (r < nq) {
      beta2 = row_max[hb * nq + r] * kLog2e + log2f(row_sum[hb * nq + r]);
      if (r < w) {
        wr = 1.f / (float)w;
        last = n - w + r;
      } else {
        wr = lambda_l * omega[(long)b * m + (r - w) / t] / (float)t;
        last = n - 1;
      }
    }
    consts[hb * 64 + r] = make_float4(beta2, pi, wr, __int_as_float(last));
  }
}

// The same outputs for 16-bit value types, on the matrix cores.  One block
// per (query head, sequence); wave w takes rows 16w..16w+15.  G~ is exact in
// fp16, so y = G~ o is formed as G~ o_hi + G~ o_lo with o scaled per row by a
// power of two (largest |o| in [2^14, 2^15)) and split into fp16 hi + lo
// parts: the products are exact and the sum is an fp32 accumulation, as in
// a plain fp32 dot product.  G~ is symmetric, so its rows serve as the
// columns of the B operand.  y is stored as fp16 y_hi plus y_lo = y - y_hi as
// fp8 e4m3 scaled per row by a power of two (see the y_lo block below).
template <int D>
__global__ void __launch_bounds__(256)
prep_mfma_kernel(const f16 *__restrict__ Gv, const float *__restrict__ O,
                 const float *__restrict__ row_max, const float *__restrict__ row_sum,
                 const float *__restrict__ omega, int h_q, int n, int nq, int w, int m, int t,
                 float lambda_l, f16 *__restrict__ Yhi, uint8_t *__restrict__ Ylo8,
                 float4 *__restrict__ consts) {
  constexpr int KS = D / 32, NB = D / 16;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int h = blockIdx.x, b = blockIdx.y;
  const long hb = (long)b * h_q + h;
  const f16 *G = Gv + (long)h * D * D;
  // A operand: lane (col, grp) holds o[16w + col][32 ks + 8 grp + e]
  const int ra = wv * 16 + col;
  // the row constants' inputs are requested first, so their loads are not a
  // round trip of their own after the products
  const int rc = wv * 16 + 4 * grp + (col & 3);
  float rmax = 0.f, rsum = 1.f, om = 0.f;
  if (col < 4 && rc < nq) {
    rmax = row_max[hb * nq + rc];
    rsum = row_sum[hb * nq + rc];
    if (rc >= w) om = omega[(long)b * m + (rc - w) / t];
  }
  float oa[KS][8];
  float amax = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const float4 *src = reinterpret_cast<const float4 *>(O + (hb * nq + ra) * D + ks * 32 + 8 * grp);
    const float4 v0 = ra < nq ? src[0] : make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 v1 = ra < nq ? src[1] : make_float4(0.f, 0.f, 0.f, 0.f);
    oa[ks][0] = v0.x; oa[ks][1] = v0.y; oa[ks][2] = v0.z; oa[ks][3] = v0.w;
    oa[ks][4] = v1.x; oa[ks][5] = v1.y; oa[ks][6] = v1.z; oa[ks][7] = v1.w;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(oa[ks][e]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
  // power-of-two row scale: exponent of amax -> 14
  const int ex = amax > 0.f ? max(((__float_as_int(amax) >> 23) & 0xFF) - 127, -100) : 14;
  const float sc = ldexpf(1.f, 14 - ex), unsc = ldexpf(1.f, ex - 14);
  f16x8 ahi[KS], alo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = oa[ks][e] * sc;
      const f16 hi = (f16)v;
      ahi[ks][e] = hi;
      alo[ks][e] = (f16)(v - (float)hi);
    }
  // output rows 16w + 4 grp + j: their unscale factors live in lanes 4 grp + j
  float unr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) unr[j] = __shfl(unsc, 4 * grp + j, 64);
  // every G~ fragment and every o element the pi sums need are requested up
  // front, so the block waits for one round of loads rather than one per
  // column block
  f16x8 bfa[NB][KS];
  float oc[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) bfa[nb][ks] = load8<f16>(G + (nb * 16 + col) * D + ks * 32 + 8 * grp);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wv * 16 + 4 * grp + j;
      oc[nb][j] = r < nq ? O[(hb * nq + r) * D + nb * 16 + col] : 0.f;
    }
  }
  float pij[4] = {0.f, 0.f, 0.f, 0.f};
  float ylo[NB][4], lmax[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const f16x8 (&bf)[KS] = bfa[nb];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mma(ahi[ks], bf[ks], acc);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = mma(alo[ks], bf[ks], acc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wv * 16 + 4 * grp + j, c = nb * 16 + col;
      const float y = r < nq ? acc[j] * unr[j] : 0.f;
      const f16 hi = (f16)y;
      Yhi[(hb * 64 + r) * D + c] = hi;
      ylo[nb][j] = y - (float)hi;
      lmax[j] = fmaxf(lmax[j], fabsf(ylo[nb][j]));
      pij[j] = fmaf(oc[nb][j], y, pij[j]);
    }
  }
  // y_lo as fp8 e4m3 with a power-of-two row scale 2^k putting the row's
  // largest |y_lo| in [128, 256); the score pass's block-scaled MFMA applies
  // 2^-k through the row's E8M0 scale byte 127 - k.  Per head: 64 rows of D
  // bytes, then 64 int32 scale bytes.
  uint8_t *yb = Ylo8 + hb * (64 * D + 256);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float am = row16_max(lmax[j]);
    const int e = am > 0.f ? ((__float_as_int(am) >> 23) & 0xFF) - 127 : 7;
    const int k = min(max(7 - e, -120), 120);
    const float sc = ldexpf(1.f, k);
    const int r = wv * 16 + 4 * grp + j;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      yb[r * D + nb * 16 + col] =
          (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(ylo[nb][j] * sc, 0.f, 0, false) & 0xFF);
    if (col == 0) reinterpret_cast<int *>(yb + 64 * D)[r] = 127 - k;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) pij[j] = row16_sum(pij[j]);
  if (col < 4) {
    const int r = wv * 16 + 4 * grp + col;
    const float pi = col == 0 ? pij[0] : col == 1 ? pij[1] : col == 2 ? pij[2] : pij[3];
    float beta2 = 0.f, wr = 0.f;
    int last = -1;
    if (r < nq) {
      beta2 = rmax * kLog2e + log2f(rsum);
      if (r < w) {
        wr = 1.f / (float)w;
        last = n - w + r;
      } else {
        wr = lambda_l * om / (float)t;
        last = n - 1;
      }
    }
    consts[hb * 64 + r] = make_float4(beta2, pi, wr, __int_as_float(last));
  }
}

// ---------------------------------------------------------------------------
// N[b][h][i] = v_i^T G~_h v_i.  A workgroup of 4 waves serves up to 4 query
// heads of one KV head over a token range: 64-token V tiles are read from
// global memory once, converted to the value type once and staged in LDS
// (double-buffered: the next tile's loads are in flight while the current one
// is computed), and every wave applies its own head's G~_h to the tile.  With
// fewer than 4 heads in the group the spare waves split the tile's 16-token
// blocks instead.  Each wave holds G~_h as A fragments with its rows permuted
// by sigma(db, m) = 32*(db/2) + 8*(m/4) + 4*(db%2) + m%4, which lands output
// row 4*(lane/16)+j of block db on the head-dim index whose V value the lane
// already holds in its own B fragment (k-step db/2, element 4*(db%2)+j): the
// quadratic form then needs no data exchange until the final two cross-lane
// adds.  G~ is symmetric, so only its block upper triangle is used (32x32
// blocks: the diagonal blocks whole, the blocks above them doubled, exact in
// the value type): 20 of the 32 products per 16 tokens.
template <typename Tin, int D, int TPARTS>
__global__ void __launch_bounds__(256)
vnorm_kernel(const Tin *__restrict__ V, const typename ValueType<Tin>::type *__restrict__ Gv,
             int n, int n_pad, int h_q, int h_kv, int tpw, int nchunk, float *__restrict__ Nn) {
  typedef typename ValueType<Tin>::type TV;
  typedef typename FragOf<TV>::type FV;
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  constexpr int TN = 64;
  constexpr int EPC = 16 / (int)sizeof(Tin);
  constexpr int CPR = D / EPC;
  // 16-bit rows padded by 32 bytes: conflict-free fragment reads (as in the score pass)
  constexpr int VROW = D + (sizeof(TV) == 2 ? 16 : 4);
  constexpr int PF = (TN * CPR + 255) / 256;
  __shared__ __align__(16) TV Vs[2][TN * VROW];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int G = h_q / h_kv;
  const int hpw = G < 4 ? G : 4;          // heads per workgroup
  const int ngrp = (G + hpw - 1) / hpw;   // workgroups per KV head and token range
  static_assert(TPARTS == 1 || TPARTS == 2 || TPARTS == 4, "waves per head's tile");
  // logical (sequence, KV head, head group, token chunk) of this block
  const long L = blockIdx.x;
  const int chunk_i = (int)(L % nchunk);
  const long rest = L / nchunk;
  const int hgi = (int)(rest % ngrp);
  const int kvh = (int)((rest / ngrp) % h_kv);
  const int b = (int)(rest / ((long)ngrp * h_kv));
  const int tp = wv / hpw;  // (launch: TPARTS == 4 / hpw)
  const int hg = hgi * hpw + wv % hpw;
  const bool active = tp < TPARTS && hg < G;
  const int h = kvh * G + (active ? hg : 0);

  // block (db, ks) is used when ks >= db/2 and doubled when ks > db/2
  FV gf[DB][KS];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int row = 32 * (db >> 1) + 8 * (col >> 2) + 4 * (db & 1) + (col & 3);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks < (db >> 1)) continue;
      FV f = active ? load8<TV>(Gv + ((long)h * D + row) * D + ks * 32 + 8 * grp) : zero8<TV>();
      if (ks > (db >> 1)) {
        float t[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = 2.f * frag_elem(f, e);
        f = pack8<TV>(t);
      }
      gf[db][ks] = f;
    }
  }
  const Tin *Vg = V + ((long)b * h_kv + kvh) * (long)n * D;
  float *Nh = Nn + ((long)b * h_q + h) * n_pad;
  const int t_begin = chunk_i * tpw;
  const int t_end = min(n_pad, t_begin + tpw);
  const int nt = (t_end - t_begin + TN - 1) / TN;

  // Tile loads run one tile ahead (issued before the current tile is
  // computed, stored to the other LDS buffer after it).
  U128 pv[PF];
  constexpr uint32_t RB = D * sizeof(Tin);
  // V has n rows; tokens n..n_pad-1 read as zeros (N = 0 there)
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(Vg + (long)t_begin * D, range_bytes(t_begin, min(t_end, n), RB));
  const __amdgpu_buffer_rsrc_t rn = make_rsrc(Nh + t_begin, range_bytes(t_begin, t_end, 4));
  auto prefetch = [&](int t0) {
    const uint32_t toff = (uint32_t)(t0 - t_begin) * RB;
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int idx = threadIdx.x + u * 256;
      const int row = idx / CPR, ch = idx % CPR;
      if ((TN * CPR) % 256 == 0 || idx < TN * CPR)
        pv[u] = buf_load16(rv, toff + (uint32_t)(row * D + ch * EPC) * sizeof(Tin));
    }
  };
  auto stash = [&](int buf) {
    const U128 *regs = pv;
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int idx = threadIdx.x + u * 256;
      if ((TN * CPR) % 256 == 0 || idx < TN * CPR) {
        const int row = idx / CPR, ch = idx % CPR;
        store_converted16<Tin, TV>(regs[u], &Vs[buf][row * VROW + ch * EPC]);
      }
    }
  };
  // A wave takes blocks tb = tp, tp + TPARTS, ...; the V fragments of the
  // next block are read from LDS while the current block's products run.
  constexpr int NB = 4 / TPARTS;
  auto compute = [&](int cur, int t0) {
    if (!active) return;
    FV vb[2][KS];
    auto load_v = [&](int tb, FV (&vf)[KS]) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        vf[ks] = load8<TV>(&Vs[cur][(tb * 16 + col) * VROW + ks * 32 + 8 * grp]);
    };
    load_v(tp, vb[0]);
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int tb = tp + k * TPARTS;
      if (k + 1 < NB) load_v(tb + TPARTS, vb[(k + 1) & 1]);
      sched_fence();
      const FV (&vf)[KS] = vb[k & 1];
      const int tok = t0 + tb * 16 + col;
      // four partial sums, one per accumulator row, keep the chains short
      float npj[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = db >> 1; ks < KS; ++ks) acc = mma(gf[db][ks], vf[ks], acc);
#pragma unroll
        for (int j = 0; j < 4; ++j) npj[j] += acc[j] * frag_elem(vf[db >> 1], 4 * (db & 1) + j);
      }
      const float np = group4_sum((npj[0] + npj[1]) + (npj[2] + npj[3]));
      // tiles end at or before t_end (a multiple of 64): the lanes of group 0
      // store, the others are dropped by the range check
      buf_store_f32(rn, grp == 0 ? (uint32_t)(tok - t_begin) * 4u : kNoLoad, np);
    }
  };

  // (loads of tiles past the range read nothing, so they are unconditional)
  wait_vmem_all();
  prefetch(t_begin);
  stash(0);
  __syncthreads();
  for (int it = 0; it < nt; ++it) {
    const int t0 = t_begin + it * TN;
    const int cur = it & 1;
    prefetch(t0 + TN);
    compute(cur, t0);
    stash(cur ^ 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Score pass.  One workgroup per (token range, KV head, sequence) serves a
// subset of the group's query heads (all of them when they fit in 8 waves;
// otherwise the host launches the subsets one after another, the later ones
// adding to S).  Each query head's 64 rows are spread over 4/QBW waves.  K
// (and V, converted to the value type) tiles of 64 tokens are staged in LDS
// and shared by the workgroup, double-buffered: the next tile's loads are in
// flight while the current one is computed.  Logits are formed as S = Q K^T
// with tokens across the 16 MFMA columns: a lane owns one token and four
// query rows of each 16-row block, so the sum over query rows is in-lane
// plus two cross-lane adds per 16 tokens; the per-wave partial sums are
// combined across waves in a fixed order.
//   MODE 0 (LORE): out = out_scale * sum_h sum_q wr_q * a/(1-a+eps) * sqrt(|N - 2x + pi|),
//                  x = v . (y_hi + y_lo) as MFMA products whose accumulator
//                  starts at -pi/2, so N - 2*acc = N - 2x + pi; for 16-bit
//                  inputs y_hi . v runs on fp16 MFMA and y_lo . v as one
//                  block-scaled fp8 MFMA (y_lo e4m3 with its row's power-of-
//                  two scale, v e5m2 taken as the upper byte of its fp16
//                  value): y_lo is about 2^-11 of y, so the fp8 roundings
//                  stay near 2^-14 of x;
//                  sqrt(q2)/(1+eps-a) is formed as |q2| * rsqrt(|q2| (1+eps-a)^2
//                  + FLT_MIN).  N - 2x + pi = (v-o)^T G~ (v-o) >= 0 in exact
//                  arithmetic; it goes negative only by rounding when v ~ o,
//                  where |q2| and max(0, q2) give the same magnitude to the
//                  score's accuracy, and the absolute value is a free source
//                  modifier where a clamp would cost an instruction.  Rows of
//                  weight below FLT_MIN contribute nothing.
//   MODE 1 (H2O):  out = sum over causal rows of a
template <typename Tin, int D, int MODE, int MAXW, int QBW>
__global__ void __launch_bounds__(64 * MAXW)
score_kernel(const Tin *__restrict__ Q, const Tin *__restrict__ K, const Tin *__restrict__ V,
             const typename ValueType<Tin>::type *__restrict__ Yhi,
             const typename ValueType<Tin>::type *__restrict__ Ylo,
             const float4 *__restrict__ consts, const float *__restrict__ Nn, int n_pad,
             RowGeom geo, int h_kv, int hv0, int hcount, int accumulate, int tpw, float eps,
             float out_scale, float *__restrict__ S) {
  typedef typename ValueType<Tin>::type TV;
  typedef typename FragOf<Tin>::type FQ;
  typedef typename FragOf<TV>::type FV;
  constexpr bool SPLIT_Y = (MODE == 0) && sizeof(TV) == 2;
  constexpr int KS = D / 32;
  constexpr int TN = 64;
  constexpr int NT = 64 * MAXW;
  constexpr int WPH = 4 / QBW;
  constexpr int EPC = 16 / (int)sizeof(Tin);
  constexpr int CPR = D / EPC;
  // 16-bit rows are padded by 32 bytes: the fragment reads (16 consecutive
  // rows, four 16-byte k-slices per half-wave) then fall in distinct LDS
  // banks, where a 16-byte pad left a two-way conflict on every read
  constexpr int KROW = D + (sizeof(Tin) == 2 ? 16 : EPC);
  constexpr int VROW = D + (sizeof(TV) == 2 ? 16 : 4);
  constexpr int ITEMS = TN * CPR;
  constexpr int PF = (ITEMS + NT - 1) / NT;
  constexpr float kTiny = 1.17549435e-38f;  // FLT_MIN
  // fp8 V row: 128 k-slots (zero past D) in 160 bytes; odd rows hold each
  // pair of 16-byte chunks swapped, which makes the 32-byte fragment reads
  // bank-conflict-free
  constexpr int V8ROW = 128 + 32;
  __shared__ __align__(16) Tin Ks[2][TN * KROW];
  __shared__ __align__(16) TV Vs[MODE == 0 ? 2 : 1][MODE == 0 ? TN * VROW : 8];
  // V as fp8 e5m2 for the y_lo product (one block-scaled 16x16x128 MFMA)
  __shared__ __align__(16) uint8_t V8s[SPLIT_Y ? 2 : 1][SPLIT_Y ? TN * V8ROW : 16];
  // per-lane partial sums: row (wave, row group) of TN tokens.  Rows are 82
  // floats apart: the reads of the per-tile sum (8 consecutive tokens x 8
  // waves, row stride 4*82 = 8 mod 32 banks) hit 32 distinct banks per half-wave.
  constexpr int RROW = TN + 18;
  __shared__ __align__(16) float red[2][MAXW * 4 * RROW];
  // N of the tile's tokens for each wave's own query head
  __shared__ float Ns[MODE == 0 ? 2 : 1][MODE == 0 ? MAXW : 1][MODE == 0 ? TN : 1];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int hl = wv / WPH, qb0 = (wv % WPH) * QBW;
  const int hv = hv0 + hl;
  const bool spare = hl >= hcount;
  const int col = lane & 15, grp = lane >> 4;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int n = geo.n, G = geo.group;
  const long kv_base = ((long)b * h_kv + kvh) * (long)n * D;
  const Tin *Kb = K + kv_base;
  const Tin *Vb = V + kv_base;
  const long head = ((long)b * h_kv + kvh) * G + (spare ? 0 : hv);  // LORE: b*h_q + h
  const float c = kLog2e * rsqrtf((float)D);

  // A fragments: lane (col, grp) supplies query row 16*qb + col.  Results:
  // lane holds query rows 16*qb + 4*grp + j (j = 0..3) for token column col.
  FQ qf[QBW][KS];
  FV yhf[MODE == 0 ? QBW : 1][KS];
  i32x8 yl8[SPLIT_Y ? QBW : 1];  // y_lo row as fp8 e4m3 (k = 32 grp .. 32 grp + 31)
  int ysc[SPLIT_Y ? QBW : 1];     // its E8M0 scale byte
  float beta[QBW][4], rwr[QBW][4];
  f32x4 xinit[QBW];
  int lim[QBW][4];
  int wave_last = -1, wave_first = 0x7FFFFFFF;
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = (qb0 + qb) * 16 + 4 * grp + j;
      const float4 cs = spare ? make_float4(0.f, 0.f, 0.f, __int_as_float(-1)) : consts[head * 64 + r];
      lim[qb][j] = __float_as_int(cs.w);
      // rows without keys get a = 2^-inf = 0 on every path, masked or not
      beta[qb][j] = lim[qb][j] >= 0 ? cs.x : INFINITY;
      xinit[qb][j] = -0.5f * cs.y;
      rwr[qb][j] = 0.f;
      if (MODE == 0) {
        // a * w_r = 2^(e - beta + log2 w_r): the exponent carries the row
        // weight and 1/w_r recovers a for the denominator.  Rows of weight
        // below FLT_MIN contribute nothing: the weights are a softmax times a
        // nonnegative lambda, and below FLT_MIN 1/w_r would overflow to inf
        // and turn 0 * inf into NaN for every token whose a*w_r underflows
        const float w_r = cs.z;
        if (w_r >= kTiny) {
          beta[qb][j] -= log2f(w_r);
          rwr[qb][j] = 1.f / w_r;
        } else {
          beta[qb][j] = INFINITY;
        }
      }
      if (lim[qb][j] >= 0) {
        wave_last = max(wave_last, lim[qb][j]);
        wave_first = min(wave_first, lim[qb][j]);
      }
    }
    const int r = (qb0 + qb) * 16 + col;
    const bool valid = !spare && (geo.mode == 0 ? r < geo.nq : hv * 64 + r < n);
    long qrow;
    if (geo.mode == 0) qrow = head * geo.nq + r;
    else qrow = ((long)b * h_kv + kvh) * n + (long)hv * 64 + r;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[qb][ks] = valid ? load8<Tin>(Q + qrow * D + ks * 32 + 8 * grp) : zero8<Tin>();
      if (MODE == 0)
        yhf[qb][ks] = spare ? zero8<TV>() : load8<TV>(Yhi + (head * 64 + r) * D + ks * 32 + 8 * grp);
    }
    if (SPLIT_Y) {
      const uint8_t *yb = reinterpret_cast<const uint8_t *>(Ylo) + head * (64 * D + 256);
      const bool in_d = 32 * grp < D;  // D = 64: the upper k-slots are zero
      yl8[qb] = (spare || !in_d) ? i32x8{0, 0, 0, 0, 0, 0, 0, 0}
                                 : *reinterpret_cast<const i32x8 *>(yb + r * D + 32 * grp);
      ysc[qb] = spare ? 127 : reinterpret_cast<const int *>(yb + 64 * D)[r];
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    wave_last = max(wave_last, __shfl_xor(wave_last, o, 64));
    wave_first = min(wave_first, __shfl_xor(wave_first, o, 64));
  }

  const int t_begin = blockIdx.x * tpw;
  int t_end = min(n, t_begin + tpw);
  if (MODE == 1 && geo.mode == 1 && accumulate) {
    // causal prompt rows: no row of this head subset sees a token after its
    // last row, so an accumulating launch leaves those tokens untouched
    t_end = min(t_end, min(n, (hv0 + hcount) * 64));
    if (t_end <= t_begin) return;  // (workgroup-uniform)
  }
  const float *Nh = Nn + head * (long)n_pad;
  float *Sout = S + ((long)b * h_kv + kvh) * n;
  const int nt = (t_end - t_begin + TN - 1) / TN;

  U128 pk[PF], pv[MODE == 0 ? PF : 1];
  float pn = 0.f;  // N of token t0 + lane for this wave's head
  constexpr uint32_t RB = D * sizeof(Tin);
  const uint32_t rbytes = range_bytes(t_begin, t_end, RB);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kb + (long)t_begin * D, rbytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vb + (long)t_begin * D, MODE == 0 ? rbytes : 0u);
  const __amdgpu_buffer_rsrc_t rn =
      make_rsrc(Nh + t_begin, MODE == 0 ? range_bytes(t_begin, t_end, 4) : 0u);
  auto prefetch = [&](int t0) {
    const uint32_t toff = (uint32_t)(t0 - t_begin) * RB;
    if (MODE == 0) pn = buf_load_f32(rn, (uint32_t)(t0 - t_begin + lane) * 4u);
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int idx = threadIdx.x + u * NT;
      const int row = idx / CPR, ch = idx % CPR;
      const uint32_t off = toff + (uint32_t)(row * D + ch * EPC) * sizeof(Tin);
      if (ITEMS % NT == 0 || idx < ITEMS) {
        pk[u] = buf_load16(rk, off);
        if (MODE == 0) pv[u] = buf_load16(rv, off);
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int idx = threadIdx.x + u * NT;
      if (ITEMS % NT == 0 || idx < ITEMS) {
        const int row = idx / CPR, ch = idx % CPR;
        *reinterpret_cast<U128 *>(&Ks[buf][row * KROW + ch * EPC]) = pk[u];
        if (MODE == 0) {
          const U128 hv = convert16<Tin, TV>(pv[u]);
          *reinterpret_cast<U128 *>(&Vs[buf][row * VROW + ch * EPC]) = hv;
          if constexpr (SPLIT_Y)  // 8 fp8 bytes: half ch % 2 of 16-byte chunk ch / 2
            *reinterpret_cast<uint2 *>(&V8s[buf][row * V8ROW + ((((ch >> 1) ^ (row & 1)) << 4) | ((ch & 1) << 3))]) =
                e5m2_of_f16x8(hv);
        }
      }
    }
    if (MODE == 0) Ns[buf][wv][lane] = pn;
  };

  // One 16-token block: this lane's sum over its 4*QBW query rows for token
  // tok0 + col.  The K and V fragments of a block are read from LDS one block
  // ahead, so their latency hides behind the previous block's work.
  auto load_frags = [&](int cur, int tb, FQ (&kf)[KS], FV (&vf)[MODE == 0 ? KS : 1],
                        i32x8 &v8) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = load8<Tin>(&Ks[cur][(tb * 16 + col) * KROW + ks * 32 + 8 * grp]);
      if (MODE == 0) vf[ks] = load8<TV>(&Vs[cur][(tb * 16 + col) * VROW + ks * 32 + 8 * grp]);
    }
    if constexpr (SPLIT_Y) {
      // B fragment of the 16x16x128 product: token tb*16 + col, k = 32 grp .. +31
      // (with D = 64 the upper lanes hold zeros: their LDS slots are never written)
      if (32 * grp < D) {
        const int r8 = tb * 16 + col;
        const uint8_t *p8 = &V8s[cur][r8 * V8ROW];
        const U128 a = *reinterpret_cast<const U128 *>(p8 + (((2 * grp) ^ (r8 & 1)) << 4));
        const U128 b2 = *reinterpret_cast<const U128 *>(p8 + (((2 * grp + 1) ^ (r8 & 1)) << 4));
        v8 = i32x8{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b2.x, (int)b2.y, (int)b2.z, (int)b2.w};
      } else {
        v8 = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  };
  auto block = [&](auto masked, int tok0, float nv, const FQ (&kf)[KS],
                   const FV (&vf)[MODE == 0 ? KS : 1], const i32x8 &v8) -> float {
    constexpr bool MASKED = decltype(masked)::value;
    f32x4 sa[QBW], xa[QBW];
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s4 = mma(qf[qb][ks], kf[ks], s4);
      sa[qb] = s4;
    }
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
      f32x4 x4 = xinit[qb];
      if (MODE == 0) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) x4 = mma(yhf[qb][ks], vf[ks], x4);
      }
      if constexpr (SPLIT_Y)  // y_lo (e4m3, row scale 2^-k) times V (e5m2), K = 128
        x4 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(yl8[qb], v8, x4, 0, 1, 0, ysc[qb],
                                                               0, 127);
      xa[qb] = x4;
    }
    const int tok = tok0 + col;
    float tacc = 0.f;
#pragma unroll
    for (int qb = 0; qb < QBW; ++qb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float e = fmaf(sa[qb][j], c, -beta[qb][j]);
        if (MASKED && tok > lim[qb][j]) e = -INFINITY;
        if (MODE == 1) {
          tacc += hw_exp2(e);
        } else {
          // aw = a * w_r;  u = sqrt(|q2|) / (1 + eps - a) as |q2| rsqrt(|q2| den^2 + tiny)
          const float aw = hw_exp2(e);
          const float den = fmaf(-aw, rwr[qb][j], 1.f + eps);
          const float q2 = fabsf(fmaf(-2.f, xa[qb][j], nv));
          const float p = q2 * den;
          const float u = q2 * hw_rsq(fmaf(p, den, kTiny));
          tacc = fmaf(aw, u, tacc);
        }
      }
    }
    return tacc;
  };
  // Every wave sums the partials of TN / MAXW tokens of a finished tile: lane
  // (token u, wave part p) adds the four row groups of wave p, then the MAXW
  // parts of a token are added across lanes (u + TPW * p, p = 0..MAXW-1).
  constexpr int TPW = TN / MAXW;
  auto reduce_load = [&](int buf) -> float {
    const int u = lane % TPW, p = lane / TPW;
    const float *rp = &red[buf][(p * 4) * RROW + wv * TPW + u];
    return (rp[0] + rp[RROW]) + (rp[2 * RROW] + rp[3 * RROW]);
  };
  auto reduce_store = [&](float sum, int t0p) {
    if (TPW <= 8) sum = sum_xor8(sum);
    if (TPW <= 16) sum = sum_xor16(sum);
    if (TPW <= 32) sum = sum_xor32(sum);
    const int tok = t0p + wv * TPW + lane % TPW;
    if (lane < TPW && tok < t_end) {
      sum *= out_scale;
      // a later head-subset launch adds to S with a non-returning atomic:
      // no wait on a load of S (which would also wait for the tile loads in
      // flight), and one add per element per launch in stream order is the
      // same sum as a load-add-store
      if (accumulate) unsafeAtomicAdd(&Sout[tok], sum);
      else Sout[tok] = sum;
    }
  };
  auto tile = [&](auto masked, int cur, int t0, bool pending, float part) {
    FQ kb[2][KS];
    FV vb[2][MODE == 0 ? KS : 1];
    i32x8 v8b[2];
    float nv[TN / 16];
#pragma unroll
    for (int tb = 0; tb < TN / 16; ++tb) nv[tb] = (MODE == 0) ? Ns[cur][wv][tb * 16 + col] : 0.f;
    load_frags(cur, 0, kb[0], vb[0], v8b[0]);
#pragma unroll
    for (int tb = 0; tb < TN / 16; ++tb) {
      if (tb + 1 < TN / 16)
        load_frags(cur, tb + 1, kb[(tb + 1) & 1], vb[(tb + 1) & 1], v8b[(tb + 1) & 1]);
      sched_fence();
      const float tsum = block(masked, t0 + tb * 16, nv[tb], kb[tb & 1], vb[tb & 1], v8b[tb & 1]);
      red[cur][(wv * 4 + grp) * RROW + tb * 16 + col] = tsum;
      if (tb == 0 && pending) reduce_store(part, t0 - TN);
      // a wave further ahead in the tile yields issue priority to the wave
      // sharing its SIMD, so both reach the tile barrier together
      if (tb == 0) __builtin_amdgcn_s_setprio(2);
      else if (tb == 1) __builtin_amdgcn_s_setprio(1);
      else if (tb == 2) __builtin_amdgcn_s_setprio(0);
    }
    __builtin_amdgcn_s_setprio(3);
  };

  __builtin_amdgcn_s_setprio(3);
  wait_vmem_all();
  prefetch(t_begin);
  stash(0);
  __syncthreads();
#pragma clang loop unroll(disable)
  for (int it = 0; it < nt; ++it) {
    const int t0 = t_begin + it * TN;
    const int cur = it & 1;
    prefetch(t0 + TN);  // past the range this reads nothing
    // the previous tile's sums are read now and finished after this tile's
    // first block, so their LDS latency hides behind the products
    const float part = it > 0 ? reduce_load(cur ^ 1) : 0.f;
    if (t0 > wave_last) {
#pragma unroll
      for (int tb = 0; tb < TN / 16; ++tb) red[cur][(wv * 4 + grp) * RROW + tb * 16 + col] = 0.f;
      if (it > 0) reduce_store(part, t0 - TN);
    } else if (t0 + TN - 1 > wave_first) {
      tile(std::true_type{}, cur, t0, it > 0, part);
    } else {
      tile(std::false_type{}, cur, t0, it > 0, part);
    }
    stash(cur ^ 1);
    __syncthreads();
  }
  if (nt > 0) reduce_store(reduce_load((nt - 1) & 1), t_begin + (nt - 1) * TN);
}

// ---------------------------------------------------------------------------
template <typename Tin, int D>
static hipError_t run_gram(const void *W, int dm, int h_q, int splits, float *Gpart,
                           hipStream_t st) {
  constexpr int SR = GramStage<Tin>::rows;
  const int slabs = (dm + SR - 1) / SR;
  const int rps = (slabs + splits - 1) / splits * SR;
  if (rps > kGramStages * SR) return hipErrorInvalidValue;  // splits from gram_splits()
  {
    TimedLaunch tl_("gram", st);
    hipLaunchKernelGGL((gram_kernel<Tin, D>), dim3(splits, h_q), dim3(256), 0, st, (const Tin *)W,
                       dm, h_q, rps, Gpart);
  }
  return hipGetLastError();
}

hipError_t launch_gram(int etype, int d, const void *W_O, int d_model, int h_q, int splits,
                       float *Gpart, hipStream_t st) {
#define KVS_G(T, DD) return run_gram<T, DD>(W_O, d_model, h_q, splits, Gpart, st)
  if (etype == E_F32) { if (d == 64) KVS_G(float, 64); KVS_G(float, 128); }
  if (etype == E_BF16) { if (d == 64) KVS_G(bf16, 64); KVS_G(bf16, 128); }
  if (d == 64) KVS_G(f16, 64);
  KVS_G(f16, 128);
#undef KVS_G
}

// Row constants of the prompt-side baselines, read by score_kernel<1> (a
// plain sum of probabilities): window row r keeps beta2 = row_max*log2(e) +
// log2(row_sum) and its last visible key n - w + r; rows outside the chosen
// set (lookahead rows, padding, and for the single-query form every window
// row but the last) get last = -1, which the score pass treats as a row
// without keys (a = 0).
__global__ void __launch_bounds__(64)
baseline_prep_kernel(const float *__restrict__ row_max, const float *__restrict__ row_sum,
                     int n, int nq, int w, int last_only, float4 *__restrict__ consts) {
  const long hb = blockIdx.x;
  const int r = threadIdx.x;
  const bool used = r < nq && r < w && (!last_only || r == w - 1);
  float beta2 = 0.f;
  int last = -1;
  if (used) {
    beta2 = row_max[hb * nq + r] * kLog2e + log2f(row_sum[hb * nq + r]);
    last = n - w + r;
  }
  consts[hb * 64 + r] = make_float4(beta2, 0.f, 1.f, __int_as_float(last));
}

hipError_t launch_baseline_prep(const float *row_max, const float *row_sum, int batch, int h_q,
                                int n, int nq, int w, bool last_only, float4 *consts,
                                hipStream_t st) {
  {
    TimedLaunch tl_("baseline_prep", st);
    hipLaunchKernelGGL(baseline_prep_kernel, dim3(batch * h_q), dim3(64), 0, st, row_max, row_sum,
                       n, nq, w, last_only ? 1 : 0, consts);
  }
  return hipGetLastError();
}

template <int D, typename TV>
static hipError_t run_prep(const float *Gpart, int gsplits, const float *O, const float *row_max,
                           const float *row_sum, const float *omega, int batch, int h_q, int n,
                           int nq, int w, int m, int t, float lambda_l, void *Gv, float *Gr,
                           void *Yhi, void *Ylo, float4 *consts, hipStream_t st) {
  {
    TimedLaunch tl_("gram_reduce", st);
    constexpr int NT = D / 32;
    hipLaunchKernelGGL((gram_reduce_kernel<D, TV>), dim3(NT * (NT + 1) / 2, h_q), dim3(256), 0, st,
                       Gpart, gsplits, h_q, (TV *)Gv, Gr);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    TimedLaunch tl_("deletion_prep", st);
    if constexpr (sizeof(TV) == 2)
      hipLaunchKernelGGL((prep_mfma_kernel<D>), dim3(h_q, batch), dim3(256), 0, st,
                         (const f16 *)Gv, O, row_max, row_sum, omega, h_q, n, nq, w, m, t,
                         lambda_l, (f16 *)Yhi, (uint8_t *)Ylo, consts);
    else
      hipLaunchKernelGGL((prep_kernel<D, TV>), dim3(h_q, batch, 4), dim3(256), 0, st, Gr, O,
                         row_max, row_sum, omega, h_q, n, nq, w, m, t, lambda_l, (TV *)Yhi,
                         (TV *)Ylo, consts);
  }
  return hipGetLastError();
}

hipError_t launch_deletion_prep(int etype, int d, const float *Gpart, int gsplits, const float *O,
                                const float *row_max, const float *row_sum, const float *omega,
                                int batch, int h_q, int n, int nq, int w, int m, int t,
                                float lambda_l, void *Gv, float *Gr, void *Yhi, void *Ylo,
                                float4 *consts, hipStream_t st) {
#define KVS_P(DD, TV) \
  return run_prep<DD, TV>(Gpart, gsplits, O, row_max, row_sum, omega, batch, h_q, n, nq, w, m, t, \
                          lambda_l, Gv, Gr, Yhi, Ylo, consts, st)
  if (etype == E_F32) { if (d == 64) KVS_P(64, float); KVS_P(128, float); }
  if (d == 64) KVS_P(64, f16);
  KVS_P(128, f16);
#undef KVS_P
}

template <typename Tin, int D>
static hipError_t run_vnorm(const void *V, const void *Gv, int batch, int n, int n_pad, int h_q,
                            int h_kv, float *Nn, hipStream_t st) {
  typedef typename ValueType<Tin>::type TV;
  // about 768 workgroups (three per CU at <= 168 VGPRs) of whole 64-token tiles
  const int G = h_q / h_kv;
  const int hpw = G < 4 ? G : 4;
  const long units = (long)((G + hpw - 1) / hpw) * h_kv * batch;
  const int tiles = n_pad / 64;
  const long want = std::max(1L, 768L / units);  // three workgroups per CU
  const int tpw = std::min(64 * (int)((tiles + want - 1) / want), kMaxRangeTokens);
  const int nchunk = (n_pad + tpw - 1) / tpw;
  const long blocks = (long)nchunk * units;
  {
    TimedLaunch tl_("vnorm", st);
#define KVS_VN(TP)                                                                            \
  hipLaunchKernelGGL((vnorm_kernel<Tin, D, TP>), dim3((unsigned)blocks), dim3(256), 0, st,    \
                     (const Tin *)V, (const TV *)Gv, n, n_pad, h_q, h_kv, tpw, nchunk, Nn)
    if (4 / hpw == 4) KVS_VN(4);
    else if (4 / hpw == 2) KVS_VN(2);
    else KVS_VN(1);
#undef KVS_VN
  }
  return hipGetLastError();
}

hipError_t launch_vnorm(int etype, int d, const void *V, const void *Gv, int batch, int n,
                        int n_pad, int h_q, int h_kv, float *Nn, hipStream_t st) {
#define KVS_V(T, DD) return run_vnorm<T, DD>(V, Gv, batch, n, n_pad, h_q, h_kv, Nn, st)
  if (etype == E_F32) { if (d == 64) KVS_V(float, 64); KVS_V(float, 128); }
  if (etype == E_BF16) { if (d == 64) KVS_V(bf16, 64); KVS_V(bf16, 128); }
  if (d == 64) KVS_V(f16, 64);
  KVS_V(f16, 128);
#undef KVS_V
}

template <typename Tin, int D, int MODE, int MAXW, int QBW>
static hipError_t run_score_w(const void *Q, const void *K, const void *V, const void *Yhi,
                              const void *Ylo, const float4 *consts, const float *Nn, int n_pad,
                              RowGeom geo, int batch, int h_kv, int hpw, float eps,
                              float out_scale, float *S, hipStream_t st) {
  typedef typename ValueType<Tin>::type TV;
  if (hpw < 1 || hpw * (4 / QBW) > MAXW) return hipErrorInvalidConfiguration;
  const long units = (long)batch * h_kv;
  // LORE (MODE 0): about one workgroup per CU (256 on MI355X; its LDS admits
  // one per CU), each over a long token range, so each workgroup's set-up
  // (query and y fragments, row constants) is paid once per CU: 11% faster
  // than ~1024 shorter workgroups.  MODE 1 (no value tiles, two workgroups
  // per CU fit) takes ~512: 5% faster than 1024 on the window score, while
  // 256 left half of each CU's slots empty (22% slower).
  const long target = MODE == 0 ? 256 : 512;
  long tpw = ((long)geo.n * units + target - 1) / target;
  tpw = (tpw + 63) / 64 * 64;
  if (tpw < 64) tpw = 64;
  if (tpw > kMaxRangeTokens) tpw = kMaxRangeTokens;
  const int blocks = (int)((geo.n + tpw - 1) / tpw);
  // head subsets in stream order, the later ones adding to S.  Causal prompt
  // rows (geo.mode 1) go from the last subset to the first: the first launch
  // covers (and writes) every token, and each later one only the tokens up
  // to its own last row.
  const int nsub = (geo.group + hpw - 1) / hpw;
  for (int k = 0; k < nsub; ++k) {
    const int hv0 = (geo.mode == 1 ? nsub - 1 - k : k) * hpw;
    const int hcount = std::min(hpw, geo.group - hv0);
    {
      TimedLaunch tl_((MODE == 0 ? "score_lore" : "score_h2o_colsum"), st);
      hipLaunchKernelGGL((score_kernel<Tin, D, MODE, MAXW, QBW>), dim3(blocks, h_kv, batch),
                         dim3(64 * MAXW), 0, st, (const Tin *)Q, (const Tin *)K, (const Tin *)V,
                         (const TV *)Yhi, (const TV *)Ylo, consts, Nn, n_pad, geo, h_kv, hv0,
                         hcount, k > 0 ? 1 : 0, (int)tpw, eps, out_scale, S);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// At most 8 waves per workgroup: a query head takes 4/QBW waves (QBW = 2 for
// LORE, whose row constants and y fragments fill the registers; 4 for H2O),
// and larger groups run as several launches over head subsets of balanced size.
template <typename Tin, int D>
static hipError_t run_score(int mode, const void *Q, const void *K, const void *V, const void *Yhi,
                            const void *Ylo, const float4 *consts, const float *Nn, int n_pad,
                            RowGeom geo, int batch, int h_kv, float eps, float out_scale, float *S,
                            hipStream_t st) {
  const int wph = mode == 1 ? 1 : 2;
  const int hmax = 8 / wph;
  const int nl = (geo.group + hmax - 1) / hmax;
  const int hpw = (geo.group + nl - 1) / nl;
  const int waves = hpw * wph;
#define KVS_RS(MODE, MAXW, QBW)                                                                \
  return run_score_w<Tin, D, MODE, MAXW, QBW>(Q, K, V, Yhi, Ylo, consts, Nn, n_pad, geo, batch, \
                                              h_kv, hpw, eps, out_scale, S, st)
  if (mode == 1) {
    if (waves <= 2) KVS_RS(1, 2, 4);
    if (waves <= 4) KVS_RS(1, 4, 4);
    KVS_RS(1, 8, 4);
  }
  if (waves <= 2) KVS_RS(0, 2, 2);
  if (waves <= 4) KVS_RS(0, 4, 2);
  KVS_RS(0, 8, 2);
#undef KVS_RS
}

hipError_t launch_score(int etype, int d, int mode, const void *Q, const void *K, const void *V,
                        const void *Yhi, const void *Ylo, const float4 *consts, const float *Nn,
                        int n_pad, RowGeom geo, int batch, int h_kv, float eps, float out_scale,
                        float *S, hipStream_t st) {
#define KVS_S(T, DD) \
  return run_score<T, DD>(mode, Q, K, V, Yhi, Ylo, consts, Nn, n_pad, geo, batch, h_kv, eps, \
                          out_scale, S, st)
  if (etype == E_F32) { if (d == 64) KVS_S(float, 64); KVS_S(float, 128); }
  if (etype == E_BF16) { if (d == 64) KVS_S(bf16, 64); KVS_S(bf16, 128); }
  if (d == 64) KVS_S(f16, 64);
  KVS_S(f16, 128);
#undef KVS_S
}

}  // namespace kvs
