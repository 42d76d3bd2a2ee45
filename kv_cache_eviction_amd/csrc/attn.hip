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
// One workgroup per (token split, KV head, sequence) holds 4/QBW wavefronts
// per query head for up to 8 waves (larger groups are split over several
// workgroups), so a K/V tile staged in LDS is read once for all the query
// heads it serves.  The logits are formed transposed, S^T = K Q^T (tokens down the
// rows, query rows across the 16 columns): every lane then owns one query
// column, keeps that row's running max/sum in registers, and its eight
// accumulator values are eight tokens of that row.  Loading the K rows in the
// permuted order token(tb, rho) = 8*(rho/4) + 4*tb + rho%4 makes those eight
// tokens consecutive (8*(lane/16) + 0..7), which is exactly the k-slot order
// of a B fragment, so P^T enters the P.V product straight from registers.
// V is staged transposed (and converted to fp16 for 16-bit inputs) so the A
// fragment of O^T = V^T P^T is one 16-byte LDS read.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "timing.hpp"

namespace kvs {

// Mode 2 (counter-causal): virtual head hv = (query head in the group) * nq
// + j, and j names 64-row block rev_block(j): row position R = block * 64 + r
// sees keys R+1 .. n-1, so early blocks see most of the cache and late ones
// little.  A workgroup takes four consecutive virtual heads, the 2 x 4 waves
// two per head, and wave w runs on SIMD w % 4.  The blocks are laid out so
// that each group of four j holds two early and two late blocks, in the
// order (a, a+1, n_b-1-a, n_b-2-a): every workgroup then carries about the
// same work, and every SIMD pairs a wave of an early block with one of a
// late block, so a SIMD whose short wave has finished still has a long one.
// (The zigzag 0, n_b-1, 1, n_b-2, ... with the middle two of each full group
// of four swapped; a bijection on the n_b blocks.)
__device__ __forceinline__ int rev_block(const RowGeom &g, int hv) {
  const int nb = g.nq, j = hv % nb;
  const int q = (j < nb - nb % 4 && (j & 3) == 1) ? j + 1 : (j < nb - nb % 4 && (j & 3) == 2) ? j - 1 : j;
  return (q & 1) ? nb - 1 - (q >> 1) : (q >> 1);
}

// Last key row r of virtual head hv sees (-1: none).  The counter-causal
// forms (REV) are compiled only into the kernels launched with mode 2.
template <bool REV>
__device__ __forceinline__ int row_last(const RowGeom &g, int hv, int r) {
  if constexpr (REV) {
    const int R = rev_block(g, hv) * 64 + r;
    return R < g.n - 1 ? g.n - 1 : -1;
  }
  if (g.mode == 0) {
    if (r >= g.nq) return -1;
    return r < g.w ? g.n - g.w + r : g.n - 1;
  }
  const int R = hv * 64 + r;
  return R < g.n ? R : -1;
}

// First key row r of virtual head hv sees (mode 2 only; 0 otherwise).
template <bool REV>
__device__ __forceinline__ int row_first(const RowGeom &g, int hv, int r) {
  if constexpr (REV) return rev_block(g, hv) * 64 + r + 1;
  return 0;
}

// Index of scoring row r of query head hv (within KV head kvh's group) in Q.
template <bool REV>
__device__ __forceinline__ long q_row(const RowGeom &g, int b, int h_kv, int kvh, int hv, int r) {
  if constexpr (REV)  // Q [b][h_q][n][d], query head kvh * G + hv / nq
    return (((long)b * h_kv + kvh) * (g.group / g.nq) + hv / g.nq) * g.n + (long)rev_block(g, hv) * 64 + r;
  if (g.mode == 0) return (((long)b * h_kv + kvh) * g.group + hv) * g.nq + r;
  return ((long)b * h_kv + kvh) * g.n + (long)hv * 64 + r;
}

// LDS row of tile token t in the pass-1 K tile.  Block tb of the tile takes
// token t = 32 (tb / 2) + 8 (col / 4) + 4 (tb % 2) + col % 4 into MFMA column
// col (the order that makes each lane's logits the B-fragment k order of the
// P.V product); storing that token in row 16 tb + col makes the fragment
// reads walk 16 consecutive rows.
__device__ __forceinline__ int kslot(int t) {
  const int tb = ((t >> 5) << 1) | ((t >> 2) & 1);
  const int cl = (((t >> 3) & 3) << 2) | (t & 3);
  return tb * 16 + cl;
}

// QBW = 16-row query blocks per wave: a query head's 64 rows are spread over
// 4/QBW waves.  Tiles of 64 tokens are double-buffered in LDS: the next tile's
// global loads go to registers before the current tile is computed and into
// the other buffer after, so one barrier per tile separates the two.
//
// Online softmax with a lazy reference: p = 2^(s*c - m_ref) is formed against
// a per-row reference m_ref that is raised (and O, l rescaled) only when a
// tile's maximum exceeds it by more than kSlack, so most tiles skip the
// rescale; p then stays below 2^kSlack, well inside fp16.  The exact running
// maximum is tracked beside it and the partial (l, O) are brought to it once
// at the end, so the split outputs are the plain (max, sum, unnormalised O).
// The visibility mask is applied only on tiles that cross some row's last
// visible key (or the end of the cache).  REV (counter-causal rows, mode 2)
// adds a first visible key per row: tiles wholly before a wave's rows are
// skipped, a workgroup starts at the tile of its rows' earliest key, and the
// tiles that cross a row's first key are masked too.  Counter-causal rows are
// launched unsplit and write their final rows from the epilogue.
template <typename Tin, int D, bool WITH_O, int MAXW, int QBW, bool REV = false>
__global__ void __launch_bounds__(64 * MAXW)
attn_partial_kernel(const Tin *__restrict__ Q, const Tin *__restrict__ K, const Tin *__restrict__ V,
                    RowGeom geo, int h_kv, int hsplit, int hpw, int tps, int splits,
                    float *__restrict__ pm, float *__restrict__ pl, float *__restrict__ pO) {
  typedef typename ValueType<Tin>::type TV;
  typedef typename FragOf<Tin>::type FQ;
  typedef typename FragOf<TV>::type FV;
  constexpr int KS = D / 32;
  constexpr int DB = D / 16;
  constexpr int TN = 64;
  constexpr int TB = TN / 16;                 // 16-token blocks per tile
  constexpr int WPH = 4 / QBW;                // waves per query head
  constexpr int EPC = 16 / (int)sizeof(Tin);  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                // chunks per row
  constexpr bool V16 = sizeof(TV) == 2;
  // padded LDS rows (elements).  16-bit rows carry 32 bytes of pad, which
  // puts the 16-byte fragment reads of 16 consecutive rows (four k-slices
  // per half-wave) in distinct banks; a 16-byte pad conflicted two ways
  constexpr int KROW = D + (sizeof(Tin) == 2 ? 16 : EPC);
  constexpr int VROW = TN + (V16 ? 16 : 4);
  constexpr float kSlack = 8.f;
  // K items: one 16-byte chunk; V items: a row pair (16-bit) or one row (fp32)
  constexpr int KITEMS = TN * CPR;
  constexpr int VITEMS = V16 ? (TN / 2) * CPR : TN * CPR;
  constexpr int NT = 64 * MAXW;  // threads per workgroup
  constexpr int PFK = (KITEMS + NT - 1) / NT;
  constexpr int PFV = (VITEMS + NT - 1) / NT;
  __shared__ __align__(16) Tin Ks[2][TN * KROW];
  __shared__ __align__(16) TV Vt[WITH_O ? 2 : 1][WITH_O ? D * VROW : 8];

  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int s = blockIdx.x, kvh = blockIdx.y / hsplit, b = blockIdx.z;
  // this workgroup serves query heads [hs*hpw, hs*hpw + hpw) of the group
  const int hs = blockIdx.y % hsplit, hl = wv / WPH;
  const int hv = hs * hpw + hl, qb0 = (wv % WPH) * QBW;
  const bool spare = hl >= hpw || hv >= geo.group;
  const int col = lane & 15, grp = lane >> 4;
  const int n = geo.n;
  const long kv_base = ((long)b * h_kv + kvh) * (long)n * D;
  const Tin *Kb = K + kv_base;
  const Tin *Vb = V + kv_base;
  const int t_begin = s * tps;
  const int t_end = min(n, t_begin + tps);
  const int nt = (t_end - t_begin + TN - 1) / TN;
  const float c = kLog2e * rsqrtf((float)D);

  FQ qf[QBW][KS];
  int lim[QBW], lo[QBW];
  int wave_last = -1, wave_first = 0x7FFFFFFF;  // over this wave's visible rows
  int wave_lo_min = 0x7FFFFFFF, wave_lo_max = 0;  // REV: earliest and latest first keys
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int r = (qb0 + qb) * 16 + col;
    lim[qb] = spare ? -1 : row_last<REV>(geo, hv, r);  // spare waves only stage tiles
    lo[qb] = row_first<REV>(geo, hv, r);
    if (lim[qb] >= 0) {
      wave_last = max(wave_last, lim[qb]);
      wave_first = min(wave_first, lim[qb]);
      if (REV) {
        wave_lo_min = min(wave_lo_min, lo[qb]);
        wave_lo_max = max(wave_lo_max, lo[qb]);
      }
      const Tin *qp = Q + q_row<REV>(geo, b, h_kv, kvh, hv, r) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = load8<Tin>(qp + ks * 32 + 8 * grp);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[qb][ks] = zero8<Tin>();
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    wave_last = max(wave_last, __shfl_xor(wave_last, o, 64));
    wave_first = min(wave_first, __shfl_xor(wave_first, o, 64));
    if (REV) {
      wave_lo_min = min(wave_lo_min, __shfl_xor(wave_lo_min, o, 64));
      wave_lo_max = max(wave_lo_max, __shfl_xor(wave_lo_max, o, 64));
    }
  }

  // mref: reference max of the exponentials (log2 units), negm = -mref (0
  // while no key has been visible); mtop: exact running max; lsum: this
  // lane's share of the row sum against mref.
  float mref[QBW], negm[QBW], mtop[QBW], lsum[QBW];
  f32x4 oacc[WITH_O ? DB : 1][QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    mref[qb] = -INFINITY;
    negm[qb] = 0.f;
    mtop[qb] = -INFINITY;
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
  // Tile loads go through a buffer resource over the tile's valid rows: rows
  // past the end of the cache read as zeros (their logits are masked).
  constexpr uint32_t RB = D * sizeof(Tin);  // row bytes
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kb + (long)t_begin * D, range_bytes(t_begin, t_end, RB));
  const __amdgpu_buffer_rsrc_t rv =
      make_rsrc(Vb + (long)t_begin * D, WITH_O ? range_bytes(t_begin, t_end, RB) : 0u);
  auto prefetch = [&](int t0) {
    const uint32_t toff = (uint32_t)(t0 - t_begin) * RB;
#pragma unroll
    for (int u = 0; u < PFK; ++u) {
      const int idx = threadIdx.x + u * NT;
      const int row = idx / CPR, ch = idx % CPR;
      if (KITEMS % NT == 0 || idx < KITEMS)
        pk[u] = buf_load16(rk, toff + (uint32_t)(row * D + ch * EPC) * sizeof(Tin));
    }
    if (WITH_O) {
#pragma unroll
      for (int u = 0; u < PFV; ++u) {
        const int idx = threadIdx.x + u * NT;
        if (VITEMS % NT != 0 && idx >= VITEMS) continue;
        if constexpr (V16) {
          const int kp = idx % (TN / 2), ch = idx / (TN / 2);
          const uint32_t off = toff + (uint32_t)(2 * kp * D + ch * EPC) * sizeof(Tin);
          pv[u][0] = buf_load16(rv, off);
          pv[u][V16 ? 1 : 0] = buf_load16(rv, off + D * sizeof(Tin));
        } else {
          const int r = idx % TN, ch = idx / TN;
          pv[u][0] = buf_load16(rv, toff + (uint32_t)(r * D + ch * EPC) * sizeof(Tin));
        }
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PFK; ++u) {
      const int idx = threadIdx.x + u * NT;
      if (KITEMS % NT == 0 || idx < KITEMS) {
        const int row = idx / CPR, ch = idx % CPR;
        *reinterpret_cast<U128 *>(&Ks[buf][kslot(row) * KROW + ch * EPC]) = pk[u];
      }
    }
    if (WITH_O) {
#pragma unroll
      for (int u = 0; u < PFV; ++u) {
        const int idx = threadIdx.x + u * NT;
        if (VITEMS % NT != 0 && idx >= VITEMS) continue;
        if constexpr (V16) {
          const int kp = idx % (TN / 2), ch = idx / (TN / 2);
          const Elems16<Tin> ae = elems16<Tin>(pv[u][0]);
          const Elems16<Tin> be = elems16<Tin>(pv[u][V16 ? 1 : 0]);
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            uint32_t packed;
            if constexpr (__is_same(Tin, bf16) && __is_same(TV, f16))
              // exact in the fp16 normal range: round-toward-zero changes nothing there
              packed = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(to_f32(ae.e[e]), to_f32(be.e[e])));
            else
              packed = bits16(from_f32<TV>(to_f32(ae.e[e]))) | (bits16(from_f32<TV>(to_f32(be.e[e]))) << 16);
            *reinterpret_cast<uint32_t *>(&Vt[buf][(ch * EPC + e) * VROW + 2 * kp]) = packed;
          }
        } else {
          const int r = idx % TN, ch = idx / TN;
          const Elems16<Tin> ae = elems16<Tin>(pv[u][0]);
#pragma unroll
          for (int e = 0; e < EPC; ++e) Vt[buf][(ch * EPC + e) * VROW + r] = from_f32<TV>(to_f32(ae.e[e]));
        }
      }
    }
  };

  // REV: no row of this workgroup sees a key before its heads' earliest first
  // key, so the tiles before it are neither loaded nor computed
  int it0 = 0;
  if (REV) {
    int wg_lo = 0x7FFFFFFF;
    for (int h2 = 0; h2 < hpw; ++h2) {
      const int v = hs * hpw + h2;
      if (v < geo.group) wg_lo = min(wg_lo, rev_block(geo, v) * 64 + 1);
    }
    if (wg_lo > t_begin) it0 = min(nt, (wg_lo - t_begin) / TN);
  }
  // causal prompt rows (mode 1): no row of this workgroup sees a key after
  // its last head's last row, so the tiles past it are neither loaded nor
  // stepped through (their rows' statistics come out empty for this split)
  int it_end = nt;
  if (!REV && geo.mode == 1) {
    const int wg_last = min(n - 1, min(geo.group, hs * hpw + hpw) * 64 - 1);
    it_end = wg_last < t_begin ? 0 : min(nt, (wg_last - t_begin) / TN + 1);
  }
  wait_vmem_all();
  prefetch(t_begin + it0 * TN);
  stash(it0 & 1);
  __syncthreads();
  for (int it = it0; it < it_end; ++it) {
    const int t0 = t_begin + it * TN;
    const int cur = it & 1;
    prefetch(t0 + TN);  // past the split end this reads nothing
    // a tile's causal masking is compiled only into the tiles that need it
    auto tile = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
      // S^T for the tile: block tb holds tokens (tb/2)*32 + 8*(row/4) + 4*(tb%2) + row%4.
      // LDS fragments are read one step ahead of the products that use them.
      // (the stash put that token in LDS row 16 tb + col)
      auto load_k = [&](int tb, FQ (&kf)[KS]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = load8<Tin>(&Ks[cur][(tb * 16 + col) * KROW + ks * 32 + 8 * grp]);
      };
      // P.V steps: (half h of the tile, 16-row block db of d), step = h * DB + db
      constexpr int PVS = WITH_O ? (TB / 2) * DB : 1;
      constexpr int VW = 4;  // V fragments in flight
      auto load_v = [&](int step) -> FV {
        const int h = step / DB, db = step % DB;
        return load8<TV>(&Vt[cur][(db * 16 + col) * VROW + h * 32 + 8 * grp]);
      };
      f32x4 sacc[TB][QBW];
      FQ kb[2][KS];
      load_k(0, kb[0]);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        if (tb + 1 < TB) load_k(tb + 1, kb[(tb + 1) & 1]);
        sched_fence();
        const FQ (&kf)[KS] = kb[tb & 1];
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) acc = mma(kf[ks], qf[qb][ks], acc);
          sacc[tb][qb] = acc;
        }
      }
      // Lane (col, grp) holds tokens t0 + (tb/2)*32 + 8*grp + 4*(tb%2) + j.
      if constexpr (MASKED) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int qb = 0; qb < QBW; ++qb)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int tok = t0 + (tb >> 1) * 32 + 8 * grp + 4 * (tb & 1) + j;
              if (tok > lim[qb] || (REV && tok < lo[qb])) sacc[tb][qb][j] = -INFINITY;
            }
      }

      // the first V fragments land while the softmax runs
      FV vq[VW];
      if (WITH_O) {
#pragma unroll
        for (int k = 0; k < VW; ++k) vq[k] = load_v(k);
      }
      sched_fence();
      FV pf[TB / 2][QBW];
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sacc[tb][qb][j]);
        mx = group4_max(mx);
        const float mxs = mx * c;
        mtop[qb] = fmaxf(mtop[qb], mxs);
        if (__any(mxs > mref[qb] + kSlack)) {
          const float mnew = fmaxf(mref[qb], mxs);
          const float alpha = (mnew == -INFINITY) ? 1.f : hw_exp2(mref[qb] - mnew);
          mref[qb] = mnew;
          negm[qb] = (mnew == -INFINITY) ? 0.f : -mnew;
          lsum[qb] *= alpha;
          if (WITH_O) {
#pragma unroll
            for (int db = 0; db < (WITH_O ? DB : 1); ++db) oacc[db][qb] *= alpha;
          }
        }
        float p[TB * 4];
        float psum = 0.f;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            p[4 * tb + j] = hw_exp2(fmaf(sacc[tb][qb][j], c, negm[qb]));
            psum += p[4 * tb + j];
          }
        lsum[qb] += psum;
        if (WITH_O) {
#pragma unroll
          for (int h = 0; h < TB / 2; ++h) pf[h][qb] = pack8<TV>(&p[8 * h]);
        }
      }
      if (WITH_O) {
#pragma unroll
        for (int step = 0; step < PVS; ++step) {
          const int h = step / DB, db = step % DB;
          const FV vf = vq[step % VW];
          if (step + VW < PVS) vq[step % VW] = load_v(step + VW);
#pragma unroll
          for (int qb = 0; qb < QBW; ++qb)
            oacc[db % (WITH_O ? DB : 1)][qb] = mma(vf, pf[h][qb], oacc[db % (WITH_O ? DB : 1)][qb]);
        }
      }
    };
    if (t0 <= wave_last && (!REV || t0 + TN - 1 >= wave_lo_min)) {
      if (t0 + TN - 1 > wave_first || (REV && t0 < wave_lo_max)) tile(std::true_type{});
      else tile(std::false_type{});
    }
    stash(cur ^ 1);
    __syncthreads();
  }

  if (spare) return;
  const long head = ((long)b * h_kv + kvh) * geo.group + hv;
  if constexpr (REV && WITH_O) {
    if (splits == 1) {
      // counter-causal rows run unsplit: this workgroup saw every key of its
      // rows, so it writes the final row_max (natural units), row_sum and
      // normalised O rows itself (pm, pl, pO are then row_max [.][n],
      // row_sum [.][n] and O [.][n][D])
      const long ohead = (((long)b * h_kv + kvh) * (geo.group / geo.nq) + hv / geo.nq);
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        const float fix = (mtop[qb] == -INFINITY) ? 1.f : hw_exp2(mref[qb] - mtop[qb]);
        const float l = group4_sum(lsum[qb] * fix);
        const int pos = rev_block(geo, hv) * 64 + (qb0 + qb) * 16 + col;
        if (pos < n) {
          const long orow = ohead * n + pos;
          if (grp == 0) {
            pm[orow] = mtop[qb] * kLn2;
            pl[orow] = l;
          }
          const float sc = l > 0.f ? fix / l : 0.f;
#pragma unroll
          for (int db = 0; db < DB; ++db)
            *reinterpret_cast<float4 *>(pO + orow * D + db * 16 + 4 * grp) =
                make_float4(oacc[db][qb][0] * sc, oacc[db][qb][1] * sc, oacc[db][qb][2] * sc,
                            oacc[db][qb][3] * sc);
        }
      }
      return;
    }
  }
  const long pbase = (head * splits + s) * 64;
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    // bring (l, O) from the reference max to the exact max
    const float fix = (mtop[qb] == -INFINITY) ? 1.f : hw_exp2(mref[qb] - mtop[qb]);
    float l = lsum[qb] * fix;
    l = group4_sum(l);
    const int r = (qb0 + qb) * 16 + col;
    if (grp == 0) {
      pm[pbase + r] = mtop[qb];
      pl[pbase + r] = l;
    }
    if (WITH_O) {
      float *po = pO + (head * splits + s) * (long)D * 64;
#pragma unroll
      for (int db = 0; db < (WITH_O ? DB : 1); ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          po[(db * 16 + 4 * grp + j) * 64 + (qb0 + qb) * 16 + col] = oacc[db][qb][j] * fix;
    }
  }
}

// LORE: merge the splits of every scoring row into row_max (natural units of
// q.k/sqrt(d)), row_sum and the normalised O.  One block per (query head,
// 4-wide slice of d), thread (q = tid % 64, d = slice + tid / 64).  A thread
// first puts its column of partial O (one value per split) in flight, then
// the four waves share the split weights: each takes every fourth split for
// the row maximum and the weighted row sum, combined through LDS, so no
// thread waits on a serial chain of loads.
template <int D>
__global__ void __launch_bounds__(256)
attn_combine_lore_kernel(const float *__restrict__ pm, const float *__restrict__ pl,
                         const float *__restrict__ pO, int splits, int nq,
                         float *__restrict__ row_max, float *__restrict__ row_sum,
                         float *__restrict__ O) {
  constexpr int CH = 32;           // partial-O values held in registers per pass
  extern __shared__ float wsh[];   // [splits][64] split weights, [4][64] max, [4][64] sums
  float *pmax = wsh + splits * 64, *psum = pmax + 256;
  const long head = blockIdx.x;
  const int q = threadIdx.x & 63, part = threadIdx.x >> 6;
  const int d = blockIdx.y * 4 + part;
  const float *hm = pm + head * splits * 64;
  const float *hl = pl + head * splits * 64;
  const float *ho = pO + (head * splits * (long)D + d) * 64 + q;  // split stride D * 64
  // splits per thread held in registers in the weight phase (every fourth
  // split: up to 32 splits); further splits are read again in a loop.  Few
  // registers keep four waves per SIMD, so the grid runs in one round.
  constexpr int SPT = 8;
  float ov[CH], mv[SPT], lv[SPT];
#pragma unroll
  for (int u = 0; u < CH; ++u) ov[u] = u < splits ? ho[(long)u * D * 64] : 0.f;
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int s = part + 4 * u;
    mv[u] = s < splits ? hm[s * 64 + q] : -INFINITY;
    lv[u] = s < splits ? hl[s * 64 + q] : 0.f;
  }
  float mloc = -INFINITY;
#pragma unroll
  for (int u = 0; u < SPT; ++u) mloc = fmaxf(mloc, mv[u]);
  for (int s = part + 4 * SPT; s < splits; s += 4) mloc = fmaxf(mloc, hm[s * 64 + q]);
  pmax[part * 64 + q] = mloc;
  __syncthreads();
  const float M = fmaxf(fmaxf(pmax[q], pmax[64 + q]), fmaxf(pmax[128 + q], pmax[192 + q]));
  const float muse = (M == -INFINITY) ? 0.f : M;
  float lloc = 0.f;
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int s = part + 4 * u;
    if (s < splits) {
      const float wgt = exp2f(mv[u] - muse);
      wsh[s * 64 + q] = wgt;
      lloc += lv[u] * wgt;
    }
  }
  for (int s = part + 4 * SPT; s < splits; s += 4) {
    const float wgt = exp2f(hm[s * 64 + q] - muse);
    wsh[s * 64 + q] = wgt;
    lloc += hl[s * 64 + q] * wgt;
  }
  psum[part * 64 + q] = lloc;
  __syncthreads();
  const float L = (psum[q] + psum[64 + q]) + (psum[128 + q] + psum[192 + q]);
  if (part == 0 && q < nq && blockIdx.y == 0) {
    row_max[head * nq + q] = M * kLn2;
    row_sum[head * nq + q] = L;
  }
  float o = 0.f;
  for (int s0 = 0; s0 < splits; s0 += CH) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < CH; ++u) ov[u] = s0 + u < splits ? ho[(long)(s0 + u) * D * 64] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < CH; ++u)
      if (s0 + u < splits) o += ov[u] * wsh[(s0 + u) * 64 + q];
  }
  if (q < nq) O[(head * nq + q) * D + d] = o * (1.f / L);
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

// The dense probabilities a_{q,i} of the scoring rows (an optional output of
// kvscore_probs): P[b][h][r][i] = 2^(s c - beta2_r) for the tokens row r sees
// and exactly 0 for the others, beta2_r = row_max_r log2(e) + log2(row_sum_r)
// from the combined statistics.  One workgroup per (64-token tile, query head,
// sequence), one wave per 16-row block: the K tile is staged in LDS, S = Q K^T
// runs on the matrix cores with the tokens across the columns, and each store
// instruction writes 16 consecutive tokens of 4 rows.
template <typename Tin, int D>
__global__ void __launch_bounds__(256)
probs_write_kernel(const Tin *__restrict__ Q, const Tin *__restrict__ K,
                   const float *__restrict__ row_max, const float *__restrict__ row_sum,
                   RowGeom geo, int h_kv, float *__restrict__ P) {
  typedef typename FragOf<Tin>::type FQ;
  constexpr int KS = D / 32;
  constexpr int TN = 64;
  constexpr int EPC = 16 / (int)sizeof(Tin);
  constexpr int CPR = D / EPC;
  constexpr int KROW = D + (sizeof(Tin) == 2 ? 16 : EPC);  // conflict-free fragment reads
  constexpr int ITEMS = TN * CPR;
  __shared__ __align__(16) Tin Ks[TN * KROW];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int t0 = blockIdx.x * TN, h = blockIdx.y, b = blockIdx.z;
  const int n = geo.n, nq = geo.nq, G = geo.group;
  const long head = (long)b * h_kv * G + h;  // b * h_q + h
  const Tin *Kb = K + ((long)b * h_kv + h / G) * (long)n * D;
  constexpr uint32_t RB = D * sizeof(Tin);
  // rows past the end of the cache read as zeros (their tokens are not stored)
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kb + (long)t0 * D, range_bytes(t0, min(n, t0 + TN), RB));
#pragma unroll
  for (int u = 0; u < (ITEMS + 255) / 256; ++u) {
    const int idx = threadIdx.x + u * 256;
    if (ITEMS % 256 == 0 || idx < ITEMS) {
      const int row = idx / CPR, ch = idx % CPR;
      *reinterpret_cast<U128 *>(&Ks[row * KROW + ch * EPC]) =
          buf_load16(rk, (uint32_t)(row * D + ch * EPC) * sizeof(Tin));
    }
  }
  // A fragment: query row 16 wv + col; results: rows 16 wv + 4 grp + j
  const int rq = 16 * wv + col;
  FQ qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = rq < nq ? load8<Tin>(Q + (head * nq + rq) * D + ks * 32 + 8 * grp) : zero8<Tin>();
  float beta[4];
  int last[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * wv + 4 * grp + j;
    beta[j] = r < nq ? row_max[head * nq + r] * kLog2e + log2f(row_sum[head * nq + r]) : 0.f;
    last[j] = r < nq ? (r < geo.w ? n - geo.w + r : n - 1) : -1;
  }
  const float c = kLog2e * rsqrtf((float)D);
  __syncthreads();
#pragma unroll
  for (int tb = 0; tb < TN / 16; ++tb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = mma(qf[ks], load8<Tin>(&Ks[(tb * 16 + col) * KROW + ks * 32 + 8 * grp]), acc);
    const int tok = t0 + tb * 16 + col;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 16 * wv + 4 * grp + j;
      if (r < nq && tok < n)
        P[(head * nq + r) * (long)n + tok] =
            tok <= last[j] ? hw_exp2(fmaf(acc[j], c, -beta[j])) : 0.f;
    }
  }
}

hipError_t launch_probs_write(int etype, int d, const void *Q, const void *K,
                              const float *row_max, const float *row_sum, RowGeom geo, int batch,
                              int h_kv, float *P, hipStream_t st) {
  const dim3 grid((geo.n + 63) / 64, h_kv * geo.group, batch);
  {
    TimedLaunch tl_("probs_write", st);
#define KVS_PW(T, DD) \
  hipLaunchKernelGGL((probs_write_kernel<T, DD>), grid, dim3(256), 0, st, (const T *)Q, (const T *)K, \
                     row_max, row_sum, geo, h_kv, P)
    if (etype == E_F32) { if (d == 64) KVS_PW(float, 64); else KVS_PW(float, 128); }
    else if (etype == E_BF16) { if (d == 64) KVS_PW(bf16, 64); else KVS_PW(bf16, 128); }
    else { if (d == 64) KVS_PW(f16, 64); else KVS_PW(f16, 128); }
#undef KVS_PW
  }
  return hipGetLastError();
}

SplitPlan attn_split_plan(int units, int n) {
  const int target = 256;  // about one workgroup per CU; fewer splits mean less partial-O traffic
  int splits = (target + units - 1) / units;
  const int max_splits = (n + 511) / 512;
  if (splits > max_splits) splits = max_splits;
  if (splits > 128) splits = 128;
  if (splits < 1) splits = 1;
  if (splits < (n + kMaxRangeTokens - 1) / kMaxRangeTokens)
    splits = (n + kMaxRangeTokens - 1) / kMaxRangeTokens;
  int tps = (n + splits - 1) / splits;
  tps = (tps + 63) / 64 * 64;
  splits = (n + tps - 1) / tps;
  return SplitPlan{splits, tps};
}

// A workgroup holds at most 8 waves: a group needing more (G query heads x
// 4/QBW waves each) is served by hsplit workgroups of hpw heads.  With O the
// waves take 2 query blocks each (the O accumulators fill the registers),
// without O 4.
HeadSplit attn_head_split(int group, bool with_o) {
  HeadSplit h;
  h.qbw = with_o ? 2 : 4;
  const int wph = 4 / h.qbw;
  // without O (H2O prefill rows, causal) groups of at most 4 virtual heads:
  // the waves of a workgroup then differ less in how many tiles they need
  // (measured 4% faster than 8 on the OPT-30B prompt, 2 was slower)
  h.hsplit = with_o ? (group * wph + 7) / 8 : (group + 3) / 4;
  h.hpw = (group + h.hsplit - 1) / h.hsplit;
  h.maxw = 2;
  while (h.maxw < h.hpw * wph) h.maxw *= 2;
  return h;
}

template <typename Tin, int D, bool WITH_O, int MAXW, int QBW, bool REV = false>
static hipError_t run_partial(const void *Q, const void *K, const void *V, RowGeom geo, int batch,
                              int h_kv, HeadSplit hs, SplitPlan plan, float *pm, float *pl,
                              float *pO, hipStream_t st) {
  // The block is always MAXW waves; waves beyond the heads' share stage
  // tiles but compute nothing.
  dim3 grid(plan.splits, h_kv * hs.hsplit, batch), block(64 * MAXW);
  const int need = hs.hpw * (4 / QBW);
  if (need < 1 || need > MAXW || hs.hsplit * hs.hpw < geo.group) return hipErrorInvalidConfiguration;
  {
    TimedLaunch tl_("attn_partial", st);
    hipLaunchKernelGGL((attn_partial_kernel<Tin, D, WITH_O, MAXW, QBW, REV>), grid, block, 0, st,
                       (const Tin *)Q, (const Tin *)K, (const Tin *)V, geo, h_kv, hs.hsplit,
                       hs.hpw, plan.tps, plan.splits, pm, pl, pO);
  }
  return hipGetLastError();
}

template <typename Tin, int D>
static hipError_t run_partial_d(bool with_o, const void *Q, const void *K, const void *V,
                                RowGeom geo, int batch, int h_kv, SplitPlan plan, float *pm,
                                float *pl, float *pO, hipStream_t st) {
  const HeadSplit hs = attn_head_split(geo.group, with_o);
#define KVS_RP(O, MAXW, QBW) \
  return run_partial<Tin, D, O, MAXW, QBW>(Q, K, V, geo, batch, h_kv, hs, plan, pm, pl, pO, st)
  if (geo.mode == 2) {  // counter-causal rows: always with O
    if (!with_o) return hipErrorInvalidValue;
    if (hs.maxw == 2) return run_partial<Tin, D, true, 2, 2, true>(Q, K, V, geo, batch, h_kv, hs, plan, pm, pl, pO, st);
    if (hs.maxw == 4) return run_partial<Tin, D, true, 4, 2, true>(Q, K, V, geo, batch, h_kv, hs, plan, pm, pl, pO, st);
    return run_partial<Tin, D, true, 8, 2, true>(Q, K, V, geo, batch, h_kv, hs, plan, pm, pl, pO, st);
  }
  if (!with_o) {
    if (hs.maxw == 2) KVS_RP(false, 2, 4);
    if (hs.maxw == 4) KVS_RP(false, 4, 4);
    KVS_RP(false, 8, 4);
  }
  if (hs.maxw == 2) KVS_RP(true, 2, 2);
  if (hs.maxw == 4) KVS_RP(true, 4, 2);
  KVS_RP(true, 8, 2);
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
  const size_t shm = sizeof(float) * 64 * ((size_t)splits + 8);
  {
    TimedLaunch tl_("attn_combine", st);
    if (d == 64)
      hipLaunchKernelGGL(attn_combine_lore_kernel<64>, dim3(heads, 64 / 4), dim3(256), shm, st,
                         part_m, part_l, part_O, splits, nq, row_max, row_sum, O);
    else
      hipLaunchKernelGGL(attn_combine_lore_kernel<128>, dim3(heads, 128 / 4), dim3(256), shm, st,
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
