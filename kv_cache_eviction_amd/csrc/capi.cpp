// C ABI of the library: argument checks, workspace planning and dispatch.
// Every check runs on the host before anything is enqueued; see kvscore.h.
#include "kvscore.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <initializer_list>
#include <string>

#include "launch.hpp"
#include "timing.hpp"

#define KVS_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_err;

kvs_status fail(kvs_status st, const std::string &msg) {
  g_err = msg;
  return st;
}

// Element-type tensors (and O) are read and written with 16-byte vector
// accesses, so their base addresses must be 16-byte aligned.
kvs_status check_aligned(const char *who, std::initializer_list<const void *> ptrs) {
  for (const void *p : ptrs)
    if (p && (reinterpret_cast<uintptr_t>(p) & 15u))
      return fail(KVS_ERR_INVALID, std::string(who) + ": tensor pointers must be 16-byte aligned");
  return KVS_OK;
}

kvs_status ok() {
  g_err.clear();
  return KVS_OK;
}

kvs_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(KVS_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }

// Sequences x heads (and the query heads of a layer) index one grid
// dimension of the scoring, selection and compaction launches, which holds
// at most 65535 workgroups.
constexpr long kMaxRows = 65535;
kvs_status check_rows(long rows, const char *what) {
  if (rows > kMaxRows) return fail(KVS_ERR_UNSUPPORTED, std::string(what) + " above 65535");
  return KVS_OK;
}

int n_pad_of(int n) { return (n + 63) / 64 * 64; }

// Plans of the LORE workspace; every entry point lays out its scratch from
// offset 0 of the same buffer.
struct LorePlan {
  kvs::SplitPlan split;
  int gsplits;
  size_t probs_bytes, deletion_bytes, topb_bytes, reliability_bytes;
  // deletion layout
  size_t off_gpart, off_gv, off_gr, off_yhi, off_ylo, off_consts, off_n;
  // probs layout
  size_t off_pm, off_pl, off_po;
};

kvs_status check_lore(const kvs_lore_desc *d) {
  if (!d) return fail(KVS_ERR_INVALID, "descriptor is NULL");
  if (d->batch < 1 || d->n < 1 || d->h_q < 1 || d->h_kv < 1 || d->d_model < 1)
    return fail(KVS_ERR_INVALID, "batch, n, h_q, h_kv and d_model must be >= 1");
  if (check_rows((long)d->batch * d->h_kv, "batch * h_kv") != KVS_OK) return KVS_ERR_UNSUPPORTED;
  if (check_rows(d->h_q, "h_q") != KVS_OK) return KVS_ERR_UNSUPPORTED;
  if (d->h_q % d->h_kv != 0) return fail(KVS_ERR_INVALID, "h_q must be a multiple of h_kv");
  if (d->h_q / d->h_kv > 16) return fail(KVS_ERR_UNSUPPORTED, "query-head group larger than 16");
  if (d->d != 64 && d->d != 128) return fail(KVS_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (d->w < 0 || d->m < 0 || d->t < 0) return fail(KVS_ERR_INVALID, "w, m and t must be >= 0");
  if (d->m > 0 && d->t < 1) return fail(KVS_ERR_INVALID, "t must be >= 1 when m > 0");
  const long nq = (long)d->w + (long)d->m * d->t;
  if (nq < 1 || nq > 64) return fail(KVS_ERR_UNSUPPORTED, "w + m*t must be in [1, 64]");
  if (d->n_sink < 0 || d->budget < 0) return fail(KVS_ERR_INVALID, "n_sink and budget must be >= 0");
  if ((long)d->n_sink + d->w > d->n) return fail(KVS_ERR_INVALID, "n must be >= n_sink + w");
  if (d->chunk < 1) return fail(KVS_ERR_INVALID, "chunk must be >= 1");
  if (d->n > (1 << 28)) return fail(KVS_ERR_UNSUPPORTED, "n above 2^28 tokens");
  if (!(std::isfinite(d->eps) && d->eps >= 0.f)) return fail(KVS_ERR_INVALID, "eps must be finite and >= 0");
  if (!(std::isfinite(d->lambda_l) && d->lambda_l >= 0.f))
    return fail(KVS_ERR_INVALID, "lambda_l must be finite and >= 0");
  if (d->dtype != KVS_F32 && d->dtype != KVS_BF16 && d->dtype != KVS_F16)
    return fail(KVS_ERR_INVALID, "unknown dtype");
  return ok();
}

size_t topb_bytes_of(const kvs_lore_desc *d);

LorePlan plan_lore(const kvs_lore_desc *d) {
  LorePlan p{};
  const size_t heads = (size_t)d->batch * d->h_q;
  const size_t D = d->d;
  const size_t vbytes = d->dtype == KVS_F32 ? 4 : 2;  // value-side element type
  p.split = kvs::attn_split_plan(
      d->batch * d->h_kv * kvs::attn_head_split(d->h_q / d->h_kv, true).hsplit, d->n);
  const size_t S = p.split.splits;
  p.off_pm = 0;
  p.off_pl = align_up(p.off_pm + heads * S * 64 * 4);
  p.off_po = align_up(p.off_pl + heads * S * 64 * 4);
  p.probs_bytes = align_up(p.off_po + heads * S * D * 64 * 4);

  p.gsplits = kvs::gram_splits(d->h_q, d->d_model, d->dtype == KVS_F32 ? 4 : 2);
  p.off_gpart = 0;
  p.off_gv = align_up(p.off_gpart + (size_t)p.gsplits * d->h_q * D * D * 4);
  p.off_gr = align_up(p.off_gv + (size_t)d->h_q * D * D * vbytes);
  p.off_yhi = align_up(p.off_gr + (size_t)d->h_q * D * D * 4);
  p.off_ylo = align_up(p.off_yhi + heads * 64 * D * vbytes);
  p.off_consts = align_up(p.off_ylo + heads * 64 * D * vbytes);
  p.off_n = align_up(p.off_consts + heads * 64 * 16);
  p.deletion_bytes = align_up(p.off_n + heads * (size_t)n_pad_of(d->n) * 4);

  p.topb_bytes = topb_bytes_of(d);
  p.reliability_bytes = align_up(kvs::reliability_ws_bytes(d->batch, d->h_q, d->m));
  return p;
}

// Selection reads only the shape and selection fields of the descriptor.
kvs_status check_select(const kvs_lore_desc *d) {
  if (!d) return fail(KVS_ERR_INVALID, "descriptor is NULL");
  if (d->batch < 1 || d->h_kv < 1 || d->n < 1)
    return fail(KVS_ERR_INVALID, "batch, h_kv and n must be >= 1");
  if (check_rows((long)d->batch * d->h_kv, "batch * h_kv") != KVS_OK) return KVS_ERR_UNSUPPORTED;
  if (d->n_sink < 0 || d->w < 0 || d->budget < 0)
    return fail(KVS_ERR_INVALID, "n_sink, w and budget must be >= 0");
  if ((long)d->n_sink + d->w > d->n) return fail(KVS_ERR_INVALID, "n must be >= n_sink + w");
  if (d->chunk < 1) return fail(KVS_ERR_INVALID, "chunk must be >= 1");
  if (d->n > (1 << 28)) return fail(KVS_ERR_UNSUPPORTED, "n above 2^28 tokens");
  return ok();
}

size_t topb_bytes_of(const kvs_lore_desc *d) {
  return align_up(kvs::topb_workspace_bytes(d->batch * d->h_kv, d->n, d->chunk));
}

kvs_status check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need) {
    char buf[160];
    snprintf(buf, sizeof buf, "workspace of %zu bytes is smaller than the %zu bytes needed",
             ws_bytes, need);
    return fail(KVS_ERR_WORKSPACE, buf);
  }
  if (need > 0 && !ws) return fail(KVS_ERR_WORKSPACE, "workspace pointer is NULL");
  return ok();
}

kvs::RowGeom lore_geom(const kvs_lore_desc *d) {
  return kvs::RowGeom{0, d->n, d->w + d->m * d->t, d->w, d->h_q / d->h_kv};
}

template <typename T> T *at(void *base, size_t off) {
  return reinterpret_cast<T *>(static_cast<char *>(base) + off);
}

}  // namespace

KVS_API const char *kvs_last_error(void) { return g_err.c_str(); }

KVS_API size_t kvs_lore_workspace_bytes(const kvs_lore_desc *desc) {
  if (check_lore(desc) != KVS_OK) return 0;
  const LorePlan p = plan_lore(desc);
  size_t m = p.probs_bytes;
  if (p.deletion_bytes > m) m = p.deletion_bytes;
  if (p.topb_bytes > m) m = p.topb_bytes;
  if (p.reliability_bytes > m) m = p.reliability_bytes;
  return m;
}

KVS_API kvs_status kvscore_probs(const kvs_lore_desc *desc, int32_t mask, const void *Q,
                                 const void *K, const void *V, float *row_max, float *row_sum,
                                 float *O, float *P, void *ws, size_t ws_bytes, void *stream) {
  kvs_status st = check_lore(desc);
  if (st != KVS_OK) return st;
  if (mask == KVS_MASK_CAUSAL || mask == KVS_MASK_SLOTS)
    return fail(KVS_ERR_UNSUPPORTED, "kvscore_probs: the causal and slot masks are the H2O modes "
                                     "of kvscore_h2o_accumulate");
  if (mask != KVS_MASK_NONE && mask != KVS_MASK_WINDOW_CAUSAL)
    return fail(KVS_ERR_INVALID, "kvscore_probs: unknown mask");
  if (!Q || !K || !V || !row_max || !row_sum || !O)
    return fail(KVS_ERR_INVALID, "kvscore_probs: a required pointer is NULL");
  st = check_aligned("kvscore_probs", {Q, K, V, O});
  if (st != KVS_OK) return st;
  const LorePlan p = plan_lore(desc);
  st = check_ws(ws, ws_bytes, p.probs_bytes);
  if (st != KVS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  kvs::RowGeom geo = lore_geom(desc);
  if (mask == KVS_MASK_NONE) geo.w = 0;  // no row is causal: every row sees all n tokens
  float *pm = at<float>(ws, p.off_pm), *pl = at<float>(ws, p.off_pl), *po = at<float>(ws, p.off_po);
  hipError_t e = kvs::launch_attn_partial(desc->dtype, desc->d, true, Q, K, V, geo, desc->batch,
                                          desc->h_kv, p.split, pm, pl, po, s);
  if (e != hipSuccess) return hip_status(e, "attention pass");
  e = kvs::launch_attn_combine_lore(desc->d, pm, pl, po, desc->batch * desc->h_q, p.split.splits,
                                    geo.nq, row_max, row_sum, O, s);
  if (e != hipSuccess || !P) return hip_status(e, "attention combine");
  e = kvs::launch_probs_write(desc->dtype, desc->d, Q, K, row_max, row_sum, geo, desc->batch,
                              desc->h_kv, P, s);
  return hip_status(e, "probabilities");
}

KVS_API kvs_status kvscore_deletion(const kvs_lore_desc *desc, const void *Q, const void *K,
                                    const void *V, const void *W_O, const float *omega,
                                    const float *row_max, const float *row_sum, const float *O,
                                    float *S, void *ws, size_t ws_bytes, void *stream) {
  kvs_status st = check_lore(desc);
  if (st != KVS_OK) return st;
  if (!Q || !K || !V || !W_O || !row_max || !row_sum || !O || !S)
    return fail(KVS_ERR_INVALID, "kvscore_deletion: a required pointer is NULL");
  if (desc->m > 0 && !omega) return fail(KVS_ERR_INVALID, "kvscore_deletion: omega is NULL");
  st = check_aligned("kvscore_deletion", {Q, K, V, W_O, O});
  if (st != KVS_OK) return st;
  const LorePlan p = plan_lore(desc);
  st = check_ws(ws, ws_bytes, p.deletion_bytes);
  if (st != KVS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const kvs::RowGeom geo = lore_geom(desc);
  float *gpart = at<float>(ws, p.off_gpart);
  void *gv = at<void>(ws, p.off_gv);
  float *gr = at<float>(ws, p.off_gr);
  void *yhi = at<void>(ws, p.off_yhi), *ylo = at<void>(ws, p.off_ylo);
  float4 *consts = at<float4>(ws, p.off_consts);
  float *nn = at<float>(ws, p.off_n);
  const int npad = n_pad_of(desc->n);
  hipError_t e = kvs::launch_gram(desc->dtype, desc->d, W_O, desc->d_model, desc->h_q, p.gsplits,
                                  gpart, s);
  if (e != hipSuccess) return hip_status(e, "gram");
  e = kvs::launch_deletion_prep(desc->dtype, desc->d, gpart, p.gsplits, O, row_max, row_sum, omega,
                                desc->batch, desc->h_q, desc->n, geo.nq, desc->w, desc->m, desc->t,
                                desc->lambda_l, gv, gr, yhi, ylo, consts, s);
  if (e != hipSuccess) return hip_status(e, "deletion prep");
  e = kvs::launch_vnorm(desc->dtype, desc->d, V, gv, desc->batch, desc->n, npad, desc->h_q,
                        desc->h_kv, nn, s);
  if (e != hipSuccess) return hip_status(e, "value norms");
  e = kvs::launch_score(desc->dtype, desc->d, 0, Q, K, V, yhi, ylo, consts, nn, npad, geo,
                        desc->batch, desc->h_kv, desc->eps, 1.f / (float)geo.group, S, s);
  return hip_status(e, "deletion score");
}

KVS_API kvs_status kvscore_baseline_scores(const kvs_lore_desc *desc, int kind, const void *Q,
                                           const void *K, const float *row_max,
                                           const float *row_sum, float *S, void *ws,
                                           size_t ws_bytes, void *stream) {
  kvs_status st = check_lore(desc);
  if (st != KVS_OK) return st;
  if (kind != KVS_BASELINE_WINDOW && kind != KVS_BASELINE_TOVA)
    return fail(KVS_ERR_INVALID, "kvscore_baseline_scores: unknown kind");
  if (desc->w < 1) return fail(KVS_ERR_INVALID, "kvscore_baseline_scores: needs w >= 1 window rows");
  if (!Q || !K || !row_max || !row_sum || !S)
    return fail(KVS_ERR_INVALID, "kvscore_baseline_scores: a required pointer is NULL");
  st = check_aligned("kvscore_baseline_scores", {Q, K});
  if (st != KVS_OK) return st;
  const LorePlan p = plan_lore(desc);
  st = check_ws(ws, ws_bytes, p.deletion_bytes);
  if (st != KVS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const kvs::RowGeom geo = lore_geom(desc);
  float4 *consts = at<float4>(ws, p.off_consts);
  hipError_t e = kvs::launch_baseline_prep(row_max, row_sum, desc->batch, desc->h_q, desc->n,
                                           geo.nq, desc->w, kind == KVS_BASELINE_TOVA, consts, s);
  if (e != hipSuccess) return hip_status(e, "baseline prep");
  e = kvs::launch_score(desc->dtype, desc->d, 1, Q, K, nullptr, nullptr, nullptr, consts, nullptr,
                        n_pad_of(desc->n), geo, desc->batch, desc->h_kv, desc->eps,
                        1.f / (float)geo.group, S, s);
  return hip_status(e, "baseline score");
}

KVS_API kvs_status kvscore_reliability_weights(const kvs_lore_desc *desc, const void *Q,
                                               const float *logp, const float *entropy,
                                               float beta, float gamma, float lambda_d,
                                               float *omega, float *dhat, void *ws,
                                               size_t ws_bytes, void *stream) {
  kvs_status st = check_lore(desc);
  if (st != KVS_OK) return st;
  if (desc->m < 1) return ok();  // no trajectories: nothing to weight
  if (desc->m > 64) return fail(KVS_ERR_UNSUPPORTED, "kvscore_reliability_weights: m above 64");
  if (!Q || !logp || !entropy || !omega)
    return fail(KVS_ERR_INVALID, "kvscore_reliability_weights: a required pointer is NULL");
  st = check_aligned("kvscore_reliability_weights", {Q});
  if (st != KVS_OK) return st;
  if (!(std::isfinite(beta) && std::isfinite(gamma) && std::isfinite(lambda_d)))
    return fail(KVS_ERR_INVALID, "kvscore_reliability_weights: beta, gamma, lambda_d must be finite");
  const LorePlan p = plan_lore(desc);
  if (desc->m > 1) {
    st = check_ws(ws, ws_bytes, p.reliability_bytes);
    if (st != KVS_OK) return st;
  }
  const int nq = desc->w + desc->m * desc->t;
  hipError_t e = kvs::launch_reliability(desc->dtype, Q, desc->batch, desc->h_q, nq, desc->d,
                                         desc->w, desc->m, desc->t, logp, entropy, beta, gamma,
                                         lambda_d, omega, dhat, at<double>(ws, 0),
                                         static_cast<hipStream_t>(stream));
  return hip_status(e, "reliability weights");
}

// ---------------------------------------------------------------------------
// Output fidelity: the attention pass on the full and on the kept cache, then
// per-row cosines.

kvs_status check_fidelity(const kvs_lore_desc *d, int n_f, int n_keep) {
  if (!d) return fail(KVS_ERR_INVALID, "descriptor is NULL");
  if (d->batch < 1 || d->n < 1 || d->h_q < 1 || d->h_kv < 1)
    return fail(KVS_ERR_INVALID, "batch, n, h_q and h_kv must be >= 1");
  if (check_rows((long)d->batch * d->h_kv, "batch * h_kv") != KVS_OK) return KVS_ERR_UNSUPPORTED;
  if (check_rows(d->h_q, "h_q") != KVS_OK) return KVS_ERR_UNSUPPORTED;
  if (d->h_q % d->h_kv != 0) return fail(KVS_ERR_INVALID, "h_q must be a multiple of h_kv");
  if (d->h_q / d->h_kv > 16) return fail(KVS_ERR_UNSUPPORTED, "query-head group larger than 16");
  if (d->d != 64 && d->d != 128) return fail(KVS_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (d->n > (1 << 28)) return fail(KVS_ERR_UNSUPPORTED, "n above 2^28 tokens");
  if (d->dtype != KVS_F32 && d->dtype != KVS_BF16 && d->dtype != KVS_F16)
    return fail(KVS_ERR_INVALID, "unknown dtype");
  if (n_f < 1 || n_f > 64) return fail(KVS_ERR_UNSUPPORTED, "n_f must be in [1, 64]");
  if (n_keep < 1 || n_keep > d->n) return fail(KVS_ERR_INVALID, "n_keep must be in [1, n]");
  return ok();
}

struct FidelityPlan {
  kvs::SplitPlan full, kept;
  size_t off_pm, off_pl, off_po, off_m, off_l, off_of, off_ok, bytes;
};

FidelityPlan plan_fidelity(const kvs_lore_desc *d, int n_f, int n_keep) {
  FidelityPlan p{};
  const size_t heads = (size_t)d->batch * d->h_q, D = d->d;
  const int units = d->batch * d->h_kv * kvs::attn_head_split(d->h_q / d->h_kv, true).hsplit;
  p.full = kvs::attn_split_plan(units, d->n);
  p.kept = kvs::attn_split_plan(units, n_keep);
  const size_t S = p.full.splits > p.kept.splits ? p.full.splits : p.kept.splits;
  p.off_pm = 0;
  p.off_pl = align_up(p.off_pm + heads * S * 64 * 4);
  p.off_po = align_up(p.off_pl + heads * S * 64 * 4);
  p.off_m = align_up(p.off_po + heads * S * D * 64 * 4);
  p.off_l = align_up(p.off_m + heads * n_f * 4);
  p.off_of = align_up(p.off_l + heads * n_f * 4);
  p.off_ok = align_up(p.off_of + heads * n_f * D * 4);
  p.bytes = align_up(p.off_ok + heads * n_f * D * 4);
  return p;
}

KVS_API size_t kvs_fidelity_workspace_bytes(const kvs_lore_desc *desc, int32_t n_f,
                                            int32_t n_keep) {
  if (check_fidelity(desc, n_f, n_keep) != KVS_OK) return 0;
  return plan_fidelity(desc, n_f, n_keep).bytes;
}

KVS_API kvs_status kvscore_output_fidelity(const kvs_lore_desc *desc, int32_t n_f, int32_t n_keep,
                                           const void *Qf, const void *K, const void *V,
                                           const void *K_keep, const void *V_keep,
                                           float *cos_out, float *fidelity, void *ws,
                                           size_t ws_bytes, void *stream) {
  kvs_status st = check_fidelity(desc, n_f, n_keep);
  if (st != KVS_OK) return st;
  if (!Qf || !K || !V || !K_keep || !V_keep || !cos_out || !fidelity)
    return fail(KVS_ERR_INVALID, "kvscore_output_fidelity: a required pointer is NULL");
  st = check_aligned("kvscore_output_fidelity", {Qf, K, V, K_keep, V_keep});
  if (st != KVS_OK) return st;
  const FidelityPlan p = plan_fidelity(desc, n_f, n_keep);
  st = check_ws(ws, ws_bytes, p.bytes);
  if (st != KVS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int group = desc->h_q / desc->h_kv, heads = desc->batch * desc->h_q;
  float *pm = at<float>(ws, p.off_pm), *pl = at<float>(ws, p.off_pl), *po = at<float>(ws, p.off_po);
  float *rm = at<float>(ws, p.off_m), *rl = at<float>(ws, p.off_l);
  float *Of = at<float>(ws, p.off_of), *Ok = at<float>(ws, p.off_ok);
  // every held-out row sees every token of its cache (no window rows)
  const kvs::RowGeom gf{0, desc->n, n_f, 0, group}, gk{0, n_keep, n_f, 0, group};
  hipError_t e = kvs::launch_attn_partial(desc->dtype, desc->d, true, Qf, K, V, gf, desc->batch,
                                          desc->h_kv, p.full, pm, pl, po, s);
  if (e != hipSuccess) return hip_status(e, "full-cache attention");
  e = kvs::launch_attn_combine_lore(desc->d, pm, pl, po, heads, p.full.splits, n_f, rm, rl, Of, s);
  if (e != hipSuccess) return hip_status(e, "full-cache combine");
  e = kvs::launch_attn_partial(desc->dtype, desc->d, true, Qf, K_keep, V_keep, gk, desc->batch,
                               desc->h_kv, p.kept, pm, pl, po, s);
  if (e != hipSuccess) return hip_status(e, "kept-cache attention");
  e = kvs::launch_attn_combine_lore(desc->d, pm, pl, po, heads, p.kept.splits, n_f, rm, rl, Ok, s);
  if (e != hipSuccess) return hip_status(e, "kept-cache combine");
  e = kvs::launch_output_cosine(desc->d, Of, Ok, desc->batch, desc->h_q * n_f, cos_out, fidelity,
                                s);
  return hip_status(e, "output cosine");
}

// ---------------------------------------------------------------------------
// Counter-causal attention: every cached position's fresh query over the keys
// after it (RowGeom mode 2, virtual heads of 64 positions).

kvs_status check_counter_causal(const kvs_lore_desc *d) {
  if (!d) return fail(KVS_ERR_INVALID, "descriptor is NULL");
  if (d->batch < 1 || d->n < 1 || d->h_q < 1 || d->h_kv < 1)
    return fail(KVS_ERR_INVALID, "batch, n, h_q and h_kv must be >= 1");
  if (check_rows((long)d->batch * d->h_kv, "batch * h_kv") != KVS_OK) return KVS_ERR_UNSUPPORTED;
  if (check_rows(d->h_q, "h_q") != KVS_OK) return KVS_ERR_UNSUPPORTED;
  if (d->h_q % d->h_kv != 0) return fail(KVS_ERR_INVALID, "h_q must be a multiple of h_kv");
  if (d->d != 64 && d->d != 128) return fail(KVS_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (d->n > (1 << 22)) return fail(KVS_ERR_UNSUPPORTED, "n above 2^22 tokens");
  if (d->dtype != KVS_F32 && d->dtype != KVS_BF16 && d->dtype != KVS_F16)
    return fail(KVS_ERR_INVALID, "unknown dtype");
  // workgroups per KV head (grid y) grow with the query heads' 64-row blocks
  const long group = (long)(d->h_q / d->h_kv) * ((d->n + 63) / 64);
  if ((long)d->h_kv * ((group * 2 + 7) / 8) > 65535)
    return fail(KVS_ERR_UNSUPPORTED, "counter-causal: h_q * ceil(n/64) too large for one launch");
  return ok();
}

KVS_API kvs_status kvscore_counter_causal(const kvs_lore_desc *desc, const void *Q, const void *K,
                                          const void *V, float *row_max, float *row_sum,
                                          float *O, void *stream) {
  kvs_status st = check_counter_causal(desc);
  if (st != KVS_OK) return st;
  if (!Q || !K || !V || !row_max || !row_sum || !O)
    return fail(KVS_ERR_INVALID, "kvscore_counter_causal: a required pointer is NULL");
  st = check_aligned("kvscore_counter_causal", {Q, K, V, O});
  if (st != KVS_OK) return st;
  // one split over all n keys (a workgroup starts at its rows' earliest key),
  // so the attention pass writes the final rows and no workspace is needed
  const int G = desc->h_q / desc->h_kv, nblk = (desc->n + 63) / 64;
  const kvs::RowGeom geo{2, desc->n, nblk, 0, G * nblk};
  const int tps = (desc->n + 63) / 64 * 64;
  hipError_t e = kvs::launch_attn_partial(desc->dtype, desc->d, true, Q, K, V, geo, desc->batch,
                                          desc->h_kv, kvs::SplitPlan{1, tps}, row_max, row_sum,
                                          O, static_cast<hipStream_t>(stream));
  return hip_status(e, "counter-causal attention");
}

// ---------------------------------------------------------------------------
// Memory refresh: keep the J most surprising of the n cached tokens (system
// prompt and last token protected), then gather K, V and the token ids with
// one token-level kept list per sequence.

KVS_API size_t kvs_refresh_workspace_bytes(int32_t batch, int32_t n) {
  if (batch < 1 || n < 1) {
    fail(KVS_ERR_INVALID, "kvs_refresh_workspace_bytes: batch and n must be >= 1");
    return 0;
  }
  return align_up(kvs::topb_workspace_bytes(batch, n, 1));
}

KVS_API kvs_status kvscore_refresh(int32_t batch, int32_t heads, int32_t n, int32_t d,
                                   int32_t dtype, int32_t n_sys, int32_t J,
                                   const float *surprise, const void *K, const void *V,
                                   const int32_t *ids, int32_t *kept, void *K_out, void *V_out,
                                   int32_t *ids_out, void *ws, size_t ws_bytes, void *stream) {
  if (batch < 1 || heads < 1 || n < 1)
    return fail(KVS_ERR_INVALID, "kvscore_refresh: batch, heads and n must be >= 1");
  if (check_rows((long)batch * heads, "kvscore_refresh: batch * heads") != KVS_OK)
    return KVS_ERR_UNSUPPORTED;
  if (n > (1 << 28)) return fail(KVS_ERR_UNSUPPORTED, "kvscore_refresh: n above 2^28 tokens");
  if (d != 64 && d != 128) return fail(KVS_ERR_UNSUPPORTED, "kvscore_refresh: head dim must be 64 or 128");
  if (dtype != KVS_F32 && dtype != KVS_BF16 && dtype != KVS_F16)
    return fail(KVS_ERR_INVALID, "kvscore_refresh: unknown dtype");
  if (n_sys < 0 || J < 0) return fail(KVS_ERR_INVALID, "kvscore_refresh: n_sys and J must be >= 0");
  if (J == 0) return ok();  // nothing survives the refresh
  const int keep = J < n ? J : n;
  const int n_sink = n_sys < n - 1 ? n_sys : n - 1;
  if (keep < n_sink + 1)
    return fail(KVS_ERR_INVALID, "kvscore_refresh: J leaves no room beside the system prompt for the last token");
  if (!surprise || !K || !V || !kept || !K_out || !V_out)
    return fail(KVS_ERR_INVALID, "kvscore_refresh: a required pointer is NULL");
  if ((ids == nullptr) != (ids_out == nullptr))
    return fail(KVS_ERR_INVALID, "kvscore_refresh: ids and ids_out go together");
  kvs_status st = check_aligned("kvscore_refresh", {K, V, K_out, V_out});
  if (st != KVS_OK) return st;
  st = check_ws(ws, ws_bytes, align_up(kvs::topb_workspace_bytes(batch, n, 1)));
  if (st != KVS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = kvs::launch_topb(surprise, batch, n, n_sink, 1, 1, keep - n_sink - 1, keep, ws,
                                  kept, nullptr, s);
  if (e != hipSuccess) return hip_status(e, "refresh selection");
  const int row_bytes = d * (int)kvs::elem_bytes(dtype);
  e = kvs::launch_compact(batch * heads, n, keep, keep, row_bytes, K, V, kept, K_out, V_out,
                          nullptr, ids, ids_out, s, heads);
  return hip_status(e, "refresh gather");
}

KVS_API size_t kvs_topb_workspace_bytes(const kvs_lore_desc *desc) {
  if (check_select(desc) != KVS_OK) return 0;
  return topb_bytes_of(desc);
}

KVS_API kvs_status kvscore_topb_select(const kvs_lore_desc *desc, const float *S, int32_t *kept,
                                       float *pooled, void *ws, size_t ws_bytes, void *stream) {
  kvs_status st = check_select(desc);
  if (st != KVS_OK) return st;
  if (!S || !kept) return fail(KVS_ERR_INVALID, "kvscore_topb_select: S or kept is NULL");
  st = check_ws(ws, ws_bytes, topb_bytes_of(desc));
  if (st != KVS_OK) return st;
  const int n_cand = desc->n - desc->n_sink - desc->w;
  const int B = desc->budget < n_cand ? desc->budget : n_cand;
  const int n_keep = desc->n_sink + B + desc->w;
  hipError_t e = kvs::launch_topb(S, desc->batch * desc->h_kv, desc->n, desc->n_sink, desc->w,
                                  desc->chunk, desc->budget, n_keep, ws, kept,
                                  pooled, static_cast<hipStream_t>(stream));
  return hip_status(e, "top-B select");
}

KVS_API kvs_status kvscore_retention_shift(int32_t rows, int32_t n_keep, int32_t n,
                                          int32_t n_sink, int32_t w, const int32_t *kept_a,
                                          const int32_t *kept_b, float *shift, void *stream) {
  if (rows < 1 || n_keep < 1 || n < 1)
    return fail(KVS_ERR_INVALID, "kvscore_retention_shift: rows, n_keep and n must be >= 1");
  if (n_sink < 0 || w < 0 || (long)n_sink + w > n || n_keep > n)
    return fail(KVS_ERR_INVALID, "kvscore_retention_shift: need n_sink, w >= 0, n_sink + w <= n, n_keep <= n");
  if (!kept_a || !kept_b || !shift)
    return fail(KVS_ERR_INVALID, "kvscore_retention_shift: a required pointer is NULL");
  const hipError_t e = kvs::launch_retention_shift(rows, n_keep, n_sink, w, n, kept_a, kept_b,
                                                   shift, static_cast<hipStream_t>(stream));
  return hip_status(e, "retention shift");
}

static_assert(kvs::kTopbScratchBytes == KVS_TOPB_NOALLOC_MAX_BYTES,
              "the header states the library's scratch size");

KVS_API kvs_status kvscore_topb_select_noalloc(const kvs_lore_desc *desc, const float *S,
                                               int32_t *kept, float *pooled, void *stream) {
  kvs_status st = check_select(desc);
  if (st != KVS_OK) return st;
  if (!S || !kept) return fail(KVS_ERR_INVALID, "kvscore_topb_select_noalloc: S or kept is NULL");
  const size_t need = topb_bytes_of(desc);
  if (need > kvs::kTopbScratchBytes) {
    char buf[200];
    snprintf(buf, sizeof buf,
             "kvscore_topb_select_noalloc: needs %zu bytes of scratch, above the library's "
             "%zu-byte maximum (use kvscore_topb_select with a workspace)",
             need, kvs::kTopbScratchBytes);
    return fail(KVS_ERR_UNSUPPORTED, buf);
  }
  void *scratch = nullptr;
  hipError_t e = kvs::topb_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "kvscore_topb_select_noalloc: scratch address");
  const int n_cand = desc->n - desc->n_sink - desc->w;
  const int B = desc->budget < n_cand ? desc->budget : n_cand;
  const int n_keep = desc->n_sink + B + desc->w;
  e = kvs::launch_topb(S, desc->batch * desc->h_kv, desc->n, desc->n_sink, desc->w, desc->chunk,
                       desc->budget, n_keep, scratch, kept, pooled,
                       static_cast<hipStream_t>(stream));
  return hip_status(e, "top-B select (library scratch)");
}

KVS_API kvs_status kv_compact(int32_t batch, int32_t heads, int32_t n_src, int32_t n_keep,
                              int32_t cap_dst, int32_t d, int32_t dtype, const void *K,
                              const void *V, const int32_t *kept, void *K_out, void *V_out,
                              int32_t *pos_out, const float *score_in, float *score_out,
                              void *stream) {
  if (batch < 1 || heads < 1 || n_src < 1 || n_keep < 0 || cap_dst < 1)
    return fail(KVS_ERR_INVALID, "kv_compact: batch, heads, n_src, cap_dst must be >= 1, n_keep >= 0");
  if (n_keep > n_src || n_keep > cap_dst)
    return fail(KVS_ERR_INVALID, "kv_compact: n_keep exceeds n_src or cap_dst");
  if (check_rows((long)batch * heads, "kv_compact: batch * heads") != KVS_OK)
    return KVS_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return fail(KVS_ERR_UNSUPPORTED, "kv_compact: head dim must be 64 or 128");
  if (dtype != KVS_F32 && dtype != KVS_BF16 && dtype != KVS_F16)
    return fail(KVS_ERR_INVALID, "kv_compact: unknown dtype");
  if (!K || !V || !K_out || !V_out || (n_keep > 0 && !kept))
    return fail(KVS_ERR_INVALID, "kv_compact: a required pointer is NULL");
  if ((score_in == nullptr) != (score_out == nullptr))
    return fail(KVS_ERR_INVALID, "kv_compact: score_in and score_out go together");
  if (check_aligned("kv_compact", {K, V, K_out, V_out}) != KVS_OK) return KVS_ERR_INVALID;
  const int row_bytes = d * (int)kvs::elem_bytes(dtype);
  hipError_t e = kvs::launch_compact(batch * heads, n_src, n_keep, cap_dst, row_bytes, K, V, kept,
                                     K_out, V_out, pos_out, score_in, score_out,
                                     static_cast<hipStream_t>(stream));
  return hip_status(e, "compaction");
}

namespace {

// Longest prompt the prefill takes: an fp32 prompt's column-sum pass runs one
// launch per eight 64-row blocks (32 launches at 16384 tokens); 16-bit
// prompts run two launches at any length.
constexpr int kMaxPrefill = 16384;

kvs_status check_h2o(const kvs_h2o_desc *d, int mode) {
  if (!d) return fail(KVS_ERR_INVALID, "descriptor is NULL");
  if (d->batch < 1 || d->heads < 1 || d->cap < 1)
    return fail(KVS_ERR_INVALID, "batch, heads and cap must be >= 1");
  if (check_rows((long)d->batch * d->heads, "batch * heads") != KVS_OK) return KVS_ERR_UNSUPPORTED;
  if (d->d != 64 && d->d != 128) return fail(KVS_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (d->dtype != KVS_F32 && d->dtype != KVS_BF16 && d->dtype != KVS_F16)
    return fail(KVS_ERR_INVALID, "unknown dtype");
  if (mode == KVS_H2O_PREFILL) {
    if (d->cap > kMaxPrefill)
      return fail(KVS_ERR_UNSUPPORTED, "prefill prompt longer than 16384");
    // the attention pass launches heads * ceil(cap/64 / 4) workgroups along grid y
    if ((long)d->heads * (((d->cap + 63) / 64 + 3) / 4) > 65535)
      return fail(KVS_ERR_UNSUPPORTED, "prefill: heads * ceil(cap / 256) above 65535");
  } else if (mode == KVS_H2O_DECODE) {
    if (d->cap > 2048) return fail(KVS_ERR_UNSUPPORTED, "decode slot count above 2048");
    if (d->cur_len < 1 || d->k_heavy < 0 || d->k_recent < 0)
      return fail(KVS_ERR_INVALID, "cur_len >= 1, k_heavy >= 0, k_recent >= 0 required");
  } else {
    return fail(KVS_ERR_INVALID, "unknown H2O mode");
  }
  return ok();
}

struct H2OPlan {
  int group;
  kvs::SplitPlan split;
  size_t off_pm, off_pl, off_consts, bytes;
};

H2OPlan plan_h2o(const kvs_h2o_desc *d) {
  H2OPlan p{};
  p.group = (d->cap + 63) / 64;
  p.split = kvs::attn_split_plan(
      d->batch * d->heads * kvs::attn_head_split(p.group, false).hsplit, d->cap);
  const size_t heads = (size_t)d->batch * d->heads * p.group;
  p.off_pm = 0;
  p.off_pl = align_up(heads * p.split.splits * 64 * 4);
  p.off_consts = align_up(p.off_pl + heads * p.split.splits * 64 * 4);
  p.bytes = align_up(p.off_consts + heads * 64 * 16);
  return p;
}

}  // namespace

KVS_API size_t kvs_h2o_workspace_bytes(const kvs_h2o_desc *desc, int32_t mode) {
  if (check_h2o(desc, mode) != KVS_OK) return 0;
  if (mode == KVS_H2O_DECODE) return 0;
  return plan_h2o(desc).bytes;
}

KVS_API kvs_status kvscore_h2o_accumulate(const kvs_h2o_desc *desc, int32_t mode, const void *q,
                                          void *K, void *V, const void *k_new,
                                          const void *v_new, const int32_t *write_slot,
                                          int32_t *slot_pos, float *acc, void *O,
                                          int32_t *evict_slot, void *ws, size_t ws_bytes,
                                          void *stream) {
  kvs_status st = check_h2o(desc, mode);
  if (st != KVS_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (mode == KVS_H2O_PREFILL) {
    if (!q || !K || !acc) return fail(KVS_ERR_INVALID, "prefill: q, K and acc are required");
    st = check_aligned("prefill", {q, K});
    if (st != KVS_OK) return st;
    const H2OPlan p = plan_h2o(desc);
    st = check_ws(ws, ws_bytes, p.bytes);
    if (st != KVS_OK) return st;
    const kvs::RowGeom geo{1, desc->cap, 64, 0, p.group};
    float *pm = at<float>(ws, p.off_pm), *pl = at<float>(ws, p.off_pl);
    float4 *consts = at<float4>(ws, p.off_consts);
    if (desc->dtype != KVS_F32)  // 16-bit prompts: the balanced two-pass kernels
      return hip_status(kvs::launch_prefill(desc->dtype, desc->d, q, K, desc->batch, desc->heads,
                                            desc->cap, consts, acc, s),
                        "prefill accumulate");
    hipError_t e = kvs::launch_attn_partial(desc->dtype, desc->d, false, q, K, nullptr, geo,
                                            desc->batch, desc->heads, p.split, pm, pl, nullptr, s);
    if (e != hipSuccess) return hip_status(e, "prefill row statistics");
    e = kvs::launch_attn_combine_rows(pm, pl, desc->batch * desc->heads * p.group, p.split.splits,
                                      p.group, desc->cap, consts, s);
    if (e != hipSuccess) return hip_status(e, "prefill row combine");
    e = kvs::launch_score(desc->dtype, desc->d, 1, q, K, nullptr, nullptr, nullptr, consts, nullptr,
                          0, geo, desc->batch, desc->heads, 0.f, 1.f, acc, s);
    return hip_status(e, "prefill column sums");
  }
  if (!q || !K || !V || !k_new || !v_new || !slot_pos || !acc)
    return fail(KVS_ERR_INVALID, "decode: q, K, V, k_new, v_new, slot_pos and acc are required");
  st = check_aligned("decode", {q, K, V, k_new, v_new, O});
  if (st != KVS_OK) return st;
  hipError_t e = kvs::launch_h2o_decode(desc->dtype, desc->d, desc->batch * desc->heads, desc->cap,
                                        desc->cur_len, desc->k_heavy, desc->k_recent, q, K, V,
                                        k_new, v_new, write_slot,
                                        slot_pos, acc, O, evict_slot, s);
  return hip_status(e, "decode step");
}

KVS_API kvs_status kvs_measure_peaks(void *buf, size_t bytes, float *mfma_bf16_tflops,
                                     float *hbm_read_gbs, void *stream) {
  if (!buf || !mfma_bf16_tflops || !hbm_read_gbs)
    return fail(KVS_ERR_INVALID, "kvs_measure_peaks: a required pointer is NULL");
  if (bytes < ((size_t)66 << 20))
    return fail(KVS_ERR_INVALID, "kvs_measure_peaks: the buffer must hold at least 66 MiB");
  if (check_aligned("kvs_measure_peaks", {buf}) != KVS_OK) return KVS_ERR_INVALID;
  const hipError_t e = kvs::measure_peaks(buf, bytes, mfma_bf16_tflops, hbm_read_gbs,
                                          static_cast<hipStream_t>(stream));
  return hip_status(e, "kvs_measure_peaks");
}

KVS_API kvs_status kvs_timing_enable(int32_t on) {
  kvs::timing_enable(on);
  return ok();
}

KVS_API int32_t kvs_timing_count(void) { return kvs::timing_count(); }

KVS_API kvs_status kvs_timing_read(int32_t i, const char **kernel, float *ms) {
  if (!kernel || !ms) return fail(KVS_ERR_INVALID, "kvs_timing_read: NULL output");
  const int rc = kvs::timing_read(i, kernel, ms);
  if (rc == 1) return fail(KVS_ERR_INVALID, "kvs_timing_read: index out of range");
  if (rc == 2) return fail(KVS_ERR_HIP, "kvs_timing_read: event query failed");
  return ok();
}

KVS_API void kvs_timing_reset(void) { kvs::timing_reset(); }
