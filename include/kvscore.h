/*
 * kvscore.h -- C ABI of the KV-cache scoring and eviction library (gfx950).
 *
 * The library scores every cached key/value token of every KV head against a
 * set of scoring queries, keeps each head's top-B tokens plus a protected set,
 * and compacts the cache.  Two methods are covered:
 *
 *  * LORE-KV (project page "Monte Carlo Estimation for KV-Cache Eviction",
 *    Method section): the projected deletion score of Eqs. 5-7 under the
 *    w prompt-window queries and the M x T Monte Carlo lookahead queries,
 *    per-KV-head top-B selection with the attention sink and window protected
 *    (Eq. 8), chunk pooling ("chunk", Hyperparameters table), compaction.
 *  * H2O (summary page "H2O: Heavy-Hitter Oracle", 3.4 and System
 *    Implementation Details): accumulated attention per cached token, and the
 *    decode-time eviction of the lowest-accumulated non-recent token from a
 *    preallocated slot cache.
 *
 * Conventions shared by every entry point
 *  - Every tensor pointer is a DEVICE pointer to memory the caller owns and
 *    keeps alive until the enqueued work has finished.  The library keeps no
 *    device memory between calls; scratch comes from a caller workspace.
 *  - Tensors are dense, row-major, in the layouts stated per argument.  The
 *    base address of every tensor of the descriptor's dtype (and of O) must
 *    be 16-byte aligned (KVS_ERR_INVALID otherwise): rows are moved with
 *    16-byte vector accesses.
 *    Element type of Q, K, V, W_O (and of the H2O inputs) is the descriptor's
 *    dtype; statistics and scores are fp32; indices are int32.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the default stream).  No call synchronises the device or copies between
 *    host and device.
 *  - Arguments are checked on the host before anything is enqueued.  A failed
 *    check returns KVS_ERR_INVALID / KVS_ERR_UNSUPPORTED / KVS_ERR_WORKSPACE
 *    and enqueues nothing.  A failed launch returns KVS_ERR_HIP.  The reason
 *    is available from kvs_last_error() (thread-local).  Nothing aborts or
 *    prints.
 *  - Outputs must not alias inputs unless an argument says it is in/out.
 *  - Sequences x heads (batch * h_kv, batch * heads) and the query heads h_q
 *    of one call are at most 65535: each indexes one grid dimension of a
 *    launch.  More returns KVS_ERR_UNSUPPORTED.
 *  - Calls on one stream run in order; calls on different streams that share
 *    a workspace race.
 */
#ifndef KVSCORE_H
#define KVSCORE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KVS_F32 = 0, KVS_BF16 = 1, KVS_F16 = 2 } kvs_dtype;

typedef enum {
  KVS_OK = 0,
  KVS_ERR_INVALID = 1,     /* malformed shape, null pointer, out-of-range hyperparameter */
  KVS_ERR_UNSUPPORTED = 2, /* well-formed but outside what the kernels implement */
  KVS_ERR_WORKSPACE = 3,   /* workspace missing or smaller than kvs_lore_workspace_bytes() */
  KVS_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} kvs_status;

/*
 * One LORE-KV eviction over one layer of `batch` independent sequences.
 *
 *  n        cached tokens per sequence and KV head (the prompt length).
 *  h_q,h_kv query heads and KV heads; query head h reads KV head h/(h_q/h_kv).
 *           h_q % h_kv == 0 and the group size h_q/h_kv is at most 16.
 *  d        head dimension, 64 or 128.
 *  d_model  rows of W_O.
 *  w,m,t    scoring rows per query head: n_q = w + m*t, 1 <= n_q <= 64.
 *           Rows 0..w-1 are the window queries of the last w prompt tokens
 *           (LORE-KV "Prefill"); row r < w sits at position n-w+r and attends
 *           to tokens 0..n-w+r.  Row w + j*t + u is lookahead query u of
 *           trajectory j (Eq. 1) and attends to all n tokens.
 *  n_sink   protected prefix (the attention sink); the last w tokens are
 *           protected too.  Candidates are [n_sink, n - w); n >= n_sink + w.
 *  chunk    adjacent-token grouping: a candidate's ranking score is the mean
 *           score of the candidates in its aligned group [chunk*floor(i/chunk),
 *           +chunk).  chunk >= 1.
 *  budget   B: candidates kept per KV head.  n_keep = n_sink + min(B, n-n_sink-w) + w.
 *  eps      the renormalisation guard of Eq. 5 (>= 0).
 *  lambda_l weight of the lookahead term in Eq. 7 (finite, >= 0).
 *  dtype    element type of Q, K, V and W_O.
 *
 * Scores use softmax(q.k / sqrt(d)) probabilities a, attention outputs
 * o = sum_i a_i v_i, e = a/(1-a+eps) * ||W_h (v_i - o)|| with W_h the d_model
 * x d column slice h*d..h*d+d-1 of W_O, the arithmetic mean over each query
 * set (window; each trajectory), lookahead trajectories weighted by omega
 * and lambda_l, and the mean over the query heads of a KV head's group.
 */
typedef struct {
  int32_t batch, n, h_q, h_kv, d, d_model;
  int32_t w, m, t;
  int32_t n_sink, chunk, budget;
  float eps, lambda_l;
  int32_t dtype; /* kvs_dtype */
} kvs_lore_desc;

/* Bytes of workspace any LORE entry point below needs for `desc` (0 if the
 * descriptor is invalid; kvs_last_error() then says why).  One workspace may
 * serve all of them in turn on one stream. */
size_t kvs_lore_workspace_bytes(const kvs_lore_desc *desc);

/* Visibility of the cached tokens to the query rows. */
typedef enum {
  KVS_MASK_NONE = 0,           /* every row sees all n tokens */
  KVS_MASK_WINDOW_CAUSAL = 1,  /* LORE-KV scoring rows: window row r < w sees tokens
                                  0..n-w+r (causal at its own position), lookahead rows all n */
  KVS_MASK_CAUSAL = 2,         /* prompt row r sees 0..r (H2O prefill: KVS_H2O_PREFILL) */
  KVS_MASK_SLOTS = 3           /* the occupied slots of a slot cache (H2O decode: KVS_H2O_DECODE) */
} kvs_mask;

/*
 * Pass 1: softmax statistics and attention outputs of the scoring rows.
 * (LORE-KV Method: a_{q,i} and o_q of Eq. 5.)
 *
 *  mask     KVS_MASK_WINDOW_CAUSAL (the LORE-KV scoring rows; the statistics
 *           kvscore_deletion needs) or KVS_MASK_NONE (every row sees every
 *           token, e.g. held-out queries).  The causal and slot masks are
 *           the H2O modes of kvscore_h2o_accumulate: KVS_ERR_UNSUPPORTED here.
 *  Q        [batch][h_q][n_q][d]      scoring queries (window rows first).
 *  K, V     [batch][h_kv][n][d]       the cache.
 *  row_max  [batch][h_q][n_q] fp32    out: max_i q.k_i / sqrt(d) over visible i.
 *  row_sum  [batch][h_q][n_q] fp32    out: sum_i exp(q.k_i/sqrt(d) - row_max).
 *  O        [batch][h_q][n_q][d] fp32 out: o_q = sum_i a_{q,i} v_i.
 *  P        [batch][h_q][n_q][n] fp32 out, nullable: the probabilities a_{q,i}
 *           themselves, 0 where the mask hides token i from row q.  The path
 *           does not need them (the score pass recomputes each probability
 *           from q.k and the row statistics), so they are formed only when P
 *           is given, by an extra pass over K after the statistics
 *           (1 GiB per layer of the 128K workload).
 *  ws, ws_bytes                       workspace (>= kvs_lore_workspace_bytes).
 */
kvs_status kvscore_probs(const kvs_lore_desc *desc, int32_t mask, const void *Q, const void *K,
                         const void *V, float *row_max, float *row_sum, float *O, float *P,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * Pass 2: projected deletion score of every cached token, per KV head
 * (LORE-KV "Projected deletion score", Eqs. 5-7, grouped per KV head as the
 * selection of Eq. 8 needs).
 *
 *  Q, K, V                  as for kvscore_probs.
 *  W_O      [d_model][h_q*d] the attention output projection (linear-layer layout).
 *  omega    [batch][m] fp32  trajectory reliability weights (Eq. 10 output, a
 *           softmax).  The domain is omega >= 0.  A row whose weight
 *           lambda_l * omega_j / t is below FLT_MIN (1.2e-38) -- in particular
 *           any omega_j <= 0, which lies outside the domain -- contributes
 *           nothing to S: the kernel folds log2 of the row weight into the
 *           exponent of a, so it cannot carry a negative or subnormal weight.
 *           For omega_j < 0 this differs from Eq. 7 read literally (which
 *           would subtract that trajectory's term); no error is raised, since
 *           omega lives in device memory and is not read on the host.
 *  row_max, row_sum, O      kvscore_probs outputs for the same inputs, under
 *                           KVS_MASK_WINDOW_CAUSAL (the score recomputes the
 *                           probabilities with that mask).
 *  S        [batch][h_kv][n] fp32 out: the KV head's score of every token
 *           (protected tokens are scored too; selection ignores them).
 *
 * For bf16 input the value-side products (V.G_h, V.y, P.V) run in fp16 after
 * a bf16->fp16 conversion of V.  That conversion is exact in fp16's normal
 * range (2^-14 <= |v| < 65504); smaller magnitudes become fp16 subnormals,
 * truncated (absolute error below 2^-24); |V| must stay below 65504.
 */
kvs_status kvscore_deletion(const kvs_lore_desc *desc, const void *Q, const void *K, const void *V,
                            const void *W_O, const float *omega,
                            const float *row_max, const float *row_sum, const float *O,
                            float *S, void *ws, size_t ws_bytes, void *stream);

/*
 * Trajectory reliability weights omega, the input of kvscore_deletion's
 * lookahead term (LORE-KV Method, "Reliability weights", Eqs. 2-4 and 10):
 *   c_u = log q(y_u) + H_u per sampled token; cbar_m, Hbar_m = means over the
 *   trajectory's t tokens; R_m = beta cbar_m - gamma Hbar_m - lambda_d Dhat_m;
 *   omega = softmax(R) over the m trajectories of each sequence.
 * Dhat_m is the trajectory's standardized cosine disagreement, read as: D_m =
 * mean of (1 - cos) over every query head and every pair (a query of
 * trajectory m, a query of another trajectory) at that head (a zero query has
 * cosine 0); Dhat = (D - mean D) / std D over the trajectories (population
 * std), and 0 when that std is below 1e-6 (m = 2 always gives 0).  The window
 * rows are not read.  Presets: LORE-KV /E (beta, gamma, lambda_d) = (1, 1.3, 0),
 * /D = (1, 1, 0.3) (KVS_RELIABILITY_E / KVS_RELIABILITY_D below).
 *
 *  Q        [batch][h_q][n_q][d]  the scoring queries (as for kvscore_probs);
 *           rows w + j*t .. w + j*t + t - 1 are trajectory j's.
 *  logp     [batch][m][t] fp32    log-probability of each sampled token.
 *  entropy  [batch][m][t] fp32    entropy of the distribution it was drawn from.
 *  omega    [batch][m] fp32       out: the weights (each row sums to 1).
 *  dhat     [batch][m] fp32       out, nullable: Dhat.
 *  ws, ws_bytes                   workspace (>= kvs_lore_workspace_bytes; not
 *                                 read when m = 1).
 * m = 0 is a no-op; m above 64 is KVS_ERR_UNSUPPORTED.  Cosines, norms and all
 * sums run in fp64 in a fixed order (deterministic).
 */
#define KVS_RELIABILITY_E 1.0f, 1.3f, 0.0f
#define KVS_RELIABILITY_D 1.0f, 1.0f, 0.3f
kvs_status kvscore_reliability_weights(const kvs_lore_desc *desc, const void *Q,
                                       const float *logp, const float *entropy,
                                       float beta, float gamma, float lambda_d,
                                       float *omega, float *dhat,
                                       void *ws, size_t ws_bytes, void *stream);

/*
 * Attention-output fidelity of a retained cache (LORE-KV page, "Why it
 * works", "Output fidelity": how closely the retained cache reproduces the
 * full cache's attention outputs), read as: for each held-out query row r of
 * query head h, the cosine between o_full = softmax(q K^T / sqrt(d)) V over all
 * n tokens of the head's KV head and o_kept, the same over the n_keep kept
 * tokens (renormalised), in the head's value space; fidelity = the mean over
 * the sequence's heads and rows.  Two zero outputs agree (1); one zero output
 * gives 0.  Reads desc->batch, n, h_q, h_kv, d, dtype only.
 *
 *  Qf       [batch][h_q][n_f][d]      held-out queries, 1 <= n_f <= 64; every
 *                                     row sees every token (no mask).
 *  K, V     [batch][h_kv][n][d]       the full cache.
 *  K_keep, V_keep [batch][h_kv][n_keep][d]  the retained cache (e.g.
 *                                     kv_compact's output), 1 <= n_keep <= n.
 *  cos_out  [batch][h_q][n_f] fp32    out: per-row cosines.
 *  fidelity [batch] fp32              out: their mean per sequence.
 *  ws, ws_bytes                       workspace (>= kvs_fidelity_workspace_bytes).
 * The attention outputs carry the precision of kvscore_probs' O; the cosines
 * are fp32.
 */
size_t kvs_fidelity_workspace_bytes(const kvs_lore_desc *desc, int32_t n_f, int32_t n_keep);
kvs_status kvscore_output_fidelity(const kvs_lore_desc *desc, int32_t n_f, int32_t n_keep,
                                   const void *Qf, const void *K, const void *V,
                                   const void *K_keep, const void *V_keep,
                                   float *cos_out, float *fidelity,
                                   void *ws, size_t ws_bytes, void *stream);

/*
 * Counter-causal attention over a cache (counter-causal review "Back from the
 * Future", 3.2: a strictly upper-triangular mask over the cached keys and
 * values, with fresh queries at the original positions).  The query of cached
 * position i attends to the keys of positions j > i only; the last position
 * sees none (row_max -inf, row_sum 0, O 0; the refresh keeps it regardless).
 * The outputs feed the caller's layer output and LM head, which turn them into
 * the surprise logits that kvscore_refresh ranks.  Reads desc->batch, n, h_q,
 * h_kv, d, dtype only.
 *
 *  Q        [batch][h_q][n][d]      the fresh query of every cached position.
 *  K, V     [batch][h_kv][n][d]     the cache (query head h uses KV head h / (h_q/h_kv)).
 *  row_max  [batch][h_q][n] fp32    out: max_{j>i} q_i.k_j / sqrt(d).
 *  row_sum  [batch][h_q][n] fp32    out: sum_{j>i} exp(q_i.k_j/sqrt(d) - row_max).
 *  O        [batch][h_q][n][d] fp32 out: the attention output of each position.
 * No workspace.  Cost: about n^2/2 key visits per query head.  n above 2^22,
 * or h_q * ceil(n/64) above about 262000 (one launch's grid), is
 * KVS_ERR_UNSUPPORTED.
 */
kvs_status kvscore_counter_causal(const kvs_lore_desc *desc, const void *Q, const void *K,
                                  const void *V, float *row_max, float *row_sum, float *O,
                                  void *stream);

/*
 * Memory refresh (counter-causal review, Alg. 3 "Memory refresh step", design
 * choice 4, and the last-token rule of 3.2 Step 5): of the n cached tokens
 * (memory J plus buffer h) keep the J of largest surprise, with the n_sys
 * system-prompt tokens never evicted and the last token always kept; ties go
 * to the lower position.  One token-level kept list per sequence serves every
 * head; K, V and the token ids are gathered with it, in ascending position
 * order.  J = 0 keeps nothing (no work is enqueued); J >= n keeps all.
 *
 *  surprise [batch][n] fp32          the score of each token (larger = keep).
 *  K, V     [batch][heads][n][d]     the cache (dtype).
 *  ids      [batch][n] int32, nullable  token ids (with ids_out).
 *  kept     [batch][min(J,n)] int32  out: kept positions, ascending.
 *  K_out, V_out [batch][heads][min(J,n)][d]  out: the new memory.
 *  ids_out  [batch][min(J,n)] int32, nullable  out: their token ids.
 *  ws, ws_bytes                      workspace (>= kvs_refresh_workspace_bytes).
 * J in [1, n_sys] (no room for the last token beside the system prompt) is
 * KVS_ERR_INVALID.
 */
size_t kvs_refresh_workspace_bytes(int32_t batch, int32_t n);
kvs_status kvscore_refresh(int32_t batch, int32_t heads, int32_t n, int32_t d, int32_t dtype,
                           int32_t n_sys, int32_t J, const float *surprise, const void *K,
                           const void *V, const int32_t *ids, int32_t *kept, void *K_out,
                           void *V_out, int32_t *ids_out, void *ws, size_t ws_bytes,
                           void *stream);

/* Which prompt-side baseline kvscore_baseline_scores computes. */
typedef enum { KVS_BASELINE_WINDOW = 0, KVS_BASELINE_TOVA = 1 } kvs_baseline;

/*
 * Prompt-side attention scores of every cached token, per KV head, for the
 * same selector: the baselines the LORE-KV page sets its score against
 * ("The query-reference mismatch", "Prompt-side eviction": tokens ranked by
 * how the last w prompt tokens attend to them), and the single-query form of
 * the counter-causal review's background paragraph on TOVA ("Prerequisites":
 * the most recent token's attention over the cache).  Lookahead rows are not
 * read.
 *
 *  kind     KVS_BASELINE_WINDOW: S_i = mean over the KV head's query heads of
 *           sum_{r<w} a_{r,i}.  KVS_BASELINE_TOVA: the same with the last
 *           window row only (r = w - 1, the last prompt token).
 *  Q, K     as for kvscore_probs (V is not read).
 *  row_max, row_sum  kvscore_probs outputs for the same inputs.
 *  S        [batch][h_kv][n] fp32 out.
 *  ws, ws_bytes  the LORE workspace (>= kvs_lore_workspace_bytes).
 * Errors: KVS_ERR_INVALID for an unknown kind, w < 1 or a NULL pointer.
 */
kvs_status kvscore_baseline_scores(const kvs_lore_desc *desc, int kind, const void *Q,
                                   const void *K, const float *row_max, const float *row_sum,
                                   float *S, void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace kvscore_topb_select needs (0 if the selection fields of
 * the descriptor are invalid).  No larger than kvs_lore_workspace_bytes(). */
size_t kvs_topb_workspace_bytes(const kvs_lore_desc *desc);

/*
 * Per-KV-head top-B selection (LORE-KV Eq. 8 with chunk pooling).
 * Reads only batch, h_kv, n, n_sink, w, chunk and budget of the descriptor,
 * so it also serves any other per-row score (the H2O prompt reduction uses
 * n_sink = 0, w = recent budget, chunk = 1, budget = heavy budget).
 *
 *  S       [batch][h_kv][n] fp32   scores (kvscore_deletion output, or any score).
 *  kept    [batch][h_kv][n_keep] int32 out: kept token indices, ascending:
 *          [0, n_sink) + the B best candidates by (pooled score desc, index asc)
 *          + [n - w, n).
 *  pooled  [batch][h_kv][n] fp32 out, nullable: each candidate's pooled score;
 *          protected tokens get NaN.
 * NaN scores rank above every number.
 */
kvs_status kvscore_topb_select(const kvs_lore_desc *desc, const float *S, int32_t *kept,
                               float *pooled, void *ws, size_t ws_bytes, void *stream);

/*
 * Retention-order shift between two selections of the same budget (LORE-KV
 * page, "More analyses", "Retention-order shift"): per row, the share of
 * selection A's kept candidates -- indices in [n_sink, n - w) -- that
 * selection B does not keep; the protected tokens, kept by both, are left
 * out.  0 when A keeps no candidate.  With equal budgets the measure is
 * symmetric.
 *
 *  rows          number of kept lists (e.g. batch * h_kv).
 *  kept_a, kept_b [rows][n_keep] int32: kvscore_topb_select outputs.  kept_b
 *                must be ascending (as kvscore_topb_select writes it; an
 *                unsorted kept_b gives a wrong count, never an invalid read).
 *  shift         [rows] fp32 out.
 * Errors: KVS_ERR_INVALID for sizes out of range or NULL pointers.
 */
kvs_status kvscore_retention_shift(int32_t rows, int32_t n_keep, int32_t n, int32_t n_sink,
                                   int32_t w, const int32_t *kept_a, const int32_t *kept_b,
                                   float *shift, void *stream);

/*
 * kvscore_topb_select without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, outputs and results as
 * kvscore_topb_select; its scratch is a fixed array the library owns on each
 * GPU it runs on, KVS_TOPB_NOALLOC_MAX_BYTES bytes, held until the process
 * ends.  Nothing is allocated or freed by the call.
 *
 * Limit: kvs_topb_workspace_bytes(desc) must not exceed
 * KVS_TOPB_NOALLOC_MAX_BYTES (e.g. 1 x 8 KV heads x 131072 tokens with chunk
 * 4 needs 2 MiB; 3584 rows x 1024 tokens with chunk 1 needs 29 MiB); larger
 * inputs return KVS_ERR_UNSUPPORTED before anything is enqueued.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller.  A call rewrites everything of the scratch it reads, so the
 * contents left by an earlier call never matter.
 * Errors: as kvscore_topb_select; KVS_ERR_HIP if the scratch's device address
 * cannot be looked up on the current device.
 */
#define KVS_TOPB_NOALLOC_MAX_BYTES ((size_t)32 << 20)
kvs_status kvscore_topb_select_noalloc(const kvs_lore_desc *desc, const float *S, int32_t *kept,
                                       float *pooled, void *stream);

/*
 * Gather kept rows into a compact cache (LORE-KV: decoding then runs on the
 * compressed cache).  Also used to load the H2O slot cache after the prompt
 * reduction.
 *
 *  K, V      [batch][heads][n_src][d]  (dtype)   source cache.
 *  kept      [batch][heads][n_keep] int32         rows to copy.
 *  K_out, V_out [batch][heads][cap_dst][d]        out: rows 0..n_keep-1 get the copies;
 *            rows n_keep..cap_dst-1 are left untouched.
 *  pos_out   [batch][heads][cap_dst] int32, nullable   out: kept index per row, -1 beyond n_keep.
 *  score_in  [batch][heads][n_src] fp32, nullable       optional per-token score to carry along;
 *  score_out [batch][heads][cap_dst] fp32               out (needed iff score_in): gathered, 0 beyond n_keep.
 * The copy is bit-exact.  A kept index outside [0, n_src) copies nothing
 * (its output rows are left as they were) and records -1 / 0.
 */
kvs_status kv_compact(int32_t batch, int32_t heads, int32_t n_src, int32_t n_keep, int32_t cap_dst,
                      int32_t d, int32_t dtype, const void *K, const void *V, const int32_t *kept,
                      void *K_out, void *V_out, int32_t *pos_out,
                      const float *score_in, float *score_out, void *stream);

/* H2O modes: the mode fixes the mask (prefill: KVS_MASK_CAUSAL over the
 * prompt; decode: KVS_MASK_SLOTS over the occupied slots plus the new token). */
typedef enum {
  KVS_H2O_PREFILL = 0, /* accumulated attention of a causal prompt */
  KVS_H2O_DECODE = 1   /* one decode step on the slot cache */
} kvs_h2o_mode;

/*
 *  batch, heads, d   rows are (sequence, head) pairs, each independent (MHA).
 *  d                 64 or 128.
 *  cap               PREFILL: the prompt length P, at most 16384 (and
 *                    heads * ceil(P/256) at most 65535).  DECODE: slots
 *                    per row, at most 2048 (each row keeps its slot map,
 *                    accumulators and probabilities in LDS).  Larger values
 *                    return KVS_ERR_UNSUPPORTED before any launch.
 *  cur_len           DECODE: sequence length after appending this step's token
 *                    (the new token's position is cur_len - 1).
 *  k_heavy, k_recent DECODE: budget for this step; a token is recent if its
 *                    position is >= cur_len - k_recent.
 *  dtype             element type of q, K, V, k_new, v_new, O.
 */
typedef struct {
  int32_t batch, heads, d, cap;
  int32_t cur_len, k_heavy, k_recent;
  int32_t dtype;
} kvs_h2o_desc;

/*
 * H2O accumulated attention (H2O page 3.4: the accumulated score of a token is
 * the sum of the attention weights later queries give it; the new query
 * attends over the retained cache and itself; o~_i = o~_{i-1} + o_i; the
 * evictee is the retained non-recent token with the lowest accumulated score,
 * later position first on ties, at most one per step, Def. 2.1).
 *
 * KVS_H2O_PREFILL:
 *   q, K    [batch][heads][cap][d]  prompt queries and keys (row r attends to keys 0..r).
 *   acc     [batch][heads][cap] fp32 out: acc_i = sum_{r >= i} a_{r,i}.
 *   V, k_new, v_new, write_slot, slot_pos, O, evict_slot: unused (may be NULL).
 *   ws, ws_bytes: workspace of at least kvs_h2o_workspace_bytes(desc, mode).
 *
 * KVS_H2O_DECODE (one step; rows independent):
 *   q, k_new, v_new [batch][heads][d]   this step's query, key and value.
 *   K, V            [batch][heads][cap][d]  slot cache, in/out: the new token is
 *                   written into slot write_slot[row], or, with write_slot NULL,
 *                   into the lowest-index free slot.
 *   write_slot      [batch][heads] int32, nullable: the slot each row's new token
 *                   goes into; it must be free (slot_pos -1) and in [0, cap).  A
 *                   row whose write_slot is occupied or out of range is left
 *                   unchanged and reports evict_slot -2 (checked on the device).
 *   slot_pos        [batch][heads][cap] int32, in/out: position held by each slot,
 *                   -1 = free.  At least one slot must be free on entry.
 *   acc             [batch][heads][cap] fp32, in/out: accumulated attention per slot.
 *   O               [batch][heads][d] (dtype), nullable: out, attention output.
 *   evict_slot      [batch][heads] int32, nullable: out, slot evicted this step
 *                   (its slot_pos becomes -1) or -1 if the row is within
 *                   budget; -2 if the row had no free slot, or its write_slot
 *                   was not a free slot in range (nothing changed).
 *   ws, ws_bytes: unused.
 */
size_t kvs_h2o_workspace_bytes(const kvs_h2o_desc *desc, int32_t mode);

kvs_status kvscore_h2o_accumulate(const kvs_h2o_desc *desc, int32_t mode,
                                  const void *q, void *K, void *V,
                                  const void *k_new, const void *v_new,
                                  const int32_t *write_slot, int32_t *slot_pos, float *acc,
                                  void *O, int32_t *evict_slot,
                                  void *ws, size_t ws_bytes, void *stream);

/*
 * Measured ceilings, reported beside the published peaks (a diagnostic, not
 * part of the path): the dense bf16 MFMA rate of v_mfma_f32_16x16x32_bf16
 * issued back to back on four independent accumulators per wave (2048
 * workgroups of four waves), and the streaming HBM read rate of waves that
 * each read one contiguous 64 KiB range with eight 16-byte-per-lane loads in
 * flight (the row-read pattern of the H2O decode and the compaction).
 *
 *  buf, bytes  caller-owned device buffer, >= 66 MiB (use >= 1 GiB so the
 *              read exceeds the 256 MB last-level cache); its contents are
 *              read and partly overwritten.
 *  mfma_bf16_tflops, hbm_read_gbs  host outputs: best of three timed runs
 *              after a warm-up (HIP events on `stream`).
 * Unlike every other entry point this one waits for its own work.
 * Errors: KVS_ERR_INVALID for NULL pointers, a small or misaligned buffer.
 */
kvs_status kvs_measure_peaks(void *buf, size_t bytes, float *mfma_bf16_tflops,
                             float *hbm_read_gbs, void *stream);

/*
 * Per-launch kernel timing, for benchmarks and profiling.  While enabled,
 * every kernel the library launches is bracketed by two HIP events recorded
 * on its launch stream (process-wide).  kvs_timing_read synchronises on the
 * i-th record's stop event and returns the kernel's name (a static string)
 * and its event-to-event time in milliseconds.  kvs_timing_reset waits for
 * and drops every record.  Off by default.
 */
kvs_status kvs_timing_enable(int32_t on);
int32_t kvs_timing_count(void);
kvs_status kvs_timing_read(int32_t i, const char **kernel, float *ms);
void kvs_timing_reset(void);

/* Reason for the last non-OK status on the calling thread ("" if none). */
const char *kvs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVSCORE_H */
