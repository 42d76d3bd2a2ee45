// Host-side launchers of the gfx950 kernels (one per kernel family).  The C ABI
// in capi.cpp validates arguments, sizes workspaces and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvs {

enum ElemType { E_F32 = 0, E_BF16 = 1, E_F16 = 2 };

inline size_t elem_bytes(int t) { return t == E_F32 ? 4 : 2; }

// Geometry of the scoring rows (see attn.hip).
struct RowGeom {
  int mode;   // 0: LORE scoring rows; 1: causal prompt rows (H2O prefill);
              // 2: counter-causal rows (row at position R sees keys R+1 .. n-1)
  int n;      // keys per KV head (LORE: cache length; H2O: prompt length)
  int nq;     // LORE: rows per query head; counter-causal: 64-row blocks per query head
  int w;      // LORE: window rows
  int group;  // query heads (H2O: virtual heads of 64 prompt rows) per KV head
};

// Split-K plan of the attention pass.
struct SplitPlan {
  int splits;
  int tps;  // tokens per split, a multiple of 32
};
// Token ranges handled by one workgroup stay below this many tokens, so a
// range's rows (at most 512 bytes each) fit a 32-bit buffer offset.
constexpr int kMaxRangeTokens = 1 << 22;

SplitPlan attn_split_plan(int units, int n);
struct HeadSplit { int hsplit, hpw, maxw, qbw; };
HeadSplit attn_head_split(int group, bool with_o);

// Pass 1 partials -> combined statistics.  Counter-causal rows (RowGeom mode
// 2, one split covering all n keys) take part_m, part_l, part_O as the final
// row_max [batch*h_q][n], row_sum and O [batch*h_q][n][d] instead.
// part_m/part_l: [heads][splits][64]; part_O: [heads][splits][d][64].
hipError_t launch_attn_partial(int etype, int d, bool with_o, const void *Q, const void *K,
                               const void *V, RowGeom geo, int batch, int h_kv, SplitPlan plan,
                               float *part_m, float *part_l, float *part_O, hipStream_t st);
// LORE: writes row_max, row_sum [heads][nq] and O [heads][nq][d].
hipError_t launch_attn_combine_lore(int d, const float *part_m, const float *part_l,
                                    const float *part_O, int heads, int splits, int nq,
                                    float *row_max, float *row_sum, float *O, hipStream_t st);
// LORE: the dense probabilities P [batch][h_q][nq][n] from the combined
// statistics (geo.w = 0: every row sees every token).
hipError_t launch_probs_write(int etype, int d, const void *Q, const void *K,
                              const float *row_max, const float *row_sum, RowGeom geo, int batch,
                              int h_kv, float *P, hipStream_t st);
// H2O: writes per-row constants {beta2, 0, 1, last-visible bits} [heads][64].
hipError_t launch_attn_combine_rows(const float *part_m, const float *part_l, int heads,
                                    int splits, int group, int P, float4 *consts, hipStream_t st);

// Trajectory reliability weights: per-head cosine sums per trajectory pair
// (pair_sum: reliability_ws_bytes), then D, Dhat, R and omega per sequence.
size_t reliability_ws_bytes(int batch, int h_q, int m);
hipError_t launch_reliability(int etype, const void *Q, int batch, int h_q, int nq, int d, int w,
                              int m, int t, const float *logp, const float *entropy, float beta,
                              float gamma, float lambda_d, float *omega, float *dhat,
                              double *pair_sum, hipStream_t st);

// Output fidelity: cos_out [batch][rows] and its mean per sequence, from the
// fp32 attention outputs over the full and the kept cache, [batch][rows][d].
hipError_t launch_output_cosine(int d, const float *Of, const float *Ok, int batch, int rows,
                                float *cos_out, float *fidelity, hipStream_t st);

// Deletion score pieces.
int gram_splits(int h_q, int d_model, int elem_bytes);
// Row constants for the prompt-side baselines (window rows, or the last one).
hipError_t launch_baseline_prep(const float *row_max, const float *row_sum, int batch, int h_q,
                                int n, int nq, int w, bool last_only, float4 *consts,
                                hipStream_t st);
hipError_t launch_gram(int etype, int d, const void *W_O, int d_model, int h_q, int splits,
                       float *Gpart, hipStream_t st);
hipError_t launch_deletion_prep(int etype, int d, const float *Gpart, int gsplits, const float *O,
                                const float *row_max, const float *row_sum, const float *omega,
                                int batch, int h_q, int n, int nq, int w, int m, int t,
                                float lambda_l, void *Gv, float *Gr, void *Yhi, void *Ylo,
                                float4 *consts, hipStream_t st);
hipError_t launch_vnorm(int etype, int d, const void *V, const void *Gv, int batch, int n,
                        int n_pad, int h_q, int h_kv, float *Nn, hipStream_t st);
// mode 0: LORE deletion score (Yhi/Ylo, consts, Nn used); mode 1: causal column sums.
hipError_t launch_score(int etype, int d, int mode, const void *Q, const void *K, const void *V,
                        const void *Yhi, const void *Ylo, const float4 *consts, const float *Nn,
                        int n_pad, RowGeom geo, int batch, int h_kv, float eps, float out_scale,
                        float *S, hipStream_t st);

// Selection and compaction.
size_t topb_workspace_bytes(int rows, int n, int chunk);
// Retention-order shift between two ascending kept lists per row.
hipError_t launch_retention_shift(int rows, int n_keep, int n_sink, int w, int n,
                                  const int32_t *kept_a, const int32_t *kept_b, float *shift,
                                  hipStream_t st);
// The library-owned scratch of the allocation-free selection: its size, and
// its device address on the current device (looked up once per device).
constexpr size_t kTopbScratchBytes = (size_t)32 << 20;
hipError_t topb_scratch(void **ptr);
hipError_t launch_topb(const float *S, int rows, int n, int n_sink, int w, int chunk, int budget,
                       int n_keep, void *ws, int32_t *kept, float *pooled, hipStream_t st);
// kept [rows / kept_div][n_keep]: rows share lists in groups of kept_div;
// pos_out and the 32-bit payload have one row per list.
hipError_t launch_compact(int rows, int n_src, int n_keep, int cap_dst, int row_bytes,
                          const void *K, const void *V, const int32_t *kept, void *K_out,
                          void *V_out, int32_t *pos_out, const void *payload_in,
                          void *payload_out, hipStream_t st, int kept_div = 1);

// Measured ceilings: dense bf16 MFMA TFLOP/s and streaming HBM read GB/s,
// on the caller's buffer (>= 64 MiB + 2 MiB); waits for its own work.
hipError_t measure_peaks(void *buf, size_t bytes, float *mfma_tflops, float *read_gbs,
                         hipStream_t st);

// H2O decode step.
// write_slot (nullable): the slot each row's new token goes into (else the
// lowest free one).
// H2O prefill accumulate for bf16/fp16 prompts (prefill.hip): row constants
// of the causal prompt rows into consts [batch*heads*ceil(P/64)][64], then
// the column sums into acc [batch*heads][P].
hipError_t launch_prefill(int etype, int d, const void *Q, const void *K, int batch, int heads,
                          int P, float4 *consts, float *acc, hipStream_t st);

hipError_t launch_h2o_decode(int etype, int d, int rows, int cap, int cur_len, int k_heavy,
                             int k_recent, const void *q, void *K, void *V, const void *k_new,
                             const void *v_new, const int32_t *write_slot, int32_t *slot_pos,
                             float *acc, void *O, int32_t *evict_slot, hipStream_t st);

}  // namespace kvs
