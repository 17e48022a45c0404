/*
 * tg_oracle.h -- plain, slow CPU oracle for the token-gated prefill path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link
 * or call this; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no source with the HIP library.
 *
 * All floating-point work is fp64 on the exact input values.  Every
 * function follows the plain definition of its step; parallelism (OpenMP)
 * is only across independent outputs and never changes the arithmetic of
 * one output.
 *
 * Sources (the pages describing TokenGate):
 *   [S1] "TokenGate: Adapting LLMs for Fast and Memory-Efficient Prefill with
 *        Learned Token Pruning" (ai.info AI summary), sections "Key
 *        Contributions", "Methodology in Plain English", "Main Findings".
 *   [S2] "TokenGate Learned Token Pruning LLM Prefill Explained"
 *        (techbycountry), section "how the gate works".
 *   [S5] "TokenGate: Adapting LLMs for pre-fill with learned skimming for
 *        ~11x speedup" (wpnews mirror of the project README), sections
 *        "How it works" and "Quick start".
 */
#ifndef TG_ORACLE_H
#define TG_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Gate scorer, [S1] Key Contributions item 1, [S2] how the gate works,
 * [S5] How it works: RMSNorm of the post-attention residual, then an MLP
 * d -> h (SiLU) -> 1.  Non-prunable rows get score 0.
 * resid [T][d], w1 [h][d], gamma [d] or NULL (=1), b1 [h] or NULL (=0),
 * w2 [h]; scores [T] out. */
void tgo_gate_score(int64_t T, int64_t d, int64_t h, const double* resid,
                    const uint8_t* prunable, const double* gamma, double eps,
                    const double* w1, const double* b1, const double* w2,
                    double b2, double* scores);

/* Top-K selection and order-preserving compaction, [S1] Key Contributions
 * item 1 and Methodology: the K highest-scoring prunable tokens plus every
 * non-prunable token are kept; kept tokens keep their original order.
 * Scores are fp32 (the precision the selection is taken in); ties go to the
 * lower index; NaN ranks below every number; -0 equals +0.  K >= |P| keeps
 * every prunable token.  Writes the kept indices ascending into kept_idx
 * (capacity T) and returns their number, or -1 if K < 0 or T < 0. */
int64_t tgo_topk_select(int64_t T, const float* scores,
                        const uint8_t* prunable, int64_t K, int32_t* kept_idx);

/* Row gather into kept order, [S1] Key Contributions item 1 and [S5] How it
 * works: upper layers see only the kept rows.  Copies row bytes verbatim;
 * pos_kept[r] = kept_idx[r]; score_kept[r] = scores[kept_idx[r]]. */
void tgo_compact_gather(int64_t N, int64_t row_bytes, const uint8_t* resid,
                        int64_t resid_row_bytes, const float* scores,
                        const int32_t* kept_idx, uint8_t* resid_kept,
                        int32_t* pos_kept, float* score_kept);

/* Lower layers' KV cache gathered to the kept tokens ([S1] Key
 * Contributions item 1: upper layers hold no KV entries for pruned tokens;
 * the lower layers' entries are compacted with the same kept indices):
 * out[l][r] = cache[l][kept_idx[r]] for l < L, r < N; rows of row_bytes
 * bytes, cache [L][T] rows, out [L][N] rows. */
void tgo_kv_gather(int64_t L, int64_t T, int64_t N, int64_t row_bytes,
                   const uint8_t* cache, const int32_t* kept_idx, uint8_t* out);

/* Token-gated attention forward, [S1] Key Contributions item 2 and 3,
 * Methodology ("added before the online softmax"), [S2] how the gate works:
 * for query row r, query head hq, key c (c <= r when causal):
 *   z = c_r * ( scale * <Q[r,hq], K[c,kv]> + gain[hq] * key_score[c] ),
 *   kv = hq / (Hq / Hkv),
 *   O[r,hq] = sum_c softmax_c(z) V[c,kv],  LSE[hq,r] = log sum_c exp(z).
 * q [N][Hq][D], k and v [N][Hkv][D], key_score [N], gain [Hq],
 * q_scale [N] or NULL (=1).  rows selects which query rows to compute
 * (NULL = all N rows, n_rows ignored); out [n_rows][Hq][D],
 * lse [Hq][n_rows] or NULL.  A row whose logits are all -inf gets O = 0
 * and LSE = -inf. */
void tgo_bias_attn(int64_t N, int64_t Hq, int64_t Hkv, int64_t D,
                   const double* q, const double* k, const double* v,
                   const double* key_score, const double* gain,
                   const double* q_scale, double scale, int causal,
                   const int64_t* rows, int64_t n_rows, double* out,
                   double* lse);

/* Number of threads the OpenMP loops above use (1 without OpenMP). */
/* Gradients of token-gated attention (TokenGate pages: ai.info summary "Key
 * Contributions" items 2 and 3 -- the gate is trained end to end through the
 * attention bias, which needs the gradient of the logits with respect to the
 * key scores and the per-head gains).  With the forward of tgo_bias_attn and
 * an upstream gradient dout [N][Hq][D], writes dq [N][Hq][D], dk, dv
 * [N][Hkv][D], dscore [N] and dgain [Hq], all fp64.  Recomputes the
 * softmax from its definition. */
void tgo_bias_attn_bwd(int64_t N, int64_t Hq, int64_t Hkv, int64_t D,
                       const double* q, const double* k, const double* v,
                       const double* key_score, const double* gain,
                       const double* q_scale, double scale, int causal,
                       const double* dout, double* dq, double* dk, double* dv,
                       double* dscore, double* dgain);

int tgo_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
