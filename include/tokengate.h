/*
 * tokengate.h -- C ABI of the token-gated prefill path on AMD Instinct
 * MI355X (gfx950).
 *
 * TokenGate (pages: "TokenGate: Adapting LLMs for Fast and Memory-Efficient
 * Prefill with Learned Token Pruning", ai.info summary; the techbycountry
 * explainer "TokenGate Learned Token Pruning LLM Prefill Explained"; the
 * README mirror "TokenGate: Adapting LLMs for pre-fill with learned skimming
 * for ~11x speedup") inserts a small gate at one layer L of a trained
 * transformer.  The gate scores every prunable token of the prompt, keeps the
 * K best plus every non-prunable token, and the layers above L run only on
 * the kept tokens, with the gate score added as a per-key, per-head bias to
 * their attention logits.  This library is that path's hot core:
 *
 *   tg_gate_score      RMSNorm + MLP scorer over the residual rows   [a1]
 *   tg_gate_pack_w1 / tg_gate_score_packed
 *                      the same scorer with W1 packed once at load   [a1]
 *   tg_topk_select     top-K selection and ordered compaction        [a2,a3]
 *   tg_compact_gather  gather of residual rows/positions/scores      [a4]
 *   tg_bias_attn_fwd   causal GQA attention with the gate bias       [a5]
 *   tg_kv_gather       lower layers' KV cache gathered to kept tokens
 *   tg_chain_*         the four calls captured as one HIP graph
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every data pointer is DEVICE memory owned by the caller.  The compute
 *   calls allocate no device memory; their scratch memory is caller-provided
 *   workspace, sized by a query: tg_topk_select's (tg_topk_workspace_size),
 *   the split attention's (tg_bias_attn_workspace_size) and the backward's
 *   (tg_bias_attn_bwd_workspace_size).  Only tg_chain_create allocates (the
 *   runtime's graph objects).
 * - Host-side state: the split attention's plans depend only on the shape
 *   and are kept in a bounded cache of the last 256 shapes, guarded by a
 *   mutex, so every call is thread-safe; the device properties are read
 *   once per device.
 * - Every call only enqueues work on `stream` (a hipStream_t; NULL means the
 *   null stream) and returns; nothing synchronises the device and nothing
 *   is read back to the host.  Results are valid once the stream reaches
 *   them.
 * - Errors are return codes.  All shape, dtype, pointer and alignment
 *   checks run on the host BEFORE any device work, so a call that returns
 *   anything but TG_OK has enqueued nothing (except TG_ERR_LAUNCH).  The
 *   library never aborts and never throws across this boundary.
 *   tg_last_error() returns a thread-local description of the last failure.
 * - Sizes are int64_t; token counts must fit in int32 (T <= 2^31 - 1).
 * - "bf16" is bfloat16 (1-8-7), "f32" is IEEE binary32; matrices are
 *   row-major with the stated row strides in ELEMENTS.
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tg_status {
  TG_OK = 0,
  TG_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative or inconsistent size, misalignment */
  TG_ERR_UNSUPPORTED = 2,      /* valid request outside what the kernels implement */
  TG_ERR_WORKSPACE = 3,        /* workspace missing or smaller than tg_topk_workspace_size() */
  TG_ERR_LAUNCH = 4            /* the HIP runtime refused a kernel launch */
} tg_status;

typedef enum tg_dtype { TG_DTYPE_F32 = 0, TG_DTYPE_BF16 = 1 } tg_dtype;

/* Static, never-NULL name of a status code. */
const char* tg_status_str(int status);

/* Thread-local, human-readable detail of the last failed call on this
 * thread ("" if none).  Valid until the next call on the same thread. */
const char* tg_last_error(void);

/* --------------------------------------------------------------------------
 * [a1] Gate scorer.  Pages: ai.info summary "Key Contributions" item 1 (a
 * scoring MLP over each token's RMSNorm-normalised post-attention residual
 * scores the prunable tokens) and the README mirror "How it works".
 *
 *   for prunable t:  u = gamma * x_t / sqrt(mean_i x_{t,i}^2 + eps)
 *                    s_t = b2 + sum_j w2_j * SiLU((W1 u)_j + b1_j)
 *   otherwise:       s_t = 0   (non-prunable tokens are never pruned, so
 *                               they carry no gate bias)
 *
 * dt          TG_DTYPE_BF16 or TG_DTYPE_F32: dtype of resid and w1.  The
 *             bf16 path multiplies on bf16 MFMA with fp32 accumulation; the
 *             f32 path is fp32 throughout.
 * T, d, h     tokens, hidden size, gate MLP width.  T >= 0 (T == 0 is a
 *             no-op), d >= 1, h >= 1.  bf16 path: d % 8 == 0 and
 *             h in {64, 128, 192, 256}.
 * resid       [T][resid_row_stride] of dt; row t's first d elements are x_t.
 *             bf16 path: resid and resid_row_stride*2 16-byte aligned.
 * prunable    [T] bytes, nonzero = prunable.
 * rms_weight  [d] f32 RMSNorm weight gamma, or NULL for all ones.
 * eps         >= 0.
 * w1          [h][d] of dt (Linear layout), 16-byte aligned on the bf16 path.
 * b1          [h] f32 or NULL (zeros).  w2 [h] f32.  b2 scalar.
 * scores      out [T] f32.
 * ------------------------------------------------------------------------ */
tg_status tg_gate_score(tg_dtype dt, int64_t T, int64_t d, int64_t h,
                        const void* resid, int64_t resid_row_stride,
                        const uint8_t* prunable, const float* rms_weight,
                        float eps, const void* w1, const float* b1,
                        const float* w2, float b2, float* scores,
                        void* stream);

/* --------------------------------------------------------------------------
 * [a1] Gate scorer with a packed W1.  The same operation as tg_gate_score
 * (same pages, same formula) for the bf16 path with a unit RMSNorm weight.
 * W1 is a constant of the trained gate, so it can be rearranged once, when
 * the weights are loaded, into the order in which the scorer's matrix-core
 * instructions consume it: then each 64-wide slice of the hidden dimension
 * is one contiguous block instead of h rows d*2 bytes apart.  The packed
 * bytes are an opaque layout (a permutation of W1's elements, no rounding);
 * only tg_gate_score_packed reads them.  Results equal tg_gate_score's for
 * the same W1, up to fp32 summation order.
 *
 * tg_gate_w1_packed_bytes  bytes of the packed W1 for (dt, h, d), or 0 when
 *             the layout does not cover them (it needs dt == TG_DTYPE_BF16,
 *             d % 64 == 0, d >= 128, h in {64, 128, 192, 256}).
 * tg_gate_pack_w1  reads w1 [h][d] bf16 (row-major, 16-byte aligned) and
 *             writes w1_packed (tg_gate_w1_packed_bytes bytes, 16-byte
 *             aligned, not overlapping w1).  Enqueued on `stream`.
 * tg_gate_score_packed  arguments as tg_gate_score, with w1_packed in place
 *             of w1; dt must be TG_DTYPE_BF16 and rms_weight NULL
 *             (TG_ERR_UNSUPPORTED otherwise).
 * ------------------------------------------------------------------------ */
size_t tg_gate_w1_packed_bytes(tg_dtype dt, int64_t h, int64_t d);

tg_status tg_gate_pack_w1(tg_dtype dt, int64_t h, int64_t d, const void* w1,
                          void* w1_packed, void* stream);

tg_status tg_gate_score_packed(tg_dtype dt, int64_t T, int64_t d, int64_t h,
                               const void* resid, int64_t resid_row_stride,
                               const uint8_t* prunable, const float* rms_weight,
                               float eps, const void* w1_packed, const float* b1,
                               const float* w2, float b2, float* scores,
                               void* stream);

/* --------------------------------------------------------------------------
 * [a2, a3] Top-K selection and order-preserving compaction.  Pages: ai.info
 * summary "Key Contributions" item 1 and "Methodology in Plain English": the
 * K highest-scoring prunable tokens plus ALL non-prunable tokens continue
 * upward; the README "Quick start" budget K = None keeps every prunable
 * token.
 *
 * Kept set = { t : !prunable[t] }  U  the first min(K, |P|) prunable tokens
 * ordered by (score descending, index ascending).  Scores compare as fp32
 * values: -0 == +0, +-inf are ordinary values, NaN ranks below every
 * number (NaNs tie, lower index first).  kept_idx lists the kept tokens in
 * ascending original order, so its length is N = min(K, |P|) + |not P|.
 *
 * T              tokens, 0 <= T <= 2^31 - 1.
 * scores         [T] f32 (values at non-prunable positions are ignored).
 * prunable       [T] bytes, nonzero = prunable.
 * K              budget, K >= 0.  K >= |P| keeps every token; K = 0 keeps
 *                only the non-prunable tokens.
 * kept_idx       out, [kept_capacity] int32.  Entries beyond the kept count
 *                are left untouched; kept entries at positions >=
 *                kept_capacity are dropped (so a capacity of T is always
 *                enough).
 * n_kept         out, [1] int32 on the device: the kept count N (may exceed
 *                kept_capacity, which signals a too-small capacity).  For
 *                24576 < T <= 524288 the selection is one launch of at most
 *                32 workgroups that wait for each other (at most one per
 *                CU); a wait is bounded, and if one gives up (the workgroups
 *                were not all running together) n_kept is -1 and kept_idx
 *                is invalid.
 * workspace      device scratch of at least tg_topk_workspace_size(T) bytes,
 *                256-byte aligned.  It must be all-zero before its first use;
 *                every call leaves it all-zero again when its kernels finish.
 *                Calls sharing a workspace must be ordered on one stream.
 * ------------------------------------------------------------------------ */
size_t tg_topk_workspace_size(int64_t T);

tg_status tg_topk_select(int64_t T, const float* scores,
                         const uint8_t* prunable, int64_t K,
                         int32_t* kept_idx, int64_t kept_capacity,
                         int32_t* n_kept, void* workspace,
                         size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------
 * tg_topk_select without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same operation, arguments, kernels
 * and results as tg_topk_select (bit for bit); its scratch is instead a
 * static device array of 64 KiB in the library, one copy per GPU, held until
 * the process ends, which covers every T up to 2^31 - 1 (the workspace of
 * the largest T is 53.5 KiB; a T whose workspace exceeded the array would
 * return TG_ERR_UNSUPPORTED).  The first call on a device looks the array up
 * and enqueues one kernel on `stream` that clears it; no call allocates.
 * Every call on one GPU shares that GPU's array, so calls that can overlap
 * on one GPU (unordered streams, threads) race: order them on one stream.
 * ------------------------------------------------------------------------ */
tg_status tg_topk_select_noalloc(int64_t T, const float* scores,
                                 const uint8_t* prunable, int64_t K,
                                 int32_t* kept_idx, int64_t kept_capacity,
                                 int32_t* n_kept, void* stream);

/* --------------------------------------------------------------------------
 * [a4] Gather into kept order.  Pages: ai.info summary "Key Contributions"
 * item 1 and the README mirror "How it works": layers above the gate
 * process, and keep KV entries for, only the kept tokens.
 *
 *   resid_kept[r][:] = resid[kept_idx[r]][:]   (bit copy of d elements)
 *   pos_kept[r]      = kept_idx[r]             (original position)
 *   score_kept[r]    = scores[kept_idx[r]]     (bit copy)
 *
 * T            rows in resid (bounds for kept_idx).  N >= 0 kept rows
 *              (N == 0 is a no-op).  d >= 1.
 * resid        [T][resid_row_stride] of dt.  resid_kept [N][kept_row_stride].
 *              Both pointers and both strides (in bytes) 16-byte aligned,
 *              resid_kept may be NULL (no rows copied).
 * scores       [T] f32; may be NULL only if score_kept is NULL.
 * kept_idx     [N] int32.  An index outside [0, T) yields a zero row,
 *              pos_kept = -1 and score_kept = 0 for that r (no fault).
 * pos_kept, score_kept   out [N], each may be NULL.
 * ------------------------------------------------------------------------ */
tg_status tg_compact_gather(tg_dtype dt, int64_t T, int64_t N, int64_t d,
                            const void* resid, int64_t resid_row_stride,
                            const float* scores, const int32_t* kept_idx,
                            void* resid_kept, int64_t kept_row_stride,
                            int32_t* pos_kept, float* score_kept,
                            void* stream);

/* --------------------------------------------------------------------------
 * [a5] Token-gated attention, forward.  Pages: ai.info summary "Key
 * Contributions" items 2 and 3 and "Methodology in Plain English": each kept
 * key's gate score, times a per-layer per-head gain, is added to the
 * attention logits of the upper layers before the online softmax; a
 * per-query temperature (driven by the ratio of the query's original
 * position to its rank among kept tokens) rescales the logits.
 *
 * For query row r, query head h, key c (c <= r when causal),
 *   kv = h / (Hq / Hkv)
 *   z  = q_scale[r] * ( softmax_scale * <Q[r,h,:], K[c,kv,:]> + gain[h] * key_score[c] )
 *   O[r,h,:] = sum_c softmax_c(z) * V[c,kv,:],   lse[h][r] = log sum_c exp(z)
 * A row whose logits are all -inf gets O = 0 and lse = -inf.  Inputs are
 * finite, except key_score, which may be -inf (the key is deleted); a NaN
 * anywhere gives unspecified results (the kernels are built assuming none).
 *
 * dt            TG_DTYPE_BF16 (bf16 MFMA, fp32 softmax; the weights are
 *               rounded to bf16 for the PV product and the normaliser sums
 *               those rounded weights, so lse carries their rounding, about
 *               4e-3 at most) or TG_DTYPE_F32.
 * N             kept tokens, 0 <= N <= 2^31 - 1 (N == 0 is a no-op).
 * Hq, Hkv       query / KV heads, Hkv >= 1, Hq % Hkv == 0.
 * D             head dim: 64, 128 or 256 (ai.info summary "Main Findings":
 *               the pages' kernel serves 128 for Qwen3 and 256 for Qwen3.5).
 * q             [N][Hq][D] of dt, contiguous.  k, v: [N][Hkv][D] of dt.
 *               16-byte aligned.
 * key_score     [N] f32 gate scores of the kept tokens, or NULL for no bias
 *               (plain attention; gain is then ignored).
 * gain          [Hq] f32, required when key_score != NULL.  Expected > 0
 *               (a softplus output); gain 0 with an infinite score is NaN.
 * q_scale       [N] f32 per-query logit scale, or NULL for all ones.
 *               Expected > 0.  A -inf key_score deletes its key exactly
 *               whenever softmax_scale * q_scale[r] > 2^-80.
 * softmax_scale <= 0 selects 1/sqrt(D).
 * causal        nonzero: key c is visible to query r only if c <= r.
 * out           out [N][Hq][D] of dt.  lse: out [Hq][N] f32, or NULL.
 * ------------------------------------------------------------------------ */
tg_status tg_bias_attn_fwd(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv,
                           int64_t D, const void* q, const void* k,
                           const void* v, const float* key_score,
                           const float* gain, const float* q_scale,
                           float softmax_scale, int causal, void* out,
                           float* lse, void* stream);

/* --------------------------------------------------------------------------
 * tg_bias_attn_fwd with a split of the key range (same operation, ai.info
 * summary "Key Contributions" items 2 and 3; results equal tg_bias_attn_fwd's
 * within the bf16 tolerance, rounding order aside).  On a bf16 prompt too
 * short for its workgroups to fill the chip, the longest causal rows alone
 * set the time; with a workspace the call cuts every long row's key tiles
 * into chunks run by separate workgroups, each chunk keeps the online-softmax
 * state of its keys (running max and sum in fp32; the unnormalised output
 * scaled by a power of two folded into the max, and rounded to fp16), and a
 * second kernel combines the chunks of each row as the online softmax
 * combines key tiles.  A cost model decides per shape whether
 * the split pays.
 *
 * tg_bias_attn_workspace_size  bytes the split needs for this shape, or 0
 *           when the shape runs unsplit (fp32, a grid that fills the chip,
 *           rows too short to cut, or a split the cost model prices above
 *           the unsplit launch).  Depends only on the arguments; invalid
 *           arguments also give 0.
 * workspace device memory of at least that many bytes, 16-byte aligned, or
 *           NULL: the call then runs unsplit, as tg_bias_attn_fwd.  Needs no
 *           initialisation; left undefined.  Calls sharing a workspace must
 *           be ordered on one stream.
 * Errors: those of tg_bias_attn_fwd, and TG_ERR_WORKSPACE when workspace is
 * given with workspace_bytes below the size query's value.
 * ------------------------------------------------------------------------ */
size_t tg_bias_attn_workspace_size(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv,
                                   int64_t D, int causal);

tg_status tg_bias_attn_fwd_ws(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv,
                              int64_t D, const void* q, const void* k,
                              const void* v, const float* key_score,
                              const float* gain, const float* q_scale,
                              float softmax_scale, int causal, void* out,
                              float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------
 * Token-gated attention, backward.  Pages: ai.info summary "Key
 * Contributions" items 2 and 3: the gate is trained end to end, and its
 * scores reach the loss only through the per-key bias gain_h * score_c, so
 * training needs the gradients of the biased attention with respect to the
 * scores and the gains as well as Q, K and V.
 *
 * With the forward of tg_bias_attn_fwd (same arguments) and an upstream
 * gradient dO, for z[h,r,c] = c_r (alpha <q_r,k_c> + gain_h score_c):
 *   dZ = P (dO V^T - <dO, O>)           (P the forward's softmax)
 *   dQ = c alpha dZ K,  dK = sum_h (c alpha dZ)^T Q,  dV = sum_h P^T dO
 *   dscore[c] = sum_{h,r} gain_h c_r dZ[h,r,c]
 *   dgain[h]  = sum_{r,c} score_c c_r dZ[h,r,c]   (keys with P = 0 add 0)
 *
 * dt            TG_DTYPE_BF16 only (TG_ERR_UNSUPPORTED otherwise).
 * D             64, 128 or 256 (TG_ERR_UNSUPPORTED otherwise).
 * q, k, v, key_score, gain, q_scale, softmax_scale, causal
 *               as given to tg_bias_attn_fwd.
 * out, lse      the forward's outputs: out [N][Hq][D] bf16 and lse [Hq][N]
 *               f32 (both required).
 * dout          [N][Hq][D] bf16, the gradient of the loss w.r.t. out.
 * dq            out, [N][Hq][D] bf16.  dk, dv: out, [N][Hkv][D] bf16.
 * dscore        out, [N] f32; dgain: out, [Hq] f32.  Required when
 *               key_score != NULL, ignored (not written) when it is NULL.
 * workspace     device memory of at least tg_bias_attn_bwd_workspace_size
 *               bytes (0 for invalid shapes), 16-byte aligned; needs no
 *               initialisation.  It holds Delta, the log-sum-exp in log2
 *               units and the fp32 partial sums of the dK/dV workgroups,
 *               which split each key block's query range into chunks when
 *               the prompt is short.  Calls sharing it must be ordered on
 *               one stream.
 * All tensors 16-byte aligned.  Results are deterministic (fixed-order
 * reductions, no atomics).  Errors: TG_ERR_INVALID_ARGUMENT,
 * TG_ERR_UNSUPPORTED, TG_ERR_WORKSPACE, with nothing enqueued.
 * ------------------------------------------------------------------------ */
size_t tg_bias_attn_bwd_workspace_size(int64_t N, int64_t Hq, int64_t Hkv,
                                       int64_t D);

tg_status tg_bias_attn_bwd(tg_dtype dt, int64_t N, int64_t Hq, int64_t Hkv,
                           int64_t D, const void* q, const void* k,
                           const void* v, const float* key_score,
                           const float* gain, const float* q_scale,
                           float softmax_scale, int causal, const void* out,
                           const void* dout, const float* lse, void* dq,
                           void* dk, void* dv, float* dscore, float* dgain,
                           void* workspace, size_t workspace_bytes,
                           void* stream);

/* --------------------------------------------------------------------------
 * Lower layers' KV cache gathered to the kept tokens.  Pages: ai.info summary
 * "Key Contributions" item 1 (layers above the gate never create KV entries
 * for pruned tokens) and "Methodology in Plain English" (the layers below
 * the gate ran on every token): compacting the lower layers' cache with the
 * same kept_idx leaves the prompt's whole KV cache holding kept tokens only.
 *
 *   k_kept[l][r] = k_cache[l][kept_idx[r]],  v_kept[l][r] = v_cache[l][kept_idx[r]]
 *
 * dt        dtype of the caches (bit copy; any dtype of that size works).
 * L, T, N   lower layers, prompt tokens, kept tokens (L, T, N >= 0).
 * Hkv, D    KV heads and head dim; Hkv * D * element size % 16 == 0.
 * k_cache, v_cache  [L][T][Hkv][D] contiguous, 16-byte aligned; either may
 *           be NULL together with its output (that tensor is skipped).
 * kept_idx  [N] int32, as written by tg_topk_select.  An index outside
 *           [0, T) yields a zero row.
 * k_kept, v_kept    out, [L][N][Hkv][D] contiguous, 16-byte aligned.
 * Enqueued on `stream`; meant for a second stream that waits for
 * tg_topk_select and runs beside tg_bias_attn_fwd.
 * ------------------------------------------------------------------------ */
tg_status tg_kv_gather(tg_dtype dt, int64_t L, int64_t T, int64_t N, int64_t Hkv,
                       int64_t D, const void* k_cache, const void* v_cache,
                       const int32_t* kept_idx, void* k_kept, void* v_kept,
                       void* stream);

/* --------------------------------------------------------------------------
 * The four calls captured once as a HIP graph and replayed.  Pages: ai.info
 * summary "Key Contributions" item 4 (the serving recipe captures the pruned
 * forward pass as a graph per padded length, so the short kernels of a small
 * budget are not paced by launches).  The four calls above enqueue only
 * kernels and never synchronise, so they are capturable as they stand.
 *
 * tg_chain_desc holds the arguments of the four calls, field for field as
 * documented above (w1_packed selects tg_gate_score_packed; attn_key_score
 * is the attention's key_score, normally score_kept; attn_workspace, if not
 * NULL, selects tg_bias_attn_fwd_ws; the kv_ fields, if kv_L > 0, add
 * tg_kv_gather with the desc's T, N, Hkv, D and kept_idx), with these
 * differences that make one graph serve a bucket of prompts:
 *   - N is a capacity.  The gather, the KV gather and the attention read the
 *     kept count from n_kept (device memory the select writes) at every
 *     replay: kept rows r >= n_kept are padding (zero residual and KV rows,
 *     pos_kept -1, score_kept 0, attention output 0 and lse -inf), and keys
 *     at or past n_kept are masked.  A kept count above N keeps its first N
 *     rows (n_kept still holds the full count, so the caller can see it).
 *   - prompt_len: NULL (T is the prompt's length), or a device int32 read at
 *     every replay, 0 <= *prompt_len <= T: the gate and the select then take
 *     only tokens [0, *prompt_len) of the T-token buffers (later tokens are
 *     neither scored, kept nor counted).  T, and the buffers, are then the
 *     bucket's capacity: a graph captured at (T, N) serves every prompt up
 *     to T tokens whose kept count is at most N, with its inputs refilled in
 *     place and *prompt_len set before the replay.
 * tg_chain_create validates the arguments through the calls themselves (a
 * failing call's status and tg_last_error() come back unchanged and nothing
 * is captured), captures the chain on an internal stream and instantiates
 * it.  The graph keeps the pointers: the caller keeps every buffer alive and
 * refills inputs in place.  tg_chain_launch enqueues one replay on
 * `stream`; replays on one stream are ordered and may not overlap a replay
 * of the same chain on another stream (they share the workspace and
 * outputs).  tg_chain_destroy frees the graph (NULL is a no-op).  Creating a
 * chain allocates the runtime's graph objects (host memory and whatever the
 * runtime keeps per graph); replays allocate nothing.
 * ------------------------------------------------------------------------ */
typedef struct tg_chain tg_chain;

typedef struct tg_chain_desc {
  /* tg_gate_score / tg_gate_score_packed */
  tg_dtype dt;
  int64_t T, d, h;
  const void* resid;
  int64_t resid_row_stride;
  const uint8_t* prunable;
  const float* rms_weight;
  float eps;
  const void* w1;
  int w1_packed;
  const float* b1;
  const float* w2;
  float b2;
  float* scores;
  /* tg_topk_select */
  int64_t K;
  int32_t* kept_idx;
  int64_t kept_capacity;
  int32_t* n_kept;
  void* workspace;
  size_t workspace_bytes;
  /* tg_compact_gather */
  int64_t N;
  void* resid_kept;
  int64_t kept_row_stride;
  int32_t* pos_kept;
  float* score_kept;
  /* tg_bias_attn_fwd */
  int64_t Hq, Hkv, D;
  const void* q;
  const void* k;
  const void* v;
  const float* attn_key_score;
  const float* gain;
  const float* q_scale;
  float softmax_scale;
  int causal;
  void* out;
  float* lse;
  /* optional tg_kv_gather of kv_L lower layers (0: none), captured on a
   * second stream that forks after tg_compact_gather and joins after
   * tg_bias_attn_fwd, so the two run side by side in every replay */
  int64_t kv_L;
  const void* kv_k_cache;
  const void* kv_v_cache;
  void* kv_k_kept;
  void* kv_v_kept;
  /* optional workspace of tg_bias_attn_fwd_ws (NULL: unsplit attention) */
  void* attn_workspace;
  size_t attn_workspace_bytes;
  /* optional run-time prompt length: NULL, or a device int32 (see above) */
  const int32_t* prompt_len;
} tg_chain_desc;

tg_status tg_chain_create(const tg_chain_desc* desc, tg_chain** chain);

tg_status tg_chain_launch(const tg_chain* chain, void* stream);

void tg_chain_destroy(tg_chain* chain);

#ifdef __cplusplus
}
#endif
#endif /* TOKENGATE_H */
