/*
 * tg_oracle.c -- plain fp64 CPU oracle for the token-gated prefill path.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU baseline, never by the product path.  Shares no code with
 * the HIP library.  Each function is the plain definition of its step,
 * written out loop by loop; the comments in tg_oracle.h name the passage of
 * the TokenGate pages each one follows.
 *
 * Readings of points the pages leave open (kept in one place here so a
 * reader can check them against the pages):
 *   - non-prunable tokens are not scored: their score is 0;
 *   - the gate bias added to a logit is gain[head] * raw score (no squashing);
 *   - the per-query scale c_r multiplies the whole logit (dot-product term
 *     and bias alike), as a softmax temperature would;
 *   - one gain per query head; query head hq reads KV head hq / (Hq/Hkv);
 *   - the dot-product scale is 1/sqrt(D) unless the caller passes another;
 *   - ties in score go to the lower token index; NaN ranks lowest;
 *     -0 and +0 are equal; kept tokens stay in original order.
 */
#include "tg_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int tgo_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ---------------------------------------------------------------------- */
/* Gate: s_t = b2 + sum_j w2_j * SiLU(b1_j + sum_i W1[j,i] * u_i),          */
/*       u_i = gamma_i * x_i / sqrt(mean_i(x_i^2) + eps).                   */
/* ---------------------------------------------------------------------- */
void tgo_gate_score(int64_t T, int64_t d, int64_t h, const double* resid,
                    const uint8_t* prunable, const double* gamma, double eps,
                    const double* w1, const double* b1, const double* w2,
                    double b2, double* scores) {
#pragma omp parallel
  {
    double* u = (double*)malloc((size_t)(d > 0 ? d : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
      if (!prunable[t]) {
        scores[t] = 0.0;
        continue;
      }
      const double* x = resid + t * d;
      /* RMSNorm */
      double sumsq = 0.0;
      for (int64_t i = 0; i < d; ++i) sumsq += x[i] * x[i];
      const double rms = sqrt(sumsq / (double)d + eps);
      for (int64_t i = 0; i < d; ++i) {
        const double g = gamma ? gamma[i] : 1.0;
        u[i] = g * (x[i] / rms);
      }
      /* MLP: d -> h, SiLU, h -> 1 */
      double s = b2;
      for (int64_t j = 0; j < h; ++j) {
        double z = b1 ? b1[j] : 0.0;
        const double* wrow = w1 + j * d;
        for (int64_t i = 0; i < d; ++i) z += wrow[i] * u[i];
        const double silu = z / (1.0 + exp(-z));
        s += w2[j] * silu;
      }
      scores[t] = s;
    }
    free(u);
  }
}

/* ---------------------------------------------------------------------- */
/* Selection: sort the prunable tokens by (score descending, index          */
/* ascending), keep the first min(K, |P|), add every non-prunable token and */
/* list the kept set in ascending index order.                              */
/* ---------------------------------------------------------------------- */
typedef struct {
  float s;
  int64_t t;
} scored_token;

/* qsort comparator: a comes first if it has the higher score, or equal
 * score and lower index.  NaN is below every number (NaNs tie among
 * themselves); -0 == +0 by IEEE comparison. */
static int rank_order(const void* pa, const void* pb) {
  const scored_token* a = (const scored_token*)pa;
  const scored_token* b = (const scored_token*)pb;
  const int an = isnan(a->s), bn = isnan(b->s);
  if (an != bn) return an ? 1 : -1;
  if (!an) {
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
  }
  return (a->t < b->t) ? -1 : (a->t > b->t) ? 1 : 0;
}

int64_t tgo_topk_select(int64_t T, const float* scores,
                        const uint8_t* prunable, int64_t K, int32_t* kept_idx) {
  if (K < 0 || T < 0) return -1;
  int64_t nP = 0;
  for (int64_t t = 0; t < T; ++t) nP += prunable[t] ? 1 : 0;
  scored_token* cand =
      (scored_token*)malloc((size_t)(nP > 0 ? nP : 1) * sizeof(scored_token));
  int64_t c = 0;
  for (int64_t t = 0; t < T; ++t)
    if (prunable[t]) {
      cand[c].s = scores[t];
      cand[c].t = t;
      ++c;
    }
  qsort(cand, (size_t)nP, sizeof(scored_token), rank_order);
  const int64_t keepP = K < nP ? K : nP;
  uint8_t* keep = (uint8_t*)calloc((size_t)(T > 0 ? T : 1), 1);
  for (int64_t i = 0; i < keepP; ++i) keep[cand[i].t] = 1;
  for (int64_t t = 0; t < T; ++t)
    if (!prunable[t]) keep[t] = 1;
  int64_t n = 0;
  for (int64_t t = 0; t < T; ++t)
    if (keep[t]) kept_idx[n++] = (int32_t)t;
  free(keep);
  free(cand);
  return n;
}

/* ---------------------------------------------------------------------- */
/* Gather into kept order.                                                  */
/* ---------------------------------------------------------------------- */
void tgo_compact_gather(int64_t N, int64_t row_bytes, const uint8_t* resid,
                        int64_t resid_row_bytes, const float* scores,
                        const int32_t* kept_idx, uint8_t* resid_kept,
                        int32_t* pos_kept, float* score_kept) {
  for (int64_t r = 0; r < N; ++r) {
    const int64_t t = kept_idx[r];
    memcpy(resid_kept + r * row_bytes, resid + t * resid_row_bytes,
           (size_t)row_bytes);
    if (pos_kept) pos_kept[r] = (int32_t)t;
    if (score_kept) score_kept[r] = scores[t];
  }
}

/* ---------------------------------------------------------------------- */
/* Lower layers' KV cache gathered to the kept tokens: for every layer l and */
/* kept rank r, row (l, r) of the output is row (l, kept_idx[r]) of the     */
/* cache, byte for byte.                                                    */
/* ---------------------------------------------------------------------- */
void tgo_kv_gather(int64_t L, int64_t T, int64_t N, int64_t row_bytes,
                   const uint8_t* cache, const int32_t* kept_idx, uint8_t* out) {
  for (int64_t l = 0; l < L; ++l)
    for (int64_t r = 0; r < N; ++r)
      memcpy(out + (l * N + r) * row_bytes,
             cache + (l * T + (int64_t)kept_idx[r]) * row_bytes, (size_t)row_bytes);
}

/* ---------------------------------------------------------------------- */
/* Token-gated attention, one (query row, query head) at a time.            */
/* ---------------------------------------------------------------------- */
void tgo_bias_attn(int64_t N, int64_t Hq, int64_t Hkv, int64_t D,
                   const double* q, const double* k, const double* v,
                   const double* key_score, const double* gain,
                   const double* q_scale, double scale, int causal,
                   const int64_t* rows, int64_t n_rows, double* out,
                   double* lse) {
  if (rows == NULL) n_rows = N;
  const int64_t G = Hq / Hkv;
#pragma omp parallel
  {
    double* z = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 1) collapse(2)
    for (int64_t i = 0; i < n_rows; ++i) {
      for (int64_t hq = 0; hq < Hq; ++hq) {
        const int64_t r = rows ? rows[i] : i;
        const int64_t kv = hq / G;
        const double cr = q_scale ? q_scale[r] : 1.0;
        const double* qr = q + (r * Hq + hq) * D;
        const int64_t nkeys = causal ? r + 1 : N;
        /* logits */
        double m = -INFINITY;
        for (int64_t c = 0; c < nkeys; ++c) {
          const double* kc = k + (c * Hkv + kv) * D;
          double dot = 0.0;
          for (int64_t e = 0; e < D; ++e) dot += qr[e] * kc[e];
          z[c] = cr * (scale * dot + gain[hq] * key_score[c]);
          if (z[c] > m) m = z[c];
        }
        double* o = out + (i * Hq + hq) * D;
        for (int64_t e = 0; e < D; ++e) o[e] = 0.0;
        if (m == -INFINITY) { /* every key masked out */
          if (lse) lse[hq * n_rows + i] = -INFINITY;
          continue;
        }
        /* softmax-weighted sum of values */
        double denom = 0.0;
        for (int64_t c = 0; c < nkeys; ++c) {
          const double w = exp(z[c] - m);
          denom += w;
          const double* vc = v + (c * Hkv + kv) * D;
          for (int64_t e = 0; e < D; ++e) o[e] += w * vc[e];
        }
        for (int64_t e = 0; e < D; ++e) o[e] /= denom;
        if (lse) lse[hq * n_rows + i] = m + log(denom);
      }
    }
    free(z);
  }
}

/* ---------------------------------------------------------------------- */
/* Token-gated attention backward: the gradients of sum(O * dO) with      */
/* respect to Q, K, V, the key scores and the per-head gains.             */
/*   P = softmax_c(z), z[c] = c_r (alpha <q_r, k_c> + g_h s_c)            */
/*   dP[c] = <dO_r, v_c>,  Delta = sum_c P[c] dP[c]                       */
/*   dZ[c] = P[c] (dP[c] - Delta)                                         */
/*   dq_r += dZ c_r alpha k_c,  dk_c += dZ c_r alpha q_r,  dv_c += P dO_r */
/*   dscore_c += dZ c_r g_h,    dgain_h += dZ c_r s_c                     */
/* A key with P = 0 (masked or outside the causal range) contributes      */
/* nothing, also to dgain where its score may be -inf.                    */
/* ---------------------------------------------------------------------- */
void tgo_bias_attn_bwd(int64_t N, int64_t Hq, int64_t Hkv, int64_t D,
                       const double* q, const double* k, const double* v,
                       const double* key_score, const double* gain,
                       const double* q_scale, double scale, int causal,
                       const double* dout, double* dq, double* dk, double* dv,
                       double* dscore, double* dgain) {
  const int64_t G = Hq / Hkv;
  memset(dq, 0, (size_t)(N * Hq * D) * sizeof(double));
  memset(dk, 0, (size_t)(N * Hkv * D) * sizeof(double));
  memset(dv, 0, (size_t)(N * Hkv * D) * sizeof(double));
  memset(dgain, 0, (size_t)Hq * sizeof(double));
  /* per KV head: its keys' dk/dv are written by that head's query heads only */
  double* ds_part = (double*)calloc((size_t)(Hkv * (N > 0 ? N : 1)), sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t kvh = 0; kvh < Hkv; ++kvh) {
    double* P = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    double* dZ = (double*)malloc((size_t)(N > 0 ? N : 1) * sizeof(double));
    for (int64_t hq = kvh * G; hq < (kvh + 1) * G; ++hq) {
      double dg = 0.0;
      for (int64_t r = 0; r < N; ++r) {
        const double c_r = q_scale ? q_scale[r] : 1.0;
        const double* q_r = q + (r * Hq + hq) * D;
        const double* do_r = dout + (r * Hq + hq) * D;
        const int64_t n_vis = causal ? (r + 1) : N;
        double zmax = -INFINITY;
        for (int64_t c = 0; c < n_vis; ++c) {
          const double* k_c = k + (c * Hkv + kvh) * D;
          double qk = 0.0;
          for (int64_t e = 0; e < D; ++e) qk += q_r[e] * k_c[e];
          P[c] = c_r * (scale * qk + key_score[c] * gain[hq]);
          if (P[c] > zmax) zmax = P[c];
        }
        if (zmax == -INFINITY) continue; /* no visible key: no gradient */
        double sum = 0.0;
        for (int64_t c = 0; c < n_vis; ++c) {
          P[c] = exp(P[c] - zmax);
          sum += P[c];
        }
        double delta = 0.0;
        for (int64_t c = 0; c < n_vis; ++c) {
          P[c] /= sum;
          const double* v_c = v + (c * Hkv + kvh) * D;
          double dp = 0.0;
          for (int64_t e = 0; e < D; ++e) dp += do_r[e] * v_c[e];
          dZ[c] = dp;
          delta += P[c] * dp;
        }
        double* dq_r = dq + (r * Hq + hq) * D;
        for (int64_t c = 0; c < n_vis; ++c) {
          if (P[c] == 0.0) continue;
          const double dz = P[c] * (dZ[c] - delta);
          const double* k_c = k + (c * Hkv + kvh) * D;
          double* dk_c = dk + (c * Hkv + kvh) * D;
          double* dv_c = dv + (c * Hkv + kvh) * D;
          for (int64_t e = 0; e < D; ++e) {
            dq_r[e] += dz * c_r * scale * k_c[e];
            dk_c[e] += dz * c_r * scale * q_r[e];
            dv_c[e] += P[c] * do_r[e];
          }
          ds_part[kvh * N + c] += dz * c_r * gain[hq];
          dg += dz * c_r * key_score[c];
        }
      }
      dgain[hq] = dg;
    }
    free(P);
    free(dZ);
  }
  for (int64_t c = 0; c < N; ++c) {
    double acc = 0.0;
    for (int64_t kvh = 0; kvh < Hkv; ++kvh) acc += ds_part[kvh * N + c];
    dscore[c] = acc;
  }
  free(ds_part);
}
