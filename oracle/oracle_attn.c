/*
 * oracle_attn.c -- the fp64 CPU oracle for exact causal grouped-query attention.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The HIP product path never links,
 * imports or calls it, and it includes no header of the product path.
 *
 * What it computes is the plain definition of the attention forward that the
 * memory-efficient kernel reproduces exactly up to rounding: the result SDPA's
 * math path gives by materialising the score matrix and a row softmax
 * (kev pull request 202, sections "Why fp32 fell to the L x L kernel" and
 * "The change"). Grouped-query attention: 16 query heads share 4 key/value
 * heads (same section; system1-omni issue 27, "The closest planned or
 * implemented model"), read here as query head h using key/value head
 * h / (Hq/Hkv), the map that repeating K/V per query head produces.
 * Segment ids follow the splash-attention pull request (maxtext 4929, the
 * problem statement and the review): key j is visible to query i only when
 * their ids are equal; constant ids give the non-segmented result.
 * Causality is by position with an offset for queries that start later, the
 * branch "positions restarting at the state length" (system1-omni issue 27,
 * "Three differences from Cua-S1 that matter", item 3).
 *
 * Everything is fp64. Inputs arrive as fp32 (bf16 inputs are widened to fp32
 * by the caller, which is exact), and fp32 -> fp64 is exact. The scale is
 * 1/sqrt(D). No fast-math: the build uses -O2 and no reassociation.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Key/value head read by query head h: contiguous groups of Hq/Hkv heads. */
static int64_t kv_head_of(int64_t h, int64_t Hq, int64_t Hkv) { return h / (Hq / Hkv); }

/* The score scale 1/sqrt(D). */
static double score_scale(int64_t D) { return 1.0 / sqrt((double)D); }

/* Key j visible to query row i of batch b? Causal part: j <= q_offset + i.
 * Segment part: seg_q[b,i] == seg_k[b,j] when ids are given. */
static int visible(int64_t b, int64_t i, int64_t j, int64_t Lq, int64_t Lk, int64_t q_offset,
                   const int32_t* seg_q, const int32_t* seg_k, int causal) {
  if (causal && j > q_offset + i) return 0;
  if (seg_q && seg_q[b * Lq + i] != seg_k[b * Lk + j]) return 0;
  return 1;
}

/* One output row (b, h, i): scores s_j = (1/sqrt(D)) q.k_j for visible j,
 * M = max s_j, l = sum exp(s_j - M), lse = M + log l (natural log),
 * o = sum exp(s_j - M) v_j / l. An empty row gives o = 0, lse = -inf.
 * `s` is caller scratch of Lk doubles. If `w` is non-null it receives the
 * softmax weights of every key (0 for invisible keys). */
static void one_row(const float* q, const float* k, const float* v,
                    int64_t b, int64_t h, int64_t i,
                    int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                    int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k, int causal,
                    double* s, double* o_row, double* lse_out, double* w) {
  const int64_t g = kv_head_of(h, Hq, Hkv);
  const double scale = score_scale(D);
  const float* qi = q + ((b * Hq + h) * Lq + i) * D;
  const float* kb = k + (b * Hkv + g) * Lk * D;
  const float* vb = v + (b * Hkv + g) * Lk * D;
  double M = -INFINITY;
  int64_t nvis = 0;
  for (int64_t j = 0; j < Lk; ++j) {
    if (!visible(b, i, j, Lq, Lk, q_offset, seg_q, seg_k, causal)) { s[j] = -INFINITY; continue; }
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += (double)qi[d] * (double)kb[j * D + d];
    s[j] = scale * dot;
    if (s[j] > M) M = s[j];
    ++nvis;
  }
  for (int64_t d = 0; d < D; ++d) o_row[d] = 0.0;
  if (nvis == 0) {
    *lse_out = -INFINITY;
    if (w) for (int64_t j = 0; j < Lk; ++j) w[j] = 0.0;
    return;
  }
  double l = 0.0;
  for (int64_t j = 0; j < Lk; ++j) {
    if (s[j] == -INFINITY) continue;
    const double p = exp(s[j] - M);
    s[j] = p;
    l += p;
    for (int64_t d = 0; d < D; ++d) o_row[d] += p * (double)vb[j * D + d];
  }
  for (int64_t d = 0; d < D; ++d) o_row[d] /= l;
  *lse_out = M + log(l);
  if (w) for (int64_t j = 0; j < Lk; ++j) w[j] = (s[j] == -INFINITY) ? 0.0 : s[j] / l;
}

/* Attention forward for a subset of query rows.
 *   q [B,Hq,Lq,D], k,v [B,Hkv,Lk,D] fp32 row-major; seg_q [B,Lq], seg_k [B,Lk] int32 or both NULL.
 *   rows: nrows query indices in [0,Lq), or NULL for all rows (nrows must equal Lq).
 *   o [B,Hq,nrows,D] fp64, lse [B,Hq,nrows] fp64.
 *   nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 for an invalid argument. */
int oracle_attn(const float* q, const float* k, const float* v,
                int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k, int causal,
                const int64_t* rows, int64_t nrows, double* o, double* lse, int nthreads) {
  if (!q || !k || !v || !o || !lse) return -1;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || Lk <= 0 || D <= 0 || Hq % Hkv) return -1;
  if ((seg_q == NULL) != (seg_k == NULL) || q_offset < 0 || nrows <= 0) return -1;
  if (!rows && nrows != Lq) return -1;
  if (rows) for (int64_t r = 0; r < nrows; ++r) if (rows[r] < 0 || rows[r] >= Lq) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  const int64_t total = B * Hq * nrows;
  int err = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc((size_t)Lk * sizeof(double));
    if (!s) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t t = 0; t < total; ++t) {
      if (!s) continue;
      const int64_t r = t % nrows, h = (t / nrows) % Hq, b = t / (nrows * Hq);
      const int64_t i = rows ? rows[r] : r;
      one_row(q, k, v, b, h, i, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal,
              s, o + t * D, lse + t, NULL);
    }
    free(s);
  }
  return err ? -1 : 0;
}

/* Softmax weights of one row (b, h, i) over all Lk keys, for the
 * normalisation check; w has Lk entries. Returns 0 or -1. */
int oracle_attn_weights(const float* q, const float* k, const float* v,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                        int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k, int causal,
                        int64_t b, int64_t h, int64_t i, double* w) {
  if (!q || !k || !v || !w || b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Lq) return -1;
  if (Hq % Hkv || (seg_q == NULL) != (seg_k == NULL)) return -1;
  double* s = (double*)malloc((size_t)Lk * sizeof(double));
  double* orow = (double*)malloc((size_t)D * sizeof(double));
  double lse;
  if (!s || !orow) { free(s); free(orow); return -1; }
  one_row(q, k, v, b, h, i, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal, s, orow, &lse, w);
  free(s);
  free(orow);
  return 0;
}

/* Combine two attention results over disjoint key sets A1 and A2 of the same
 * query rows into the result over A1 u A2, from their log-sum-exps:
 *   M = max(l1, l2), w_x = exp(l_x - M), o = (w1 o1 + w2 o2) / (w1 + w2),
 *   lse = M + log(w1 + w2); both empty gives o = 0, lse = -inf.
 * This is how the shared-prefix branch (system1-omni issue 27, "Three
 * differences from Cua-S1 that matter", item 3) splits into a prefix part and
 * a suffix part. rows x D values, fp64. */
void oracle_merge(const double* o1, const double* lse1, const double* o2, const double* lse2,
                  int64_t rows, int64_t D, double* o, double* lse) {
  for (int64_t r = 0; r < rows; ++r) {
    const double l1 = lse1[r], l2 = lse2[r];
    const double M = l1 > l2 ? l1 : l2;
    if (M == -INFINITY) {
      for (int64_t d = 0; d < D; ++d) o[r * D + d] = 0.0;
      lse[r] = -INFINITY;
      continue;
    }
    const double w1 = exp(l1 - M), w2 = exp(l2 - M);
    for (int64_t d = 0; d < D; ++d) o[r * D + d] = (w1 * o1[r * D + d] + w2 * o2[r * D + d]) / (w1 + w2);
    lse[r] = M + log(w1 + w2);
  }
}

/* ---- Backward: gradients of a scalar loss whose gradient with respect to o
 * is dout ---------------------------------------------------------------------
 *
 * The pages train at these lengths (kev pull request 202, the title of the
 * change: states of 64k tokens are trained and served; system1-omni issue 27,
 * the model trains end to end), so the backward is the gradient of the same
 * forward, by the chain rule through its definition. With the scores
 * s_ij = (1/sqrt(D)) q_i.k_j over the visible keys A_i, the weights
 * p_ij = exp(s_ij - lse_i) and o_i = sum_j p_ij v_j:
 *   dp_ij = dout_i . v_j
 *   ds_ij = p_ij (dp_ij - sum_{k in A_i} p_ik dp_ik)      (softmax Jacobian)
 *   dq_i  = (1/sqrt(D)) sum_{j in A_i} ds_ij k_j
 *   dk_j  = (1/sqrt(D)) sum_{(h,i): j in A_i} ds_ij q_i
 *   dv_j  = sum_{(h,i): j in A_i} p_ij dout_i
 * where the key/value sums run over every query head h that shares the key's
 * head (the heads that repeating K/V would have copied it to). Rows with no
 * visible key contribute nothing and get dq = 0. */

/* Statistics of one row (b, h, i): lse_i (natural log; -inf when empty) and
 * r_i = sum_j p_ij dp_ij. `s` is scratch of Lk doubles, `w` receives p_ij. */
static void bwd_row_stats(const float* q, const float* k, const float* v, const float* dout,
                          int64_t b, int64_t h, int64_t i,
                          int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                          int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k, int causal,
                          double* s, double* orow, double* w, double* lse_out, double* r_out) {
  one_row(q, k, v, b, h, i, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal, s, orow, lse_out, w);
  const int64_t g = kv_head_of(h, Hq, Hkv);
  const float* di = dout + ((b * Hq + h) * Lq + i) * D;
  const float* vb = v + (b * Hkv + g) * Lk * D;
  double r = 0.0;
  for (int64_t j = 0; j < Lk; ++j) {
    if (w[j] == 0.0) continue;
    double dp = 0.0;
    for (int64_t d = 0; d < D; ++d) dp += (double)di[d] * (double)vb[j * D + d];
    r += w[j] * dp;
  }
  *r_out = r;
}

/* dq for a subset of query rows (rows == NULL: all, nrows == Lq).
 * dq [B,Hq,nrows,D] fp64. Returns 0 or -1. */
int oracle_attn_bwd_dq(const float* q, const float* k, const float* v, const float* dout,
                       int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                       int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k, int causal,
                       const int64_t* rows, int64_t nrows, double* dq, int nthreads) {
  if (!q || !k || !v || !dout || !dq) return -1;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || Lk <= 0 || D <= 0 || Hq % Hkv) return -1;
  if ((seg_q == NULL) != (seg_k == NULL) || q_offset < 0 || nrows <= 0) return -1;
  if (!rows && nrows != Lq) return -1;
  if (rows) for (int64_t r = 0; r < nrows; ++r) if (rows[r] < 0 || rows[r] >= Lq) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  const double scale = score_scale(D);
  const int64_t total = B * Hq * nrows;
  int err = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc((size_t)Lk * sizeof(double));
    double* w = (double*)malloc((size_t)Lk * sizeof(double));
    double* orow = (double*)malloc((size_t)D * sizeof(double));
    if (!s || !w || !orow) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t t = 0; t < total; ++t) {
      if (!s || !w || !orow) continue;
      const int64_t r = t % nrows, h = (t / nrows) % Hq, b = t / (nrows * Hq);
      const int64_t i = rows ? rows[r] : r;
      double lse, rsum;
      bwd_row_stats(q, k, v, dout, b, h, i, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal,
                    s, orow, w, &lse, &rsum);
      const int64_t g = kv_head_of(h, Hq, Hkv);
      const float* di = dout + ((b * Hq + h) * Lq + i) * D;
      const float* kb = k + (b * Hkv + g) * Lk * D;
      const float* vb = v + (b * Hkv + g) * Lk * D;
      double* out = dq + t * D;
      for (int64_t d = 0; d < D; ++d) out[d] = 0.0;
      for (int64_t j = 0; j < Lk; ++j) {
        if (w[j] == 0.0) continue;
        double dp = 0.0;
        for (int64_t d = 0; d < D; ++d) dp += (double)di[d] * (double)vb[j * D + d];
        const double ds = w[j] * (dp - rsum);
        for (int64_t d = 0; d < D; ++d) out[d] += scale * ds * (double)kb[j * D + d];
      }
    }
    free(s);
    free(w);
    free(orow);
  }
  return err ? -1 : 0;
}

/* dk and dv for a subset of keys (keys == NULL: all, nkeys == Lk).
 * dk, dv [B,Hkv,nkeys,D] fp64. The row statistics are computed only for the
 * rows that see at least one selected key. Returns 0 or -1. */
int oracle_attn_bwd_dkdv(const float* q, const float* k, const float* v, const float* dout,
                         int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                         int64_t q_offset, const int32_t* seg_q, const int32_t* seg_k, int causal,
                         const int64_t* keys, int64_t nkeys, double* dk, double* dv, int nthreads) {
  if (!q || !k || !v || !dout || !dk || !dv) return -1;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || Lk <= 0 || D <= 0 || Hq % Hkv) return -1;
  if ((seg_q == NULL) != (seg_k == NULL) || q_offset < 0 || nkeys <= 0) return -1;
  if (!keys && nkeys != Lk) return -1;
  if (keys) for (int64_t r = 0; r < nkeys; ++r) if (keys[r] < 0 || keys[r] >= Lk) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#endif
  const double scale = score_scale(D);
  /* rows (per batch) that see some selected key */
  char* need = (char*)calloc((size_t)(B * Lq), 1);
  double* lse = (double*)malloc((size_t)(B * Hq * Lq) * sizeof(double));
  double* rsum = (double*)malloc((size_t)(B * Hq * Lq) * sizeof(double));
  if (!need || !lse || !rsum) { free(need); free(lse); free(rsum); return -1; }
#pragma omp parallel for schedule(dynamic, 16)
  for (int64_t t = 0; t < B * Lq; ++t) {
    const int64_t b = t / Lq, i = t % Lq;
    for (int64_t r = 0; r < nkeys; ++r) {
      const int64_t j = keys ? keys[r] : r;
      if (visible(b, i, j, Lq, Lk, q_offset, seg_q, seg_k, causal)) { need[t] = 1; break; }
    }
  }
  int err = 0;
#pragma omp parallel
  {
    double* s = (double*)malloc((size_t)Lk * sizeof(double));
    double* w = (double*)malloc((size_t)Lk * sizeof(double));
    double* orow = (double*)malloc((size_t)D * sizeof(double));
    if (!s || !w || !orow) {
#pragma omp atomic write
      err = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t t = 0; t < B * Hq * Lq; ++t) {
      const int64_t i = t % Lq, h = (t / Lq) % Hq, b = t / (Lq * Hq);
      if (!s || !w || !orow || !need[b * Lq + i]) continue;
      bwd_row_stats(q, k, v, dout, b, h, i, Hq, Hkv, Lq, Lk, D, q_offset, seg_q, seg_k, causal,
                    s, orow, w, &lse[t], &rsum[t]);
    }
    free(s);
    free(w);
    free(orow);
  }
  if (err) { free(need); free(lse); free(rsum); return -1; }
  const int64_t n_rep = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < B * Hkv * nkeys; ++t) {
    const int64_t r = t % nkeys, g = (t / nkeys) % Hkv, b = t / (nkeys * Hkv);
    const int64_t j = keys ? keys[r] : r;
    const float* kj = k + ((b * Hkv + g) * Lk + j) * D;
    const float* vj = v + ((b * Hkv + g) * Lk + j) * D;
    double* dkj = dk + t * D;
    double* dvj = dv + t * D;
    for (int64_t d = 0; d < D; ++d) { dkj[d] = 0.0; dvj[d] = 0.0; }
    for (int64_t h = g * n_rep; h < (g + 1) * n_rep; ++h) {
      for (int64_t i = 0; i < Lq; ++i) {
        if (!visible(b, i, j, Lq, Lk, q_offset, seg_q, seg_k, causal)) continue;
        const int64_t row = (b * Hq + h) * Lq + i;
        const float* qi = q + row * D;
        const float* di = dout + row * D;
        double sd = 0.0, dp = 0.0;
        for (int64_t d = 0; d < D; ++d) {
          sd += (double)qi[d] * (double)kj[d];
          dp += (double)di[d] * (double)vj[d];
        }
        const double p = exp(scale * sd - lse[row]);
        const double ds = p * (dp - rsum[row]);
        for (int64_t d = 0; d < D; ++d) {
          dvj[d] += p * (double)di[d];
          dkj[d] += scale * ds * (double)qi[d];
        }
      }
    }
  }
  free(need);
  free(lse);
  free(rsum);
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
