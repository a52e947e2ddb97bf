/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the fused
 * attention forward pass.  TEST INFRASTRUCTURE ONLY: it is loaded by the
 * tests, by the smoke check and by the benchmark's CPU-baseline leg, never by
 * the product path.  It shares no code, header, table or helper with the HIP
 * library; both sides see only the same seeded input tensors.
 *
 * Arithmetic is fp64 throughout.  Inputs arrive already widened to double
 * (a bf16 or fp16 value widens to double exactly), outputs are double.
 *
 * What is computed (the plain definition the tiled online-softmax method
 * reaches up to rounding order):
 *
 *   JAX Pallas Mosaic-GPU "FlashAttention3" page, function
 *   `attention_reference`: upcast, logits = q.k per (query, key) with the
 *   q-heads of one kv-head taken as a contiguous group (q reshaped to
 *   (B, Sq, Hkv, Hq/Hkv, D)), mask, row max m, unnormalized = exp(logits - m),
 *   l = row sum, weights = unnormalized / l, out = weights . v, and the
 *   residual lse = m + log(l) (that page writes it in base 2; here it is the
 *   natural log, see the header of oracle/__init__.py for the reading).
 *
 *   The logits are multiplied by `scale` (the Croqtile `flash_atten` page
 *   folds 1/sqrt(128) into its exponent; the JAX reference applies none,
 *   i.e. scale = 1).  The causal mask is aligned bottom-right: key j is
 *   visible from query i iff j <= i + (Skv - Sq).  For Sq == Skv this is the
 *   JAX reference's `arange(Sq)[:, None] >= arange(Skv)[None, :]`.  A row
 *   with no visible key gets O = 0 and LSE = -inf (the log of an empty sum;
 *   the same (-inf, 0, 0) identity the kernbench merge is seeded with).
 *
 * Two passes per row, as the definition reads: pass 1 computes every visible
 * logit and the max, pass 2 the exponentials, their sum and the weighted sum
 * of V rows, then one division.
 *
 * Parallelism: rows are independent; an OpenMP loop over rows changes no
 * arithmetic (each row is computed start to finish by one thread, in key
 * order).
 *
 * Layouts (all contiguous, row-major):
 *   q, o : [B, Sq, Hq, D]      k, v : [B, Skv, Hkv, D]      lse : [B, Hq, Sq]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of threads the OpenMP loops use; 0 means the OpenMP default. */
static int g_threads = 0;

void oracle_set_threads(int n) { g_threads = n; }

int oracle_threads(void) {
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

/* Largest visible key index + 1 for query row i (0 if none is visible). */
static int64_t visible_end(int64_t i, int64_t Sq, int64_t Skv, int causal) {
  if (!causal) return Skv;
  int64_t last = i + (Skv - Sq); /* bottom-right alignment */
  if (last < 0) return 0;
  if (last >= Skv) return Skv;
  return last + 1;
}

/*
 * One output row (b, hq, i).  `s` is caller-provided scratch of Skv doubles.
 * Visible keys are the range [j_lo, j_hi) intersected with the causal set;
 * the full definition uses j_lo = 0, j_hi = Skv.
 *
 * Writes m (the max logit, -inf if no key is visible), l (sum of
 * exp(logit - m), 0 if none) and acc[D] (sum of exp(logit - m) * V_j,
 * unnormalized).
 */
static void row_partial(const double* q, const double* k, const double* v,
                        int64_t b, int64_t hq, int64_t i, int64_t Sq,
                        int64_t Skv, int64_t Hq, int64_t Hkv, int64_t D,
                        int causal, double scale, int64_t j_lo, int64_t j_hi,
                        double* s, double* m_out, double* l_out, double* acc) {
  const int64_t group = Hq / Hkv;  /* q-heads per kv-head */
  const int64_t hk = hq / group;   /* contiguous grouping */
  int64_t end = visible_end(i, Sq, Skv, causal);
  if (j_hi > end) j_hi = end;
  if (j_lo < 0) j_lo = 0;

  const double* qrow = q + ((b * Sq + i) * Hq + hq) * D;

  /* pass 1: logits and their max */
  double m = -INFINITY;
  for (int64_t j = j_lo; j < j_hi; ++j) {
    const double* krow = k + ((b * Skv + j) * Hkv + hk) * D;
    double dot = 0.0;
    for (int64_t d = 0; d < D; ++d) dot += qrow[d] * krow[d];
    s[j] = scale * dot;
    if (s[j] > m) m = s[j];
  }

  /* pass 2: exponentials, their sum and the weighted sum of V rows */
  double l = 0.0;
  for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
  for (int64_t j = j_lo; j < j_hi; ++j) {
    double p = exp(s[j] - m);
    l += p;
    const double* vrow = v + ((b * Skv + j) * Hkv + hk) * D;
    for (int64_t d = 0; d < D; ++d) acc[d] += p * vrow[d];
  }
  *m_out = m;
  *l_out = l;
}

static int check_shape(int64_t B, int64_t Sq, int64_t Skv, int64_t Hq,
                       int64_t Hkv, int64_t D) {
  if (B < 1 || Sq < 1 || Skv < 1 || Hq < 1 || Hkv < 1 || D < 1) return -1;
  if (Hq % Hkv != 0) return -1;
  return 0;
}

/*
 * Full forward: every (b, hq, i) row.  lse may be NULL.
 * Returns 0, or -1 on a bad shape, -2 if scratch cannot be allocated.
 */
int oracle_attn_fwd(const double* q, const double* k, const double* v,
                    double* o, double* lse, int64_t B, int64_t Sq, int64_t Skv,
                    int64_t Hq, int64_t Hkv, int64_t D, int causal,
                    double scale) {
  if (check_shape(B, Sq, Skv, Hq, Hkv, D)) return -1;
  const int64_t rows = B * Hq * Sq;
  int failed = 0;
#pragma omp parallel num_threads(oracle_threads())
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Skv);
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!s || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / (Hq * Sq);
        int64_t hq = (r / Sq) % Hq;
        int64_t i = r % Sq;
        double m, l;
        row_partial(q, k, v, b, hq, i, Sq, Skv, Hq, Hkv, D, causal, scale, 0,
                    Skv, s, &m, &l, acc);
        double* orow = o + ((b * Sq + i) * Hq + hq) * D;
        if (l > 0.0) {
          for (int64_t d = 0; d < D; ++d) orow[d] = acc[d] / l;
          if (lse) lse[(b * Hq + hq) * Sq + i] = m + log(l);
        } else {
          for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
          if (lse) lse[(b * Hq + hq) * Sq + i] = -INFINITY;
        }
      }
    }
    free(s);
    free(acc);
  }
  return failed ? -2 : 0;
}

/*
 * Selected rows only, for checks at sizes where the full forward is too slow.
 * rows_bhi holds n triples (b, hq, i).  o_rows is [n, D], lse_rows is [n].
 */
int oracle_attn_rows(const double* q, const double* k, const double* v,
                     int64_t B, int64_t Sq, int64_t Skv, int64_t Hq,
                     int64_t Hkv, int64_t D, int causal, double scale,
                     const int64_t* rows_bhi, int64_t n, double* o_rows,
                     double* lse_rows) {
  if (check_shape(B, Sq, Skv, Hq, Hkv, D)) return -1;
  for (int64_t r = 0; r < n; ++r) {
    int64_t b = rows_bhi[3 * r], hq = rows_bhi[3 * r + 1],
            i = rows_bhi[3 * r + 2];
    if (b < 0 || b >= B || hq < 0 || hq >= Hq || i < 0 || i >= Sq) return -1;
  }
  int failed = 0;
#pragma omp parallel num_threads(oracle_threads())
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Skv);
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!s || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < n; ++r) {
        int64_t b = rows_bhi[3 * r], hq = rows_bhi[3 * r + 1],
                i = rows_bhi[3 * r + 2];
        double m, l;
        row_partial(q, k, v, b, hq, i, Sq, Skv, Hq, Hkv, D, causal, scale, 0,
                    Skv, s, &m, &l, acc);
        double* orow = o_rows + r * D;
        if (l > 0.0) {
          for (int64_t d = 0; d < D; ++d) orow[d] = acc[d] / l;
          lse_rows[r] = m + log(l);
        } else {
          for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;
          lse_rows[r] = -INFINITY;
        }
      }
    }
    free(s);
    free(acc);
  }
  return failed ? -2 : 0;
}

/*
 * Unnormalized partial state of every row over the keys [j_lo, j_hi) (still
 * subject to the causal mask): m [B,Hq,Sq], l [B,Hq,Sq], acc [B,Sq,Hq,D].
 * This is the (m, l, O) triple of one tile of the kernbench tile sweep, whose
 * O is left unnormalized until the root divides by l.
 */
int oracle_attn_partial(const double* q, const double* k, const double* v,
                        int64_t B, int64_t Sq, int64_t Skv, int64_t Hq,
                        int64_t Hkv, int64_t D, int causal, double scale,
                        int64_t j_lo, int64_t j_hi, double* m_out,
                        double* l_out, double* acc_out) {
  if (check_shape(B, Sq, Skv, Hq, Hkv, D)) return -1;
  const int64_t rows = B * Hq * Sq;
  int failed = 0;
#pragma omp parallel num_threads(oracle_threads())
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Skv);
    if (!s) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / (Hq * Sq);
        int64_t hq = (r / Sq) % Hq;
        int64_t i = r % Sq;
        double* acc = acc_out + ((b * Sq + i) * Hq + hq) * D;
        row_partial(q, k, v, b, hq, i, Sq, Skv, Hq, Hkv, D, causal, scale,
                    j_lo, j_hi, s, &m_out[r], &l_out[r], acc);
      }
    }
    free(s);
  }
  return failed ? -2 : 0;
}

/*
 * Online-softmax merge of two partial triples, following the kernbench
 * prefill page, `_merge_running`: the new max is the larger of the two, each
 * side is weighted by exp(its max - new max), the sums and the unnormalized
 * outputs are added with those weights.  One guard is added: when both maxima
 * are -inf (neither side saw a visible key) the result is the identity
 * (-inf, 0, 0) instead of exp(-inf - -inf) = NaN.
 *
 * n rows; acc arrays are [n, D].  Output arrays may alias the first input.
 */
void oracle_merge(int64_t n, int64_t D, const double* m1, const double* l1,
                  const double* acc1, const double* m2, const double* l2,
                  const double* acc2, double* m_out, double* l_out,
                  double* acc_out) {
  for (int64_t r = 0; r < n; ++r) {
    double m = m1[r] > m2[r] ? m1[r] : m2[r];
    if (m == -INFINITY) {
      m_out[r] = -INFINITY;
      l_out[r] = 0.0;
      for (int64_t d = 0; d < D; ++d) acc_out[r * D + d] = 0.0;
      continue;
    }
    double a = exp(m1[r] - m);
    double c = exp(m2[r] - m);
    l_out[r] = l1[r] * a + l2[r] * c;
    for (int64_t d = 0; d < D; ++d)
      acc_out[r * D + d] = acc1[r * D + d] * a + acc2[r * D + d] * c;
    m_out[r] = m;
  }
}

/*
 * Backward pass: the gradients of a scalar loss L with respect to q, k and v,
 * given dout = dL/dO, for the same forward definition as oracle_attn_fwd.
 *
 * The textbook softmax gradient, following the backward of the JAX Pallas
 * FlashAttention3 page (`_attention_bwd`: delta = rowsum(O * dO); dP = dO.V^T;
 * dS = P * (dP - delta); dQ = dS.K; dK = dS^T.Q; dV = P^T.dO, the dK and dV of
 * a kv-head summed over the q-heads of its group) with the scale applied to
 * the logits, so that dQ and dK carry one factor of scale:
 *
 *   P[i,j]  = exp(s[i,j] - LSE[i])        over the visible keys j of row i
 *   delta_i = sum_j P[i,j] * (dO_i . V_j)      (= dO_i . O_i)
 *   dS[i,j] = P[i,j] * (dO_i . V_j - delta_i)
 *   dQ_i    = scale * sum_j dS[i,j] * K_j
 *   dK_j    = scale * sum_{q-heads of j's kv-head} sum_i dS[i,j] * Q_i
 *   dV_j    =         sum_{q-heads of j's kv-head} sum_i P[i,j]  * dO_i
 *
 * Three steps, each a plain sum per output element so that no two threads
 * write one element: (1) per row, LSE and delta from the logits; (2) per
 * row, dQ; (3) per key row of a kv-head, dK and dV over every (q-head, row)
 * that sees it.  Rows without a visible key contribute nothing.
 */

/* Step 1 for every row (b, hq, i), row index (b*Hq+hq)*Sq+i.  0 or -2. */
static int bwd_lse_delta(const double* q, const double* k, const double* v,
                         const double* dout, int64_t B, int64_t Sq, int64_t Skv,
                         int64_t Hq, int64_t Hkv, int64_t D, int causal,
                         double scale, double* lse, double* delta) {
  const int64_t rows = B * Hq * Sq;
  int failed = 0;
#pragma omp parallel num_threads(oracle_threads())
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)Skv);
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!s || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < rows; ++r) {
        int64_t b = r / (Hq * Sq);
        int64_t hq = (r / Sq) % Hq;
        int64_t i = r % Sq;
        double m, l;
        row_partial(q, k, v, b, hq, i, Sq, Skv, Hq, Hkv, D, causal, scale, 0,
                    Skv, s, &m, &l, acc);
        const double* dorow = dout + ((b * Sq + i) * Hq + hq) * D;
        if (l > 0.0) {
          lse[r] = m + log(l);
          double dl = 0.0; /* dO . O, with O = acc / l */
          for (int64_t d = 0; d < D; ++d) dl += dorow[d] * (acc[d] / l);
          delta[r] = dl;
        } else {
          lse[r] = -INFINITY;
          delta[r] = 0.0;
        }
      }
    }
    free(s);
    free(acc);
  }
  return failed ? -2 : 0;
}

/* Step 2: dQ of row (b, hq, i) into dqrow[D]. */
static void bwd_dq_row(const double* q, const double* k, const double* v,
                       const double* dout, const double* lse,
                       const double* delta, int64_t b, int64_t hq, int64_t i,
                       int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv,
                       int64_t D, int causal, double scale, double* dqrow) {
  const int64_t group = Hq / Hkv;
  const int64_t hk = hq / group;
  const int64_t r = (b * Hq + hq) * Sq + i;
  const double* qrow = q + ((b * Sq + i) * Hq + hq) * D;
  const double* dorow = dout + ((b * Sq + i) * Hq + hq) * D;
  for (int64_t d = 0; d < D; ++d) dqrow[d] = 0.0;
  int64_t end = visible_end(i, Sq, Skv, causal);
  for (int64_t j = 0; j < end; ++j) {
    const double* krow = k + ((b * Skv + j) * Hkv + hk) * D;
    const double* vrow = v + ((b * Skv + j) * Hkv + hk) * D;
    double dot = 0.0, dp = 0.0;
    for (int64_t d = 0; d < D; ++d) {
      dot += qrow[d] * krow[d];
      dp += dorow[d] * vrow[d];
    }
    double p = exp(scale * dot - lse[r]);
    double ds = p * (dp - delta[r]);
    for (int64_t d = 0; d < D; ++d) dqrow[d] += scale * ds * krow[d];
  }
}

/* Step 3: dK and dV of key row (b, j, hk) into dkrow[D], dvrow[D]. */
static void bwd_dkdv_key(const double* q, const double* k, const double* v,
                         const double* dout, const double* lse,
                         const double* delta, int64_t b, int64_t hk, int64_t j,
                         int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv,
                         int64_t D, int causal, double scale, double* dkrow,
                         double* dvrow) {
  const int64_t group = Hq / Hkv;
  const double* krow = k + ((b * Skv + j) * Hkv + hk) * D;
  const double* vrow = v + ((b * Skv + j) * Hkv + hk) * D;
  for (int64_t d = 0; d < D; ++d) {
    dkrow[d] = 0.0;
    dvrow[d] = 0.0;
  }
  for (int64_t hq = hk * group; hq < (hk + 1) * group; ++hq) {
    for (int64_t i = 0; i < Sq; ++i) {
      if (j >= visible_end(i, Sq, Skv, causal)) continue;
      int64_t r = (b * Hq + hq) * Sq + i;
      const double* qrow = q + ((b * Sq + i) * Hq + hq) * D;
      const double* dorow = dout + ((b * Sq + i) * Hq + hq) * D;
      double dot = 0.0, dp = 0.0;
      for (int64_t d = 0; d < D; ++d) {
        dot += qrow[d] * krow[d];
        dp += dorow[d] * vrow[d];
      }
      double p = exp(scale * dot - lse[r]);
      double ds = p * (dp - delta[r]);
      for (int64_t d = 0; d < D; ++d) {
        dkrow[d] += scale * ds * qrow[d];
        dvrow[d] += p * dorow[d];
      }
    }
  }
}

/*
 * Every gradient: dq [B,Sq,Hq,D]; dk, dv [B,Skv,Hkv,D].  Returns 0, -1 on a
 * bad shape, -2 if scratch cannot be allocated.
 */
int oracle_attn_bwd(const double* q, const double* k, const double* v,
                    const double* dout, double* dq, double* dk, double* dv,
                    int64_t B, int64_t Sq, int64_t Skv, int64_t Hq, int64_t Hkv,
                    int64_t D, int causal, double scale) {
  if (check_shape(B, Sq, Skv, Hq, Hkv, D)) return -1;
  const int64_t rows = B * Hq * Sq;
  double* lse = (double*)malloc(sizeof(double) * (size_t)rows);
  double* delta = (double*)malloc(sizeof(double) * (size_t)rows);
  int rc = (!lse || !delta) ? -2
                            : bwd_lse_delta(q, k, v, dout, B, Sq, Skv, Hq, Hkv,
                                            D, causal, scale, lse, delta);
  if (rc == 0) {
#pragma omp parallel for schedule(dynamic, 16) num_threads(oracle_threads())
    for (int64_t r = 0; r < rows; ++r) {
      int64_t b = r / (Hq * Sq), hq = (r / Sq) % Hq, i = r % Sq;
      bwd_dq_row(q, k, v, dout, lse, delta, b, hq, i, Sq, Skv, Hq, Hkv, D,
                 causal, scale, dq + ((b * Sq + i) * Hq + hq) * D);
    }
    const int64_t krows = B * Skv * Hkv;
#pragma omp parallel for schedule(dynamic, 16) num_threads(oracle_threads())
    for (int64_t kr = 0; kr < krows; ++kr) {
      int64_t b = kr / (Skv * Hkv), j = (kr / Hkv) % Skv, hk = kr % Hkv;
      bwd_dkdv_key(q, k, v, dout, lse, delta, b, hk, j, Sq, Skv, Hq, Hkv, D,
                   causal, scale, dk + ((b * Skv + j) * Hkv + hk) * D,
                   dv + ((b * Skv + j) * Hkv + hk) * D);
    }
  }
  free(lse);
  free(delta);
  return rc;
}

/*
 * Selected gradients, for checks at sizes where every gradient is too slow:
 * dQ of the nq query rows qrows (triples b, hq, i) into dq_rows [nq, D], and
 * dK, dV of the nk key rows krows (triples b, hk, j) into dk_rows, dv_rows
 * [nk, D].  Step 1 still runs over every row.  Returns 0, -1 on a bad shape
 * or index, -2 if scratch cannot be allocated.
 */
int oracle_attn_bwd_rows(const double* q, const double* k, const double* v,
                         const double* dout, int64_t B, int64_t Sq, int64_t Skv,
                         int64_t Hq, int64_t Hkv, int64_t D, int causal,
                         double scale, const int64_t* qrows, int64_t nq,
                         double* dq_rows, const int64_t* krows, int64_t nk,
                         double* dk_rows, double* dv_rows) {
  if (check_shape(B, Sq, Skv, Hq, Hkv, D)) return -1;
  for (int64_t n = 0; n < nq; ++n) {
    const int64_t* t = qrows + 3 * n;
    if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= Hq || t[2] < 0 || t[2] >= Sq) return -1;
  }
  for (int64_t n = 0; n < nk; ++n) {
    const int64_t* t = krows + 3 * n;
    if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= Hkv || t[2] < 0 || t[2] >= Skv) return -1;
  }
  const int64_t rows = B * Hq * Sq;
  double* lse = (double*)malloc(sizeof(double) * (size_t)rows);
  double* delta = (double*)malloc(sizeof(double) * (size_t)rows);
  int rc = (!lse || !delta) ? -2
                            : bwd_lse_delta(q, k, v, dout, B, Sq, Skv, Hq, Hkv,
                                            D, causal, scale, lse, delta);
  if (rc == 0) {
#pragma omp parallel for schedule(dynamic, 4) num_threads(oracle_threads())
    for (int64_t n = 0; n < nq; ++n) {
      const int64_t* t = qrows + 3 * n;
      bwd_dq_row(q, k, v, dout, lse, delta, t[0], t[1], t[2], Sq, Skv, Hq, Hkv,
                 D, causal, scale, dq_rows + n * D);
    }
#pragma omp parallel for schedule(dynamic, 4) num_threads(oracle_threads())
    for (int64_t n = 0; n < nk; ++n) {
      const int64_t* t = krows + 3 * n;
      bwd_dkdv_key(q, k, v, dout, lse, delta, t[0], t[1], t[2], Sq, Skv, Hq,
                   Hkv, D, causal, scale, dk_rows + n * D, dv_rows + n * D);
    }
  }
  free(lse);
  free(delta);
  return rc;
}
