/*
 * ORACLE -- test infrastructure only.
 *
 * A plain, slow CPU statement of what one rank's share of an Ulysses
 * sequence-parallel attention layer computes.  Only the tests, the smoke
 * check and the benchmark's CPU-baseline leg may load it; the product path
 * never does.  It shares no code with the HIP library.
 *
 * Sources (the pages' titles and sections):
 *  - "Ulysses Sequence Parallelism: Training with Million-Token Contexts"
 *    (Hugging Face blog, Chinese translation), section "The challenge of
 *    long-sequence training" -> how Ulysses works: sequence sharding, an
 *    all-to-all that leaves every GPU with all positions for a subset of the
 *    heads, local attention per head, and an inverse all-to-all.
 *  - "DeepSpeed Ulysses SP and ALST integration guide for HF Transformers"
 *    (zwxr.cn), sections on the attention adapter (tensor layout
 *    [sl, bs, hc, hs]; causality from position ids instead of a 4D mask;
 *    GQA/MQA head rules; packed samples reset position ids).
 *  - Transformers "DeepSpeed ALST/Ulysses" guide walkthrough
 *    (demingchina.com), the two-GPU layout diagram.
 *  - "DeepSpeed Ulysses: system optimizations for training extremely long
 *    sequence Transformer models" (DeepSpeed blog, Chinese), the design
 *    section (per-head attention after the first all-to-all).
 *
 * Readings where the pages are silent:
 *  - attention is standard scaled dot-product softmax attention per head
 *    (the formula on the DeepSpeed blog is an image that did not survive);
 *  - query head h uses key/value head floor(h / (hq / hkv));
 *  - causal mask is j <= i (queries and keys share positions);
 *  - with documents (cu_seqlens) a query attends only inside its own
 *    document; without causality it attends to its whole document;
 *  - LSE is the natural-log log-sum-exp of the scaled scores;
 *  - the backward pass is the gradient of O with respect to Q, K and V.
 *
 * Arithmetic: every float sum and product is carried out in double from the
 * exact input values; exp and log are the C library's double functions.
 * Loops over independent output rows may run on several threads
 * (OpenMP); every output element is computed by one thread in a fixed
 * order, so results do not depend on the thread count.
 *
 * Parity pins for every function are in tests/test_oracle_pins.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------
 * Layout exchange, one rank's view.
 *
 * Seq-sharded: chunk c (held by rank c before the exchange) is
 * [n, bs, heads, hd] and holds tokens [c*n, (c+1)*n) with all heads.
 * Head-sharded: rank r holds [P*n, bs, heads_l, hd], all tokens for its
 * head slice.  heads_l = heads / P; when heads < P (and P % heads == 0) the
 * head is replicated: heads_l = 1 and rank r takes head floor(r*heads/P).
 * ---------------------------------------------------------------------- */

static int local_heads(int heads, int P) { return heads >= P ? heads / P : 1; }

static int source_head(int heads, int P, int rank, int h) {
  if (heads >= P) return rank * (heads / P) + h;
  return (int)(((long)rank * heads) / P);
}

/* out[c*n + s, b, h, :] = chunk_c[s, b, source_head(h), :] */
int oracle_seq_to_head(const void* const* chunks, int P, int rank, int64_t n, int bs,
                       int heads, int hd, int esize, void* out) {
  if (P <= 0 || rank < 0 || rank >= P || n < 0 || bs <= 0 || heads <= 0 || hd <= 0) return -1;
  if (heads >= P ? heads % P : P % heads) return -1;
  const int hl = local_heads(heads, P);
  const size_t row = (size_t)hd * esize;
  for (int c = 0; c < P; ++c) {
    const char* src = (const char*)chunks[c];
    for (int64_t s = 0; s < n; ++s)
      for (int b = 0; b < bs; ++b)
        for (int h = 0; h < hl; ++h) {
          const int64_t t = (int64_t)c * n + s;
          const size_t o_off = ((((size_t)t * bs + b) * hl) + h) * row;
          const size_t i_off = ((((size_t)s * bs + b) * heads) + source_head(heads, P, rank, h)) * row;
          memcpy((char*)out + o_off, src + i_off, row);
        }
  }
  return 0;
}

/* chunk_c[s, b, rank*hl + h, :] = in[c*n + s, b, h, :]; other head slots of
 * the chunks are not written (they belong to the other ranks). */
int oracle_head_to_seq(const void* in, int P, int rank, int64_t n, int bs, int heads,
                       int hd, int esize, void* const* chunks) {
  if (P <= 0 || rank < 0 || rank >= P || n < 0 || bs <= 0 || heads <= 0 || hd <= 0) return -1;
  if (heads % P) return -1;
  const int hl = heads / P;
  const size_t row = (size_t)hd * esize;
  for (int c = 0; c < P; ++c) {
    char* dst = (char*)chunks[c];
    for (int64_t s = 0; s < n; ++s)
      for (int b = 0; b < bs; ++b)
        for (int h = 0; h < hl; ++h) {
          const int64_t t = (int64_t)c * n + s;
          const size_t i_off = ((((size_t)t * bs + b) * hl) + h) * row;
          const size_t o_off = ((((size_t)s * bs + b) * heads) + rank * hl + h) * row;
          memcpy(dst + o_off, (const char*)in + i_off, row);
        }
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Attention.
 *
 * Tensors are [N, bs, heads, hd] (row-major, the pages' [sl, bs, hc, hs]).
 * cu is NULL (one document) or cu[0]=0 < cu[1] < ... < cu[ndocs]=N.
 * ---------------------------------------------------------------------- */

typedef struct {
  const double *q, *k, *v;
  int64_t N;
  int bs, hq, hkv, hd;
  double scale;
  int causal;
  const int64_t* cu;
  int ndocs;
} attn_t;

static double qv(const attn_t* a, const double* x, int heads, int64_t t, int b, int h, int e) {
  return x[(((size_t)t * a->bs + b) * heads + h) * a->hd + e];
}

/* Document index of position i. */
static int doc_of(const attn_t* a, int64_t i) {
  if (!a->cu) return 0;
  int d = 0;
  while (d + 1 < a->ndocs && a->cu[d + 1] <= i) ++d;
  return d;
}

static int64_t doc_start(const attn_t* a, int64_t i) { return a->cu ? a->cu[doc_of(a, i)] : 0; }
static int64_t doc_end(const attn_t* a, int64_t i) { return a->cu ? a->cu[doc_of(a, i) + 1] : a->N; }

/* Keys j that query i may attend to: [lo, hi). */
static void key_range(const attn_t* a, int64_t i, int64_t* lo, int64_t* hi) {
  *lo = doc_start(a, i);
  *hi = a->causal ? i + 1 : doc_end(a, i);
}

/* Queries i that attend to key j: [lo, hi). */
static void query_range(const attn_t* a, int64_t j, int64_t* lo, int64_t* hi) {
  *lo = a->causal ? j : doc_start(a, j);
  *hi = doc_end(a, j);
}

static int kv_head(const attn_t* a, int h) { return h / (a->hq / a->hkv); }

/* s_ij = scale * <q_i, k_j> */
static double score(const attn_t* a, int64_t i, int64_t j, int b, int h) {
  const int kh = kv_head(a, h);
  double acc = 0.0;
  for (int e = 0; e < a->hd; ++e)
    acc += qv(a, a->q, a->hq, i, b, h, e) * qv(a, a->k, a->hkv, j, b, kh, e);
  return a->scale * acc;
}

/* Row statistics of query (i, b, h): LSE_i = m_i + ln sum_j exp(s_ij - m_i)
 * and, if o != NULL, O_i = sum_j exp(s_ij - LSE_i) v_j.  s is scratch of
 * length >= number of keys. */
static double row_forward(const attn_t* a, int64_t i, int b, int h, double* s, double* o,
                          double* o_mag) {
  int64_t lo, hi;
  key_range(a, i, &lo, &hi);
  double m = -INFINITY;
  for (int64_t j = lo; j < hi; ++j) {
    s[j - lo] = score(a, i, j, b, h);
    if (s[j - lo] > m) m = s[j - lo];
  }
  double l = 0.0;
  for (int64_t j = lo; j < hi; ++j) l += exp(s[j - lo] - m);
  const double lse = m + log(l);
  if (o) {
    const int kh = kv_head(a, h);
    for (int e = 0; e < a->hd; ++e) o[e] = 0.0;
    if (o_mag)
      for (int e = 0; e < a->hd; ++e) o_mag[e] = 0.0;
    for (int64_t j = lo; j < hi; ++j) {
      const double p = exp(s[j - lo] - lse);
      for (int e = 0; e < a->hd; ++e) {
        o[e] += p * qv(a, a->v, a->hkv, j, b, kh, e);
        if (o_mag) o_mag[e] += p * fabs(qv(a, a->v, a->hkv, j, b, kh, e));
      }
    }
  }
  return lse;
}

static int check_docs(const int64_t* cu, int ndocs, int64_t N) {
  if (!cu) return 0;
  if (ndocs < 1 || cu[0] != 0 || cu[ndocs] != N) return -1;
  for (int d = 0; d < ndocs; ++d)
    if (cu[d + 1] <= cu[d]) return -1;
  return 0;
}

/*
 * Forward.  rows: NULL for all N positions, else nrows positions.  Outputs
 * are compact over the selected positions: o[t, b, h, :] for t < nrows and
 * lse[b, h, t].  o_mag (optional, same layout as o) receives the magnitude
 * of each output sum, sum_j P_ij |v_j|: the scale of the rounding error a
 * finite-precision evaluation of that sum can make.  Returns 0, or -1 on
 * malformed arguments.
 */
int oracle_attn_fwd(const double* q, const double* k, const double* v, int64_t N, int bs,
                    int hq, int hkv, int hd, double scale, int causal, const int64_t* cu,
                    int ndocs, const int64_t* rows, int64_t nrows, double* o, double* lse,
                    double* o_mag) {
  if (N <= 0 || bs <= 0 || hq <= 0 || hkv <= 0 || hd <= 0 || hq % hkv) return -1;
  if (check_docs(cu, ndocs, N)) return -1;
  const attn_t a = {q, k, v, N, bs, hq, hkv, hd, scale, causal, cu, ndocs};
  const int64_t nsel = rows ? nrows : N;
  for (int64_t t = 0; t < nsel; ++t)
    if (rows && (rows[t] < 0 || rows[t] >= N)) return -1;
  const int64_t total = nsel * bs * hq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
    for (int64_t w = 0; w < total; ++w) {
      const int64_t t = w / (bs * hq);
      const int b = (int)((w / hq) % bs);
      const int h = (int)(w % hq);
      const int64_t i = rows ? rows[t] : t;
      const size_t off = (((size_t)t * bs + b) * hq + h) * hd;
      lse[((size_t)b * hq + h) * nsel + t] =
          row_forward(&a, i, b, h, s, o + off, o_mag ? o_mag + off : NULL);
    }
    free(s);
  }
  return 0;
}

/*
 * Backward of O with respect to Q, K, V for upstream gradient dO:
 *   D_i    = sum_e dO_ie O_ie
 *   P_ij   = exp(s_ij - LSE_i)
 *   dP_ij  = <dO_i, v_j>
 *   dS_ij  = P_ij (dP_ij - D_i)
 *   dQ_i   = scale * sum_j dS_ij k_j
 *   dK_j   = scale * sum_{h in group} sum_i dS_ij q_i
 *   dV_j   = sum_{h in group} sum_i P_ij dO_i
 * where j ranges over the keys query i attends to, and i over the queries
 * that attend to key j.  LSE_i and O_i are this file's own forward values.
 *
 * dq_rows: NULL for all positions, else the positions whose dQ is wanted
 * (dq is compact [t, bs, hq, hd]).  dkv_cols likewise for dK/dV
 * (compact [t, bs, hkv, hd]).  Pass n = 0 with a non-NULL pointer to skip.
 * o_in, lse_in (optional): the forward's O ([N, bs, hq, hd]) and LSE
 * ([bs, hq, N]) to use in place of this file's own values, as the backward
 * receives them from a forward call: D_i = <dO_i, o_in_i> and
 * P_ij = exp(s_ij - lse_in_i).
 * dq_mag, dk_mag, dv_mag (optional, NULL to skip; layouts as dq, dk, dv)
 * receive the magnitude of each output sum -- the same sum with every term
 * replaced by its absolute value:
 *   scale sum_j |dS_ij| |k_j|,  scale sum_h sum_i |dS_ij| |q_i|,  sum_h sum_i P_ij |dO_i|.
 * dq_dmag, dk_dmag (optional) receive how strongly dQ and dK depend on D:
 *   scale A_i sum_j P_ij |k_j|  and  scale sum_h sum_i P_ij A_i |q_i|,
 * with A_i = sum_e |dO_ie| sum_j P_ij |v_je| the magnitude of D_i's sum; an
 * error dD_i in D (e.g. from O rounded to a short format) moves dQ_i and
 * dK_j by at most these times |dD_i| / A_i.
 */
int oracle_attn_bwd(const double* q, const double* k, const double* v, const double* dout,
                    int64_t N, int bs, int hq, int hkv, int hd, double scale, int causal,
                    const int64_t* cu, int ndocs, const int64_t* dq_rows, int64_t n_dq,
                    const int64_t* dkv_cols, int64_t n_dkv, const double* o_in,
                    const double* lse_in, double* dq, double* dk, double* dv, double* dq_mag,
                    double* dk_mag, double* dv_mag, double* dq_dmag, double* dk_dmag) {
  if (N <= 0 || bs <= 0 || hq <= 0 || hkv <= 0 || hd <= 0 || hq % hkv) return -1;
  if (check_docs(cu, ndocs, N)) return -1;
  const attn_t a = {q, k, v, N, bs, hq, hkv, hd, scale, causal, cu, ndocs};
  const int64_t nq = dq_rows ? n_dq : N;
  const int64_t nk = dkv_cols ? n_dkv : N;
  for (int64_t t = 0; t < nq; ++t)
    if (dq_rows && (dq_rows[t] < 0 || dq_rows[t] >= N)) return -1;
  for (int64_t t = 0; t < nk; ++t)
    if (dkv_cols && (dkv_cols[t] < 0 || dkv_cols[t] >= N)) return -1;
  const int g = hq / hkv;

  /* Which query rows need LSE and D: the dQ rows, and every query that
   * attends to a requested key. */
  char* need = (char*)calloc((size_t)N, 1);
  for (int64_t t = 0; t < nq; ++t) need[dq_rows ? dq_rows[t] : t] = 1;
  for (int64_t t = 0; t < nk; ++t) {
    int64_t lo, hi;
    query_range(&a, dkv_cols ? dkv_cols[t] : t, &lo, &hi);
    for (int64_t i = lo; i < hi; ++i) need[i] = 1;
  }
  double* LSE = (double*)malloc(sizeof(double) * (size_t)N * bs * hq);
  double* D = (double*)malloc(sizeof(double) * (size_t)N * bs * hq);
  double* A = (double*)malloc(sizeof(double) * (size_t)N * bs * hq);
  const int want_dmag = dq_dmag != NULL || dk_dmag != NULL;
  const int64_t total = N * bs * hq;
#pragma omp parallel
  {
    double* s = (double*)malloc(sizeof(double) * (size_t)N);
    double* o = (double*)malloc(sizeof(double) * (size_t)hd);
    double* om = (double*)malloc(sizeof(double) * (size_t)hd);
#pragma omp for schedule(dynamic, 16)
    for (int64_t w = 0; w < total; ++w) {
      const int64_t i = w / (bs * hq);
      if (!need[i]) continue;
      const int b = (int)((w / hq) % bs);
      const int h = (int)(w % hq);
      const size_t idx = ((size_t)b * hq + h) * N + i;
      const int fwd = !(o_in && lse_in) || want_dmag;
      const double lse = fwd ? row_forward(&a, i, b, h, s, o, om) : 0.0;
      LSE[idx] = lse_in ? lse_in[idx] : lse;
      double d = 0.0, mag = 0.0;
      for (int e = 0; e < hd; ++e) {
        const double oe = o_in ? qv(&a, o_in, hq, i, b, h, e) : o[e];
        d += qv(&a, dout, hq, i, b, h, e) * oe;
        if (fwd) mag += fabs(qv(&a, dout, hq, i, b, h, e)) * om[e];
      }
      D[idx] = d;
      A[idx] = mag;
    }
    free(s);
    free(o);
    free(om);
  }

  /* dQ rows. */
  const int64_t totq = nq * bs * hq;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t w = 0; w < totq; ++w) {
    const int64_t t = w / (bs * hq);
    const int b = (int)((w / hq) % bs);
    const int h = (int)(w % hq);
    const int64_t i = dq_rows ? dq_rows[t] : t;
    const int kh = kv_head(&a, h);
    const size_t idx = ((size_t)b * hq + h) * N + i;
    double* out = dq + (((size_t)t * bs + b) * hq + h) * hd;
    double* mag = dq_mag ? dq_mag + (((size_t)t * bs + b) * hq + h) * hd : NULL;
    double* dmag = dq_dmag ? dq_dmag + (((size_t)t * bs + b) * hq + h) * hd : NULL;
    for (int e = 0; e < hd; ++e) out[e] = 0.0;
    if (mag)
      for (int e = 0; e < hd; ++e) mag[e] = 0.0;
    if (dmag)
      for (int e = 0; e < hd; ++e) dmag[e] = 0.0;
    int64_t lo, hi;
    key_range(&a, i, &lo, &hi);
    for (int64_t j = lo; j < hi; ++j) {
      const double p = exp(score(&a, i, j, b, h) - LSE[idx]);
      double dp = 0.0;
      for (int e = 0; e < hd; ++e) dp += qv(&a, dout, hq, i, b, h, e) * qv(&a, v, hkv, j, b, kh, e);
      const double ds = p * (dp - D[idx]);
      for (int e = 0; e < hd; ++e) {
        out[e] += ds * qv(&a, k, hkv, j, b, kh, e);
        if (mag) mag[e] += fabs(ds) * fabs(qv(&a, k, hkv, j, b, kh, e));
        if (dmag) dmag[e] += p * A[idx] * fabs(qv(&a, k, hkv, j, b, kh, e));
      }
    }
    for (int e = 0; e < hd; ++e) out[e] *= scale;
    if (mag)
      for (int e = 0; e < hd; ++e) mag[e] *= scale;
    if (dmag)
      for (int e = 0; e < hd; ++e) dmag[e] *= scale;
  }

  /* dK, dV columns. */
  const int64_t totk = nk * bs * hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t w = 0; w < totk; ++w) {
    const int64_t t = w / (bs * hkv);
    const int b = (int)((w / hkv) % bs);
    const int kh = (int)(w % hkv);
    const int64_t j = dkv_cols ? dkv_cols[t] : t;
    const size_t off = (((size_t)t * bs + b) * hkv + kh) * hd;
    double* okk = dk + off;
    double* ovv = dv + off;
    double* mk = dk_mag ? dk_mag + off : NULL;
    double* mv = dv_mag ? dv_mag + off : NULL;
    double* dmk = dk_dmag ? dk_dmag + off : NULL;
    for (int e = 0; e < hd; ++e) okk[e] = ovv[e] = 0.0;
    if (dmk)
      for (int e = 0; e < hd; ++e) dmk[e] = 0.0;
    if (mk)
      for (int e = 0; e < hd; ++e) mk[e] = 0.0;
    if (mv)
      for (int e = 0; e < hd; ++e) mv[e] = 0.0;
    int64_t lo, hi;
    query_range(&a, j, &lo, &hi);
    for (int h = kh * g; h < (kh + 1) * g; ++h)
      for (int64_t i = lo; i < hi; ++i) {
        const size_t idx = ((size_t)b * hq + h) * N + i;
        const double p = exp(score(&a, i, j, b, h) - LSE[idx]);
        double dp = 0.0;
        for (int e = 0; e < hd; ++e) dp += qv(&a, dout, hq, i, b, h, e) * qv(&a, v, hkv, j, b, kh, e);
        const double ds = p * (dp - D[idx]);
        for (int e = 0; e < hd; ++e) {
          okk[e] += ds * qv(&a, q, hq, i, b, h, e);
          ovv[e] += p * qv(&a, dout, hq, i, b, h, e);
          if (mk) mk[e] += fabs(ds) * fabs(qv(&a, q, hq, i, b, h, e));
          if (mv) mv[e] += p * fabs(qv(&a, dout, hq, i, b, h, e));
          if (dmk) dmk[e] += p * A[idx] * fabs(qv(&a, q, hq, i, b, h, e));
        }
      }
    for (int e = 0; e < hd; ++e) okk[e] *= scale;
    if (mk)
      for (int e = 0; e < hd; ++e) mk[e] *= scale;
    if (dmk)
      for (int e = 0; e < hd; ++e) dmk[e] *= scale;
  }
  free(need);
  free(LSE);
  free(D);
  free(A);
  return 0;
}

/* ------------------------------------------------------------------------
 * Merge of two partial attention results over disjoint key sets A and B:
 * the combination step of ring (blockwise) attention, which the Hugging Face
 * Ulysses blog compares with Ulysses in "Ulysses vs Ring Attention" (the key/
 * value blocks travel around a ring and every block's result is folded into
 * the running one).  Each partial O is its block's sum of exp(s_ij) v_j
 * divided by its block's exp(LSE), so over A and B together
 *   LSE = ln(exp(LSE_a) + exp(LSE_b)),
 *   O   = exp(LSE_a - LSE) O_a + exp(LSE_b - LSE) O_b.
 * A partial whose LSE is -inf saw no key: it contributes nothing, whatever
 * its O holds; if both are -inf the row has no key at all: O = 0 and
 * LSE = -inf.
 * O tensors are [N, bs, heads, hd], LSE tensors [bs, heads, N].
 * ---------------------------------------------------------------------- */
int oracle_attn_merge(const double* o_a, const double* lse_a, const double* o_b,
                      const double* lse_b, int64_t N, int bs, int heads, int hd, double* o,
                      double* lse) {
  if (N < 0 || bs < 1 || heads < 1 || hd < 1 || !o_a || !lse_a || !o_b || !lse_b || !o || !lse)
    return 1;
  for (int64_t i = 0; i < N; ++i)
    for (int b = 0; b < bs; ++b)
      for (int h = 0; h < heads; ++h) {
        const size_t r = ((size_t)b * heads + h) * (size_t)N + (size_t)i;
        const double la = lse_a[r], lb = lse_b[r];
        const double m = la > lb ? la : lb;
        double L = -INFINITY, wa = 0.0, wb = 0.0;
        if (m != -INFINITY) {
          L = m + log(exp(la - m) + exp(lb - m));
          wa = exp(la - L);
          wb = exp(lb - L);
        }
        lse[r] = L;
        const size_t row = (((size_t)i * bs + b) * heads + h) * (size_t)hd;
        for (int e = 0; e < hd; ++e) {
          double x = 0.0;
          if (la != -INFINITY) x += wa * o_a[row + e];
          if (lb != -INFINITY) x += wb * o_b[row + e];
          o[row + e] = x;
        }
      }
  return 0;
}

/* ----------------------------------------------------------------------
 * Language-model loss over the hidden states and its gradients: the
 * computation that the integration guide's tiled fused logits loss
 * (section on tiled loss computation) shards over the sequence so that
 * the [tokens, vocab] logits never exist in full.  Sharding does not change
 * the result, so the oracle states it whole, by definition:
 *   z_iv   = <h_i, w_v>                       (lm_head, no bias)
 *   lse_i  = ln sum_v exp(z_iv)
 *   loss_i = lse_i - z_i,y_i   for a token whose label y_i is not the
 *            ignore index (labels arrive already shifted, so label i is
 *            the target of position i); 0 for an ignored token
 *   loss_sum = sum_i loss_i,  n_good = number of tokens not ignored
 *   G_iv   = s (softmax(z_i)_v - [v == y_i]) for a kept token, 0 otherwise,
 *            the gradient of s * loss_sum with respect to z_iv
 *   dh = G W   ([T, d]),   dW = G^T H   ([V, d]).
 * The caller picks s: 1 / (total good tokens over all ranks) gives the
 * gradient of the guide's loss aggregation (sum of per-rank losses
 * weighted by good tokens, divided by the total good tokens).
 * Optional magnitude outputs (any may be NULL) bound the rounding of a
 * low-precision implementation: zmag_i = max_v sum_k |h_ik w_vk|,
 * dh_mag = |G| |W|, dw_mag = |G|^T |H|.
 * h is [T, d], w is [V, d], labels [T]; every output is row-major.
 * ---------------------------------------------------------------------- */
int oracle_logits_loss(const double* h, const double* w, const int64_t* labels, int64_t T,
                       int64_t d, int64_t V, int64_t ignore_index, double s, double* loss_rows,
                       double* loss_sum, int64_t* n_good, double* dh, double* dw, double* zmag,
                       double* dh_mag, double* dw_mag) {
  if (T < 0 || d < 1 || V < 1 || !h || !w || !labels || !loss_rows || !loss_sum || !n_good ||
      !dh || !dw)
    return 1;
  for (int64_t i = 0; i < T; ++i)
    if (labels[i] != ignore_index && (labels[i] < 0 || labels[i] >= V)) return 2;
  double* G = (double*)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * (size_t)V);
  if (!G) return 3;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < T; ++i) {
    double* z = G + (size_t)i * (size_t)V;
    double zm = 0.0;
    for (int64_t v = 0; v < V; ++v) {
      double acc = 0.0, mag = 0.0;
      for (int64_t k = 0; k < d; ++k) {
        acc += h[i * d + k] * w[v * d + k];
        mag += fabs(h[i * d + k] * w[v * d + k]);
      }
      z[v] = acc;
      if (mag > zm) zm = mag;
    }
    if (zmag) zmag[i] = zm;
    if (labels[i] == ignore_index) {
      loss_rows[i] = 0.0;
      for (int64_t v = 0; v < V; ++v) z[v] = 0.0;
      continue;
    }
    double m = z[0];
    for (int64_t v = 1; v < V; ++v)
      if (z[v] > m) m = z[v];
    double sum = 0.0;
    for (int64_t v = 0; v < V; ++v) sum += exp(z[v] - m);
    const double lse = m + log(sum);
    loss_rows[i] = lse - z[labels[i]];
    for (int64_t v = 0; v < V; ++v) z[v] = s * (exp(z[v] - lse) - (v == labels[i] ? 1.0 : 0.0));
  }
  double total = 0.0;
  int64_t good = 0;
  for (int64_t i = 0; i < T; ++i) {
    total += loss_rows[i];
    if (labels[i] != ignore_index) ++good;
  }
  *loss_sum = total;
  *n_good = good;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < T; ++i)
    for (int64_t k = 0; k < d; ++k) {
      double acc = 0.0, mag = 0.0;
      for (int64_t v = 0; v < V; ++v) {
        acc += G[(size_t)i * V + v] * w[v * d + k];
        mag += fabs(G[(size_t)i * V + v] * w[v * d + k]);
      }
      dh[i * d + k] = acc;
      if (dh_mag) dh_mag[i * d + k] = mag;
    }
#pragma omp parallel for schedule(static)
  for (int64_t v = 0; v < V; ++v)
    for (int64_t k = 0; k < d; ++k) {
      double acc = 0.0, mag = 0.0;
      for (int64_t i = 0; i < T; ++i) {
        acc += G[(size_t)i * V + v] * h[i * d + k];
        mag += fabs(G[(size_t)i * V + v] * h[i * d + k]);
      }
      dw[v * d + k] = acc;
      if (dw_mag) dw_mag[v * d + k] = mag;
    }
  free(G);
  return 0;
}

/* ----------------------------------------------------------------------
 * Sequence-tiled SwiGLU MLP (the integration guide's TiledMLP, section on
 * the ALST memory tricks): the MLP of a Llama-style block,
 *   g = x Wg^T,  u = x Wu^T   ([T, I]; Wg, Wu are [I, d])
 *   a = silu(g) * u,  silu(g) = g / (1 + e^-g)
 *   y = a Wd^T                ([T, d]; Wd is [d, I])
 * which TiledMLP runs a shard of tokens at a time to bound the [T, I]
 * intermediates; rows are independent, so the result is the whole-sequence
 * MLP and the oracle states that.  Backward, for the upstream gradient dy:
 *   da = dy Wd,  dWd = dy^T a
 *   dg = da * u * silu'(g),  silu'(g) = s (1 + g (1 - s)),  s = 1/(1+e^-g)
 *   du = da * silu(g)
 *   dx = dg Wg + du Wu,  dWg = dg^T x,  dWu = du^T x.
 * dy == NULL: forward only (dx, dwg, dwu, dwd unused).  Optional magnitude
 * outputs (NULL to skip) bound the rounding of a low-precision
 * implementation that rounds a, dg and du before the products that use them:
 *   y_mag = |a| |Wd|^T, dx_mag = |dg| |Wg| + |du| |Wu|, dwg_mag = |dg|^T |x|,
 *   dwu_mag = |du|^T |x|, dwd_mag = |dy|^T |a|.
 * All matrices row-major.
 * ---------------------------------------------------------------------- */
static double sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }

int oracle_swiglu_mlp(const double* x, const double* wg, const double* wu, const double* wd,
                      const double* dy, int64_t T, int64_t d, int64_t I, double* y, double* dx,
                      double* dwg, double* dwu, double* dwd, double* y_mag, double* dx_mag,
                      double* dwg_mag, double* dwu_mag, double* dwd_mag) {
  if (T < 0 || d < 1 || I < 1 || !x || !wg || !wu || !wd || !y) return 1;
  if (dy && (!dx || !dwg || !dwu || !dwd)) return 1;
  const size_t TI = (size_t)(T > 0 ? T : 1) * (size_t)I;
  double* a = (double*)malloc(sizeof(double) * TI);
  double* dg = (double*)malloc(sizeof(double) * TI);
  double* du = (double*)malloc(sizeof(double) * TI);
  if (!a || !dg || !du) {
    free(a);
    free(dg);
    free(du);
    return 3;
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < T; ++i) {
    for (int64_t j = 0; j < I; ++j) {
      double g = 0.0, u = 0.0;
      for (int64_t k = 0; k < d; ++k) {
        g += x[i * d + k] * wg[j * d + k];
        u += x[i * d + k] * wu[j * d + k];
      }
      const double s = sigmoid(g);
      a[(size_t)i * I + j] = g * s * u;
      if (dy) {
        double da = 0.0;
        for (int64_t k = 0; k < d; ++k) da += dy[i * d + k] * wd[k * I + j];
        dg[(size_t)i * I + j] = da * u * s * (1.0 + g * (1.0 - s));
        du[(size_t)i * I + j] = da * g * s;
      }
    }
    for (int64_t k = 0; k < d; ++k) {
      double acc = 0.0, mag = 0.0;
      for (int64_t j = 0; j < I; ++j) {
        acc += a[(size_t)i * I + j] * wd[k * I + j];
        mag += fabs(a[(size_t)i * I + j] * wd[k * I + j]);
      }
      y[i * d + k] = acc;
      if (y_mag) y_mag[i * d + k] = mag;
    }
    if (dy)
      for (int64_t k = 0; k < d; ++k) {
        double acc = 0.0, mag = 0.0;
        for (int64_t j = 0; j < I; ++j) {
          const double p = dg[(size_t)i * I + j] * wg[j * d + k];
          const double q = du[(size_t)i * I + j] * wu[j * d + k];
          acc += p + q;
          mag += fabs(p) + fabs(q);
        }
        dx[i * d + k] = acc;
        if (dx_mag) dx_mag[i * d + k] = mag;
      }
  }
  if (dy) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < I; ++j)
      for (int64_t k = 0; k < d; ++k) {
        double sg = 0.0, su = 0.0, mg = 0.0, mu = 0.0;
        for (int64_t i = 0; i < T; ++i) {
          sg += dg[(size_t)i * I + j] * x[i * d + k];
          su += du[(size_t)i * I + j] * x[i * d + k];
          mg += fabs(dg[(size_t)i * I + j] * x[i * d + k]);
          mu += fabs(du[(size_t)i * I + j] * x[i * d + k]);
        }
        dwg[j * d + k] = sg;
        dwu[j * d + k] = su;
        if (dwg_mag) dwg_mag[j * d + k] = mg;
        if (dwu_mag) dwu_mag[j * d + k] = mu;
      }
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < d; ++k)
      for (int64_t j = 0; j < I; ++j) {
        double acc = 0.0, mag = 0.0;
        for (int64_t i = 0; i < T; ++i) {
          acc += dy[i * d + k] * a[(size_t)i * I + j];
          mag += fabs(dy[i * d + k] * a[(size_t)i * I + j]);
        }
        dwd[k * I + j] = acc;
        if (dwd_mag) dwd_mag[k * I + j] = mag;
      }
  }
  free(a);
  free(dg);
  free(du);
  return 0;
}
