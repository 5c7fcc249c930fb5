/*
 * pfa_oracle.c -- plain, slow, fp64 CPU oracle for packed (block-diagonal) attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load this
 * file; only the tests, the smoke check and the benchmark's CPU-baseline leg use it.
 * It shares no code, header or constant with the HIP library.
 *
 * What it computes (the plain definition, written out):
 *   Tokens of several images are concatenated into one sequence; cu_seqlens[s] is the
 *   offset of image s, so image s owns rows [cu[s], cu[s+1]) of q, k and v, each laid
 *   out as [total_tokens, heads, dim].  (Mage-Flow page, hankli.space, section
 *   "原生分辨率序列打包 / Packing + Flash Attention Varlen": the packed_attention
 *   listing's q/k/v shape and cu_seqlens = [0, len0, len0+len1, ...].)
 *   Tokens of different images never attend to each other (same page, the sentence
 *   after that listing: the varlen call applies a block-diagonal mask); attention is
 *   non-causal (causal=False in the same listing).
 *   Within a segment, for query i and head h, with scale the caller's factor
 *   (1/sqrt(d) in the pages' dense definition: lmnt.cn GigaPath-Flash page, section 4.1
 *   naive_attention; jefxiong.cn SparseAttn article, section 3.1, the s_ij equation):
 *       s_ij   = scale * sum_t q[i,h,t] k[j,h,t]        j in the segment of i
 *       M_i    = max_j s_ij
 *       Z_i    = sum_j exp(s_ij - M_i)
 *       O[i,h] = sum_j exp(s_ij - M_i) v[j,h,:] / Z_i
 *       LSE[h,i] = M_i + ln Z_i
 *   Restricting the softmax to the key set of the query's own segment is the
 *   "restricted softmax over a retained set" of the SparseAttn article, section 3.1:
 *   renormalising the full-row probabilities over the retained set equals a softmax
 *   over only the retained keys.  The retained set here always contains the query
 *   itself, so it is never empty.
 *
 * Separate query and key tables (pfa_oracle_fwd_qk): the varlen call of the same
 * listing takes cu_seqlens_q and cu_seqlens_k (and max_seqlen_q / max_seqlen_k) as
 * separate arguments; with different tables, the queries of segment s are rows
 * [cu_q[s], cu_q[s+1]) of q and attend exactly the keys [cu_k[s], cu_k[s+1]) of k and v.
 * That is the cross-attention of the xxmr.cn editing-network article (section 3.1: Q
 * from the draft features, K and V from the condition or edit sequence; section 4.1:
 * those sequences are much shorter than the query sequence).  A segment with queries but
 * no keys has no softmax; the reading taken here is a zero output and LSE = ln 0 = -inf.
 *
 * Deliberately two-pass (exact row max first, then the sums), not the blocked online
 * recurrence of the GigaPath-Flash page, section 3.2: the oracle must not share the
 * method's algorithm.  All arithmetic is fp64 on the exact input values.
 *
 * Inputs are either fp64 arrays or bf16 bit patterns (uint16, the top half of an
 * IEEE float32); bf16 values are widened exactly.  dv may differ from d (the
 * SparseAttn worked example uses d = 20, dv = 3).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_ENOMEM (-2)

enum { ELEM_F64 = 0, ELEM_BF16 = 1 };

static double widen_bf16(uint16_t bits) {
  uint32_t u = ((uint32_t)bits) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_elem(int kind, const void* base, int64_t idx) {
  if (kind == ELEM_F64) return ((const double*)base)[idx];
  return widen_bf16(((const uint16_t*)base)[idx]);
}

/* Segment that owns token t: the s with cu[s] <= t < cu[s+1] (binary search over a
 * non-decreasing table; zero-length segments are skipped naturally). */
static int owner_segment(const int32_t* cu, int num_seqs, int64_t t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

static int check_table(const int32_t* cu, int num_seqs) {
  if (!cu || num_seqs < 1) return ORACLE_EINVAL;
  if (cu[0] != 0) return ORACLE_EINVAL;
  for (int s = 0; s < num_seqs; ++s)
    if (cu[s + 1] < cu[s]) return ORACLE_EINVAL;
  return ORACLE_OK;
}

/* One (query row, head): writes dv outputs and the LSE.  score[] has room for the
 * segment length. */
static void one_row(int kind, const void* q, const void* k, const void* v, int64_t a, int64_t b,
                    int64_t i, int h, int heads, int d, int dv, double scale, double* score,
                    double* o, double* lse_out) {
  const int64_t qoff = (i * heads + h) * (int64_t)d;
  if (b <= a) { /* no keys: zero output, LSE of an empty sum */
    for (int c = 0; c < dv; ++c) o[c] = 0.0;
    *lse_out = -INFINITY;
    return;
  }
  /* pass 1: scores and their exact maximum */
  double m = -INFINITY;
  for (int64_t j = a; j < b; ++j) {
    const int64_t koff = (j * heads + h) * (int64_t)d;
    double dot = 0.0;
    for (int t = 0; t < d; ++t) dot += load_elem(kind, q, qoff + t) * load_elem(kind, k, koff + t);
    double s = scale * dot;
    score[j - a] = s;
    if (s > m) m = s;
  }
  /* pass 2: normaliser and weighted sum of values */
  double z = 0.0;
  for (int c = 0; c < dv; ++c) o[c] = 0.0;
  for (int64_t j = a; j < b; ++j) {
    double w = exp(score[j - a] - m);
    z += w;
    const int64_t voff = (j * heads + h) * (int64_t)dv;
    for (int c = 0; c < dv; ++c) o[c] += w * load_elem(kind, v, voff + c);
  }
  for (int c = 0; c < dv; ++c) o[c] /= z;
  *lse_out = m + log(z);
}

static int max_segment_length(const int32_t* cu, int num_seqs) {
  int mx = 0;
  for (int s = 0; s < num_seqs; ++s) if (cu[s + 1] - cu[s] > mx) mx = cu[s + 1] - cu[s];
  return mx;
}

/*
 * Full or row-sampled forward with separate query and key tables.
 *   q is [Tq, heads, d], k is [Tk, heads, d], v is [Tk, heads, dv], with
 *   Tq = cu_q[num_seqs] and Tk = cu_k[num_seqs].
 *   rows == NULL: every query token; out is [Tq, heads, dv], lse is [heads, Tq].
 *   rows != NULL: only query tokens rows[0..n_rows); out is [n_rows, heads, dv],
 *                 lse is [heads, n_rows].
 * Returns 0, or ORACLE_EINVAL for a malformed table / row index, ORACLE_ENOMEM.
 */
int pfa_oracle_fwd_qk(int kind, const void* q, const void* k, const void* v, const int32_t* cu_q,
                      const int32_t* cu_k, int num_seqs, int heads, int d, int dv, double scale,
                      const int64_t* rows, int64_t n_rows, double* out, double* lse) {
  if (kind != ELEM_F64 && kind != ELEM_BF16) return ORACLE_EINVAL;
  if (!q || !k || !v || !out || !lse || heads < 1 || d < 1 || dv < 1) return ORACLE_EINVAL;
  if (check_table(cu_q, num_seqs) != ORACLE_OK || check_table(cu_k, num_seqs) != ORACLE_OK)
    return ORACLE_EINVAL;
  const int64_t total = cu_q[num_seqs];
  const int64_t n = rows ? n_rows : total;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= total) return ORACLE_EINVAL;
  const int maxlen = max_segment_length(cu_k, num_seqs);
  int failed = 0;
#pragma omp parallel
  {
    double* score = (double*)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)dv);
    if (!score || !o) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t w = 0; w < n * heads; ++w) {
        const int64_t r = w / heads;
        const int h = (int)(w % heads);
        const int64_t i = rows ? rows[r] : r;
        const int s = owner_segment(cu_q, num_seqs, i);
        double l;
        one_row(kind, q, k, v, cu_k[s], cu_k[s + 1], i, h, heads, d, dv, scale, score, o, &l);
        memcpy(out + (r * heads + h) * (int64_t)dv, o, sizeof(double) * (size_t)dv);
        lse[(int64_t)h * n + r] = l;
      }
    }
    free(score);
    free(o);
  }
  return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* Self-attention over one table: queries and keys share cu (the listing passes the same
 * cu_seqlens for both). */
int pfa_oracle_fwd(int kind, const void* q, const void* k, const void* v, const int32_t* cu,
                   int num_seqs, int heads, int d, int dv, double scale, const int64_t* rows,
                   int64_t n_rows, double* out, double* lse) {
  return pfa_oracle_fwd_qk(kind, q, k, v, cu, cu, num_seqs, heads, d, dv, scale, rows, n_rows,
                           out, lse);
}

/*
 * Debug view of one row of the block-diagonal probability matrix: p_out[j] for every
 * token j in [0, T), zero outside the query's own segment.  Same two-pass arithmetic.
 */
int pfa_oracle_probs(int kind, const void* q, const void* k, const int32_t* cu, int num_seqs,
                     int heads, int d, double scale, int64_t i, int h, double* p_out) {
  if (kind != ELEM_F64 && kind != ELEM_BF16) return ORACLE_EINVAL;
  if (!q || !k || !p_out || heads < 1 || d < 1 || h < 0 || h >= heads) return ORACLE_EINVAL;
  if (check_table(cu, num_seqs) != ORACLE_OK) return ORACLE_EINVAL;
  const int64_t total = cu[num_seqs];
  if (i < 0 || i >= total) return ORACLE_EINVAL;
  const int s = owner_segment(cu, num_seqs, i);
  const int64_t a = cu[s], b = cu[s + 1];
  const int64_t qoff = (i * heads + h) * (int64_t)d;
  for (int64_t j = 0; j < total; ++j) p_out[j] = 0.0;
  double m = -INFINITY;
  for (int64_t j = a; j < b; ++j) {
    const int64_t koff = (j * heads + h) * (int64_t)d;
    double dot = 0.0;
    for (int t = 0; t < d; ++t) dot += load_elem(kind, q, qoff + t) * load_elem(kind, k, koff + t);
    p_out[j] = scale * dot;
    if (p_out[j] > m) m = p_out[j];
  }
  double z = 0.0;
  for (int64_t j = a; j < b; ++j) {
    p_out[j] = exp(p_out[j] - m);
    z += p_out[j];
  }
  for (int64_t j = a; j < b; ++j) p_out[j] /= z;
  return ORACLE_OK;
}

/*
 * Backward of the same definition, for upstream gradient dO of O (one table, as in
 * self-attention).  The pages train with this path (Mage-Flow page: the packing gains are
 * training throughput), but print no gradient formulas; these are the plain chain rule of
 * the forward definition above, written out (fp64, exact input values):
 *     P_ij  = exp(s_ij - LSE_i)                    (softmax over the segment of i)
 *     dV_j  = sum_i P_ij dO_i                      (O_i = sum_j P_ij v_j)
 *     dP_ij = dO_i . v_j
 *     dS_ij = P_ij (dP_ij - sum_t P_it dP_it)      (softmax Jacobian)
 *     dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i   (s_ij = scale q_i.k_j)
 * Rows are processed one query at a time: scores, exact max, normaliser, probabilities,
 * then dP, the row term sum_t P_it dP_it, dS, and the row's contributions to dQ, dK, dV.
 * Outputs are fp64 [T, heads, d]; (segment, head) pairs run in parallel, each owning its
 * key rows of dK / dV.
 */
int pfa_oracle_bwd(int kind, const void* q, const void* k, const void* v, const void* dout,
                   const int32_t* cu, int num_seqs, int heads, int d, double scale, double* dq,
                   double* dk, double* dv) {
  if (kind != ELEM_F64 && kind != ELEM_BF16) return ORACLE_EINVAL;
  if (!q || !k || !v || !dout || !dq || !dk || !dv || heads < 1 || d < 1) return ORACLE_EINVAL;
  if (check_table(cu, num_seqs) != ORACLE_OK) return ORACLE_EINVAL;
  const int64_t total = cu[num_seqs];
  const int maxlen = max_segment_length(cu, num_seqs);
  for (int64_t x = 0; x < total * heads * (int64_t)d; ++x) dq[x] = dk[x] = dv[x] = 0.0;
  int failed = 0;
#pragma omp parallel
  {
    double* p = (double*)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
    if (!p || !dp) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t w = 0; w < (int64_t)num_seqs * heads; ++w) {
        const int s = (int)(w / heads);
        const int h = (int)(w % heads);
        const int64_t a = cu[s], b = cu[s + 1];
        for (int64_t i = a; i < b; ++i) {
          const int64_t qi = (i * heads + h) * (int64_t)d;
          /* probabilities of row i (two passes: exact max, then normaliser) */
          double m = -INFINITY;
          for (int64_t j = a; j < b; ++j) {
            const int64_t kj = (j * heads + h) * (int64_t)d;
            double dot = 0.0;
            for (int t = 0; t < d; ++t) dot += load_elem(kind, q, qi + t) * load_elem(kind, k, kj + t);
            p[j - a] = scale * dot;
            if (p[j - a] > m) m = p[j - a];
          }
          double z = 0.0;
          for (int64_t j = a; j < b; ++j) {
            p[j - a] = exp(p[j - a] - m);
            z += p[j - a];
          }
          for (int64_t j = a; j < b; ++j) p[j - a] /= z;
          /* dP_ij = dO_i . v_j and the row term sum_j P_ij dP_ij */
          double rowterm = 0.0;
          for (int64_t j = a; j < b; ++j) {
            const int64_t vj = (j * heads + h) * (int64_t)d;
            double dot = 0.0;
            for (int t = 0; t < d; ++t) dot += load_elem(kind, dout, qi + t) * load_elem(kind, v, vj + t);
            dp[j - a] = dot;
            rowterm += p[j - a] * dot;
          }
          /* dS, then this row's contributions */
          for (int64_t j = a; j < b; ++j) {
            const double ds = p[j - a] * (dp[j - a] - rowterm);
            const int64_t kj = (j * heads + h) * (int64_t)d;
            for (int t = 0; t < d; ++t) {
              dq[qi + t] += scale * ds * load_elem(kind, k, kj + t);
              dk[kj + t] += scale * ds * load_elem(kind, q, qi + t);
              dv[kj + t] += p[j - a] * load_elem(kind, dout, qi + t);
            }
          }
        }
      }
    }
    free(p);
    free(dp);
  }
  return failed ? ORACLE_ENOMEM : ORACLE_OK;
}

/* Threads an OpenMP parallel region of the oracle uses (1 without OpenMP). */
int pfa_oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
