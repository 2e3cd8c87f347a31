/*
 * Exact-attention oracle: plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can compare the HIP kernels against an
 * obviously correct definition.  It shares no code, header or constant with
 * the GPU library.
 *
 * What it computes (FlashAttention pages):
 *   - "FlashAttention：让精确注意力服从内存层次" (wineandchord.com), opening
 *     formula softmax(Q K^T / sqrt(d)) V and section "前序瓶颈" (S = QK^T,
 *     P = softmax(S), O = PV): the dense definition, written row by row.
 *   - Same page, section "Online softmax": per-tile statistics
 *     (m, l, u) and their pairwise merge; used by oracle_fwd_blockwise.
 *   - "FlashAttention" paper story (ai.tomabc.com), conceptual forward
 *     pseudocode: Q row-blocks in the outer loop, K/V column-blocks in the
 *     inner loop; the blockwise variant follows that loop order.
 *   - Same story, backward paragraph: only the softmax statistics are kept
 *     and P is recomputed.  The pages drop the gradient formulas, so the
 *     backward here is the textbook gradient of O = softmax(scale*QK^T) V.
 *
 * Conventions (readings where the pages are silent):
 *   - Layout: dense row-major [B, H, N, d]; K and V have Hkv heads, query
 *     head h reads kv head h / (Hq / Hkv).
 *   - Causal: key j is visible to query i iff j <= i (top-left alignment).
 *   - A row with no visible key has O = 0 and LSE = -inf.
 *   - LSE is the natural-log logsumexp of the scaled scores: m + ln(l).
 *   - Inputs are fp64 arrays; callers upcast bf16/fp32 values exactly.
 *
 * All arithmetic is fp64.  Build with -O2 -ffp-contract=off, without
 * -ffast-math, so every sum is evaluated in source order.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEM 2

/* Threads an OpenMP parallel region of this library will use. */
int oracle_threads(void) { return omp_get_max_threads(); }

static int check_args(int B, int Hq, int Hkv, int Nq, int Nk, int dk, int dv) {
  if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0 || dk < 1 || dv < 1)
    return ORACLE_BAD_ARG;
  if (Hq % Hkv != 0) return ORACLE_BAD_ARG;
  return ORACLE_OK;
}

/* Number of keys visible to query row i: all of them, or with the causal
 * mask keys j <= i + off (off = 0: top-left alignment; off = Nk - Nq:
 * bottom-right alignment, the last query sees every key). */
static int64_t visible_keys_off(int64_t i, int64_t Nk, int causal, int64_t off) {
  if (!causal) return Nk;
  const int64_t n = i + 1 + off;
  if (n < 0) return 0;
  return (n < Nk) ? n : Nk;
}

static int64_t visible_keys(int64_t i, int64_t Nk, int causal) {
  return visible_keys_off(i, Nk, causal, 0);
}

/* Plain dot product in index order. */
static double dot(const double* a, const double* b, int n) {
  double s = 0.0;
  for (int c = 0; c < n; ++c) s += a[c] * b[c];
  return s;
}

/*
 * One output row of the dense definition: s_j = scale q.k_j over the visible
 * keys, m = max s_j, l = sum exp(s_j - m), o = sum exp(s_j - m) v_j / l,
 * lse = m + ln l.  `scores` is scratch of Nk doubles (one row, never N x N).
 */
static void dense_row(const double* qi, const double* Kh, const double* Vh,
                      int64_t nvis, int dk, int dv, double scale,
                      double* scores, double* orow, double* lse) {
  for (int c = 0; c < dv; ++c) orow[c] = 0.0;
  if (nvis == 0) {
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (int64_t j = 0; j < nvis; ++j) {
    scores[j] = scale * dot(qi, Kh + j * dk, dk);
    if (scores[j] > m) m = scores[j];
  }
  double l = 0.0;
  for (int64_t j = 0; j < nvis; ++j) {
    double w = exp(scores[j] - m);
    l += w;
    const double* vj = Vh + j * dv;
    for (int c = 0; c < dv; ++c) orow[c] += w * vj[c];
  }
  for (int c = 0; c < dv; ++c) orow[c] /= l;
  *lse = m + log(l);
}

/*
 * Dense forward.  q [B,Hq,Nq,dk], k [B,Hkv,Nk,dk], v [B,Hkv,Nk,dv];
 * o [B,Hq,Nq,dv], lse [B,Hq,Nq].
 */
int oracle_fwd(const double* q, const double* k, const double* v, double* o,
               double* lse, int B, int Hq, int Hkv, int Nq, int Nk, int dk,
               int dv, int causal, double scale) {
  int rc = check_args(B, Hq, Hkv, Nq, Nk, dk, dv);
  if (rc) return rc;
  const int64_t rows = (int64_t)B * Hq * Nq;
  const int group = Hq / Hkv;
  int bad = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (Nk > 0 ? Nk : 1));
    if (!scores) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < rows; ++r) {
        const int64_t i = r % Nq;
        const int64_t h = (r / Nq) % Hq;
        const int64_t b = r / ((int64_t)Nq * Hq);
        const int64_t g = h / group;
        const double* Kh = k + (b * Hkv + g) * (int64_t)Nk * dk;
        const double* Vh = v + (b * Hkv + g) * (int64_t)Nk * dv;
        dense_row(q + r * dk, Kh, Vh, visible_keys(i, Nk, causal), dk, dv,
                  scale, scores, o + r * dv, lse + r);
      }
      free(scores);
    }
  }
  return bad ? ORACLE_NO_MEM : ORACLE_OK;
}

/*
 * Dense forward with the causal mask aligned to the bottom-right corner:
 * query i (of Nq) sees keys j <= i + (Nk - Nq), as when the Nq queries are
 * the last Nq positions of a sequence of Nk keys (decode and append).  For
 * Nq == Nk this is oracle_fwd.  Rows that see no key get O = 0, LSE = -inf.
 */
int oracle_fwd_bottom_right(const double* q, const double* k, const double* v, double* o,
                            double* lse, int B, int Hq, int Hkv, int Nq, int Nk, int dk,
                            int dv, int causal, double scale) {
  int rc = check_args(B, Hq, Hkv, Nq, Nk, dk, dv);
  if (rc) return rc;
  const int64_t rows = (int64_t)B * Hq * Nq;
  const int group = Hq / Hkv;
  const int64_t off = (int64_t)Nk - Nq;
  int bad = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (Nk > 0 ? Nk : 1));
    if (!scores) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < rows; ++r) {
        const int64_t i = r % Nq;
        const int64_t h = (r / Nq) % Hq;
        const int64_t b = r / ((int64_t)Nq * Hq);
        const int64_t g = h / group;
        const double* Kh = k + (b * Hkv + g) * (int64_t)Nk * dk;
        const double* Vh = v + (b * Hkv + g) * (int64_t)Nk * dv;
        dense_row(q + r * dk, Kh, Vh, visible_keys_off(i, Nk, causal, off), dk, dv, scale,
                  scores, o + r * dv, lse + r);
      }
      free(scores);
    }
  }
  return bad ? ORACLE_NO_MEM : ORACLE_OK;
}

/*
 * Block-sparse forward ("FlashAttention" paper story, block-sparse
 * paragraph: a 0/1 mask over the grid of (Br rows) x (Bc keys) score blocks,
 * whose zero blocks are never computed).  Square problem, N queries and N
 * keys.  Query i of head h sees key j iff
 *     mask[hm][i / bm][j / bn] != 0   and   (causal == 0 or j <= i),
 * with hm = h when mask_heads == Hq and hm = 0 when mask_heads == 1; the
 * mask is row-major [mask_heads][ceil(N/bm)][ceil(N/bn)] bytes and is shared
 * by every batch.  Each row's visible keys are gathered in index order and
 * the dense softmax is taken over them (dense_row), so the result is the
 * definition itself.  A row that sees no key gets O = 0 and LSE = -inf.
 */
int oracle_fwd_blockmask(const double* q, const double* k, const double* v, double* o,
                         double* lse, const uint8_t* mask, int mask_heads, int bm, int bn,
                         int B, int Hq, int Hkv, int N, int dk, int dv, int causal,
                         double scale) {
  int rc = check_args(B, Hq, Hkv, N, N, dk, dv);
  if (rc) return rc;
  if (!(mask_heads == 1 || mask_heads == Hq) || bm < 1 || bn < 1) return ORACLE_BAD_ARG;
  const int64_t nbq = ((int64_t)N + bm - 1) / bm, nbk = ((int64_t)N + bn - 1) / bn;
  const int64_t rows = (int64_t)B * Hq * N;
  const int group = Hq / Hkv;
  int bad = 0;
#pragma omp parallel
  {
    const int64_t n1 = N > 0 ? N : 1;
    double* scores = (double*)malloc(sizeof(double) * n1);
    double* kg = (double*)malloc(sizeof(double) * n1 * dk);
    double* vg = (double*)malloc(sizeof(double) * n1 * dv);
    if (!scores || !kg || !vg) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < rows; ++r) {
        const int64_t i = r % N;
        const int64_t h = (r / N) % Hq;
        const int64_t b = r / ((int64_t)N * Hq);
        const int64_t g = h / group;
        const int64_t hm = (mask_heads == 1) ? 0 : h;
        const uint8_t* mrow = mask + (hm * nbq + i / bm) * nbk;
        const double* Kh = k + (b * Hkv + g) * (int64_t)N * dk;
        const double* Vh = v + (b * Hkv + g) * (int64_t)N * dv;
        int64_t nvis = 0;
        for (int64_t j = 0; j < N; ++j) {
          if (!mrow[j / bn]) continue;
          if (causal && j > i) continue;
          memcpy(kg + nvis * dk, Kh + j * dk, sizeof(double) * dk);
          memcpy(vg + nvis * dv, Vh + j * dv, sizeof(double) * dv);
          ++nvis;
        }
        dense_row(q + r * dk, kg, vg, nvis, dk, dv, scale, scores, o + r * dv, lse + r);
      }
    }
    free(scores);
    free(kg);
    free(vg);
  }
  return bad ? ORACLE_NO_MEM : ORACLE_OK;
}

/*
 * Variable-length (packed) forward: nseq sequences laid end to end along the
 * token axis, sequence s occupying tokens [cu[s], cu[s+1]) of T.  Each token
 * attends only to keys of its own sequence (a document mask), with the
 * causal rule inside the sequence.  q [Hq, T, dk], k [Hkv, T, dk],
 * v [Hkv, T, dv]; o [Hq, T, dv], lse [Hq, T].  cu must be non-decreasing from
 * 0 to T.  Every (sequence, head) is one dense problem (dense_row on that
 * sequence's keys); an empty sequence has no rows.
 */
int oracle_fwd_varlen(const double* q, const double* k, const double* v, double* o, double* lse,
                      const int32_t* cu, int nseq, int Hq, int Hkv, int T, int dk, int dv,
                      int causal, double scale) {
  int rc = check_args(1, Hq, Hkv, T, T, dk, dv);
  if (rc) return rc;
  if (nseq < 0 || (nseq == 0 && T != 0) || (nseq > 0 && (cu[0] != 0 || cu[nseq] != T)))
    return ORACLE_BAD_ARG;
  for (int s = 0; s < nseq; ++s)
    if (cu[s + 1] < cu[s]) return ORACLE_BAD_ARG;
  const int group = Hq / Hkv;
  const int64_t rows = (int64_t)Hq * T;
  int bad = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (T > 0 ? T : 1));
    if (!scores) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < rows; ++r) {
        const int64_t h = r / T;
        const int64_t t = r % T;
        int s = 0;
        while (cu[s + 1] <= t) ++s;  /* sequence holding token t */
        const int64_t start = cu[s], len = (int64_t)cu[s + 1] - cu[s];
        const int64_t i = t - start;  /* position inside the sequence */
        const int64_t g = h / group;
        const double* Kh = k + (g * T + start) * dk;
        const double* Vh = v + (g * T + start) * dv;
        dense_row(q + r * dk, Kh, Vh, visible_keys(i, len, causal), dk, dv, scale, scores,
                  o + r * dv, lse + r);
      }
      free(scores);
    }
  }
  return bad ? ORACLE_NO_MEM : ORACLE_OK;
}

/*
 * Dense forward on a chosen subset of rows.  rows[t] is the flat row index
 * (b * Hq + h) * Nq + i; o is [nrows, dv], lse is [nrows].  Used to check
 * sampled rows of large problems one by one.
 */
int oracle_fwd_rows(const double* q, const double* k, const double* v,
                    const int64_t* rows, int64_t nrows, double* o, double* lse,
                    int B, int Hq, int Hkv, int Nq, int Nk, int dk, int dv,
                    int causal, double scale) {
  int rc = check_args(B, Hq, Hkv, Nq, Nk, dk, dv);
  if (rc) return rc;
  const int64_t total = (int64_t)B * Hq * Nq;
  for (int64_t t = 0; t < nrows; ++t)
    if (rows[t] < 0 || rows[t] >= total) return ORACLE_BAD_ARG;
  const int group = Hq / Hkv;
  int bad = 0;
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (Nk > 0 ? Nk : 1));
    if (!scores) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t t = 0; t < nrows; ++t) {
        const int64_t r = rows[t];
        const int64_t i = r % Nq;
        const int64_t h = (r / Nq) % Hq;
        const int64_t b = r / ((int64_t)Nq * Hq);
        const int64_t g = h / group;
        const double* Kh = k + (b * Hkv + g) * (int64_t)Nk * dk;
        const double* Vh = v + (b * Hkv + g) * (int64_t)Nk * dv;
        dense_row(q + r * dk, Kh, Vh, visible_keys(i, Nk, causal), dk, dv,
                  scale, scores, o + t * dv, lse + t);
      }
      free(scores);
    }
  }
  return bad ? ORACLE_NO_MEM : ORACLE_OK;
}

/*
 * Blockwise forward with the online (m, l, u) merge.
 *
 * Outer loop over query blocks of br rows, inner loop over key/value blocks
 * of bc keys (the tiling of the forward pseudocode; tail blocks are partial).
 * For every row and key block the tile statistics are formed from the
 * visible keys of that block:
 *   m_b = max s,  l_b = sum exp(s - m_b),  u_b = sum exp(s - m_b) v,
 * and merged into the running state (m_a, l_a, u_a):
 *   m = max(m_a, m_b),  l = e^{m_a - m} l_a + e^{m_b - m} l_b,
 *   u = e^{m_a - m} u_a + e^{m_b - m} u_b.
 * A block with no visible key for a row leaves that row's state unchanged
 * (the empty state is the identity of the merge).  At the end o = u / l and
 * lse = m + ln l.
 */
int oracle_fwd_blockwise(const double* q, const double* k, const double* v,
                         double* o, double* lse, int B, int Hq, int Hkv, int Nq,
                         int Nk, int dk, int dv, int causal, double scale,
                         int br, int bc) {
  int rc = check_args(B, Hq, Hkv, Nq, Nk, dk, dv);
  if (rc) return rc;
  if (br < 1 || bc < 1) return ORACLE_BAD_ARG;
  const int group = Hq / Hkv;
  const int64_t nqb = (Nq + br - 1) / br;
  const int64_t units = (int64_t)B * Hq * nqb;
  int bad = 0;
#pragma omp parallel
  {
    double* m_run = (double*)malloc(sizeof(double) * br);
    double* l_run = (double*)malloc(sizeof(double) * br);
    double* u_run = (double*)malloc(sizeof(double) * (size_t)br * dv);
    double* s_blk = (double*)malloc(sizeof(double) * bc);
    double* u_blk = (double*)malloc(sizeof(double) * dv);
    if (!m_run || !l_run || !u_run || !s_blk || !u_blk) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t unit = 0; unit < units; ++unit) {
        const int64_t qb = unit % nqb;
        const int64_t h = (unit / nqb) % Hq;
        const int64_t b = unit / (nqb * Hq);
        const int64_t g = h / group;
        const double* Qh = q + (b * Hq + h) * (int64_t)Nq * dk;
        const double* Kh = k + (b * Hkv + g) * (int64_t)Nk * dk;
        const double* Vh = v + (b * Hkv + g) * (int64_t)Nk * dv;
        double* Oh = o + (b * Hq + h) * (int64_t)Nq * dv;
        double* Lh = lse + (b * Hq + h) * (int64_t)Nq;
        const int64_t i0 = qb * br;
        const int64_t i1 = (i0 + br < Nq) ? i0 + br : Nq;
        for (int64_t i = i0; i < i1; ++i) {
          m_run[i - i0] = -INFINITY;
          l_run[i - i0] = 0.0;
          for (int c = 0; c < dv; ++c) u_run[(i - i0) * dv + c] = 0.0;
        }
        for (int64_t j0 = 0; j0 < Nk; j0 += bc) {
          const int64_t j1 = (j0 + bc < Nk) ? j0 + bc : Nk;
          for (int64_t i = i0; i < i1; ++i) {
            const int64_t nvis = visible_keys(i, Nk, causal);
            const int64_t jend = (j1 < nvis) ? j1 : nvis;
            if (jend <= j0) continue; /* no visible key: identity merge */
            const double* qi = Qh + i * dk;
            double m_b = -INFINITY;
            for (int64_t j = j0; j < jend; ++j) {
              s_blk[j - j0] = scale * dot(qi, Kh + j * dk, dk);
              if (s_blk[j - j0] > m_b) m_b = s_blk[j - j0];
            }
            double l_b = 0.0;
            for (int c = 0; c < dv; ++c) u_blk[c] = 0.0;
            for (int64_t j = j0; j < jend; ++j) {
              const double w = exp(s_blk[j - j0] - m_b);
              l_b += w;
              for (int c = 0; c < dv; ++c) u_blk[c] += w * Vh[j * dv + c];
            }
            double* ua = u_run + (i - i0) * dv;
            const double m_a = m_run[i - i0];
            if (l_run[i - i0] == 0.0 && m_a == -INFINITY) {
              /* running state empty: the merge returns the block state */
              m_run[i - i0] = m_b;
              l_run[i - i0] = l_b;
              for (int c = 0; c < dv; ++c) ua[c] = u_blk[c];
              continue;
            }
            const double m_new = (m_a > m_b) ? m_a : m_b;
            const double fa = exp(m_a - m_new);
            const double fb = exp(m_b - m_new);
            l_run[i - i0] = fa * l_run[i - i0] + fb * l_b;
            for (int c = 0; c < dv; ++c) ua[c] = fa * ua[c] + fb * u_blk[c];
            m_run[i - i0] = m_new;
          }
        }
        for (int64_t i = i0; i < i1; ++i) {
          double* orow = Oh + i * dv;
          if (l_run[i - i0] == 0.0) {
            for (int c = 0; c < dv; ++c) orow[c] = 0.0;
            Lh[i] = -INFINITY;
          } else {
            for (int c = 0; c < dv; ++c)
              orow[c] = u_run[(i - i0) * dv + c] / l_run[i - i0];
            Lh[i] = m_run[i - i0] + log(l_run[i - i0]);
          }
        }
      }
    }
    free(m_run);
    free(l_run);
    free(u_run);
    free(s_blk);
    free(u_blk);
  }
  return bad ? ORACLE_NO_MEM : ORACLE_OK;
}

/*
 * Backward: textbook gradient of O = softmax(scale * Q K^T [+ causal]) V
 * for an upstream gradient dO, with P recomputed from the oracle's own
 * statistics (never taken from the GPU):
 *   P_ij  = exp(s_ij - LSE_i) on visible keys, 0 elsewhere
 *   dP_ij = dO_i . v_j
 *   D_i   = dO_i . O_i
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i  = scale sum_j dS_ij k_j
 *   dK_j  = scale sum_{h in group} sum_i dS_ij q_i
 *   dV_j  = sum_{h in group} sum_i P_ij dO_i
 * Three passes: row statistics (LSE, O, D), then dQ row by row, then dK/dV
 * key by key.  lse_out/o_out/dsum_out (may be NULL) receive the forward
 * statistics [B,Hq,Nq], [B,Hq,Nq,dv], [B,Hq,Nq].
 */
int oracle_bwd(const double* q, const double* k, const double* v,
               const double* dout, double* dq, double* dk_out, double* dv_out,
               double* lse_out, double* o_out, double* dsum_out, int B, int Hq,
               int Hkv, int Nq, int Nk, int dk, int dv, int causal,
               double scale) {
  int rc = check_args(B, Hq, Hkv, Nq, Nk, dk, dv);
  if (rc) return rc;
  const int group = Hq / Hkv;
  const int64_t rows = (int64_t)B * Hq * Nq;
  double* lse = (double*)malloc(sizeof(double) * (rows > 0 ? rows : 1));
  double* obuf = (double*)malloc(sizeof(double) * (rows > 0 ? rows : 1) * dv);
  double* dsum = (double*)malloc(sizeof(double) * (rows > 0 ? rows : 1));
  if (!lse || !obuf || !dsum) {
    free(lse);
    free(obuf);
    free(dsum);
    return ORACLE_NO_MEM;
  }
  int bad = 0;

  /* Pass 1: forward statistics of every row, and D_i = dO_i . O_i. */
#pragma omp parallel
  {
    double* scores = (double*)malloc(sizeof(double) * (Nk > 0 ? Nk : 1));
    if (!scores) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t r = 0; r < rows; ++r) {
        const int64_t i = r % Nq;
        const int64_t h = (r / Nq) % Hq;
        const int64_t b = r / ((int64_t)Nq * Hq);
        const int64_t g = h / group;
        const double* Kh = k + (b * Hkv + g) * (int64_t)Nk * dk;
        const double* Vh = v + (b * Hkv + g) * (int64_t)Nk * dv;
        dense_row(q + r * dk, Kh, Vh, visible_keys(i, Nk, causal), dk, dv,
                  scale, scores, obuf + r * dv, lse + r);
        dsum[r] = dot(dout + r * dv, obuf + r * dv, dv);
      }
      free(scores);
    }
  }

  /* Pass 2: dQ_i = scale sum_j P_ij (dP_ij - D_i) k_j. */
  if (!bad) {
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t r = 0; r < rows; ++r) {
      const int64_t i = r % Nq;
      const int64_t h = (r / Nq) % Hq;
      const int64_t b = r / ((int64_t)Nq * Hq);
      const int64_t g = h / group;
      const double* Kh = k + (b * Hkv + g) * (int64_t)Nk * dk;
      const double* Vh = v + (b * Hkv + g) * (int64_t)Nk * dv;
      const double* qi = q + r * dk;
      const double* doi = dout + r * dv;
      double* dqi = dq + r * dk;
      for (int c = 0; c < dk; ++c) dqi[c] = 0.0;
      const int64_t nvis = visible_keys(i, Nk, causal);
      for (int64_t j = 0; j < nvis; ++j) {
        const double p = exp(scale * dot(qi, Kh + j * dk, dk) - lse[r]);
        const double dp = dot(doi, Vh + j * dv, dv);
        const double ds = p * (dp - dsum[r]);
        for (int c = 0; c < dk; ++c) dqi[c] += ds * Kh[j * dk + c];
      }
      for (int c = 0; c < dk; ++c) dqi[c] *= scale;
    }
  }

  /* Pass 3: dK_j, dV_j, summed over the query heads of the kv group. */
  if (!bad) {
    const int64_t cols = (int64_t)B * Hkv * Nk;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t cidx = 0; cidx < cols; ++cidx) {
      const int64_t j = cidx % Nk;
      const int64_t g = (cidx / Nk) % Hkv;
      const int64_t b = cidx / ((int64_t)Nk * Hkv);
      const double* kj = k + cidx * dk;
      const double* vj = v + cidx * dv;
      double* dkj = dk_out + cidx * dk;
      double* dvj = dv_out + cidx * dv;
      for (int c = 0; c < dk; ++c) dkj[c] = 0.0;
      for (int c = 0; c < dv; ++c) dvj[c] = 0.0;
      for (int64_t hh = 0; hh < group; ++hh) {
        const int64_t h = g * group + hh;
        const int64_t rbase = (b * Hq + h) * (int64_t)Nq;
        for (int64_t i = 0; i < Nq; ++i) {
          if (j >= visible_keys(i, Nk, causal)) continue;
          const int64_t r = rbase + i;
          const double* qi = q + r * dk;
          const double* doi = dout + r * dv;
          const double p = exp(scale * dot(qi, kj, dk) - lse[r]);
          const double dp = dot(doi, vj, dv);
          const double ds = p * (dp - dsum[r]);
          for (int c = 0; c < dv; ++c) dvj[c] += p * doi[c];
          for (int c = 0; c < dk; ++c) dkj[c] += ds * qi[c];
        }
      }
      for (int c = 0; c < dk; ++c) dkj[c] *= scale;
    }
  }

  if (!bad) {
    if (lse_out) memcpy(lse_out, lse, sizeof(double) * rows);
    if (o_out) memcpy(o_out, obuf, sizeof(double) * rows * dv);
    if (dsum_out) memcpy(dsum_out, dsum, sizeof(double) * rows);
  }
  free(lse);
  free(obuf);
  free(dsum);
  return bad ? ORACLE_NO_MEM : ORACLE_OK;
}

/*
 * Backward restricted to whole (b, kv-group) slices: the gradients of every
 * row and key of the listed (b, g) pairs, for sampled checks of large
 * problems.  slices[t] = b * Hkv + g.  Outputs are packed per slice:
 * dq [nslices, group, Nq, dk], dk/dv [nslices, Nk, dk|dv].
 */
int oracle_bwd_slices(const double* q, const double* k, const double* v,
                      const double* dout, const int64_t* slices,
                      int64_t nslices, double* dq, double* dk_out,
                      double* dv_out, int B, int Hq, int Hkv, int Nq, int Nk,
                      int dk, int dv, int causal, double scale) {
  int rc = check_args(B, Hq, Hkv, Nq, Nk, dk, dv);
  if (rc) return rc;
  const int group = Hq / Hkv;
  for (int64_t t = 0; t < nslices; ++t) {
    const int64_t s = slices[t];
    if (s < 0 || s >= (int64_t)B * Hkv) return ORACLE_BAD_ARG;
    const int64_t b = s / Hkv, g = s % Hkv;
    /* One slice is a B=1, Hq=group, Hkv=1 problem. */
    const double* qs = q + (b * Hq + g * group) * (int64_t)Nq * dk;
    const double* dos = dout + (b * Hq + g * group) * (int64_t)Nq * dv;
    const double* ks = k + (b * Hkv + g) * (int64_t)Nk * dk;
    const double* vs = v + (b * Hkv + g) * (int64_t)Nk * dv;
    rc = oracle_bwd(qs, ks, vs, dos, dq + t * (int64_t)group * Nq * dk,
                    dk_out + t * (int64_t)Nk * dk, dv_out + t * (int64_t)Nk * dv,
                    NULL, NULL, NULL, 1, group, 1, Nq, Nk, dk, dv, causal,
                    scale);
    if (rc) return rc;
  }
  return ORACLE_OK;
}
