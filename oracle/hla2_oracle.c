/*
 * hla2_oracle.c -- plain, slow fp64 CPU oracle for strictly causal second-order
 * Higher-order Linear Attention (HLA2).  TEST INFRASTRUCTURE ONLY: nothing on the
 * product path may link, load or call this file; only the tests, the smoke check
 * and the benchmark's CPU-baseline leg do.  It shares no code, header or table
 * with the GPU library.
 *
 * Sources (web pages about arXiv 2510.27258):
 *   [SUM] "Technische Samenvatting: Hogere-orde Lineaire Aandacht (HLA)",
 *         gist.science -- the technical summary; primary authority.
 *   [ABS] "Высокоуровневое линейное внимание", chatpaper.ai -- the abstract.
 *
 * Everything works on ONE head: q, k are n x d row-major, v is n x dv row-major,
 * tokens t = 0..n-1.  All arithmetic is IEEE double.
 *
 * What is computed (readings of the pages, stated once here):
 *  - Prefix summaries [SUM §1 "Onderhoud van de toestand"]: key moment
 *    S_t = sum_{i<=t} k_i k_i^T (d x d), query-value accumulator
 *    C_t = sum_{i<=t} q_i v_i^T (d x dv), query mass m_t = sum_{i<=t} q_i (d).
 *  - Cross summaries G_t (d x dv), h_t (d) [SUM §1 "Strenge causaliteit"] remove
 *    from the naive product S_t C_t the pairs (i, j) where the query index j
 *    comes BEFORE the key index i.  The pages name G and h but print no update;
 *    the update used here, G_t = G_{t-1} + k_t (k_t^T C_{t-1}), is the unique one
 *    that collects exactly those pairs, because at step t the new key k_t pairs
 *    with every earlier query j <= t-1.  h likewise with m_{t-1}.
 *  - Output [SUM §1 "Outputformulering"]: num_t = q_t^T (S_t C_t - G_t).
 *    Expanding, num_t = sum_{j<=t} sum_{i<=j} (q_t.k_i)(q_j.k_i) v_j, i.e. row t
 *    of L o (A A^T) V with A = L o (Q K^T) and L the lower triangle including
 *    the diagonal; so the output at t depends on tokens j <= t only
 *    [SUM "Resultaten en claims", causality bullet].
 *  - Ratio normalisation [SUM §1 "Normalisatie"]: the masked denominator built
 *    from the same kind of summaries, den_t = q_t^T (S_t m_t - h_t) = the row sum
 *    of the same masked matrix; o_t = num_t / den_t with plain IEEE division
 *    (the pages give no epsilon).
 *  - Exponential decay [SUM "Belangrijkste bijdragen" 2 names decayed variants
 *    but prints no formula].  Reading: every first-order summary decays by
 *    gamma per token, S <- gamma S + k k^T, C <- gamma C + q v^T,
 *    m <- gamma m + q.  Keeping o_t = q_t^T (S_t C_t - G_t) exact then forces
 *    G <- gamma^2 G + gamma k (k^T C_{t-1}) (and h likewise), and the pair
 *    (i <= j <= t) carries weight gamma^{(t-i)+(t-j)}.  gamma = 1 is no decay.
 *  - Chunk-parallel form [SUM §4 "Associatieve operatoren", "Scan-equivalentie"]:
 *    a segment of tokens is summarised by (Gamma, S, C, m, G, h), Gamma =
 *    gamma^{len}; two consecutive segments A then B concatenate by the
 *    semidirect-product rule
 *      S = Gamma_B S_A + S_B,  C = Gamma_B C_A + C_B,  m = Gamma_B m_A + m_B,
 *      G = Gamma_B^2 G_A + G_B + Gamma_B S_B C_A,
 *      h = Gamma_B^2 h_A + h_B + Gamma_B S_B m_A,   Gamma = Gamma_A Gamma_B,
 *    whose cross term S_B C_A is the one [SUM §4] names.  An exclusive Blelloch
 *    scan over chunk summaries gives every chunk its incoming state, from which
 *    the chunk's outputs follow; the result equals the serial recurrence.
 *
 * State block layout (one head), shared by decode and the final-state outputs:
 *   S[d*d] | C[d*dv] | m[d] | G[d*dv] | h[d], all row-major.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

#define HLA2_ORACLE_ABI_VERSION 1

int hla2_oracle_abi_version(void) { return HLA2_ORACLE_ABI_VERSION; }

long hla2_oracle_state_len(int d, int dv) { return (long)d * d + 2L * d * dv + 2L * d; }

/* Summary block layout used by the chunked path and the combine:
 *   Gamma[1] | S[d*d] | C[d*dv] | m[d] | G[d*dv] | h[d]. */
long hla2_oracle_summary_len(int d, int dv) { return 1 + hla2_oracle_state_len(d, dv); }

/* ---------------------------------------------------------------------------
 * One streaming step [SUM §1; ABS: constant-size state, per-token update].
 * state (in/out) is the layout above; q[d], k[d], v[dv] are token t.
 * Writes num[dv] and *den for token t; with num == NULL only the state is
 * updated (the readout does not touch it).
 * Order: the cross summaries use C_{t-1}, m_{t-1}; then S, C, m take token t;
 * then the readout uses the updated state.
 * ------------------------------------------------------------------------- */
void hla2_oracle_step(int d, int dv, double gamma, double *state,
                      const double *q, const double *k, const double *v,
                      double *num, double *den) {
  double *S = state;
  double *C = S + (long)d * d;
  double *m = C + (long)d * dv;
  double *G = m + d;
  double *h = G + (long)d * dv;
  double g2 = gamma * gamma;
  int a, b, c;

  /* kC = k^T C_{t-1} (dv), km = k^T m_{t-1} */
  double *kC = (double *)calloc((size_t)dv, sizeof(double));
  double km = 0.0;
  for (a = 0; a < d; ++a) {
    for (c = 0; c < dv; ++c) kC[c] += k[a] * C[(long)a * dv + c];
    km += k[a] * m[a];
  }
  /* cross summaries */
  for (a = 0; a < d; ++a) {
    for (c = 0; c < dv; ++c)
      G[(long)a * dv + c] = g2 * G[(long)a * dv + c] + gamma * k[a] * kC[c];
    h[a] = g2 * h[a] + gamma * k[a] * km;
  }
  /* first-order summaries */
  for (a = 0; a < d; ++a) {
    for (b = 0; b < d; ++b) S[(long)a * d + b] = gamma * S[(long)a * d + b] + k[a] * k[b];
    for (c = 0; c < dv; ++c) C[(long)a * dv + c] = gamma * C[(long)a * dv + c] + q[a] * v[c];
    m[a] = gamma * m[a] + q[a];
  }
  if (!num) {
    free(kC);
    return;
  }
  /* readout: p = S^T q (S is symmetric), num = p^T C - q^T G, den = p.m - q.h */
  double *p = (double *)calloc((size_t)d, sizeof(double));
  for (a = 0; a < d; ++a)
    for (b = 0; b < d; ++b) p[b] += q[a] * S[(long)a * d + b];
  for (c = 0; c < dv; ++c) {
    double s = 0.0;
    for (a = 0; a < d; ++a) s += p[a] * C[(long)a * dv + c] - q[a] * G[(long)a * dv + c];
    num[c] = s;
  }
  double sd = 0.0;
  for (a = 0; a < d; ++a) sd += p[a] * m[a] - q[a] * h[a];
  *den = sd;
  free(p);
  free(kC);
}

/* ---------------------------------------------------------------------------
 * Serial recurrence over a whole sequence (one head).
 * state: nullable.  If given, it is the state before token 0 and receives the
 * state after token n-1; if NULL the run starts from the all-zero state.
 * num: n*dv, den: n (nullable).  num == NULL skips the readouts (den is then
 * ignored): only the state advances, as when a prefix is absorbed.
 * ------------------------------------------------------------------------- */
int hla2_oracle_serial(int n, int d, int dv, double gamma,
                       const double *q, const double *k, const double *v,
                       double *num, double *den, double *state) {
  if (n < 0 || d <= 0 || dv <= 0) return -1;
  long L = hla2_oracle_state_len(d, dv);
  double *st = state ? state : (double *)calloc((size_t)L, sizeof(double));
  double dummy;
  int t;
  for (t = 0; t < n; ++t)
    hla2_oracle_step(d, dv, gamma, st, q + (long)t * d, k + (long)t * d, v + (long)t * dv,
                     num ? num + (long)t * dv : NULL, den ? den + t : &dummy);
  if (!state) free(st);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Serial recurrence that also reports, per token, the Euclidean norm of the
 * denominator state u_t = S_t m_t - h_t (so den_t = q_t . u_t).  The ratio
 * q_t . u_t / (|q_t| |u_t|) measures how well-conditioned the ratio-normalised
 * output is at t [SUM §1 "Normalisatie"]: where it is tiny, den_t is a
 * cancellation of large terms and num_t / den_t amplifies any rounding.
 * Arguments as hla2_oracle_serial plus unorm (n).
 * ------------------------------------------------------------------------- */
int hla2_oracle_serial_unorm(int n, int d, int dv, double gamma,
                             const double *q, const double *k, const double *v,
                             double *num, double *den, double *unorm, double *state) {
  if (n < 0 || d <= 0 || dv <= 0) return -1;
  long L = hla2_oracle_state_len(d, dv);
  double *st = state ? state : (double *)calloc((size_t)L, sizeof(double));
  const double *S = st, *m = st + (long)d * d + (long)d * dv, *h = m + d + (long)d * dv;
  double dummy;
  int t, a, b;
  for (t = 0; t < n; ++t) {
    hla2_oracle_step(d, dv, gamma, st, q + (long)t * d, k + (long)t * d, v + (long)t * dv,
                     num + (long)t * dv, den ? den + t : &dummy);
    double ss = 0.0;
    for (a = 0; a < d; ++a) {
      double u = -h[a];
      for (b = 0; b < d; ++b) u += S[(long)a * d + b] * m[b];
      ss += u * u;
    }
    unorm[t] = sqrt(ss);
  }
  if (!state) free(st);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Brute force straight from the definition (small n only):
 *   num_t = sum_{j<=t} sum_{i<=j} gamma^{(t-i)+(t-j)} (q_t.k_i)(q_j.k_i) v_j
 *   den_t = the same sum without v_j.
 * Cost O(n^2 (n + d) + n^2 dv).
 * ------------------------------------------------------------------------- */
int hla2_oracle_bruteforce(int n, int d, int dv, double gamma,
                           const double *q, const double *k, const double *v,
                           double *num, double *den) {
  if (n < 0 || d <= 0 || dv <= 0) return -1;
  double *dot = (double *)malloc(sizeof(double) * (size_t)n * (size_t)(n > 0 ? n : 1));
  int t, i, j, a, c;
  /* dot[t*n + i] = q_t . k_i */
  for (t = 0; t < n; ++t)
    for (i = 0; i < n; ++i) {
      double s = 0.0;
      for (a = 0; a < d; ++a) s += q[(long)t * d + a] * k[(long)i * d + a];
      dot[(long)t * n + i] = s;
    }
  for (t = 0; t < n; ++t) {
    for (c = 0; c < dv; ++c) num[(long)t * dv + c] = 0.0;
    double dsum = 0.0;
    for (j = 0; j <= t; ++j) {
      double w = 0.0;
      for (i = 0; i <= j; ++i)
        w += pow(gamma, (double)((t - i) + (t - j))) * dot[(long)t * n + i] * dot[(long)j * n + i];
      for (c = 0; c < dv; ++c) num[(long)t * dv + c] += w * v[(long)j * dv + c];
      dsum += w;
    }
    if (den) den[t] = dsum;
  }
  free(dot);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Summary of one segment of `len` tokens, built by definition (pairs inside
 * the segment, weights measured from the segment's last token T = len-1):
 *   S = sum_i g^{T-i} k_i k_i^T,  C = sum_j g^{T-j} q_j v_j^T,  m = sum_j g^{T-j} q_j,
 *   G = sum_{j<i} g^{(T-i)+(T-j)} k_i (k_i.q_j) v_j^T,   h likewise without v,
 *   Gamma = g^{len}.
 * ------------------------------------------------------------------------- */
void hla2_oracle_segment_summary(int len, int d, int dv, double gamma,
                                 const double *q, const double *k, const double *v,
                                 double *sum) {
  long L = hla2_oracle_summary_len(d, dv);
  double *Gam = sum, *S = sum + 1;
  double *C = S + (long)d * d, *m = C + (long)d * dv, *G = m + d, *h = G + (long)d * dv;
  int i, j, a, b, c;
  memset(sum, 0, sizeof(double) * (size_t)L);
  *Gam = pow(gamma, (double)len);
  int T = len - 1;
  for (i = 0; i < len; ++i) {
    double wi = pow(gamma, (double)(T - i));
    const double *ki = k + (long)i * d, *qi = q + (long)i * d, *vi = v + (long)i * dv;
    for (a = 0; a < d; ++a) {
      for (b = 0; b < d; ++b) S[(long)a * d + b] += wi * ki[a] * ki[b];
      for (c = 0; c < dv; ++c) C[(long)a * dv + c] += wi * qi[a] * vi[c];
      m[a] += wi * qi[a];
    }
    for (j = 0; j < i; ++j) {
      double wj = pow(gamma, (double)(T - j));
      const double *qj = q + (long)j * d, *vj = v + (long)j * dv;
      double kq = 0.0;
      for (a = 0; a < d; ++a) kq += ki[a] * qj[a];
      for (a = 0; a < d; ++a) {
        double f = wi * wj * ki[a] * kq;
        for (c = 0; c < dv; ++c) G[(long)a * dv + c] += f * vj[c];
        h[a] += f;
      }
    }
  }
}

/* Identity element of the combine: Gamma = 1, everything else zero. */
void hla2_oracle_identity(int d, int dv, double *sum) {
  memset(sum, 0, sizeof(double) * (size_t)hla2_oracle_summary_len(d, dv));
  sum[0] = 1.0;
}

/* ---------------------------------------------------------------------------
 * Semidirect-product combine: out = A then B (A earlier in the sequence).
 * [SUM §4 "Associatieve operatoren"]; out may alias neither input.
 * ------------------------------------------------------------------------- */
void hla2_oracle_combine(int d, int dv, const double *A, const double *B, double *out) {
  const double GA = A[0], GB = B[0];
  const double *SA = A + 1, *CA = SA + (long)d * d, *mA = CA + (long)d * dv,
               *GgA = mA + d, *hA = GgA + (long)d * dv;
  const double *SB = B + 1, *CB = SB + (long)d * d, *mB = CB + (long)d * dv,
               *GgB = mB + d, *hB = GgB + (long)d * dv;
  double *So = out + 1, *Co = So + (long)d * d, *mo = Co + (long)d * dv,
         *Go = mo + d, *ho = Go + (long)d * dv;
  int a, b, c;
  out[0] = GA * GB;
  for (a = 0; a < d; ++a) {
    for (b = 0; b < d; ++b) So[(long)a * d + b] = GB * SA[(long)a * d + b] + SB[(long)a * d + b];
    for (c = 0; c < dv; ++c) Co[(long)a * dv + c] = GB * CA[(long)a * dv + c] + CB[(long)a * dv + c];
    mo[a] = GB * mA[a] + mB[a];
  }
  /* G = GB^2 G_A + G_B + GB * S_B C_A ;  h = GB^2 h_A + h_B + GB * S_B m_A */
  for (a = 0; a < d; ++a) {
    for (c = 0; c < dv; ++c) {
      double s = 0.0;
      for (b = 0; b < d; ++b) s += SB[(long)a * d + b] * CA[(long)b * dv + c];
      Go[(long)a * dv + c] = GB * GB * GgA[(long)a * dv + c] + GgB[(long)a * dv + c] + GB * s;
    }
    double s = 0.0;
    for (b = 0; b < d; ++b) s += SB[(long)a * d + b] * mA[b];
    ho[a] = GB * GB * hA[a] + hB[a] + GB * s;
  }
}

/* ---------------------------------------------------------------------------
 * Exclusive Blelloch scan, in place, over `count` summaries laid out back to
 * back (stride = summary length).  The array is padded to a power of two with
 * identity elements; the up-sweep builds partial products in a balanced tree,
 * the root is replaced by the identity, and the down-sweep hands every node
 * the product of everything to its left.  Afterwards element c holds the
 * combination of elements 0..c-1 (the identity for c = 0).
 * ------------------------------------------------------------------------- */
int hla2_oracle_exclusive_scan(int d, int dv, int count, double *sums) {
  long L = hla2_oracle_summary_len(d, dv);
  int P = 1, i;
  if (count <= 0) return 0;
  while (P < count) P <<= 1;
  double *x = (double *)malloc(sizeof(double) * (size_t)L * (size_t)P);
  double *tmp = (double *)malloc(sizeof(double) * (size_t)L);
  double *left = (double *)malloc(sizeof(double) * (size_t)L);
  if (!x || !tmp || !left) { free(x); free(tmp); free(left); return -2; }
  memcpy(x, sums, sizeof(double) * (size_t)L * (size_t)count);
  for (i = count; i < P; ++i) hla2_oracle_identity(d, dv, x + (long)i * L);
  /* up-sweep: x[r] <- x[l] then x[r], r = right child of each pair */
  int stride;
  for (stride = 1; stride < P; stride <<= 1) {
    for (i = 2 * stride - 1; i < P; i += 2 * stride) {
      double *xl = x + (long)(i - stride) * L, *xr = x + (long)i * L;
      hla2_oracle_combine(d, dv, xl, xr, tmp);
      memcpy(xr, tmp, sizeof(double) * (size_t)L);
    }
  }
  /* root gets the identity */
  hla2_oracle_identity(d, dv, x + (long)(P - 1) * L);
  /* down-sweep: (left, right) <- (right, right then left-subtree total) */
  for (stride = P >> 1; stride >= 1; stride >>= 1) {
    for (i = 2 * stride - 1; i < P; i += 2 * stride) {
      double *xl = x + (long)(i - stride) * L, *xr = x + (long)i * L;
      memcpy(left, xl, sizeof(double) * (size_t)L);  /* total of left subtree */
      memcpy(xl, xr, sizeof(double) * (size_t)L);    /* prefix before this node */
      hla2_oracle_combine(d, dv, xr, left, tmp);     /* prefix, then left subtree */
      memcpy(xr, tmp, sizeof(double) * (size_t)L);
    }
  }
  memcpy(sums, x, sizeof(double) * (size_t)L * (size_t)count);
  free(x); free(tmp); free(left);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Outputs of one chunk of `len` tokens from its incoming state (S0, C0, m0,
 * G0, h0), written out in the chunk-local matrix form.  With tau the local
 * index, D[tau][i] = gamma^{tau-i} for i <= tau (else 0), A = L o (Q K^T):
 *   U0 = S0 C0 - G0,  u0 = S0 m0 - h0,
 *   W[tau][j] = D[tau][j] * ( gamma^{tau+1} q_tau^T S0 q_j
 *                            + sum_{i<=j} D[tau][i] A[tau][i] A[j][i] ),  j <= tau
 *   num_tau = gamma^{2(tau+1)} q_tau^T U0 + sum_{j<=tau} W[tau][j] v_j
 *   den_tau = gamma^{2(tau+1)} q_tau^T u0 + sum_{j<=tau} W[tau][j].
 * The first term carries every pair with both indices before the chunk, the
 * q^T S0 q term the pairs whose key index lies before the chunk and whose query
 * index lies inside, the last sum the pairs inside the chunk.
 * ------------------------------------------------------------------------- */
static void chunk_outputs(int len, int d, int dv, double gamma, const double *state_in,
                          const double *q, const double *k, const double *v,
                          double *num, double *den) {
  const double *S0 = state_in + 1, *C0 = S0 + (long)d * d, *m0 = C0 + (long)d * dv,
               *G0 = m0 + d, *h0 = G0 + (long)d * dv;
  double *U0 = (double *)malloc(sizeof(double) * (size_t)d * dv);
  double *u0 = (double *)malloc(sizeof(double) * (size_t)d);
  double *A = (double *)malloc(sizeof(double) * (size_t)len * len);
  double *QS = (double *)malloc(sizeof(double) * (size_t)len * d);
  int a, b, c, tau, i, j;
  for (a = 0; a < d; ++a) {
    for (c = 0; c < dv; ++c) {
      double s = 0.0;
      for (b = 0; b < d; ++b) s += S0[(long)a * d + b] * C0[(long)b * dv + c];
      U0[(long)a * dv + c] = s - G0[(long)a * dv + c];
    }
    double s = 0.0;
    for (b = 0; b < d; ++b) s += S0[(long)a * d + b] * m0[b];
    u0[a] = s - h0[a];
  }
  for (tau = 0; tau < len; ++tau) {
    for (i = 0; i < len; ++i) {
      double s = 0.0;
      if (i <= tau)
        for (a = 0; a < d; ++a) s += q[(long)tau * d + a] * k[(long)i * d + a];
      A[(long)tau * len + i] = s;
    }
    for (b = 0; b < d; ++b) {
      double s = 0.0;
      for (a = 0; a < d; ++a) s += q[(long)tau * d + a] * S0[(long)a * d + b];
      QS[(long)tau * d + b] = s;
    }
  }
  for (tau = 0; tau < len; ++tau) {
    double carry = pow(gamma, 2.0 * (tau + 1));
    double *o = num + (long)tau * dv;
    for (c = 0; c < dv; ++c) {
      double s = 0.0;
      for (a = 0; a < d; ++a) s += q[(long)tau * d + a] * U0[(long)a * dv + c];
      o[c] = carry * s;
    }
    double dn = 0.0;
    for (a = 0; a < d; ++a) dn += q[(long)tau * d + a] * u0[a];
    dn *= carry;
    for (j = 0; j <= tau; ++j) {
      double qsq = 0.0;
      for (b = 0; b < d; ++b) qsq += QS[(long)tau * d + b] * q[(long)j * d + b];
      double inner = 0.0;
      for (i = 0; i <= j; ++i)
        inner += pow(gamma, (double)(tau - i)) * A[(long)tau * len + i] * A[(long)j * len + i];
      double w = pow(gamma, (double)(tau - j)) * (pow(gamma, (double)(tau + 1)) * qsq + inner);
      for (c = 0; c < dv; ++c) o[c] += w * v[(long)j * dv + c];
      dn += w;
    }
    if (den) den[tau] = dn;
  }
  free(U0); free(u0); free(A); free(QS);
}

/* ---------------------------------------------------------------------------
 * Chunk-parallel path (one head): summaries of every chunk of `chunk` tokens
 * (the last may be shorter), exclusive Blelloch scan, then chunk outputs from
 * each chunk's incoming state.  If `state_out` is non-NULL it receives the
 * state after the last token (the inclusive total, Gamma dropped).
 * ------------------------------------------------------------------------- */
int hla2_oracle_chunked(int n, int d, int dv, double gamma, int chunk,
                        const double *q, const double *k, const double *v,
                        double *num, double *den, double *state_out) {
  if (n < 0 || d <= 0 || dv <= 0 || chunk <= 0) return -1;
  if (n == 0) {
    if (state_out) memset(state_out, 0, sizeof(double) * (size_t)hla2_oracle_state_len(d, dv));
    return 0;
  }
  int nc = (n + chunk - 1) / chunk, c;
  long L = hla2_oracle_summary_len(d, dv);
  double *sums = (double *)malloc(sizeof(double) * (size_t)L * (size_t)nc);
  double *incl = (double *)malloc(sizeof(double) * (size_t)L);
  if (!sums || !incl) { free(sums); free(incl); return -2; }
  for (c = 0; c < nc; ++c) {
    int t0 = c * chunk, len = (n - t0 < chunk) ? n - t0 : chunk;
    hla2_oracle_segment_summary(len, d, dv, gamma, q + (long)t0 * d, k + (long)t0 * d,
                                v + (long)t0 * dv, sums + (long)c * L);
  }
  double *last = (double *)malloc(sizeof(double) * (size_t)L);
  memcpy(last, sums + (long)(nc - 1) * L, sizeof(double) * (size_t)L);
  int rc = hla2_oracle_exclusive_scan(d, dv, nc, sums);
  if (rc) { free(sums); free(incl); free(last); return rc; }
  for (c = 0; c < nc; ++c) {
    int t0 = c * chunk, len = (n - t0 < chunk) ? n - t0 : chunk;
    chunk_outputs(len, d, dv, gamma, sums + (long)c * L, q + (long)t0 * d, k + (long)t0 * d,
                  v + (long)t0 * dv, num + (long)t0 * dv, den ? den + t0 : NULL);
  }
  if (state_out) {
    hla2_oracle_combine(d, dv, sums + (long)(nc - 1) * L, last, incl);
    memcpy(state_out, incl + 1, sizeof(double) * (size_t)(L - 1));
  }
  free(sums); free(incl); free(last);
  return 0;
}

/* ---------------------------------------------------------------------------
 * Gradients of the forward pass (one head): the adjoint of the serial
 * recurrence, run backwards in time.  The pages train through the scan but
 * print no backward formulas [SUM §4]; this is the chain rule applied to the
 * recurrence above, for the loss L = sum_t dout_t . o_t.
 *
 * Change of variables: U_t = S_t C_t - G_t and u_t = S_t m_t - h_t.  Expanding
 * S_t C_t with S_t = gamma S_{t-1} + k k^T and C_t = gamma C_{t-1} + q v^T, the
 * part gamma k (k^T C_{t-1}) is exactly G's new term, so
 *     U_t = gamma^2 U_{t-1} + (S_t q_t) v_t^T   (and u_t with v_t -> 1).
 * With z_t = S_t q_t and the augmented value v'_t = [v_t, 1] (dv + 1 columns),
 *     U'_t = gamma^2 U'_{t-1} + z_t v'_t^T,   [num_t, den_t] = U'_t^T q_t.
 * Upstream gradient of [num_t, den_t]: g'_t = [dout_t, 0] unnormalised, or
 * [dout_t / den_t, -(dout_t . out_t) / den_t] for the ratio, where out and den
 * are the forward's outputs (passed in, so both sides of a comparison use the
 * same values).
 * Adjoint states (gradients w.r.t. U'_t and S_t, including every later use):
 *     Ubar_t = q_t g'_t^T + gamma^2 Ubar_{t+1},   zbar_t = Ubar_t v'_t,
 *     Sbar_t = zbar_t q_t^T + gamma Sbar_{t+1},
 *     dq_t = U'_t g'_t + S_t zbar_t   (S_t symmetric),
 *     dv_t = (Ubar_t^T z_t)[0 .. dv-1],
 *     dk_t = (Sbar_t + Sbar_t^T) k_t.
 * Three passes: forward for z_t; backward for the adjoints, dk and dv; forward
 * again (S_t, U'_t rebuilt) for dq.
 * out, den: n*dv and n, read only when normalize = 1.
 * ------------------------------------------------------------------------- */
int hla2_oracle_backward_serial(int n, int d, int dv, double gamma, int normalize,
                                const double *q, const double *k, const double *v,
                                const double *dout, const double *out, const double *den,
                                double *dq, double *dk, double *dvv) {
  const int dvp = dv + 1;
  const double gsq = gamma * gamma;
  int t, a, b, c;
  if (n <= 0) return 0;
  if (normalize && (!out || !den)) return -1;
  double *gp = (double *)calloc((size_t)n * dvp, sizeof(double));
  double *z = (double *)calloc((size_t)n * d, sizeof(double));
  double *zb = (double *)calloc((size_t)n * d, sizeof(double));
  double *S = (double *)calloc((size_t)d * d, sizeof(double));
  double *U = (double *)calloc((size_t)d * dvp, sizeof(double));
  double *Ub = (double *)calloc((size_t)d * dvp, sizeof(double));
  double *Sb = (double *)calloc((size_t)d * d, sizeof(double));
  if (!gp || !z || !zb || !S || !U || !Ub || !Sb) {
    free(gp); free(z); free(zb); free(S); free(U); free(Ub); free(Sb);
    return -2;
  }
  /* upstream gradient of [num, den] */
  for (t = 0; t < n; ++t) {
    const double *g = dout + (long)t * dv;
    double *gt = gp + (long)t * dvp;
    if (normalize) {
      double dot = 0.0;
      for (c = 0; c < dv; ++c) dot += g[c] * out[(long)t * dv + c];
      for (c = 0; c < dv; ++c) gt[c] = g[c] / den[t];
      gt[dv] = -dot / den[t];
    } else {
      for (c = 0; c < dv; ++c) gt[c] = g[c];
      gt[dv] = 0.0;
    }
  }
  /* pass 1: z_t = S_t q_t */
  for (t = 0; t < n; ++t) {
    const double *qt = q + (long)t * d, *kt = k + (long)t * d;
    for (a = 0; a < d; ++a)
      for (b = 0; b < d; ++b) S[(long)a * d + b] = gamma * S[(long)a * d + b] + kt[a] * kt[b];
    for (a = 0; a < d; ++a) {
      double s = 0.0;
      for (b = 0; b < d; ++b) s += S[(long)a * d + b] * qt[b];
      z[(long)t * d + a] = s;
    }
  }
  /* pass 2: adjoints backwards in time; dk, dv */
  for (t = n - 1; t >= 0; --t) {
    const double *qt = q + (long)t * d, *kt = k + (long)t * d, *vt = v + (long)t * dv;
    const double *gt = gp + (long)t * dvp;
    double *zbt = zb + (long)t * d;
    for (a = 0; a < d; ++a)
      for (c = 0; c < dvp; ++c) Ub[(long)a * dvp + c] = gsq * Ub[(long)a * dvp + c] + qt[a] * gt[c];
    for (a = 0; a < d; ++a) {
      double s = Ub[(long)a * dvp + dv];  /* the ones column of v' */
      for (c = 0; c < dv; ++c) s += Ub[(long)a * dvp + c] * vt[c];
      zbt[a] = s;
    }
    for (a = 0; a < d; ++a)
      for (b = 0; b < d; ++b) Sb[(long)a * d + b] = gamma * Sb[(long)a * d + b] + zbt[a] * qt[b];
    for (a = 0; a < d; ++a) {
      double s = 0.0;
      for (b = 0; b < d; ++b) s += (Sb[(long)a * d + b] + Sb[(long)b * d + a]) * kt[b];
      dk[(long)t * d + a] = s;
    }
    for (c = 0; c < dv; ++c) {
      double s = 0.0;
      for (a = 0; a < d; ++a) s += Ub[(long)a * dvp + c] * z[(long)t * d + a];
      dvv[(long)t * dv + c] = s;
    }
  }
  /* pass 3: forward again; dq */
  memset(S, 0, sizeof(double) * (size_t)d * d);
  for (t = 0; t < n; ++t) {
    const double *kt = k + (long)t * d, *vt = v + (long)t * dv;
    const double *gt = gp + (long)t * dvp, *zt = z + (long)t * d, *zbt = zb + (long)t * d;
    for (a = 0; a < d; ++a)
      for (b = 0; b < d; ++b) S[(long)a * d + b] = gamma * S[(long)a * d + b] + kt[a] * kt[b];
    for (a = 0; a < d; ++a) {
      for (c = 0; c < dv; ++c) U[(long)a * dvp + c] = gsq * U[(long)a * dvp + c] + zt[a] * vt[c];
      U[(long)a * dvp + dv] = gsq * U[(long)a * dvp + dv] + zt[a];
    }
    for (a = 0; a < d; ++a) {
      double s = 0.0;
      for (c = 0; c < dvp; ++c) s += U[(long)a * dvp + c] * gt[c];
      for (b = 0; b < d; ++b) s += S[(long)a * d + b] * zbt[b];
      dq[(long)t * d + a] = s;
    }
  }
  free(gp); free(z); free(zb); free(S); free(U); free(Ub); free(Sb);
  return 0;
}

/* ===========================================================================
 * AHLA, the asymmetric variant [SUM §2]: the operator Q (K^T Q)(K^T V), with
 * the streaming summaries P^KV_t, m^K_t, E_t, n_t the page names.  Masked as
 * the second-order case (every index at or before t), row t is
 *     num_t = sum_{j<=t} sum_{i<=j} (q_t.k_j)(q_j.k_i) v_i,
 * i.e. A A V with A = L o (Q K^T): the value of key i reaches query t through
 * the intermediate key index j.  Reading of the summaries (the page gives only
 * their names): P^KV_t = sum_{i<=t} k_i v_i^T and m^K_t = sum_{i<=t} k_i are
 * the key-value and key-mass prefixes; E_t = sum_{j<=t} k_j (q_j^T P^KV_j) and
 * n_t = sum_{j<=t} k_j (q_j . m^K_j) carry the inner sums already masked at
 * their own index j, so num_t = q_t^T E_t and den_t = q_t^T n_t.  With decay
 * every summary decays by gamma per token (as in the second-order case), so
 * the term (j, i) carries gamma^{t-i}: num = A_g A_g V with A_g = D o A.
 * State block: P[d*dv] | m[d] | E[d*dv] | n[d].
 * ------------------------------------------------------------------------- */
long hla2_oracle_ahla_state_len(int d, int dv) { return 2L * d * dv + 2L * d; }

/* One token: P, m absorb (k, v); then E, n absorb k (q^T P_t), k (q . m_t); readout. */
void hla2_oracle_ahla_step(int d, int dv, double gamma, double *state, const double *q, const double *k,
                           const double *v, double *num, double *den) {
  double *P = state, *m = P + (long)d * dv, *E = m + d, *nn = E + (long)d * dv;
  int a, c;
  double *qP = (double *)calloc((size_t)dv, sizeof(double));
  double qm = 0.0;
  for (a = 0; a < d; ++a) {
    for (c = 0; c < dv; ++c) P[(long)a * dv + c] = gamma * P[(long)a * dv + c] + k[a] * v[c];
    m[a] = gamma * m[a] + k[a];
  }
  for (a = 0; a < d; ++a) {
    for (c = 0; c < dv; ++c) qP[c] += q[a] * P[(long)a * dv + c];
    qm += q[a] * m[a];
  }
  for (a = 0; a < d; ++a) {
    for (c = 0; c < dv; ++c) E[(long)a * dv + c] = gamma * E[(long)a * dv + c] + k[a] * qP[c];
    nn[a] = gamma * nn[a] + k[a] * qm;
  }
  for (c = 0; c < dv; ++c) {
    double s = 0.0;
    for (a = 0; a < d; ++a) s += q[a] * E[(long)a * dv + c];
    num[c] = s;
  }
  double sd = 0.0;
  for (a = 0; a < d; ++a) sd += q[a] * nn[a];
  *den = sd;
  free(qP);
}

/* Serial recurrence (state nullable: zero start; else in/out). */
int hla2_oracle_ahla_serial(int n, int d, int dv, double gamma, const double *q, const double *k,
                            const double *v, double *num, double *den, double *state) {
  long L = hla2_oracle_ahla_state_len(d, dv);
  double *st = state ? state : (double *)calloc((size_t)L, sizeof(double));
  int t;
  if (!st) return -2;
  for (t = 0; t < n; ++t) {
    double dd;
    hla2_oracle_ahla_step(d, dv, gamma, st, q + (long)t * d, k + (long)t * d, v + (long)t * dv,
                          num + (long)t * dv, &dd);
    if (den) den[t] = dd;
  }
  if (!state) free(st);
  return 0;
}

/* Serial recurrence that also reports, per token, |n_t|, the norm of the den column of the state
 * (den_t = q_t . n_t): the natural scale of den_t, against which its cancellation is measured
 * [SUM §1 "Normalisatie", as for the second order's u_t].  Arguments as hla2_oracle_ahla_serial plus
 * unorm (n). */
int hla2_oracle_ahla_serial_unorm(int n, int d, int dv, double gamma, const double *q, const double *k,
                                  const double *v, double *num, double *den, double *unorm, double *state) {
  long L = hla2_oracle_ahla_state_len(d, dv);
  double *st = state ? state : (double *)calloc((size_t)L, sizeof(double));
  const double *nn = st + 2L * d * dv + d;
  int t, a;
  if (!st) return -2;
  for (t = 0; t < n; ++t) {
    double dd, ss = 0.0;
    hla2_oracle_ahla_step(d, dv, gamma, st, q + (long)t * d, k + (long)t * d, v + (long)t * dv,
                          num + (long)t * dv, &dd);
    if (den) den[t] = dd;
    for (a = 0; a < d; ++a) ss += nn[a] * nn[a];
    unorm[t] = sqrt(ss);
  }
  if (!state) free(st);
  return 0;
}

/* The definition as a triple sum (small n). */
int hla2_oracle_ahla_bruteforce(int n, int d, int dv, double gamma, const double *q, const double *k,
                                const double *v, double *num, double *den) {
  int t, j, i, a, c;
  for (t = 0; t < n; ++t) {
    for (c = 0; c < dv; ++c) num[(long)t * dv + c] = 0.0;
    double sd = 0.0;
    for (j = 0; j <= t; ++j) {
      double qk_tj = 0.0;
      for (a = 0; a < d; ++a) qk_tj += q[(long)t * d + a] * k[(long)j * d + a];
      for (i = 0; i <= j; ++i) {
        double qk_ji = 0.0;
        for (a = 0; a < d; ++a) qk_ji += q[(long)j * d + a] * k[(long)i * d + a];
        double w = pow(gamma, (double)(t - i)) * qk_tj * qk_ji;
        for (c = 0; c < dv; ++c) num[(long)t * dv + c] += w * v[(long)i * dv + c];
        sd += w;
      }
    }
    if (den) den[t] = sd;
  }
  return 0;
}

/* Segment summary for the chunk-parallel form: (Gamma, P, m, E, n, M) of a run
 * of len tokens from the zero state, with M = sum_j k_j q_j^T (d x d, no decay:
 * for a later segment B, the term gamma^{end-1-j} k_j q_j^T (gamma^{j-start+1} P_A)
 * loses every power of j, so E_{AB} = Gamma_B E_A + E_B + Gamma_B M_B P_A).
 * Layout: Gamma | P | m | E | n | M. */
long hla2_oracle_ahla_summary_len(int d, int dv) { return 1 + hla2_oracle_ahla_state_len(d, dv) + (long)d * d; }

void hla2_oracle_ahla_summary(int len, int d, int dv, double gamma, const double *q, const double *k,
                              const double *v, double *sum) {
  long L = hla2_oracle_ahla_state_len(d, dv);
  double *num = (double *)malloc(sizeof(double) * (size_t)(len > 0 ? len : 1) * dv);
  double *M = sum + 1 + L;
  int t, a, b;
  memset(sum, 0, sizeof(double) * (size_t)hla2_oracle_ahla_summary_len(d, dv));
  sum[0] = pow(gamma, (double)len);
  hla2_oracle_ahla_serial(len, d, dv, gamma, q, k, v, num, NULL, sum + 1);
  for (t = 0; t < len; ++t)
    for (a = 0; a < d; ++a)
      for (b = 0; b < d; ++b) M[(long)a * d + b] += k[(long)t * d + a] * q[(long)t * d + b];
  free(num);
}

/* A then B: P = G_B P_A + P_B, m likewise, E = G_B E_A + E_B + G_B M_B P_A,
 * n = G_B n_A + n_B + G_B M_B m_A, M = M_A + M_B, Gamma = G_A G_B. */
void hla2_oracle_ahla_combine(int d, int dv, const double *A, const double *B, double *out) {
  long L = hla2_oracle_ahla_state_len(d, dv);
  const double GB = B[0];
  const double *PA = A + 1, *mA = PA + (long)d * dv, *EA = mA + d, *nA = EA + (long)d * dv, *MA = A + 1 + L;
  const double *PB = B + 1, *mB = PB + (long)d * dv, *EB = mB + d, *nB = EB + (long)d * dv, *MB = B + 1 + L;
  double *tmp = (double *)malloc(sizeof(double) * (size_t)hla2_oracle_ahla_summary_len(d, dv));
  double *Po = tmp + 1, *mo = Po + (long)d * dv, *Eo = mo + d, *no = Eo + (long)d * dv, *Mo = tmp + 1 + L;
  int a, b, c;
  tmp[0] = A[0] * GB;
  for (a = 0; a < d; ++a) {
    for (c = 0; c < dv; ++c) {
      double s = 0.0;
      for (b = 0; b < d; ++b) s += MB[(long)a * d + b] * PA[(long)b * dv + c];
      Po[(long)a * dv + c] = GB * PA[(long)a * dv + c] + PB[(long)a * dv + c];
      Eo[(long)a * dv + c] = GB * EA[(long)a * dv + c] + EB[(long)a * dv + c] + GB * s;
    }
    double s = 0.0;
    for (b = 0; b < d; ++b) s += MB[(long)a * d + b] * mA[b];
    mo[a] = GB * mA[a] + mB[a];
    no[a] = GB * nA[a] + nB[a] + GB * s;
    for (b = 0; b < d; ++b) Mo[(long)a * d + b] = MA[(long)a * d + b] + MB[(long)a * d + b];
  }
  memcpy(out, tmp, sizeof(double) * (size_t)hla2_oracle_ahla_summary_len(d, dv));
  free(tmp);
}

/* ===========================================================================
 * Third-order HLA [SUM §3]: the interaction A A^T A with A = Q K^T, masked so
 * that no index passes t.  Reading (the page names the moments S^K, S^Q, P^KV
 * and six cross summaries but prints no formula): with the middle query index
 * l, the key j of the A A^T factor and the key i of the last A factor,
 *   num_t = sum_{l<=t} sum_{j<=l} sum_{i<=l} g^{(t-j)+(t-l)+(t-i)}
 *                                 (q_t.k_j)(q_l.k_j)(q_l.k_i) v_i,
 * den_t likewise with v_i -> 1; unmasked and undecayed this is
 * q_t^T S^K S^Q P^KV, and every one of the three moments decays by g per token.
 * In matrix form num = (L o D_{g^2} o (A_g A^T)) (A_g V) with A = L o (Q K^T)
 * and A_g = D_g o A.
 * Streaming form used here (the cross summaries are folded into one corrected
 * accumulator, as U = S C - G for the second order): with z_l = S^K_l q_l and
 * y'_l = P'_l^T q_l, P' = [P^KV | m^K] (key-value and key-mass prefixes),
 *   W'_t = g^3 W'_{t-1} + z_t y'_t^T,   [num | den]_t = W'_t^T q_t.
 * State block: S[d*d] | P[d*dv] | m[d] | W[d*dv] | w[d]  (W' = [W | w]).
 * ------------------------------------------------------------------------- */
long hla2_oracle_ho3_state_len(int d, int dv) { return (long)d * d + 2L * d * (dv + 1); }

void hla2_oracle_ho3_step(int d, int dv, double gamma, double *state, const double *q, const double *k,
                          const double *v, double *num, double *den) {
  const int dvp = dv + 1;
  double *S = state, *P = S + (long)d * d, *W = P + (long)d * dvp;  /* P, W with the extra column */
  const double g3 = gamma * gamma * gamma;
  int a, b, c;
  double *z = (double *)calloc((size_t)d, sizeof(double));
  double *y = (double *)calloc((size_t)dvp, sizeof(double));
  for (a = 0; a < d; ++a) {
    for (b = 0; b < d; ++b) S[(long)a * d + b] = gamma * S[(long)a * d + b] + k[b] * k[a];
    for (c = 0; c < dv; ++c) P[(long)a * dvp + c] = gamma * P[(long)a * dvp + c] + k[a] * v[c];
    P[(long)a * dvp + dv] = gamma * P[(long)a * dvp + dv] + k[a];
  }
  for (a = 0; a < d; ++a) {
    for (b = 0; b < d; ++b) z[a] += S[(long)a * d + b] * q[b];
    for (c = 0; c < dvp; ++c) y[c] += q[a] * P[(long)a * dvp + c];
  }
  for (a = 0; a < d; ++a)
    for (c = 0; c < dvp; ++c) W[(long)a * dvp + c] = g3 * W[(long)a * dvp + c] + z[a] * y[c];
  for (c = 0; c < dvp; ++c) {
    double s = 0.0;
    for (a = 0; a < d; ++a) s += q[a] * W[(long)a * dvp + c];
    if (c < dv) num[c] = s;
    else *den = s;
  }
  free(z);
  free(y);
}

int hla2_oracle_ho3_serial(int n, int d, int dv, double gamma, const double *q, const double *k,
                           const double *v, double *num, double *den, double *state) {
  long L = hla2_oracle_ho3_state_len(d, dv);
  double *st = state ? state : (double *)calloc((size_t)L, sizeof(double));
  int t;
  if (!st) return -2;
  for (t = 0; t < n; ++t) {
    double dd;
    hla2_oracle_ho3_step(d, dv, gamma, st, q + (long)t * d, k + (long)t * d, v + (long)t * dv,
                         num + (long)t * dv, &dd);
    if (den) den[t] = dd;
  }
  if (!state) free(st);
  return 0;
}

/* Serial recurrence that also reports, per token, |w_t|, the norm of the den column of the corrected
 * accumulator W' (den_t = q_t . w_t): the natural scale of den_t [SUM §1 "Normalisatie", as for the
 * second order's u_t].  Arguments as hla2_oracle_ho3_serial plus unorm (n). */
int hla2_oracle_ho3_serial_unorm(int n, int d, int dv, double gamma, const double *q, const double *k,
                                 const double *v, double *num, double *den, double *unorm, double *state) {
  long L = hla2_oracle_ho3_state_len(d, dv);
  double *st = state ? state : (double *)calloc((size_t)L, sizeof(double));
  const int dvp = dv + 1;
  const double *W = st + (long)d * d + (long)d * dvp;
  int t, a;
  if (!st) return -2;
  for (t = 0; t < n; ++t) {
    double dd, ss = 0.0;
    hla2_oracle_ho3_step(d, dv, gamma, st, q + (long)t * d, k + (long)t * d, v + (long)t * dv,
                         num + (long)t * dv, &dd);
    if (den) den[t] = dd;
    for (a = 0; a < d; ++a) ss += W[(long)a * dvp + dv] * W[(long)a * dvp + dv];
    unorm[t] = sqrt(ss);
  }
  if (!state) free(st);
  return 0;
}

static double ho3_dot(int d, const double *x, const double *y) {
  double s = 0.0;
  int a;
  for (a = 0; a < d; ++a) s += x[a] * y[a];
  return s;
}

/* The definition as a quadruple sum (small n). */
int hla2_oracle_ho3_bruteforce(int n, int d, int dv, double gamma, const double *q, const double *k,
                               const double *v, double *num, double *den) {
  int t, l, j, i, c;
  for (t = 0; t < n; ++t) {
    double sd = 0.0;
    for (c = 0; c < dv; ++c) num[(long)t * dv + c] = 0.0;
    for (l = 0; l <= t; ++l)
      for (j = 0; j <= l; ++j) {
        double f1 = ho3_dot(d, q + (long)t * d, k + (long)j * d) * ho3_dot(d, q + (long)l * d, k + (long)j * d);
        for (i = 0; i <= l; ++i) {
          double w = pow(gamma, (double)((t - j) + (t - l) + (t - i))) * f1 * ho3_dot(d, q + (long)l * d, k + (long)i * d);
          for (c = 0; c < dv; ++c) num[(long)t * dv + c] += w * v[(long)i * dv + c];
          sd += w;
        }
      }
    if (den) den[t] = sd;
  }
  return 0;
}

/* Segment summary for the chunk-parallel form, from the zero state over len
 * tokens (u = 0 .. len-1 inside the segment, z^B, y'^B the segment-local values):
 *   the state part (S, P', W') and the maps that fold an incoming state
 *   (S_A, P'_A) into W' at the segment end:
 *     Q2 = sum_u g^{3len-1-u} q_u q_u^T            (d x d)
 *     X1 = sum_u g^{3len-2-2u} q_u y'^B_u^T         (d x (dv+1))
 *     X2 = sum_u g^{3len-2-2u} z^B_u q_u^T          (d x d)
 *   W'_end = g^{3len} W'_A + W'_B + S_A Q2 P'_A + S_A X1 + X2 P'_A,
 *   S_end = g^len S_A + S_B,  P'_end = g^len P'_A + P'_B.
 * (Inside the segment z_u = g^{u+1} S_A q_u + z^B_u and y'_u = g^{u+1} P'_A^T q_u + y'^B_u;
 * the powers collect into the weights above.)
 * Layout: Gamma | state | Q2 | X1 | X2. */
long hla2_oracle_ho3_summary_len(int d, int dv) {
  return 1 + hla2_oracle_ho3_state_len(d, dv) + 2L * d * d + (long)d * (dv + 1);
}

void hla2_oracle_ho3_summary(int len, int d, int dv, double gamma, const double *q, const double *k,
                             const double *v, double *sum) {
  const int dvp = dv + 1;
  long L = hla2_oracle_ho3_state_len(d, dv);
  double *st = sum + 1, *Q2 = sum + 1 + L, *X1 = Q2 + (long)d * d, *X2 = X1 + (long)d * dvp;
  double *num = (double *)malloc(sizeof(double) * (size_t)dv), dd;
  double *S = st, *P = S + (long)d * d;
  double *z = (double *)malloc(sizeof(double) * (size_t)d), *y = (double *)malloc(sizeof(double) * (size_t)dvp);
  int u, a, b, c;
  memset(sum, 0, sizeof(double) * (size_t)hla2_oracle_ho3_summary_len(d, dv));
  sum[0] = pow(gamma, (double)len);
  for (u = 0; u < len; ++u) {
    const double *qu = q + (long)u * d;
    hla2_oracle_ho3_step(d, dv, gamma, st, qu, k + (long)u * d, v + (long)u * dv, num, &dd);
    /* segment-local z, y' after the token */
    for (a = 0; a < d; ++a) {
      z[a] = 0.0;
      for (b = 0; b < d; ++b) z[a] += S[(long)a * d + b] * qu[b];
    }
    for (c = 0; c < dvp; ++c) {
      y[c] = 0.0;
      for (a = 0; a < d; ++a) y[c] += qu[a] * P[(long)a * dvp + c];
    }
    const double wq = pow(gamma, (double)(3 * len - 1 - u)), wx = pow(gamma, (double)(3 * len - 2 - 2 * u));
    for (a = 0; a < d; ++a) {
      for (b = 0; b < d; ++b) {
        Q2[(long)a * d + b] += wq * qu[a] * qu[b];
        X2[(long)a * d + b] += wx * z[a] * qu[b];
      }
      for (c = 0; c < dvp; ++c) X1[(long)a * dvp + c] += wx * qu[a] * y[c];
    }
  }
  free(num); free(z); free(y);
}

/* Fold a segment summary into a state (the exclusive scan's step). */
void hla2_oracle_ho3_apply(int d, int dv, const double *sum, double *state) {
  const int dvp = dv + 1;
  long L = hla2_oracle_ho3_state_len(d, dv);
  const double G = sum[0], G3 = G * G * G;
  const double *SB = sum + 1, *PB = SB + (long)d * d, *WB = PB + (long)d * dvp;
  const double *Q2 = sum + 1 + L, *X1 = Q2 + (long)d * d, *X2 = X1 + (long)d * dvp;
  double *S = state, *P = S + (long)d * d, *W = P + (long)d * dvp;
  double *SQ = (double *)calloc((size_t)d * d, sizeof(double));
  double *Wn = (double *)calloc((size_t)d * dvp, sizeof(double));
  int a, b, c;
  for (a = 0; a < d; ++a)
    for (b = 0; b < d; ++b)
      for (c = 0; c < d; ++c) SQ[(long)a * d + b] += S[(long)a * d + c] * Q2[(long)c * d + b];
  for (a = 0; a < d; ++a)
    for (c = 0; c < dvp; ++c) {
      double s = G3 * W[(long)a * dvp + c] + WB[(long)a * dvp + c];
      for (b = 0; b < d; ++b)
        s += SQ[(long)a * d + b] * P[(long)b * dvp + c] + S[(long)a * d + b] * X1[(long)b * dvp + c] +
             X2[(long)a * d + b] * P[(long)b * dvp + c];
      Wn[(long)a * dvp + c] = s;
    }
  for (a = 0; a < d; ++a) {
    for (b = 0; b < d; ++b) S[(long)a * d + b] = G * S[(long)a * d + b] + SB[(long)a * d + b];
    for (c = 0; c < dvp; ++c) {
      P[(long)a * dvp + c] = G * P[(long)a * dvp + c] + PB[(long)a * dvp + c];
      W[(long)a * dvp + c] = Wn[(long)a * dvp + c];
    }
  }
  free(SQ); free(Wn);
}
