/*
 * elsaa_oracle.c -- CPU reference for the ELSAA attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or call
 * this file: it exists so that tests, the smoke check and the CPU-baseline leg
 * of the benchmark can compare the GPU library against a plain, slow, obviously
 * correct computation.  It shares no code, header, table or constant with the
 * GPU library.
 *
 * Arithmetic: IEEE binary64 throughout, on inputs that arrive already upcast
 * (exactly) from their stored precision (fp32 or bf16).  Compile without
 * fast-math and with -ffp-contract=off so that every operation below is the
 * rounded binary64 operation it is written as.
 *
 * Sources (page titles and sections; no formula survives in the pages' text,
 * so each step names the passage it follows and the reading taken where the
 * text is silent):
 *   [A] "ELSAA: Efficient Low-Rank and Sparse Attention Approximation for
 *       Training Transformers" (arxivlens summary), first paragraph: sparse
 *       branch + low-rank branch, denominator-aware fusion that scales the
 *       sparse branch by its estimated attention mass relative to the
 *       low-rank branch, gates, lambda.
 *   [B] "Two Efficient Attentions, One Denominator Problem", section
 *       "Two efficient branches can still be mis-scaled": the sparse branch
 *       computes selected query-key interactions exactly; the RACE branch is a
 *       hash-bucket summary; each branch is normalised over its own
 *       denominator; the sparse multiplier for query i, then independent gates.
 *   [C] same page, "The ablation isolates the actual contribution": the
 *       Sort_Lsh_RACE ablation fixes the sparse multiplier to one, i.e. the
 *       multiplier acts on the sparse branch only.
 *   [D] same page, "Linear interactions are not yet production economics":
 *       the cost is a count of attention/bucket interactions, linear in N.
 * Mechanics the pages leave open (SRP hashing, stable sort by bucket, chunks of
 * w attending their own and the previous chunk, RACE scatter/gather, the mass
 * ratio Z_s/(Z_s + lambda Z_lr), sigmoid gates) follow the operator's
 * specification and the readings recorded in the design notes of this
 * repository; each function states the reading it implements.
 *
 * Parity pins: every function here is checked by tests under tests/ against
 * closed forms, brute force on tiny inputs, library routines (numpy stable
 * argsort, math.fsum, dense softmax) and invariants -- never against the GPU.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MAX_D 4096

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ------------------------------------------------------------------------- */
/* Exact sign of a dot product.                                               */
/*                                                                           */
/* Reading: a hash bit is 1 iff the exact real dot product of the stored     */
/* vectors with the hyperplane normal is > 0 (a zero product gives 0).  Each */
/* product of two values with at most 24 significant bits is exact in       */
/* binary64; the sum of the products is carried exactly as a nonoverlapping  */
/* floating-point expansion grown one term at a time with Knuth's TwoSum     */
/* (Shewchuk, "Adaptive Precision Floating-Point Arithmetic and Fast Robust  */
/* Geometric Predicates", 1997: Grow-Expansion with zero elimination).  The  */
/* sign of a nonoverlapping expansion is the sign of its largest component, */
/* which Grow-Expansion leaves last.                                          */
/* ------------------------------------------------------------------------- */
static void two_sum(double a, double b, double *s, double *err) {
  double x = a + b;
  double b_virtual = x - a;
  double a_virtual = x - b_virtual;
  double b_round = b - b_virtual;
  double a_round = a - a_virtual;
  *s = x;
  *err = a_round + b_round;
}

int oracle_exact_dot_sign(const double *x, const double *r, int d) {
  double expansion[ORACLE_MAX_D + 1];
  int m = 0;
  for (int i = 0; i < d; ++i) {
    double q = x[i] * r[i]; /* exact: each factor has <= 24 significant bits */
    int k = 0;
    for (int j = 0; j < m; ++j) {
      double s, h;
      two_sum(q, expansion[j], &s, &h);
      q = s;
      if (h != 0.0) expansion[k++] = h;
    }
    if (q != 0.0) expansion[k++] = q;
    m = k;
  }
  if (m == 0) return 0;
  return expansion[m - 1] > 0.0 ? 1 : -1;
}

/* ------------------------------------------------------------------------- */
/* SRP (sign random projection) codes.                                        */
/* For each of `rows` vectors x (length d) and planes[first .. first+nbits),  */
/* bit t of the code is [<x, plane[first+t]> > 0], least significant first.   */
/* codes[row * code_stride + code_offset] receives the code.                  */
/* ------------------------------------------------------------------------- */
void oracle_srp_codes(const double *x, long rows, int d, const double *planes,
                      int first, int nbits, int32_t *codes, int code_stride,
                      int code_offset) {
  long r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < rows; ++r) {
    const double *xr = x + (size_t)r * d;
    int32_t code = 0;
    for (int t = 0; t < nbits; ++t) {
      const double *plane = planes + (size_t)(first + t) * d;
      if (oracle_exact_dot_sign(xr, plane, d) > 0) code |= (int32_t)1 << t;
    }
    codes[(size_t)r * code_stride + code_offset] = code;
  }
}

/* ------------------------------------------------------------------------- */
/* Stable sort by bucket: per segment s of n codes, perm[s][rank] is the       */
/* original position of the element with that rank when elements are ordered */
/* by (code ascending, original position ascending).  Counting sort.          */
/* ------------------------------------------------------------------------- */
int oracle_stable_sort(const int32_t *codes, long segments, int n, int nbuckets,
                       int32_t *perm) {
  int fail = 0;
  long s;
#pragma omp parallel for schedule(dynamic) reduction(| : fail)
  for (s = 0; s < segments; ++s) {
    const int32_t *c = codes + (size_t)s * n;
    int32_t *p = perm + (size_t)s * n;
    long *start = (long *)calloc((size_t)nbuckets + 1, sizeof(long));
    if (!start) { fail = 1; continue; }
    for (int i = 0; i < n; ++i) start[c[i] + 1] += 1;
    for (int b = 0; b < nbuckets; ++b) start[b + 1] += start[b];
    for (int i = 0; i < n; ++i) p[start[c[i]]++] = i;
    free(start);
  }
  return fail ? -1 : 0;
}

/* ------------------------------------------------------------------------- */
/* Chunked exact attention ([B]: exact on the selected pairs).                */
/* The query at sorted rank r lies in chunk c = floor(r / w) and attends the  */
/* keys at sorted ranks [max(0, (c-1) w), (c+1) w): its own chunk and the     */
/* previous one, with no wrap-around, no mask.  Scores s = <q, k> / sqrt(d).  */
/* Outputs (at the query's original position): o = sum_j softmax(s)_j v_j    */
/* and lse = log sum_j exp(s_j), the log of the sparse mass Z_s.              */
/* Returns the number of (query, key) pairs evaluated per segment summed over */
/* all segments.                                                              */
/* ------------------------------------------------------------------------- */
long oracle_chunk_attention(const double *q, const double *k, const double *v,
                            const int32_t *perm_q, const int32_t *perm_k,
                            long segments, int n, int d, int w, double *o,
                            double *lse) {
  const double scale = 1.0 / sqrt((double)d);
  long pairs = 0;
  long idx;
  const long total = segments * (long)n;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs)
  for (idx = 0; idx < total; ++idx) {
    const long s = idx / n;
    const int rank = (int)(idx % n);
    const int c = rank / w;
    const int lo = c > 0 ? (c - 1) * w : 0;
    const int hi = (c + 1) * w;
    const int i = perm_q[(size_t)s * n + rank];
    const double *qi = q + ((size_t)s * n + i) * d;
    double *scores = (double *)malloc(sizeof(double) * (size_t)(hi - lo));
    double m = -INFINITY;
    for (int t = lo; t < hi; ++t) {
      const int j = perm_k[(size_t)s * n + t];
      const double *kj = k + ((size_t)s * n + j) * d;
      double dot = 0.0;
      for (int e = 0; e < d; ++e) dot += qi[e] * kj[e];
      scores[t - lo] = dot * scale;
      if (scores[t - lo] > m) m = scores[t - lo];
    }
    double total_w = 0.0;
    double *oi = o + ((size_t)s * n + i) * d;
    for (int e = 0; e < d; ++e) oi[e] = 0.0;
    for (int t = lo; t < hi; ++t) {
      const int j = perm_k[(size_t)s * n + t];
      const double *vj = v + ((size_t)s * n + j) * d;
      const double p = exp(scores[t - lo] - m);
      total_w += p;
      for (int e = 0; e < d; ++e) oi[e] += p * vj[e];
    }
    for (int e = 0; e < d; ++e) oi[e] /= total_w;
    lse[(size_t)s * n + i] = m + log(total_w);
    pairs += hi - lo;
    free(scores);
  }
  return pairs;
}

/* ------------------------------------------------------------------------- */
/* RACE tables ([B]: hash-bucket summaries).  For every segment, table l and  */
/* bucket b: count[s][l][b] = #{keys j : code_l(k_j) = b} and                 */
/* sum[s][l][b][:] = sum of v_j over those keys.  kcodes is [s][n][L].        */
/* ------------------------------------------------------------------------- */
void oracle_race_tables(const double *v, const int32_t *kcodes, long segments,
                        int n, int d, int L, int P, double *sums, double *counts) {
  const long nb = 1L << P;
  long sl;
#pragma omp parallel for schedule(dynamic)
  for (sl = 0; sl < segments * L; ++sl) {
    const long s = sl / L;
    const int l = (int)(sl % L);
    double *tsum = sums + (size_t)sl * nb * d;
    double *tcnt = counts + (size_t)sl * nb;
    memset(tsum, 0, sizeof(double) * (size_t)nb * d);
    memset(tcnt, 0, sizeof(double) * (size_t)nb);
    for (int j = 0; j < n; ++j) {
      const int b = kcodes[((size_t)s * n + j) * L + l];
      const double *vj = v + ((size_t)s * n + j) * d;
      tcnt[b] += 1.0;
      for (int e = 0; e < d; ++e) tsum[(size_t)b * d + e] += vj[e];
    }
  }
}

/* ------------------------------------------------------------------------- */
/* RACE query side.  Each query gathers, in every table, the bucket it hashes */
/* to.  Reading: both the numerator and the collision-count mass are means    */
/* over the L tables:                                                         */
/*   Z_lr = (1/L) sum_l count_l[code_l(q)],  num = (1/L) sum_l sum_l[...],    */
/*   o_lr = num / Z_lr, and o_lr = 0 when Z_lr = 0 (no key shares a bucket).  */
/* ------------------------------------------------------------------------- */
void oracle_race_query(const int32_t *qcodes, const double *sums,
                       const double *counts, long segments, int n, int d, int L,
                       int P, double *o_lr, double *z_lr) {
  const long nb = 1L << P;
  long idx;
  const long total = segments * (long)n;
#pragma omp parallel for schedule(static)
  for (idx = 0; idx < total; ++idx) {
    const long s = idx / n;
    double *out = o_lr + (size_t)idx * d;
    double z = 0.0;
    for (int e = 0; e < d; ++e) out[e] = 0.0;
    for (int l = 0; l < L; ++l) {
      const int b = qcodes[(size_t)idx * L + l];
      const size_t t = ((size_t)s * L + l) * nb + b;
      z += counts[t];
      for (int e = 0; e < d; ++e) out[e] += sums[t * d + e];
    }
    z /= (double)L;
    for (int e = 0; e < d; ++e) out[e] /= (double)L;
    if (z > 0.0) {
      for (int e = 0; e < d; ++e) out[e] /= z;
    } else {
      for (int e = 0; e < d; ++e) out[e] = 0.0;
    }
    z_lr[idx] = z;
  }
}

/* ------------------------------------------------------------------------- */
/* Token-wise gates ([A], [B]: independent gates per branch).  Reading: one   */
/* gate input x_gate[b][i][:] per token shared by the heads, weights per head */
/* and per branch: g[br][b][h][i] = sigmoid(<x_gate[b][i], W[br][h]> + c[br][h]) */
/* with br = 0 the sparse gate and br = 1 the low-rank gate.                  */
/* ------------------------------------------------------------------------- */
void oracle_gates(const double *x_gate, const double *gate_w, const double *gate_b,
                  int B, int H, int n, int dg, double *g_s, double *g_lr) {
  long idx;
  const long total = (long)B * H * n;
#pragma omp parallel for schedule(static)
  for (idx = 0; idx < total; ++idx) {
    const int i = (int)(idx % n);
    const int h = (int)((idx / n) % H);
    const int b = (int)(idx / ((long)n * H));
    const double *x = x_gate + ((size_t)b * n + i) * dg;
    for (int br = 0; br < 2; ++br) {
      const double *wv = gate_w + ((size_t)br * H + h) * dg;
      double a = gate_b[(size_t)br * H + h];
      for (int e = 0; e < dg; ++e) a += x[e] * wv[e];
      const double g = 1.0 / (1.0 + exp(-a));
      if (br == 0) g_s[idx] = g; else g_lr[idx] = g;
    }
  }
}

/* ------------------------------------------------------------------------- */
/* Denominator-aware fusion ([A], [B], [C]).                                  */
/* alpha_i = Z_s / (Z_s + lambda Z_lr) with Z_s = exp(lse), evaluated as      */
/* 1 / (1 + exp(log(lambda Z_lr) - lse)); alpha = 1 when lambda Z_lr = 0.     */
/* y_i = g_s alpha o_s + g_lr o_lr: the multiplier scales the sparse branch   */
/* only ([C]), then each branch is weighted by its own gate.                  */
/* ------------------------------------------------------------------------- */
void oracle_fuse(const double *o_s, const double *lse, const double *o_lr,
                 const double *z_lr, const double *g_s, const double *g_lr,
                 double lambda, long rows, int d, double *alpha, double *y) {
  long idx;
#pragma omp parallel for schedule(static)
  for (idx = 0; idx < rows; ++idx) {
    const double mass_lr = lambda * z_lr[idx];
    double a = 1.0;
    if (mass_lr > 0.0) a = 1.0 / (1.0 + exp(log(mass_lr) - lse[idx]));
    if (alpha) alpha[idx] = a;
    for (int e = 0; e < d; ++e)
      y[(size_t)idx * d + e] = g_s[idx] * a * o_s[(size_t)idx * d + e] +
                               g_lr[idx] * o_lr[(size_t)idx * d + e];
  }
}

/* ------------------------------------------------------------------------- */
/* Backward pass: the exact gradient of the forward output above, for          */
/* training ("ELSAA: Efficient Low-Rank and Sparse Attention Approximation for */
/* Training Transformers", first paragraph: a framework for training, with a   */
/* learnable lambda; "ELSAA combines sparsity and low-rank methods to reduce   */
/* transformer attention complexity": it acts on the attention computation at */
/* run time, so gradients flow through it).  Given dL/dy, it returns dL/dq,    */
/* dL/dk, dL/dv, dL/dx_gate, dL/dW_g, dL/db_g and dL/dlambda.  Hash codes,     */
/* permutations and bucket counts are piecewise constant in the inputs and     */
/* carry no gradient.  Derivation, per query i (original index):               */
/*   y = c_s o_s + c_lr o_lr with (c_s, c_lr) = (g_s alpha, g_lr) for the full */
/*   operator, (g_s, g_lr) with alpha fixed to one, (0, 1) RACE only, (1, 0)   */
/*   sparse only;                                                              */
/*   alpha = Z_s / (Z_s + lambda Z_lr), Z_s = exp(lse):                        */
/*     d alpha / d lse = alpha (1 - alpha),                                    */
/*     d alpha / d lambda = -alpha^2 Z_lr / Z_s;                               */
/*   sparse branch: p_ij = exp(s_ij - lse_i) over the window, o_s = sum p v,   */
/*     lse = log sum exp s:  with do = dL/do_s and D_i = do_i . o_s,i,         */
/*     ds_ij = p_ij (do_i . v_j - D_i + dL/dlse_i), s_ij = q_i . k_j / sqrt d; */
/*   low-rank branch: o_lr = num / Z_lr, num = (1/L) sum_l T_l[c_l(q)], Z_lr   */
/*     constant: dT_l[b] = (1/L) sum over queries in bucket b of do_lr / Z_lr, */
/*     and dv_j = sum_l dT_l[c_l(k_j)] (T_l[b] sums the values of its keys);   */
/*   gates: g = sigmoid(a), da = dg g (1 - g), a = <x_gate, W> + b.            */
/* Arrays are [B][H][n][...] (x_gate [B][n][dg], W_g [2][H][dg], b_g [2][H]);  */
/* perms [B H][n], RACE codes [B H][n][L].  The outputs are overwritten.       */
/* ------------------------------------------------------------------------- */
int oracle_backward(const double *q, const double *k, const double *v, const double *x_gate,
                    const double *gate_w, const int32_t *perm_q, const int32_t *perm_k,
                    const int32_t *rq, const int32_t *rk, const double *o_s, const double *lse,
                    const double *o_lr, const double *z_lr, const double *g_s, const double *g_lr,
                    const double *alpha, const double *dy, int B, int H, int n, int d, int dg,
                    int w, int L, int P, double lambda, int variant, double *dq, double *dk,
                    double *dv, double *dx_gate, double *dgate_w, double *dgate_b,
                    double *dlambda) {
  const long segs = (long)B * H;
  const long rows = segs * n;
  const long nb = 1L << P;
  const double scale = 1.0 / sqrt((double)d);
  double *da_s = (double *)calloc((size_t)rows, sizeof(double));
  double *da_lr = (double *)calloc((size_t)rows, sizeof(double));
  double *dlam_seg = (double *)calloc((size_t)segs, sizeof(double));
  int fail = (!da_s || !da_lr || !dlam_seg);
  long s;
  if (!fail) {
#pragma omp parallel for schedule(dynamic) reduction(| : fail)
    for (s = 0; s < segs; ++s) {
      const size_t base = (size_t)s * n;
      double *do_s = (double *)malloc(sizeof(double) * (size_t)n * d);
      double *dlse = (double *)malloc(sizeof(double) * (size_t)n);
      double *dT = (double *)calloc((size_t)L * nb * d, sizeof(double));
      if (!do_s || !dlse || !dT) {
        free(do_s); free(dlse); free(dT);
        fail = 1;
        continue;
      }
      for (size_t e = base * d; e < (base + n) * d; ++e) dq[e] = dk[e] = dv[e] = 0.0;
      double dlam = 0.0;
      /* 1. the fusion, per query */
      for (int i = 0; i < n; ++i) {
        const size_t r = base + i;
        const double *dyi = dy + r * d, *osi = o_s + r * d, *olri = o_lr + r * d;
        double dy_os = 0.0, dy_olr = 0.0;
        for (int e = 0; e < d; ++e) {
          dy_os += dyi[e] * osi[e];
          dy_olr += dyi[e] * olri[e];
        }
        double c_s, c_lr;
        dlse[i] = 0.0;
        if (variant == 0) {  /* full operator */
          c_s = g_s[r] * alpha[r];
          c_lr = g_lr[r];
          const double dalpha = g_s[r] * dy_os;
          dlse[i] = dalpha * alpha[r] * (1.0 - alpha[r]);
          if (z_lr[r] > 0.0) dlam += dalpha * (-alpha[r] * alpha[r] * exp(log(z_lr[r]) - lse[r]));
          da_s[r] = alpha[r] * dy_os * g_s[r] * (1.0 - g_s[r]);
          da_lr[r] = dy_olr * g_lr[r] * (1.0 - g_lr[r]);
        } else if (variant == 1) {  /* alpha fixed to one */
          c_s = g_s[r];
          c_lr = g_lr[r];
          da_s[r] = dy_os * g_s[r] * (1.0 - g_s[r]);
          da_lr[r] = dy_olr * g_lr[r] * (1.0 - g_lr[r]);
        } else if (variant == 2) {  /* RACE only */
          c_s = 0.0;
          c_lr = 1.0;
        } else {  /* sparse only */
          c_s = 1.0;
          c_lr = 0.0;
        }
        for (int e = 0; e < d; ++e) do_s[(size_t)i * d + e] = c_s * dyi[e];
        /* low-rank branch: scatter do_lr / (L Z_lr) into the query's buckets */
        if (c_lr != 0.0 && z_lr[r] > 0.0) {
          for (int l = 0; l < L; ++l) {
            double *t = dT + ((size_t)l * nb + rq[r * L + l]) * d;
            for (int e = 0; e < d; ++e) t[e] += c_lr * dyi[e] / ((double)L * z_lr[r]);
          }
        }
      }
      dlam_seg[s] = dlam;
      /* 2. sparse branch: every (query, key) pair of every window */
      for (int rank = 0; rank < n; ++rank) {
        const int c = rank / w;
        const int lo = c > 0 ? (c - 1) * w : 0;
        const int hi = (c + 1) * w;
        const int i = perm_q[base + rank];
        const double *qi = q + (base + i) * d, *doi = do_s + (size_t)i * d, *osi = o_s + (base + i) * d;
        double D = 0.0;
        for (int e = 0; e < d; ++e) D += doi[e] * osi[e];
        for (int t = lo; t < hi; ++t) {
          const int j = perm_k[base + t];
          const double *kj = k + (base + j) * d, *vj = v + (base + j) * d;
          double sij = 0.0, dp = 0.0;
          for (int e = 0; e < d; ++e) {
            sij += qi[e] * kj[e];
            dp += doi[e] * vj[e];
          }
          const double p = exp(sij * scale - lse[base + i]);
          const double ds = p * (dp - D + dlse[i]);
          for (int e = 0; e < d; ++e) {
            dq[(base + i) * d + e] += ds * kj[e] * scale;
            dk[(base + j) * d + e] += ds * qi[e] * scale;
            dv[(base + j) * d + e] += p * doi[e];
          }
        }
      }
      /* 3. low-rank branch: each key collects its buckets' gradients */
      for (int j = 0; j < n; ++j) {
        for (int l = 0; l < L; ++l) {
          const double *t = dT + ((size_t)l * nb + rk[(base + j) * L + l]) * d;
          for (int e = 0; e < d; ++e) dv[(base + j) * d + e] += t[e];
        }
      }
      free(do_s); free(dlse); free(dT);
    }
  }
  if (fail) {
    free(da_s); free(da_lr); free(dlam_seg);
    return -1;
  }
  /* 4. gates: dW_g, db_g over every (batch, token); dx_gate over the heads */
  for (long e = 0; e < 2L * H * dg; ++e) dgate_w[e] = 0.0;
  for (long e = 0; e < 2L * H; ++e) dgate_b[e] = 0.0;
  for (long e = 0; e < (long)B * n * dg; ++e) dx_gate[e] = 0.0;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int i = 0; i < n; ++i) {
        const size_t r = ((size_t)b * H + h) * n + i;
        const double *x = x_gate + ((size_t)b * n + i) * dg;
        double *dx = dx_gate + ((size_t)b * n + i) * dg;
        const double *w0 = gate_w + (size_t)h * dg, *w1 = gate_w + ((size_t)H + h) * dg;
        double *dw0 = dgate_w + (size_t)h * dg, *dw1 = dgate_w + ((size_t)H + h) * dg;
        for (int e = 0; e < dg; ++e) {
          dw0[e] += da_s[r] * x[e];
          dw1[e] += da_lr[r] * x[e];
          dx[e] += da_s[r] * w0[e] + da_lr[r] * w1[e];
        }
        dgate_b[h] += da_s[r];
        dgate_b[H + h] += da_lr[r];
      }
  double dl = 0.0;
  for (s = 0; s < segs; ++s) dl += dlam_seg[s];
  *dlambda = variant == 0 ? dl : 0.0;
  (void)lambda;
  free(da_s); free(da_lr); free(dlam_seg);
  return 0;
}
