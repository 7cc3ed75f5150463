/*
 * Retention oracle: plain, slow, fp64 CPU reference for multi-scale retention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library; the two are built
 * separately and neither includes or links the other.
 *
 * Sources (the web pages this build follows):
 *   [P2] "Retentive Network: A Successor to Transformer for Large Language
 *        Models" -- paper summary, blog.csdn.net/weixin_45378275/article/
 *        details/132817411.  Sec. 2.1 "Retention" (recurrence, diagonalisation,
 *        scalar-gamma form, and the three representations: (1) parallel,
 *        (2) recurrent, (3) chunkwise recurrent) and Sec. 2.2 "Gated
 *        Multi-Scale Retention" (gamma per head, GroupNorm, swish gate).
 *   [P1] "RetNet dual-mode hands-on manual", lanjinlin.com.cn/news/2041318.
 *        Sec. 1 (the decay matrix), Sec. 3.1 (parallel/recurrent equivalence).
 *
 * Conventions (readings of the pages where they leave a choice open):
 *   - Arrays are row-major fp64.  Q, K: [B,H,L,dk]; V, O: [B,H,L,dv];
 *     state S: [B,H,dk,dv].  Token n of a call sits at absolute position
 *     p = pos0 + n (0-based).
 *   - Rotation pairs coordinates (2i, 2i+1) as the complex number
 *     x_{2i} + i*x_{2i+1} and multiplies it by exp(i*p*theta_i).  Q and K are
 *     rotated the same way; the score is the real part of q_rot * conj(k_rot),
 *     i.e. the real dot product of the rotated vectors (P2 Sec. 2.1, the
 *     conjugate-transpose form of scalar-gamma retention).
 *   - theta == NULL means no rotation.
 *   - Decay D[n][m] = gamma^(n-m) for n >= m, else 0 (P2 Sec. 2.1 (1);
 *     P1 Sec. 1).  pow(0, 0) == 1, so gamma = 0 gives D = I.
 *   - No 1/sqrt(dk) scaling anywhere: the formulas have none.
 *
 * Every function below is pinned by a CPU test against closed forms,
 * special cases, brute force or a library routine (tests/test_oracle_*.py).
 */
#include <complex.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>


/* Rotate one row x[0..dk) that sits at absolute position p (P2 Sec. 2.1:
 * Q is multiplied by Theta_n = exp(i n theta), K by its conjugate inside the
 * conjugate-transpose).  out may not alias x. */
static void rotate_row(const double *x, long dk, long long p, const double *theta,
                       double *out) {
  if (!theta) {
    memcpy(out, x, sizeof(double) * dk);
    return;
  }
  for (long i = 0; i < dk / 2; ++i) {
    double ang = (double)p * theta[i];
    double c = cos(ang), s = sin(ang);
    double re = x[2 * i], im = x[2 * i + 1];
    out[2 * i] = re * c - im * s;
    out[2 * i + 1] = re * s + im * c;
  }
  if (dk & 1) out[dk - 1] = x[dk - 1]; /* an unpaired last coordinate is not rotated */
}

/* Rotate a whole [BH, L, dk] tensor into out. */
void orc_rotate(const double *x, double *out, long BH, long L, long dk, const double *theta,
                long long pos0) {
#pragma omp parallel for collapse(2) schedule(static)
  for (long u = 0; u < BH; ++u)
    for (long n = 0; n < L; ++n)
      rotate_row(x + (u * L + n) * dk, dk, pos0 + n, theta, out + (u * L + n) * dk);
}

static double dot(const double *a, const double *b, long d) {
  double s = 0.0;
  for (long j = 0; j < d; ++j) s += a[j] * b[j];
  return s;
}

/* Parallel representation, P2 Sec. 2.1 (1): Retention(X) = (Q K^T (.) D) V,
 * written as the literal double sum o_n = sum_{m<=n} gamma^(n-m) (q_n . k_m) v_m
 * on rotated q, k. */
void orc_parallel(const double *q, const double *k, const double *v, double *o, long B, long H,
                  long L, long dk, long dv, const double *gamma, const double *theta,
                  long long pos0) {
  double *qr = malloc(sizeof(double) * B * H * L * dk);
  double *kr = malloc(sizeof(double) * B * H * L * dk);
  orc_rotate(q, qr, B * H, L, dk, theta, pos0);
  orc_rotate(k, kr, B * H, L, dk, theta, pos0);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (long u = 0; u < B * H; ++u)
    for (long n = 0; n < L; ++n) {
      double g = gamma[u % H];
      double *on = o + (u * L + n) * dv;
      for (long j = 0; j < dv; ++j) on[j] = 0.0;
      for (long m = 0; m <= n; ++m) {
        double d = pow(g, (double)(n - m));
        double a = dot(qr + (u * L + n) * dk, kr + (u * L + m) * dk, dk);
        const double *vm = v + (u * L + m) * dv;
        for (long j = 0; j < dv; ++j) on[j] += d * a * vm[j];
      }
    }
  free(qr);
  free(kr);
}

/* Complex transcription of the scalar-gamma form, P2 Sec. 2.1:
 * o_n = sum_{m<=n} gamma^(n-m) (Q_n e^{i n theta}) (K_m e^{i m theta})^dagger v_m,
 * with Q_n, K_m viewed as vectors in C^(dk/2) (pairs (2i, 2i+1)); the real part
 * of the scalar is taken.  Independent of rotate_row: used to pin it. */
void orc_parallel_complex(const double *q, const double *k, const double *v, double *o, long B,
                          long H, long L, long dk, long dv, const double *gamma,
                          const double *theta, long long pos0) {
  long P = dk / 2;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (long u = 0; u < B * H; ++u)
    for (long n = 0; n < L; ++n) {
      double g = gamma[u % H];
      double *on = o + (u * L + n) * dv;
      for (long j = 0; j < dv; ++j) on[j] = 0.0;
      for (long m = 0; m <= n; ++m) {
        double complex acc = 0.0;
        for (long i = 0; i < P; ++i) {
          const double *qn = q + (u * L + n) * dk, *km = k + (u * L + m) * dk;
          double complex qh = qn[2 * i] + I * qn[2 * i + 1];
          double complex kh = km[2 * i] + I * km[2 * i + 1];
          double th = theta ? theta[i] : 0.0;
          double complex a = qh * cexp(I * (double)(pos0 + n) * th);
          double complex b = kh * cexp(I * (double)(pos0 + m) * th);
          acc += a * conj(b);
        }
        double w = pow(g, (double)(n - m)) * creal(acc);
        const double *vm = v + (u * L + m) * dv;
        for (long j = 0; j < dv; ++j) on[j] += w * vm[j];
      }
    }
}

/* Recurrent representation, P2 Sec. 2.1 (2): S_n = gamma S_{n-1} + K_n^T V_n
 * (an outer product, dk x dv), Retention(X_n) = Q_n S_n.  s_in may be NULL
 * (zero state); s_out may be NULL. */
void orc_recurrent(const double *q, const double *k, const double *v, double *o, long B, long H,
                   long L, long dk, long dv, const double *gamma, const double *theta,
                   long long pos0, const double *s_in, double *s_out) {
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < B * H; ++u) {
    double g = gamma[u % H];
    double *S = calloc(dk * dv, sizeof(double));
    double *qr = malloc(sizeof(double) * dk), *kr = malloc(sizeof(double) * dk);
    if (s_in) memcpy(S, s_in + u * dk * dv, sizeof(double) * dk * dv);
    for (long n = 0; n < L; ++n) {
      rotate_row(q + (u * L + n) * dk, dk, pos0 + n, theta, qr);
      rotate_row(k + (u * L + n) * dk, dk, pos0 + n, theta, kr);
      const double *vn = v + (u * L + n) * dv;
      for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) S[i * dv + j] = g * S[i * dv + j] + kr[i] * vn[j];
      double *on = o + (u * L + n) * dv;
      for (long j = 0; j < dv; ++j) on[j] = 0.0;
      for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) on[j] += qr[i] * S[i * dv + j];
    }
    if (s_out) memcpy(s_out + u * dk * dv, S, sizeof(double) * dk * dv);
    free(S);
    free(qr);
    free(kr);
  }
}

/* Chunkwise recurrent representation, P2 Sec. 2.1 (3): parallel inside a
 * chunk, recurrent across chunks.  The pages give it in words only; the form
 * here is obtained from the recurrence by induction (the state entering chunk
 * c is S_c, chunk c holds tokens c0..c0+Cc-1, the last chunk may be short):
 *   o_{c0+j} = gamma^(j+1) q_{c0+j} S_c + sum_{i<=j} gamma^(j-i) (q_{c0+j} . k_{c0+i}) v_{c0+i}
 *   S_{c+1}  = gamma^Cc S_c + sum_i gamma^(Cc-1-i) k_{c0+i}^T v_{c0+i}
 * with all q, k rotated at their absolute positions. */
void orc_chunkwise(const double *q, const double *k, const double *v, double *o, long B, long H,
                   long L, long dk, long dv, long chunk, const double *gamma,
                   const double *theta, long long pos0, const double *s_in, double *s_out) {
  double *qr = malloc(sizeof(double) * B * H * L * dk);
  double *kr = malloc(sizeof(double) * B * H * L * dk);
  orc_rotate(q, qr, B * H, L, dk, theta, pos0);
  orc_rotate(k, kr, B * H, L, dk, theta, pos0);
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < B * H; ++u) {
    double g = gamma[u % H];
    double *S = calloc(dk * dv, sizeof(double));
    double *Sn = malloc(sizeof(double) * dk * dv);
    if (s_in) memcpy(S, s_in + u * dk * dv, sizeof(double) * dk * dv);
    for (long c0 = 0; c0 < L; c0 += chunk) {
      long Cc = (L - c0 < chunk) ? (L - c0) : chunk;
      for (long j = 0; j < Cc; ++j) {
        const double *qn = qr + (u * L + c0 + j) * dk;
        double *on = o + (u * L + c0 + j) * dv;
        double xi = pow(g, (double)(j + 1));
        for (long jj = 0; jj < dv; ++jj) {
          double cross = 0.0;
          for (long i = 0; i < dk; ++i) cross += qn[i] * S[i * dv + jj];
          on[jj] = xi * cross;
        }
        for (long i = 0; i <= j; ++i) {
          double w = pow(g, (double)(j - i)) * dot(qn, kr + (u * L + c0 + i) * dk, dk);
          const double *vi = v + (u * L + c0 + i) * dv;
          for (long jj = 0; jj < dv; ++jj) on[jj] += w * vi[jj];
        }
      }
      double gc = pow(g, (double)Cc);
      for (long e = 0; e < dk * dv; ++e) Sn[e] = gc * S[e];
      for (long i = 0; i < Cc; ++i) {
        double zeta = pow(g, (double)(Cc - 1 - i));
        const double *ki = kr + (u * L + c0 + i) * dk;
        const double *vi = v + (u * L + c0 + i) * dv;
        for (long a = 0; a < dk; ++a)
          for (long b = 0; b < dv; ++b) Sn[a * dv + b] += zeta * ki[a] * vi[b];
      }
      memcpy(S, Sn, sizeof(double) * dk * dv);
    }
    if (s_out) memcpy(s_out + u * dk * dv, S, sizeof(double) * dk * dv);
    free(S);
    free(Sn);
  }
  free(qr);
  free(kr);
}

/* Selected output rows of the defining sum (P2 Sec. 2.1, scalar-gamma form),
 * one by one, for spot checks at sizes where a full oracle run is too slow.
 * idx holds nidx triples (b, h, n); out receives nidx rows of dv values.
 * s_in (may be NULL) is the state entering token 0: it adds
 * gamma^(n+1) q_n S_in, the recurrence unrolled over the tokens before the call. */
void orc_rows(const double *q, const double *k, const double *v, long B, long H, long L,
              long dk, long dv, const double *gamma, const double *theta, long long pos0,
              const double *s_in, const long *idx, long nidx, double *out) {
#pragma omp parallel for schedule(dynamic)
  for (long r = 0; r < nidx; ++r) {
    long b = idx[3 * r], h = idx[3 * r + 1], n = idx[3 * r + 2];
    if (b < 0 || b >= B || h < 0 || h >= H || n < 0 || n >= L) {
      for (long j = 0; j < dv; ++j) out[r * dv + j] = NAN;
      continue;
    }
    long u = b * H + h;
    double g = gamma[h];
    double *qn = malloc(sizeof(double) * dk), *km = malloc(sizeof(double) * dk);
    rotate_row(q + (u * L + n) * dk, dk, pos0 + n, theta, qn);
    double *on = out + r * dv;
    for (long j = 0; j < dv; ++j) on[j] = 0.0;
    if (s_in) {
      double xi = pow(g, (double)(n + 1));
      const double *S = s_in + u * dk * dv;
      for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) on[j] += xi * qn[i] * S[i * dv + j];
    }
    for (long m = 0; m <= n; ++m) {
      rotate_row(k + (u * L + m) * dk, dk, pos0 + m, theta, km);
      double w = pow(g, (double)(n - m)) * dot(qn, km, dk);
      const double *vm = v + (u * L + m) * dv;
      for (long j = 0; j < dv; ++j) on[j] += w * vm[j];
    }
    free(qn);
    free(km);
  }
}

/* The transpose of the rotation at position p: pair i multiplied by
 * exp(-i p theta_i).  The rotation is orthogonal, so this is also its inverse. */
static void unrotate_row(const double *x, long dk, long long p, const double *theta, double *out) {
  if (!theta) {
    memcpy(out, x, sizeof(double) * dk);
    return;
  }
  for (long i = 0; i < dk / 2; ++i) {
    double ang = (double)p * theta[i];
    double c = cos(ang), s = sin(ang);
    double re = x[2 * i], im = x[2 * i + 1];
    out[2 * i] = re * c + im * s;
    out[2 * i + 1] = -re * s + im * c;
  }
  if (dk & 1) out[dk - 1] = x[dk - 1];
}

/* Gradients of the defining sum (P2 Sec. 2.1, scalar-gamma form; no GroupNorm)
 * with respect to q, k and v, for an output gradient dO.  With a_nm =
 * gamma^(n-m) for n >= m and the rotated rows q~, k~:
 *   dv_m  = sum_{n >= m} a_nm (q~_n . k~_m) dO_n
 *   dq~_n = sum_{m <= n} a_nm (dO_n . v_m) k~_m,   dq_n = R_n^T dq~_n
 *   dk~_m = sum_{n >= m} a_nm (dO_n . v_m) q~_n,   dk_m = R_m^T dk~_m
 * (each term of o_n is bilinear in (q~_n, k~_m) and linear in v_m).  Written
 * as one double loop over n >= m per (b, h). */
void orc_backward(const double *q, const double *k, const double *v, const double *dO, long B, long H,
                  long L, long dk, long dv, const double *gamma, const double *theta, long long pos0,
                  double *dq, double *dkk, double *dvv) {
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < B * H; ++u) {
    long h = u % H;
    double g = gamma[h];
    double *qr = malloc(sizeof(double) * L * dk), *kr = malloc(sizeof(double) * L * dk);
    double *dqr = calloc(L * dk, sizeof(double)), *dkr = calloc(L * dk, sizeof(double));
    for (long n = 0; n < L; ++n) {
      rotate_row(q + (u * L + n) * dk, dk, pos0 + n, theta, qr + n * dk);
      rotate_row(k + (u * L + n) * dk, dk, pos0 + n, theta, kr + n * dk);
    }
    double *dvu = dvv + u * L * dv;
    for (long i = 0; i < L * dv; ++i) dvu[i] = 0.0;
    for (long n = 0; n < L; ++n) {
      const double *don = dO + (u * L + n) * dv;
      for (long m = 0; m <= n; ++m) {
        double a = pow(g, (double)(n - m));
        double s = dot(qr + n * dk, kr + m * dk, dk);
        double t = dot(don, v + (u * L + m) * dv, dv);
        for (long j = 0; j < dv; ++j) dvu[m * dv + j] += a * s * don[j];
        for (long i = 0; i < dk; ++i) {
          dqr[n * dk + i] += a * t * kr[m * dk + i];
          dkr[m * dk + i] += a * t * qr[n * dk + i];
        }
      }
    }
    for (long n = 0; n < L; ++n) {
      unrotate_row(dqr + n * dk, dk, pos0 + n, theta, dq + (u * L + n) * dk);
      unrotate_row(dkr + n * dk, dk, pos0 + n, theta, dkk + (u * L + n) * dk);
    }
    free(qr);
    free(kr);
    free(dqr);
    free(dkr);
  }
}

/* The same gradients from the recurrent representation (P2 Sec. 2.1 (2)) by
 * its adjoint, a derivation independent of the double sum above and O(L dk dv)
 * per (b, h).  The forward state S_n = gamma S_{n-1} + k~_n^T v_n (zero before
 * token 0) gives o_n = q~_n S_n, so
 *   dq~_n = S_n dO_n^T                                  (forward sweep)
 * and the reverse-time state G_n = gamma G_{n+1} + q~_n^T dO_n (zero after the
 * last token), which gathers the pull of every query at or after n, gives
 *   dk~_n = G_n v_n^T,   dv_n = k~_n G_n                 (backward sweep)
 * with dq_n = R_n^T dq~_n and dk_n = R_n^T dk~_n. */
void orc_backward_recurrent(const double *q, const double *k, const double *v, const double *dO, long B,
                            long H, long L, long dk, long dv, const double *gamma, const double *theta,
                            long long pos0, double *dq, double *dkk, double *dvv) {
#pragma omp parallel for schedule(dynamic)
  for (long u = 0; u < B * H; ++u) {
    double g = gamma[u % H];
    double *S = calloc(dk * dv, sizeof(double));
    double *xr = malloc(sizeof(double) * dk), *acc = malloc(sizeof(double) * dk);
    for (long n = 0; n < L; ++n) { /* forward sweep: dq */
      rotate_row(k + (u * L + n) * dk, dk, pos0 + n, theta, xr);
      const double *vn = v + (u * L + n) * dv, *don = dO + (u * L + n) * dv;
      for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) S[i * dv + j] = g * S[i * dv + j] + xr[i] * vn[j];
      for (long i = 0; i < dk; ++i) acc[i] = dot(S + i * dv, don, dv);
      unrotate_row(acc, dk, pos0 + n, theta, dq + (u * L + n) * dk);
    }
    double *G = S;
    for (long i = 0; i < dk * dv; ++i) G[i] = 0.0;
    for (long n = L - 1; n >= 0; --n) { /* backward sweep: dk, dv */
      rotate_row(q + (u * L + n) * dk, dk, pos0 + n, theta, xr);
      const double *vn = v + (u * L + n) * dv, *don = dO + (u * L + n) * dv;
      for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) G[i * dv + j] = g * G[i * dv + j] + xr[i] * don[j];
      for (long i = 0; i < dk; ++i) acc[i] = dot(G + i * dv, vn, dv);
      unrotate_row(acc, dk, pos0 + n, theta, dkk + (u * L + n) * dk);
      rotate_row(k + (u * L + n) * dk, dk, pos0 + n, theta, xr);
      double *dvn = dvv + (u * L + n) * dv;
      for (long j = 0; j < dv; ++j) dvn[j] = 0.0;
      for (long i = 0; i < dk; ++i)
        for (long j = 0; j < dv; ++j) dvn[j] += xr[i] * G[i * dv + j];
    }
    free(S);
    free(xr);
    free(acc);
  }
}

/* Selected rows of the gradients above: which = 0 gives dq row n (a sum over
 * m <= n), 1 gives dk row n and 2 gives dv row n (sums over later tokens).
 * idx holds (b, h, n) triples; out receives dk values per row for which 0 and 1,
 * dv values for which 2 (NaN for an index out of range). */
void orc_backward_rows(const double *q, const double *k, const double *v, const double *dO, long B,
                       long H, long L, long dk, long dv, const double *gamma, const double *theta,
                       long long pos0, int which, const long *idx, long nidx, double *out) {
  const long w = which == 2 ? dv : dk;
#pragma omp parallel for schedule(dynamic)
  for (long r = 0; r < nidx; ++r) {
    long b = idx[3 * r], h = idx[3 * r + 1], n = idx[3 * r + 2];
    double *o = out + r * w;
    if (b < 0 || b >= B || h < 0 || h >= H || n < 0 || n >= L || which < 0 || which > 2) {
      for (long j = 0; j < w; ++j) o[j] = NAN;
      continue;
    }
    long u = b * H + h;
    double g = gamma[h];
    double *xr = malloc(sizeof(double) * dk), *yr = malloc(sizeof(double) * dk);
    double *acc = calloc(w, sizeof(double));
    if (which == 0) { /* dq~_n = sum_{m <= n} a_nm (dO_n . v_m) k~_m */
      const double *don = dO + (u * L + n) * dv;
      for (long m = 0; m <= n; ++m) {
        rotate_row(k + (u * L + m) * dk, dk, pos0 + m, theta, xr);
        double c = pow(g, (double)(n - m)) * dot(don, v + (u * L + m) * dv, dv);
        for (long i = 0; i < dk; ++i) acc[i] += c * xr[i];
      }
      unrotate_row(acc, dk, pos0 + n, theta, o);
    } else if (which == 1) { /* dk~_n = sum_{t >= n} a_tn (dO_t . v_n) q~_t */
      const double *vn = v + (u * L + n) * dv;
      for (long t = n; t < L; ++t) {
        rotate_row(q + (u * L + t) * dk, dk, pos0 + t, theta, xr);
        double c = pow(g, (double)(t - n)) * dot(dO + (u * L + t) * dv, vn, dv);
        for (long i = 0; i < dk; ++i) acc[i] += c * xr[i];
      }
      unrotate_row(acc, dk, pos0 + n, theta, o);
    } else { /* dv_n = sum_{t >= n} a_tn (q~_t . k~_n) dO_t */
      rotate_row(k + (u * L + n) * dk, dk, pos0 + n, theta, yr);
      for (long t = n; t < L; ++t) {
        rotate_row(q + (u * L + t) * dk, dk, pos0 + t, theta, xr);
        double c = pow(g, (double)(t - n)) * dot(xr, yr, dk);
        const double *dot_ = dO + (u * L + t) * dv;
        for (long j = 0; j < dv; ++j) acc[j] += c * dot_[j];
      }
      for (long j = 0; j < dv; ++j) o[j] = acc[j];
    }
    free(xr);
    free(yr);
    free(acc);
  }
}

/* Selected entries of the state after all L tokens of a call: the recurrence
 * S_n = gamma S_{n-1} + k_n^T v_n (P2 Sec. 2.1 (2)) unrolled,
 *   S_L[a][b] = gamma^L S_in[a][b] + sum_m gamma^(L-1-m) k_m[a] v_m[b].
 * idx holds nidx quadruples (b, h, a, bcol). */
void orc_state_entries(const double *k, const double *v, long B, long H, long L, long dk,
                       long dv, const double *gamma, const double *theta, long long pos0,
                       const double *s_in, const long *idx, long nidx, double *out) {
#pragma omp parallel for schedule(dynamic)
  for (long r = 0; r < nidx; ++r) {
    long b = idx[4 * r], h = idx[4 * r + 1], a = idx[4 * r + 2], c = idx[4 * r + 3];
    if (b < 0 || b >= B || h < 0 || h >= H || a < 0 || a >= dk || c < 0 || c >= dv) {
      out[r] = NAN;
      continue;
    }
    long u = b * H + h;
    double g = gamma[h];
    double *km = malloc(sizeof(double) * dk);
    double acc = s_in ? pow(g, (double)L) * s_in[(u * dk + a) * dv + c] : 0.0;
    for (long m = 0; m < L; ++m) {
      rotate_row(k + (u * L + m) * dk, dk, pos0 + m, theta, km);
      acc += pow(g, (double)(L - 1 - m)) * km[a] * v[(u * L + m) * dv + c];
    }
    out[r] = acc;
    free(km);
  }
}

/* Per-head GroupNorm of P2 Sec. 2.2 ("GroupNorm normalises each head's
 * output"): every row of dv values (one token, one head) is shifted to mean 0
 * and divided by sqrt(var + eps), biased variance, no affine. In place. */
void orc_groupnorm(double *x, long rows, long dv, double eps) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) {
    double *xr = x + r * dv;
    double mu = 0.0;
    for (long j = 0; j < dv; ++j) mu += xr[j];
    mu /= (double)dv;
    double var = 0.0;
    for (long j = 0; j < dv; ++j) var += (xr[j] - mu) * (xr[j] - mu);
    var /= (double)dv;
    double inv = 1.0 / sqrt(var + eps);
    for (long j = 0; j < dv; ++j) xr[j] = (xr[j] - mu) * inv;
  }
}

/* y[M][N] = x[M][K] . w^T, with w stored [N][K] (each output column's weights
 * contiguous).  A plain triple loop. */
void orc_matmul_nt(const double *x, const double *w, double *y, long M, long N, long K) {
#pragma omp parallel for collapse(2) schedule(static)
  for (long m = 0; m < M; ++m)
    for (long n = 0; n < N; ++n) y[m * N + n] = dot(x + m * K, w + n * K, K);
}

/* swish(x) = x * sigmoid(x) = x / (1 + exp(-x)) (P2 Sec. 2.2). In place. */
void orc_swish(double *x, long n) {
#pragma omp parallel for schedule(static)
  for (long i = 0; i < n; ++i) x[i] = x[i] / (1.0 + exp(-x[i]));
}

/* LayerNorm of the block equations (P2, the pre-LN residual block): each row of
 * d values becomes (x - mean) / sqrt(var + eps), biased variance, no affine
 * parameters (the identity they start from).  In place. */
void orc_layernorm(double *x, long rows, long d, double eps) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) {
    double *xr = x + r * d, mu = 0.0, var = 0.0;
    for (long j = 0; j < d; ++j) mu += xr[j];
    mu /= (double)d;
    for (long j = 0; j < d; ++j) var += (xr[j] - mu) * (xr[j] - mu);
    var /= (double)d;
    double inv = 1.0 / sqrt(var + eps);
    for (long j = 0; j < d; ++j) xr[j] = (xr[j] - mu) * inv;
  }
}

/* gelu of the FFN (P2: FFN(X) = gelu(X W_1) W_2), the exact form
 * x * Phi(x) = x (1 + erf(x / sqrt 2)) / 2.  In place. */
void orc_gelu(double *x, long n) {
#pragma omp parallel for schedule(static)
  for (long i = 0; i < n; ++i) x[i] = 0.5 * x[i] * (1.0 + erf(x[i] / sqrt(2.0)));
}
