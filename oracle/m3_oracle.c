/*
 * m3_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, sequential fp64 CPU evaluation of the Mamba-3 SSM core
 * recurrence.  It exists to check the HIP library; nothing in the library
 * may call, link or load it.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header or
 * constant with the HIP path.
 *
 * What it computes (one (batch, head) pair at a time, one token at a time):
 *
 *   exponential-trapezoidal three-term update
 *     [xxxxx.co.kr Mamba-3 article ("2배 작은 상태 크기와 향상된 MIMO 디코딩
 *      하드웨어 효율..."), section 1.1, the h_t equation]:
 *       alpha_t = exp(dt_t * A_t)
 *       beta_t  = (1 - lam_t) * dt_t * alpha_t
 *       gamma_t = lam_t * dt_t
 *       h_t = alpha_t h_{t-1} + beta_t B_{t-1} x_{t-1} + gamma_t B_t x_t
 *
 *   complex-valued state [same article, section 1.2 ("RoPE trick")]: the
 *     state's N columns are N/2 complex numbers (column 2k = real part,
 *     2k+1 = imaginary part).  The discretised transition of pair k is the
 *     complex number exp(dt_t (A_t + i theta_{t,k})); its modulus is
 *     alpha_t and its phase phi_{t,k} = dt_t * theta_{t,k}.  Both the
 *     decayed state and the left-endpoint (beta) term carry that factor;
 *     the right-endpoint (gamma) term is taken at the current time and is
 *     not rotated.  The output is the real dot product y = h C, i.e.
 *     Re(sum_k conj(c_k) h_k).
 *
 *   MIMO rank R [same article, section 1.3]: x_t is P x R, B_t and C_t are
 *     N x R, the input terms are the P x N matrix products X B^T and the
 *     output is the P x R matrix h C.  R = 1 is the single-input form.
 *
 * Readings where the pages leave a choice open (each is shared with the
 * HIP path and listed in the design notes): phase = dt * theta unless
 * M3REF_THETA_IS_ANGLE; theta has one angle per complex pair per head per
 * token; pairs are adjacent columns (2k, 2k+1); the state is multiplied by
 * e^{+i phi}; the token before t = 0 is x_prev/B_prev (zero when NULL);
 * A is per head unless M3REF_A_PER_TOKEN; dt and lam arrive already
 * activated; no skip term or gate is applied, and B and C enter the
 * recurrence as given (m3ref_bc_prep below prepares them when the
 * normalisation and bias of section 2 are wanted).
 *
 * Layouts (dense, row-major, last index fastest):
 *   x      [Bsz, T, H, P, R]      B, C  [Bsz, T, H, N, R]
 *   dt,lam [Bsz, T, H]            theta [Bsz, T, H, N/2]
 *   A      [H] (or [Bsz, T, H] with M3REF_A_PER_TOKEN)
 *   h0, hT [Bsz, H, P, N]         x_prev [Bsz, H, P, R]   B_prev [Bsz, H, N, R]
 *   y      [Bsz, T, H, P, R]
 * The decode step uses the same layouts without the T axis.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define M3REF_THETA_IS_ANGLE 1u
#define M3REF_A_PER_TOKEN 2u

typedef struct {
  int64_t batch, seqlen, nheads, headdim, dstate, rank;
  uint32_t flags;
} m3ref_dims;

/* One token of the recurrence for one (batch, head): S is P x N, updated in
 * place; xp/bp are the previous token's x (P x R) and B (N x R) or NULL for
 * zero; x/b/c the current token's; y (P x R) receives S C. */
static void m3ref_token(int64_t P, int64_t N, int64_t R, uint32_t flags,
                        double* S, const double* xp, const double* bp,
                        const double* x, const double* b, const double* c,
                        double dt, double A, double lam, const double* theta,
                        double* y) {
  const double alpha = exp(dt * A);
  const double beta = (1.0 - lam) * dt * alpha;
  const double gamma = lam * dt;

  /* decay, then the left-endpoint input term (both get the full-step factor) */
  for (int64_t p = 0; p < P; ++p)
    for (int64_t n = 0; n < N; ++n) {
      double s = alpha * S[p * N + n];
      if (xp && bp) {
        double u = 0.0;
        for (int64_t r = 0; r < R; ++r) u += xp[p * R + r] * bp[n * R + r];
        s += beta * u;
      }
      S[p * N + n] = s;
    }

  /* phase of the complex eigenvalue: rotate every (2k, 2k+1) pair by +phi */
  for (int64_t k = 0; k < N / 2; ++k) {
    const double phi = (flags & M3REF_THETA_IS_ANGLE) ? theta[k] : dt * theta[k];
    const double cs = cos(phi), sn = sin(phi);
    for (int64_t p = 0; p < P; ++p) {
      const double re = S[p * N + 2 * k], im = S[p * N + 2 * k + 1];
      S[p * N + 2 * k] = cs * re - sn * im;
      S[p * N + 2 * k + 1] = sn * re + cs * im;
    }
  }

  /* right-endpoint input term, taken at the current time: not rotated */
  for (int64_t p = 0; p < P; ++p)
    for (int64_t n = 0; n < N; ++n) {
      double u = 0.0;
      for (int64_t r = 0; r < R; ++r) u += x[p * R + r] * b[n * R + r];
      S[p * N + n] += gamma * u;
    }

  /* output y = S C  (P x R) */
  for (int64_t p = 0; p < P; ++p)
    for (int64_t r = 0; r < R; ++r) {
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) acc += S[p * N + n] * c[n * R + r];
      y[p * R + r] = acc;
    }
}

static int m3ref_check(const m3ref_dims* d) {
  if (!d) return 1;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads < 0) return 2;
  if (d->headdim <= 0 || d->dstate <= 0 || d->rank <= 0) return 2;
  if (d->dstate % 2) return 2;
  return 0;
}

/* Full sequential scan: y (and hT when non-NULL) from x, dt, A, lam, theta,
 * B, C, the initial state h0 (NULL = 0) and the token before the first one
 * (x_prev/B_prev, NULL = 0).  nthreads <= 0 lets OpenMP choose. */
int m3ref_scan(const m3ref_dims* d, const double* x, const double* dt,
               const double* A, const double* lam, const double* theta,
               const double* B, const double* C, const double* h0,
               const double* x_prev, const double* B_prev, double* y,
               double* hT, int nthreads) {
  int rc = m3ref_check(d);
  if (rc) return rc;
  const int64_t Bsz = d->batch, T = d->seqlen, H = d->nheads, P = d->headdim,
                N = d->dstate, R = d->rank;
  const int64_t units = Bsz * H;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t u = 0; u < units; ++u) {
    const int64_t b = u / H, h = u % H;
    double* S = (double*)malloc(sizeof(double) * P * N);
    if (h0)
      memcpy(S, h0 + (b * H + h) * P * N, sizeof(double) * P * N);
    else
      memset(S, 0, sizeof(double) * P * N);
    const double* xp = x_prev ? x_prev + (b * H + h) * P * R : NULL;
    const double* bp = B_prev ? B_prev + (b * H + h) * N * R : NULL;
    if (xp == NULL || bp == NULL) xp = bp = NULL; /* both or neither */
    for (int64_t t = 0; t < T; ++t) {
      const int64_t bth = (b * T + t) * H + h;
      const double* xt = x + bth * P * R;
      const double* bt = B + bth * N * R;
      const double* ct = C + bth * N * R;
      const double a = (d->flags & M3REF_A_PER_TOKEN) ? A[bth] : A[h];
      m3ref_token(P, N, R, d->flags, S, xp, bp, xt, bt, ct, dt[bth], a,
                  lam[bth], theta + bth * (N / 2), y + bth * P * R);
      xp = xt;
      bp = bt;
    }
    if (hT) memcpy(hT + (b * H + h) * P * N, S, sizeof(double) * P * N);
    free(S);
  }
  return 0;
}

/* One decode step: h (in/out, [Bsz,H,P,N]) advances by one token; y_t gets
 * the output.  x_prev/B_prev NULL = 0.  A is [H] (or [Bsz,H] with the
 * per-token flag).  seqlen is ignored. */
int m3ref_decode_step(const m3ref_dims* d, double* h, const double* x_t,
                      const double* x_prev, const double* B_t,
                      const double* B_prev, const double* C_t,
                      const double* dt_t, const double* A,
                      const double* lam_t, const double* theta_t, double* y_t,
                      int nthreads) {
  int rc = m3ref_check(d);
  if (rc) return rc;
  const int64_t Bsz = d->batch, H = d->nheads, P = d->headdim, N = d->dstate,
                R = d->rank;
  const int64_t units = Bsz * H;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t u = 0; u < units; ++u) {
    const int64_t h_ = u % H;
    const double* xp = (x_prev && B_prev) ? x_prev + u * P * R : NULL;
    const double* bp = (x_prev && B_prev) ? B_prev + u * N * R : NULL;
    const double a = (d->flags & M3REF_A_PER_TOKEN) ? A[u] : A[h_];
    m3ref_token(P, N, R, d->flags, h + u * P * N, xp, bp, x_t + u * P * R,
                B_t + u * N * R, C_t + u * N * R, dt_t[u], a, lam_t[u],
                theta_t + u * (N / 2), y_t + u * P * R);
  }
  return 0;
}

/*
 * Gradients of the scan (reverse-mode, the adjoint of the token recurrence
 * above, taken step by step in reverse order).  Given dL/dy (dy) and
 * dL/dhT (dhT, NULL = 0) it returns dL/d of every input: x, dt, A, lam,
 * theta, B, C, h0, x_prev, B_prev (any output may be NULL).  Per token t,
 * with U = alpha S_{t-1} + beta X_{t-1} B_{t-1}^T, W = R(phi) U and
 * S_t = W + gamma X_t B_t^T, and G the gradient of S_t:
 *   G += dy_t C_t^T;  dC_t = S_t^T dy_t;  dgamma = <G, X_t B_t^T>;
 *   dX_t += gamma G B_t;  dB_t += gamma G^T X_t;
 *   dphi_k = sum_p <G_pair, J W_pair>, J (a, b) = (-b, a)  (d R(phi)/dphi = J R(phi));
 *   V = R(-phi) G;  dalpha = <V, S_{t-1}>;  dbeta = <V, X_{t-1} B_{t-1}^T>;
 *   dX_{t-1} += beta V B_{t-1};  dB_{t-1} += beta V^T X_{t-1};  G <- alpha V;
 * then the chain through alpha = exp(dt A), beta = (1 - lam) dt alpha,
 * gamma = lam dt and phi = dt theta (theta with M3REF_THETA_IS_ANGLE).
 * dA is [H] (summed over batch and time) or [Bsz, T, H] with
 * M3REF_A_PER_TOKEN.  The forward states of a (batch, head) are kept
 * (T + 1 of them), so this is for small cases.
 */
int m3ref_scan_backward(const m3ref_dims* d, const double* x, const double* dt,
                        const double* A, const double* lam, const double* theta,
                        const double* B, const double* C, const double* h0,
                        const double* x_prev, const double* B_prev, const double* dy,
                        const double* dhT, double* dx, double* ddt, double* dA,
                        double* dlam, double* dtheta, double* dB, double* dC,
                        double* dh0, double* dx_prev, double* dB_prev, int nthreads) {
  int rc = m3ref_check(d);
  if (rc) return rc;
  if (!x || !dt || !A || !lam || !theta || !B || !C || !dy) return 3;
  const int64_t Bsz = d->batch, T = d->seqlen, H = d->nheads, P = d->headdim,
                N = d->dstate, R = d->rank, K = N / 2;
  const int64_t units = Bsz * H, PN = P * N;
  const int angle = (d->flags & M3REF_THETA_IS_ANGLE) != 0;
  const int a_tok = (d->flags & M3REF_A_PER_TOKEN) != 0;
  /* per-token dA, summed per head at the end unless A is per token */
  double* dA_tok = (double*)calloc((size_t)(Bsz * T * H > 0 ? Bsz * T * H : 1), sizeof(double));
  if (!dA_tok) return 4;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (int64_t u = 0; u < units; ++u) {
    const int64_t b = u / H, h = u % H;
    const int prev = x_prev && B_prev;
    const double* xp0 = prev ? x_prev + u * P * R : NULL;
    const double* bp0 = prev ? B_prev + u * N * R : NULL;
    /* forward: states S_{-1} .. S_{T-1} */
    double* St = (double*)calloc((size_t)((T + 1) * PN), sizeof(double));
    double* G = (double*)calloc((size_t)PN, sizeof(double));
    double* V = (double*)calloc((size_t)PN, sizeof(double));
    double* yt = (double*)calloc((size_t)(P * R), sizeof(double));
    double* gx = (double*)calloc((size_t)((T + 1) * P * R), sizeof(double));  /* dX_{-1..T-1} */
    double* gb = (double*)calloc((size_t)((T + 1) * N * R), sizeof(double));  /* dB_{-1..T-1} */
    if (h0) memcpy(St, h0 + u * PN, sizeof(double) * PN);
    for (int64_t t = 0; t < T; ++t) {
      const int64_t bth = (b * T + t) * H + h;
      memcpy(St + (t + 1) * PN, St + t * PN, sizeof(double) * PN);
      const double* xp = t == 0 ? xp0 : x + (bth - H) * P * R;
      const double* bp = t == 0 ? bp0 : B + (bth - H) * N * R;
      m3ref_token(P, N, R, d->flags, St + (t + 1) * PN, xp, bp, x + bth * P * R, B + bth * N * R,
                  C + bth * N * R, dt[bth], a_tok ? A[bth] : A[h], lam[bth], theta + bth * K, yt);
    }
    /* reverse */
    if (dhT) memcpy(G, dhT + u * PN, sizeof(double) * PN);
    for (int64_t t = T - 1; t >= 0; --t) {
      const int64_t bth = (b * T + t) * H + h;
      const double* S1 = St + (t + 1) * PN; /* S_t */
      const double* S0 = St + t * PN;       /* S_{t-1} */
      const double* xt = x + bth * P * R;
      const double* bt = B + bth * N * R;
      const double* ct = C + bth * N * R;
      const double* dyt = dy + bth * P * R;
      const double* xp = t == 0 ? xp0 : x + (bth - H) * P * R;
      const double* bp = t == 0 ? bp0 : B + (bth - H) * N * R;
      const double DT = dt[bth], LM = lam[bth], AA = a_tok ? A[bth] : A[h];
      const double alpha = exp(DT * AA), beta = (1.0 - LM) * DT * alpha, gamma = LM * DT;
      /* the output of token t */
      for (int64_t p = 0; p < P; ++p)
        for (int64_t n = 0; n < N; ++n) {
          double v = 0.0;
          for (int64_t r = 0; r < R; ++r) v += dyt[p * R + r] * ct[n * R + r];
          G[p * N + n] += v;
        }
      if (dC)
        for (int64_t n = 0; n < N; ++n)
          for (int64_t r = 0; r < R; ++r) {
            double v = 0.0;
            for (int64_t p = 0; p < P; ++p) v += S1[p * N + n] * dyt[p * R + r];
            dC[bth * N * R + n * R + r] = v;
          }
      /* the gamma term */
      double dgamma = 0.0;
      for (int64_t p = 0; p < P; ++p)
        for (int64_t n = 0; n < N; ++n) {
          double xb = 0.0;
          for (int64_t r = 0; r < R; ++r) xb += xt[p * R + r] * bt[n * R + r];
          dgamma += G[p * N + n] * xb;
        }
      for (int64_t p = 0; p < P; ++p)
        for (int64_t r = 0; r < R; ++r) {
          double v = 0.0;
          for (int64_t n = 0; n < N; ++n) v += G[p * N + n] * bt[n * R + r];
          gx[(t + 1) * P * R + p * R + r] += gamma * v;
        }
      for (int64_t n = 0; n < N; ++n)
        for (int64_t r = 0; r < R; ++r) {
          double v = 0.0;
          for (int64_t p = 0; p < P; ++p) v += G[p * N + n] * xt[p * R + r];
          gb[(t + 1) * N * R + n * R + r] += gamma * v;
        }
      /* the rotation: W = S_t - gamma X_t B_t^T */
      double dphi_dt = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const double phi = angle ? theta[bth * K + k] : DT * theta[bth * K + k];
        const double cs = cos(phi), sn = sin(phi);
        double dphi = 0.0;
        for (int64_t p = 0; p < P; ++p) {
          double w0 = S1[p * N + 2 * k], w1 = S1[p * N + 2 * k + 1];
          for (int64_t r = 0; r < R; ++r) {
            w0 -= gamma * xt[p * R + r] * bt[(2 * k) * R + r];
            w1 -= gamma * xt[p * R + r] * bt[(2 * k + 1) * R + r];
          }
          const double g0 = G[p * N + 2 * k], g1 = G[p * N + 2 * k + 1];
          dphi += -g0 * w1 + g1 * w0;
          V[p * N + 2 * k] = cs * g0 + sn * g1;
          V[p * N + 2 * k + 1] = -sn * g0 + cs * g1;
        }
        if (dtheta) dtheta[bth * K + k] = angle ? dphi : DT * dphi;
        dphi_dt += theta[bth * K + k] * dphi;
      }
      /* decay and the beta term */
      double dalpha = 0.0, dbeta = 0.0;
      for (int64_t p = 0; p < P; ++p)
        for (int64_t n = 0; n < N; ++n) {
          dalpha += V[p * N + n] * S0[p * N + n];
          if (xp) {
            double xb = 0.0;
            for (int64_t r = 0; r < R; ++r) xb += xp[p * R + r] * bp[n * R + r];
            dbeta += V[p * N + n] * xb;
          }
        }
      if (xp) {
        for (int64_t p = 0; p < P; ++p)
          for (int64_t r = 0; r < R; ++r) {
            double v = 0.0;
            for (int64_t n = 0; n < N; ++n) v += V[p * N + n] * bp[n * R + r];
            gx[t * P * R + p * R + r] += beta * v;
          }
        for (int64_t n = 0; n < N; ++n)
          for (int64_t r = 0; r < R; ++r) {
            double v = 0.0;
            for (int64_t p = 0; p < P; ++p) v += V[p * N + n] * xp[p * R + r];
            gb[t * N * R + n * R + r] += beta * v;
          }
      }
      for (int64_t i = 0; i < PN; ++i) G[i] = alpha * V[i];
      /* chain to dt, lam, A */
      if (ddt)
        ddt[bth] = AA * alpha * dalpha + (1.0 - LM) * alpha * (1.0 + DT * AA) * dbeta + LM * dgamma +
                   (angle ? 0.0 : dphi_dt);
      if (dlam) dlam[bth] = -DT * alpha * dbeta + DT * dgamma;
      dA_tok[bth] = DT * alpha * dalpha + (1.0 - LM) * DT * DT * alpha * dbeta;
    }
    if (dh0) memcpy(dh0 + u * PN, G, sizeof(double) * PN);
    for (int64_t t = 0; t < T; ++t) {
      const int64_t bth = (b * T + t) * H + h;
      if (dx) memcpy(dx + bth * P * R, gx + (t + 1) * P * R, sizeof(double) * P * R);
      if (dB) memcpy(dB + bth * N * R, gb + (t + 1) * N * R, sizeof(double) * N * R);
    }
    if (prev && dx_prev) memcpy(dx_prev + u * P * R, gx, sizeof(double) * P * R);
    if (prev && dB_prev) memcpy(dB_prev + u * N * R, gb, sizeof(double) * N * R);
    free(St); free(G); free(V); free(yt); free(gx); free(gb);
  }
  if (dA) {
    if (a_tok) {
      memcpy(dA, dA_tok, sizeof(double) * Bsz * T * H);
    } else {
      for (int64_t h = 0; h < H; ++h) dA[h] = 0.0;
      for (int64_t i = 0; i < Bsz * T * H; ++i) dA[i % H] += dA_tok[i];
    }
  }
  free(dA_tok);
  return 0;
}

/*
 * Preparation of B and C for the recurrence [the same article, section 2:
 * B and C go through an RMS normalisation, the way attention normalises Q
 * and K, and then get a learned bias per head and per channel].  For each
 * row (one token of one batch), each head h of group g = h / (H / G) and
 * each rank column r:
 *   rms = sqrt( (1/N) sum_n in[g][n][r]^2 + eps )          (when rms_on)
 *   out[h][n][r] = w[n] * in[g][n][r] / rms + bias[h][n][r]
 * With rms_on == 0 the division is skipped; w NULL means 1, bias NULL
 * means 0.  Readings: the normalisation runs over the N state channels of
 * one rank column; the weight has one value per channel, shared by heads
 * and ranks; the bias is per head (so heads of one group differ after it)
 * and is added after the normalisation and the weight.
 * Layouts: in [rows, G, N, R], w [N], bias [H, N, R], out [rows, H, N, R].
 */
int m3ref_bc_prep(int64_t rows, int64_t G, int64_t H, int64_t N, int64_t R,
                  const double* in, const double* w, const double* bias,
                  double eps, int rms_on, double* out) {
  if (rows < 0 || G <= 0 || H <= 0 || H % G != 0 || N <= 0 || R <= 0 || !in || !out)
    return 1;
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t h = 0; h < H; ++h) {
      const int64_t g = h / (H / G);
      const double* v = in + (i * G + g) * N * R;
      double* o = out + (i * H + h) * N * R;
      for (int64_t r = 0; r < R; ++r) {
        double scale = 1.0;
        if (rms_on) {
          double ms = 0.0;
          for (int64_t n = 0; n < N; ++n) ms += v[n * R + r] * v[n * R + r];
          scale = 1.0 / sqrt(ms / (double)N + eps);
        }
        for (int64_t n = 0; n < N; ++n) {
          const double wn = w ? w[n] : 1.0;
          const double bn = bias ? bias[(h * N + n) * R + r] : 0.0;
          o[n * R + r] = wn * v[n * R + r] * scale + bn;
        }
      }
    }
  return 0;
}

/*
 * Angle projection [the same article, section 1.2: the rotation angles of
 * the complex state are data-dependent, produced from the layer's input like
 * B and C].  For each row (one token of one batch), group g and pair k:
 *   out[g][k] = sum_j W[g][k][j] * u[j]
 * Layouts: u [rows, D], W [G, K, D], out [rows, G, K] (K = N/2 pairs).
 * Reading: one linear map per head group, of the same input row that feeds
 * the group's B and C; no bias and no activation.
 */
int m3ref_theta_proj(int64_t rows, int64_t G, int64_t K, int64_t D, const double* u,
                     const double* W, double* out) {
  if (rows < 0 || G <= 0 || K <= 0 || D <= 0 || !u || !W || !out) return 1;
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t g = 0; g < G; ++g)
      for (int64_t k = 0; k < K; ++k) {
        double acc = 0.0;
        for (int64_t j = 0; j < D; ++j) acc += W[(g * K + k) * D + j] * u[i * D + j];
        out[(i * G + g) * K + k] = acc;
      }
  return 0;
}

int m3ref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
