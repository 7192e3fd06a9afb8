/*
 * Plain fp64 CPU oracle for the Mamba-2 mixer hot path:
 *   causal depthwise conv1d (+SiLU)  ->  selective SSD recurrence  ->  SiLU(z) gate,
 * and the backward pass of each stage.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the GPU library; the two never include or link each other.
 *
 * Sources (the pages this follows):
 *  - Video-Ma2mba review (pith.science verdict for arXiv 2411.19460), skeptic
 *    critique and referee report, Eq. (1): the mixer state obeys the first-order
 *    recurrence h_t = A_t h_{t-1} + B_t x_t.  The selective (Mamba / Mamba-2,
 *    both in the reference list of the arXiv index page) form of that equation is
 *    used: A_t = exp(dt_t * A_h) (one scalar per head), input term dt_t * B_t x_t^T,
 *    readout y_t = C_t^T h_t + D_h x_t, output gated by SiLU(z).
 *  - Same review, skeptic critique ("load-bearing attack", "concrete test"): a
 *    causal Conv1d of width k precedes the SSD, so the state needed to resume a
 *    sequence at step s is (h_s, the last k-1 conv inputs).  Both are carried in
 *    and out here.
 *
 * Everything is the literal sequential definition: one time step at a time, per
 * independent lane (batch b, head h, head channel p).  The only parallelism is
 * across lanes (or across heads / channels in the backward pass); the time loop is
 * strictly sequential.  Build with -ffp-contract=off so that recomputation is
 * bitwise identical to the first computation.
 *
 * Layouts (all contiguous, row-major, float64):
 *   x, z, y, out        [B][L][H][P]
 *   dt_raw, ddt         [B][L][H]
 *   Bm, Cm              [B][L][G][N]     head h reads group h / (H/G)
 *   h0, h_final         [B][H][P][N]     (state transposed: p outer, n inner)
 *   conv input / output [B][L][Cd]
 *   conv state          [B][K-1][Cd]     the last K-1 conv *inputs*, oldest first
 *   conv weight         [Cd][K]          w[c][K-1] multiplies the current token
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double sigm(double u) { return 1.0 / (1.0 + exp(-u)); }

/* softplus(u) = log(1 + e^u), evaluated without overflow. */
static double softplus(double u) { return (u > 0.0 ? u : 0.0) + log1p(exp(-fabs(u))); }

static double silu(double u) { return u * sigm(u); }

/* d/du [u * sigmoid(u)] = s * (1 + u * (1 - s)), s = sigmoid(u). */
static double dsilu(double u) {
  double s = sigm(u);
  return s * (1.0 + u * (1.0 - s));
}

int oracle_abi_version(void) { return 1; }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* Causal depthwise conv1d.                                                   */
/* ------------------------------------------------------------------------- */

/* Conv input at time tau in [-(K-1), L): the carried state for tau < 0. */
static double conv_in(const double* xraw, const double* state_in, int64_t L, int64_t Cd, int K,
                      int64_t b, int64_t tau, int64_t c) {
  if (tau >= 0) return xraw[(b * L + tau) * Cd + c];
  if (!state_in) return 0.0;
  return state_in[(b * (K - 1) + (tau + K - 1)) * Cd + c];
}

/* pre[t,c] = bias[c] + sum_k w[c][k] * xin[t-(K-1)+k, c];  out = silu(pre) or pre. */
void oracle_conv1d_fwd(int64_t B, int64_t L, int64_t Cd, int K, const double* xraw,
                       const double* state_in, const double* w, const double* bias, int use_silu,
                       double* out, double* state_out) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t c = 0; c < Cd; ++c) {
      for (int64_t t = 0; t < L; ++t) {
        double pre = bias ? bias[c] : 0.0;
        for (int k = 0; k < K; ++k)
          pre += w[c * K + k] * conv_in(xraw, state_in, L, Cd, K, b, t - (K - 1) + k, c);
        out[(b * L + t) * Cd + c] = use_silu ? silu(pre) : pre;
      }
      if (state_out)
        for (int j = 0; j < K - 1; ++j)
          state_out[(b * (K - 1) + j) * Cd + c] =
              conv_in(xraw, state_in, L, Cd, K, b, L - (K - 1) + j, c);
    }
}

/* Backward of oracle_conv1d_fwd.  dstate_out is the gradient arriving at the
 * returned conv state (from a later segment); dstate_in is the gradient of the
 * carried-in state.  dw, db are overwritten (not accumulated). */
void oracle_conv1d_bwd(int64_t B, int64_t L, int64_t Cd, int K, const double* xraw,
                       const double* state_in, const double* w, const double* bias, int use_silu,
                       const double* dout, const double* dstate_out, double* dx, double* dw,
                       double* db, double* dstate_in) {
  const int64_t T = L + K - 1; /* tau = -(K-1) .. L-1 */
  if (K < 1 || K > 16) return;
#pragma omp parallel for schedule(static)
  for (int64_t c = 0; c < Cd; ++c) {
    double* dpre = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double* dxin = (double*)malloc(sizeof(double) * (size_t)T);
    double dwc[16];
    for (int k = 0; k < K; ++k) dwc[k] = 0.0;
    double dbc = 0.0;
    for (int64_t b = 0; b < B; ++b) {
      for (int64_t t = 0; t < L; ++t) {
        double g = dout[(b * L + t) * Cd + c];
        if (use_silu) {
          double pre = bias ? bias[c] : 0.0;
          for (int k = 0; k < K; ++k)
            pre += w[c * K + k] * conv_in(xraw, state_in, L, Cd, K, b, t - (K - 1) + k, c);
          g *= dsilu(pre);
        }
        dpre[t] = g;
      }
      for (int64_t t = 0; t < L; ++t) {
        dbc += dpre[t];
        for (int k = 0; k < K; ++k)
          dwc[k] += dpre[t] * conv_in(xraw, state_in, L, Cd, K, b, t - (K - 1) + k, c);
      }
      /* dxin[tau] = sum_k dpre[tau + (K-1) - k] * w[c][k] over valid output times */
      for (int64_t i = 0; i < T; ++i) {
        int64_t tau = i - (K - 1);
        double acc = 0.0;
        for (int k = 0; k < K; ++k) {
          int64_t t = tau + (K - 1) - k;
          if (t >= 0 && t < L) acc += dpre[t] * w[c * K + k];
        }
        dxin[i] = acc;
      }
      if (dstate_out)
        for (int j = 0; j < K - 1; ++j) {
          int64_t tau = L - (K - 1) + j;
          dxin[tau + (K - 1)] += dstate_out[(b * (K - 1) + j) * Cd + c];
        }
      for (int64_t t = 0; t < L; ++t) dx[(b * L + t) * Cd + c] = dxin[t + (K - 1)];
      if (dstate_in)
        for (int j = 0; j < K - 1; ++j) dstate_in[(b * (K - 1) + j) * Cd + c] = dxin[j];
    }
    for (int k = 0; k < K; ++k) dw[c * K + k] = dwc[k];
    if (db) db[c] = dbc;
    free(dpre);
    free(dxin);
  }
}

/* ------------------------------------------------------------------------- */
/* Selective SSD recurrence.                                                  */
/* ------------------------------------------------------------------------- */

typedef struct {
  int64_t B, L, H, P, N, G;
  const double *x, *dt_raw, *dt_bias, *A, *Bm, *Cm, *D, *z, *h0;
  int use_softplus;
} ssd_in;

static double dt_of(const ssd_in* s, int64_t b, int64_t t, int64_t h) {
  double u = s->dt_raw[(b * s->L + t) * s->H + h] + (s->dt_bias ? s->dt_bias[h] : 0.0);
  return s->use_softplus ? softplus(u) : u;
}

/* One step of Eq. (1) for one lane: s <- exp(dt*A) * s + (dt * x) * B_t.
 * The same function is used for the first pass and for every recomputation. */
static void ssd_step(int64_t N, double* st, double a, double dtx, const double* Bt) {
  for (int64_t n = 0; n < N; ++n) st[n] = a * st[n] + dtx * Bt[n];
}

static double ssd_read(int64_t N, const double* st, const double* Ct) {
  double acc = 0.0;
  for (int64_t n = 0; n < N; ++n) acc += st[n] * Ct[n];
  return acc;
}

/* Forward.  out = y * silu(z) (or y when z is NULL); y_pre (optional) receives
 * the ungated y; h_final (optional) the state after the last step. */
void oracle_ssd_fwd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                    const double* x, const double* dt_raw, const double* dt_bias,
                    int use_softplus, const double* A, const double* Bm, const double* Cm,
                    const double* D, const double* z, const double* h0, double* out,
                    double* y_pre, double* h_final) {
  ssd_in s = {B, L, H, P, N, G, x, dt_raw, dt_bias, A, Bm, Cm, D, z, h0, use_softplus};
  const int64_t hpg = H / G;
#pragma omp parallel for collapse(3) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t p = 0; p < P; ++p) {
        const int64_t g = h / hpg;
        double* st = (double*)malloc(sizeof(double) * (size_t)N);
        for (int64_t n = 0; n < N; ++n) st[n] = h0 ? h0[((b * H + h) * P + p) * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
          const double dt = dt_of(&s, b, t, h);
          const double a = exp(dt * A[h]);
          const int64_t xi = ((b * L + t) * H + h) * P + p;
          const double* Bt = Bm + ((b * L + t) * G + g) * N;
          const double* Ct = Cm + ((b * L + t) * G + g) * N;
          ssd_step(N, st, a, dt * x[xi], Bt);
          double y = ssd_read(N, st, Ct) + (D ? D[h] * x[xi] : 0.0);
          if (y_pre) y_pre[xi] = y;
          out[xi] = z ? y * silu(z[xi]) : y;
        }
        if (h_final)
          for (int64_t n = 0; n < N; ++n) h_final[((b * H + h) * P + p) * N + n] = st[n];
        free(st);
      }
}

/* Backward with full-storage semantics.
 *
 * Per lane the reverse sweep needs the state before and after every step.  The
 * states are kept only at the start of each time block of `block` steps and each
 * block is recomputed with ssd_step before its reverse sweep; with
 * -ffp-contract=off this reproduces the stored states bit for bit, so every
 * output equals literal full storage (block >= L) exactly.
 *
 * Reverse sweep for one lane, g = dLoss/d(state after step t):
 *   g   += dy_t * C_t
 *   dC_t += dy_t * s_t;   q = <g, B_t>;   dx_t = dt_t q + D dy_t;   dB_t += dt_t x_t g
 *   dl   = a_t <g, s_{t-1}>             (gradient of log-decay l_t = dt_t A)
 *   ddt_t += x_t q + A dl;   dA += dt_t dl;   dD += dy_t x_t;   g <- a_t g
 * with dy = dout * silu(z) and dz = dout * y * silu'(z).  After t = 0, dh0 = g.
 * ddt is returned with respect to dt_raw (softplus and bias chain applied).
 * dA, dD, ddt_bias are overwritten (not accumulated). */
void oracle_ssd_bwd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                    const double* x, const double* dt_raw, const double* dt_bias,
                    int use_softplus, const double* A, const double* Bm, const double* Cm,
                    const double* D, const double* z, const double* h0, const double* dout,
                    const double* dh_final, double* dx, double* ddt, double* dBm, double* dCm,
                    double* dz, double* dA, double* dD, double* ddt_bias, double* dh0,
                    int64_t block) {
  ssd_in s = {B, L, H, P, N, G, x, dt_raw, dt_bias, A, Bm, Cm, D, z, h0, use_softplus};
  const int64_t hpg = H / G;
  if (block <= 0 || block > L) block = L > 0 ? L : 1;
  const int64_t nblk = L > 0 ? (L + block - 1) / block : 0;
  const int64_t lanes_b = H * P;

  /* per-lane carried quantities */
  double* ck = (double*)malloc(sizeof(double) * (size_t)(lanes_b * (nblk > 0 ? nblk : 1) * N));
  double* gst = (double*)malloc(sizeof(double) * (size_t)(lanes_b * N));
  double* dA_lane = (double*)malloc(sizeof(double) * (size_t)lanes_b);
  double* dD_lane = (double*)malloc(sizeof(double) * (size_t)lanes_b);
  /* per-head block buffers for the group reductions */
  double* dBh = (double*)malloc(sizeof(double) * (size_t)(H * block * N));
  double* dCh = (double*)malloc(sizeof(double) * (size_t)(H * block * N));
  double* ddth = (double*)malloc(sizeof(double) * (size_t)(H * block));
  double* dAh = (double*)calloc((size_t)H, sizeof(double));
  double* dDh = (double*)calloc((size_t)H, sizeof(double));

  for (int64_t b = 0; b < B; ++b) {
    /* 1. forward pass storing the state at the start of each block */
#pragma omp parallel for schedule(static)
    for (int64_t lane = 0; lane < lanes_b; ++lane) {
      const int64_t h = lane / P, p = lane % P, g = h / hpg;
      double* st = (double*)malloc(sizeof(double) * (size_t)N);
      for (int64_t n = 0; n < N; ++n) st[n] = h0 ? h0[((b * H + h) * P + p) * N + n] : 0.0;
      for (int64_t t = 0; t < L; ++t) {
        if (t % block == 0) memcpy(ck + (lane * nblk + t / block) * N, st, sizeof(double) * N);
        const double dt = dt_of(&s, b, t, h);
        const double a = exp(dt * A[h]);
        ssd_step(N, st, a, dt * x[((b * L + t) * H + h) * P + p], Bm + ((b * L + t) * G + g) * N);
      }
      for (int64_t n = 0; n < N; ++n)
        gst[lane * N + n] = dh_final ? dh_final[((b * H + h) * P + p) * N + n] : 0.0;
      dA_lane[lane] = 0.0;
      dD_lane[lane] = 0.0;
      free(st);
    }

    /* 2. reverse sweep, one block at a time, parallel over heads */
    for (int64_t blk = nblk - 1; blk >= 0; --blk) {
      const int64_t t0 = blk * block;
      const int64_t t1 = (t0 + block < L) ? t0 + block : L;
      const int64_t len = t1 - t0;
#pragma omp parallel for schedule(static)
      for (int64_t h = 0; h < H; ++h) {
        const int64_t g = h / hpg;
        double* sb = (double*)malloc(sizeof(double) * (size_t)((len + 1) * N));
        double* dBl = dBh + h * block * N;
        double* dCl = dCh + h * block * N;
        double* ddl = ddth + h * block;
        memset(dBl, 0, sizeof(double) * (size_t)(len * N));
        memset(dCl, 0, sizeof(double) * (size_t)(len * N));
        memset(ddl, 0, sizeof(double) * (size_t)len);
        for (int64_t p = 0; p < P; ++p) {
          const int64_t lane = h * P + p;
          /* recompute s_{t0-1} .. s_{t1-1} into sb[0 .. len] */
          memcpy(sb, ck + (lane * nblk + blk) * N, sizeof(double) * N);
          for (int64_t t = t0; t < t1; ++t) {
            double* cur = sb + (t - t0 + 1) * N;
            memcpy(cur, cur - N, sizeof(double) * N);
            const double dt = dt_of(&s, b, t, h);
            const double a = exp(dt * A[h]);
            ssd_step(N, cur, a, dt * x[((b * L + t) * H + h) * P + p],
                     Bm + ((b * L + t) * G + g) * N);
          }
          double* gl = gst + lane * N;
          for (int64_t t = t1 - 1; t >= t0; --t) {
            const int64_t xi = ((b * L + t) * H + h) * P + p;
            const double dt = dt_of(&s, b, t, h);
            const double a = exp(dt * A[h]);
            const double* Bt = Bm + ((b * L + t) * G + g) * N;
            const double* Ct = Cm + ((b * L + t) * G + g) * N;
            const double* s_t = sb + (t - t0 + 1) * N;
            const double* s_prev = sb + (t - t0) * N;
            const double xv = x[xi];
            double dy = dout[xi];
            if (z) {
              const double y = ssd_read(N, s_t, Ct) + (D ? D[h] * xv : 0.0);
              if (dz) dz[xi] = dout[xi] * y * dsilu(z[xi]);
              dy = dout[xi] * silu(z[xi]);
            } else if (dz) {
              dz[xi] = 0.0;
            }
            for (int64_t n = 0; n < N; ++n) gl[n] += dy * Ct[n];
            double* dCt = dCl + (t - t0) * N;
            double* dBt = dBl + (t - t0) * N;
            for (int64_t n = 0; n < N; ++n) dCt[n] += dy * s_t[n];
            const double q = ssd_read(N, gl, Bt);
            dx[xi] = dt * q + (D ? D[h] * dy : 0.0);
            for (int64_t n = 0; n < N; ++n) dBt[n] += dt * xv * gl[n];
            const double dl = a * ssd_read(N, gl, s_prev);
            ddl[t - t0] += xv * q + A[h] * dl;
            dA_lane[lane] += dt * dl;
            dD_lane[lane] += dy * xv;
            for (int64_t n = 0; n < N; ++n) gl[n] *= a;
          }
        }
        /* chain ddt to dt_raw */
        for (int64_t t = t0; t < t1; ++t) {
          double v = ddl[t - t0];
          if (use_softplus) {
            double u = dt_raw[(b * L + t) * H + h] + (dt_bias ? dt_bias[h] : 0.0);
            v *= sigm(u);
          }
          ddt[(b * L + t) * H + h] = v;
        }
        free(sb);
      }
      /* group reductions, heads summed in increasing order */
      for (int64_t t = t0; t < t1; ++t)
        for (int64_t g = 0; g < G; ++g)
          for (int64_t n = 0; n < N; ++n) {
            double accB = 0.0, accC = 0.0;
            for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
              accB += dBh[(h * block + (t - t0)) * N + n];
              accC += dCh[(h * block + (t - t0)) * N + n];
            }
            dBm[((b * L + t) * G + g) * N + n] = accB;
            dCm[((b * L + t) * G + g) * N + n] = accC;
          }
    }

    /* 3. per-batch outputs and ordered parameter reductions */
    for (int64_t h = 0; h < H; ++h)
      for (int64_t p = 0; p < P; ++p) {
        const int64_t lane = h * P + p;
        dAh[h] += dA_lane[lane];
        dDh[h] += dD_lane[lane];
        if (dh0)
          for (int64_t n = 0; n < N; ++n) dh0[((b * H + h) * P + p) * N + n] = gst[lane * N + n];
      }
  }
  for (int64_t h = 0; h < H; ++h) {
    dA[h] = dAh[h];
    if (dD) dD[h] = dDh[h];
    if (ddt_bias) {
      double acc = 0.0;
      for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < L; ++t) acc += ddt[(b * L + t) * H + h];
      ddt_bias[h] = acc;
    }
  }
  free(ck);
  free(gst);
  free(dA_lane);
  free(dD_lane);
  free(dBh);
  free(dCh);
  free(ddth);
  free(dAh);
  free(dDh);
}
