/*
 * Sequential fp64 CPU oracle for the selective state-space scan (Mamba S6)
 * and its Mamba-2 SSD form.  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the benchmark's CPU-baseline leg call it; the GPU library never
 * links, includes or calls anything here, and this file includes nothing of
 * the GPU library.
 *
 * Everything is double precision.  Callers convert their stored inputs
 * (bf16 or fp32) to double exactly before calling.  Each function walks the
 * recurrence one time step at a time, in the order the sources write it; no
 * blocking, no reordering, no fusion beyond what the formulas state.
 *
 * Sources (cited by page title and section):
 *  [P1] "Mamba / State Space Models complete guide" (youngju.dev):
 *       section 2 (continuous SSM; discretization, ZOH; convolution kernel),
 *       section 5 (MambaBlock.ssm / selective_scan listing).
 *  [P2] "Paper explainer: Mamba (2312.00752)" (0h-n0.github.io):
 *       "Technical details" (ZOH, selection mechanism with softplus,
 *       hardware-aware parallel scan listing).
 *  [P3] "SSM & Mamba" (disassemble-channel.com): "Discretization / ZOH",
 *       "Equivalence with convolution", "Python implementation"
 *       (discretize_zoh, recurrent and convolution modes).
 *  [P5] "Mamba-2 / Structured State Space Duality" (abeam guide):
 *       "Basic idea", "Linear and quadratic forms".
 *
 * Readings taken where the sources are silent (each also listed in the
 * design notes):
 *  - B-bar is the exact diagonal ZOH form g = expm1(dt*a)/a (P3, ZOH with
 *    diagonal A); g = dt when a == 0 (the limit of that expression).
 *  - The state before token 0 is h0 (zero when absent) and y_t reads the
 *    state *after* token t's update, so y_0 = C_0 . Bbar_0 x_0 (P1 sec. 2,
 *    the expansion of y[0], y[1], y[2]).
 *  - The skip term is added before the gate: y = (C.h + Dskip*x) * silu(z)
 *    (P1 sec. 5: selective_scan adds u*D, the block then multiplies by
 *    silu(z)).
 *  - softplus(v) = log(1 + e^v) (P2, selection mechanism), evaluated in the
 *    overflow-free form max(v,0) + log1p(exp(-|v|)); an optional per-channel
 *    bias is added to v first (the dt projection carries a bias, P1 sec. 5).
 *  - silu(z) = z / (1 + exp(-z)).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include <stdlib.h>

static double softplus(double v) {
  /* log(1 + e^v), written so that neither branch overflows */
  return (v > 0 ? v : 0.0) + log1p(exp(-fabs(v)));
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* ZOH input gain for one diagonal entry: Bbar_n / B_n = (e^{dt a} - 1)/a. */
static double zoh_gain(double dt, double a) {
  if (a == 0.0) return dt;
  return expm1(dt * a) / a;
}

/*
 * O1. Selective scan (S6) with exact ZOH, diagonal A.
 *
 *   x, delta, z, y : (batch, seqlen, dim)   row-major
 *   A              : (dim, dstate)
 *   B, C           : (batch, seqlen, dstate), shared by every channel
 *   Dskip, bias    : (dim)
 *   h0, h_final    : (batch, dim, dstate)
 * Optional pointers may be NULL (Dskip, z, bias, h0, y, h_final).
 * Only the (batch, channel) slices s in [s_begin, s_end) are computed,
 * s = b*dim + d, so a caller may split the work over threads.
 *
 *   h_t = exp(dt_t a) * h_{t-1} + expm1(dt_t a)/a * B_t * x_t     (P3 ZOH;
 *         P1 sec. 2 "x[t] = A_bar x[t-1] + B_bar u[t]")
 *   y_t = sum_n C_t,n h_t,n + Dskip x_t, then * silu(z_t)         (P1 sec. 5)
 */
static void selective_scan_impl(const double* x, const double* delta, const double* A,
                                const double* B, const double* C, const double* Dskip,
                                const double* z, const double* delta_bias, int delta_softplus,
                                const double* h0, double* y, double* h_final,
                                int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                int64_t s_begin, int64_t s_end, int euler) {
  double* h = (double*)malloc(sizeof(double) * (size_t)(dstate > 0 ? dstate : 1));
  for (int64_t s = s_begin; s < s_end; ++s) {
    int64_t b = s / dim, d = s % dim;
    for (int64_t n = 0; n < dstate; ++n)
      h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      int64_t i = (b * seqlen + t) * dim + d;        /* (b, t, d) */
      int64_t r = (b * seqlen + t) * dstate;         /* (b, t, :) */
      double v = delta[i] + (delta_bias ? delta_bias[d] : 0.0);
      double dt = delta_softplus ? softplus(v) : v;
      double acc = 0.0;
      for (int64_t n = 0; n < dstate; ++n) {
        double a = A[d * dstate + n];
        double abar = exp(dt * a);
        double g = euler ? dt : zoh_gain(dt, a);
        h[n] = abar * h[n] + g * B[r + n] * x[i];
        acc += C[r + n] * h[n];
      }
      double out = acc + (Dskip ? Dskip[d] * x[i] : 0.0);
      if (z) out *= silu(z[i]);
      if (y) y[i] = out;
    }
    if (h_final)
      for (int64_t n = 0; n < dstate; ++n) h_final[(b * dim + d) * dstate + n] = h[n];
  }
  free(h);
}

void oracle_selective_scan(const double* x, const double* delta, const double* A,
                           const double* B, const double* C, const double* Dskip,
                           const double* z, const double* delta_bias, int delta_softplus,
                           const double* h0, double* y, double* h_final,
                           int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                           int64_t s_begin, int64_t s_end) {
  selective_scan_impl(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, y, h_final, batch, seqlen, dim,
                      dstate, s_begin, s_end, 0);
}

/*
 * O1e. The same scan with the Euler input discretization of the pages'
 * listings, Bbar = dt * B (P1 sec. 5 selective_scan: deltaB_u = delta * B * u;
 * P2 listing), keeping Abar = exp(dt a).
 */
void oracle_selective_scan_euler(const double* x, const double* delta, const double* A,
                                 const double* B, const double* C, const double* Dskip,
                                 const double* z, const double* delta_bias, int delta_softplus,
                                 const double* h0, double* y, double* h_final,
                                 int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                 int64_t s_begin, int64_t s_end) {
  selective_scan_impl(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, y, h_final, batch, seqlen, dim,
                      dstate, s_begin, s_end, 1);
}

/*
 * O2. Mamba-2 SSD, recurrent (linear) form.  One scalar decay per head
 * (P1 sec. 6: A_log has one entry per head), dt per (token, head), B and C
 * per (token, group) with heads split evenly over groups, head dim P.
 *
 *   x, z, y   : (batch, seqlen, nheads, headdim)
 *   dt        : (batch, seqlen, nheads)
 *   A, Dskip, dt_bias : (nheads)
 *   B, C      : (batch, seqlen, ngroups, dstate)
 *   h0, h_final : (batch, nheads, headdim, dstate)
 * Slices s in [s_begin, s_end), s = b*nheads + h.
 *
 *   S_t[p][n] = exp(dt a) S_{t-1}[p][n] + expm1(dt a)/a * B_t[n] * x_t[p]
 *   y_t[p]    = sum_n C_t[n] S_t[p][n] (+ Dskip x_t[p]) (* silu z_t[p])
 * (P5 "Basic idea": h_t = A_t h_{t-1} + B_t x_t, y_t = C_t h_t, with the
 * same ZOH discretization as the selective scan.)
 */
void oracle_ssd_recurrent(const double* x, const double* dt, const double* A,
                          const double* B, const double* C, const double* Dskip,
                          const double* z, const double* dt_bias, int dt_softplus,
                          const double* h0, double* y, double* h_final,
                          int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                          int64_t ngroups, int64_t dstate, int64_t s_begin, int64_t s_end) {
  int64_t hpg = nheads / ngroups;
  double* S = (double*)malloc(sizeof(double) * (size_t)(headdim * dstate > 0 ? headdim * dstate : 1));
  for (int64_t s = s_begin; s < s_end; ++s) {
    int64_t b = s / nheads, hd = s % nheads, grp = hd / hpg;
    double a = A[hd];
    for (int64_t k = 0; k < headdim * dstate; ++k)
      S[k] = h0 ? h0[(b * nheads + hd) * headdim * dstate + k] : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      double v = dt[(b * seqlen + t) * nheads + hd] + (dt_bias ? dt_bias[hd] : 0.0);
      double del = dt_softplus ? softplus(v) : v;
      double abar = exp(del * a);
      double g = zoh_gain(del, a);
      const double* Bt = B + ((b * seqlen + t) * ngroups + grp) * dstate;
      const double* Ct = C + ((b * seqlen + t) * ngroups + grp) * dstate;
      for (int64_t p = 0; p < headdim; ++p) {
        int64_t i = ((b * seqlen + t) * nheads + hd) * headdim + p;
        double acc = 0.0;
        for (int64_t n = 0; n < dstate; ++n) {
          S[p * dstate + n] = abar * S[p * dstate + n] + g * Bt[n] * x[i];
          acc += Ct[n] * S[p * dstate + n];
        }
        double out = acc + (Dskip ? Dskip[hd] * x[i] : 0.0);
        if (z) out *= silu(z[i]);
        if (y) y[i] = out;
      }
    }
    if (h_final)
      for (int64_t k = 0; k < headdim * dstate; ++k)
        h_final[(b * nheads + hd) * headdim * dstate + k] = S[k];
  }
  free(S);
}

/*
 * O2'. Mamba-2 SSD, quadratic ("attention-like") form (P5 "Linear and
 * quadratic forms"): the same map written as a causal, decayed matrix
 * product over the whole sequence, O(L^2):
 *
 *   y_t = sum_{s<=t} (C_t . B_s) * exp(a * sum_{r=s+1..t} dt_r) * g_s * x_s
 *       + sum_n C_t[n] * exp(a * sum_{r=0..t} dt_r) * h0[p][n]
 *       (+ Dskip x_t) (* silu z_t)
 * with g_s = expm1(dt_s a)/a.  The decay is evaluated directly from the
 * partial sums of dt (never as a ratio of cumulative exponentials).
 * Same layouts and slicing as oracle_ssd_recurrent; y required.
 */
void oracle_ssd_quadratic(const double* x, const double* dt, const double* A,
                          const double* B, const double* C, const double* Dskip,
                          const double* z, const double* dt_bias, int dt_softplus,
                          const double* h0, double* y,
                          int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim,
                          int64_t ngroups, int64_t dstate, int64_t s_begin, int64_t s_end) {
  int64_t hpg = nheads / ngroups;
  double* del = (double*)malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
  for (int64_t s = s_begin; s < s_end; ++s) {
    int64_t b = s / nheads, hd = s % nheads, grp = hd / hpg;
    double a = A[hd];
    for (int64_t t = 0; t < seqlen; ++t) {
      double v = dt[(b * seqlen + t) * nheads + hd] + (dt_bias ? dt_bias[hd] : 0.0);
      del[t] = dt_softplus ? softplus(v) : v;
    }
    for (int64_t t = 0; t < seqlen; ++t) {
      const double* Ct = C + ((b * seqlen + t) * ngroups + grp) * dstate;
      for (int64_t p = 0; p < headdim; ++p) {
        int64_t i = ((b * seqlen + t) * nheads + hd) * headdim + p;
        double acc = 0.0;
        double span = 0.0;                       /* sum_{r=s+1..t} dt_r */
        for (int64_t s2 = t; s2 >= 0; --s2) {
          const double* Bs = B + ((b * seqlen + s2) * ngroups + grp) * dstate;
          double cb = 0.0;
          for (int64_t n = 0; n < dstate; ++n) cb += Ct[n] * Bs[n];
          int64_t j = ((b * seqlen + s2) * nheads + hd) * headdim + p;
          acc += cb * exp(a * span) * zoh_gain(del[s2], a) * x[j];
          span += del[s2];
        }
        if (h0) {                                /* span = sum_{r=0..t} dt_r */
          const double* H = h0 + ((b * nheads + hd) * headdim + p) * dstate;
          for (int64_t n = 0; n < dstate; ++n) acc += Ct[n] * exp(a * span) * H[n];
        }
        double out = acc + (Dskip ? Dskip[hd] * x[i] : 0.0);
        if (z) out *= silu(z[i]);
        y[i] = out;
      }
    }
  }
  free(del);
}

/*
 * O3. Linear time-invariant SSM as a causal convolution (P1 sec. 2 "SSM as
 * a convolution kernel"; P3 "Equivalence with convolution" and its
 * convolution-mode code): one channel, dt, B, C held constant,
 *
 *   K_i = sum_n C_n * Abar_n^i * Bbar_n,   Abar_n = exp(dt a_n),
 *   Bbar_n = expm1(dt a_n)/a_n * B_n,
 *   y_t = sum_{j=0..t} K_{t-j} x_j + Dskip x_t.
 * The powers Abar^i are built by repeated multiplication, as the kernel is
 * defined.  A, B, C: (dstate); x, y: (seqlen).
 */
void oracle_lti_conv(const double* x, const double* A, const double* B, const double* C,
                     double dt, double Dskip, double* y, int64_t seqlen, int64_t dstate) {
  double* K = (double*)malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
  double* pw = (double*)malloc(sizeof(double) * (size_t)(dstate > 0 ? dstate : 1));
  for (int64_t n = 0; n < dstate; ++n) pw[n] = 1.0;
  for (int64_t i = 0; i < seqlen; ++i) {
    double k = 0.0;
    for (int64_t n = 0; n < dstate; ++n) {
      k += C[n] * pw[n] * zoh_gain(dt, A[n]) * B[n];
      pw[n] *= exp(dt * A[n]);
    }
    K[i] = k;
  }
  for (int64_t t = 0; t < seqlen; ++t) {
    double acc = 0.0;
    for (int64_t j = 0; j <= t; ++j) acc += K[t - j] * x[j];
    y[t] = acc + Dskip * x[t];
  }
  free(pw);
  free(K);
}

/*
 * O4. Causal depthwise 1-D convolution of the Mamba block's x branch, then
 * SiLU (P1 sec. 5, the Mamba block: Conv1d with one group per channel,
 * padding width-1 and the output trimmed to the first seqlen positions,
 * then silu).  Per batch b and channel d, with weights w[d][0..W-1]:
 *
 *   out[t] = silu( bias_d + sum_{k=0..W-1} w[d][k] * xx[t - (W-1) + k] )
 *
 * where xx[i] = x[b, i, d] for i >= 0, and for -(W-1) <= i < 0 the inputs
 * carried in from a previous segment, state_in[b, d, (W-1) + i] (oldest
 * first; zeros when state_in is NULL, which is the padding of the block).
 * state_out[b, d, j] = xx[seqlen - (W-1) + j], the last W-1 inputs of the
 * extended sequence, so that a later segment (or a single decode token)
 * continues the same convolution.  silu_on = 0 leaves out the SiLU.
 *
 *   x, out : (batch, seqlen, dim); w : (dim, width); bias : (dim) or NULL
 *   state_in, state_out : (batch, dim, width-1) or NULL
 * Slices s = b*dim + d in [s_begin, s_end).
 */
static double conv_ext(const double* x, const double* state_in, int64_t b, int64_t d, int64_t i,
                       int64_t seqlen, int64_t dim, int64_t width) {
  if (i >= 0) return x[(b * seqlen + i) * dim + d];
  if (!state_in) return 0.0;
  return state_in[(b * dim + d) * (width - 1) + (width - 1) + i];
}

void oracle_causal_conv1d(const double* x, const double* w, const double* bias, const double* state_in,
                          int silu_on, double* out, double* state_out, int64_t batch, int64_t seqlen,
                          int64_t dim, int64_t width, int64_t s_begin, int64_t s_end) {
  (void)batch;
  for (int64_t s = s_begin; s < s_end; ++s) {
    const int64_t b = s / dim, d = s % dim;
    double* keep = NULL;
    if (state_out && width > 1) {
      /* read the carried-in values first: state_out may be the same buffer */
      keep = (double*)malloc(sizeof(double) * (size_t)(width - 1));
      for (int64_t j = 0; j < width - 1; ++j)
        keep[j] = conv_ext(x, state_in, b, d, seqlen - (width - 1) + j, seqlen, dim, width);
    }
    if (out) {
      for (int64_t t = 0; t < seqlen; ++t) {
        double acc = bias ? bias[d] : 0.0;
        for (int64_t k = 0; k < width; ++k)
          acc += w[d * width + k] * conv_ext(x, state_in, b, d, t - (width - 1) + k, seqlen, dim, width);
        out[(b * seqlen + t) * dim + d] = silu_on ? silu(acc) : acc;
      }
    }
    if (keep) {
      for (int64_t j = 0; j < width - 1; ++j) state_out[(b * dim + d) * (width - 1) + j] = keep[j];
      free(keep);
    }
  }
}

/* d/da of the ZOH gain expm1(dt a)/a: (dt e^{dt a} - g)/a, written as
 * dt^2 * psi(q), psi(q) = sum_{k>=2} (k-1) q^{k-2} / k!, q = dt a, by its
 * series for small |q| (where the quotient cancels) and directly otherwise;
 * dt^2/2 at a = 0. */
static double zoh_gain_da(double dt, double a) {
  double q = dt * a;
  if (fabs(q) < 0.1) {
    double psi = 0.0, term = 0.5; /* term = q^{k-2} / k!, from k = 2 */
    for (int k = 2; k < 20; ++k) {
      psi += (double)(k - 1) * term;
      term *= q / (double)(k + 1);
    }
    return dt * dt * psi;
  }
  return (dt * exp(q) - expm1(q) / a) / a;
}

/*
 * O5. Gradient of the selective scan O1 (reverse-mode, exact in fp64).  The
 * pages give no backward pass; this is the adjoint of the recurrence as O1
 * writes it, pinned against central finite differences of O1.  For the scalar
 *   loss = sum_{b,t,d} dout[b,t,d] * out[b,t,d] + sum dh_final * h_final
 * it returns, per slice s = b*dim + d in [s_begin, s_end):
 *   dx, ddelta, dz (batch, seqlen, dim) and dh0 (batch, dim, dstate)   -- written;
 *   dA (dim, dstate), dB, dC (batch, seqlen, dstate), dDskip, ddelta_bias (dim)
 *                                                                     -- ADDED to;
 * (ddelta is the gradient with respect to the delta input, i.e. through the
 * bias and the softplus when they are used).  The caller gives each thread
 * its own accumulation buffers.  Optional inputs as in O1; dh_final, dz,
 * dh0, dDskip and ddelta_bias may be NULL.
 *
 * Adjoint of one step (lam = dloss/dh_t, then carried to h_{t-1}):
 *   dy = dout * silu(z);  dz = dout * y * silu'(z)
 *   lam_n += C_n dy;      dC_n += h_n dy
 *   dE = lam_n h_{t-1,n}; dg = lam_n B_n x
 *   dB_n += lam_n g x;    dx += lam_n g B_n  (+ Dskip dy)
 *   ddt += dE E a + dg E;           (d g/d dt = e^{dt a} = E)
 *   dA_n += dE E dt + dg dg/da;
 *   lam_n *= E
 */
static void selective_scan_bwd_impl(const double* x, const double* delta, const double* A,
                                    const double* B, const double* C, const double* Dskip,
                                    const double* z, const double* delta_bias, int delta_softplus,
                                    const double* h0, const double* dout, const double* dh_final,
                                    double* dx, double* ddelta, double* dA, double* dB, double* dC,
                                    double* dDskip, double* dz, double* ddelta_bias, double* dh0,
                                    int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                    int64_t s_begin, int64_t s_end, int euler) {
  (void)batch;
  size_t nh = (size_t)((seqlen + 1) * dstate > 0 ? (seqlen + 1) * dstate : 1);
  double* hs = (double*)malloc(sizeof(double) * nh);       /* h_t for t = -1 .. L-1 */
  double* dts = (double*)malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
  double* ys = (double*)malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
  double* lam = (double*)malloc(sizeof(double) * (size_t)(dstate > 0 ? dstate : 1));
  for (int64_t s = s_begin; s < s_end; ++s) {
    int64_t b = s / dim, d = s % dim;
    /* forward, keeping every state */
    for (int64_t n = 0; n < dstate; ++n) hs[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;
    for (int64_t t = 0; t < seqlen; ++t) {
      int64_t i = (b * seqlen + t) * dim + d, r = (b * seqlen + t) * dstate;
      double v = delta[i] + (delta_bias ? delta_bias[d] : 0.0);
      double dt = delta_softplus ? softplus(v) : v;
      dts[t] = dt;
      double acc = 0.0;
      for (int64_t n = 0; n < dstate; ++n) {
        double a = A[d * dstate + n];
        double g = euler ? dt : zoh_gain(dt, a);
        double h = exp(dt * a) * hs[t * dstate + n] + g * B[r + n] * x[i];
        hs[(t + 1) * dstate + n] = h;
        acc += C[r + n] * h;
      }
      ys[t] = acc + (Dskip ? Dskip[d] * x[i] : 0.0);
    }
    /* reverse */
    for (int64_t n = 0; n < dstate; ++n) lam[n] = dh_final ? dh_final[(b * dim + d) * dstate + n] : 0.0;
    for (int64_t t = seqlen - 1; t >= 0; --t) {
      int64_t i = (b * seqlen + t) * dim + d, r = (b * seqlen + t) * dstate;
      double dy = dout[i];
      if (z) {
        double sg = 1.0 / (1.0 + exp(-z[i]));
        if (dz) dz[i] = dout[i] * ys[t] * (sg + z[i] * sg * (1.0 - sg));
        dy = dout[i] * z[i] * sg;
      }
      double dxi = Dskip ? Dskip[d] * dy : 0.0;
      if (dDskip) dDskip[d] += dy * x[i];
      double dt = dts[t], ddt = 0.0;
      for (int64_t n = 0; n < dstate; ++n) {
        double a = A[d * dstate + n];
        double E = exp(dt * a), g = euler ? dt : zoh_gain(dt, a);
        lam[n] += C[r + n] * dy;
        dC[r + n] += hs[(t + 1) * dstate + n] * dy;
        double dE = lam[n] * hs[t * dstate + n];
        double dg = lam[n] * B[r + n] * x[i];
        dB[r + n] += lam[n] * g * x[i];
        dxi += lam[n] * g * B[r + n];
        /* dg/ddt: E for ZOH, 1 for Euler; dg/da: zoh_gain_da for ZOH, 0 for Euler */
        ddt += dE * E * a + dg * (euler ? 1.0 : E);
        dA[d * dstate + n] += dE * E * dt + (euler ? 0.0 : dg * zoh_gain_da(dt, a));
        lam[n] *= E;
      }
      dx[i] = dxi;
      double v = delta[i] + (delta_bias ? delta_bias[d] : 0.0);
      double dv = delta_softplus ? ddt / (1.0 + exp(-v)) : ddt;   /* softplus' = sigmoid */
      ddelta[i] = dv;
      if (ddelta_bias) ddelta_bias[d] += dv;
    }
    if (dh0)
      for (int64_t n = 0; n < dstate; ++n) dh0[(b * dim + d) * dstate + n] = lam[n];
  }
  free(hs);
  free(dts);
  free(ys);
  free(lam);
}

void oracle_selective_scan_bwd(const double* x, const double* delta, const double* A,
                               const double* B, const double* C, const double* Dskip,
                               const double* z, const double* delta_bias, int delta_softplus,
                               const double* h0, const double* dout, const double* dh_final,
                               double* dx, double* ddelta, double* dA, double* dB, double* dC,
                               double* dDskip, double* dz, double* ddelta_bias, double* dh0,
                               int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                               int64_t s_begin, int64_t s_end) {
  selective_scan_bwd_impl(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, dout, dh_final, dx,
                          ddelta, dA, dB, dC, dDskip, dz, ddelta_bias, dh0, batch, seqlen, dim, dstate, s_begin,
                          s_end, 0);
}

/* O5e. The gradient of O1e (Euler input discretization, gain dt): the same
 * adjoint with dg/ddt = 1 and dg/da = 0. */
void oracle_selective_scan_bwd_euler(const double* x, const double* delta, const double* A,
                                     const double* B, const double* C, const double* Dskip,
                                     const double* z, const double* delta_bias, int delta_softplus,
                                     const double* h0, const double* dout, const double* dh_final,
                                     double* dx, double* ddelta, double* dA, double* dB, double* dC,
                                     double* dDskip, double* dz, double* ddelta_bias, double* dh0,
                                     int64_t batch, int64_t seqlen, int64_t dim, int64_t dstate,
                                     int64_t s_begin, int64_t s_end) {
  selective_scan_bwd_impl(x, delta, A, B, C, Dskip, z, delta_bias, delta_softplus, h0, dout, dh_final, dx,
                          ddelta, dA, dB, dC, dDskip, dz, ddelta_bias, dh0, batch, seqlen, dim, dstate, s_begin,
                          s_end, 1);
}
