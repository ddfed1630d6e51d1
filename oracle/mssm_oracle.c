/*
 * mssm_oracle.c -- fp64 CPU oracle for the selective scan and its
 * single-token decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  The product path (the HIP
 * library under selective_state_space_52_amd/) shares no code with it and
 * never calls it.
 *
 * What is computed, and where it comes from:
 *
 *   - The continuous model h'(t) = A h(t) + B x(t), y(t) = C h(t) + D x(t)
 *     (page "Mamba: Selective State Space Models", section "Mathematical
 *     Foundation / State Space Model").  D enters as a skip term on the input.
 *   - B, C and the step size Delta depend on the token; Delta is the
 *     activation tau_Delta applied to (parameter + projection)
 *     (same page, "Mathematical Foundation / Selective Mechanism").  The
 *     parameter is the per-channel delta_bias below; tau_Delta is read as
 *     softplus(x) = log(1 + e^x) and may be switched off.
 *   - Delta drives the discretisation (same page, "Architecture").  The pages
 *     do not write the discrete rule out.  Reading used here: zero-order hold
 *     on A and an Euler step on B, i.e.
 *         h_t[n] = exp(Delta_t * A[n]) * h_{t-1}[n] + Delta_t * B_t[n] * u_t
 *         y_t    = sum_n C_t[n] * h_t[n] + D * u_t
 *     with y_t read from the state AFTER token t has been absorbed.
 *   - The output is gated by silu(z) = z / (1 + e^-z); the skip term sits
 *     inside the gate (same page, "Features": the block is gated).
 *   - Inference runs the recurrence token by token with a fixed-size state
 *     (same page, "Mathematical Foundation / Efficient Scan", sequential
 *     scan with constant memory).  This file is that sequential form, plain
 *     and in fp64.  The parallel scan of the same page reaches the same
 *     result up to rounding order, so no parallel form is needed here.
 *
 * Layouts (row-major, last index fastest), for one call:
 *   u, delta, z, out : (batch, dim, seqlen)
 *   B, C             : (batch, seqlen, dstate)   one N-vector per token
 *   A                : (dim, dstate)
 *   D, delta_bias    : (dim)
 *   h0, last_state   : (batch, dim, dstate)
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* largest state size the oracle's per-row arrays hold */
#define MSSM_ORACLE_MAX_N 256

/* tau_Delta = softplus, evaluated without a large-x threshold.  For x > 0
 * the form x + log1p(e^-x) avoids overflow; for x <= 0 log1p(e^x) keeps
 * relative accuracy when e^x is tiny. */
static double oracle_softplus(double x)
{
    if (x > 0.0)
        return x + log1p(exp(-x));
    return log1p(exp(x));
}

/* silu(z) = z * sigmoid(z) */
static double oracle_silu(double z)
{
    return z / (1.0 + exp(-z));
}

/*
 * One (batch, channel) row of the scan.
 *   u, delta, z, out : seqlen values of this row (z may be NULL: no gate)
 *   A_row            : dstate values A[d, :]
 *   B_b, C_b         : (seqlen, dstate) for this row's batch entry
 *   D_d, bias_d      : the channel's skip weight and delta bias
 *   h0               : dstate initial state, or NULL for zero
 *   last_state       : dstate final state, or NULL
 * h0 and last_state may point to the same memory.
 */
void mssm_oracle_scan_row(int64_t seqlen, int64_t dstate,
                          const double *u, const double *delta,
                          const double *z, const double *A_row,
                          const double *B_b, const double *C_b,
                          double D_d, double bias_d, int softplus,
                          const double *h0, double *out,
                          double *last_state)
{
    double h[MSSM_ORACLE_MAX_N];
    int64_t n, t;
    for (n = 0; n < dstate; ++n)
        h[n] = h0 ? h0[n] : 0.0;

    for (t = 0; t < seqlen; ++t) {
        double x = delta[t] + bias_d;
        double dt = softplus ? oracle_softplus(x) : x;
        double y = 0.0;
        for (n = 0; n < dstate; ++n) {
            double decay = exp(dt * A_row[n]);            /* Abar = exp(Delta A) */
            double drive = dt * B_b[t * dstate + n] * u[t]; /* Bbar u = Delta B u */
            h[n] = decay * h[n] + drive;
            y += C_b[t * dstate + n] * h[n];
        }
        y += D_d * u[t];
        out[t] = z ? y * oracle_silu(z[t]) : y;
    }

    if (last_state)
        for (n = 0; n < dstate; ++n)
            last_state[n] = h[n];
}

/*
 * B/C groups.  With ngroups = G, B and C hold G vectors per token, layout
 * (batch, seqlen, G, dstate), and channel d reads group d / (dim / G): the
 * first dim / G channels share group 0, and so on.  G = 1 is the single
 * shared vector of page "Mamba: Selective State Space Models", "Mathematical
 * Foundation / Selective Mechanism"; more groups are the layout variant of
 * the Mamba-2 block (page "Mamba State Space Model", "Use the Mamba2 block",
 * which takes a group count), read here as contiguous channel blocks.
 *
 * gather_groups copies X (batch, seqlen, G, dstate) into a new array
 * (batch, G, seqlen, dstate), so that each (batch entry, group) is one
 * contiguous (seqlen, dstate) block as the row routines take it.
 */
static double *gather_groups(const double *X, int64_t batch, int64_t seqlen,
                             int64_t ngroups, int64_t dstate)
{
    double *o = (double *)malloc(sizeof(double) * (size_t)(batch * ngroups * seqlen * dstate));
    int64_t b, t, g, n;
    if (!o)
        return NULL;
    for (b = 0; b < batch; ++b)
        for (t = 0; t < seqlen; ++t)
            for (g = 0; g < ngroups; ++g)
                for (n = 0; n < dstate; ++n)
                    o[((b * ngroups + g) * seqlen + t) * dstate + n] =
                        X[((b * seqlen + t) * ngroups + g) * dstate + n];
    return o;
}

/* the group of channel d */
static int64_t group_of(int64_t d, int64_t dim, int64_t ngroups)
{
    return d / (dim / ngroups);
}

/*
 * Whole scan.  D, z, delta_bias and h0 may be NULL (zero skip, no gate, zero
 * bias, zero initial state).  last_state may be NULL.  Rows are independent,
 * so they are spread over nthreads OpenMP threads (nthreads <= 0: default).
 * B, C are (batch, seqlen, ngroups, dstate).
 * Returns 0, -1 if dstate is outside 1..MSSM_ORACLE_MAX_N, -3 if ngroups
 * does not divide dim, -2 if out of memory.
 */
int mssm_oracle_scan(int64_t batch, int64_t dim, int64_t dstate,
                     int64_t seqlen, int64_t ngroups, const double *u,
                     const double *delta,
                     const double *A, const double *B, const double *C,
                     const double *D, const double *z,
                     const double *delta_bias, int softplus,
                     const double *h0, double *out, double *last_state,
                     int nthreads)
{
    int64_t rows = batch * dim;
    int64_t r;
    double *Bg, *Cg;
    if (dstate < 1 || dstate > MSSM_ORACLE_MAX_N)
        return -1;
    if (ngroups < 1 || dim % ngroups != 0)
        return -3;
    if (nthreads <= 0)
        nthreads = 1;
    Bg = gather_groups(B, batch, seqlen, ngroups, dstate);
    Cg = gather_groups(C, batch, seqlen, ngroups, dstate);
    if (!Bg || !Cg) {
        free(Bg);
        free(Cg);
        return -2;
    }
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (r = 0; r < rows; ++r) {
        int64_t b = r / dim, d = r % dim;
        size_t row = (size_t)r * (size_t)seqlen;
        size_t bc = (size_t)(b * ngroups + group_of(d, dim, ngroups)) *
                    (size_t)seqlen * (size_t)dstate;
        mssm_oracle_scan_row(seqlen, dstate, u + row, delta + row,
                             z ? z + row : NULL, A + d * dstate, Bg + bc,
                             Cg + bc, D ? D[d] : 0.0,
                             delta_bias ? delta_bias[d] : 0.0, softplus,
                             h0 ? h0 + r * dstate : NULL, out + row,
                             last_state ? last_state + r * dstate : NULL);
    }
    free(Bg);
    free(Cg);
    return 0;
}

/*
 * Single-token decode step: the scan above with seqlen = 1, starting from
 * `state` and writing the new state back into it (the fixed-size state that
 * inference carries from token to token).
 *   state            : (batch, dim, dstate), in/out
 *   x, dt, z, out    : (batch, dim)
 *   B, C             : (batch, ngroups, dstate)
 *   A                : (dim, dstate);  D, dt_bias : (dim)
 */
int mssm_oracle_state_update(int64_t batch, int64_t dim, int64_t dstate,
                             int64_t ngroups, double *state, const double *x,
                             const double *dt, const double *A,
                             const double *B, const double *C,
                             const double *D, const double *z,
                             const double *dt_bias, int softplus,
                             double *out, int nthreads)
{
    int64_t rows = batch * dim;
    int64_t r;
    if (dstate < 1 || dstate > MSSM_ORACLE_MAX_N)
        return -1;
    if (ngroups < 1 || dim % ngroups != 0)
        return -3;
    if (nthreads <= 0)
        nthreads = 1;
#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (r = 0; r < rows; ++r) {
        int64_t b = r / dim, d = r % dim;
        int64_t bg = (b * ngroups + group_of(d, dim, ngroups)) * dstate;
        double *h = state + r * dstate;
        mssm_oracle_scan_row(1, dstate, x + r, dt + r, z ? z + r : NULL,
                             A + d * dstate, B + bg, C + bg,
                             D ? D[d] : 0.0, dt_bias ? dt_bias[d] : 0.0,
                             softplus, h, out + r, h);
    }
    return 0;
}

/*
 * Gradients of one row of the scan (the reverse of mssm_oracle_scan_row).
 *
 * With the loss sum_t dout_t * out_t + sum_n dlast[n] * last_state[n], the
 * chain rule through the recurrence above gives, backwards in time, the
 * total gradient of the state
 *     g_t[n] = dy_t * C_t[n] + exp(Delta_{t+1} A[n]) * g_{t+1}[n],
 *     g_{L-1} = dlast + dy_{L-1} C_{L-1},   dy_t = dout_t * silu(z_t),
 * and from it every input's gradient (the derivative of each forward step
 * written out; softplus'(x) = sigmoid(x), silu'(z) = s(z)(1 + z(1 - s(z)))):
 *     du_t     = dy_t D + sum_n g_t[n] Delta_t B_t[n]
 *     dDelta_t = sum_n g_t[n] (B_t[n] u_t + A[n] exp(Delta_t A[n]) h_{t-1}[n])
 *     ddelta_t = dDelta_t * softplus'(delta_t + bias)   (or dDelta_t)
 *     dz_t     = dout_t * y_t * silu'(z_t)
 *     dA[n]   += sum_t g_t[n] Delta_t exp(Delta_t A[n]) h_{t-1}[n]
 *     dB_t[n] += g_t[n] Delta_t u_t       dC_t[n] += dy_t h_t[n]
 *     dD      += sum_t dy_t u_t           dbias   += sum_t ddelta_t
 *     dh0[n]   = exp(Delta_0 A[n]) g_0[n]
 * du, ddelta, dz are written; dA (dstate), dB_b, dC_b (seqlen x dstate),
 * *dD and *dbias are ADDED to (they sum over rows).  z, h0, dlast, dz, dh0
 * may be NULL.  Uses a scratch of 2 * seqlen * dstate + 3 * seqlen doubles.
 */
void mssm_oracle_scan_bwd_row(int64_t seqlen, int64_t dstate,
                              const double *u, const double *delta,
                              const double *z, const double *A_row,
                              const double *B_b, const double *C_b,
                              double D_d, double bias_d, int softplus,
                              const double *h0, const double *dout,
                              const double *dlast, double *du, double *ddelta,
                              double *dz, double *dA_row, double *dB_b,
                              double *dC_b, double *dD, double *dbias,
                              double *dh0, double *scratch)
{
    double *H = scratch;                      /* h_t, seqlen x dstate */
    double *E = H + seqlen * dstate;          /* exp(Delta_t A), same */
    double *DT = E + seqlen * dstate;         /* Delta_t */
    double *X = DT + seqlen;                  /* delta_t + bias */
    double *Y = X + seqlen;                   /* y_t before the gate */
    double g[MSSM_ORACLE_MAX_N];
    int64_t n, t;

    /* forward again, keeping every state */
    for (t = 0; t < seqlen; ++t) {
        double x = delta[t] + bias_d;
        double dt = softplus ? oracle_softplus(x) : x;
        double y = 0.0;
        X[t] = x;
        DT[t] = dt;
        for (n = 0; n < dstate; ++n) {
            double prev = t > 0 ? H[(t - 1) * dstate + n] : (h0 ? h0[n] : 0.0);
            double e = exp(dt * A_row[n]);
            E[t * dstate + n] = e;
            H[t * dstate + n] = e * prev + dt * B_b[t * dstate + n] * u[t];
            y += C_b[t * dstate + n] * H[t * dstate + n];
        }
        Y[t] = y + D_d * u[t];
    }

    for (n = 0; n < dstate; ++n)
        g[n] = dlast ? dlast[n] : 0.0;

    for (t = seqlen - 1; t >= 0; --t) {
        double dy, ddt = 0.0, dut;
        if (z) {
            double sg = 1.0 / (1.0 + exp(-z[t]));
            dy = dout[t] * z[t] * sg;
            if (dz)
                dz[t] = dout[t] * Y[t] * sg * (1.0 + z[t] * (1.0 - sg));
        } else {
            dy = dout[t];
        }
        dut = dy * D_d;
        *dD += dy * u[t];
        for (n = 0; n < dstate; ++n) {
            double prev = t > 0 ? H[(t - 1) * dstate + n] : (h0 ? h0[n] : 0.0);
            double e = E[t * dstate + n];
            double Bn = B_b[t * dstate + n];
            g[n] += dy * C_b[t * dstate + n];
            dC_b[t * dstate + n] += dy * H[t * dstate + n];
            dB_b[t * dstate + n] += g[n] * DT[t] * u[t];
            dut += g[n] * DT[t] * Bn;
            ddt += g[n] * (Bn * u[t] + A_row[n] * e * prev);
            dA_row[n] += g[n] * DT[t] * e * prev;
            g[n] *= e;
        }
        du[t] = dut;
        if (softplus)
            ddt *= 1.0 / (1.0 + exp(-X[t]));
        ddelta[t] = ddt;
        *dbias += ddt;
    }
    if (dh0)
        for (n = 0; n < dstate; ++n)
            dh0[n] = g[n];
}

/*
 * Gradients of the whole scan (serial over rows; the oracle is for tests).
 * Shapes as mssm_oracle_scan; dout (batch, dim, seqlen); dlast, dh0
 * (batch, dim, dstate) or NULL; outputs du, ddelta, dz (batch, dim, seqlen),
 * dA (dim, dstate), dB, dC (batch, seqlen, ngroups, dstate; each group sums
 * over its own channels), dD, dbias (dim), all overwritten.  Returns 0, -1
 * for an unsupported dstate, -3 if ngroups does not divide dim, -2 if out of
 * memory.
 */
int mssm_oracle_scan_bwd(int64_t batch, int64_t dim, int64_t dstate,
                         int64_t seqlen, int64_t ngroups, const double *u,
                         const double *delta,
                         const double *A, const double *B, const double *C,
                         const double *D, const double *z,
                         const double *delta_bias, int softplus,
                         const double *h0, const double *dout,
                         const double *dlast, double *du, double *ddelta,
                         double *dz, double *dA, double *dB, double *dC,
                         double *dD, double *dbias, double *dh0)
{
    int64_t r, i, b, t, g, n;
    const int64_t nbc = batch * ngroups * seqlen * dstate;
    double *scratch, *Bg, *Cg, *dBg, *dCg;
    if (dstate < 1 || dstate > MSSM_ORACLE_MAX_N)
        return -1;
    if (ngroups < 1 || dim % ngroups != 0)
        return -3;
    scratch = (double *)malloc(sizeof(double) * (size_t)(2 * seqlen * dstate + 3 * seqlen));
    Bg = gather_groups(B, batch, seqlen, ngroups, dstate);
    Cg = gather_groups(C, batch, seqlen, ngroups, dstate);
    dBg = (double *)calloc((size_t)nbc, sizeof(double));
    dCg = (double *)calloc((size_t)nbc, sizeof(double));
    if (!scratch || !Bg || !Cg || !dBg || !dCg) {
        free(scratch);
        free(Bg);
        free(Cg);
        free(dBg);
        free(dCg);
        return -2;
    }
    for (i = 0; i < dim * dstate; ++i)
        dA[i] = 0.0;
    for (i = 0; i < dim; ++i)
        dD[i] = dbias[i] = 0.0;
    for (r = 0; r < batch * dim; ++r) {
        int64_t bb = r / dim, d = r % dim;
        size_t row = (size_t)r * (size_t)seqlen;
        size_t bc = (size_t)(bb * ngroups + group_of(d, dim, ngroups)) *
                    (size_t)seqlen * (size_t)dstate;
        mssm_oracle_scan_bwd_row(
            seqlen, dstate, u + row, delta + row, z ? z + row : NULL,
            A + d * dstate, Bg + bc, Cg + bc, D ? D[d] : 0.0,
            delta_bias ? delta_bias[d] : 0.0, softplus,
            h0 ? h0 + r * dstate : NULL, dout + row,
            dlast ? dlast + r * dstate : NULL, du + row, ddelta + row,
            dz ? dz + row : NULL, dA + d * dstate, dBg + bc, dCg + bc, dD + d,
            dbias + d, dh0 ? dh0 + r * dstate : NULL, scratch);
    }
    /* back to (batch, seqlen, ngroups, dstate) */
    for (b = 0; b < batch; ++b)
        for (t = 0; t < seqlen; ++t)
            for (g = 0; g < ngroups; ++g)
                for (n = 0; n < dstate; ++n) {
                    const int64_t src = ((b * ngroups + g) * seqlen + t) * dstate + n;
                    const int64_t dst = ((b * seqlen + t) * ngroups + g) * dstate + n;
                    dB[dst] = dBg[src];
                    dC[dst] = dCg[src];
                }
    free(scratch);
    free(Bg);
    free(Cg);
    free(dBg);
    free(dCg);
    return 0;
}

/*
 * Causal depthwise convolution over time, ahead of the scan in the Mamba
 * block.  The pages give its width (d_conv = 4, "Local convolution width",
 * page "Mamba State Space Model" and page "Mamba: Selective State Space
 * Models", "Quick Start") and name the causal-conv1d package that provides
 * it, but not the formula.  Reading used here (the plain meaning of a causal
 * depthwise convolution of width K with a bias, as a framework's Conv1d with
 * K - 1 steps of left padding computes it):
 *     v[b,d,t] = bias[d] + sum_{k=0}^{K-1} w[d,k] * x[b,d,t-(K-1)+k]
 * so w[d,K-1] weighs the current step, and x at t < 0 is taken from `init`
 * (x[b,d,-(K-1)..-1], layout (batch, dim, K-1)) or is 0 when init is NULL.
 * With `silu` the output is silu(v) (the block feeds the scan the activated
 * convolution); without it, v.
 *   x, out : (batch, dim, seqlen);   w : (dim, K);   bias : (dim) or NULL
 */
int mssm_oracle_causal_conv1d(int64_t batch, int64_t dim, int64_t seqlen,
                              int64_t K, const double *x, const double *w,
                              const double *bias, const double *init,
                              int silu, double *out)
{
    if (K < 1)
        return -1;
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const double *xr = x + (b * dim + d) * seqlen;
            const double *wr = w + d * K;
            const double *ir = init ? init + (b * dim + d) * (K - 1) : NULL;
            double *o = out + (b * dim + d) * seqlen;
            for (int64_t t = 0; t < seqlen; ++t) {
                double v = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t s = t - (K - 1) + k;   /* source step */
                    double xv = 0.0;
                    if (s >= 0)
                        xv = xr[s];
                    else if (ir)
                        xv = ir[(K - 1) + s];          /* s in [-(K-1), -1] */
                    v += wr[k] * xv;
                }
                o[t] = silu ? oracle_silu(v) : v;
            }
        }
    }
    return 0;
}

/*
 * Gradients of the causal convolution above for an incoming dout = dLoss/d
 * out (the training step of the conv-fed block: the scan's backward gives
 * du, the gradient of its input u, which is this convolution's output).
 * Plain chain rule through v[b,d,t] = bias[d] + sum_k w[d,k] x[b,d,t-(K-1)+k]
 * and out = silu(v) (or v):
 *     g[t]       = dout[t] * silu'(v[t])   (or dout[t]),
 *                  silu'(v) = s (1 + v (1 - s)),  s = 1 / (1 + e^-v)
 *     dx[s]     += w[d,k] g[t]    for every t, k with s = t-(K-1)+k >= 0
 *     dinit[j]  += w[d,k] g[t]    for s = t-(K-1)+k < 0, j = (K-1) + s
 *     dw[d,k]   += g[t] x[s]      (x[s] from init, or 0, for s < 0)
 *     dbias[d]  += g[t]
 * dw and dbias sum over the batch and time; dx and dinit are per row.
 *   x, dout, dx : (batch, dim, seqlen);  w, dw : (dim, K);  bias, dbias :
 *   (dim) (bias may be NULL);  init, dinit : (batch, dim, K-1) (init may be
 *   NULL for zeros; dinit is the gradient of those values either way)
 */
int mssm_oracle_causal_conv1d_bwd(int64_t batch, int64_t dim, int64_t seqlen,
                                  int64_t K, const double *x, const double *w,
                                  const double *bias, const double *init,
                                  int silu, const double *dout, double *dx,
                                  double *dw, double *dbias, double *dinit)
{
    if (K < 1)
        return -1;
    for (int64_t d = 0; d < dim; ++d) {
        for (int64_t k = 0; k < K; ++k)
            dw[d * K + k] = 0.0;
        dbias[d] = 0.0;
    }
    for (int64_t b = 0; b < batch; ++b) {
        for (int64_t d = 0; d < dim; ++d) {
            const double *xr = x + (b * dim + d) * seqlen;
            const double *gr = dout + (b * dim + d) * seqlen;
            const double *wr = w + d * K;
            const double *ir = init ? init + (b * dim + d) * (K - 1) : NULL;
            double *dxr = dx + (b * dim + d) * seqlen;
            double *dir = dinit + (b * dim + d) * (K - 1);
            for (int64_t t = 0; t < seqlen; ++t)
                dxr[t] = 0.0;
            for (int64_t j = 0; j < K - 1; ++j)
                dir[j] = 0.0;
            for (int64_t t = 0; t < seqlen; ++t) {
                double v = bias ? bias[d] : 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t s = t - (K - 1) + k;
                    double xv = 0.0;
                    if (s >= 0)
                        xv = xr[s];
                    else if (ir)
                        xv = ir[(K - 1) + s];
                    v += wr[k] * xv;
                }
                double g = gr[t];
                if (silu) {
                    const double sg = 1.0 / (1.0 + exp(-v));
                    g *= sg * (1.0 + v * (1.0 - sg));
                }
                dbias[d] += g;
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t s = t - (K - 1) + k;
                    double xv = 0.0;
                    if (s >= 0) {
                        xv = xr[s];
                        dxr[s] += wr[k] * g;
                    } else {
                        if (ir)
                            xv = ir[(K - 1) + s];
                        dir[(K - 1) + s] += wr[k] * g;
                    }
                    dw[d * K + k] += g * xv;
                }
            }
        }
    }
    return 0;
}

int mssm_oracle_version(void) { return 1; }
