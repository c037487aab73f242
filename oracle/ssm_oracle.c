/*
 * Selective-scan ORACLE: plain, slow, sequential fp64 CPU code.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU library never
 * links, includes or calls it, and it shares no code with the GPU path.
 *
 * What it computes is the textbook definition of the Mamba-1 selective scan,
 * written out with no blocking, fusion or reordering:
 *
 *   Delta discretisation  -- "Mamba State Space Models complete guide"
 *       (youngju.dev), section 5, "core innovation: selective mechanism":
 *       Delta is made positive by a softplus of its projection; here the
 *       projection output is `delta` plus an optional per-channel bias.
 *   Per-state decay       -- same page, section 2 "Discretization" (ZOH):
 *       Abar = exp(Delta * A).  A is diagonal, so this is one scalar exp per
 *       (channel d, state n).
 *   Input term            -- same page, section 5, the pure-PyTorch
 *       selective_scan of the "complete Mamba implementation": the input is
 *       injected as Delta * B * x (the simplified Bbar, not the ZOH one).
 *   Recurrence, readout   -- same page, section 2: x[t] = Abar x[t-1] + Bbar u[t],
 *       y[t] = C x[t]; plus the D skip term of the continuous SSM (section 2,
 *       "continuous-time SSM") and of the selective_scan listing.
 *   Gate                  -- same page, section 5 MambaBlock.forward: the SSM
 *       output is multiplied by SiLU(z).
 *   Initial / final state -- the state enters as h0 (as in the SM1 closed
 *       form, "Windows SM1 (Scalar Mamba1)" page, detailed-sections part) and
 *       the state after the last step is returned for continuation.
 *
 * Layouts (row-major, all fp64 here):
 *   x, delta, z, y : (B, T, D)      B, C : (B, T, N)      A : (D, N)
 *   D, delta_bias  : (D)            h0, last_state : (B, D, N)
 * Optional pointers may be NULL: delta_bias (no bias), D (no skip), z (no
 * gate), h0 (zero state), last_state (not written).  h0 and last_state may be
 * the same array: each chain reads its h0 before it writes its last_state.
 *
 * Chains (b, d) are independent; [chain_begin, chain_end) selects a range of
 * chain index c = b * D + d so a caller may run disjoint ranges on several
 * threads.  Nothing is shared between chains.
 *
 * The entry points used by the tests:
 *   oracle_selective_scan      -- the general scan (any N >= 1)
 *   oracle_state_update        -- one decode step: the scan with T = 1, state in/out
 *   oracle_sm1_scan            -- the d_state = 1 special case (same definition)
 *   oracle_selective_scan_bwd  -- the gradient of the general scan (below)
 *   oracle_causal_conv1d       -- the block's causal depthwise convolution + SiLU
 *                                 that produces the scan's x (below)
 *   oracle_conv1d_update       -- the same for one decode token, with the rolling
 *                                 window of past inputs
 *   oracle_ssd_scan            -- the Mamba-2 multi-head scan (scalar decay per head)
 *   oracle_dt_proj             -- the projection that produces the scan's delta input
 */
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

/* softplus(v) = log(1 + exp(v)), evaluated without overflow:
 * for v > 0, log(1 + e^v) = v + log(1 + e^-v). */
static double softplus(double v)
{
    if (v > 0.0)
        return v + log1p(exp(-v));
    return log1p(exp(v));
}

/* SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)). */
static double silu(double v)
{
    return v / (1.0 + exp(-v));
}

void oracle_selective_scan(const double *x, const double *delta, const double *delta_bias,
                           int delta_softplus, const double *A, const double *Bm,
                           const double *Cm, const double *Dv, const double *z,
                           const double *h0, double *y, double *last_state,
                           long nbatch, long seqlen, long dim, long dstate,
                           long chain_begin, long chain_end)
{
    if (dstate < 1)
        return;
    double h[dstate];
    for (long c = chain_begin; c < chain_end && c < nbatch * dim; ++c) {
        const long b = c / dim;
        const long d = c % dim;

        for (long n = 0; n < dstate; ++n)
            h[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;

        for (long t = 0; t < seqlen; ++t) {
            const long bt = b * seqlen + t;     /* row of the (B, T, .) tensors */
            const double xv = x[bt * dim + d];

            double v = delta[bt * dim + d];
            if (delta_bias)
                v += delta_bias[d];
            const double dt = delta_softplus ? softplus(v) : v;

            /* h[n] <- exp(dt * A[d,n]) * h[n] + dt * B[b,t,n] * x[b,t,d] */
            for (long n = 0; n < dstate; ++n) {
                const double decay = exp(dt * A[d * dstate + n]);
                h[n] = decay * h[n] + dt * Bm[bt * dstate + n] * xv;
            }

            /* y = sum_n C[b,t,n] h[n]  (+ D[d] x)  (* SiLU(z)) */
            double out = 0.0;
            for (long n = 0; n < dstate; ++n)
                out += Cm[bt * dstate + n] * h[n];
            if (Dv)
                out += Dv[d] * xv;
            if (z)
                out *= silu(z[bt * dim + d]);
            y[bt * dim + d] = out;
        }

        if (last_state)
            for (long n = 0; n < dstate; ++n)
                last_state[(b * dim + d) * dstate + n] = h[n];
    }
}

/* One recurrent decode step: the scan above with T = 1, the state read from
 * and written back to `state` (B, D, N).  x, delta, z, y are (B, D); B, C are
 * (B, N). */
void oracle_state_update(double *state, const double *x, const double *delta,
                         const double *delta_bias, int delta_softplus, const double *A,
                         const double *Bm, const double *Cm, const double *Dv, const double *z,
                         double *y, long nbatch, long dim, long dstate,
                         long chain_begin, long chain_end)
{
    oracle_selective_scan(x, delta, delta_bias, delta_softplus, A, Bm, Cm, Dv, z,
                          state, y, state, nbatch, 1, dim, dstate, chain_begin, chain_end);
}

/* SM1: the d_state = 1 case.  A is (D); B, C are (B, T); h0, last_state are
 * (B, D) -- the general layouts with N = 1. */
void oracle_sm1_scan(const double *x, const double *delta, const double *delta_bias,
                     int delta_softplus, const double *A, const double *Bm, const double *Cm,
                     const double *Dv, const double *z, const double *h0, double *y,
                     double *last_state, long nbatch, long seqlen, long dim,
                     long chain_begin, long chain_end)
{
    oracle_selective_scan(x, delta, delta_bias, delta_softplus, A, Bm, Cm, Dv, z, h0, y,
                          last_state, nbatch, seqlen, dim, 1, chain_begin, chain_end);
}

/* ---------------------------------------------------------------------------
 * The gradient of the scan above.
 *
 * Training a Mamba model differentiates the loss through the selective scan
 * (youngju.dev guide, the training loop of its practical section calls
 * loss.backward(); the "Windows SM1" page trains its scalar-state model the
 * same way through native PyTorch autograd).  The pages give no backward
 * formulas: what is computed here is the exact derivative of the forward
 * definition, by the chain rule applied to each statement of the forward
 * body in reverse order (reverse-mode differentiation), with the states of
 * the forward pass kept for every step.
 *
 * Given dout = dL/dout (B, T, D) and, optionally, dlast = dL/dlast_state
 * (B, D, N), it produces
 *   per element  : dx, ddelta, dz (B, T, D)      (dz only when z is given)
 *   per chain    : dh0 (B, D, N)                 (optional)
 *   accumulated  : dA (D, N), dB, dC (B, T, N), dD (D), ddelta_bias (D)
 * The accumulated ones are ADDED to what the arrays hold (the caller zeroes
 * them; several threads use separate arrays and sum them).  Any output
 * pointer may be NULL (not computed); dD / ddelta_bias / dz are skipped when
 * the forward had no D / bias / z.
 *
 * Per chain (b, d), with a_t[n] = exp(dt_t A[d,n]) and h_{-1} = h0:
 *   forward   h_t[n] = a_t[n] h_{t-1}[n] + dt_t B[t,n] x_t
 *             yv_t   = sum_n C[t,n] h_t[n] + D x_t ;  out_t = yv_t SiLU(z_t)
 *   backward  g[n]   = dlast[n]                        (dL/dh after the last step)
 *             for t = T-1 .. 0:
 *               dyv   = dout_t SiLU(z_t)
 *               dz_t  = dout_t yv_t SiLU'(z_t),  SiLU'(z) = s (1 + z (1 - s)), s = sigmoid(z)
 *               dD   += dyv x_t ;  dx_t = dyv D
 *               dC[t,n] += dyv h_t[n] ;  g[n] += dyv C[t,n]        (g = dL/dh_t)
 *               ddt   = sum_n g[n] (A[d,n] a_t[n] h_{t-1}[n] + B[t,n] x_t)
 *               dA[d,n] += g[n] dt_t a_t[n] h_{t-1}[n]
 *               dB[t,n] += g[n] dt_t x_t ;  dx_t += sum_n g[n] dt_t B[t,n]
 *               g[n]  = g[n] a_t[n]                                (now dL/dh_{t-1})
 *               ddelta_t = ddt sigmoid(v_t) with softplus (its derivative), else ddt
 *               dbias += ddelta_t
 *             dh0[n] = g[n]
 */
static double sigmoid(double v)
{
    return 1.0 / (1.0 + exp(-v));
}

void oracle_selective_scan_bwd(const double *x, const double *delta, const double *delta_bias,
                               int delta_softplus, const double *A, const double *Bm,
                               const double *Cm, const double *Dv, const double *z,
                               const double *h0, const double *dout, const double *dlast,
                               double *dx, double *ddelta, double *ddelta_bias, double *dA,
                               double *dB, double *dC, double *dD, double *dz, double *dh0,
                               long nbatch, long seqlen, long dim, long dstate,
                               long chain_begin, long chain_end)
{
    if (dstate < 1)
        return;
    /* hs[(t + 1) * N + n] = h_t[n], hs[n] = h0 ; dts[t] = Delta_t ; vs[t] = v_t */
    double *hs = malloc(sizeof(double) * (size_t)(seqlen + 1) * (size_t)dstate);
    double *dts = malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
    double *vs = malloc(sizeof(double) * (size_t)(seqlen > 0 ? seqlen : 1));
    double g[dstate];
    if (!hs || !dts || !vs) {
        free(hs); free(dts); free(vs);
        return;
    }
    for (long c = chain_begin; c < chain_end && c < nbatch * dim; ++c) {
        const long b = c / dim;
        const long d = c % dim;

        /* forward, keeping every state */
        for (long n = 0; n < dstate; ++n)
            hs[n] = h0 ? h0[(b * dim + d) * dstate + n] : 0.0;
        for (long t = 0; t < seqlen; ++t) {
            const long bt = b * seqlen + t;
            const double xv = x[bt * dim + d];
            double v = delta[bt * dim + d];
            if (delta_bias)
                v += delta_bias[d];
            const double dt = delta_softplus ? softplus(v) : v;
            vs[t] = v;
            dts[t] = dt;
            for (long n = 0; n < dstate; ++n) {
                const double decay = exp(dt * A[d * dstate + n]);
                hs[(t + 1) * dstate + n] = decay * hs[t * dstate + n] + dt * Bm[bt * dstate + n] * xv;
            }
        }

        /* backward */
        for (long n = 0; n < dstate; ++n)
            g[n] = dlast ? dlast[(b * dim + d) * dstate + n] : 0.0;
        for (long t = seqlen - 1; t >= 0; --t) {
            const long bt = b * seqlen + t;
            const double xv = x[bt * dim + d];
            const double dt = dts[t];
            const double *h_now = &hs[(t + 1) * dstate];
            const double *h_prev = &hs[t * dstate];
            const double go = dout[bt * dim + d];

            double dyv = go;
            if (z) {
                const double zv = z[bt * dim + d];
                const double s = sigmoid(zv);
                double yv = 0.0;
                for (long n = 0; n < dstate; ++n)
                    yv += Cm[bt * dstate + n] * h_now[n];
                if (Dv)
                    yv += Dv[d] * xv;
                dyv = go * zv * s;
                if (dz)
                    dz[bt * dim + d] = go * yv * s * (1.0 + zv * (1.0 - s));
            }
            double dxv = Dv ? dyv * Dv[d] : 0.0;
            if (Dv && dD)
                dD[d] += dyv * xv;
            double ddt = 0.0;
            for (long n = 0; n < dstate; ++n) {
                const double a = exp(dt * A[d * dstate + n]);
                if (dC)
                    dC[bt * dstate + n] += dyv * h_now[n];
                g[n] += dyv * Cm[bt * dstate + n];
                ddt += g[n] * (A[d * dstate + n] * a * h_prev[n] + Bm[bt * dstate + n] * xv);
                if (dA)
                    dA[d * dstate + n] += g[n] * dt * a * h_prev[n];
                if (dB)
                    dB[bt * dstate + n] += g[n] * dt * xv;
                dxv += g[n] * dt * Bm[bt * dstate + n];
                g[n] *= a;
            }
            const double dv = delta_softplus ? ddt * sigmoid(vs[t]) : ddt;
            if (dx)
                dx[bt * dim + d] = dxv;
            if (ddelta)
                ddelta[bt * dim + d] = dv;
            if (delta_bias && ddelta_bias)
                ddelta_bias[d] += dv;
        }
        if (dh0)
            for (long n = 0; n < dstate; ++n)
                dh0[(b * dim + d) * dstate + n] = g[n];
    }
    free(hs);
    free(dts);
    free(vs);
}

/* ---------------------------------------------------------------------------
 * The causal depthwise convolution in front of the scan.
 *
 * youngju.dev guide, section 5, "complete Mamba implementation": the x branch
 * of the input projection goes through nn.Conv1d with groups = d_inner (one
 * filter per channel), kernel size d_conv, padding d_conv - 1 on both sides
 * and the output cut to the first seqlen steps (causal), then SiLU, and only
 * then into the selective scan.  Written out for one channel d with filter
 * w[d, 0..K-1] (PyTorch's Conv1d is a cross-correlation):
 *     out[t] = bias[d] + sum_{k=0}^{K-1} w[d, k] * x[t - (K - 1) + k]
 * where x at a step before 0 is the value the caller hands in as the state
 * (the K - 1 inputs before the sequence, oldest first) or 0 without one.
 *
 * Layouts: x, out (B, T, D); w (D, K); bias (D) or NULL; state_in, state_out
 * (B, D, K - 1) or NULL.  state_out receives the last K - 1 inputs of the
 * extended sequence (state_in followed by x), oldest first, which is the
 * state the next call (or the decode step) continues from.  silu != 0 applies
 * SiLU to out.
 */
void oracle_causal_conv1d(const double *x, const double *w, const double *bias,
                          const double *state_in, double *out, double *state_out, int silu_on,
                          long nbatch, long seqlen, long dim, long width,
                          long chain_begin, long chain_end)
{
    const long H = width - 1;      /* inputs of history */
    for (long c = chain_begin; c < chain_end && c < nbatch * dim; ++c) {
        const long b = c / dim;
        const long d = c % dim;
        /* the extended input: step s in [-H, T) */
        for (long t = 0; t < seqlen; ++t) {
            double acc = bias ? bias[d] : 0.0;
            for (long k = 0; k < width; ++k) {
                const long s = t - H + k;
                double v;
                if (s >= 0)
                    v = x[(b * seqlen + s) * dim + d];
                else
                    v = state_in ? state_in[(b * dim + d) * H + (H + s)] : 0.0;
                acc += w[d * width + k] * v;
            }
            out[(b * seqlen + t) * dim + d] = silu_on ? silu(acc) : acc;
        }
        if (state_out)
            for (long j = 0; j < H; ++j) {
                const long s = seqlen - H + j;     /* extended step of state slot j */
                double v;
                if (s >= 0)
                    v = x[(b * seqlen + s) * dim + d];
                else
                    v = state_in ? state_in[(b * dim + d) * H + (H + s)] : 0.0;
                state_out[(b * dim + d) * H + j] = v;
            }
    }
}

/* One decode token: x, out (B, D); state (B, D, K - 1) in/out (read, then
 * replaced by the window shifted by one with x appended). */
void oracle_conv1d_update(double *state, const double *x, const double *w, const double *bias,
                          double *out, int silu_on, long nbatch, long dim, long width,
                          long chain_begin, long chain_end)
{
    const long H = width - 1;
    for (long c = chain_begin; c < chain_end && c < nbatch * dim; ++c) {
        const long b = c / dim;
        const long d = c % dim;
        double *st = &state[(b * dim + d) * H];
        double acc = bias ? bias[d] : 0.0;
        for (long k = 0; k < H; ++k)
            acc += w[d * width + k] * st[k];
        acc += w[d * width + H] * x[b * dim + d];
        out[b * dim + d] = silu_on ? silu(acc) : acc;
        for (long k = 0; k + 1 < H; ++k)
            st[k] = st[k + 1];
        if (H > 0)
            st[H - 1] = x[b * dim + d];
    }
}

/* ---------------------------------------------------------------------------
 * The Mamba-2 scan (youngju.dev guide, section 6 "Mamba 2"): a multi-head SSM
 * whose decay is one scalar per head.  The block's input projection gives,
 * per step, x and z (H heads of P channels each), one B and one C of N
 * values shared by every head, and one dt per head; A is a scalar per head
 * (the block keeps one A_log per head; A = -exp(A_log) as for Mamba-1).  The
 * section's sketch of the operation is the same recurrence as Mamba-1,
 * x[t] = A[t] x[t-1] + B[t] u[t], y[t] = C[t]^T x[t]; here, with the
 * discretisation of the Mamba-1 sections, every channel p of head h carries
 * an N-vector state:
 *
 *   Delta = softplus(dt[b,t,h] + dt_bias[h])       (or without the softplus)
 *   s[n] <- exp(Delta * A[h]) * s[n] + Delta * B[b,t,n] * x[b,t,h,p]
 *   y[b,t,h,p] = (sum_n C[b,t,n] s[n] + D[h] x[b,t,h,p]) * SiLU(z[b,t,h,p])
 *
 * The section's chunked evaluation (matrix products inside a chunk, the
 * recurrence between chunks) is an algorithm for the same result and is not
 * used here: this is the step-by-step definition.
 *
 * Layouts: x, z, y (B, T, H, P); dt (B, T, H); B, C (B, T, N); A, D,
 * dt_bias (H); h0, last_state (B, H, P, N).  Optional: dt_bias, D, z, h0,
 * last_state (NULL).  Chains c = (b * H + h) * P + p are independent.
 */
void oracle_ssd_scan(const double *x, const double *dt, const double *dt_bias, int dt_softplus,
                     const double *A, const double *Bm, const double *Cm, const double *Dv,
                     const double *z, const double *h0, double *y, double *last_state,
                     long nbatch, long seqlen, long nheads, long headdim, long dstate,
                     long chain_begin, long chain_end)
{
    if (dstate < 1)
        return;
    double s[dstate];
    const long nchains = nbatch * nheads * headdim;
    for (long c = chain_begin; c < chain_end && c < nchains; ++c) {
        const long p = c % headdim;
        const long h = (c / headdim) % nheads;
        const long b = c / (headdim * nheads);

        for (long n = 0; n < dstate; ++n)
            s[n] = h0 ? h0[c * dstate + n] : 0.0;

        for (long t = 0; t < seqlen; ++t) {
            const long bt = b * seqlen + t;                 /* row of (B, T, .) */
            const long xi = (bt * nheads + h) * headdim + p;  /* element of (B, T, H, P) */
            const double xv = x[xi];

            double v = dt[bt * nheads + h];
            if (dt_bias)
                v += dt_bias[h];
            const double delta = dt_softplus ? softplus(v) : v;
            const double decay = exp(delta * A[h]);

            for (long n = 0; n < dstate; ++n)
                s[n] = decay * s[n] + delta * Bm[bt * dstate + n] * xv;

            double out = 0.0;
            for (long n = 0; n < dstate; ++n)
                out += Cm[bt * dstate + n] * s[n];
            if (Dv)
                out += Dv[h] * xv;
            if (z)
                out *= silu(z[xi]);
            y[xi] = out;
        }

        if (last_state)
            for (long n = 0; n < dstate; ++n)
                last_state[c * dstate + n] = s[n];
    }
}


/*
 * dt_proj: the projection that produces the scan's delta input ("Mamba State
 * Space Models complete guide" (youngju.dev), section 5, the MambaBlock of the
 * complete implementation: a linear layer from dt_rank = d_model / 16 inputs
 * to d_inner outputs, applied to the first dt_rank columns of the x_proj
 * output, then softplus).  Its bias is the scan's delta_bias, which the scan
 * adds inside the softplus, so the product alone is computed here:
 *     out[m, d] = sum_{k=0}^{rank-1} xdt[m * ldx + k] * W[d * rank + k]
 * Layouts: xdt rows of stride ldx >= rank, of which only the first `rank`
 * columns are read (the rest of an x_proj row holds B and C); W (dim, rank)
 * row-major, the layer's weight; out (rows, dim).  Rows [row_begin, row_end)
 * are computed.
 */
void oracle_dt_proj(const double *xdt, long ldx, const double *W, double *out,
                    long rows, long rank, long dim, long row_begin, long row_end)
{
    for (long m = row_begin; m < row_end && m < rows; ++m) {
        for (long d = 0; d < dim; ++d) {
            double acc = 0.0;
            for (long k = 0; k < rank; ++k)
                acc += xdt[m * ldx + k] * W[d * rank + k];
            out[m * dim + d] = acc;
        }
    }
}
