/*
 * ss_oracle.c -- CPU reference of the Mamba-1 S6 selective scan.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct oracle
 * the HIP path is checked against. Only the tests, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the product path never does.
 * It shares no code, header or constant with the HIP library.
 *
 * Arithmetic is IEEE double with libm exp/log1p; build without fast-math.
 * Every (batch, channel) row is an independent sequential token loop.
 *
 * What is computed (nnterp "selective_scan" page, class docstring: the
 * per-channel recurrence and the step size; TransformerLens "ssm_mixer" page,
 * compute_ssm_state: the same recurrence written per state coordinate):
 *
 *   dt_t = softplus(dt_raw_t + dt_bias)           (or dt_raw_t + dt_bias)
 *   h_t  = exp(dt_t * A) * h_{t-1} + dt_t * B_t * x_t
 *   y_t  = (C_t . h_t + D * x_t) * silu(z_t)       (gate optional)
 *
 * Readings where the pages leave a step open:
 *  - B is discretised as dt * B (both pages print it that way).
 *  - y_t reads the updated state h_t.
 *  - The gate multiplies the whole pre-gate output, D * x included (the
 *    ssm_mixer page calls y before the gate "the pre-gate scan output" and
 *    includes D * x in it).
 *  - A prompt without an initial state starts from zeros.
 *  - Hard reset ("s6_reset" post, Enforced Boundary Resetting, in the
 *    convention "the state is zeroed before a document's first token"):
 *    reset_t != 0 makes the decay of that token zero, so h_t = dt_t*B_t*x_t.
 *  - The decode step is the same body for one token, the state read and
 *    written in place, y from the updated state.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* softplus(v) = log(1 + e^v), written in the form that does not overflow. */
double oracle_softplus(double v) {
    return fmax(v, 0.0) + log1p(exp(-fabs(v)));
}

/* silu(z) = z * sigmoid(z) */
static double silu(double z) {
    return z / (1.0 + exp(-z));
}

/* Step size of one token of one channel. */
static double step_size(double dt_raw, const double* dt_bias, int64_t c, int dt_softplus) {
    double v = dt_raw + (dt_bias ? dt_bias[c] : 0.0);
    return dt_softplus ? oracle_softplus(v) : v;
}

/*
 * One token of one channel: update h[0..N) in place and return y before the
 * gate. Bt, Ct point at state coordinate 0 of this token; consecutive state
 * coordinates are bc_stride elements apart.
 */
static double s6_token(int64_t N, double* h, double d, double xv, const double* A_row,
                       const double* Bt, const double* Ct, int64_t bc_stride, int reset) {
    double y = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        double a = reset ? 0.0 : exp(d * A_row[n]);
        h[n] = a * h[n] + d * Bt[n * bc_stride] * xv;
        y += Ct[n * bc_stride] * h[n];
    }
    return y;
}

/*
 * Prompt scan over the flattened rows r = b * channels + c, r in
 * [row_begin, row_end). Layouts (all contiguous, C order):
 *   x, dt, z, y : [batch, channels, L]
 *   Bm, Cm      : [batch, N, L]
 *   A           : [channels, N];  D, dt_bias : [channels]
 *   h0, h_last  : [batch, channels, N]
 *   reset       : [batch, L] (uint8, nonzero = first token of a document)
 *   states      : [batch, channels, L, N] (optional: state after every token)
 * Optional pointers may be NULL: D (= 0), z (no gate), dt_bias (= 0),
 * h0 (zeros), reset (none), h_last, states.
 */
int oracle_scan(int64_t batch, int64_t channels, int64_t N, int64_t L,
                const double* x, const double* dt, const double* A,
                const double* Bm, const double* Cm, const double* D, const double* z,
                const double* dt_bias, const double* h0, const uint8_t* reset,
                int dt_softplus, double* y, double* h_last, double* states,
                int64_t row_begin, int64_t row_end) {
    if (batch < 0 || channels < 0 || N < 1 || N > 4096 || L < 0) return ORACLE_BAD_ARG;
    if (!x || !dt || !A || !Bm || !Cm || !y) return ORACLE_BAD_ARG;
    if (row_begin < 0 || row_end > batch * channels || row_begin > row_end) return ORACLE_BAD_ARG;
    double h[4096];
    for (int64_t r = row_begin; r < row_end; ++r) {
        const int64_t b = r / channels, c = r % channels;
        for (int64_t n = 0; n < N; ++n) h[n] = h0 ? h0[r * N + n] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const int64_t i = r * L + t;
            const double d = step_size(dt[i], dt_bias, c, dt_softplus);
            const int rs = reset ? (reset[b * L + t] != 0) : 0;
            double yt = s6_token(N, h, d, x[i], A + c * N, Bm + b * N * L + t, Cm + b * N * L + t, L, rs);
            yt += (D ? D[c] : 0.0) * x[i];
            if (z) yt *= silu(z[i]);
            y[i] = yt;
            if (states)
                for (int64_t n = 0; n < N; ++n) states[i * N + n] = h[n];
        }
        if (h_last)
            for (int64_t n = 0; n < N; ++n) h_last[r * N + n] = h[n];
    }
    return ORACLE_OK;
}

/*
 * Single-token decode step (nnterp "selective_scan" page: the state-update
 * kernel call on one token; the updated state is what the cache receives).
 *   state       : [batch, channels, N], read and written in place
 *   x, dt, z, y : [batch, channels]
 *   Bm, Cm      : [batch, N]
 * Rows r = b * channels + c in [row_begin, row_end).
 */
int oracle_update(int64_t batch, int64_t channels, int64_t N,
                  double* state, const double* x, const double* dt, const double* A,
                  const double* Bm, const double* Cm, const double* D, const double* z,
                  const double* dt_bias, int dt_softplus, double* y,
                  int64_t row_begin, int64_t row_end) {
    if (batch < 0 || channels < 0 || N < 1 || N > 4096) return ORACLE_BAD_ARG;
    if (!state || !x || !dt || !A || !Bm || !Cm || !y) return ORACLE_BAD_ARG;
    if (row_begin < 0 || row_end > batch * channels || row_begin > row_end) return ORACLE_BAD_ARG;
    for (int64_t r = row_begin; r < row_end; ++r) {
        const int64_t b = r / channels, c = r % channels;
        const double d = step_size(dt[r], dt_bias, c, dt_softplus);
        double yt = s6_token(N, state + r * N, d, x[r], A + c * N, Bm + b * N, Cm + b * N, 1, 0);
        yt += (D ? D[c] : 0.0) * x[r];
        if (z) yt *= silu(z[r]);
        y[r] = yt;
    }
    return ORACLE_OK;
}

/*
 * Scalar-gated state scan ("Mamba 2 Gated State Scan" problem page,
 * statement): per batch item a state matrix S of dk x dv numbers,
 *
 *   S_t = gamma_t * S_{t-1} + k_t v_t^T
 *   y_t = q_t^T S_t                       (the output reads the updated state)
 *
 * starting from s0 (zeros when s0 is NULL; the page starts every batch state
 * at zero). Layouts (contiguous, C order):
 *   q, k  : [batch, L, dk];  v, y : [batch, L, dv];  gamma : [batch, L]
 *   s0, final_state : [batch, dk, dv]
 * Batch items b in [b_begin, b_end); each is a sequential token loop.
 */
int oracle_gated_scan(int64_t batch, int64_t L, int64_t dk, int64_t dv,
                      const double* q, const double* k, const double* v, const double* gamma,
                      const double* s0, double* y, double* final_state,
                      int64_t b_begin, int64_t b_end) {
    if (batch < 0 || L < 0 || dk < 1 || dv < 1) return ORACLE_BAD_ARG;
    if (!q || !k || !v || !gamma || !y) return ORACLE_BAD_ARG;
    if (b_begin < 0 || b_end > batch || b_begin > b_end) return ORACLE_BAD_ARG;
    double* S = (double*)malloc((size_t)(dk * dv) * sizeof(double));
    if (!S) return ORACLE_BAD_ARG;
    for (int64_t b = b_begin; b < b_end; ++b) {
        for (int64_t e = 0; e < dk * dv; ++e) S[e] = s0 ? s0[b * dk * dv + e] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            const double g = gamma[b * L + t];
            const double* kt = k + (b * L + t) * dk;
            const double* vt = v + (b * L + t) * dv;
            const double* qt = q + (b * L + t) * dk;
            for (int64_t i = 0; i < dk; ++i)
                for (int64_t j = 0; j < dv; ++j) S[i * dv + j] = g * S[i * dv + j] + kt[i] * vt[j];
            for (int64_t j = 0; j < dv; ++j) {
                double acc = 0.0;
                for (int64_t i = 0; i < dk; ++i) acc += qt[i] * S[i * dv + j];
                y[(b * L + t) * dv + j] = acc;
            }
        }
        if (final_state)
            for (int64_t e = 0; e < dk * dv; ++e) final_state[b * dk * dv + e] = S[e];
    }
    free(S);
    return ORACLE_OK;
}

/*
 * Effective attention of the selective scan (TransformerLens "ssm_mixer"
 * page, compute_effective_attention): per batch item and channel,
 *
 *   M[c, i, j] = sum_n C[i, n] * prod_{k=j+1..i} exp(A[c, n] * dt[c, k]) * B[j, n]
 *
 * for j <= i (the product is empty, 1, at j == i) and 0 for j > i (causal).
 * dt is the step size (softplus of dt_raw + dt_bias, or dt_raw + dt_bias, as
 * in the scan). With include_dt nonzero column j is multiplied by dt[c, j]
 * (the page's reconstruction form, y = M x + D x before the gate). With
 * per_state nonzero the sum over n is not taken.
 *   dt          : [batch, channels, L]
 *   Bm, Cm      : [batch, N, L];  A : [channels, N];  dt_bias : [channels]
 *   out         : [batch, channels, L, L], or [batch, channels, N, L, L]
 * The product for column j is accumulated over i = j+1, j+2, ... one factor
 * at a time, in the order the page writes it. Rows r = b * channels + c in
 * [row_begin, row_end).
 */
int oracle_effective_attention(int64_t batch, int64_t channels, int64_t N, int64_t L,
                               const double* dt, const double* A, const double* Bm, const double* Cm,
                               const double* dt_bias, int dt_softplus, int include_dt, int per_state,
                               double* out, int64_t row_begin, int64_t row_end) {
    if (batch < 0 || channels < 0 || N < 1 || N > 4096 || L < 0) return ORACLE_BAD_ARG;
    if (!dt || !A || !Bm || !Cm || !out) return ORACLE_BAD_ARG;
    if (row_begin < 0 || row_end > batch * channels || row_begin > row_end) return ORACLE_BAD_ARG;
    double* d = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double prod[4096];
    if (!d) return ORACLE_BAD_ARG;
    for (int64_t r = row_begin; r < row_end; ++r) {
        const int64_t b = r / channels, c = r % channels;
        const double* Bb = Bm + b * N * L;
        const double* Cb = Cm + b * N * L;
        for (int64_t t = 0; t < L; ++t) d[t] = step_size(dt[r * L + t], dt_bias, c, dt_softplus);
        double* o = out + r * (per_state ? N : 1) * L * L;
        for (int64_t j = 0; j < L; ++j) {
            for (int64_t n = 0; n < N; ++n) prod[n] = 1.0;
            const double colscale = include_dt ? d[j] : 1.0;
            for (int64_t i = 0; i < L; ++i) {
                if (i > j)
                    for (int64_t n = 0; n < N; ++n) prod[n] *= exp(A[c * N + n] * d[i]);
                double m = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double term = i >= j ? Cb[n * L + i] * prod[n] * Bb[n * L + j] * colscale : 0.0;
                    if (per_state) o[(n * L + i) * L + j] = term;
                    m += term;
                }
                if (!per_state) o[i * L + j] = m;
            }
        }
    }
    free(d);
    return ORACLE_OK;
}

/*
 * Input side of the scan (nnterp "selective_scan" page, class docstring: the
 * scan's x is the causal conv1d output after SiLU, and its dt the dt_proj
 * output; TransformerLens "ssm_mixer" page: x is the post-conv SiLU input,
 * dt is read from dt_proj's output).
 *
 * Depthwise causal convolution of width W over the sequence, then SiLU:
 *   x[b, c, t] = silu(conv_b[c] + sum_{k=0}^{W-1} conv_w[c, k] * x_pre[b, c, t - (W-1) + k])
 * where a tap reading a position before 0, or before the first token of the
 * current document when a reset mask is given (reset[b, s] != 0 marks a
 * document's first token), reads 0: a document's convolution does not see
 * the previous document. conv_b may be NULL (= 0), reset NULL (one document).
 *   x_pre, x : [batch, channels, L];  conv_w : [channels, W];  reset : [batch, L]
 * Rows r = b * channels + c in [row_begin, row_end).
 */
int oracle_conv1d_silu(int64_t batch, int64_t channels, int64_t L, int64_t W,
                       const double* x_pre, const double* conv_w, const double* conv_b,
                       const uint8_t* reset, double* x, int64_t row_begin, int64_t row_end) {
    if (batch < 0 || channels < 0 || L < 0 || W < 1) return ORACLE_BAD_ARG;
    if (!x_pre || !conv_w || !x) return ORACLE_BAD_ARG;
    if (row_begin < 0 || row_end > batch * channels || row_begin > row_end) return ORACLE_BAD_ARG;
    for (int64_t r = row_begin; r < row_end; ++r) {
        const int64_t b = r / channels, c = r % channels;
        int64_t doc_start = 0;
        for (int64_t t = 0; t < L; ++t) {
            if (reset && reset[b * L + t]) doc_start = t;
            double acc = conv_b ? conv_b[c] : 0.0;
            for (int64_t k = 0; k < W; ++k) {
                const int64_t s = t - (W - 1) + k;
                if (s >= doc_start) acc += conv_w[c * W + k] * x_pre[r * L + s];
            }
            x[r * L + t] = silu(acc);
        }
    }
    return ORACLE_OK;
}

/*
 * dt_proj: the step sizes from the low-rank projection,
 *   dt[b, c, t] = sum_{k=0}^{R-1} w_dt[c, k] * delta[b, t, k]
 * and, with apply nonzero, dt <- softplus(dt + dt_bias[c]) (dt_bias NULL = 0),
 * the step size the scan would otherwise form from it.
 *   w_dt : [channels, R];  delta : [batch, L, R] (token-major, as the
 *   projection of the tokens produces it);  dt : [batch, channels, L]
 * Rows r = b * channels + c in [row_begin, row_end).
 */
int oracle_dt_proj(int64_t batch, int64_t channels, int64_t L, int64_t R,
                   const double* w_dt, const double* delta, const double* dt_bias, int apply,
                   double* dt, int64_t row_begin, int64_t row_end) {
    if (batch < 0 || channels < 0 || L < 0 || R < 1) return ORACLE_BAD_ARG;
    if (!w_dt || !delta || !dt) return ORACLE_BAD_ARG;
    if (row_begin < 0 || row_end > batch * channels || row_begin > row_end) return ORACLE_BAD_ARG;
    for (int64_t r = row_begin; r < row_end; ++r) {
        const int64_t b = r / channels, c = r % channels;
        for (int64_t t = 0; t < L; ++t) {
            double acc = 0.0;
            for (int64_t k = 0; k < R; ++k) acc += w_dt[c * R + k] * delta[(b * L + t) * R + k];
            dt[r * L + t] = apply ? oracle_softplus(acc + (dt_bias ? dt_bias[c] : 0.0)) : acc;
        }
    }
    return ORACLE_OK;
}
