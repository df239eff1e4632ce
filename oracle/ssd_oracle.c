/*
 * ssd_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, sequential fp64 CPU reference for the two operations of the SSD
 * hot path.  Only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  It shares no code, header or helper with the
 * HIP library in selective_state_space_ssd_amd/csrc and must never be called by
 * the product path.
 *
 * What it computes (the definition, written out, no blocking or reordering):
 *
 *   For every (batch b, head h), with group g = h / (H/G):
 *     s <- init_state[b,h]            (zeros when no initial state is given)
 *     for t = 0 .. L-1:
 *       s[p][n] <- exp(dt[b,t,h] * A[h]) * s[p][n] + dt[b,t,h] * x[b,t,h,p] * B[b,t,g,n]
 *       y[b,t,h,p] = sum_n C[b,t,g,n] * s[p][n] + D[h] * x[b,t,h,p]
 *     final_state[b,h] = s
 *
 * Sources (page title, section):
 *  - "另辟蹊径--Mamba介绍", «The Recurrent Representation»: the discrete state is
 *    the previous state times the discretised A plus the discretised B times the
 *    input, and the output C times the UPDATED state (so y_t sees x_t).
 *  - same page, «What is a State Space Model?» (output equation): D is a direct
 *    input-to-output skip term.
 *  - same page, «From a Continuous to a Discrete Signal» / «Zero-order hold实现»:
 *    the step size Delta discretises A; here Abar = exp(dt*A) and Bbar = dt*B
 *    (the pages strip the formulas; dt*B is the reading this library takes).
 *  - same page, «Selectively Retain Information»: B, C and Delta vary per token,
 *    A does not.
 *  - Bi-Mamba page, «Preliminary: Mamba Series»: in SSD, A is a scalar times the
 *    identity per head and the head dimension P is larger than one.
 *  - Mamba-2 article (msbhsh.com), «SSD 层» (grouped-value attention heads): B and
 *    C are shared by the heads of one group; head h uses group h / (H/G).
 *  - "如何将 Llama 变成 Mamba？...", «推测解码»: Mamba keeps only the current state,
 *    so the verify step must hand back the state at the accepted position.
 *
 * Precision: every product and sum is fp64 (no fused multiply-add contraction is
 * requested; build with -O2 -ffp-contract=off).  Inputs are the exact values the
 * GPU receives (bf16 or fp32 values widened to double).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_DIM 1
#define ORACLE_ERR_GROUPS 2
#define ORACLE_ERR_ACCEPT 3
#define ORACLE_ERR_ALLOC 4

/* One (batch, head) unit of the recurrence over tokens [0, T).  Token t of the
 * unit reads x at x_base + t*x_tstride etc.  s holds the P x N state (row p, col n)
 * on entry and on exit.  If states_out is non-null, the state after token t is
 * copied to states_out + t*states_tstride. */
static void recurrence_unit(double *s, const double *x, long x_tstride, const double *dt,
                            long dt_tstride, double A, const double *B, const double *C,
                            long bc_tstride, double D, double *y, long y_tstride, long T,
                            long P, long N, double *states_out, long states_tstride)
{
    for (long t = 0; t < T; ++t) {
        const double d = dt[t * dt_tstride];
        const double decay = exp(d * A);
        const double *xt = x + t * x_tstride;
        const double *Bt = B + t * bc_tstride;
        const double *Ct = C + t * bc_tstride;
        for (long p = 0; p < P; ++p) {
            const double u = d * xt[p];
            double *row = s + p * N;
            for (long n = 0; n < N; ++n)
                row[n] = decay * row[n] + u * Bt[n];
        }
        double *yt = y + t * y_tstride;
        for (long p = 0; p < P; ++p) {
            const double *row = s + p * N;
            double acc = 0.0;
            for (long n = 0; n < N; ++n)
                acc += Ct[n] * row[n];
            yt[p] = acc + D * xt[p];
        }
        if (states_out)
            memcpy(states_out + t * states_tstride, s, (size_t)(P * N) * sizeof(double));
    }
}

/*
 * Full-sequence recurrence (what the chunked scan must reproduce).
 * Layouts, row-major contiguous: x[b,L,H,P], dt[b,L,H], A[H], B,C[b,L,G,N], D[H],
 * init_state[b,H,P,N] (nullable -> zeros), y[b,L,H,P], final_state[b,H,P,N]
 * (nullable -> not written).  Only the (batch*H + head) units in
 * [bh_begin, bh_end) are computed, so a caller can evaluate a sample of heads or
 * split the units over threads; entries of y for other units are left untouched.
 */
int ssd_oracle_scan_f64(const double *x, const double *dt, const double *A, const double *B,
                        const double *C, const double *D, const double *init_state, double *y,
                        double *final_state, long b, long L, long H, long P, long N, long G,
                        long bh_begin, long bh_end)
{
    if (b < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0)
        return ORACLE_ERR_DIM;
    if (H % G != 0)
        return ORACLE_ERR_GROUPS;
    if (bh_begin < 0 || bh_end > b * H || bh_begin > bh_end)
        return ORACLE_ERR_DIM;
    const long heads_per_group = H / G;
    double *s = (double *)malloc((size_t)(P * N) * sizeof(double));
    if (!s)
        return ORACLE_ERR_ALLOC;
    for (long bh = bh_begin; bh < bh_end; ++bh) {
        const long bi = bh / H, h = bh % H, g = h / heads_per_group;
        if (init_state)
            memcpy(s, init_state + bh * P * N, (size_t)(P * N) * sizeof(double));
        else
            memset(s, 0, (size_t)(P * N) * sizeof(double));
        recurrence_unit(s, x + (bi * L * H + h) * P, H * P, dt + bi * L * H + h, H, A[h],
                        B + (bi * L * G + g) * N, C + (bi * L * G + g) * N, G * N, D[h],
                        y + (bi * L * H + h) * P, H * P, L, P, N, NULL, 0);
        if (final_state)
            memcpy(final_state + bh * P * N, s, (size_t)(P * N) * sizeof(double));
    }
    free(s);
    return ORACLE_OK;
}

/*
 * Verify step for K draft tokens applied to an existing state.
 * state_in[b,H,P,N], x[b,K,H,P], dt[b,K,H], B,C[b,K,G,N], accept_len[b] in [0,K].
 * Outputs: y[b,K,H,P] for all K positions; states_all[b,K,H,P,N] (nullable) =
 * state after k+1 tokens; state_out[b,H,P,N] = state after accept_len[b] tokens
 * (= state_in when accept_len is 0).  An accept_len outside [0,K] is an error here;
 * the oracle never clamps.
 */
int ssd_oracle_verify_f64(const double *state_in, const double *x, const double *dt,
                          const double *A, const double *B, const double *C, const double *D,
                          const int32_t *accept_len, double *y, double *state_out,
                          double *states_all, long b, long K, long H, long P, long N, long G)
{
    if (b < 0 || K <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0)
        return ORACLE_ERR_DIM;
    if (H % G != 0)
        return ORACLE_ERR_GROUPS;
    for (long bi = 0; bi < b; ++bi)
        if (accept_len[bi] < 0 || accept_len[bi] > K)
            return ORACLE_ERR_ACCEPT;
    const long heads_per_group = H / G;
    const long PN = P * N;
    double *s = (double *)malloc((size_t)PN * sizeof(double));
    double *hist = (double *)malloc((size_t)(K * PN) * sizeof(double));
    if (!s || !hist) {
        free(s);
        free(hist);
        return ORACLE_ERR_ALLOC;
    }
    for (long bi = 0; bi < b; ++bi) {
        for (long h = 0; h < H; ++h) {
            const long g = h / heads_per_group;
            const long bh = bi * H + h;
            memcpy(s, state_in + bh * PN, (size_t)PN * sizeof(double));
            recurrence_unit(s, x + (bi * K * H + h) * P, H * P, dt + bi * K * H + h, H, A[h],
                            B + (bi * K * G + g) * N, C + (bi * K * G + g) * N, G * N, D[h],
                            y + (bi * K * H + h) * P, H * P, K, P, N, hist, PN);
            const long a = accept_len[bi];
            const double *keep = (a == 0) ? state_in + bh * PN : hist + (a - 1) * PN;
            memcpy(state_out + bh * PN, keep, (size_t)PN * sizeof(double));
            if (states_all)
                for (long k = 0; k < K; ++k)
                    memcpy(states_all + ((bi * K + k) * H + h) * PN, hist + k * PN,
                           (size_t)PN * sizeof(double));
        }
    }
    free(s);
    free(hist);
    return ORACLE_OK;
}

/*
 * Selective scan with one channel per head and a diagonal state matrix (the
 * "selective SSM" the SSD layer replaces; kept as the comparison kernel):
 *
 *   For every (batch b, channel d), with group g = d / (Dch/G), and every state
 *   index n (each has its own decay A[d][n]):
 *     s[n] <- init_state[b,d,n]           (zeros when no initial state is given)
 *     for t = 0 .. L-1:
 *       s[n] <- exp(dt[b,t,d] * A[d][n]) * s[n] + dt[b,t,d] * x[b,t,d] * B[b,t,g,n]
 *       y[b,t,d] = sum_n C[b,t,g,n] * s[n] + D[d] * x[b,t,d]
 *     final_state[b,d] = s
 *
 * Sources (page title, section):
 *  - "另辟蹊径--Mamba介绍", «Selectively Retain Information»: B, C and the step size
 *    Delta are computed per token (they depend on the input), A is fixed.
 *  - same page, «The Scan Operation»: each state is the previous state times A
 *    plus the current input times B, computed with a scan.
 *  - Bi-Mamba page, «Preliminary: Mamba Series»: SSD restricts A to a scalar times
 *    the identity and uses a head dimension larger than the Mamba one, which is 1;
 *    so here every channel is its own head and A is a full diagonal (N values).
 *  - the discretisation and the output equation are those of ssd_oracle_scan_f64.
 *
 * Layouts: x, y [b,L,Dch]; dt [b,L,Dch]; A [Dch,N]; B, C [b,L,G,N]; D [Dch];
 * init_state, final_state [b,Dch,N] (init_state may be NULL).
 */
int ssd_oracle_selective_scan_f64(const double *x, const double *dt, const double *A,
                                  const double *B, const double *C, const double *D,
                                  const double *init_state, double *y, double *final_state,
                                  long b, long L, long Dch, long N, long G)
{
    if (b < 0 || L < 0 || Dch <= 0 || N <= 0 || G <= 0)
        return ORACLE_ERR_DIM;
    if (Dch % G != 0)
        return ORACLE_ERR_GROUPS;
    const long per_group = Dch / G;
    double *s = (double *)malloc((size_t)N * sizeof(double));
    if (!s)
        return ORACLE_ERR_ALLOC;
    for (long bi = 0; bi < b; ++bi) {
        for (long d = 0; d < Dch; ++d) {
            const long g = d / per_group;
            for (long n = 0; n < N; ++n)
                s[n] = init_state ? init_state[(bi * Dch + d) * N + n] : 0.0;
            for (long t = 0; t < L; ++t) {
                const double xv = x[(bi * L + t) * Dch + d];
                const double dv = dt[(bi * L + t) * Dch + d];
                const double *Bt = B + ((bi * L + t) * G + g) * N;
                const double *Ct = C + ((bi * L + t) * G + g) * N;
                double acc = 0.0;
                for (long n = 0; n < N; ++n) {
                    s[n] = exp(dv * A[d * N + n]) * s[n] + dv * xv * Bt[n];
                    acc += Ct[n] * s[n];
                }
                y[(bi * L + t) * Dch + d] = acc + D[d] * xv;
            }
            for (long n = 0; n < N; ++n)
                final_state[(bi * Dch + d) * N + n] = s[n];
        }
    }
    free(s);
    return ORACLE_OK;
}
