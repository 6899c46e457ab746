/*
 * CPU oracle for the Mamba-2 SSD selective-scan forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code with the HIP library.
 *
 * What it computes is the plain definition, one timestep at a time, in fp64:
 *
 *   dt_t   = clamp(softplus(dt_raw_t + dt_bias_h), dt_min, dt_max)
 *   a_t    = exp(dt_t * A_h)                       (scalar decay per head)
 *   h_t    = a_t * h_{t-1} + dt_t * x_t (outer) B_t   h_{-1} = initial state
 *   y_t    = C_t . h_t + D_h * x_t
 *   out_t  = y_t * silu(z_t)                         (only when z is given)
 *
 * Sources, by page (the pages are GitHub threads about the mamba kernels):
 *  - The recurrence is the Mamba-2 state-space-duality (SSD) layer of
 *    Dao & Gu, "Transformers are SSMs" (2024), which the flash-linear-attention
 *    PR #49 page refers to ("Section 7.2 of the Mamba-2 paper").
 *  - dt is a discretization input absorbed into the log-gate dt*A, A is
 *    constant in time, there is no 1/sqrt(d) scaling of C.B, and B/C are shared
 *    by groups of heads like grouped-query keys: the same page, its list of
 *    differences between the simple_gla kernel and the mamba2_ssd kernel.
 *  - dt_bias, dt_limit, D (one value per head), the SiLU gate applied before
 *    any norm, initial_states and return_final_states: mamba issue #647, the
 *    repro script's arguments.
 *  - Continuation from a given state (chunked prefill): mamba issue #488.
 *  - seq_idx (several sequences packed along one batch row): an argument of
 *    the chunked-scan call in mamba issue #647's repro script.
 *
 * Readings taken where the pages are silent:
 *  - the state is stored as h[p][n] (headdim x dstate), the transpose of the
 *    B x^T form; the mathematics are identical;
 *  - y_t includes token t's own contribution (h_t is updated before use);
 *  - the input is scaled by dt (not the zero-order-hold (e^{dtA}-1)/A);
 *  - head h reads group g = h / (nheads / ngroups) (contiguous blocks);
 *  - dt_limit clamps after softplus; softplus is always applied;
 *  - the D skip is added before the gate: out = (C.h + D x) * silu(z);
 *  - seq_idx [batch, seqlen] (optional) labels the packed sequence each step
 *    belongs to; wherever it changes between steps t-1 and t a new sequence
 *    starts and the state is reset to zero before step t's update (nothing
 *    flows across the boundary).  initial_states is the state entering step
 *    0, i.e. that of the row's first sequence, and final_states the state
 *    after the last step, i.e. that of the row's last sequence.
 *
 * Layouts (row-major, contiguous):
 *   x, z        [batch, seqlen, nheads, headdim]           float32 values
 *   dt_raw      [batch, seqlen, nheads]                    float32 values
 *   B, C        [batch, seqlen, ngroups, dstate]           float32 values
 *   A, D, dt_bias [nheads]                                 float32 values
 *   seq_idx     [batch, seqlen]                            int32 labels
 *   init, final [batch, nheads, headdim, dstate]           fp64
 *   out         [batch, seqlen, nheads, headdim]           fp64
 * The inputs arrive as float32 because every input of the method is an fp32
 * or bf16 value, which float32 holds exactly; all arithmetic is fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(u) = log(1 + e^u), in the form that neither overflows nor
 * cancels: max(u,0) + log1p(e^{-|u|}). */
static double softplus(double u) { return (u > 0.0 ? u : 0.0) + log1p(exp(-fabs(u))); }

/* True when step t of batch row b starts a new packed sequence: its label
 * differs from step t-1's.  Step 0 continues from the initial state. */
static int new_sequence(const int32_t* seq_idx, int64_t L, int64_t b, int64_t t) {
    return seq_idx && t > 0 && seq_idx[b * L + t] != seq_idx[b * L + t - 1];
}

/* Discretization step of one (b, t, h): softplus of the biased raw value,
 * clamped to [dt_min, dt_max] (mamba issue #647 passes dt_limit=(0, inf)). */
static double step_dt(const float* dt_raw, const float* dt_bias, double dt_min, double dt_max,
                      int64_t L, int64_t H, int64_t b, int64_t t, int64_t h) {
    double u = (double)dt_raw[(b * L + t) * H + h] + (dt_bias ? (double)dt_bias[h] : 0.0);
    double dt = softplus(u);
    if (dt < dt_min) dt = dt_min;
    if (dt > dt_max) dt = dt_max;
    return dt;
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int oracle_max_threads(int nthreads) { return set_threads(nthreads); }

/*
 * The whole forward: out (and final state) for every (b, h) whose entry in
 * head_mask is non-zero (head_mask == NULL: all).  Entries of out for masked-
 * out heads are left untouched, so a caller can sample a few heads of a large
 * problem.  Returns 0, or -1 on bad shapes.
 */
int oracle_ssd_fwd(const float* x, const float* dt_raw, const float* A, const float* B,
                   const float* C, const float* D, const float* z, const float* dt_bias,
                   double dt_min, double dt_max, const double* init, double* out,
                   double* final_states, const int32_t* seq_idx, int64_t batch,
                   int64_t seqlen, int64_t nheads, int64_t headdim, int64_t dstate,
                   int64_t ngroups, const unsigned char* head_mask, int nthreads) {
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
        nheads % ngroups != 0)
        return -1;
    set_threads(nthreads);
    const int64_t L = seqlen, H = nheads, P = headdim, N = dstate, G = ngroups;
    const int64_t heads_per_group = H / G;
    const int64_t pairs = batch * H;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
        if (head_mask && !head_mask[bh]) continue;
        const int64_t b = bh / H, h = bh % H;
        const int64_t g = h / heads_per_group;
        double* S = (double*)malloc(sizeof(double) * (size_t)(P * N));
        if (init)
            memcpy(S, init + (b * H + h) * P * N, sizeof(double) * (size_t)(P * N));
        else
            memset(S, 0, sizeof(double) * (size_t)(P * N));
        const double Ah = (double)A[h];
        const double Dh = D ? (double)D[h] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            if (new_sequence(seq_idx, L, b, t)) memset(S, 0, sizeof(double) * (size_t)(P * N));
            const double dt = step_dt(dt_raw, dt_bias, dt_min, dt_max, L, H, b, t, h);
            const double a = exp(dt * Ah);
            const float* xt = x + ((b * L + t) * H + h) * P;
            const float* Bt = B + ((b * L + t) * G + g) * N;
            const float* Ct = C + ((b * L + t) * G + g) * N;
            for (int64_t p = 0; p < P; ++p) {
                const double u = dt * (double)xt[p];
                double* Sp = S + p * N;
                double y = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    Sp[n] = a * Sp[n] + u * (double)Bt[n];
                    y += Sp[n] * (double)Ct[n];
                }
                y += Dh * (double)xt[p];
                if (z) {
                    const double zz = (double)z[((b * L + t) * H + h) * P + p];
                    y *= zz / (1.0 + exp(-zz));
                }
                out[((b * L + t) * H + h) * P + p] = y;
            }
        }
        if (final_states) memcpy(final_states + (b * H + h) * P * N, S, sizeof(double) * (size_t)(P * N));
        free(S);
    }
    return 0;
}

/*
 * Per-chunk intermediates of the chunked form, each written out from its
 * definition (chunk c covers t in [c*Q, min((c+1)*Q, L))):
 *   dt_out  [b, H, nc, Q]      dt_t                      (0 past the end)
 *   cum_out [b, H, nc, Q]      sum_{r=cQ..t} dt_r*A_h    (held constant past the end)
 *   chunk_states [b, nc, H, P, N]  the recurrence run over chunk c alone,
 *                              starting from a zero state
 *   states_in    [b, nc, H, P, N]  the state of the full recurrence just
 *                              before chunk c's first step (init for c = 0)
 * With seq_idx both recurrences reset to zero where a new sequence starts.
 * Any output pointer may be NULL.  Returns 0, or -1 on bad shapes.
 */
int oracle_ssd_chunk_intermediates(const float* x, const float* dt_raw, const float* A,
                                   const float* B, const float* dt_bias, double dt_min,
                                   double dt_max, const double* init, double* dt_out,
                                   double* cum_out, double* chunk_states, double* states_in,
                                   const int32_t* seq_idx, int64_t batch, int64_t seqlen,
                                   int64_t nheads,
                                   int64_t headdim, int64_t dstate, int64_t ngroups,
                                   int64_t chunk_size, int nthreads) {
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
        nheads % ngroups != 0 || chunk_size <= 0)
        return -1;
    set_threads(nthreads);
    const int64_t L = seqlen, H = nheads, P = headdim, N = dstate, G = ngroups, Q = chunk_size;
    const int64_t nc = (L + Q - 1) / Q;
    const int64_t heads_per_group = H / G;
    const int64_t pairs = batch * H;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        const int64_t g = h / heads_per_group;
        const double Ah = (double)A[h];
        double* S = (double*)malloc(sizeof(double) * (size_t)(P * N));  /* full recurrence */
        double* Sc = (double*)malloc(sizeof(double) * (size_t)(P * N)); /* chunk-local */
        if (init)
            memcpy(S, init + (b * H + h) * P * N, sizeof(double) * (size_t)(P * N));
        else
            memset(S, 0, sizeof(double) * (size_t)(P * N));
        for (int64_t c = 0; c < nc; ++c) {
            const size_t state_off = (size_t)(((b * nc + c) * H + h) * P * N);
            if (states_in) memcpy(states_in + state_off, S, sizeof(double) * (size_t)(P * N));
            memset(Sc, 0, sizeof(double) * (size_t)(P * N));
            double cum = 0.0;
            for (int64_t q = 0; q < Q; ++q) {
                const int64_t t = c * Q + q;
                const size_t k = (size_t)(((b * H + h) * nc + c) * Q + q);
                if (t >= L) {
                    if (dt_out) dt_out[k] = 0.0;
                    if (cum_out) cum_out[k] = cum;
                    continue;
                }
                if (new_sequence(seq_idx, L, b, t)) {
                    memset(S, 0, sizeof(double) * (size_t)(P * N));
                    memset(Sc, 0, sizeof(double) * (size_t)(P * N));
                }
                const double dt = step_dt(dt_raw, dt_bias, dt_min, dt_max, L, H, b, t, h);
                cum += dt * Ah;
                if (dt_out) dt_out[k] = dt;
                if (cum_out) cum_out[k] = cum;
                const double a = exp(dt * Ah);
                const float* xt = x + ((b * L + t) * H + h) * P;
                const float* Bt = B + ((b * L + t) * G + g) * N;
                for (int64_t p = 0; p < P; ++p) {
                    const double u = dt * (double)xt[p];
                    for (int64_t n = 0; n < N; ++n) {
                        S[p * N + n] = a * S[p * N + n] + u * (double)Bt[n];
                        Sc[p * N + n] = a * Sc[p * N + n] + u * (double)Bt[n];
                    }
                }
            }
            if (chunk_states) memcpy(chunk_states + state_off, Sc, sizeof(double) * (size_t)(P * N));
        }
        free(S);
        free(Sc);
    }
    return 0;
}

/*
 * Backward of oracle_ssd_fwd: gradients of the loss
 *     l = sum(dout * out) + sum(dfinal * final_states)
 * with respect to every input, written out as the adjoint of the recurrence
 * (reverse-mode derivative, one timestep at a time, fp64).  With
 *     u_t = dt_raw_t + dt_bias_h,  dt_t = clamp(softplus(u_t), dt_min, dt_max),
 *     a_t = exp(dt_t A_h),  h_t = a_t h_{t-1} + dt_t x_t B_t^T,
 *     y_t = h_t C_t + D_h x_t,  out_t = y_t silu(z_t),
 * going backwards from g = dfinal (g is dl/dh_t):
 *     dy_t  = dout_t silu(z_t);   dz_t = dout_t y_t silu'(z_t)
 *     dC_t  = h_t^T dy_t                        (summed over the group's heads)
 *     g    += dy_t C_t^T                        (h_t feeds y_t)
 *     dx_t  = D_h dy_t + dt_t g B_t;   dD_h += dy_t . x_t
 *     dB_t += dt_t g^T x_t                      (summed over the group's heads)
 *     ddt_t = <g, x_t B_t^T> + A_h a_t <g, h_{t-1}>;  dA_h += dt_t a_t <g, h_{t-1}>
 *     g     = a_t g                             (on to h_{t-1})
 *     ddt_raw_t = ddt_t sigmoid(u_t) where softplus(u_t) lies in
 *                 [dt_min, dt_max] (the clamp passes it), else 0;
 *     ddt_bias_h = sum_t ddt_raw_t;   dinit = g after step 0.
 * (A seq_idx reset cuts g to zero where the state was reset.)  States are
 * kept at every 64th step in the forward pass and each 64-step segment is
 * recomputed from its checkpoint on the way back, so memory stays
 * O((L/64 + 64) P N) per (b, h).
 *
 * Outputs (fp64, all required): dx, dz (ignored when z is NULL) [b,L,H,P];
 * ddt_raw [b,L,H]; dA, dD, ddt_bias [H]; dB, dC [b,L,G,N]; dinit [b,H,P,N].
 * dout is required; dfinal may be NULL (zero).  Returns 0, or -1 on bad
 * shapes or failed allocation.
 */
int oracle_ssd_bwd(const float* x, const float* dt_raw, const float* A, const float* B,
                   const float* C, const float* D, const float* z, const float* dt_bias,
                   double dt_min, double dt_max, const double* init, const int32_t* seq_idx,
                   const double* dout, const double* dfinal, double* dx, double* dz,
                   double* ddt_raw, double* dA, double* dB, double* dC, double* dD,
                   double* ddt_bias, double* dinit, int64_t batch, int64_t seqlen,
                   int64_t nheads, int64_t headdim, int64_t dstate, int64_t ngroups,
                   int nthreads) {
    if (batch < 0 || seqlen < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
        nheads % ngroups != 0)
        return -1;
    set_threads(nthreads);
    const int64_t L = seqlen, H = nheads, P = headdim, N = dstate, G = ngroups;
    const int64_t heads_per_group = H / G, PN = P * N, SEG = 64;
    const int64_t nseg = (L + SEG - 1) / SEG;
    const int64_t pairs = batch * H;
    /* per-head partials of the group-shared gradients, summed afterwards */
    double* dBh = (double*)calloc((size_t)(batch * L * H * N), sizeof(double));
    double* dCh = (double*)calloc((size_t)(batch * L * H * N), sizeof(double));
    double* dAp = (double*)calloc((size_t)pairs, sizeof(double));
    double* dDp = (double*)calloc((size_t)pairs, sizeof(double));
    double* dbp = (double*)calloc((size_t)pairs, sizeof(double));
    if (!dBh || !dCh || !dAp || !dDp || !dbp) {
        free(dBh); free(dCh); free(dAp); free(dDp); free(dbp);
        return -1;
    }
    int failed = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        const int64_t g = h / heads_per_group;
        const double Ah = (double)A[h];
        const double Dh = D ? (double)D[h] : 0.0;
        double* ck = (double*)malloc(sizeof(double) * (size_t)((nseg + 1) * PN)); /* h before each segment */
        double* seg = (double*)malloc(sizeof(double) * (size_t)((SEG + 1) * PN)); /* h_{t0-1} .. h_{t0+SEG-1} */
        double* gs = (double*)malloc(sizeof(double) * (size_t)PN);
        if (!ck || !seg || !gs) {
            free(ck); free(seg); free(gs);
#pragma omp atomic write
            failed = 1;
            continue;
        }
        /* forward pass, keeping the state before every segment */
        double* S = seg;
        if (init) memcpy(S, init + (b * H + h) * PN, sizeof(double) * (size_t)PN);
        else memset(S, 0, sizeof(double) * (size_t)PN);
        for (int64_t t = 0; t < L; ++t) {
            if (t % SEG == 0) memcpy(ck + (t / SEG) * PN, S, sizeof(double) * (size_t)PN);
            if (new_sequence(seq_idx, L, b, t)) memset(S, 0, sizeof(double) * (size_t)PN);
            const double dtv = step_dt(dt_raw, dt_bias, dt_min, dt_max, L, H, b, t, h);
            const double a = exp(dtv * Ah);
            const float* xt = x + ((b * L + t) * H + h) * P;
            const float* Bt = B + ((b * L + t) * G + g) * N;
            for (int64_t p = 0; p < P; ++p)
                for (int64_t n = 0; n < N; ++n)
                    S[p * N + n] = a * S[p * N + n] + dtv * (double)xt[p] * (double)Bt[n];
        }
        /* backward, segment by segment from the end */
        if (dfinal) memcpy(gs, dfinal + (b * H + h) * PN, sizeof(double) * (size_t)PN);
        else memset(gs, 0, sizeof(double) * (size_t)PN);
        double dA_acc = 0.0, dD_acc = 0.0, db_acc = 0.0;
        for (int64_t sgi = nseg - 1; sgi >= 0; --sgi) {
            const int64_t t0 = sgi * SEG, t1 = (t0 + SEG < L) ? t0 + SEG : L;
            /* recompute h_{t0-1} .. h_{t1-1}: seg[(t - t0 + 1) * PN] = h_t */
            memcpy(seg, ck + sgi * PN, sizeof(double) * (size_t)PN);
            for (int64_t t = t0; t < t1; ++t) {
                double* prev = seg + (t - t0) * PN;
                double* cur = seg + (t - t0 + 1) * PN;
                const int reset = new_sequence(seq_idx, L, b, t);
                const double dtv = step_dt(dt_raw, dt_bias, dt_min, dt_max, L, H, b, t, h);
                const double a = exp(dtv * Ah);
                const float* xt = x + ((b * L + t) * H + h) * P;
                const float* Bt = B + ((b * L + t) * G + g) * N;
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n)
                        cur[p * N + n] = (reset ? 0.0 : a * prev[p * N + n]) +
                                         dtv * (double)xt[p] * (double)Bt[n];
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const double* prev = seg + (t - t0) * PN; /* h_{t-1} (before any reset) */
                const double* cur = seg + (t - t0 + 1) * PN;
                const int reset = new_sequence(seq_idx, L, b, t);
                const double u = (double)dt_raw[(b * L + t) * H + h] +
                                 (dt_bias ? (double)dt_bias[h] : 0.0);
                const double sp = softplus(u);
                const double dtv = step_dt(dt_raw, dt_bias, dt_min, dt_max, L, H, b, t, h);
                const double a = exp(dtv * Ah);
                const float* xt = x + ((b * L + t) * H + h) * P;
                const float* Bt = B + ((b * L + t) * G + g) * N;
                const float* Ct = C + ((b * L + t) * G + g) * N;
                const int64_t xo = ((b * L + t) * H + h) * P;
                /* gate and output */
                double dy[4096];
                double* dyp = P <= 4096 ? dy : (double*)malloc(sizeof(double) * (size_t)P);
                for (int64_t p = 0; p < P; ++p) {
                    double y = Dh * (double)xt[p];
                    for (int64_t n = 0; n < N; ++n) y += cur[p * N + n] * (double)Ct[n];
                    const double d = dout[xo + p];
                    if (z) {
                        const double zz = (double)z[xo + p];
                        const double sg = 1.0 / (1.0 + exp(-zz));
                        dyp[p] = d * zz * sg;
                        dz[xo + p] = d * y * sg * (1.0 + zz * (1.0 - sg));
                    } else {
                        dyp[p] = d;
                    }
                    dD_acc += dyp[p] * (double)xt[p];
                }
                /* dC_t = h_t^T dy_t ; g += dy_t C_t^T */
                double* dCt = dCh + ((b * L + t) * H + h) * N;
                for (int64_t n = 0; n < N; ++n) {
                    double s = 0.0;
                    for (int64_t p = 0; p < P; ++p) s += cur[p * N + n] * dyp[p];
                    dCt[n] = s;
                }
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n) gs[p * N + n] += dyp[p] * (double)Ct[n];
                /* through h_t = a h_{t-1} + dt x B^T */
                double* dBt = dBh + ((b * L + t) * H + h) * N;
                double gxb = 0.0, gh = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    double s = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        s += gs[p * N + n] * (double)Bt[n];
                        gh += gs[p * N + n] * prev[p * N + n];
                    }
                    dx[xo + p] = Dh * dyp[p] + dtv * s;
                    gxb += s * (double)xt[p];
                }
                for (int64_t n = 0; n < N; ++n) {
                    double s = 0.0;
                    for (int64_t p = 0; p < P; ++p) s += gs[p * N + n] * (double)xt[p];
                    dBt[n] = dtv * s;
                }
                if (reset) gh = 0.0; /* h_{t-1} did not reach h_t */
                const double ddt = gxb + Ah * a * gh;
                dA_acc += dtv * a * gh;
                const double pass = (sp >= dt_min && sp <= dt_max) ? 1.0 : 0.0;
                const double dr = ddt * pass / (1.0 + exp(-u));
                ddt_raw[(b * L + t) * H + h] = dr;
                db_acc += dr;
                /* on to h_{t-1} */
                for (int64_t k = 0; k < PN; ++k) gs[k] = reset ? 0.0 : a * gs[k];
                if (dyp != dy) free(dyp);
            }
        }
        memcpy(dinit + (b * H + h) * PN, gs, sizeof(double) * (size_t)PN);
        dAp[bh] = dA_acc;
        dDp[bh] = dD_acc;
        dbp[bh] = db_acc;
        free(ck);
        free(seg);
        free(gs);
    }
    if (!failed) {
        for (int64_t hh = 0; hh < H; ++hh) {
            double sa = 0.0, sd = 0.0, sb = 0.0;
            for (int64_t b = 0; b < batch; ++b) {
                sa += dAp[b * H + hh];
                sd += dDp[b * H + hh];
                sb += dbp[b * H + hh];
            }
            dA[hh] = sa;
            dD[hh] = sd;
            ddt_bias[hh] = sb;
        }
        for (int64_t bt = 0; bt < batch * L; ++bt)
            for (int64_t g = 0; g < G; ++g)
                for (int64_t n = 0; n < N; ++n) {
                    double sb = 0.0, sc = 0.0;
                    for (int64_t k = 0; k < heads_per_group; ++k) {
                        const int64_t hh = g * heads_per_group + k;
                        sb += dBh[(bt * H + hh) * N + n];
                        sc += dCh[(bt * H + hh) * N + n];
                    }
                    dB[(bt * G + g) * N + n] = sb;
                    dC[(bt * G + g) * N + n] = sc;
                }
    }
    free(dBh); free(dCh); free(dAp); free(dDp); free(dbp);
    return failed ? -1 : 0;
}
