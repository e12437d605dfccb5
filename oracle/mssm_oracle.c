/*
 * CPU oracle for the selective-scan forward pass.  TEST INFRASTRUCTURE ONLY:
 * nothing in the product library links or calls this file; only the tests,
 * the smoke check and the benchmark's CPU-baseline leg use it.
 *
 * Plain, slow, sequential fp64 recurrences written straight from the
 * definitions.  No blocking, no chunking, no reordering: one (batch, channel)
 * row (Mamba-1) or one (batch, head) pair (Mamba-2 form) is walked step by
 * step in time.  Threads split independent rows only.
 *
 * Sources (page title + section):
 *  - "Mamba-2 y state-space models", 4.1: the recurrence h_t = A h_{t-1} + B x_t
 *    and the readout y_t = C h_t.
 *  - "P20 - Mamba", 5 (minimal maths): the selective SSM makes the recurrence
 *    and readout parameters depend on the current token.
 *  - "03 - Modelos de espacio de estados", "El mecanismo selectivo de Mamba":
 *    B, C and the step delta are per token; "Discretizacion": zero-order hold
 *    with A diagonal, so exp(delta*A) is taken elementwise; "Parallel scan":
 *    h_t = Abar_t h_{t-1} + Bbar_t x_t.
 *  - "Mamba-3" (blog), introduction: in Mamba-2 the transition is a scalar
 *    times the identity, so each head has one scalar A.
 *  - "Mamba-2 y state-space models", 4.3 notes: Mamba-2 organises the state
 *    in heads of size headdim.
 * Readings where the pages are silent or garbled:
 *  - Bbar x = delta * B * x (Euler step for the input, zero-order hold for A).
 *  - A is a fixed parameter (negative reals), delta arrives final.
 *  - out = (C.h + D*x) * silu(z), silu(z) = z / (1 + exp(-z)); D and z optional.
 *  - y_t reads the state after step t; h_{-1} = h0 (zero when absent).
 *  - Mamba-2 form: head h reads group g = h / (H / G) of B and C; D per head.
 *
 * Parity status of each function is stated in the oracle's Python wrapper.
 */
#include <complex.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define IO_F32 0
#define IO_BF16 1

/* bf16 bit pattern -> value (the upper half of an fp32) */
static double bf16_value(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_io(const void* p, int io, int64_t i) {
    if (io == IO_BF16) return bf16_value(((const uint16_t*)p)[i]);
    return (double)((const float*)p)[i];
}

static double silu(double v) { return v / (1.0 + exp(-v)); }

/* ------------------------------------------------------------------------- */
/* Mamba-1 selective scan                                                     */
/* ------------------------------------------------------------------------- */
typedef struct {
    int64_t Bsz, L, D, N;
    int io;
    const void *x, *delta, *Bm, *Cm, *z;
    const float *A, *Dv, *h0;
    const double* x64;       /* nullable: x already computed in fp64 (the convolution front end) */
    int64_t c0, c1;          /* channel range [c0, c1) */
    double *out, *final_state;
    int64_t row_begin, row_end;  /* rows = b * (c1 - c0) + (c - c0) */
} scan_job;

static void scan_row(const scan_job* j, int64_t b, int64_t c, double* h) {
    const int64_t N = j->N, D = j->D, L = j->L, nc = j->c1 - j->c0;
    for (int64_t n = 0; n < N; ++n) h[n] = j->h0 ? (double)j->h0[(b * D + c) * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const int64_t i = (b * L + t) * D + c;      /* [B, L, D] */
        const int64_t r = (b * L + t) * N;          /* [B, L, N] */
        const double d = load_io(j->delta, j->io, i);
        const double u = j->x64 ? j->x64[i] : load_io(j->x, j->io, i);
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            const double dA = exp(d * (double)j->A[c * N + n]);
            const double dBx = d * load_io(j->Bm, j->io, r + n) * u;
            h[n] = dA * h[n] + dBx;
            acc += load_io(j->Cm, j->io, r + n) * h[n];
        }
        double y = acc + (j->Dv ? (double)j->Dv[c] * u : 0.0);
        if (j->z) y *= silu(load_io(j->z, j->io, i));
        j->out[(b * L + t) * nc + (c - j->c0)] = y;
    }
    if (j->final_state)
        for (int64_t n = 0; n < N; ++n) j->final_state[(b * nc + (c - j->c0)) * N + n] = h[n];
}

static void* scan_worker(void* arg) {
    const scan_job* j = (const scan_job*)arg;
    const int64_t nc = j->c1 - j->c0;
    double* h = (double*)malloc(sizeof(double) * (size_t)j->N);
    for (int64_t row = j->row_begin; row < j->row_end; ++row)
        scan_row(j, row / nc, j->c0 + row % nc, h);
    free(h);
    return NULL;
}

/*
 * out [Bsz, L, c1-c0] fp64; final_state [Bsz, c1-c0, N] fp64 (nullable).
 * x, delta, z: [Bsz, L, D]; Bm, Cm: [Bsz, L, N] in io dtype; A [D, N], Dv [D],
 * h0 [Bsz, D, N] fp32 (Dv, z, h0 nullable).  Returns 0, or -1 on bad sizes.
 */
static int scan_fwd_impl(int64_t Bsz, int64_t L, int64_t D, int64_t N, int io,
                         const void* x, const double* x64, const void* delta, const float* A, const void* Bm,
                         const void* Cm, const float* Dv, const void* z, const float* h0, int64_t c0, int64_t c1,
                         double* out, double* final_state, int nthreads) {
    if (Bsz < 0 || L < 0 || D <= 0 || N <= 0 || c0 < 0 || c1 > D || c1 < c0) return -1;
    if (io != IO_F32 && io != IO_BF16) return -1;
    const int64_t rows = Bsz * (c1 - c0);
    if (rows == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > rows) nthreads = (int)rows;
    scan_job* jobs = (scan_job*)calloc((size_t)nthreads, sizeof(scan_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int k = 0; k < nthreads; ++k) {
        scan_job* j = &jobs[k];
        j->Bsz = Bsz; j->L = L; j->D = D; j->N = N; j->io = io;
        j->x = x; j->delta = delta; j->Bm = Bm; j->Cm = Cm; j->z = z;
        j->A = A; j->Dv = Dv; j->h0 = h0; j->x64 = x64; j->c0 = c0; j->c1 = c1;
        j->out = out; j->final_state = final_state;
        j->row_begin = rows * k / nthreads;
        j->row_end = rows * (k + 1) / nthreads;
    }
    for (int k = 1; k < nthreads; ++k) pthread_create(&th[k], NULL, scan_worker, &jobs[k]);
    scan_worker(&jobs[0]);
    for (int k = 1; k < nthreads; ++k) pthread_join(th[k], NULL);
    free(jobs);
    free(th);
    return 0;
}

int oracle_scan_fwd(int64_t Bsz, int64_t L, int64_t D, int64_t N, int io,
                    const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                    const float* Dv, const void* z, const float* h0, int64_t c0, int64_t c1,
                    double* out, double* final_state, int nthreads) {
    return scan_fwd_impl(Bsz, L, D, N, io, x, NULL, delta, A, Bm, Cm, Dv, z, h0, c0, c1, out, final_state,
                         nthreads);
}

/* ------------------------------------------------------------------------- */
/* Short causal convolution + SiLU in front of the scan                      */
/* ------------------------------------------------------------------------- */
/*
 * The short causal convolution of the Mamba-1/2 block ("Mamba-3" blog,
 * "Arquitectura": the layer Mamba-3 drops applied one to the state input;
 * "Mamba-2 y state-space models" 4.3 installs its kernel package beside the
 * scan's), read as a per-channel (depthwise) causal convolution over time of
 * width W followed by SiLU, its output being the scan's x:
 *   x[b,t,c] = silu(bias[c] + sum_{k<W} w[c,k] * xin[b, t-(W-1)+k, c])
 * where xin at a step before 0 is init[b, W-1+s, c] (the W-1 inputs that
 * precede the sequence, oldest first), or 0 without init.  fp64 out.
 */
int oracle_conv_silu(int64_t Bsz, int64_t L, int64_t D, int64_t W, int io, const void* xin, const float* w,
                     const float* bias, const void* init, double* x) {
    if (Bsz < 0 || L < 0 || D <= 0 || W < 1) return -1;
    if (io != IO_F32 && io != IO_BF16) return -1;
    for (int64_t b = 0; b < Bsz; ++b)
        for (int64_t t = 0; t < L; ++t)
            for (int64_t c = 0; c < D; ++c) {
                double acc = bias ? (double)bias[c] : 0.0;
                for (int64_t k = 0; k < W; ++k) {
                    const int64_t s = t - (W - 1) + k;
                    double v = 0.0;
                    if (s >= 0)
                        v = load_io(xin, io, (b * L + s) * D + c);
                    else if (init)
                        v = load_io(init, io, (b * (W - 1) + (W - 1) + s) * D + c);
                    acc += (double)w[c * W + k] * v;
                }
                x[(b * L + t) * D + c] = silu(acc);
            }
    return 0;
}

/* The scan of oracle_scan_fwd with x = oracle_conv_silu(xin, ...). */
int oracle_conv_scan_fwd(int64_t Bsz, int64_t L, int64_t D, int64_t N, int64_t W, int io,
                         const void* xin, const float* w, const float* bias, const void* init,
                         const void* delta, const float* A, const void* Bm, const void* Cm,
                         const float* Dv, const void* z, const float* h0, int64_t c0, int64_t c1,
                         double* out, double* final_state, int nthreads) {
    if (Bsz < 0 || L < 0 || D <= 0 || W < 1) return -1;
    double* x = (double*)malloc(sizeof(double) * (size_t)(Bsz * L * D > 0 ? Bsz * L * D : 1));
    int rc = oracle_conv_silu(Bsz, L, D, W, io, xin, w, bias, init, x);
    if (rc == 0)
        rc = scan_fwd_impl(Bsz, L, D, N, io, NULL, x, delta, A, Bm, Cm, Dv, z, h0, c0, c1, out, final_state,
                           nthreads);
    free(x);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Mamba-2 scalar-A multi-head form (its own loop, not a call into the above) */
/* ------------------------------------------------------------------------- */
typedef struct {
    int64_t Bsz, L, H, P, N, G;
    int io;
    const void *x, *delta, *Bm, *Cm, *z;
    const float *A, *Dv, *h0;
    int64_t hd0, hd1;        /* head range [hd0, hd1) */
    double *out, *final_state;
    int64_t pair_begin, pair_end;   /* pairs = b * (hd1 - hd0) + (h - hd0) */
} ssd_job;

static void ssd_pair(const ssd_job* j, int64_t b, int64_t hd, double* S) {
    const int64_t H = j->H, P = j->P, N = j->N, L = j->L, G = j->G, nh = j->hd1 - j->hd0;
    const int64_t g = hd / (H / G);
    for (int64_t p = 0; p < P; ++p)
        for (int64_t n = 0; n < N; ++n)
            S[p * N + n] = j->h0 ? (double)j->h0[((b * H + hd) * P + p) * N + n] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
        const double d = load_io(j->delta, j->io, (b * L + t) * H + hd);
        const double a = exp(d * (double)j->A[hd]);          /* scalar decay for the whole head */
        const int64_t r = ((b * L + t) * G + g) * N;           /* [B, L, G, N] */
        for (int64_t p = 0; p < P; ++p) {
            const int64_t i = ((b * L + t) * H + hd) * P + p;  /* [B, L, H, P] */
            const double u = load_io(j->x, j->io, i);
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                S[p * N + n] = a * S[p * N + n] + d * load_io(j->Bm, j->io, r + n) * u;
                acc += load_io(j->Cm, j->io, r + n) * S[p * N + n];
            }
            double y = acc + (j->Dv ? (double)j->Dv[hd] * u : 0.0);
            if (j->z) y *= silu(load_io(j->z, j->io, i));
            j->out[((b * L + t) * nh + (hd - j->hd0)) * P + p] = y;
        }
    }
    if (j->final_state)
        for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n)
                j->final_state[((b * nh + (hd - j->hd0)) * P + p) * N + n] = S[p * N + n];
}

static void* ssd_worker(void* arg) {
    const ssd_job* j = (const ssd_job*)arg;
    const int64_t nh = j->hd1 - j->hd0;
    double* S = (double*)malloc(sizeof(double) * (size_t)(j->P * j->N));
    for (int64_t k = j->pair_begin; k < j->pair_end; ++k) ssd_pair(j, k / nh, j->hd0 + k % nh, S);
    free(S);
    return NULL;
}

/*
 * out [Bsz, L, hd1-hd0, P] fp64; final_state [Bsz, hd1-hd0, P, N] fp64 (nullable).
 * x, z: [Bsz, L, H, P]; delta [Bsz, L, H]; Bm, Cm [Bsz, L, G, N] in io dtype;
 * A [H], Dv [H], h0 [Bsz, H, P, N] fp32 (Dv, z, h0 nullable).
 */
int oracle_ssd_fwd(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int io,
                   const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                   const float* Dv, const void* z, const float* h0, int64_t hd0, int64_t hd1,
                   double* out, double* final_state, int nthreads) {
    if (Bsz < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
    if (hd0 < 0 || hd1 > H || hd1 < hd0) return -1;
    if (io != IO_F32 && io != IO_BF16) return -1;
    const int64_t pairs = Bsz * (hd1 - hd0);
    if (pairs == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > pairs) nthreads = (int)pairs;
    ssd_job* jobs = (ssd_job*)calloc((size_t)nthreads, sizeof(ssd_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int k = 0; k < nthreads; ++k) {
        ssd_job* j = &jobs[k];
        j->Bsz = Bsz; j->L = L; j->H = H; j->P = P; j->N = N; j->G = G; j->io = io;
        j->x = x; j->delta = delta; j->Bm = Bm; j->Cm = Cm; j->z = z;
        j->A = A; j->Dv = Dv; j->h0 = h0; j->hd0 = hd0; j->hd1 = hd1;
        j->out = out; j->final_state = final_state;
        j->pair_begin = pairs * k / nthreads;
        j->pair_end = pairs * (k + 1) / nthreads;
    }
    for (int k = 1; k < nthreads; ++k) pthread_create(&th[k], NULL, ssd_worker, &jobs[k]);
    ssd_worker(&jobs[0]);
    for (int k = 1; k < nthreads; ++k) pthread_join(th[k], NULL);
    free(jobs);
    free(th);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Mamba-3 SISO recurrence: exponential-trapezoidal input rule (own loop)    */
/* ------------------------------------------------------------------------- */
/*
 * "Mamba-3" (blog), "El modelo Mamba-3" item 1: the recurrence comes from an
 * exponential-trapezoidal discretisation; "Arquitectura": it applies an
 * implicit convolution to the state's input, which is why the short
 * convolution can go.  The pages give no formula; this is the plain reading.
 * Over one step of length d the exact update of h' = a h + B(s) x(s) is
 *   h_t = exp(d a) h_{t-1} + integral_0^d exp((d - s) a) B(s) x(s) ds,
 * and the integral is taken by the weighted trapezoidal rule with weight
 * (1 - lam_t) on its left end (s = 0, where the integrand is
 * exp(d a) B_{t-1} x_{t-1}) and lam_t on its right end (s = d: B_t x_t):
 *   h_t = exp(d a) h_{t-1} + (1 - lam_t) d exp(d a) B_{t-1} x_{t-1} + lam_t d B_t x_t.
 * lam = 1/2 is the trapezoidal rule; lam = 1 is the right-end rule d B_t x_t
 * of the Mamba-2 form above.  lam_t is per (batch, step, head), given by the
 * caller.  Before step 0 there is no input: B_{-1} x_{-1} = 0, and h0 is h_{-1}.
 * Readout, D and gate as in the Mamba-2 form.
 */
typedef struct {
    int64_t Bsz, L, H, P, N, G;
    int io;
    const void *x, *delta, *lam, *Bm, *Cm, *z;
    const float *A, *Dv, *h0;
    double *out, *final_state;
    int64_t pair_begin, pair_end;   /* pairs = b * H + h */
} ssd3_job;

static void ssd3_pair(const ssd3_job* j, int64_t b, int64_t hd, double* S, double* bx_prev) {
    const int64_t H = j->H, P = j->P, N = j->N, L = j->L, G = j->G;
    const int64_t g = hd / (H / G);
    for (int64_t p = 0; p < P; ++p)
        for (int64_t n = 0; n < N; ++n) {
            S[p * N + n] = j->h0 ? (double)j->h0[((b * H + hd) * P + p) * N + n] : 0.0;
            bx_prev[p * N + n] = 0.0;                           /* B_{-1} x_{-1} */
        }
    for (int64_t t = 0; t < L; ++t) {
        const double d = load_io(j->delta, j->io, (b * L + t) * H + hd);
        const double lam = load_io(j->lam, j->io, (b * L + t) * H + hd);
        const double a = exp(d * (double)j->A[hd]);
        const double w_left = (1.0 - lam) * d * a, w_right = lam * d;
        const int64_t r = ((b * L + t) * G + g) * N;
        for (int64_t p = 0; p < P; ++p) {
            const int64_t i = ((b * L + t) * H + hd) * P + p;
            const double u = load_io(j->x, j->io, i);
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                const double bx = load_io(j->Bm, j->io, r + n) * u;
                S[p * N + n] = a * S[p * N + n] + w_left * bx_prev[p * N + n] + w_right * bx;
                bx_prev[p * N + n] = bx;
                acc += load_io(j->Cm, j->io, r + n) * S[p * N + n];
            }
            double y = acc + (j->Dv ? (double)j->Dv[hd] * u : 0.0);
            if (j->z) y *= silu(load_io(j->z, j->io, i));
            j->out[i] = y;
        }
    }
    if (j->final_state)
        for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n)
                j->final_state[((b * H + hd) * P + p) * N + n] = S[p * N + n];
}

static void* ssd3_worker(void* arg) {
    const ssd3_job* j = (const ssd3_job*)arg;
    double* S = (double*)malloc(sizeof(double) * (size_t)(2 * j->P * j->N));
    for (int64_t k = j->pair_begin; k < j->pair_end; ++k) ssd3_pair(j, k / j->H, k % j->H, S, S + j->P * j->N);
    free(S);
    return NULL;
}

/*
 * out [Bsz, L, H, P] fp64; final_state [Bsz, H, P, N] fp64 (nullable).
 * x, z: [Bsz, L, H, P]; delta, lam [Bsz, L, H]; Bm, Cm [Bsz, L, G, N] in io
 * dtype; A [H], Dv [H], h0 [Bsz, H, P, N] fp32 (Dv, z, h0 nullable).
 */
int oracle_ssd3_fwd(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int io,
                    const void* x, const void* delta, const void* lam, const float* A, const void* Bm,
                    const void* Cm, const float* Dv, const void* z, const float* h0,
                    double* out, double* final_state, int nthreads) {
    if (Bsz < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return -1;
    if (io != IO_F32 && io != IO_BF16) return -1;
    const int64_t pairs = Bsz * H;
    if (pairs == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > pairs) nthreads = (int)pairs;
    ssd3_job* jobs = (ssd3_job*)calloc((size_t)nthreads, sizeof(ssd3_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int k = 0; k < nthreads; ++k) {
        ssd3_job* j = &jobs[k];
        j->Bsz = Bsz; j->L = L; j->H = H; j->P = P; j->N = N; j->G = G; j->io = io;
        j->x = x; j->delta = delta; j->lam = lam; j->Bm = Bm; j->Cm = Cm; j->z = z;
        j->A = A; j->Dv = Dv; j->h0 = h0;
        j->out = out; j->final_state = final_state;
        j->pair_begin = pairs * k / nthreads;
        j->pair_end = pairs * (k + 1) / nthreads;
    }
    for (int k = 1; k < nthreads; ++k) pthread_create(&th[k], NULL, ssd3_worker, &jobs[k]);
    ssd3_worker(&jobs[0]);
    for (int k = 1; k < nthreads; ++k) pthread_join(th[k], NULL);
    free(jobs);
    free(th);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Mamba-3 MIMO: several inputs and outputs per channel on one state (own loop) */
/* ------------------------------------------------------------------------- */
/*
 * "Mamba-3" (blog), "El modelo Mamba-3" item 3: multi-input multi-output SSMs
 * model several SSMs in parallel against the single-input single-output
 * ones; "Arquitectura": the MIMO projections widen B and C; "Tareas de
 * recuperacion": MIMO does not grow the state.  The pages give no formula;
 * plain reading (the control-theory sense of MIMO on the multi-head state):
 * each channel p of head h takes R inputs x[t,h,r,p] and gives R outputs; the
 * R input terms drive the one state S[p,n] of the head through one transition
 * (B widened to B[t,g,r,n]), and output r reads that state through its own
 * C[t,g,r,n].  With U_t[p,n] = sum_r B[t,g,r,n] x[t,h,r,p] and the
 * exponential-trapezoidal rule of oracle_ssd3_fwd:
 *   S_t = a_t S_{t-1} + (1 - lam_t) d_t a_t U_{t-1} + lam_t d_t U_t
 *   y[t,h,r,p] = sum_n C[t,g,r,n] S_t[p,n] + D[h] x[t,h,r,p],  out = y silu(z[t,h,r,p])
 * lam NULL is lam = 1 everywhere (the Mamba-2 rule d_t U_t).  R = 1 is
 * oracle_ssd3_fwd (oracle_ssd_fwd without lam).  The token before step 0 is
 * x_prev / B_prev (nullable: U_{-1} = 0).
 */
typedef struct {
    int64_t Bsz, L, H, P, N, G, R;
    int io;
    const void *x, *delta, *lam, *Bm, *Cm, *z, *x_prev, *B_prev;
    const float *A, *Dv, *h0;
    double *out, *final_state;
    int64_t pair_begin, pair_end;   /* pairs = b * H + h */
} ssdm_job;

static void ssdm_pair(const ssdm_job* j, int64_t b, int64_t hd, double* S, double* U_prev, double* U) {
    const int64_t H = j->H, P = j->P, N = j->N, L = j->L, G = j->G, R = j->R;
    const int64_t g = hd / (H / G);
    for (int64_t p = 0; p < P; ++p)
        for (int64_t n = 0; n < N; ++n) {
            S[p * N + n] = j->h0 ? (double)j->h0[((b * H + hd) * P + p) * N + n] : 0.0;
            double u = 0.0;                                           /* U_{-1}: the token before step 0 */
            if (j->x_prev && j->B_prev)
                for (int64_t r = 0; r < R; ++r)
                    u += load_io(j->B_prev, j->io, ((b * G + g) * R + r) * N + n) *
                         load_io(j->x_prev, j->io, ((b * H + hd) * R + r) * P + p);
            U_prev[p * N + n] = u;
        }
    for (int64_t t = 0; t < L; ++t) {
        const double d = load_io(j->delta, j->io, (b * L + t) * H + hd);
        const double lam = j->lam ? load_io(j->lam, j->io, (b * L + t) * H + hd) : 1.0;
        const double a = exp(d * (double)j->A[hd]);
        const double w_left = (1.0 - lam) * d * a, w_right = lam * d;
        const int64_t bc = ((b * L + t) * G + g) * R;                 /* row of rank 0 in B, C */
        const int64_t xr = ((b * L + t) * H + hd) * R;                /* row of rank 0 in x, z, out */
        for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n) {
                double u = 0.0;                                       /* sum over the R inputs */
                for (int64_t r = 0; r < R; ++r)
                    u += load_io(j->Bm, j->io, (bc + r) * N + n) * load_io(j->x, j->io, (xr + r) * P + p);
                U[p * N + n] = u;
                S[p * N + n] = a * S[p * N + n] + w_left * U_prev[p * N + n] + w_right * u;
            }
        for (int64_t r = 0; r < R; ++r)                               /* each output reads the one state */
            for (int64_t p = 0; p < P; ++p) {
                const int64_t i = (xr + r) * P + p;
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) acc += load_io(j->Cm, j->io, (bc + r) * N + n) * S[p * N + n];
                double y = acc + (j->Dv ? (double)j->Dv[hd] * load_io(j->x, j->io, i) : 0.0);
                if (j->z) y *= silu(load_io(j->z, j->io, i));
                j->out[i] = y;
            }
        memcpy(U_prev, U, sizeof(double) * (size_t)(P * N));
    }
    if (j->final_state)
        for (int64_t p = 0; p < P; ++p)
            for (int64_t n = 0; n < N; ++n)
                j->final_state[((b * H + hd) * P + p) * N + n] = S[p * N + n];
}

static void* ssdm_worker(void* arg) {
    const ssdm_job* j = (const ssdm_job*)arg;
    const int64_t n = j->P * j->N;
    double* S = (double*)malloc(sizeof(double) * (size_t)(3 * n));
    for (int64_t k = j->pair_begin; k < j->pair_end; ++k) ssdm_pair(j, k / j->H, k % j->H, S, S + n, S + 2 * n);
    free(S);
    return NULL;
}

/*
 * out [Bsz, L, H, R, P] fp64; final_state [Bsz, H, P, N] fp64 (nullable).
 * x, z [Bsz, L, H, R, P]; delta, lam [Bsz, L, H]; Bm, Cm [Bsz, L, G, R, N];
 * x_prev [Bsz, H, R, P], B_prev [Bsz, G, R, N] in io dtype; A [H], Dv [H],
 * h0 [Bsz, H, P, N] fp32.  lam, Dv, z, h0, x_prev, B_prev nullable.
 */
int oracle_ssdm_fwd(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t R, int io,
                    const void* x, const void* delta, const void* lam, const float* A, const void* Bm,
                    const void* Cm, const float* Dv, const void* z, const float* h0, const void* x_prev,
                    const void* B_prev, double* out, double* final_state, int nthreads) {
    if (Bsz < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || R <= 0 || H % G != 0) return -1;
    if (io != IO_F32 && io != IO_BF16) return -1;
    const int64_t pairs = Bsz * H;
    if (pairs == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > pairs) nthreads = (int)pairs;
    ssdm_job* jobs = (ssdm_job*)calloc((size_t)nthreads, sizeof(ssdm_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int k = 0; k < nthreads; ++k) {
        ssdm_job* j = &jobs[k];
        j->Bsz = Bsz; j->L = L; j->H = H; j->P = P; j->N = N; j->G = G; j->R = R; j->io = io;
        j->x = x; j->delta = delta; j->lam = lam; j->Bm = Bm; j->Cm = Cm; j->z = z;
        j->x_prev = x_prev; j->B_prev = B_prev;
        j->A = A; j->Dv = Dv; j->h0 = h0;
        j->out = out; j->final_state = final_state;
        j->pair_begin = pairs * k / nthreads;
        j->pair_end = pairs * (k + 1) / nthreads;
    }
    for (int k = 1; k < nthreads; ++k) pthread_create(&th[k], NULL, ssdm_worker, &jobs[k]);
    ssdm_worker(&jobs[0]);
    for (int k = 1; k < nthreads; ++k) pthread_join(th[k], NULL);
    free(jobs);
    free(th);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Mamba-3 SISO with a complex-valued state (own loop, complex arithmetic)   */
/* ------------------------------------------------------------------------- */
/*
 * "Mamba-3" (blog), "El modelo Mamba-3" item 2: the state is tracked by a
 * complex-valued SSM; "Arquitectura": the complex transitions act as
 * rotations (RoPE), data-dependent ("Kernels por todas partes").  Plain
 * reading: state pairs (2k, 2k+1) are one complex number h_k, the transition
 * of head h is the complex scalar a_h + i omega[h,k] per pair, and zero-order
 * hold gives exp(d (a_h + i omega)) -- a decay times a rotation by d*omega,
 * data-dependent through d.  B and C pairs are complex numbers too; the
 * input rule is the exponential-trapezoidal one of oracle_ssd3_fwd with the
 * complex transition, and the readout takes the real part of conj(C_k) h_k
 * (the real dot product of the pairs).  omega = 0 is oracle_ssd3_fwd.
 */
typedef struct {
    int64_t Bsz, L, H, P, N, G;
    int io;
    const void *x, *delta, *lam, *Bm, *Cm, *z;
    const float *A, *omega, *Dv, *h0;
    const void *x_prev, *B_prev;
    double *out, *final_state;
    int64_t pair_begin, pair_end;
} ssdc_job;

static void ssdc_pair(const ssdc_job* j, int64_t b, int64_t hd, double complex* S, double complex* bx_prev) {
    const int64_t H = j->H, P = j->P, N = j->N, L = j->L, G = j->G, K = N / 2;
    const int64_t g = hd / (H / G);
    for (int64_t p = 0; p < P; ++p)
        for (int64_t k = 0; k < K; ++k) {
            const int64_t i = ((b * H + hd) * P + p) * N + 2 * k;
            S[p * K + k] = j->h0 ? (double)j->h0[i] + I * (double)j->h0[i + 1] : 0.0;
            bx_prev[p * K + k] = 0.0;
            if (j->x_prev && j->B_prev) {
                const double xp = load_io(j->x_prev, j->io, (b * H + hd) * P + p);
                const int64_t r = (b * G + g) * N + 2 * k;
                bx_prev[p * K + k] = (load_io(j->B_prev, j->io, r) + I * load_io(j->B_prev, j->io, r + 1)) * xp;
            }
        }
    for (int64_t t = 0; t < L; ++t) {
        const double d = load_io(j->delta, j->io, (b * L + t) * H + hd);
        const double lam = load_io(j->lam, j->io, (b * L + t) * H + hd);
        const int64_t r = ((b * L + t) * G + g) * N;
        for (int64_t p = 0; p < P; ++p) {
            const int64_t i = ((b * L + t) * H + hd) * P + p;
            const double u = load_io(j->x, j->io, i);
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double complex a = cexp(d * ((double)j->A[hd] + I * (double)j->omega[hd * K + k]));
                const double complex bk = load_io(j->Bm, j->io, r + 2 * k) + I * load_io(j->Bm, j->io, r + 2 * k + 1);
                const double complex ck = load_io(j->Cm, j->io, r + 2 * k) + I * load_io(j->Cm, j->io, r + 2 * k + 1);
                const double complex bx = bk * u;
                S[p * K + k] = a * S[p * K + k] + (1.0 - lam) * d * a * bx_prev[p * K + k] + lam * d * bx;
                bx_prev[p * K + k] = bx;
                acc += creal(conj(ck) * S[p * K + k]);
            }
            double y = acc + (j->Dv ? (double)j->Dv[hd] * u : 0.0);
            if (j->z) y *= silu(load_io(j->z, j->io, i));
            j->out[i] = y;
        }
    }
    if (j->final_state)
        for (int64_t p = 0; p < P; ++p)
            for (int64_t k = 0; k < K; ++k) {
                const int64_t i = ((b * H + hd) * P + p) * N + 2 * k;
                j->final_state[i] = creal(S[p * K + k]);
                j->final_state[i + 1] = cimag(S[p * K + k]);
            }
}

static void* ssdc_worker(void* arg) {
    const ssdc_job* j = (const ssdc_job*)arg;
    const int64_t n = j->P * (j->N / 2);
    double complex* S = (double complex*)malloc(sizeof(double complex) * (size_t)(2 * n));
    for (int64_t k = j->pair_begin; k < j->pair_end; ++k) ssdc_pair(j, k / j->H, k % j->H, S, S + n);
    free(S);
    return NULL;
}

/*
 * As oracle_ssd3_fwd, plus omega [H, N/2] fp32 (rotation rate of each state
 * pair) and the token before step 0, x_prev [Bsz, H, P] and B_prev
 * [Bsz, G, N] in io dtype (both nullable: no previous token).  N must be even.
 */
int oracle_ssdc_fwd(int64_t Bsz, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int io,
                    const void* x, const void* delta, const void* lam, const float* A, const float* omega,
                    const void* Bm, const void* Cm, const float* Dv, const void* z, const float* h0,
                    const void* x_prev, const void* B_prev, double* out, double* final_state, int nthreads) {
    if (Bsz < 0 || L < 0 || H <= 0 || P <= 0 || N <= 0 || N % 2 != 0 || G <= 0 || H % G != 0) return -1;
    if (io != IO_F32 && io != IO_BF16) return -1;
    const int64_t pairs = Bsz * H;
    if (pairs == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > pairs) nthreads = (int)pairs;
    ssdc_job* jobs = (ssdc_job*)calloc((size_t)nthreads, sizeof(ssdc_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int k = 0; k < nthreads; ++k) {
        ssdc_job* j = &jobs[k];
        j->Bsz = Bsz; j->L = L; j->H = H; j->P = P; j->N = N; j->G = G; j->io = io;
        j->x = x; j->delta = delta; j->lam = lam; j->Bm = Bm; j->Cm = Cm; j->z = z;
        j->A = A; j->omega = omega; j->Dv = Dv; j->h0 = h0; j->x_prev = x_prev; j->B_prev = B_prev;
        j->out = out; j->final_state = final_state;
        j->pair_begin = pairs * k / nthreads;
        j->pair_end = pairs * (k + 1) / nthreads;
    }
    for (int k = 1; k < nthreads; ++k) pthread_create(&th[k], NULL, ssdc_worker, &jobs[k]);
    ssdc_worker(&jobs[0]);
    for (int k = 1; k < nthreads; ++k) pthread_join(th[k], NULL);
    free(jobs);
    free(th);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Mamba-1 selective scan: gradients (reverse mode through the same loop)    */
/* ------------------------------------------------------------------------- */
/*
 * The derivative of the forward definition above, taken step by step in
 * reverse time ("P20 - Mamba", 5: the selective recurrence; training needs
 * its gradients, which the pages discuss only as the cost of the method).
 * With a_t[n] = exp(delta_t A[n]), h_t = a_t h_{t-1} + delta_t B_t x_t,
 * y_t = C_t . h_t + D x_t and out_t = y_t silu(z_t), for an upstream gradient
 * g_t = dLoss/dout_t and dLoss/dfinal_state:
 *   dy_t          = g_t silu(z_t),  dz_t = g_t y_t silu'(z_t)
 *   lam_t         = C_t dy_t + a_{t+1} lam_{t+1}       (adjoint of h_t; lam_L = dfinal)
 *   dC_t[n]      += dy_t h_t[n]        (summed over channels)
 *   dB_t[n]      += lam_t[n] delta_t x_t   (summed over channels)
 *   ddelta_t      = sum_n lam_t[n] (h_{t-1}[n] a_t[n] A[n] + B_t[n] x_t)
 *   dx_t          = D dy_t + sum_n lam_t[n] delta_t B_t[n]
 *   dA[n]        += lam_t[n] h_{t-1}[n] a_t[n] delta_t   (summed over batch and time)
 *   dD           += dy_t x_t                             (summed over batch and time)
 *   dh0[n]        = a_0[n] lam_0[n]
 * Plain, sequential, fp64; every forward state of a row is kept (no
 * recomputation), rows of one batch entry are walked in turn by one thread.
 */
typedef struct {
    int64_t Bsz, L, D, N;
    int io;
    const void *x, *delta, *Bm, *Cm, *z, *dout;
    const float *A, *Dv, *h0, *dfinal;
    double *dx, *ddelta, *dA, *dB, *dC, *dD, *dz, *dh0;   /* dA, dD: this thread's partial sums */
    int64_t b_begin, b_end;
} bwd_job;

static double dsilu(double v) {
    const double s = 1.0 / (1.0 + exp(-v));
    return s * (1.0 + v * (1.0 - s));
}

static void* bwd_worker(void* arg) {
    const bwd_job* j = (const bwd_job*)arg;
    const int64_t N = j->N, D = j->D, L = j->L;
    double* hs = (double*)malloc(sizeof(double) * (size_t)((L + 1) * N));   /* h_{-1..L-1} */
    double* ys = (double*)malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    double* lam = (double*)malloc(sizeof(double) * (size_t)N);
    for (int64_t b = j->b_begin; b < j->b_end; ++b) {
        for (int64_t c = 0; c < D; ++c) {
            /* forward, keeping every state: hs[(t + 1) * N + n] = h_t[n] */
            for (int64_t n = 0; n < N; ++n) hs[n] = j->h0 ? (double)j->h0[(b * D + c) * N + n] : 0.0;
            for (int64_t t = 0; t < L; ++t) {
                const int64_t i = (b * L + t) * D + c, r = (b * L + t) * N;
                const double d = load_io(j->delta, j->io, i), u = load_io(j->x, j->io, i);
                double acc = 0.0;
                for (int64_t n = 0; n < N; ++n) {
                    const double h = exp(d * (double)j->A[c * N + n]) * hs[t * N + n] +
                                     d * load_io(j->Bm, j->io, r + n) * u;
                    hs[(t + 1) * N + n] = h;
                    acc += load_io(j->Cm, j->io, r + n) * h;
                }
                ys[t] = acc + (j->Dv ? (double)j->Dv[c] * u : 0.0);
            }
            /* reverse */
            for (int64_t n = 0; n < N; ++n) lam[n] = j->dfinal ? (double)j->dfinal[(b * D + c) * N + n] : 0.0;
            for (int64_t t = L - 1; t >= 0; --t) {
                const int64_t i = (b * L + t) * D + c, r = (b * L + t) * N;
                const double d = load_io(j->delta, j->io, i), u = load_io(j->x, j->io, i);
                const double g = load_io(j->dout, j->io, i);
                double dy = g;
                if (j->z) {
                    const double zz = load_io(j->z, j->io, i);
                    dy = g * silu(zz);
                    j->dz[i] = g * ys[t] * dsilu(zz);
                }
                double du = 0.0, dd = 0.0;
                if (j->Dv) {
                    du = dy * (double)j->Dv[c];
                    j->dD[c] += dy * u;
                }
                for (int64_t n = 0; n < N; ++n) {
                    const double An = (double)j->A[c * N + n];
                    const double a = exp(d * An);
                    const double Bn = load_io(j->Bm, j->io, r + n), Cn = load_io(j->Cm, j->io, r + n);
                    const double h = hs[(t + 1) * N + n], hprev = hs[t * N + n];
                    lam[n] += Cn * dy;                         /* adjoint of h_t */
                    j->dC[r + n] += dy * h;
                    j->dB[r + n] += lam[n] * d * u;
                    dd += lam[n] * (hprev * a * An + Bn * u);
                    du += lam[n] * d * Bn;
                    j->dA[c * N + n] += lam[n] * hprev * a * d;
                    lam[n] *= a;                               /* adjoint of h_{t-1} */
                }
                j->ddelta[i] = dd;
                j->dx[i] = du;
            }
            for (int64_t n = 0; n < N; ++n) j->dh0[(b * D + c) * N + n] = lam[n];
        }
    }
    free(hs);
    free(ys);
    free(lam);
    return NULL;
}

/*
 * Gradients of the selective scan for upstream gradients dout [Bsz, L, D] (io
 * dtype) and dfinal [Bsz, D, N] fp32 (nullable).  Outputs fp64: dx, ddelta,
 * dz [Bsz, L, D]; dB, dC [Bsz, L, N]; dA [D, N]; dD [D]; dh0 [Bsz, D, N]
 * (dz and dD are written only when z and Dv are given).  Returns 0, or -1 on
 * bad sizes.
 */
int oracle_scan_bwd(int64_t Bsz, int64_t L, int64_t D, int64_t N, int io,
                    const void* x, const void* delta, const float* A, const void* Bm, const void* Cm,
                    const float* Dv, const void* z, const float* h0, const void* dout, const float* dfinal,
                    double* dx, double* ddelta, double* dA, double* dB, double* dC, double* dD, double* dz,
                    double* dh0, int nthreads) {
    if (Bsz < 0 || L < 0 || D <= 0 || N <= 0) return -1;
    if (io != IO_F32 && io != IO_BF16) return -1;
    memset(dA, 0, sizeof(double) * (size_t)(D * N));
    if (dD) memset(dD, 0, sizeof(double) * (size_t)D);
    memset(dB, 0, sizeof(double) * (size_t)(Bsz * L * N));
    memset(dC, 0, sizeof(double) * (size_t)(Bsz * L * N));
    if (Bsz == 0) return 0;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > Bsz) nthreads = (int)Bsz;
    bwd_job* jobs = (bwd_job*)calloc((size_t)nthreads, sizeof(bwd_job));
    pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int k = 0; k < nthreads; ++k) {
        bwd_job* j = &jobs[k];
        j->Bsz = Bsz; j->L = L; j->D = D; j->N = N; j->io = io;
        j->x = x; j->delta = delta; j->Bm = Bm; j->Cm = Cm; j->z = z; j->dout = dout;
        j->A = A; j->Dv = Dv; j->h0 = h0; j->dfinal = dfinal;
        j->dx = dx; j->ddelta = ddelta; j->dB = dB; j->dC = dC; j->dz = dz; j->dh0 = dh0;
        j->dA = (double*)calloc((size_t)(D * N), sizeof(double));
        j->dD = (double*)calloc((size_t)D, sizeof(double));
        j->b_begin = Bsz * k / nthreads;
        j->b_end = Bsz * (k + 1) / nthreads;
    }
    for (int k = 1; k < nthreads; ++k) pthread_create(&th[k], NULL, bwd_worker, &jobs[k]);
    bwd_worker(&jobs[0]);
    for (int k = 1; k < nthreads; ++k) pthread_join(th[k], NULL);
    for (int k = 0; k < nthreads; ++k) {
        for (int64_t e = 0; e < D * N; ++e) dA[e] += jobs[k].dA[e];
        if (dD)
            for (int64_t e = 0; e < D; ++e) dD[e] += jobs[k].dD[e];
        free(jobs[k].dA);
        free(jobs[k].dD);
    }
    free(jobs);
    free(th);
    return 0;
}
