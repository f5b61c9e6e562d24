/*
 * ssu_ref.c -- CPU oracle for the Mamba2 decode-step selective_state_update.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline
 * leg use it. It shares no code with the GPU library.
 *
 * What it computes (plain fp64 from the exact stored input values; bf16 and
 * fp32 inputs convert to fp64 exactly):
 *
 *   The decode step of a Mamba2 layer advances each request's SSM state by one
 *   token. sglang PR #41223 ("[Perf] Mamba2 selective_state_update up to 2x
 *   faster on B200 ...", section "Summary") states that each step reads and
 *   writes every request's fp32 state; its section "Kernel measurement" names
 *   the operands: a state pool [pool, H, 64, 128] fp32 addressed by
 *   state_batch_indices, x [bs, H, P], B and C [bs, G, N], and dt, A, D,
 *   dt_bias broadcast per head. The pages print no formula; the update taken
 *   here is the standard one-token step of the selective-scan recurrence, the
 *   same recurrence whose exact order the COREY page's patched live scan kernel
 *   keeps while it varies the chunk size (COREY: Entropy-Guided Runtime Chunk
 *   Scheduling for Selective Scan Kernels, Table 5):
 *
 *     u      = dt[b,h] + dt_bias[h]                    (dt_bias = 0 if absent)
 *     delta  = softplus(u) if softplus is on, else u
 *     a      = exp(A[h] * delta)
 *     S'[p,n] = S[idx[b],h,p,n] * a + (delta * x[b,h,p]) * B[b,g(h),n]
 *     y[p]   = sum_n S'[p,n] * C[b,g(h),n] + D[h] * x[b,h,p]   (D = 0 if absent)
 *     out[p] = bf16_RNE(fp32_RNE(y[p]))
 *     pool[idx[b],h,p,n] = fp32_RNE(S'[p,n])
 *
 *   with g(h) = floor(h * G / H) (contiguous blocks of H/G heads per group),
 *   the output using the updated state, and the sum over n taken in order
 *   n = 0, 1, ..., N-1.
 *
 *   ssu_ref_run with nsteps = K > 1 carries S' in fp64 from one token to the
 *   next (the sequential length-K scan of the same recurrence) and writes the
 *   pool once, after the last token.
 *
 * Slot indices outside [0, pool_slots) are skipped: that request's state is
 * neither read nor written and its out rows are left untouched (the library's
 * documented behaviour for padding entries). Duplicate in-range indices are an
 * error (status 3): the step is then not a function of its inputs.
 *
 * Parity pins: every part above is pinned by tests against closed forms,
 * library routines (numpy outer product / matrix-vector product, torch's bf16
 * rounding), invariants and an independent Python brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct ssu_ref_args {
    /* problem shape */
    int32_t batch, nheads, headdim, dstate, ngroups, dt_softplus, nsteps, nthreads;
    int64_t pool_slots;
    /* state pool [pool_slots, H, P, N] fp32, n contiguous; updated in place */
    float *state;
    int64_t st_slot, st_head, st_row;
    /* state_batch_indices [batch] */
    const int32_t *idx;
    /* x [nsteps, batch, H, P] bf16 bits */
    const uint16_t *x;
    int64_t x_t, x_b, x_h, x_p;
    /* B, C [nsteps, batch, G, N] bf16 bits */
    const uint16_t *B;
    int64_t B_t, B_b, B_g, B_n;
    const uint16_t *C;
    int64_t C_t, C_b, C_g, C_n;
    /* dt [nsteps, batch, H] bf16 bits, one value per (request, head) */
    const uint16_t *dt;
    int64_t dt_t, dt_b, dt_h;
    /* per-head fp32 parameters; dt_bias and D may be NULL */
    const float *dt_bias;
    int64_t dt_bias_h;
    const float *A;
    int64_t A_h;
    const float *D;
    int64_t D_h;
    /* out [nsteps, batch, H, P] bf16 bits */
    uint16_t *out;
    int64_t out_t, out_b, out_h, out_p;
    /* optional fp64 outputs, contiguous:
     *   state_ref [batch, H, P, N] : S' after the last token
     *   y_ref     [nsteps, batch, H, P] : y before rounding
     *   tau_ref   [nsteps, batch, H, P] : sum_n |S'[p,n] C[n]| + |D x[p]| */
    double *state_ref, *y_ref, *tau_ref;
} ssu_ref_args;

/* bf16 bit pattern -> value (exact). */
static double ref_bf16_value(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* fp32 -> bf16 bit pattern, round to nearest, ties to even. NaN stays NaN
 * (quiet, sign kept); infinities and overflow to infinity follow from the
 * rounding of the bit pattern. */
uint16_t ssu_ref_bf16_rne(float f)
{
    uint32_t w;
    memcpy(&w, &f, sizeof w);
    if ((w & 0x7F800000u) == 0x7F800000u && (w & 0x007FFFFFu) != 0)
        return (uint16_t)((w >> 16) | 0x0040u);
    uint32_t lsb = (w >> 16) & 1u;
    w += 0x7FFFu + lsb;
    return (uint16_t)(w >> 16);
}

/* softplus(u) = log(1 + e^u), in the form max(u,0) + log1p(e^-|u|), which is
 * exact algebra and never overflows. */
double ssu_ref_softplus(double u)
{
    return fmax(u, 0.0) + log1p(exp(-fabs(u)));
}

/* Per-(request, head) discretisation: delta and the decay a = exp(A * delta). */
void ssu_ref_discretize(double dt, double dt_bias, double A, int32_t softplus,
                        double *delta, double *a)
{
    double u = dt + dt_bias;
    double d = softplus ? ssu_ref_softplus(u) : u;
    *delta = d;
    *a = exp(A * d);
}

int32_t ssu_ref_abi_version(void) { return 1; }

/* Returns 0 on success; 1 bad shape; 2 null pointer; 3 duplicate slot index. */
int32_t ssu_ref_run(const ssu_ref_args *g)
{
    const int32_t bs = g->batch, H = g->nheads, P = g->headdim, N = g->dstate, G = g->ngroups;
    const int32_t K = g->nsteps;
    if (bs < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0 || K <= 0 || g->pool_slots < 0)
        return 1;
    if (bs == 0)
        return 0;
    if (!g->state || !g->idx || !g->x || !g->B || !g->C || !g->dt || !g->A || !g->out)
        return 2;

    /* distinctness of the in-range slot indices */
    unsigned char *seen = (unsigned char *)calloc((size_t)(g->pool_slots > 0 ? g->pool_slots : 1), 1);
    if (!seen)
        return 2;
    for (int32_t b = 0; b < bs; ++b) {
        int64_t s = g->idx[b];
        if (s < 0 || s >= g->pool_slots)
            continue;
        if (seen[s]) {
            free(seen);
            return 3;
        }
        seen[s] = 1;
    }
    free(seen);

#ifdef _OPENMP
    int nthreads = g->nthreads > 0 ? g->nthreads : omp_get_max_threads();
#endif

#ifdef _OPENMP
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *S = (double *)malloc(sizeof(double) * (size_t)P * (size_t)N);
        if (!S)
            abort();
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t bh = 0; bh < (int64_t)bs * H; ++bh) {
            const int32_t b = (int32_t)(bh / H), h = (int32_t)(bh % H);
            const int64_t slot = g->idx[b];
            if (slot < 0 || slot >= g->pool_slots)
                continue;                       /* padding entry: skipped */
            const int32_t grp = (int32_t)(((int64_t)h * G) / H);
            float *pool = g->state + slot * g->st_slot + (int64_t)h * g->st_head;

            /* gather: S = pool[slot, h] */
            for (int32_t p = 0; p < P; ++p)
                for (int32_t n = 0; n < N; ++n)
                    S[(int64_t)p * N + n] = (double)pool[(int64_t)p * g->st_row + n];

            for (int32_t t = 0; t < K; ++t) {
                const double dtv = ref_bf16_value(g->dt[t * g->dt_t + b * g->dt_b + h * g->dt_h]);
                const double bias = g->dt_bias ? (double)g->dt_bias[h * g->dt_bias_h] : 0.0;
                const double Av = (double)g->A[h * g->A_h];
                const double Dv = g->D ? (double)g->D[h * g->D_h] : 0.0;
                double delta, a;
                ssu_ref_discretize(dtv, bias, Av, g->dt_softplus, &delta, &a);

                const uint16_t *xr = g->x + t * g->x_t + b * g->x_b + h * g->x_h;
                const uint16_t *Br = g->B + t * g->B_t + b * g->B_b + grp * g->B_g;
                const uint16_t *Cr = g->C + t * g->C_t + b * g->C_b + grp * g->C_g;

                for (int32_t p = 0; p < P; ++p) {
                    const double xp = ref_bf16_value(xr[p * g->x_p]);
                    double *Sp = S + (int64_t)p * N;
                    /* state update: S' = S * a + (delta * x[p]) * B[n] */
                    for (int32_t n = 0; n < N; ++n)
                        Sp[n] = Sp[n] * a + (delta * xp) * ref_bf16_value(Br[n * g->B_n]);
                    /* output: y = sum_n S'[p,n] C[n] + D x[p], n in order */
                    double y = 0.0, tau = 0.0;
                    for (int32_t n = 0; n < N; ++n) {
                        const double term = Sp[n] * ref_bf16_value(Cr[n * g->C_n]);
                        y += term;
                        tau += fabs(term);
                    }
                    y += Dv * xp;
                    tau += fabs(Dv * xp);

                    const int64_t oi = t * g->out_t + b * g->out_b + h * g->out_h + p * g->out_p;
                    g->out[oi] = ssu_ref_bf16_rne((float)y);
                    const int64_t ri = (((int64_t)t * bs + b) * H + h) * P + p;
                    if (g->y_ref)
                        g->y_ref[ri] = y;
                    if (g->tau_ref)
                        g->tau_ref[ri] = tau;
                }
            }

            /* write back: pool = fp32(S'), and the fp64 S' on request */
            for (int32_t p = 0; p < P; ++p)
                for (int32_t n = 0; n < N; ++n) {
                    const double v = S[(int64_t)p * N + n];
                    pool[(int64_t)p * g->st_row + n] = (float)v;
                    if (g->state_ref)
                        g->state_ref[(((int64_t)b * H + h) * P + p) * N + n] = v;
                }
        }
        free(S);
    }
    return 0;
}

/* Number of threads an ssu_ref_run call with nthreads = 0 would use. */
int32_t ssu_ref_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Block copy for prefix caching / multi-token prediction (vLLM PR #48110,
 * "[Perf][Hybrid] Vectorize _copy_mamba_state_block to uint64 for temporal",
 * section "Purpose"): for every request r and every state tensor k, the block
 * src[r] of tensor k is copied to block dst[r] of tensor k. A tensor's block
 * i occupies bytes [base + i * block_stride, base + i * block_stride +
 * block_bytes). Block ids outside [0, nblocks) skip that request (the same
 * padding rule as the decode step); src == dst is a no-op. Destinations must
 * be distinct and must not be any request's source (status 3 otherwise): the
 * result would then depend on the order of the copies.
 */
typedef struct ssu_ref_block_tensor {
    unsigned char *base;
    int64_t block_stride, block_bytes, nblocks;
} ssu_ref_block_tensor;

int32_t ssu_ref_copy_blocks(const ssu_ref_block_tensor *t, int32_t ntensors, const int32_t *src,
                            const int32_t *dst, int32_t nreqs)
{
    if (ntensors < 0 || nreqs < 0)
        return 1;
    if (nreqs == 0 || ntensors == 0)
        return 0;
    if (!t || !src || !dst)
        return 2;
    for (int32_t k = 0; k < ntensors; ++k)
        if (!t[k].base || t[k].block_bytes < 0 || t[k].nblocks < 0)
            return 1;
    /* destinations distinct and never a source (per tensor, same ids) */
    for (int32_t r = 0; r < nreqs; ++r) {
        if (src[r] == dst[r])
            continue;
        for (int32_t q = 0; q < nreqs; ++q) {
            if (q != r && dst[q] == dst[r] && src[q] != dst[q])
                return 3;
            if (src[q] == dst[r] && src[q] != dst[q])
                return 3;
        }
    }
    for (int32_t r = 0; r < nreqs; ++r)
        for (int32_t k = 0; k < ntensors; ++k) {
            const int64_t s = src[r], d = dst[r];
            if (s < 0 || s >= t[k].nblocks || d < 0 || d >= t[k].nblocks || s == d)
                continue;
            memcpy(t[k].base + d * t[k].block_stride, t[k].base + s * t[k].block_stride,
                   (size_t)t[k].block_bytes);
        }
    return 0;
}

/*
 * Selective scan over a sequence, for prefill (COREY: Entropy-Guided Runtime
 * Chunk Scheduling for Selective Scan Kernels, Table 9, Table 17 and Table 18:
 * selective_scan_fn over dim channels with d_state states each, FP16 or BF16
 * activations, the sequence cut into static chunks of tokens with one kernel
 * call per chunk and the state carried from one chunk to the next; Table 5
 * calls such a kernel recurrence-preserving). The page prints no formula; the
 * scan taken here is the standard Mamba selective scan, the length-L form of
 * the decode step above with a decay rate per (channel, state):
 *
 *   for every request b, channel d and token t = 0, 1, ..., L-1 in order:
 *     v       = delta[b,d,t] + delta_bias[d]            (delta_bias = 0 if absent)
 *     Delta   = softplus(v) if softplus is on, else v
 *     a[n]    = exp(A[d,n] * Delta)
 *     h[n]    = h[n] * a[n] + (Delta * u[b,d,t]) * B[b,g(d),n,t]
 *     y[t]    = sum_n h[n] * C[b,g(d),n,t] + D[d] * u[b,d,t]   (D = 0 if absent)
 *     out[t]  = io_RNE(fp32_RNE(y[t]))
 *   state[b,d,n] = fp32_RNE(h[n] after the last token)
 *
 * with h read from state[b,d,:] before the first token, g(d) = floor(d * G /
 * dim) (contiguous blocks of dim/G channels per group) and the sum over n in
 * order. Cutting the sequence into chunks and carrying h between them gives
 * the same recurrence, so the oracle is the unchunked scan.
 *
 * Error scales for the acceptance test (not part of the scan; ssu_ref_scan
 * returns them on request). With beta = (Delta u) B, per (b, d, n):
 *   M_t = a_t M_{t-1} + |beta_t|                        (bounds |h_t|)
 *   E_t = a_t E_{t-1} + (1 + |A Delta_t|) a_t M_{t-1} + M_t
 * from M_{-1} = E_{-1} = |h before the first token|. E_t grows by every
 * magnitude that a rounding step of fp32 arithmetic on this recurrence can
 * touch (the decay, whose relative error grows with its argument, applied to
 * the carried state, and the new state) and carries the older ones with the
 * decay, so fp32 rounding errors in h_t stay within a small multiple of
 * 2^-24 E_t in any association of the scan.
 */
typedef struct ssu_ref_scan_args {
    int32_t batch, dim, dstate, ngroups, delta_softplus, io_dtype, nthreads, reserved;
    int64_t seqlen;
    /* state [batch, dim, dstate] fp32, n contiguous; read, then overwritten */
    float *state;
    int64_t st_b, st_d;
    /* u, delta [batch, dim, L]; B, C [batch, G, dstate, L]: io_dtype bits
     * (0 = bf16, 1 = fp16) */
    const uint16_t *u;
    int64_t u_b, u_d, u_t;
    const uint16_t *delta;
    int64_t dl_b, dl_d, dl_t;
    const uint16_t *B;
    int64_t B_b, B_g, B_n, B_t;
    const uint16_t *C;
    int64_t C_b, C_g, C_n, C_t;
    /* A [dim, dstate] fp32; D, delta_bias [dim] fp32 contiguous, may be NULL */
    const float *A;
    int64_t A_d, A_n;
    const float *D, *delta_bias;
    /* out [batch, dim, L] io_dtype bits */
    uint16_t *out;
    int64_t o_b, o_d, o_t;
    /* optional fp64 outputs, contiguous:
     *   state_ref [batch, dim, dstate] : h after the last token
     *   err_ref   [batch, dim, dstate] : E after the last token
     *   y_ref     [batch, dim, L]      : y before rounding
     *   tau_ref   [batch, dim, L]      : sum_n |h[n] C[n]| + |D u|
     *   rho_ref   [batch, dim, L]      : sum_n |C[n]| E[n] */
    double *state_ref, *err_ref, *y_ref, *tau_ref, *rho_ref;
} ssu_ref_scan_args;

/* IEEE binary16 bit pattern -> value (exact): 1 sign bit, 5 exponent bits with
 * bias 15, 10 fraction bits; exponent 0 holds the subnormals m * 2^-24. */
double ssu_ref_f16_value(uint16_t bits)
{
    const int e = (bits >> 10) & 0x1F, m = bits & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m | 0x400), e - 25);
    return (bits & 0x8000u) ? -v : v;
}

/* fp32 -> binary16 bit pattern, round to nearest, ties to even (from the
 * definition: scale to an integer significand in double, where it is exact,
 * and round with rint in the default rounding mode). */
uint16_t ssu_ref_f16_rne(float f)
{
    const uint16_t sign = signbit(f) ? 0x8000u : 0u;
    const double a = fabs((double)f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7E00u);
    if (isinf(f))
        return (uint16_t)(sign | 0x7C00u);
    if (a < ldexp(1.0, -14))                     /* subnormal range */
        return (uint16_t)(sign | (uint16_t)rint(ldexp(a, 24)));
    int ex;
    frexp(a, &ex);                               /* a = fr 2^ex, fr in [0.5, 1) */
    int E = ex - 1;                              /* a in [2^E, 2^(E+1)) */
    double r = rint(ldexp(a, 10 - E));           /* in [1024, 2048] */
    if (r == 2048.0) {
        r = 1024.0;
        E += 1;
    }
    if (E + 15 >= 31)
        return (uint16_t)(sign | 0x7C00u);       /* overflow: infinity */
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)(r - 1024.0));
}

static double ref_io_value(uint16_t bits, int32_t io_dtype)
{
    return io_dtype ? ssu_ref_f16_value(bits) : ref_bf16_value(bits);
}

/* Returns 0 on success; 1 bad shape; 2 null pointer. */
int32_t ssu_ref_scan(const ssu_ref_scan_args *g)
{
    const int32_t bs = g->batch, Dm = g->dim, N = g->dstate, G = g->ngroups, io = g->io_dtype;
    const int64_t L = g->seqlen;
    if (bs < 0 || Dm <= 0 || N <= 0 || G <= 0 || Dm % G != 0 || L < 0 || (io != 0 && io != 1))
        return 1;
    if (bs == 0)
        return 0;
    if (!g->state || !g->A || (L > 0 && (!g->u || !g->delta || !g->B || !g->C || !g->out)))
        return 2;

#ifdef _OPENMP
    int nthreads = g->nthreads > 0 ? g->nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
#endif
    {
        double *h = (double *)malloc(sizeof(double) * 3 * (size_t)N);
        if (!h)
            abort();
        double *M = h + N, *E = h + 2 * N;
#ifdef _OPENMP
#pragma omp for schedule(static)
#endif
        for (int64_t bd = 0; bd < (int64_t)bs * Dm; ++bd) {
            const int32_t b = (int32_t)(bd / Dm), d = (int32_t)(bd % Dm);
            const int32_t grp = (int32_t)(((int64_t)d * G) / Dm);
            float *st = g->state + b * g->st_b + d * g->st_d;
            for (int32_t n = 0; n < N; ++n) {
                h[n] = (double)st[n];
                M[n] = E[n] = fabs(h[n]);
            }
            const double bias = g->delta_bias ? (double)g->delta_bias[d] : 0.0;
            const double Dv = g->D ? (double)g->D[d] : 0.0;
            const float *Ar = g->A + d * g->A_d;

            for (int64_t t = 0; t < L; ++t) {
                const double v = ref_io_value(g->delta[b * g->dl_b + d * g->dl_d + t * g->dl_t], io) + bias;
                const double Delta = g->delta_softplus ? ssu_ref_softplus(v) : v;
                const double ut = ref_io_value(g->u[b * g->u_b + d * g->u_d + t * g->u_t], io);
                const uint16_t *Bt = g->B + b * g->B_b + grp * g->B_g + t * g->B_t;
                const uint16_t *Ct = g->C + b * g->C_b + grp * g->C_g + t * g->C_t;
                double y = 0.0, tau = 0.0, rho = 0.0;
                for (int32_t n = 0; n < N; ++n) {
                    const double An = (double)Ar[n * g->A_n];
                    const double a = exp(An * Delta);
                    const double beta = (Delta * ut) * ref_io_value(Bt[n * g->B_n], io);
                    h[n] = h[n] * a + beta;
                    const double Mprev = M[n];
                    M[n] = a * M[n] + fabs(beta);
                    E[n] = a * E[n] + (1.0 + fabs(An * Delta)) * a * Mprev + M[n];
                    const double c = ref_io_value(Ct[n * g->C_n], io);
                    y += h[n] * c;
                    tau += fabs(h[n] * c);
                    rho += fabs(c) * E[n];
                }
                y += Dv * ut;
                tau += fabs(Dv * ut);
                const float yf = (float)y;
                g->out[b * g->o_b + d * g->o_d + t * g->o_t] = io ? ssu_ref_f16_rne(yf) : ssu_ref_bf16_rne(yf);
                const int64_t ri = ((int64_t)b * Dm + d) * L + t;
                if (g->y_ref)
                    g->y_ref[ri] = y;
                if (g->tau_ref)
                    g->tau_ref[ri] = tau;
                if (g->rho_ref)
                    g->rho_ref[ri] = rho;
            }

            for (int32_t n = 0; n < N; ++n) {
                st[n] = (float)h[n];
                const int64_t si = ((int64_t)b * Dm + d) * N + n;
                if (g->state_ref)
                    g->state_ref[si] = h[n];
                if (g->err_ref)
                    g->err_ref[si] = E[n];
            }
        }
        free(h);
    }
    return 0;
}
