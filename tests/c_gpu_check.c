/* libssu's kernels called from plain C: no Python and no torch, so the HIP
 * runtime is the system ROCm's. A decode step and a two-chunk scan run on
 * hipMalloc'd buffers and are checked against the CPU oracle, compiled into
 * this program from oracle/ssu_ref.c, under the same acceptance rules as the
 * Python parity tests; a 3-token call must equal three one-token calls
 * bitwise, and a block copy must move exactly the named blocks. Prints "ok"
 * and returns 0 when everything passes; any HIP or libssu error is printed and
 * returns 1.
 *
 * Built by __graft_entry__.build() (gcc, next to this file); run by
 * tests/test_c_gpu.py on a GPU. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ssu.h"

#include "../oracle/ssu_ref.c"

#define HIP_OK(x)                                                              \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(1);                                                           \
        }                                                                      \
    } while (0)
#define SSU_OK_(x)                                                             \
    do {                                                                       \
        ssu_status s_ = (x);                                                   \
        if (s_ != SSU_OK) {                                                    \
            printf("%s at line %d: %s\n", ssu_status_string(s_), __LINE__,    \
                   ssu_last_error());                                          \
            exit(1);                                                           \
        }                                                                      \
    } while (0)

/* inputs: xorshift64 bit patterns, values of magnitude 0.25 .. 4 */
static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next(void)
{
    rng ^= rng << 13, rng ^= rng >> 7, rng ^= rng << 17;
    return rng;
}
static uint16_t rand_bf16(void) /* sign, exponent 125..128, 7 fraction bits */
{
    uint64_t r = next();
    return (uint16_t)(((r & 1) << 15) | ((125 + ((r >> 1) & 3)) << 7) | ((r >> 3) & 0x7F));
}
static uint16_t rand_f16(void) /* sign, exponent 13..16, 10 fraction bits */
{
    uint64_t r = next();
    return (uint16_t)(((r & 1) << 15) | ((13 + ((r >> 1) & 3)) << 10) | ((r >> 3) & 0x3FF));
}
static float rand_unit(void) { return (float)((next() >> 11) * (1.0 / 9007199254740992.0)); }

static void *to_device(const void *host, size_t bytes)
{
    void *d = NULL;
    HIP_OK(hipMalloc(&d, bytes));
    HIP_OK(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}

static double bf16_value(uint16_t b)
{
    uint32_t w = (uint32_t)b << 16;
    float f;
    memcpy(&f, &w, 4);
    return f;
}
static int64_t bf16_ordered(uint16_t b) { return (b & 0x8000) ? -(int64_t)(b & 0x7FFF) : (int64_t)(b & 0x7FFF); }
static double ulp_at(double a, int frac_bits, int min_exp)
{
    int e = a > 0 ? (int)floor(log2(a)) : min_exp;
    if (e < min_exp)
        e = min_exp;
    return ldexp(1.0, e - frac_bits);
}

static int check_decode(void)
{
    enum { H = 2, P = 64, N = 128, G = 1, BS = 3, SLOTS = 5, ROW = H * P + 2 * G * N };
    const int32_t idx[BS] = {4, 1, 2};
    static float pool[SLOTS * H * P * N], pool_gpu[SLOTS * H * P * N];
    static uint16_t xbc[BS * ROW], dt[BS * H], out[BS * H * P], out_ref[BS * H * P];
    float A[H], D[H], bias[H];
    for (int i = 0; i < SLOTS * H * P * N; ++i)
        pool[i] = 2.0f * rand_unit() - 1.0f;
    for (int i = 0; i < BS * ROW; ++i)
        xbc[i] = rand_bf16();
    for (int i = 0; i < BS * H; ++i)
        dt[i] = rand_bf16();
    for (int h = 0; h < H; ++h)
        A[h] = -(0.5f + rand_unit()), D[h] = rand_unit(), bias[h] = -2.0f * rand_unit();

    float *d_pool = to_device(pool, sizeof pool);
    void *d_idx = to_device(idx, sizeof idx), *d_xbc = to_device(xbc, sizeof xbc), *d_dt = to_device(dt, sizeof dt);
    void *d_A = to_device(A, sizeof A), *d_D = to_device(D, sizeof D), *d_bias = to_device(bias, sizeof bias);
    void *d_out = NULL;
    HIP_OK(hipMalloc(&d_out, sizeof out));

    ssu_config cfg = {H, P, N, G, 1, -1, -1, 0};
    ssu_handle *h = NULL;
    SSU_OK_(ssu_create(&cfg, &h));
    ssu_args a;
    memset(&a, 0, sizeof a);
    a.batch = BS, a.pool_slots = SLOTS;
    a.state = (ssu_view){d_pool, SSU_F32, 0, {H * P * N, P * N, N, 1}};
    a.idx = (ssu_view){d_idx, SSU_I32, 0, {1, 0, 0, 0}};
    a.x = (ssu_view){d_xbc, SSU_BF16, 0, {ROW, P, 1, 0}};
    a.B = (ssu_view){(uint16_t *)d_xbc + H * P, SSU_BF16, 0, {ROW, N, 1, 0}};
    a.C = (ssu_view){(uint16_t *)d_xbc + H * P + G * N, SSU_BF16, 0, {ROW, N, 1, 0}};
    a.dt = (ssu_view){d_dt, SSU_BF16, 0, {H, 1, 0, 0}};
    a.dt_bias = (ssu_view){d_bias, SSU_F32, 0, {1, 0, 0, 0}};
    a.A = (ssu_view){d_A, SSU_F32, 0, {1, 0, 0, 0}};
    a.D = (ssu_view){d_D, SSU_F32, 0, {1, 0, 0, 0}};
    a.out = (ssu_view){d_out, SSU_BF16, 0, {H * P, P, 1, 0}};
    SSU_OK_(ssu_check_indices(&a, NULL));
    SSU_OK_(ssu_update(h, &a, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(pool_gpu, d_pool, sizeof pool, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
    ssu_destroy(h);

    static double state_ref[BS * H * P * N], y_ref[BS * H * P], tau_ref[BS * H * P];
    ssu_ref_args g;
    memset(&g, 0, sizeof g);
    g.batch = BS, g.nheads = H, g.headdim = P, g.dstate = N, g.ngroups = G, g.dt_softplus = 1, g.nsteps = 1;
    g.nthreads = 1, g.pool_slots = SLOTS;
    g.state = pool, g.st_slot = H * P * N, g.st_head = P * N, g.st_row = N;
    g.idx = idx;
    g.x = xbc, g.x_b = ROW, g.x_h = P, g.x_p = 1;
    g.B = xbc + H * P, g.B_b = ROW, g.B_g = N, g.B_n = 1;
    g.C = xbc + H * P + G * N, g.C_b = ROW, g.C_g = N, g.C_n = 1;
    g.dt = dt, g.dt_b = H, g.dt_h = 1;
    g.dt_bias = bias, g.dt_bias_h = 1, g.A = A, g.A_h = 1, g.D = D, g.D_h = 1;
    g.out = out_ref, g.out_b = H * P, g.out_h = P, g.out_p = 1;
    g.state_ref = state_ref, g.y_ref = y_ref, g.tau_ref = tau_ref;
    if (ssu_ref_run(&g) != 0) {
        printf("oracle failed\n");
        return 1;
    }

    int bad = 0;
    for (int b = 0; b < BS; ++b)
        for (int k = 0; k < H * P * N; ++k) {
            double r = state_ref[(size_t)b * H * P * N + k], v = pool_gpu[(size_t)idx[b] * H * P * N + k];
            bad += !(fabs(v - r) <= 1e-5 * (1.0 + fabs(r)));
        }
    for (int s = 0; s < SLOTS; ++s) {
        int live = 0;
        for (int b = 0; b < BS; ++b)
            live |= idx[b] == s;
        if (!live)
            bad += memcmp(pool_gpu + (size_t)s * H * P * N, pool + (size_t)s * H * P * N, sizeof(float) * H * P * N) != 0;
    }
    for (int i = 0; i < BS * H * P; ++i) {
        if (llabs(bf16_ordered(out[i]) - bf16_ordered(out_ref[i])) <= 2)
            continue;
        double mag = fmax(fabs(y_ref[i]), ldexp(tau_ref[i], -10));
        bad += !(fabs(bf16_value(out[i]) - y_ref[i]) <= 2 * ulp_at(mag, 7, -126));
    }
    hipFree(d_pool), hipFree(d_idx), hipFree(d_xbc), hipFree(d_dt), hipFree(d_A), hipFree(d_D), hipFree(d_bias);
    hipFree(d_out);
    printf("decode: %d values out of tolerance\n", bad);
    return bad != 0;
}

static int check_scan(void)
{
    enum { BS = 1, DIM = 16, N = 16, G = 1, L = 700 };
    static uint16_t u[BS * DIM * L], delta[BS * DIM * L], Bm[BS * G * N * L], Cm[BS * G * N * L];
    static uint16_t out[BS * DIM * L], out_ref[BS * DIM * L];
    static float state[BS * DIM * N], state_gpu[BS * DIM * N], state_host[BS * DIM * N];
    float A[DIM * N], D[DIM], bias[DIM];
    for (int i = 0; i < BS * DIM * L; ++i)
        u[i] = rand_f16(), delta[i] = rand_f16();
    for (int i = 0; i < BS * G * N * L; ++i)
        Bm[i] = rand_f16(), Cm[i] = rand_f16();
    for (int i = 0; i < BS * DIM * N; ++i)
        state[i] = 2.0f * rand_unit() - 1.0f;
    for (int i = 0; i < DIM * N; ++i)
        A[i] = -(float)(1 + i % N) * (0.5f + rand_unit());
    for (int d = 0; d < DIM; ++d)
        D[d] = rand_unit(), bias[d] = -3.0f - 2.0f * rand_unit();

    void *d_u = to_device(u, sizeof u), *d_dl = to_device(delta, sizeof delta);
    void *d_B = to_device(Bm, sizeof Bm), *d_C = to_device(Cm, sizeof Cm);
    void *d_A = to_device(A, sizeof A), *d_D = to_device(D, sizeof D), *d_bias = to_device(bias, sizeof bias);
    float *d_state = to_device(state, sizeof state);
    void *d_out = NULL;
    HIP_OK(hipMalloc(&d_out, sizeof out));

    ssu_scan_args a;
    memset(&a, 0, sizeof a);
    a.batch = BS, a.dim = DIM, a.dstate = N, a.ngroups = G, a.seqlen = L, a.delta_softplus = 1;
    a.state = (ssu_view){d_state, SSU_F32, 0, {DIM * N, N, 1, 0}};
    a.u = (ssu_view){d_u, SSU_F16, 0, {DIM * L, L, 1, 0}};
    a.delta = (ssu_view){d_dl, SSU_F16, 0, {DIM * L, L, 1, 0}};
    a.B = (ssu_view){d_B, SSU_F16, 0, {G * N * L, N * L, L, 1}};
    a.C = (ssu_view){d_C, SSU_F16, 0, {G * N * L, N * L, L, 1}};
    a.A = (ssu_view){d_A, SSU_F32, 0, {N, 1, 0, 0}};
    a.D = (ssu_view){d_D, SSU_F32, 0, {1, 0, 0, 0}};
    a.delta_bias = (ssu_view){d_bias, SSU_F32, 0, {1, 0, 0, 0}};
    a.out = (ssu_view){d_out, SSU_F16, 0, {DIM * L, L, 1, 0}};
    SSU_OK_(ssu_scan(&a, 512, -1, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(state_gpu, d_state, sizeof state, hipMemcpyDeviceToHost));

    static double st_ref[BS * DIM * N], err_ref[BS * DIM * N], y_ref[BS * DIM * L], tau_ref[BS * DIM * L],
        rho_ref[BS * DIM * L];
    memcpy(state_host, state, sizeof state);
    ssu_ref_scan_args g;
    memset(&g, 0, sizeof g);
    g.batch = BS, g.dim = DIM, g.dstate = N, g.ngroups = G, g.delta_softplus = 1, g.io_dtype = 1, g.nthreads = 1;
    g.seqlen = L;
    g.state = state_host, g.st_b = DIM * N, g.st_d = N;
    g.u = u, g.u_b = DIM * L, g.u_d = L, g.u_t = 1;
    g.delta = delta, g.dl_b = DIM * L, g.dl_d = L, g.dl_t = 1;
    g.B = Bm, g.B_b = G * N * L, g.B_g = N * L, g.B_n = L, g.B_t = 1;
    g.C = Cm, g.C_b = G * N * L, g.C_g = N * L, g.C_n = L, g.C_t = 1;
    g.A = A, g.A_d = N, g.A_n = 1, g.D = D, g.delta_bias = bias;
    g.out = out_ref, g.o_b = DIM * L, g.o_d = L, g.o_t = 1;
    g.state_ref = st_ref, g.err_ref = err_ref, g.y_ref = y_ref, g.tau_ref = tau_ref, g.rho_ref = rho_ref;
    if (ssu_ref_scan(&g) != 0) {
        printf("oracle failed\n");
        return 1;
    }
    const double eps = ldexp(1.0, -24);
    int bad = 0;
    for (int i = 0; i < BS * DIM * N; ++i)
        bad += !(fabs(state_gpu[i] - st_ref[i]) <= 16 * eps * err_ref[i]);
    for (int i = 0; i < BS * DIM * L; ++i) {
        double tol = ulp_at(fabs(y_ref[i]), 10, -14) + 8 * eps * (rho_ref[i] + N * tau_ref[i]);
        bad += !(fabs(ssu_ref_f16_value(out[i]) - y_ref[i]) <= tol);
    }
    hipFree(d_u), hipFree(d_dl), hipFree(d_B), hipFree(d_C), hipFree(d_A), hipFree(d_D), hipFree(d_bias);
    hipFree(d_state), hipFree(d_out);
    printf("scan: %d values out of tolerance\n", bad);
    return bad != 0;
}

/* ssu_update_tokens (3 tokens) against three ssu_update calls: bitwise. */
static int check_tokens(void)
{
    enum { H = 2, P = 64, N = 128, G = 1, BS = 3, K = 3, SLOTS = 4, ROW = H * P + 2 * G * N };
    const int32_t idx[BS] = {3, 0, 2};
    static float pool[SLOTS * H * P * N], pool_f[SLOTS * H * P * N], pool_s[SLOTS * H * P * N];
    static uint16_t xbc[BS * K * ROW], dt[BS * K * H], out_f[BS * K * H * P], out_s[BS * K * H * P];
    float A[H], D[H], bias[H];
    for (int i = 0; i < SLOTS * H * P * N; ++i)
        pool[i] = 2.0f * rand_unit() - 1.0f;
    for (int i = 0; i < BS * K * ROW; ++i)
        xbc[i] = rand_bf16();
    for (int i = 0; i < BS * K * H; ++i)
        dt[i] = rand_bf16();
    for (int h = 0; h < H; ++h)
        A[h] = -(0.5f + rand_unit()), D[h] = rand_unit(), bias[h] = -2.0f * rand_unit();

    float *d_pool = to_device(pool, sizeof pool);
    void *d_idx = to_device(idx, sizeof idx), *d_xbc = to_device(xbc, sizeof xbc), *d_dt = to_device(dt, sizeof dt);
    void *d_A = to_device(A, sizeof A), *d_D = to_device(D, sizeof D), *d_bias = to_device(bias, sizeof bias);
    void *d_out = NULL;
    HIP_OK(hipMalloc(&d_out, sizeof out_f));
    ssu_config cfg = {H, P, N, G, 1, -1, -1, 0};
    ssu_handle *h = NULL;
    SSU_OK_(ssu_create(&cfg, &h));

    /* [request, token, ...] layouts: xBC rows and dt per (request, token) */
    ssu_tokens_args a;
    memset(&a, 0, sizeof a);
    a.batch = BS, a.ntokens = K, a.pool_slots = SLOTS;
    a.state = (ssu_view){d_pool, SSU_F32, 0, {H * P * N, P * N, N, 1}};
    a.idx = (ssu_view){d_idx, SSU_I32, 0, {1, 0, 0, 0}};
    a.x = (ssu_view){d_xbc, SSU_BF16, 0, {K * ROW, ROW, P, 1}};
    a.B = (ssu_view){(uint16_t *)d_xbc + H * P, SSU_BF16, 0, {K * ROW, ROW, N, 1}};
    a.C = (ssu_view){(uint16_t *)d_xbc + H * P + G * N, SSU_BF16, 0, {K * ROW, ROW, N, 1}};
    a.dt = (ssu_view){d_dt, SSU_BF16, 0, {K * H, H, 1, 0}};
    a.dt_bias = (ssu_view){d_bias, SSU_F32, 0, {1, 0, 0, 0}};
    a.A = (ssu_view){d_A, SSU_F32, 0, {1, 0, 0, 0}};
    a.D = (ssu_view){d_D, SSU_F32, 0, {1, 0, 0, 0}};
    a.out = (ssu_view){d_out, SSU_BF16, 0, {K * H * P, H * P, P, 1}};
    SSU_OK_(ssu_update_tokens(h, &a, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(pool_f, d_pool, sizeof pool, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out_f, d_out, sizeof out_f, hipMemcpyDeviceToHost));

    HIP_OK(hipMemcpy(d_pool, pool, sizeof pool, hipMemcpyHostToDevice));
    HIP_OK(hipMemset(d_out, 0, sizeof out_f));
    for (int t = 0; t < K; ++t) {
        ssu_args s1;
        memset(&s1, 0, sizeof s1);
        s1.batch = BS, s1.pool_slots = SLOTS;
        s1.state = a.state, s1.idx = a.idx, s1.dt_bias = a.dt_bias, s1.A = a.A, s1.D = a.D;
        s1.x = (ssu_view){(uint16_t *)d_xbc + t * ROW, SSU_BF16, 0, {K * ROW, P, 1, 0}};
        s1.B = (ssu_view){(uint16_t *)d_xbc + t * ROW + H * P, SSU_BF16, 0, {K * ROW, N, 1, 0}};
        s1.C = (ssu_view){(uint16_t *)d_xbc + t * ROW + H * P + G * N, SSU_BF16, 0, {K * ROW, N, 1, 0}};
        s1.dt = (ssu_view){(uint16_t *)d_dt + t * H, SSU_BF16, 0, {K * H, 1, 0, 0}};
        s1.out = (ssu_view){(uint16_t *)d_out + t * H * P, SSU_BF16, 0, {K * H * P, P, 1, 0}};
        SSU_OK_(ssu_update(h, &s1, NULL));
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(pool_s, d_pool, sizeof pool, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(out_s, d_out, sizeof out_s, hipMemcpyDeviceToHost));
    ssu_destroy(h);
    int bad = (memcmp(pool_f, pool_s, sizeof pool) != 0) + (memcmp(out_f, out_s, sizeof out_f) != 0);
    hipFree(d_pool), hipFree(d_idx), hipFree(d_xbc), hipFree(d_dt), hipFree(d_A), hipFree(d_D), hipFree(d_bias);
    hipFree(d_out);
    printf("tokens: %s\n", bad ? "fused and successive calls differ" : "fused = successive, bitwise");
    return bad != 0;
}

/* ssu_copy_blocks over two tensors of different block sizes: destinations
 * receive their sources' bytes, every other block keeps its own. */
static int check_copy(void)
{
    enum { NB = 6, BYTES0 = 4096, BYTES1 = 640, STRIDE1 = 768 };
    static uint8_t t0[NB * BYTES0], t1[NB * STRIDE1], g0[NB * BYTES0], g1[NB * STRIDE1];
    for (int i = 0; i < NB * BYTES0; ++i)
        t0[i] = (uint8_t)next();
    for (int i = 0; i < NB * STRIDE1; ++i)
        t1[i] = (uint8_t)next();
    const int32_t src[3] = {0, 4, 2}, dst[3] = {5, 1, 2}; /* the last: src == dst, a no-op */
    void *d0 = to_device(t0, sizeof t0), *d1 = to_device(t1, sizeof t1);
    void *d_src = to_device(src, sizeof src), *d_dst = to_device(dst, sizeof dst);
    const ssu_block_tensor ts[2] = {{d0, BYTES0, BYTES0, NB}, {d1, STRIDE1, BYTES1, NB}};
    SSU_OK_(ssu_copy_blocks(ts, 2, d_src, d_dst, 3, -1, NULL));
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(g0, d0, sizeof g0, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g1, d1, sizeof g1, hipMemcpyDeviceToHost));
    for (int r = 0; r < 3; ++r) {
        memcpy(t0 + (size_t)dst[r] * BYTES0, t0 + (size_t)src[r] * BYTES0, BYTES0);
        memcpy(t1 + (size_t)dst[r] * STRIDE1, t1 + (size_t)src[r] * STRIDE1, BYTES1);
    }
    const int bad = (memcmp(g0, t0, sizeof t0) != 0) + (memcmp(g1, t1, sizeof t1) != 0);
    hipFree(d0), hipFree(d1), hipFree(d_src), hipFree(d_dst);
    printf("copy: %s\n", bad ? "blocks differ" : "blocks as expected");
    return bad != 0;
}

int main(void)
{
    int dev = 0;
    HIP_OK(hipGetDeviceCount(&dev));
    if (dev < 1) {
        printf("no GPU\n");
        return 1;
    }
    int fail = check_decode();
    fail |= check_scan();
    fail |= check_tokens();
    fail |= check_copy();
    if (fail)
        return 1;
    printf("ok\n");
    return 0;
}
