// scan.hip -- ssu_scan: the selective scan over a sequence (prefill) on
// MI355X (gfx950).
//
// What it computes (COREY: Entropy-Guided Runtime Chunk Scheduling for
// Selective Scan Kernels, Table 9, Table 17 and Table 18, the selective_scan_fn
// benchmark: dim channels with d_state states each, FP16 or BF16 activations,
// the sequence cut into static chunks of tokens, one kernel call per chunk
// with the state carried between calls): for every request b, channel d and
// token t in order,
//   Delta = softplus(delta[b,d,t] + delta_bias[d])   (or without the softplus)
//   h[n]  = h[n] * exp(A[d,n] * Delta) + (Delta * u[b,d,t]) * B[b,g,n,t]
//   y[t]  = sum_n h[n] * C[b,g,n,t] + D[d] * u[b,d,t]
// with g = d / (dim / G), h read from and written back to the fp32 state.
//
// Two kernels compute it, with the same fp32 operations in the same order,
// so every configuration of either gives the same bits:
//
//   direct (scan_t{SEG}_n{NSW}): one workgroup per (request, channel), one
//     wave per NSW of its states; each wave loads its states' B and C rows
//     straight into registers, all of a block's loads issued before any is
//     used. Few instructions stand between a launch and its first result,
//     which is what a small batch (a few thousand channels: latency bound)
//     needs.
//   staged (scan_t{SEG}_n{NSW}_w{W}_c{CPW}): a workgroup holds CPW channels of
//     one (request, group), with W waves of NSW states each. The channels of
//     a group share B and C, so the workgroup stages a block's B and C rows
//     in LDS once, W * NSW states at a time (a round; d_state above that
//     takes several rounds), and each wave reads the rows of the state it is
//     working on just before it needs them, with the carried states and
//     decay rates kept in LDS. Few registers are live, so four waves fit on
//     each SIMD, and the B/C traffic falls by CPW: what a large batch
//     (throughput bound) needs.
//
// Both split tokens into blocks of 64 * SEG: lane l owns tokens l*SEG ..
// l*SEG+SEG-1 of a block, so a block's activations are one coalesced vector
// load per lane. Per state n the recurrence h -> a h + b is a composition of
// affine maps, and composition is associative:
//   1. each lane composes its SEG pairs (a_j, b_j) into one map (P, Q);
//   2. a 64-lane inclusive scan of the maps in a fixed tree (DPP row shifts
//      1, 2, 4, 8, then row broadcasts 15 and 31) gives every lane the map
//      from the block's start to its last token; applied to the carried state
//      it is the state after that token;
//   3. shifted one lane up (lane 0 takes the carried state) it is each lane's
//      start state g; the lane's state after its token j is its prefix map
//      applied to g, h_j = P_j g + Q_j (P_j, Q_j kept from step 1), computed
//      for every j independently, and y_j += h_j C_j;
//   4. lane 63's end state is the carried state for the next block.
// The carried state is wave-uniform, so blocks, and launches that start on a
// block boundary, continue from exactly the value the previous block ended
// with: chunkings whose chunks are multiples of 64 * SEG give bitwise
// identical results.
//
// y is summed in one fixed order whatever the configuration: states in groups
// of 8, each group's partial accumulated in state order (fma), the groups
// added in group order (the channel's first wave adds the partials of the
// other waves, handed over through LDS, after its own). With the same token
// segment, every configuration and every chunking on block boundaries gives
// bitwise the same outputs.
//
// Invalid tokens (past the end of a ragged last block) get Delta = 0, u = 0
// and B = C = 0: their decay is exp2(0) = 1 and their input 0, the identity
// map, so they leave every scan value unchanged. States past d_state get
// A = 0, h = 0 and B = C = 0: the identity map and a zero contribution.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <type_traits>

#include "internal.h"

namespace ssu {
namespace {

constexpr int kLanes = 64;
constexpr int kMaxStates = 64;
constexpr int kGroup = 8;  // states per partial sum of y
constexpr float kLog2e = 1.44269504088896340736f;

struct ScanParams {
    const uint16_t *u, *delta, *B, *C;
    uint16_t *out;
    float *state;
    const float *A, *D, *bias;
    int64_t u_b, u_d, dl_b, dl_d, B_b, B_g, B_n, C_b, C_g, C_n, o_b, o_d, st_b, st_d, A_d, A_n;
    int64_t t0, t1;
    int32_t dim, dstate, ch_per_group, softplus, vec, rounds;
};

template <bool F16>
__device__ __forceinline__ float io_to_f32(uint32_t bits)
{
    if constexpr (F16)
        return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
    else
        return __uint_as_float(bits << 16);
}

template <bool F16>
__device__ __forceinline__ uint16_t f32_to_io(float f)
{
    if constexpr (F16) {
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // v_cvt_f16_f32, round to nearest even
    } else {
        uint32_t w = __float_as_uint(f);
        if ((w & 0x7fffffffu) > 0x7f800000u)
            return static_cast<uint16_t>((w >> 16) | 0x40u);  // NaN stays a quiet NaN
        w += 0x7fffu + ((w >> 16) & 1u);
        return static_cast<uint16_t>(w >> 16);
    }
}

// Tokens tok .. tok+SEG-1 of a row, packed two per word. FAST: all of them
// lie before t1 and the row is aligned for one vector load. Otherwise each is
// read from an address clamped into [0, t1) (always valid) and tokens at or
// past t1 read as 0; the loads stay unconditional, so they issue back to back.
template <int SEG, bool FAST>
__device__ __forceinline__ void load_seg(const uint16_t *row, int64_t tok, int64_t t1, uint32_t (&w)[(SEG + 1) / 2])
{
    if constexpr (FAST) {
        const uint16_t *p = row + tok;
        if constexpr (SEG == 8) {
            const auto x = *reinterpret_cast<const uint32_t __attribute__((ext_vector_type(4))) *>(p);
            w[0] = x.x, w[1] = x.y, w[2] = x.z, w[3] = x.w;
        } else if constexpr (SEG == 4) {
            const auto x = *reinterpret_cast<const u32x2 *>(p);
            w[0] = x.x, w[1] = x.y;
        } else if constexpr (SEG == 2) {
            w[0] = *reinterpret_cast<const uint32_t *>(p);
        } else {
            w[0] = *p;
        }
    } else {
        uint32_t v[SEG];
#pragma unroll
        for (int j = 0; j < SEG; ++j) {
            const int64_t t = tok + j;
            const uint32_t x = row[t < t1 ? t : t1 - 1];
            v[j] = t < t1 ? x : 0u;
        }
#pragma unroll
        for (int k = 0; k < (SEG + 1) / 2; ++k)
            w[k] = v[2 * k] | ((2 * k + 1 < SEG) ? (v[2 * k + 1] << 16) : 0u);
    }
}

// Store tokens tok .. tok+SEG-1 of a row (those before t1).
template <int SEG, bool FAST>
__device__ __forceinline__ void store_seg(uint16_t *row, int64_t tok, int64_t t1, const uint16_t (&v)[SEG])
{
    if constexpr (FAST) {
        uint16_t *p = row + tok;
        uint32_t w[(SEG + 1) / 2];
#pragma unroll
        for (int k = 0; k < (SEG + 1) / 2; ++k)
            w[k] = v[2 * k] | ((2 * k + 1 < SEG) ? (static_cast<uint32_t>(v[2 * k + 1]) << 16) : 0u);
        if constexpr (SEG == 8) {
            uint32_t __attribute__((ext_vector_type(4))) x = {w[0], w[1], w[2], w[3]};
            *reinterpret_cast<uint32_t __attribute__((ext_vector_type(4))) *>(p) = x;
        } else if constexpr (SEG == 4) {
            u32x2 x = {w[0], w[1]};
            *reinterpret_cast<u32x2 *>(p) = x;
        } else if constexpr (SEG == 2) {
            *reinterpret_cast<uint32_t *>(p) = w[0];
        } else {
            *p = v[0];
        }
    } else {
#pragma unroll
        for (int j = 0; j < SEG; ++j)
            if (tok + j < t1)
                row[tok + j] = v[j];
    }
}

template <int SEG>
__device__ __forceinline__ uint32_t half_of(const uint32_t (&w)[(SEG + 1) / 2], int j)
{
    return (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu);
}

// The 64-lane inclusive scan of the lanes' maps (P, Q), for two states at
// once or for one, as in-place DPP operations: at each level every lane
// combines its map with the map of the lane that the DPP control names (the
// earlier tokens), Q += P * Q_src, then P *= P_src. A lane without a source
// (shifted out of its row, or in a row the row mask leaves out) is not
// written, which is the same as combining with the identity map (1, 0). The
// levels: shifts 1, 2, 4, 8 within rows of 16, then lane 15 of each row into
// the next (rows 1, 3) and lane 31 into rows 2, 3. A DPP read needs two wait
// states after a VALU write of its source register: the leading s_nop 1
// covers the caller's last writes; between levels, two interleaved states
// already put three instructions between a write and its next DPP read, and
// one state needs an s_nop 0.
#define SSU_SCAN_LEVEL2(CTL)                                        \
    "v_fmac_f32_dpp %0, %0, %2 " CTL "\n\t"                         \
    "v_fmac_f32_dpp %1, %1, %3 " CTL "\n\t"                         \
    "v_mul_f32_dpp %2, %2, %2 " CTL "\n\t"                          \
    "v_mul_f32_dpp %3, %3, %3 " CTL "\n\t"
#define SSU_SCAN_TREE2(Q0, Q1, P0, P1)                                                  \
    asm("s_nop 1\n\t" SSU_SCAN_LEVEL2("row_shr:1 row_mask:0xf bank_mask:0xf")          \
            SSU_SCAN_LEVEL2("row_shr:2 row_mask:0xf bank_mask:0xf")                      \
                SSU_SCAN_LEVEL2("row_shr:4 row_mask:0xf bank_mask:0xf")                  \
                    SSU_SCAN_LEVEL2("row_shr:8 row_mask:0xf bank_mask:0xf")              \
                        SSU_SCAN_LEVEL2("row_bcast:15 row_mask:0xa bank_mask:0xf")       \
                            SSU_SCAN_LEVEL2("row_bcast:31 row_mask:0xc bank_mask:0xf")   \
        : "+v"(Q0), "+v"(Q1), "+v"(P0), "+v"(P1))
#define SSU_SCAN_LEVEL1(CTL)                                        \
    "v_fmac_f32_dpp %0, %0, %1 " CTL "\n\t"                         \
    "v_mul_f32_dpp %1, %1, %1 " CTL "\n\t"
#define SSU_SCAN_TREE1(Q0, P0)                                                                      \
    asm("s_nop 1\n\t" SSU_SCAN_LEVEL1("row_shr:1 row_mask:0xf bank_mask:0xf") "s_nop 0\n\t"          \
            SSU_SCAN_LEVEL1("row_shr:2 row_mask:0xf bank_mask:0xf") "s_nop 0\n\t"                      \
                SSU_SCAN_LEVEL1("row_shr:4 row_mask:0xf bank_mask:0xf") "s_nop 0\n\t"                  \
                    SSU_SCAN_LEVEL1("row_shr:8 row_mask:0xf bank_mask:0xf") "s_nop 0\n\t"              \
                        SSU_SCAN_LEVEL1("row_bcast:15 row_mask:0xa bank_mask:0xf") "s_nop 0\n\t"       \
                            SSU_SCAN_LEVEL1("row_bcast:31 row_mask:0xc bank_mask:0xf")                   \
        : "+v"(Q0), "+v"(P0))

// DPP control of the one-lane shift of the whole wave (GFX9 encoding).
constexpr int kWaveShr1 = 0x138;

constexpr float kLn2Hi = 0.693147182464599609375f;      // (float)ln 2
constexpr float kLn2Lo = -1.904654323148236e-09f;       // ln 2 - kLn2Hi

// softplus(v) = max(v, 0) + log1p(e) with e = exp(-|v|) in (0, 1], and
// log1p(e) = 2 atanh(s) = s q(s^2), s = e / (2 + e) in (0, 1/3]. q is a
// degree-4 polynomial fitted to 2 atanh(sqrt z) / sqrt z on z in [0, 1/9] by
// the Remez exchange (relative error 4e-9, under a tenth of an fp32 ulp;
// fit_softplus.py beside this file recomputes it). e is the hardware exp2 of
// t = -|v| log2(e) in fp32, times exp(r) ~ 1 + r for the residual
// r = -|v| - t ln 2 (ln 2 split in two, each product exact in an fma), so the
// rounding of t costs nothing. -|v| is clamped at -128, where exp2 is already
// 0 in fp32, so that infinite v give e = 0 rather than inf - inf; the
// positive part is a select that lets NaN through (fmaxf would drop it):
// softplus(+inf) = +inf, softplus(-inf) = 0, softplus(NaN) = NaN, and every
// finite v gives the same bits as without the clamp.
__device__ __forceinline__ float softplus_f32(float v)
{
    const float x = __builtin_amdgcn_fmed3f(-fabsf(v), -128.0f, 0.0f);  // NaN: carried by the select below
    const float t = x * kLog2e;
    const float ex = __builtin_amdgcn_exp2f(t);
    const float r = fmaf(-t, kLn2Lo, fmaf(-t, kLn2Hi, x));
    const float e = fmaf(ex, r, ex);
    const float sv = e * __builtin_amdgcn_rcpf(2.0f + e);
    const float z = sv * sv;
    float q = fmaf(2.817833424e-01f, z, 2.796060145e-01f);
    q = fmaf(q, z, 4.002490938e-01f);
    q = fmaf(q, z, 6.666631699e-01f);
    q = fmaf(q, z, 2.0f);
    return fmaf(sv, q, v <= 0.0f ? 0.0f : v);
}

// One state's scan over one block of 64 * SEG tokens, in this lane's SEG
// tokens: dl their step sizes, du = dl * u their inputs, dls = the sum of dl
// (in token order), Bw and Cw the state's B and C bits, A2 = A * log2(e), h
// the carried state (wave uniform). Adds the state's h_j * C_j to yy[j] and
// returns the carried state after the block.
//   1. the lane's whole map: decay exp2(A2 * dls) (the product of its
//      tokens' decays in one exponential), and the state Q reached from 0;
//   2. the 64-lane inclusive scan of the maps;
//   3. the lane's end state e (the map applied to h) and start state g (e
//      shifted one lane up, lane 0 taking h); the lane's tokens are replayed
//      from g, h_j = a_j h_{j-1} + b_j, and after its last token the state
//      is e;
//   4. lane 63's e is the carried state.
template <bool F16, int SEG>
__device__ __forceinline__ float scan_state(const float (&dl)[SEG], const float (&du)[SEG], float dls, float A2,
                                            const uint32_t (&Bw)[(SEG + 1) / 2], const uint32_t (&Cw)[(SEG + 1) / 2],
                                            float h, float (&yy)[SEG])
{
    float a[SEG], b[SEG];
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
        a[j] = __builtin_amdgcn_exp2f(dl[j] * A2);
        b[j] = fmaf(du[j], io_to_f32<F16>(half_of<SEG>(Bw, j)), 0.0f);
    }
    float Q = b[0];
#pragma unroll
    for (int j = 1; j < SEG; ++j)
        Q = fmaf(a[j], Q, b[j]);
    float P = __builtin_amdgcn_exp2f(dls * A2);
    SSU_SCAN_TREE1(Q, P);
    const float e = fmaf(P, h, Q);
    const float g = __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(h), __float_as_int(e), kWaveShr1, 0xf, 0xf, false));
    float hj = g;
#pragma unroll
    for (int j = 0; j < SEG - 1; ++j) {
        hj = fmaf(a[j], hj, b[j]);
        yy[j] = fmaf(hj, io_to_f32<F16>(half_of<SEG>(Cw, j)), yy[j]);
    }
    yy[SEG - 1] = fmaf(e, io_to_f32<F16>(half_of<SEG>(Cw, SEG - 1)), yy[SEG - 1]);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), kLanes - 1));
}

// The same for two states n, n+1 at once (their dependent steps interleave),
// with the same operations per state, so the same bits. y gets state n's
// terms before state n+1's.
template <bool F16, int SEG>
__device__ __forceinline__ void scan_state2(const float (&dl)[SEG], const float (&du)[SEG], float dls, float A20,
                                            float A21, const uint32_t (&B0)[(SEG + 1) / 2],
                                            const uint32_t (&B1)[(SEG + 1) / 2], const uint32_t (&C0)[(SEG + 1) / 2],
                                            const uint32_t (&C1)[(SEG + 1) / 2], float &h0, float &h1,
                                            float (&yy)[SEG])
{
    float a0[SEG], b0[SEG], a1[SEG], b1[SEG];
#pragma unroll
    for (int j = 0; j < SEG; ++j) {
        a0[j] = __builtin_amdgcn_exp2f(dl[j] * A20);
        a1[j] = __builtin_amdgcn_exp2f(dl[j] * A21);
        b0[j] = fmaf(du[j], io_to_f32<F16>(half_of<SEG>(B0, j)), 0.0f);
        b1[j] = fmaf(du[j], io_to_f32<F16>(half_of<SEG>(B1, j)), 0.0f);
    }
    float Q0 = b0[0], Q1 = b1[0];
#pragma unroll
    for (int j = 1; j < SEG; ++j) {
        Q0 = fmaf(a0[j], Q0, b0[j]);
        Q1 = fmaf(a1[j], Q1, b1[j]);
    }
    float P0 = __builtin_amdgcn_exp2f(dls * A20), P1 = __builtin_amdgcn_exp2f(dls * A21);
    SSU_SCAN_TREE2(Q0, Q1, P0, P1);
    const float e0 = fmaf(P0, h0, Q0), e1 = fmaf(P1, h1, Q1);
    const float g0 = __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(h0), __float_as_int(e0), kWaveShr1, 0xf, 0xf, false));
    const float g1 = __int_as_float(
        __builtin_amdgcn_update_dpp(__float_as_int(h1), __float_as_int(e1), kWaveShr1, 0xf, 0xf, false));
    float hj0 = g0, hj1 = g1;
#pragma unroll
    for (int j = 0; j < SEG - 1; ++j) {
        hj0 = fmaf(a0[j], hj0, b0[j]);
        hj1 = fmaf(a1[j], hj1, b1[j]);
        yy[j] = fmaf(hj0, io_to_f32<F16>(half_of<SEG>(C0, j)), yy[j]);
        yy[j] = fmaf(hj1, io_to_f32<F16>(half_of<SEG>(C1, j)), yy[j]);
    }
    yy[SEG - 1] = fmaf(e0, io_to_f32<F16>(half_of<SEG>(C0, SEG - 1)), yy[SEG - 1]);
    yy[SEG - 1] = fmaf(e1, io_to_f32<F16>(half_of<SEG>(C1, SEG - 1)), yy[SEG - 1]);
    h0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e0), kLanes - 1));
    h1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e1), kLanes - 1));
}

// The sum of a lane's step sizes, in token order.
template <int SEG>
__device__ __forceinline__ float step_sum(const float (&dl)[SEG])
{
    float s = dl[0];
#pragma unroll
    for (int j = 1; j < SEG; ++j)
        s += dl[j];
    return s;
}

// One wave's share of one (request, channel): its 16 states' carried values
// and decay rates (wave-uniform) and the rows it reads and writes.
template <bool F16, int SEG, int NSW, bool FULL>
struct Chan {
    static constexpr int BLOCK = kLanes * SEG;
    static constexpr int WORDS = (SEG + 1) / 2;

    const uint16_t *u_row, *dl_row, *B_row, *C_row;
    uint16_t *o_row;
    int64_t B_n, C_n;
    float bias, Dd;
    int ns, lane;
    bool softplus;
    float h0[NSW], A2[NSW];

    static constexpr int GROUPS = NSW / kGroup;

    // One block of 64 * SEG tokens starting at blk: the scan of every state
    // of this wave; yg returns the partial of y over each group of 8 states.
    // FAST: the block lies inside the chunk and every row is aligned for
    // vector access, so all loads are unconditional vector loads.
    template <bool FAST>
    __device__ __forceinline__ void block(int64_t blk, int64_t t1, float (&yg)[GROUPS][SEG], uint32_t (&uw)[WORDS])
    {
        const int64_t tok = blk + lane * SEG;

        // every load of the block first, so that one wait covers them all
        uint32_t dw[WORDS], Bw[NSW][WORDS], Cw[NSW][WORDS];
        load_seg<SEG, FAST>(u_row, tok, t1, uw);
        load_seg<SEG, FAST>(dl_row, tok, t1, dw);
#pragma unroll
        for (int n = 0; n < NSW; ++n) {
            const int r = FULL ? n : min(n, ns - 1);  // rows past dstate: read a valid row, zeroed below
            load_seg<SEG, FAST>(B_row + r * B_n, tok, t1, Bw[n]);
            load_seg<SEG, FAST>(C_row + r * C_n, tok, t1, Cw[n]);
        }
        if constexpr (!FULL) {
            // states past dstate: B = C = 0 (and A2 = 0), the identity map and a
            // zero contribution
#pragma unroll
            for (int n = 0; n < NSW; ++n)
#pragma unroll
                for (int k = 0; k < WORDS; ++k) {
                    Bw[n][k] = n < ns ? Bw[n][k] : 0u;
                    Cw[n][k] = n < ns ? Cw[n][k] : 0u;
                }
        }

        // step sizes Delta_j and inputs Delta_j u_j; invalid tokens: identity
        float dl[SEG], du[SEG];
#pragma unroll
        for (int j = 0; j < SEG; ++j) {
            // (the f16 conversions fold into mixed-precision fmas; x * 1 + bias
            // and sv * u + 0 round exactly as x + bias and sv * u)
            const float v = fmaf(io_to_f32<F16>(half_of<SEG>(dw, j)), 1.0f, bias);
            float sv = softplus ? softplus_f32(v) : v;
            if (!FAST)
                sv = tok + j < t1 ? sv : 0.0f;
            dl[j] = sv;
            du[j] = fmaf(sv, io_to_f32<F16>(half_of<SEG>(uw, j)), 0.0f);
        }
#pragma unroll
        for (int gi = 0; gi < GROUPS; ++gi)
#pragma unroll
            for (int j = 0; j < SEG; ++j)
                yg[gi][j] = 0.0f;

        const float dls = step_sum<SEG>(dl);
#pragma unroll
        for (int n = 0; n < NSW; n += 2)
            scan_state2<F16, SEG>(dl, du, dls, A2[n], A2[n + 1], Bw[n], Bw[n + 1], Cw[n], Cw[n + 1], h0[n],
                                  h0[n + 1], yg[n / kGroup]);
    }
};

template <bool F16, int SEG, int NSW, int MAXW, bool FULL>
__global__ void __launch_bounds__(kLanes * MAXW) ssu_scan_direct_kernel(const ScanParams p)
{
    using Ch = Chan<F16, SEG, NSW, FULL>;
    constexpr int BLOCK = Ch::BLOCK;
    constexpr int GROUPS = Ch::GROUPS;
    // group partials of waves 1 .. W-1
    __shared__ float ypart[MAXW > 1 ? (MAXW - 1) * GROUPS : 1][MAXW > 1 ? BLOCK : 1];

    const int lane = static_cast<int>(threadIdx.x) & (kLanes - 1);
    const int wave = MAXW > 1 ? static_cast<int>(threadIdx.x) / kLanes : 0;
    const int nwaves = MAXW > 1 ? static_cast<int>(blockDim.x) / kLanes : 1;
    const int64_t bd = blockIdx.x;
    const int64_t b = bd / p.dim;
    const int d = static_cast<int>(bd - b * p.dim);
    const int grp = d / p.ch_per_group;
    const int n0 = wave * NSW;

    Ch c;
    c.lane = lane;
    c.ns = FULL ? NSW : min(NSW, p.dstate - n0);
    c.u_row = p.u + b * p.u_b + d * p.u_d;
    c.dl_row = p.delta + b * p.dl_b + d * p.dl_d;
    c.B_row = p.B + b * p.B_b + grp * p.B_g + n0 * p.B_n;
    c.C_row = p.C + b * p.C_b + grp * p.C_g + n0 * p.C_n;
    c.o_row = p.out + b * p.o_b + d * p.o_d;
    c.B_n = p.B_n, c.C_n = p.C_n;
    c.softplus = p.softplus != 0;
    float *st = p.state + b * p.st_b + d * p.st_d + n0;

    // wave-uniform per-channel values; the state is written by this kernel,
    // so it is read with a plain load, never through the read-only path
    c.bias = p.bias ? load_ro(p.bias + d) : 0.0f;
    c.Dd = p.D ? load_ro(p.D + d) : 0.0f;
#pragma unroll
    for (int n = 0; n < NSW; ++n) {
        const int r = FULL ? n : min(n, c.ns - 1);
        const float hv = st[r], av = load_ro(p.A + d * p.A_d + (n0 + r) * p.A_n);
        c.h0[n] = (FULL || n < c.ns) ? hv : 0.0f;
        c.A2[n] = (FULL || n < c.ns) ? av * kLog2e : 0.0f;
    }
    const bool vec = p.vec != 0;

    for (int64_t blk = p.t0; blk < p.t1; blk += BLOCK) {
        float yg[GROUPS][SEG];
        uint32_t uw[Ch::WORDS];
        const bool fast = vec && blk + BLOCK <= p.t1;
        if (fast)
            c.template block<true>(blk, p.t1, yg, uw);
        else
            c.template block<false>(blk, p.t1, yg, uw);

        // y: the group partials added in group order
        float y[SEG];
#pragma unroll
        for (int j = 0; j < SEG; ++j) {
            y[j] = yg[0][j];
#pragma unroll
            for (int gi = 1; gi < GROUPS; ++gi)
                y[j] += yg[gi][j];
        }
        if constexpr (MAXW > 1) {
            if (wave > 0) {
#pragma unroll
                for (int gi = 0; gi < GROUPS; ++gi)
#pragma unroll
                    for (int j = 0; j < SEG; ++j)
                        ypart[(wave - 1) * GROUPS + gi][lane * SEG + j] = yg[gi][j];
            }
            __syncthreads();
            if (wave == 0) {
                for (int k = 0; k < (nwaves - 1) * GROUPS; ++k)
#pragma unroll
                    for (int j = 0; j < SEG; ++j)
                        y[j] += ypart[k][lane * SEG + j];
            }
            __syncthreads();
        }
        if (wave == 0) {
            uint16_t o[SEG];
#pragma unroll
            for (int j = 0; j < SEG; ++j)
                o[j] = f32_to_io<F16>(fmaf(c.Dd, io_to_f32<F16>(half_of<SEG>(uw, j)), y[j]));
            if (fast)
                store_seg<SEG, true>(c.o_row, blk + lane * SEG, p.t1, o);
            else
                store_seg<SEG, false>(c.o_row, blk + lane * SEG, p.t1, o);
        }
    }

    // final state: lane n of the wave writes state n0 + n
    float mine = 0.0f;
#pragma unroll
    for (int n = 0; n < NSW; ++n)
        mine = lane == n ? c.h0[n] : mine;
    if (lane < c.ns)
        st[lane] = mine;
}


using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

// SEG tokens of a row staged in LDS (16-bit values, packed two per word).
template <int SEG>
__device__ __forceinline__ void lds_seg(const uint16_t *p, uint32_t (&w)[(SEG + 1) / 2])
{
    if constexpr (SEG == 8) {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(p);
        w[0] = x.x, w[1] = x.y, w[2] = x.z, w[3] = x.w;
    } else if constexpr (SEG == 4) {
        const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
        w[0] = x.x, w[1] = x.y;
    } else if constexpr (SEG == 2) {
        w[0] = *reinterpret_cast<const uint32_t *>(p);
    } else {
        w[0] = *p;
    }
}

// Layout of one workgroup's LDS (dynamic, 16-byte aligned):
//   sBC [2 * RS][BLOCK] u16      the round's B rows, then its C rows;
//   sY  [W - 1][GROUPS][CPW][BLOCK] f32  partials of y that waves 1 .. W-1
//                                        of each channel hand to wave 0;
//   sH  [CPW][rounds * RS] f32   the carried states (0 past d_state);
//   sA  [CPW][rounds * RS] f32   A * log2(e) (0 past d_state).
template <int SEG, int NSW, int W, int CPW>
struct ScanShape {
    static constexpr int BLOCK = kLanes * SEG;
    static constexpr int WORDS = (SEG + 1) / 2;
    static constexpr int RS = W * NSW;            // states per round
    static constexpr int GROUPS = NSW / kGroup;
    static constexpr int NT = kLanes * W * CPW;   // threads
    static constexpr int CPR = BLOCK / 8;         // 16-byte pieces per staged row
    static constexpr int PIECES = 2 * RS * CPR;   // per round
    static constexpr int ITERS = (PIECES + NT - 1) / NT;
    static constexpr size_t BC_BYTES = size_t(2) * RS * BLOCK * 2;
    static constexpr size_t Y_BYTES = size_t(W - 1) * GROUPS * CPW * BLOCK * 4;
    static size_t lds_bytes(int rounds) { return BC_BYTES + Y_BYTES + size_t(2) * CPW * rounds * RS * 4; }
};

template <bool F16, int SEG, int NSW, int W, int CPW, bool FULL>
__global__ void __launch_bounds__(kLanes * W * CPW) __attribute__((amdgpu_waves_per_eu(4)))
ssu_scan_staged_kernel(const ScanParams p)
{
    using S = ScanShape<SEG, NSW, W, CPW>;
    constexpr int BLOCK = S::BLOCK, WORDS = S::WORDS, RS = S::RS, GROUPS = S::GROUPS, NT = S::NT;
    constexpr bool kAllPieces = S::PIECES % NT == 0;  // every thread stages ITERS pieces
    constexpr bool kSplitRows = kAllPieces && S::ITERS % 2 == 0 && NT % S::CPR == 0;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *const sBC = reinterpret_cast<uint16_t *>(smem);
    float *const sY = reinterpret_cast<float *>(smem + S::BC_BYTES);
    float *const sH = reinterpret_cast<float *>(smem + S::BC_BYTES + S::Y_BYTES);
    const int rounds = p.rounds;
    const int HP = rounds * RS;
    float *const sA = sH + CPW * HP;

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & (kLanes - 1);
    const int wv = tid / kLanes;
    const int c = wv / W;        // channel slot
    const int w = wv - c * W;    // state slice
    const int64_t bd0 = static_cast<int64_t>(blockIdx.x) * CPW;
    const int64_t b = bd0 / p.dim;                 // every channel of the group shares it
    const int d0 = static_cast<int>(bd0 - b * p.dim);
    const int d = d0 + c;
    const int grp = d0 / p.ch_per_group;
    const int dstate = p.dstate;

    const uint16_t *const Bbase = p.B + b * p.B_b + grp * p.B_g;
    const uint16_t *const Cbase = p.C + b * p.C_b + grp * p.C_g;
    const uint16_t *const u_row = p.u + b * p.u_b + d * p.u_d;
    const uint16_t *const dl_row = p.delta + b * p.dl_b + d * p.dl_d;
    const float bias = p.bias ? load_ro(p.bias + d) : 0.0f;
    const float Dd = p.D ? load_ro(p.D + d) : 0.0f;
    const bool softplus = p.softplus != 0;

    // carried states into LDS (the state is written by this kernel, so it is
    // read with plain loads, never through the read-only path)
    // and the decay rates A * log2(e)
    for (int i = tid; i < CPW * HP; i += NT) {
        const int cc = i / HP, n = i - cc * HP;
        const int nn = FULL ? n : min(n, dstate - 1);
        const float *st = p.state + b * p.st_b + (d0 + cc) * p.st_d;
        const float av = load_ro(p.A + (d0 + cc) * p.A_d + nn * p.A_n);
        sH[i] = (FULL || n < dstate) ? st[nn] : 0.0f;
        sA[i] = (FULL || n < dstate) ? av * kLog2e : 0.0f;
    }

    // One block of tokens. FAST: the block lies inside the chunk and every
    // row is aligned for vector access, so every load is an unconditional
    // vector load; otherwise each token is read from an address clamped into
    // the chunk and tokens past its end read as 0.
    auto block = [&](int64_t blk, auto fast_tag) {
        constexpr bool fast = decltype(fast_tag)::value;
        const int64_t tok = blk + lane * SEG;

        // this lane's step sizes and inputs (requested before the staging waits)
        uint32_t uw[WORDS], dw[WORDS];
        load_seg<SEG, fast>(u_row, tok, p.t1, uw);
        load_seg<SEG, fast>(dl_row, tok, p.t1, dw);
        float dl[SEG], du[SEG], y[SEG], dls = 0.0f;

        // step sizes Delta_j and inputs Delta_j u_j of this lane's tokens
        // (invalid tokens: the identity), and their sum
        auto steps = [&]() {
#pragma unroll
            for (int j = 0; j < SEG; ++j) {
                const float v = fmaf(io_to_f32<F16>(half_of<SEG>(dw, j)), 1.0f, bias);
                float sv = softplus ? softplus_f32(v) : v;
                sv = (fast || tok + j < p.t1) ? sv : 0.0f;
                dl[j] = sv;
                du[j] = fmaf(sv, io_to_f32<F16>(half_of<SEG>(uw, j)), 0.0f);
            }
            dls = step_sum<SEG>(dl);
        };

        for (int r = 0; r < rounds; ++r) {
            // stage the round's B and C rows into LDS (and, in the first
            // round, compute the step sizes while the pieces are in flight).
            // Fast blocks request all their 16-byte pieces (at most 8 per
            // thread at a time) before writing any; ragged or unaligned
            // blocks build each piece from clamped 16-bit reads, one at a time.
            {
                auto piece_src = [&](int q, bool &live) -> const uint16_t * {
                    const int row = q / S::CPR, k = q - row * S::CPR;
                    const bool isC = row >= RS;
                    const int n = r * RS + (isC ? row - RS : row);
                    const int nn = FULL ? n : min(n, dstate - 1);
                    live = FULL || n < dstate;
                    return (isC ? Cbase + nn * p.C_n : Bbase + nn * p.B_n) + blk + 8 * k;
                };
                // When the pieces divide evenly (every thread stages the same
                // number, half of them in B rows), a thread's piece `it` lies
                // in row row0 + it * RSTEP of B (first half of the iterations)
                // or of C (second half), at column piece `col`: its address is
                // the thread's base plus a uniform step.
                auto split_src = [&](int it, bool &live) -> const uint16_t * {
                    constexpr int RSTEP = NT / S::CPR;
                    const int row0 = tid / S::CPR, col = tid - row0 * S::CPR;
                    const bool isC = it >= S::ITERS / 2;
                    const int n = r * RS + row0 + (isC ? it - S::ITERS / 2 : it) * RSTEP;
                    const int nn = FULL ? n : min(n, dstate - 1);
                    live = FULL || n < dstate;
                    return (isC ? Cbase + nn * p.C_n : Bbase + nn * p.B_n) + blk + 8 * col;
                };
                bool stepped = false;
                if constexpr (fast) {
                    constexpr int BATCH = S::ITERS < 8 ? S::ITERS : 8;
#pragma unroll
                    for (int i0 = 0; i0 < S::ITERS; i0 += BATCH) {
                        u32x4 v[BATCH];
#pragma unroll
                        for (int i = 0; i < BATCH; ++i) {
                            const int q = tid + (i0 + i) * NT;
                            v[i] = u32x4{0u, 0u, 0u, 0u};
                            if (kAllPieces || q < S::PIECES) {
                                bool live;
                                const uint16_t *src = kSplitRows ? split_src(i0 + i, live) : piece_src(q, live);
                                const u32x4 x = *reinterpret_cast<const u32x4 *>(src);
                                v[i] = live ? x : u32x4{0u, 0u, 0u, 0u};
                            }
                        }
                        if (r == 0 && i0 == 0) {
                            steps();
                            stepped = true;
                        }
#pragma unroll
                        for (int i = 0; i < BATCH; ++i) {
                            const int q = tid + (i0 + i) * NT;
                            if (kAllPieces || q < S::PIECES)
                                *reinterpret_cast<u32x4 *>(sBC + 8 * q) = v[i];
                        }
                    }
                } else {
#pragma unroll 1
                    for (int q = tid; q < S::PIECES; q += NT) {
                        bool live;
                        const uint16_t *src = piece_src(q, live);
                        const int64_t t8 = blk + 8 * (q % S::CPR);
                        uint32_t e[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const int64_t t = t8 + j;
                            const uint32_t h = src[(t < p.t1 ? t : p.t1 - 1) - t8];
                            e[j] = (live && t < p.t1) ? h : 0u;
                        }
                        *reinterpret_cast<u32x4 *>(sBC + 8 * q) =
                            u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
                    }
                }
                if (r == 0 && !stepped)
                    steps();
            }
            __syncthreads();

            // this wave's states of the round, in groups of 8 and pairs: the
            // carried values and decay rates come from LDS, the B and C rows
            // of the pair from the staged block, just before they are used
            const int sbase = r * RS + w * NSW;
            const uint16_t *const sB = sBC + (w * NSW) * BLOCK + lane * SEG;
            const uint16_t *const sC = sBC + (RS + w * NSW) * BLOCK + lane * SEG;
            float *const hrow = sH + c * HP + sbase;
            const float *const arow = sA + c * HP + sbase;
#pragma unroll
            for (int gi = 0; gi < GROUPS; ++gi) {
                float yy[SEG];
#pragma unroll
                for (int j = 0; j < SEG; ++j)
                    yy[j] = 0.0f;
                // the group's carried states and decay rates, lane k holding
                // state gi * 8 + k's, read out and written back per state
                // with lane reads and writes
                float hg = lane < kGroup ? hrow[gi * kGroup + lane] : 0.0f;
                const float ag = lane < kGroup ? arow[gi * kGroup + lane] : 0.0f;
#pragma unroll 1
                for (int k = 0; k < kGroup; ++k) {
                    const int n = gi * kGroup + k;
                    const float hv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hg), k));
                    const float av = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ag), k));
                    uint32_t B0[WORDS], C0[WORDS];
                    lds_seg<SEG>(sB + n * BLOCK, B0);
                    lds_seg<SEG>(sC + n * BLOCK, C0);
                    const float hn = scan_state<F16, SEG>(dl, du, dls, av, B0, C0, hv, yy);
                    hg = lane == k ? hn : hg;
                }
                if (lane < kGroup)
                    hrow[gi * kGroup + lane] = hg;
                // the group's partial: added by wave 0 in group order, handed
                // over through LDS by the channel's other waves
                if (w == 0) {
#pragma unroll
                    for (int j = 0; j < SEG; ++j)
                        y[j] = (r == 0 && gi == 0) ? yy[j] : y[j] + yy[j];
                } else if constexpr (W > 1) {
#pragma unroll
                    for (int j = 0; j < SEG; ++j)
                        sY[(((w - 1) * GROUPS + gi) * CPW + c) * BLOCK + lane * SEG + j] = yy[j];
                }
            }

            // every wave is done with this round's rows (and has handed over
            // its partials) before they are overwritten
            if constexpr (NT > kLanes)
                __syncthreads();
            if constexpr (W > 1) {
                if (w == 0) {
                    for (int k = 0; k < (W - 1) * GROUPS; ++k)
#pragma unroll
                        for (int j = 0; j < SEG; ++j)
                            y[j] += sY[(k * CPW + c) * BLOCK + lane * SEG + j];
                }
            }
        }

        if (w == 0) {
            uint16_t o[SEG];
#pragma unroll
            for (int j = 0; j < SEG; ++j)
                o[j] = f32_to_io<F16>(fmaf(Dd, io_to_f32<F16>(half_of<SEG>(uw, j)), y[j]));
            store_seg<SEG, fast>(p.out + b * p.o_b + d * p.o_d, tok, p.t1, o);
        }
    };
    for (int64_t blk = p.t0; blk < p.t1; blk += BLOCK) {
        if (p.vec && blk + BLOCK <= p.t1)
            block(blk, std::true_type{});
        else
            block(blk, std::false_type{});
    }

    // final states: every wave wrote its own to LDS
    __syncthreads();
    for (int i = tid; i < CPW * dstate; i += NT) {
        const int cc = i / dstate, n = i - cc * dstate;
        p.state[b * p.st_b + (d0 + cc) * p.st_d + n] = sH[cc * HP + n];
    }
}

// Launchers: every configuration takes the channel count and sets its own
// grid, workgroup size and LDS.
using ScanFn = hipError_t (*)(const ScanParams &, int64_t channels, hipStream_t);

template <bool F16, int SEG, int NSW, bool FULL>
hipError_t launch_direct(const ScanParams &p, int64_t channels, hipStream_t stream)
{
    const int waves = (p.dstate + NSW - 1) / NSW;
    if constexpr (NSW == 16) {
        if (waves == 1) {  // the one-wave instantiation has the whole register file
            hipLaunchKernelGGL((ssu_scan_direct_kernel<F16, SEG, NSW, 1, FULL>), dim3(channels), dim3(kLanes), 0,
                               stream, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((ssu_scan_direct_kernel<F16, SEG, NSW, kMaxStates / NSW, FULL>), dim3(channels),
                       dim3(waves * kLanes), 0, stream, p);
    return hipGetLastError();
}

template <bool F16, int SEG, int NSW, int W, int CPW, bool FULL>
hipError_t launch_staged(const ScanParams &p, int64_t channels, hipStream_t stream)
{
    using S = ScanShape<SEG, NSW, W, CPW>;
    hipLaunchKernelGGL((ssu_scan_staged_kernel<F16, SEG, NSW, W, CPW, FULL>), dim3(channels / CPW), dim3(S::NT),
                       S::lds_bytes(p.rounds), stream, p);
    return hipGetLastError();
}

// A launch configuration: SEG tokens per lane, NSW states per wave; staged
// ones also W waves per channel and CPW channels per workgroup. rs: states
// per round (per wave for direct ones); ealign: the element alignment (of
// every row start and chunk start) its vector loads need. fn[all rounds
// full][f16].
struct ScanTile {
    int seg, nsw, waves, cpw, rs, ealign;
    bool staged;
    ScanFn fn[2][2];
    char name[32];
};

template <int SEG, int NSW>
ScanTile direct_tile()
{
    ScanTile t{};
    t.seg = SEG, t.nsw = NSW, t.waves = 0, t.cpw = 1, t.rs = NSW, t.ealign = SEG, t.staged = false;
    t.fn[0][0] = &launch_direct<false, SEG, NSW, false>;
    t.fn[0][1] = &launch_direct<true, SEG, NSW, false>;
    t.fn[1][0] = &launch_direct<false, SEG, NSW, true>;
    t.fn[1][1] = &launch_direct<true, SEG, NSW, true>;
    std::snprintf(t.name, sizeof t.name, "scan_t%d_n%d", SEG, NSW);
    return t;
}

template <int SEG, int NSW, int W, int CPW>
ScanTile staged_tile()
{
    ScanTile t{};
    t.seg = SEG, t.nsw = NSW, t.waves = W, t.cpw = CPW, t.rs = W * NSW, t.ealign = 8, t.staged = true;
    t.fn[0][0] = &launch_staged<false, SEG, NSW, W, CPW, false>;
    t.fn[0][1] = &launch_staged<true, SEG, NSW, W, CPW, false>;
    t.fn[1][0] = &launch_staged<false, SEG, NSW, W, CPW, true>;
    t.fn[1][1] = &launch_staged<true, SEG, NSW, W, CPW, true>;
    std::snprintf(t.name, sizeof t.name, "scan_t%d_n%d_w%d_c%d", SEG, NSW, W, CPW);
    return t;
}

template <int SEG>
void add_scan_tiles(ScanTile *&t)
{
    *t++ = direct_tile<SEG, 16>();
    *t++ = direct_tile<SEG, 8>();
    *t++ = staged_tile<SEG, 16, 1, 4>();
    *t++ = staged_tile<SEG, 16, 1, 8>();
    *t++ = staged_tile<SEG, 16, 1, 2>();
    *t++ = staged_tile<SEG, 8, 2, 4>();
}

constexpr int kScanTiles = 24;

const ScanTile *scan_tiles(int *count)
{
    static ScanTile table[kScanTiles];
    static const bool init = [] {
        ScanTile *t = table;
        add_scan_tiles<8>(t);
        add_scan_tiles<4>(t);
        add_scan_tiles<2>(t);
        add_scan_tiles<1>(t);
        return t == table + kScanTiles;
    }();
    (void)init;
    *count = kScanTiles;
    return table;
}

// Default launch configuration, from a sweep of the configurations on MI355X
// (d_state 16, 4096 fp16 tokens per request, 1, 2, 4, 8 and 16 requests of
// 1024 channels, static chunk 512 and one launch, cold caches): the largest
// token segment that a launch still fills (64 lanes x SEG tokens per block);
// then by the number of channels:
//   up to 1024:  the direct kernel, two waves of 8 states per channel (at one
//                request 59.95 us per sequence at chunk 512 against 64.03 for
//                the best staged one: latency bound);
//   up to 2048:  staged, two waves of 8 states per channel, four channels per
//                workgroup (two requests: 85.6 against 108.4 us direct);
//   above:       staged, one wave of 16 states per channel, four channels per
//                workgroup (16 requests: 384.5 against 595.6 us direct, and
//                355.4 against 479.4 us in one launch).
// Where a group's channels do not split into fours, the direct kernel.
constexpr int64_t kDirectChannels = 1024;
constexpr int64_t kTwoWaveChannels = 2048;

int default_scan_tile(int64_t span, int64_t channels, int ch_per_group)
{
    int count = 0;
    const ScanTile *t = scan_tiles(&count);
    int seg = 1;
    for (int sg : {8, 4, 2})
        if (span >= int64_t(kLanes) * sg) {
            seg = sg;
            break;
        }
    const bool staged = channels > kDirectChannels && ch_per_group % 4 == 0;
    const bool two_waves = channels <= kTwoWaveChannels;
    for (int i = 0; i < count; ++i) {
        const ScanTile &x = t[i];
        if (x.seg != seg || x.staged != staged)
            continue;
        if (!staged && x.nsw == 8)
            return i;
        if (staged && x.cpw == 4 && (two_waves ? (x.nsw == 8 && x.waves == 2) : (x.nsw == 16 && x.waves == 1)))
            return i;
    }
    return 0;
}

bool is_io(const ssu_view &v) { return v.dtype == SSU_F16 || v.dtype == SSU_BF16; }

}  // namespace
}  // namespace ssu

extern "C" {

int32_t ssu_scan_tile_count(void)
{
    int count = 0;
    ssu::scan_tiles(&count);
    return count;
}

const char *ssu_scan_tile_name(int32_t tile)
{
    int count = 0;
    const ssu::ScanTile *t = ssu::scan_tiles(&count);
    return (tile >= 0 && tile < count) ? t[tile].name : "";
}

ssu_status ssu_scan(const ssu_scan_args *a, int64_t chunk, int32_t tile, hipStream_t stream)
{
    using namespace ssu;
    if (!a)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: null args");
    int count = 0;
    const ScanTile *tiles = scan_tiles(&count);
    if (tile < -1 || tile >= count)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: tile %d out of range", tile);
    if (chunk < 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: negative chunk %lld", static_cast<long long>(chunk));
    const int32_t bs = a->batch, dim = a->dim, N = a->dstate, G = a->ngroups;
    const int64_t L = a->seqlen;
    if (bs < 0 || dim <= 0 || N <= 0 || G <= 0 || L < 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: bad shape batch %d dim %d dstate %d ngroups %d seqlen %lld",
                    bs, dim, N, G, static_cast<long long>(L));
    if (dim % G)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: dim %d is not a multiple of ngroups %d", dim, G);
    if (N > kMaxStates)
        return fail(SSU_ERR_UNSUPPORTED, "ssu_scan: dstate %d > %d", N, kMaxStates);
    if (static_cast<int64_t>(bs) * dim > 0x7fffffff)
        return fail(SSU_ERR_UNSUPPORTED, "ssu_scan: batch * dim too large");
    if (a->delta_softplus != 0 && a->delta_softplus != 1)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: delta_softplus must be 0 or 1");
    if (a->reserved != 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: reserved field must be 0");
    if (bs == 0)
        return SSU_OK;
    {
        const ssu_view *vs[] = {&a->state, &a->u, &a->delta, &a->B, &a->C, &a->A, &a->D, &a->delta_bias, &a->out};
        const char *names[] = {"state", "u", "delta", "B", "C", "A", "D", "delta_bias", "out"};
        const int rank[] = {3, 3, 3, 4, 4, 2, 1, 1, 3};
        for (int k = 0; k < 9; ++k) {
            if (!vs[k]->ptr)
                continue;
            if (vs[k]->reserved != 0)
                return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: %s: reserved field must be 0", names[k]);
            for (int i = 0; i < rank[k]; ++i)
                if (vs[k]->stride[i] < 0)
                    return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: %s: negative stride[%d]", names[k], i);
        }
    }

    // operands
    if (!a->state.ptr || !a->A.ptr)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: null state or A");
    if (a->state.dtype != SSU_F32 || a->A.dtype != SSU_F32)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: state and A must be F32");
    if (a->state.stride[2] != 1)
        return fail(SSU_ERR_UNSUPPORTED, "ssu_scan: the state's dstate axis must be contiguous");
    for (const ssu_view *v : {&a->D, &a->delta_bias}) {
        if (v->ptr && v->dtype != SSU_F32)
            return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: D and delta_bias must be F32");
        if (v->ptr && dim > 1 && v->stride[0] != 1)
            return fail(SSU_ERR_UNSUPPORTED, "ssu_scan: D and delta_bias must be contiguous");
    }
    for (const ssu_view *v : {&a->state, &a->A, &a->D, &a->delta_bias})
        if (reinterpret_cast<uintptr_t>(v->ptr) % 4)
            return fail(SSU_ERR_MISALIGNED, "ssu_scan: F32 operand not 4-byte aligned");
    if (L > 0) {
        const ssu_view *io[] = {&a->u, &a->delta, &a->B, &a->C, &a->out};
        const char *names[] = {"u", "delta", "B", "C", "out"};
        const int tax[] = {2, 2, 3, 3, 2};  // token axis
        for (int k = 0; k < 5; ++k) {
            if (!io[k]->ptr)
                return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: null %s", names[k]);
            if (!is_io(*io[k]) || io[k]->dtype != a->u.dtype)
                return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_scan: %s must be F16 or BF16, the same as u", names[k]);
            if (io[k]->stride[tax[k]] != 1)
                return fail(SSU_ERR_UNSUPPORTED, "ssu_scan: %s's token axis must be contiguous", names[k]);
            if (reinterpret_cast<uintptr_t>(io[k]->ptr) % 2)
                return fail(SSU_ERR_MISALIGNED, "ssu_scan: %s not 2-byte aligned", names[k]);
        }
    }

    const int ch_per_group = dim / G;
    const int64_t channels = static_cast<int64_t>(bs) * dim;
    const int t = tile >= 0 ? tile : default_scan_tile(chunk > 0 ? std::min(chunk, L) : L, channels, ch_per_group);
    const ScanTile &T = tiles[t];
    if (ch_per_group % T.cpw)
        return fail(SSU_ERR_UNSUPPORTED, "ssu_scan: %s needs the channels of a group (%d) in multiples of %d", T.name,
                    ch_per_group, T.cpw);
    const int rounds = (N + T.rs - 1) / T.rs;

    ScanParams p{};
    p.u = static_cast<const uint16_t *>(a->u.ptr);
    p.delta = static_cast<const uint16_t *>(a->delta.ptr);
    p.B = static_cast<const uint16_t *>(a->B.ptr);
    p.C = static_cast<const uint16_t *>(a->C.ptr);
    p.out = static_cast<uint16_t *>(const_cast<void *>(a->out.ptr));
    p.state = static_cast<float *>(const_cast<void *>(a->state.ptr));
    p.A = static_cast<const float *>(a->A.ptr);
    p.D = static_cast<const float *>(a->D.ptr);
    p.bias = static_cast<const float *>(a->delta_bias.ptr);
    p.u_b = a->u.stride[0], p.u_d = a->u.stride[1];
    p.dl_b = a->delta.stride[0], p.dl_d = a->delta.stride[1];
    p.B_b = a->B.stride[0], p.B_g = a->B.stride[1], p.B_n = a->B.stride[2];
    p.C_b = a->C.stride[0], p.C_g = a->C.stride[1], p.C_n = a->C.stride[2];
    p.o_b = a->out.stride[0], p.o_d = a->out.stride[1];
    p.st_b = a->state.stride[0], p.st_d = a->state.stride[1];
    p.A_d = a->A.stride[0], p.A_n = a->A.stride[1];
    p.dim = dim, p.dstate = N, p.ch_per_group = ch_per_group, p.softplus = a->delta_softplus;
    p.rounds = rounds;

    // Vector access (SEG tokens of a row per lane; for the staged kernel also
    // 16-byte pieces of the B and C rows into LDS) needs every row start and
    // every chunk start on a multiple of T.ealign elements.
    const int64_t ealign = T.ealign;  // in 16-bit elements
    bool vec = true;
    if (L > 0) {
        for (const ssu_view *v : {&a->u, &a->delta, &a->out})
            vec = vec && reinterpret_cast<uintptr_t>(v->ptr) % (2 * ealign) == 0 && v->stride[0] % ealign == 0 &&
                  v->stride[1] % ealign == 0;
        for (const ssu_view *v : {&a->B, &a->C})
            vec = vec && reinterpret_cast<uintptr_t>(v->ptr) % (2 * ealign) == 0 && v->stride[0] % ealign == 0 &&
                  v->stride[1] % ealign == 0 && v->stride[2] % ealign == 0;
    }
    const int64_t step = (chunk > 0 && chunk < L) ? chunk : L;
    const bool f16 = a->u.dtype == SSU_F16;
    const ScanFn fn = T.fn[N % T.rs == 0][f16];
    for (int64_t t0 = 0; t0 < L; t0 += step) {
        p.t0 = t0;
        p.t1 = std::min(L, t0 + step);
        p.vec = vec && (t0 % ealign == 0);
        const hipError_t e = fn(p, channels, stream);
        if (e != hipSuccess)
            return fail(SSU_ERR_HIP, "launch of %s failed: %s", T.name, hipGetErrorString(e));
    }
    return SSU_OK;
}

}  // extern "C"
