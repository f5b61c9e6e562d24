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
// Tokens go in blocks of 32 * T (T = 16, 8, 4 or 2 tokens per lane; 512
// tokens at T = 16). Both halves of a wave (lanes 0-31 and 32-63) see the
// same block: lane i of either half holds the segment of T tokens starting at
// i * T, and the two halves scan two different states of one channel (direct
// and staged kernels) or the same state of two channels (paired kernel), so
// every wave instruction advances two scans at once. Per state the recurrence
// h -> a h + b is a composition of affine maps, and composition is
// associative:
//   1. each lane composes its T pairs (a_j, b_j) into one map (P, Q);
//   2. a 32-lane inclusive scan of the maps in a fixed tree (DPP row shifts
//      1, 2, 4, 8, then lane 15 of each half into the half's second row)
//      gives every lane the map from the block's start to its last token;
//      applied to the carried state it is the state after that token;
//   3. shifted one lane up within the half (the half's first lane takes the
//      carried state) it is each lane's start state g; the lane's state after
//      its token j is its prefix map applied to g, computed by replaying its
//      tokens from g, h_j = a_j h_{j-1} + b_j, and y_j += h_j C_j;
//   4. the half's last lane's end state is the carried state for the next
//      block.
// The carried state is uniform over the half, so blocks, and launches that
// start on a block boundary, continue from exactly the value the previous
// block ended with: chunkings whose chunks are multiples of 32 * T give
// bitwise identical results.
//
// In the direct and staged kernels, work on tokens alone (the step sizes and
// their softplus, the inputs Delta u, the output's D u term and its rounding)
// is not repeated in both halves: of each segment the lower half's lane owns
// the first T/2 tokens and the upper half's lane the last T/2; each computes
// its own tokens' values and the two trade what the other needs with one
// v_permlane32_swap per value.
//
// y is summed in one fixed order whatever the configuration: states in groups
// of 4, each group's partial accumulated in state order (fma), the groups
// added in group order. In the direct and staged kernels a wave takes its
// states in passes of 8: in each pass the lower half scans the first group
// and the upper half the second, one state of each per step. After a pass the
// halves trade partials so that each lane holds both groups' partials for the
// tokens it owns, and adds them in order; partials of a channel's other waves
// are handed over through LDS. In the paired kernel each lane adds its own
// channel's groups as it finishes them. With the same T, every configuration
// and every chunking on block boundaries gives bitwise the same outputs.
//
// Three kernels compute it, with the same fp32 operations in the same order:
//
//   direct (scan_t{T}_n{NSW}): one workgroup per (request, channel), one wave
//     per NSW of its states; each wave loads its states' B and C rows straight
//     into registers, all of a block's loads issued before any is used. Few
//     instructions stand between a launch and its first result, which is what
//     a small batch (a few thousand channels: latency bound) needs.
//   staged (scan_t{T}_n{NSW}_w{W}_c{CPW}): a workgroup holds CPW channels of
//     one (request, group), with W waves of NSW states each. The channels of a
//     group share B and C, so the workgroup stages a block's B and C rows in
//     LDS once, W * NSW states at a time (a round; d_state above that takes
//     several rounds), and each wave reads the rows of the state it is working
//     on just before it needs them, with the carried states and decay rates
//     kept in LDS. Fewer registers are live (three waves fit on each SIMD at
//     T = 16, four below), and the B/C traffic falls by CPW.
//   paired (scan_t{T}_n16_pair_c{2 CPW}): staged in the same way, but each
//     half of a wave holds its own channel over the whole block and walks
//     every state of it, so that nothing is traded between the halves: each
//     lane computes the step sizes of all T tokens of its segment and sums
//     its own partials and outputs. Both halves step through the same state
//     at once and read the same staged rows. Fewest instructions per element:
//     what a large batch (throughput bound) needs.
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
constexpr int kHalf = 32;
constexpr int kMaxStates = 64;
constexpr int kGroup = 4;          // states per partial sum of y
constexpr int kPass = 2 * kGroup;  // states per pass of a wave: a group per half

using u32x4 = uint32_t __attribute__((ext_vector_type(4)));

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

// fp32 to the I/O type, round to nearest even. For fp16 the value is first
// made opaque to the compiler: otherwise it may fuse the fma that produced f
// with this conversion into one mixed-precision instruction that rounds the
// exact result to fp16 once, instead of to fp32 and then to fp16, and whether
// it does so depends on the surrounding code, so configurations would differ
// in the last bit.
template <bool F16>
__device__ __forceinline__ uint16_t f32_to_io(float f)
{
    if constexpr (F16) {
        asm("" : "+v"(f));
        return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // v_cvt_f16_f32
    } else {
        uint32_t w = __float_as_uint(f);
        if ((w & 0x7fffffffu) > 0x7f800000u)
            return static_cast<uint16_t>((w >> 16) | 0x40u);  // NaN stays a quiet NaN
        w += 0x7fffu + ((w >> 16) & 1u);
        return static_cast<uint16_t>(w >> 16);
    }
}

// Tokens tok .. tok+N-1 of a row, packed two per word. FAST: all of them lie
// before t1 and the row is aligned for vector loads. Otherwise each is read
// from an address clamped into [0, t1) (always valid) and tokens at or past t1
// read as 0; the loads stay unconditional, so they issue back to back.
template <int N, bool FAST>
__device__ __forceinline__ void load_seg(const uint16_t *row, int64_t tok, int64_t t1, uint32_t (&w)[(N + 1) / 2])
{
    if constexpr (FAST) {
        const uint16_t *p = row + tok;
        if constexpr (N >= 8) {
#pragma unroll
            for (int q = 0; q < N / 8; ++q) {
                const u32x4 x = *reinterpret_cast<const u32x4 *>(p + 8 * q);
                w[4 * q] = x.x, w[4 * q + 1] = x.y, w[4 * q + 2] = x.z, w[4 * q + 3] = x.w;
            }
        } else if constexpr (N == 4) {
            const auto x = *reinterpret_cast<const u32x2 *>(p);
            w[0] = x.x, w[1] = x.y;
        } else if constexpr (N == 2) {
            w[0] = *reinterpret_cast<const uint32_t *>(p);
        } else {
            w[0] = *p;
        }
    } else {
        uint32_t v[N];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            const int64_t t = tok + j;
            const uint32_t x = row[t < t1 ? t : t1 - 1];
            v[j] = t < t1 ? x : 0u;
        }
#pragma unroll
        for (int k = 0; k < (N + 1) / 2; ++k)
            w[k] = v[2 * k] | ((2 * k + 1 < N) ? (v[2 * k + 1] << 16) : 0u);
    }
}

// Store tokens tok .. tok+N-1 of a row (those before t1).
template <int N, bool FAST>
__device__ __forceinline__ void store_seg(uint16_t *row, int64_t tok, int64_t t1, const uint16_t (&v)[N])
{
    if constexpr (FAST) {
        uint16_t *p = row + tok;
        uint32_t w[(N + 1) / 2];
#pragma unroll
        for (int k = 0; k < (N + 1) / 2; ++k)
            w[k] = v[2 * k] | ((2 * k + 1 < N) ? (static_cast<uint32_t>(v[2 * k + 1]) << 16) : 0u);
        if constexpr (N >= 8) {
#pragma unroll
            for (int q = 0; q < N / 8; ++q) {
                u32x4 x = {w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
                *reinterpret_cast<u32x4 *>(p + 8 * q) = x;
            }
        } else if constexpr (N == 4) {
            u32x2 x = {w[0], w[1]};
            *reinterpret_cast<u32x2 *>(p) = x;
        } else if constexpr (N == 2) {
            *reinterpret_cast<uint32_t *>(p) = w[0];
        } else {
            *p = v[0];
        }
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j)
            if (tok + j < t1)
                row[tok + j] = v[j];
    }
}

// N tokens of a row staged in LDS (16-bit values, packed two per word).
template <int N>
__device__ __forceinline__ void lds_seg(const uint16_t *p, uint32_t (&w)[(N + 1) / 2])
{
    if constexpr (N >= 8) {
#pragma unroll
        for (int q = 0; q < N / 8; ++q) {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(p + 8 * q);
            w[4 * q] = x.x, w[4 * q + 1] = x.y, w[4 * q + 2] = x.z, w[4 * q + 3] = x.w;
        }
    } else if constexpr (N == 4) {
        const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
        w[0] = x.x, w[1] = x.y;
    } else {
        w[0] = *reinterpret_cast<const uint32_t *>(p);
    }
}

template <int N>
__device__ __forceinline__ uint32_t half_of(const uint32_t (&w)[(N + 1) / 2], int j)
{
    return (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu);
}

// The 32-lane inclusive scan of the lanes' maps (P, Q) in each half of the
// wave, for two states at once or for one, as in-place DPP operations: at each
// level every lane combines its map with the map of the lane that the DPP
// control names (the earlier tokens), Q += P * Q_src, then P *= P_src. A lane
// without a source (shifted out of its row, or in a row the row mask leaves
// out) is not written, which is the same as combining with the identity map
// (1, 0). The levels: shifts 1, 2, 4, 8 within rows of 16, then lane 15 of
// each row into the next row, for rows 1 and 3 only (lane 15 into row 1,
// lane 47 into row 3), so that nothing crosses from one half into the other.
// A DPP read needs two wait states after a VALU write of its source register:
// the leading s_nop 1 covers the caller's last writes; between levels, two
// interleaved states already put three instructions between a write and its
// next DPP read, and one state needs an s_nop 0.
#define SSU_SCAN_LEVEL2(CTL)                \
    "v_fmac_f32_dpp %0, %0, %2 " CTL "\n\t" \
    "v_fmac_f32_dpp %1, %1, %3 " CTL "\n\t" \
    "v_mul_f32_dpp %2, %2, %2 " CTL "\n\t"  \
    "v_mul_f32_dpp %3, %3, %3 " CTL "\n\t"
#define SSU_SCAN_TREE2(Q0, Q1, P0, P1)                                              \
    asm("s_nop 1\n\t" SSU_SCAN_LEVEL2("row_shr:1 row_mask:0xf bank_mask:0xf")      \
            SSU_SCAN_LEVEL2("row_shr:2 row_mask:0xf bank_mask:0xf")                  \
                SSU_SCAN_LEVEL2("row_shr:4 row_mask:0xf bank_mask:0xf")              \
                    SSU_SCAN_LEVEL2("row_shr:8 row_mask:0xf bank_mask:0xf")          \
                        SSU_SCAN_LEVEL2("row_bcast:15 row_mask:0xa bank_mask:0xf")   \
        : "+v"(Q0), "+v"(Q1), "+v"(P0), "+v"(P1))
#define SSU_SCAN_LEVEL1(CTL)                \
    "v_fmac_f32_dpp %0, %0, %1 " CTL "\n\t" \
    "v_mul_f32_dpp %1, %1, %1 " CTL "\n\t"
#define SSU_SCAN_TREE1_TEXT                                                                    \
    "s_nop 1\n\t" SSU_SCAN_LEVEL1("row_shr:1 row_mask:0xf bank_mask:0xf") "s_nop 0\n\t"            \
        SSU_SCAN_LEVEL1("row_shr:2 row_mask:0xf bank_mask:0xf") "s_nop 0\n\t"                        \
            SSU_SCAN_LEVEL1("row_shr:4 row_mask:0xf bank_mask:0xf") "s_nop 0\n\t"                    \
                SSU_SCAN_LEVEL1("row_shr:8 row_mask:0xf bank_mask:0xf") "s_nop 0\n\t"                \
                    SSU_SCAN_LEVEL1("row_bcast:15 row_mask:0xa bank_mask:0xf")
#define SSU_SCAN_TREE1(Q0, P0) asm(SSU_SCAN_TREE1_TEXT : "+v"(Q0), "+v"(P0))
// The same, and no memory access moves across it (the caller's loads after
// it stay after it, so their registers are not live during the scan).
#define SSU_SCAN_TREE1_FENCED(Q0, P0) asm(SSU_SCAN_TREE1_TEXT : "+v"(Q0), "+v"(P0) : : "memory")

// DPP control of the one-lane shift of the whole wave (GFX9 encoding).
constexpr int kWaveShr1 = 0x138;

// v_permlane32_swap: lanes 32..63 of x trade places with lanes 0..31 of y.
// With x and y the same per-lane values, the lower half keeps its own value
// in x and receives the upper half's in y; the upper half receives the lower
// half's in x and keeps its own in y.
__device__ __forceinline__ void swap_halves(float &x, float &y)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    x = __uint_as_float(r[0]);
    y = __uint_as_float(r[1]);
}

// The value of the last lane of this lane's half (lane 31 or lane 63), in
// every lane of the half.
__device__ __forceinline__ float half_last(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_ds_bpermute(((lane & kHalf) | (kHalf - 1)) << 2, __float_as_int(v)));
}

// One state per half over one block of 32 * T tokens, in this lane's segment
// of T tokens: dl their step sizes, du = dl * u their inputs, dls = the sum of
// dl (in token order), Bw and Cw the state's B and C bits, A2 = A * log2(e),
// h the carried state (uniform over the half), half_first: this lane is its
// half's first (lane 0 or 32). Adds the state's h_j * C_j to yy[j] and
// returns the lane's end state e (the half's last lane holds the carried
// state after the block).
//   1. the lane's whole map: decay exp2(A2 * dls) (the product of its
//      tokens' decays in one exponential), and the state Q reached from 0;
//   2. the 32-lane inclusive scan of the maps;
//   3. the lane's end state e (the map applied to h) and start state g (e
//      shifted one lane up; the half's first lane takes h instead); the
//      lane's tokens are replayed from g, h_j = a_j h_{j-1} + b_j, and after
//      its last token the state is e.
// after_scan() is called once the step no longer needs A2, Bw and h (after
// the 32-lane scan, which no memory access crosses when FENCED): a caller
// that reads the next step's operands from LDS there has them in flight
// while this step's tokens are replayed, in the registers this step's have
// just freed.
// FIRST: the pass's first state, whose terms start yy (yy[j] = h_j C_j + 0,
// the same bits as adding them to yy = +0).
template <bool F16, int T, bool FENCED = false, bool FIRST = false, typename AfterScan>
__device__ __forceinline__ float scan_step(const float (&dl)[T], const float (&du)[T], float dls, float A2,
                                           const uint32_t (&Bw)[(T + 1) / 2], const uint32_t (&Cw)[(T + 1) / 2],
                                           float h, bool half_first, float (&yy)[T], AfterScan after_scan)
{
    float a[T], b[T];
#pragma unroll
    for (int j = 0; j < T; ++j) {
        a[j] = __builtin_amdgcn_exp2f(dl[j] * A2);
        b[j] = fmaf(du[j], io_to_f32<F16>(half_of<T>(Bw, j)), 0.0f);
    }
    float Q = b[0];
#pragma unroll
    for (int j = 1; j < T; ++j)
        Q = fmaf(a[j], Q, b[j]);
    float P = __builtin_amdgcn_exp2f(dls * A2);
    if constexpr (FENCED)
        SSU_SCAN_TREE1_FENCED(Q, P);
    else
        SSU_SCAN_TREE1(Q, P);
    const float e = fmaf(P, h, Q);
    float g = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(e), kWaveShr1, 0xf, 0xf, true));
    g = half_first ? h : g;
    if constexpr (FENCED)
        asm volatile("" : "+v"(g) : : "memory");  // h is dead before after_scan's reads
    after_scan();
    float hj = g;
#pragma unroll
    for (int j = 0; j < T - 1; ++j) {
        hj = fmaf(a[j], hj, b[j]);
        yy[j] = fmaf(hj, io_to_f32<F16>(half_of<T>(Cw, j)), FIRST ? 0.0f : yy[j]);
    }
    yy[T - 1] = fmaf(e, io_to_f32<F16>(half_of<T>(Cw, T - 1)), FIRST ? 0.0f : yy[T - 1]);
    return e;
}

// The same for two states per half at once (their dependent steps
// interleave), with the same operations per state, so the same bits. y gets
// the first state's terms before the second's.
template <bool F16, int T>
__device__ __forceinline__ void scan_step2(const float (&dl)[T], const float (&du)[T], float dls, float A20,
                                           float A21, const uint32_t (&B0)[(T + 1) / 2],
                                           const uint32_t (&B1)[(T + 1) / 2], const uint32_t (&C0)[(T + 1) / 2],
                                           const uint32_t (&C1)[(T + 1) / 2], float h0, float h1, bool half_first,
                                           float (&yy)[T], float &e0, float &e1)
{
    float a0[T], b0[T], a1[T], b1[T];
#pragma unroll
    for (int j = 0; j < T; ++j) {
        a0[j] = __builtin_amdgcn_exp2f(dl[j] * A20);
        a1[j] = __builtin_amdgcn_exp2f(dl[j] * A21);
        b0[j] = fmaf(du[j], io_to_f32<F16>(half_of<T>(B0, j)), 0.0f);
        b1[j] = fmaf(du[j], io_to_f32<F16>(half_of<T>(B1, j)), 0.0f);
    }
    float Q0 = b0[0], Q1 = b1[0];
#pragma unroll
    for (int j = 1; j < T; ++j) {
        Q0 = fmaf(a0[j], Q0, b0[j]);
        Q1 = fmaf(a1[j], Q1, b1[j]);
    }
    float P0 = __builtin_amdgcn_exp2f(dls * A20), P1 = __builtin_amdgcn_exp2f(dls * A21);
    SSU_SCAN_TREE2(Q0, Q1, P0, P1);
    e0 = fmaf(P0, h0, Q0);
    e1 = fmaf(P1, h1, Q1);
    float g0 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(e0), kWaveShr1, 0xf, 0xf, true));
    float g1 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(e1), kWaveShr1, 0xf, 0xf, true));
    g0 = half_first ? h0 : g0;
    g1 = half_first ? h1 : g1;
    float hj0 = g0, hj1 = g1;
#pragma unroll
    for (int j = 0; j < T - 1; ++j) {
        hj0 = fmaf(a0[j], hj0, b0[j]);
        hj1 = fmaf(a1[j], hj1, b1[j]);
        yy[j] = fmaf(hj0, io_to_f32<F16>(half_of<T>(C0, j)), yy[j]);
        yy[j] = fmaf(hj1, io_to_f32<F16>(half_of<T>(C1, j)), yy[j]);
    }
    yy[T - 1] = fmaf(e0, io_to_f32<F16>(half_of<T>(C0, T - 1)), yy[T - 1]);
    yy[T - 1] = fmaf(e1, io_to_f32<F16>(half_of<T>(C1, T - 1)), yy[T - 1]);
}

// The sum of a segment's step sizes, in token order.
template <int T>
__device__ __forceinline__ float step_sum(const float (&dl)[T])
{
    float s = dl[0];
#pragma unroll
    for (int j = 1; j < T; ++j)
        s += dl[j];
    return s;
}

// Step sizes Delta and inputs Delta u of the T/2 tokens this lane owns (from
// their delta and u bits dw, uw; tokens at or past t1: the identity), traded
// between the halves into the whole segment's dl[T], du[T].
template <bool F16, int T, bool FAST>
__device__ __forceinline__ void segment_steps(const uint32_t (&dw)[(T / 2 + 1) / 2],
                                              const uint32_t (&uw)[(T / 2 + 1) / 2], float bias, bool softplus,
                                              int64_t own, int64_t t1, float (&dl)[T], float (&du)[T])
{
    constexpr int TH = T / 2;
#pragma unroll
    for (int j = 0; j < TH; ++j) {
        // (the f16 conversions fold into mixed-precision fmas; x * 1 + bias
        // and sv * u + 0 round exactly as x + bias and sv * u)
        const float v = fmaf(io_to_f32<F16>(half_of<TH>(dw, j)), 1.0f, bias);
        float sv = softplus ? softplus_f32(v) : v;
        if (!FAST)
            sv = own + j < t1 ? sv : 0.0f;
        float x = sv, y = sv;
        swap_halves(x, y);
        dl[j] = x, dl[TH + j] = y;
        float xu = fmaf(sv, io_to_f32<F16>(half_of<TH>(uw, j)), 0.0f), yu = xu;
        swap_halves(xu, yu);
        du[j] = xu, du[TH + j] = yu;
    }
}

// Step sizes Delta and inputs Delta u of all T tokens of this lane's segment
// (from their delta and u bits; tokens at or past t1: the identity), computed
// in the lane itself: the same operations as segment_steps, so the same bits.
template <bool F16, int T, bool FAST>
__device__ __forceinline__ void lane_steps(const uint32_t (&dw)[(T + 1) / 2], const uint32_t (&uw)[(T + 1) / 2],
                                           float bias, bool softplus, int64_t own, int64_t t1, float (&dl)[T],
                                           float (&du)[T])
{
#pragma unroll
    for (int j = 0; j < T; ++j) {
        const float v = fmaf(io_to_f32<F16>(half_of<T>(dw, j)), 1.0f, bias);
        float sv = softplus ? softplus_f32(v) : v;
        if (!FAST)
            sv = own + j < t1 ? sv : 0.0f;
        dl[j] = sv;
        du[j] = fmaf(sv, io_to_f32<F16>(half_of<T>(uw, j)), 0.0f);
    }
}

// After a pass, yy holds the lower group's partial in the lower half and the
// upper group's in the upper half, over the whole segment. Trade them so
// that each lane holds both partials of its own T/2 tokens, and add them to
// y in group order.
template <int T>
__device__ __forceinline__ void pass_partials(const float (&yy)[T], float (&lo)[T / 2], float (&hi)[T / 2])
{
    constexpr int TH = T / 2;
#pragma unroll
    for (int j = 0; j < TH; ++j) {
        float x = yy[j], z = yy[TH + j];
        swap_halves(x, z);
        lo[j] = x, hi[j] = z;
    }
}

// ONEB: the launch's tokens fit in one block (whole and aligned): that block
// alone, its loads in the order of use (see below).
template <bool F16, int T, int NSW, int MAXW, bool FULL, bool ALLFAST, bool ONEB = false>
__global__ void __launch_bounds__(kLanes * MAXW) ssu_scan_direct_kernel(const ScanParams p)
{
    static_assert(!ONEB || ALLFAST, "a one-block launch takes the aligned path");
    constexpr int TH = T / 2, BLOCK = kHalf * T, WT = (T + 1) / 2, WH = (TH + 1) / 2;
    constexpr int STEPS = NSW / 2;          // states per half of the wave
    constexpr int GROUPS = NSW / kGroup;
    // group partials of waves 1 .. W-1, by own token
    __shared__ float ypart[MAXW > 1 ? (MAXW - 1) * GROUPS : 1][MAXW > 1 ? BLOCK : 1];

    const int lane = static_cast<int>(threadIdx.x) & (kLanes - 1);
    const int li = lane & (kHalf - 1), hl = lane >> 5;
    const bool half_first = li == 0;
    const int wave = MAXW > 1 ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kLanes) : 0;
    const int nwaves = MAXW > 1 ? static_cast<int>(blockDim.x) / kLanes : 1;
    const int64_t bd = blockIdx.x;
    const int64_t b = bd / p.dim;
    const int d = static_cast<int>(bd - b * p.dim);
    const int grp = d / p.ch_per_group;
    const int n0 = wave * NSW;
    const int dstate = p.dstate;

    const uint16_t *const u_row = p.u + b * p.u_b + d * p.u_d;
    const uint16_t *const dl_row = p.delta + b * p.dl_b + d * p.dl_d;
    const uint16_t *const B_row = p.B + b * p.B_b + grp * p.B_g;
    const uint16_t *const C_row = p.C + b * p.C_b + grp * p.C_g;
    uint16_t *const o_row = p.out + b * p.o_b + d * p.o_d;
    float *const st = p.state + b * p.st_b + d * p.st_d;
    const float bias = p.bias ? load_ro(p.bias + d) : 0.0f;
    const float Dd = p.D ? load_ro(p.D + d) : 0.0f;
    const bool softplus = p.softplus != 0;

    // this half's state of step s: n0 + 8 (s / 4) + 4 hl + s % 4; its carried
    // value (read with a plain load: the state is written by this kernel) and
    // decay rate A * log2(e), both uniform over the half, read in the first
    // block after its rows are requested (one memory wait, not two in a row)
    int row[STEPS];
    bool live[STEPS];
    float hv[STEPS], A2[STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
        const int n = n0 + kPass * (s / kGroup) + kGroup * hl + s % kGroup;
        live[s] = FULL || n < dstate;
        row[s] = FULL ? n : min(n, dstate - 1);  // rows past dstate: read a valid row, zeroed below
        hv[s] = A2[s] = 0.0f;
    }
    const bool vec = p.vec != 0;

    auto block = [&](int64_t blk, auto fast_tag) {
        constexpr bool fast = decltype(fast_tag)::value;
        const int64_t seg = blk + li * T, own = seg + hl * TH;

        // every load of the block first. In a one-block launch in the order
        // of use: u and delta (the step sizes), the carried states and decay
        // rates, then the B and C rows step by step; vector-memory counters
        // retire in order, so the step sizes start once u and delta are in
        // and each step waits only for its own rows (the scheduling barriers
        // keep the compiler from reordering the groups): such a launch's
        // loads all come from far memory and nothing else hides them.
        // Otherwise all of a block's loads are issued before any is used, so
        // that one wait covers them, and in the first block the states and
        // rates follow them.
        uint32_t uw[WH], dw[WH], Bw[STEPS][WT], Cw[STEPS][WT];
        float hraw[STEPS], araw[STEPS];
        if constexpr (ONEB) {
            load_seg<TH, fast>(u_row, own, p.t1, uw);
            load_seg<TH, fast>(dl_row, own, p.t1, dw);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                hraw[s] = st[row[s]];
                araw[s] = load_ro(p.A + d * p.A_d + row[s] * p.A_n);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                load_seg<T, fast>(B_row + row[s] * p.B_n, seg, p.t1, Bw[s]);
                load_seg<T, fast>(C_row + row[s] * p.C_n, seg, p.t1, Cw[s]);
            }
            __builtin_amdgcn_sched_barrier(0);
        } else {
            load_seg<TH, fast>(u_row, own, p.t1, uw);
            load_seg<TH, fast>(dl_row, own, p.t1, dw);
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                load_seg<T, fast>(B_row + row[s] * p.B_n, seg, p.t1, Bw[s]);
                load_seg<T, fast>(C_row + row[s] * p.C_n, seg, p.t1, Cw[s]);
            }
            if (blk == p.t0) {
#pragma unroll
                for (int s = 0; s < STEPS; ++s) {
                    const float h = st[row[s]], av = load_ro(p.A + d * p.A_d + row[s] * p.A_n);
                    hv[s] = live[s] ? h : 0.0f;
                    A2[s] = live[s] ? av * kLog2e : 0.0f;
                }
            }
        }
        // states past d_state read a valid row; their B and C count as zero
        if constexpr (!FULL) {
#pragma unroll
            for (int s = 0; s < STEPS; ++s)
#pragma unroll
                for (int k = 0; k < WT; ++k) {
                    Bw[s][k] = live[s] ? Bw[s][k] : 0u;
                    Cw[s][k] = live[s] ? Cw[s][k] : 0u;
                }
        }
        float dl[T], du[T];
        segment_steps<F16, T, fast>(dw, uw, bias, softplus, own, p.t1, dl, du);
        const float dls = step_sum<T>(dl);
        if constexpr (ONEB) {
#pragma unroll
            for (int s = 0; s < STEPS; ++s) {
                hv[s] = live[s] ? hraw[s] : 0.0f;
                A2[s] = live[s] ? araw[s] * kLog2e : 0.0f;
            }
        }

        // y of the tokens this lane owns: starting from -0 (which adds exactly),
        // the groups' partials added in group order
        float y[TH];
#pragma unroll
        for (int j = 0; j < TH; ++j)
            y[j] = -0.0f;
#pragma unroll
        for (int ps = 0; ps < STEPS; ps += kGroup) {
            float yy[T];
#pragma unroll
            for (int j = 0; j < T; ++j)
                yy[j] = 0.0f;
            if constexpr (NSW == 8 && (T <= 8 || ALLFAST)) {  // (the ragged-block code leaves no room for two at T = 16)
#pragma unroll
                for (int s = ps; s < ps + kGroup; s += 2) {
                    float e0, e1;
                    scan_step2<F16, T>(dl, du, dls, A2[s], A2[s + 1], Bw[s], Bw[s + 1], Cw[s], Cw[s + 1], hv[s],
                                       hv[s + 1], half_first, yy, e0, e1);
                    hv[s] = half_last(e0, lane);
                    hv[s + 1] = half_last(e1, lane);
                }
            } else {
#pragma unroll
                for (int s = ps; s < ps + kGroup; ++s) {
                    const float e =
                        scan_step<F16, T>(dl, du, dls, A2[s], Bw[s], Cw[s], hv[s], half_first, yy, [] {});
                    hv[s] = half_last(e, lane);
                }
            }
            float lo[TH], hi[TH];
            pass_partials<T>(yy, lo, hi);
            const int gi = 2 * (ps / kGroup);  // the pass's first group within the wave
#pragma unroll
            for (int j = 0; j < TH; ++j) {
                if (wave == 0) {
                    y[j] = (y[j] + lo[j]) + hi[j];
                } else if constexpr (MAXW > 1) {
                    ypart[(wave - 1) * GROUPS + gi][li * T + hl * TH + j] = lo[j];
                    ypart[(wave - 1) * GROUPS + gi + 1][li * T + hl * TH + j] = hi[j];
                }
            }
        }
        if constexpr (MAXW > 1) {
            __syncthreads();
            if (wave == 0) {
                for (int k = 0; k < (nwaves - 1) * GROUPS; ++k)
#pragma unroll
                    for (int j = 0; j < TH; ++j)
                        y[j] += ypart[k][li * T + hl * TH + j];
            }
            __syncthreads();
        }
        if (wave == 0) {
            uint16_t o[TH];
#pragma unroll
            for (int j = 0; j < TH; ++j)
                o[j] = f32_to_io<F16>(fmaf(Dd, io_to_f32<F16>(half_of<TH>(uw, j)), y[j]));
            store_seg<TH, fast>(o_row, own, p.t1, o);
        }
    };
    if constexpr (ONEB) {
        if (p.t0 < p.t1)
            block(p.t0, std::true_type{});
    } else {
        for (int64_t blk = p.t0; blk < p.t1; blk += BLOCK) {
            if constexpr (ALLFAST) {
                block(blk, std::true_type{});
            } else {
                if (vec && blk + BLOCK <= p.t1)
                    block(blk, std::true_type{});
                else
                    block(blk, std::false_type{});
            }
        }
    }

    // final states: the first lane of each half writes its half's
    if (li == 0) {
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
            if (live[s])
                st[row[s]] = hv[s];
    }
}

// Stage round r's B and C rows of one block into LDS: RS rows of B then RS
// of C, BLOCK tokens each from token blk, as 16-byte pieces spread over the
// workgroup's NT threads (piece q lands at sBC + 8 q). FAST: the block lies
// inside the chunk with aligned rows, so every thread requests all its
// pieces (at most eight at a time) before writing any; otherwise each piece
// is built from clamped 16-bit reads, one at a time, and tokens at or past t1
// read as 0. Rows past d_state are staged as zeros. first() runs once: while
// the first batch of pieces is in flight (FAST), or after the last piece.
// When the pieces divide evenly (every thread stages the same number, half
// of them in B rows), a thread's piece `it` lies in row row0 + it * RSTEP of
// B (first half) or of C (second half) at its fixed column piece, so with
// every state live its address is a uniform row pointer plus the thread's
// fixed byte offset (offB, offC; the host keeps RS row strides below 2^30
// elements).
template <int BLOCK, int RS, int NT, bool FULL, bool FAST, typename First>
__device__ __forceinline__ void stage_rows(uint16_t *sBC, const uint16_t *Bbase, const uint16_t *Cbase, int64_t B_n,
                                           int64_t C_n, int64_t blk, int64_t t1, int r, int dstate, int tid,
                                           uint32_t offB, uint32_t offC, First first)
{
    constexpr int CPR = BLOCK / 8, PIECES = 2 * RS * CPR, ITERS = (PIECES + NT - 1) / NT;
    constexpr bool kAllPieces = PIECES % NT == 0;
    constexpr bool kSplitRows = kAllPieces && ITERS % 2 == 0 && NT % CPR == 0;
    auto piece_src = [&](int q, bool &live) -> const uint16_t * {
        const int row = q / CPR, k = q - row * CPR;
        const bool isC = row >= RS;
        const int n = r * RS + (isC ? row - RS : row);
        const int nn = FULL ? n : min(n, dstate - 1);
        live = FULL || n < dstate;
        return (isC ? Cbase + nn * C_n : Bbase + nn * B_n) + blk + 8 * k;
    };
    auto split_src = [&](int it, bool &live) -> const uint16_t * {
        constexpr int RSTEP = NT / CPR;
        const bool isC = it >= ITERS / 2;
        const int nb = r * RS + (isC ? it - ITERS / 2 : it) * RSTEP;  // the piece's row for row0 = 0
        if constexpr (FULL) {
            live = true;
            const uint16_t *rowp = (isC ? Cbase + nb * C_n : Bbase + nb * B_n) + blk;
            return reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(rowp) + (isC ? offC : offB));
        } else {
            const int row0 = tid / CPR, col = tid - row0 * CPR;
            const int n = nb + row0;
            const int nn = min(n, dstate - 1);
            live = n < dstate;
            return (isC ? Cbase + nn * C_n : Bbase + nn * B_n) + blk + 8 * col;
        }
    };
    if constexpr (FAST) {
        constexpr int BATCH = ITERS < 8 ? ITERS : 8;
#pragma unroll
        for (int i0 = 0; i0 < ITERS; i0 += BATCH) {
            u32x4 v[BATCH];
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                const int q = tid + (i0 + i) * NT;
                v[i] = u32x4{0u, 0u, 0u, 0u};
                if (kAllPieces || q < PIECES) {
                    bool live;
                    const uint16_t *src = kSplitRows ? split_src(i0 + i, live) : piece_src(q, live);
                    const u32x4 x = *reinterpret_cast<const u32x4 *>(src);
                    v[i] = live ? x : u32x4{0u, 0u, 0u, 0u};
                }
            }
            if (i0 == 0)
                first();
#pragma unroll
            for (int i = 0; i < BATCH; ++i) {
                const int q = tid + (i0 + i) * NT;
                if (kAllPieces || q < PIECES)
                    *reinterpret_cast<u32x4 *>(sBC + 8 * q) = v[i];
            }
        }
    } else {
#pragma unroll 1
        for (int q = tid; q < PIECES; q += NT) {
            bool live;
            const uint16_t *src = piece_src(q, live);
            const int64_t t8 = blk + 8 * (q % CPR);
            uint32_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t t = t8 + j;
                const uint32_t h = src[(t < t1 ? t : t1 - 1) - t8];
                e[j] = (live && t < t1) ? h : 0u;
            }
            *reinterpret_cast<u32x4 *>(sBC + 8 * q) =
                u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
        }
        first();
    }
}

// Layout of one workgroup's LDS (dynamic, 16-byte aligned):
//   sBC [2 * RS][BLOCK] u16      the round's B rows, then its C rows;
//   sY  [W - 1][GROUPS][CPW][BLOCK] f32  partials of y (by own token) that
//                                        waves 1 .. W-1 of each channel hand
//                                        to wave 0;
//   sH  [CPW][rounds * RS] f32   the carried states (0 past d_state);
//   sA  [CPW][rounds * RS] f32   A * log2(e) (0 past d_state);
//   16 bytes of padding (read, never used).
template <int T, int NSW, int W, int CPW>
struct ScanShape {
    static constexpr int BLOCK = kHalf * T;
    static constexpr int RS = W * NSW;            // states per round
    static constexpr int GROUPS = NSW / kGroup;
    static constexpr int NT = kLanes * W * CPW;   // threads
    static constexpr int CPR = BLOCK / 8;         // 16-byte pieces per staged row
    static constexpr int PIECES = 2 * RS * CPR;   // per round
    static constexpr int ITERS = (PIECES + NT - 1) / NT;
    static constexpr size_t BC_BYTES = size_t(2) * RS * BLOCK * 2;
    static constexpr size_t Y_BYTES = size_t(W - 1) * GROUPS * CPW * BLOCK * 4;
    // (+16: a step reads the next state's operands one past the last)
    static size_t lds_bytes(int rounds) { return BC_BYTES + Y_BYTES + size_t(2) * CPW * rounds * RS * 4 + 16; }
};

template <bool F16, int T, int NSW, int W, int CPW, bool FULL, bool ALLFAST>
__global__ void __launch_bounds__(kLanes * W * CPW) __attribute__((amdgpu_waves_per_eu(T >= 16 ? 3 : 4)))
ssu_scan_staged_kernel(const ScanParams p)
{
    using S = ScanShape<T, NSW, W, CPW>;
    constexpr int TH = T / 2, BLOCK = S::BLOCK, WT = (T + 1) / 2, WH = (TH + 1) / 2;
    constexpr int RS = S::RS, GROUPS = S::GROUPS, NT = S::NT;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *const sBC = reinterpret_cast<uint16_t *>(smem);
    float *const sY = reinterpret_cast<float *>(smem + S::BC_BYTES);
    float *const sH = reinterpret_cast<float *>(smem + S::BC_BYTES + S::Y_BYTES);
    const int rounds = p.rounds;
    const int HP = rounds * RS;
    float *const sA = sH + CPW * HP;

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & (kLanes - 1);
    const int li = lane & (kHalf - 1), hl = lane >> 5;
    const bool half_first = li == 0;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kLanes);  // uniform: pointers below stay scalar
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
    // read with plain loads, never through the read-only path) and the decay
    // rates A * log2(e); in the first block, after its staging loads are
    // requested (one memory wait, not two in a row)
    auto load_states = [&]() {
        for (int i = tid; i < CPW * HP; i += NT) {
            const int cc = i / HP, n = i - cc * HP;
            const int nn = FULL ? n : min(n, dstate - 1);
            const float *st = p.state + b * p.st_b + (d0 + cc) * p.st_d;
            const float av = load_ro(p.A + (d0 + cc) * p.A_d + nn * p.A_n);
            sH[i] = (FULL || n < dstate) ? st[nn] : 0.0f;
            sA[i] = (FULL || n < dstate) ? av * kLog2e : 0.0f;
        }
    };

    // Byte offset of a thread's staging pieces from the row of the first
    // thread (rows row0 = tid / CPR, column piece tid % CPR), when the pieces
    // split evenly; the host keeps RS row strides below 2^30 elements.
    const uint32_t split_offB = static_cast<uint32_t>(
        ((tid / S::CPR) * p.B_n + 8 * (tid % S::CPR)) * 2);
    const uint32_t split_offC = static_cast<uint32_t>(
        ((tid / S::CPR) * p.C_n + 8 * (tid % S::CPR)) * 2);
    const int lown = li * T + hl * TH;  // this lane's own tokens, from the block's start

    // One block of tokens. FAST: the block lies inside the chunk and every
    // row is aligned for vector access, so every load is an unconditional
    // vector load; otherwise each token is read from an address clamped into
    // the chunk and tokens past its end read as 0.
    auto block = [&](int64_t blk, auto fast_tag) {
        constexpr bool fast = decltype(fast_tag)::value;
        const int64_t own = blk + lown;

        // this lane's step sizes and inputs (requested before the staging waits)
        uint32_t uw[WH], dw[WH];
        if constexpr (fast) {
            load_seg<TH, true>(u_row + blk, lown, 0, uw);
            load_seg<TH, true>(dl_row + blk, lown, 0, dw);
        } else {
            load_seg<TH, false>(u_row, own, p.t1, uw);
            load_seg<TH, false>(dl_row, own, p.t1, dw);
        }
        float dl[T], du[T], y[TH], dls = 0.0f;
#pragma unroll
        for (int j = 0; j < TH; ++j)
            y[j] = -0.0f;

        auto steps = [&]() {
            segment_steps<F16, T, fast>(dw, uw, bias, softplus, own, p.t1, dl, du);
            dls = step_sum<T>(dl);
        };

        for (int r = 0; r < rounds; ++r) {
            // stage the round's B and C rows into LDS (and, in the first
            // round, compute the step sizes while the pieces are in flight)
            stage_rows<BLOCK, RS, NT, FULL, fast>(sBC, Bbase, Cbase, p.B_n, p.C_n, blk, p.t1, r, dstate, tid,
                                                   split_offB, split_offC, [&] {
                                                       if (r == 0) {
                                                           if (blk == p.t0)
                                                               load_states();
                                                           steps();
                                                       }
                                                   });
            __syncthreads();

            // this wave's states of the round, in passes of two groups: the
            // carried values and decay rates come from LDS, the B and C rows
            // from the staged block, just before they are used
            const int sbase = w * NSW + kGroup * hl;  // this half's first state of the wave's first pass
            const uint16_t *const sB = sBC + li * T;
            const uint16_t *const sC = sBC + RS * BLOCK + li * T;
            float *const hrow = sH + c * HP + r * RS;
            const float *const arow = sA + c * HP + r * RS;
#pragma unroll 1
            for (int ps = 0; ps < NSW; ps += kPass) {
                // a step's carried value, decay rate and B row are read from
                // LDS while the step before replays its tokens; its C row at
                // its own start
                float yy[T];
                const int n0 = sbase + ps;
                float hv = hrow[n0], av = arow[n0];
                uint32_t Bw[WT];
                lds_seg<T>(sB + n0 * BLOCK, Bw);
                auto step = [&](int k, auto first_tag) {
                    const int n = n0 + k;  // this half's state, within the round
                    const int nx = n + 1;  // past the pass's last: read, unused (LDS has a padding word)
                    uint32_t Cw[WT];
                    lds_seg<T>(sC + n * BLOCK, Cw);
                    const float e = scan_step<F16, T, true, decltype(first_tag)::value>(
                        dl, du, dls, av, Bw, Cw, hv, half_first, yy, [&] {
                            hv = hrow[nx];
                            av = arow[nx];
                            lds_seg<T>(sB + nx * BLOCK, Bw);
                        });
                    if (li == kHalf - 1)
                        hrow[n] = e;
                };
                step(0, std::true_type{});
#pragma unroll 1
                for (int k = 1; k < kGroup; ++k)
                    step(k, std::false_type{});
                // the pass's partials: added by wave 0 in group order, handed
                // over through LDS by the channel's other waves
                float lo[TH], hi[TH];
                pass_partials<T>(yy, lo, hi);
                const int gi = 2 * (ps / kPass);
                if (w == 0) {
#pragma unroll
                    for (int j = 0; j < TH; ++j)
                        y[j] = (y[j] + lo[j]) + hi[j];
                } else if constexpr (W > 1) {
#pragma unroll
                    for (int j = 0; j < TH; ++j) {
                        sY[(((w - 1) * GROUPS + gi) * CPW + c) * BLOCK + li * T + hl * TH + j] = lo[j];
                        sY[(((w - 1) * GROUPS + gi + 1) * CPW + c) * BLOCK + li * T + hl * TH + j] = hi[j];
                    }
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
                        for (int j = 0; j < TH; ++j)
                            y[j] += sY[(k * CPW + c) * BLOCK + li * T + hl * TH + j];
                }
            }
        }

        if (w == 0) {
            // u again for the D u term (read at the block's start, not kept
            // in registers across the scan)
            uint32_t uo[WH];
            uint16_t o[TH];
            if constexpr (fast)
                load_seg<TH, true>(u_row + blk, lown, 0, uo);
            else
                load_seg<TH, false>(u_row, own, p.t1, uo);
#pragma unroll
            for (int j = 0; j < TH; ++j)
                o[j] = f32_to_io<F16>(fmaf(Dd, io_to_f32<F16>(half_of<TH>(uo, j)), y[j]));
            if constexpr (fast)
                store_seg<TH, true>(p.out + b * p.o_b + d * p.o_d + blk, lown, 0, o);
            else
                store_seg<TH, false>(p.out + b * p.o_b + d * p.o_d, own, p.t1, o);
        }
    };
    for (int64_t blk = p.t0; blk < p.t1; blk += BLOCK) {
        if constexpr (ALLFAST) {
            block(blk, std::true_type{});
        } else {
            if (p.vec && blk + BLOCK <= p.t1)
                block(blk, std::true_type{});
            else
                block(blk, std::false_type{});
        }
    }

    // final states: every wave wrote its own to LDS
    __syncthreads();
    for (int i = tid; i < CPW * dstate; i += NT) {
        const int cc = i / dstate, n = i - cc * dstate;
        p.state[b * p.st_b + (d0 + cc) * p.st_d + n] = sH[cc * HP + n];
    }
}

// Layout of a paired workgroup's LDS (dynamic, 16-byte aligned):
//   sBC [2 * RS][BLOCK] u16      the round's B rows, then its C rows;
//   sH  [NCH][rounds * RS] f32   the carried states (0 past d_state);
//   sA  [NCH][rounds * RS] f32   A * log2(e) (0 past d_state);
//   16 bytes of padding (read, never used).
template <int T, int RS, int CPW>
struct PairShape {
    static constexpr int BLOCK = kHalf * T;
    static constexpr int NCH = 2 * CPW;        // channels: one per half-wave
    static constexpr int NT = kLanes * CPW;    // threads
    static constexpr size_t BC_BYTES = size_t(2) * RS * BLOCK * 2;
    static size_t lds_bytes(int rounds) { return BC_BYTES + size_t(2) * NCH * rounds * RS * 4 + 16; }
};

// The paired kernel: a workgroup holds 2 * CPW channels of one (request,
// group) in CPW waves; each half of a wave holds one channel, over the whole
// block (lane i: tokens i * T .. i * T + T - 1), and walks every state of it,
// RS states per round with the round's B and C rows staged in LDS as in the
// staged kernel. Both halves step through the same state at once, so they
// read the same staged rows. Nothing crosses from one half into the other:
// each lane computes the step sizes of its own segment and adds its own
// partials, in the same order as the other kernels (yy over a group of 4
// states by fma in state order, then y += yy in group order), so the results
// are bitwise those of the other kernels with the same T.
template <bool F16, int T, int RS, int CPW, bool FULL, bool ALLFAST>
__global__ void __launch_bounds__(kLanes * CPW) __attribute__((amdgpu_waves_per_eu(T >= 16 ? 3 : 4)))
ssu_scan_paired_kernel(const ScanParams p)
{
    using S = PairShape<T, RS, CPW>;
    constexpr int BLOCK = S::BLOCK, NT = S::NT, NCH = S::NCH, WT = (T + 1) / 2;
    constexpr int CPR = BLOCK / 8;  // 16-byte pieces per staged row
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    uint16_t *const sBC = reinterpret_cast<uint16_t *>(smem);
    float *const sH = reinterpret_cast<float *>(smem + S::BC_BYTES);
    const int rounds = p.rounds;
    const int HP = rounds * RS;
    float *const sA = sH + NCH * HP;

    const int tid = static_cast<int>(threadIdx.x);
    const int lane = tid & (kLanes - 1);
    const int li = lane & (kHalf - 1), hl = lane >> 5;
    const bool half_first = li == 0;
    const int wv = __builtin_amdgcn_readfirstlane(tid / kLanes);
    const int c = 2 * wv + hl;  // this half's channel slot
    const int64_t bd0 = static_cast<int64_t>(blockIdx.x) * NCH;
    const int64_t b = bd0 / p.dim;  // every channel of the group shares it
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

    // carried states (plain loads: this kernel writes the state) and decay
    // rates A * log2(e) into LDS, in the first block after its staging loads
    // are requested
    auto load_states = [&]() {
        for (int i = tid; i < NCH * HP; i += NT) {
            const int cc = i / HP, n = i - cc * HP;
            const int nn = FULL ? n : min(n, dstate - 1);
            const float *st = p.state + b * p.st_b + (d0 + cc) * p.st_d;
            const float av = load_ro(p.A + (d0 + cc) * p.A_d + nn * p.A_n);
            sH[i] = (FULL || n < dstate) ? st[nn] : 0.0f;
            sA[i] = (FULL || n < dstate) ? av * kLog2e : 0.0f;
        }
    };

    const uint32_t split_offB = static_cast<uint32_t>(((tid / CPR) * p.B_n + 8 * (tid % CPR)) * 2);
    const uint32_t split_offC = static_cast<uint32_t>(((tid / CPR) * p.C_n + 8 * (tid % CPR)) * 2);
    const int lown = li * T;  // this lane's tokens, from the block's start
    const uint16_t *const sB = sBC + lown;
    const uint16_t *const sC = sBC + RS * BLOCK + lown;

    auto block = [&](int64_t blk, auto fast_tag) {
        constexpr bool fast = decltype(fast_tag)::value;
        const int64_t own = blk + lown;

        uint32_t uw[WT], dw[WT];
        if constexpr (fast) {
            load_seg<T, true>(u_row + blk, lown, 0, uw);
            load_seg<T, true>(dl_row + blk, lown, 0, dw);
        } else {
            load_seg<T, false>(u_row, own, p.t1, uw);
            load_seg<T, false>(dl_row, own, p.t1, dw);
        }
        float dl[T], du[T], y[T], dls = 0.0f;
#pragma unroll
        for (int j = 0; j < T; ++j)
            y[j] = -0.0f;

        for (int r = 0; r < rounds; ++r) {
            stage_rows<BLOCK, RS, NT, FULL, fast>(sBC, Bbase, Cbase, p.B_n, p.C_n, blk, p.t1, r, dstate, tid,
                                                   split_offB, split_offC, [&] {
                                                       if (r == 0) {
                                                           if (blk == p.t0)
                                                               load_states();
                                                           lane_steps<F16, T, fast>(dw, uw, bias, softplus, own,
                                                                                    p.t1, dl, du);
                                                           dls = step_sum<T>(dl);
                                                       }
                                                   });
            __syncthreads();

            // the round's states in groups of 4; a step's carried value, decay
            // rate and B row are read from LDS while the step before replays
            // its tokens, its C row at its own start
            float *const hrow = sH + c * HP + r * RS;
            const float *const arow = sA + c * HP + r * RS;
#pragma unroll 1
            for (int n0 = 0; n0 < RS; n0 += kGroup) {
                float yy[T];
                float hv = hrow[n0], av = arow[n0];
                uint32_t Bw[WT];
                lds_seg<T>(sB + n0 * BLOCK, Bw);
                auto step = [&](int k, auto first_tag) {
                    const int n = n0 + k;
                    const int nx = n + 1;  // past the round's last: read, unused (LDS has a padding word)
                    uint32_t Cw[WT];
                    lds_seg<T>(sC + n * BLOCK, Cw);
                    const float e = scan_step<F16, T, true, decltype(first_tag)::value>(
                        dl, du, dls, av, Bw, Cw, hv, half_first, yy, [&] {
                            hv = hrow[nx];
                            av = arow[nx];
                            lds_seg<T>(sB + nx * BLOCK, Bw);
                        });
                    if (li == kHalf - 1)
                        hrow[n] = e;
                };
                step(0, std::true_type{});
#pragma unroll 1
                for (int k = 1; k < kGroup; ++k)
                    step(k, std::false_type{});
#pragma unroll
                for (int j = 0; j < T; ++j)
                    y[j] += yy[j];
            }
            // every wave is done with this round's rows before they are
            // overwritten
            __syncthreads();
        }

        // u again for the D u term
        uint32_t uo[WT];
        uint16_t o[T];
        if constexpr (fast)
            load_seg<T, true>(u_row + blk, lown, 0, uo);
        else
            load_seg<T, false>(u_row, own, p.t1, uo);
#pragma unroll
        for (int j = 0; j < T; ++j)
            o[j] = f32_to_io<F16>(fmaf(Dd, io_to_f32<F16>(half_of<T>(uo, j)), y[j]));
        if constexpr (fast)
            store_seg<T, true>(p.out + b * p.o_b + d * p.o_d + blk, lown, 0, o);
        else
            store_seg<T, false>(p.out + b * p.o_b + d * p.o_d, own, p.t1, o);
    };
    for (int64_t blk = p.t0; blk < p.t1; blk += BLOCK) {
        if constexpr (ALLFAST) {
            block(blk, std::true_type{});
        } else {
            if (p.vec && blk + BLOCK <= p.t1)
                block(blk, std::true_type{});
            else
                block(blk, std::false_type{});
        }
    }

    // final states: every half wrote its own to LDS
    __syncthreads();
    for (int i = tid; i < NCH * dstate; i += NT) {
        const int cc = i / dstate, n = i - cc * dstate;
        p.state[b * p.st_b + (d0 + cc) * p.st_d + n] = sH[cc * HP + n];
    }
}

// Launchers: every configuration takes the channel count and sets its own
// grid, workgroup size and LDS.
using ScanFn = hipError_t (*)(const ScanParams &, int64_t channels, hipStream_t);

template <bool F16, int T, int NSW, bool FULL, bool ALLFAST>
hipError_t launch_direct(const ScanParams &p, int64_t channels, hipStream_t stream)
{
    const int waves = (p.dstate + NSW - 1) / NSW;
    if constexpr (NSW == 16) {
        if (waves == 1) {  // the one-wave instantiation has the whole register file
            if constexpr (ALLFAST) {
                if (p.t1 - p.t0 <= static_cast<int64_t>(kHalf) * T) {  // one block
                    hipLaunchKernelGGL((ssu_scan_direct_kernel<F16, T, NSW, 1, FULL, true, true>), dim3(channels),
                                       dim3(kLanes), 0, stream, p);
                    return hipGetLastError();
                }
            }
            hipLaunchKernelGGL((ssu_scan_direct_kernel<F16, T, NSW, 1, FULL, ALLFAST>), dim3(channels), dim3(kLanes),
                               0, stream, p);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((ssu_scan_direct_kernel<F16, T, NSW, kMaxStates / NSW, FULL, ALLFAST>), dim3(channels),
                       dim3(waves * kLanes), 0, stream, p);
    return hipGetLastError();
}

template <bool F16, int T, int NSW, int W, int CPW, bool FULL, bool ALLFAST>
hipError_t launch_staged(const ScanParams &p, int64_t channels, hipStream_t stream)
{
    using S = ScanShape<T, NSW, W, CPW>;
    hipLaunchKernelGGL((ssu_scan_staged_kernel<F16, T, NSW, W, CPW, FULL, ALLFAST>), dim3(channels / CPW),
                       dim3(S::NT), S::lds_bytes(p.rounds), stream, p);
    return hipGetLastError();
}

template <bool F16, int T, int RS, int CPW, bool FULL, bool ALLFAST>
hipError_t launch_paired(const ScanParams &p, int64_t channels, hipStream_t stream)
{
    using S = PairShape<T, RS, CPW>;
    hipLaunchKernelGGL((ssu_scan_paired_kernel<F16, T, RS, CPW, FULL, ALLFAST>), dim3(channels / S::NCH),
                       dim3(S::NT), S::lds_bytes(p.rounds), stream, p);
    return hipGetLastError();
}

// A launch configuration: T tokens per lane, NSW states per wave; staged ones
// also W waves per channel and CPW channels per workgroup. rs: states per
// round (per wave for direct ones); ealign: the element alignment (of every
// row start and chunk start) its vector loads need. fn[all rounds
// full][f16][every block whole and aligned]: the last kernel has no code
// for ragged or unaligned blocks, so fewer registers.
struct ScanTile {
    int seg, nsw, waves, cpw, rs, ealign;
    bool staged, paired;
    ScanFn fn[2][2][2];
    char name[32];
};

template <bool FULL, bool F16, bool ALLFAST, int T, int NSW>
void set_direct(ScanTile &t)
{
    t.fn[FULL][F16][ALLFAST] = &launch_direct<F16, T, NSW, FULL, ALLFAST>;
}

template <bool FULL, bool F16, bool ALLFAST, int T, int NSW, int W, int CPW>
void set_staged(ScanTile &t)
{
    t.fn[FULL][F16][ALLFAST] = &launch_staged<F16, T, NSW, W, CPW, FULL, ALLFAST>;
}

template <bool FULL, bool F16, bool ALLFAST, int T, int RS, int CPW>
void set_paired(ScanTile &t)
{
    t.fn[FULL][F16][ALLFAST] = &launch_paired<F16, T, RS, CPW, FULL, ALLFAST>;
}

// Direct loads: a lane's own T/2 tokens of u, delta and out, its T-token
// segment of each B and C row (16-byte vectors at most). Staged ones copy
// 16-byte pieces of B and C.
template <int T, int NSW>
ScanTile direct_tile()
{
    ScanTile t{};
    t.seg = T, t.nsw = NSW, t.waves = 0, t.cpw = 1, t.rs = NSW, t.ealign = T < 8 ? T : 8, t.staged = false;
    set_direct<false, false, false, T, NSW>(t), set_direct<false, false, true, T, NSW>(t);
    set_direct<false, true, false, T, NSW>(t), set_direct<false, true, true, T, NSW>(t);
    set_direct<true, false, false, T, NSW>(t), set_direct<true, false, true, T, NSW>(t);
    set_direct<true, true, false, T, NSW>(t), set_direct<true, true, true, T, NSW>(t);
    std::snprintf(t.name, sizeof t.name, "scan_t%d_n%d", T, NSW);
    return t;
}

template <int T, int NSW, int W, int CPW>
ScanTile staged_tile()
{
    ScanTile t{};
    t.seg = T, t.nsw = NSW, t.waves = W, t.cpw = CPW, t.rs = W * NSW, t.ealign = 8, t.staged = true;
    set_staged<false, false, false, T, NSW, W, CPW>(t), set_staged<false, false, true, T, NSW, W, CPW>(t);
    set_staged<false, true, false, T, NSW, W, CPW>(t), set_staged<false, true, true, T, NSW, W, CPW>(t);
    set_staged<true, false, false, T, NSW, W, CPW>(t), set_staged<true, false, true, T, NSW, W, CPW>(t);
    set_staged<true, true, false, T, NSW, W, CPW>(t), set_staged<true, true, true, T, NSW, W, CPW>(t);
    std::snprintf(t.name, sizeof t.name, "scan_t%d_n%d_w%d_c%d", T, NSW, W, CPW);
    return t;
}

// Paired ones: rs states per round, cpw = 2 * CPW channels per workgroup (one
// per half-wave); each lane loads and stores its whole T-token segment.
template <int T, int RS, int CPW>
ScanTile paired_tile()
{
    ScanTile t{};
    t.seg = T, t.nsw = RS, t.waves = 1, t.cpw = 2 * CPW, t.rs = RS, t.ealign = 8, t.staged = true, t.paired = true;
    set_paired<false, false, false, T, RS, CPW>(t), set_paired<false, false, true, T, RS, CPW>(t);
    set_paired<false, true, false, T, RS, CPW>(t), set_paired<false, true, true, T, RS, CPW>(t);
    set_paired<true, false, false, T, RS, CPW>(t), set_paired<true, false, true, T, RS, CPW>(t);
    set_paired<true, true, false, T, RS, CPW>(t), set_paired<true, true, true, T, RS, CPW>(t);
    std::snprintf(t.name, sizeof t.name, "scan_t%d_n%d_pair_c%d", T, RS, 2 * CPW);
    return t;
}

template <int T>
void add_scan_tiles(ScanTile *&t)
{
    *t++ = direct_tile<T, 16>();
    *t++ = direct_tile<T, 8>();
    *t++ = staged_tile<T, 16, 1, 4>();
    *t++ = staged_tile<T, 16, 1, 8>();
    *t++ = staged_tile<T, 16, 1, 2>();
    *t++ = staged_tile<T, 8, 2, 4>();
    *t++ = paired_tile<T, 16, 4>();
}

constexpr int kScanTiles = 28;

const ScanTile *scan_tiles(int *count)
{
    static ScanTile table[kScanTiles];
    static const bool init = [] {
        ScanTile *t = table;
        add_scan_tiles<16>(t);
        add_scan_tiles<8>(t);
        add_scan_tiles<4>(t);
        add_scan_tiles<2>(t);
        return t == table + kScanTiles;
    }();
    (void)init;
    *count = kScanTiles;
    return table;
}

// Default launch configuration, from a sweep of the configurations on MI355X
// (d_state 16, 4096 fp16 tokens per request, 1, 2, 4, 8 and 16 requests of
// 1024 channels, static chunks 128 to 4096 and one launch, cold caches): the
// largest token segment that a launch still fills (32 lanes x T tokens per
// block); then by the number of channels:
//   up to 1024:  the direct kernel, one wave of 16 states per channel (one
//                request: 59.7 us per sequence at chunk 512 and 33.4 in one
//                launch, against 64.6 and 35.7 with two waves of 8 states;
//                staged the same at chunks up to 512, slower above: 41.5
//                against 38.9 at chunk 2048, 38.3 against 33.4 in one launch;
//                paired 81.7 and 60.4);
//   up to 2048:  staged, four channels per workgroup, where a launch spans at
//                most 1024 tokens (two requests: 77.1 against 80.3 us at
//                chunk 512, 65.0 against 66.4 at 1024, 114.4 against 117.4 at
//                256, 189.8 against 200.6 at 128); direct above (57.6 against
//                56.5 at chunk 2048, 53.9 against 50.4 in one launch; paired
//                86.4 and 62.6);
//   above:       paired, eight channels per workgroup (16 requests: 330.5
//                and 301.4 us, against 352.7 and 323.4 staged with four
//                channels per workgroup and 390.5 and 335.2 direct; 8
//                requests: 195.4 and 162.2 against 200.1 and 169.9; four
//                channels per workgroup: 439.3 and 415.4, LDS holds too few
//                workgroups; at chunks of 256, 128 and 64 tokens, 16 requests,
//                7%, 5% and 13% faster than staged).
// Where a group's channels do not split into eights, staged with four
// channels per workgroup, and where they do not split into fours either, the
// direct kernel. Configurations that stage B and C rows need their row
// strides to fit 32-bit offsets (staged_rows_fit); otherwise direct.
constexpr int64_t kDirectChannels = 1024, kStagedChannels = 2048, kStagedSpan = 1024;
// A launch of one block with up to 16 states per channel (one wave): the
// direct kernel's one-block instantiation, up to this many channels
// (measured against staged and paired at 2 to 16 requests of 1024 channels,
// d_state 16, 2 to 16 tokens per lane).
constexpr int64_t kOneBlockDirectChannels = 8192;

// The staged and paired kernels address a thread's staging pieces as a 32-bit
// byte offset from a row pointer, over at most kMaxStates rows of B and of C.
bool staged_rows_fit(int64_t B_n, int64_t C_n)
{
    return std::max(B_n, C_n) < (int64_t(1) << 30) / kMaxStates;
}

int default_scan_tile(int64_t span, int64_t channels, int ch_per_group, int dstate, bool staged_ok)
{
    int count = 0;
    const ScanTile *t = scan_tiles(&count);
    int seg = 2;
    for (int sg : {16, 8, 4})
        if (span >= int64_t(kHalf) * sg) {
            seg = sg;
            break;
        }
    const bool one_block = span <= int64_t(kHalf) * seg && channels <= kOneBlockDirectChannels && dstate <= 16;
    const bool wide = staged_ok && !one_block &&
                      (channels > kStagedChannels || (channels > kDirectChannels && span <= kStagedSpan));
    const bool paired = wide && channels > kStagedChannels && ch_per_group % 8 == 0;
    const bool staged = wide && !paired && ch_per_group % 4 == 0;
    for (int i = 0; i < count; ++i) {
        const ScanTile &x = t[i];
        if (x.seg != seg || x.nsw != 16)
            continue;
        if (paired ? (x.paired && x.cpw == 8)
                   : staged ? (x.staged && !x.paired && x.cpw == 4 && x.waves == 1) : !x.staged)
            return i;
    }
    return 0;
}

// The default for a call (sizes already checked): by the span of one launch,
// the channels, the channels per group and B's and C's state strides.
int default_scan_tile(const ssu_scan_args &a, int64_t chunk)
{
    const int64_t L = a.seqlen;
    return default_scan_tile(chunk > 0 ? std::min(chunk, L) : L, static_cast<int64_t>(a.batch) * a.dim,
                             a.dim / a.ngroups, static_cast<int>(a.dstate), staged_rows_fit(a.B.stride[2], a.C.stride[2]));
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

int32_t ssu_scan_select_tile(const ssu_scan_args *a, int64_t chunk)
{
    if (!a || chunk < 0 || a->batch < 0 || a->dim <= 0 || a->ngroups <= 0 || a->seqlen < 0 || a->dim % a->ngroups ||
        a->B.stride[2] < 0 || a->C.stride[2] < 0)
        return -1;
    return ssu::default_scan_tile(*a, chunk);
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
    const bool staged_ok = staged_rows_fit(a->B.stride[2], a->C.stride[2]);
    const int t = tile >= 0 ? tile : default_scan_tile(*a, chunk);
    const ScanTile &T = tiles[t];
    if (ch_per_group % T.cpw)
        return fail(SSU_ERR_UNSUPPORTED, "ssu_scan: %s needs the channels of a group (%d) in multiples of %d", T.name,
                    ch_per_group, T.cpw);
    if (T.staged && !staged_ok)
        return fail(SSU_ERR_UNSUPPORTED, "ssu_scan: %s needs the B and C state strides below %lld elements", T.name,
                    static_cast<long long>((int64_t(1) << 30) / kMaxStates));
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

    // Vector access (a lane's tokens of each row; for the staged kernel also
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
    const bool full = N % T.rs == 0;
    const int64_t block = int64_t(kHalf) * T.seg;
    // Each chunk: its whole, aligned blocks in one launch of the kernel
    // without the ragged-block code, then what is left (a ragged tail, or a
    // chunk that is not aligned) in one launch of the general kernel. The
    // state is carried between the two as between chunks, and the blocks are
    // the same, so the split changes no bit of the result.
    auto launch = [&](int64_t t0, int64_t t1, bool v, bool allfast) -> ssu_status {
        p.t0 = t0, p.t1 = t1, p.vec = v;
        const hipError_t e = T.fn[full][f16][allfast](p, channels, stream);
        if (e != hipSuccess)
            return fail(SSU_ERR_HIP, "launch of %s failed: %s", T.name, hipGetErrorString(e));
        return SSU_OK;
    };
    for (int64_t t0 = 0; t0 < L; t0 += step) {
        const int64_t t1 = std::min(L, t0 + step);
        const bool v = vec && (t0 % ealign == 0);
        const int64_t tf = v ? t0 + (t1 - t0) / block * block : t0;  // end of the whole blocks
        if (tf > t0)
            if (const ssu_status st = launch(t0, tf, true, true); st != SSU_OK)
                return st;
        if (t1 > tf)
            if (const ssu_status st = launch(tf, t1, v, false); st != SSU_OK)
                return st;
    }
    return SSU_OK;
}

}  // extern "C"
