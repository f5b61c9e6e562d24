// ssu.hip -- libssu: the Mamba2 decode-step selective_state_update for AMD
// Instinct MI355X (gfx950), behind the C ABI declared in include/ssu.h.
//
// What one call computes (sglang PR #41223, "[Perf] Mamba2
// selective_state_update up to 2x faster on B200 via 8x1 launch config for
// dstate 128", sections "Summary" and "Kernel measurement"): for each request
// b and head h, gather the fp32 state slot idx[b], advance it by one token in
// place, and emit out[b,h,:] in bf16. The page calls the kernel memory bound:
// every step reads and writes each request's fp32 state once, and a launch
// that gives each thread little state to move cannot keep HBM busy.
//
// Kernel design (gfx950, wave64):
//   * One workgroup owns `rows_per_group` consecutive state rows p of one
//     (b, h). A row of N fp32 values is split over LPR lanes with one 16-byte
//     (dwordx4) chunk each (two chunks 512 bytes apart when N = 256), so one
//     wave instruction moves 64 x 16 B of contiguous state and RPI = 64/LPR
//     rows at once. Each lane issues all R of its row loads before using any,
//     so R dwordx4 loads per lane are in flight.
//   * B and C: the column -> lane map is the same for every row, so each lane
//     needs only its own 4 (or 8) values of B and C. They are loaded once per
//     workgroup straight into registers as fp32 and reused for every row; LDS
//     would only add a round trip.
//   * dt', dA, D are per-(b,h) scalars computed once per lane at the start.
//   * out[p] = sum_n S'[p,n] C[n]: each lane sums its own columns in order
//     (an fma chain), then the LPR lanes of a row combine in a fixed butterfly
//     (DPP quad permutes, row half-mirror, row mirror, then a swizzle across
//     the two 16-lane rows), taken as a reduce-scatter over a lane's rows so
//     that each level adds only the rows the lane keeps. A row's order depends
//     only on N, never on the tile, so every tile gives bitwise-identical
//     results, and no atomics are used.
//   * No MFMA: 2 flops of update and 2 of contraction per 8 bytes of state is
//     far below the vector-ALU ridge; the bound is HBM bandwidth.
//   * Optional XCD-aware ordering: workgroups are dispatched round-robin over
//     the 8 XCDs; remapping gives neighbouring heads of one request (which
//     share B, C, x and idx cache lines) the same XCD and its L2.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <initializer_list>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <type_traits>
#include <utility>
#include <vector>

#include "internal.h"

namespace ssu {

struct Params {
    float *state;
    int64_t s_slot, s_head, s_row;
    const void *idx;
    int64_t pool_slots;
    // per-token operands: strides over (request, token, head|group); the token
    // stride is 0 for one-token calls
    const uint16_t *x;
    int64_t x_b, x_t, x_h;
    const uint16_t *B;
    int64_t B_b, B_t, B_g;
    const uint16_t *C;
    int64_t C_b, C_t, C_g;
    const uint32_t *dt_words;  // dt's base rounded down to 4 bytes
    int64_t dt_b, dt_t, dt_h, dt_off;  // dt_off: 1 if the base was 2 bytes past a word
    const float *dt_bias;
    int64_t dtb_h;
    const float *A;
    int64_t A_h;
    const float *D;
    int64_t D_h;
    uint16_t *out;
    int64_t o_b, o_t, o_h;
    int32_t nheads, heads_per_group, ptiles, softplus;
    int32_t idx64, xcd_remap, total_groups, ntokens;
};

// ---------------------------------------------------------------- device --

// fp32 -> bf16, round to nearest even (gfx950's v_cvt_pk_bf16_f32; NaN stays
// NaN). Kept opaque to the compiler so that it is never fused with the fma
// that produces its operand.
__device__ __forceinline__ uint16_t bf16_round(float f)
{
    asm volatile("" : "+v"(f));
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Butterfly partner of level k (0-based) within an aligned group of LPR
// lanes: lane ^ 1, lane ^ 2 (quad permutes), the mirror of each 8 and of each
// 16 lanes (row half-mirror, row mirror), then lane ^ 16 within 32 (swizzle,
// bitmask mode). Any value summed over these five pairings in this order gets
// the same bits in every lane of the group.
template <int K>
__device__ __forceinline__ float partner(float v)
{
    if constexpr (K == 0)
        return dpp<0xB1>(v);  // quad_perm [1,0,3,2]
    else if constexpr (K == 1)
        return dpp<0x4E>(v);  // quad_perm [2,3,0,1]
    else if constexpr (K == 2)
        return dpp<0x141>(v);  // row_half_mirror: lane i <-> 7 - i of each 8
    else if constexpr (K == 3)
        return dpp<0x140>(v);  // row_mirror: lane i <-> 15 - i of each 16
    else
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

// Which half of its rows a lane keeps at reduce-scatter level k: a function
// of the lane's bits that differs between the level's two partners and agrees
// between the partners of every other level (level 2 pairs lanes that differ
// in bits 0-2, level 3 in bits 0-3), so a lane and its partner always hold
// the same rows, and after the last level all lanes that share a row hold it.
__device__ __forceinline__ bool keep_upper(int lane, int k)
{
    const int b0 = lane & 1, b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1, b3 = (lane >> 3) & 1;
    switch (k) {
    case 0: return (b0 ^ b2) != 0;
    case 1: return (b1 ^ b2) != 0;
    case 2: return (b2 ^ b3) != 0;
    default: return b3 != 0;
    }
}

// a if sel, else b, as a bit blend: straight-line code that the compiler
// cannot turn into a dynamically indexed load from the caller's array (which
// it would have to place in memory).
__device__ __forceinline__ float pick(bool sel, float a, float b)
{
    const uint32_t m = 0u - static_cast<uint32_t>(sel);
    return __uint_as_float((__float_as_uint(a) & m) | (__float_as_uint(b) & ~m));
}

// base + off bytes, for a uniform base and a per-lane 32-bit byte offset: the
// offset stays a 32-bit value at the access, so the access can take the base
// from scalar registers and the offset from one vector register (no 64-bit
// address arithmetic per access).
// A pointer that is the same in every lane, held in scalar registers.
template <typename T>
__device__ __forceinline__ T *uniform_ptr(T *ptr)
{
    const uint64_t v = reinterpret_cast<uint64_t>(ptr);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    using G = __attribute__((address_space(1))) T;  // global memory: global, not flat, accesses
    return (T *)reinterpret_cast<G *>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <typename T>
__device__ __forceinline__ T *lane_at(T *base, uint32_t off)
{
    asm volatile("" : "+v"(off));  // (volatile: not hoisted into a loop-carried address)
    using C = std::conditional_t<std::is_const_v<T>, const char, char>;
    return reinterpret_cast<T *>(reinterpret_cast<C *>(base) + off);
}

// Sums of R rows, each split over an aligned group of LPR lanes (LPR in
// 4..32, R in 1..16), as a reduce-scatter: at level k every lane keeps half of
// its rows, adds its partner's partial of each kept row and sends the other
// half, until one row per lane is left (or R / LPR rows when R > LPR); the
// levels that remain sum that row as a plain butterfly. Each row's total is
// the sum over the same pairings in the same order as summing the row alone
// (fp32 addition commutes), so its bits do not depend on R. On return y[0 ..
// KEEP) hold the totals of rows first(lane) + i, and the lanes with
// writer(lane) hold each row once.
//
// With 32 lanes per row the first level pairs lane i with i ^ 16 through
// v_permlane16_swap, which exchanges the odd 16-lane rows of one register
// with the even rows of another: given a pair of rows (lo, hi), the lower
// 16 lanes get their partner's lo beside their own and the upper 16 their
// partner's hi, so the two registers' sum is the kept row in every lane, with
// no select. The other levels go from the widest pairing to the narrowest
// (row mirror, half-row mirror, quad permutes), and the choice of kept rows
// at level k is bit (4, 3, 2^3, 1)[k] of the lane. With 4 to 16 lanes per row
// the levels go the other way (quad permutes, half-row mirror, row mirror) and
// the choice is keep_upper().
template <int LPR, int R>
struct RowSums {
    static constexpr int log2(int v) { return v <= 1 ? 0 : 1 + log2(v / 2); }
    static constexpr int LEVELS = log2(LPR);
    static constexpr int SPLIT = log2(R) < LEVELS ? log2(R) : LEVELS;
    static constexpr int KEEP = R >> SPLIT;
    static constexpr bool WIDE = LPR == 32;
    static_assert(LPR >= 4 && LPR <= 32 && (LPR & (LPR - 1)) == 0, "LPR");
    static_assert(R >= 1 && R <= 16 && (R & (R - 1)) == 0, "R");

    // lane masks of the 32-lane levels, widest first
    static constexpr int wide_mask(int k) { return k == 0 ? 16 : k == 1 ? 15 : k == 2 ? 7 : k == 3 ? 2 : 1; }
    // With 32 lanes per row, lanes that end up holding the same rows differ
    // only in these bits (the remaining levels' masks, a suffix of 16, 15, 7,
    // 2, 1, span exactly the bits below their widest).
    static constexpr int plain_bits()
    {
        int m = 0;
        for (int k = SPLIT; k < LEVELS; ++k)
            m |= wide_mask(k);
        return m;
    }

    __device__ __forceinline__ static bool keeps_upper(int lane, int k)
    {
        if constexpr (WIDE) {
            const int b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1, b3 = (lane >> 3) & 1, b4 = (lane >> 4) & 1;
            return (k == 0 ? b4 : k == 1 ? b3 : k == 2 ? (b2 ^ b3) : b1) != 0;
        } else {
            return keep_upper(lane, k);
        }
    }

    // The first of the rows a lane holds at the end: a function of its bits.
    __device__ __forceinline__ static int first(int lane)
    {
        int f = 0;
#pragma unroll
        for (int k = 0; k < SPLIT; ++k)
            f += keeps_upper(lane, k) ? (R >> (k + 1)) : 0;
        return f;
    }

    // One lane of each group that holds the same rows (c = the lane within
    // its row group). With fewer lanes per row, lanes c < R hold rows first(c)
    // one to one.
    __device__ __forceinline__ static bool writer(int c)
    {
        if constexpr (WIDE)
            return (c & plain_bits()) == 0;
        else
            return R >= LPR || c < R;
    }

    template <int K>
    __device__ __forceinline__ static float wide_partner(float v)
    {
        static_assert(K >= 1 && K <= 4, "level");
        if constexpr (K == 1)
            return dpp<0x140>(v);  // row_mirror: lane i <-> 15 - i of each 16
        else if constexpr (K == 2)
            return dpp<0x141>(v);  // row_half_mirror: lane i <-> 7 - i of each 8
        else if constexpr (K == 3)
            return dpp<0x4E>(v);   // quad_perm [2,3,0,1]
        else
            return dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    }

    template <int K>
    __device__ __forceinline__ static float level_partner(float v)
    {
        if constexpr (WIDE)
            return wide_partner<K>(v);
        else
            return partner<K>(v);
    }

    // the sum of a pair's kept row in every lane (see above)
    __device__ __forceinline__ static float swap16_sum(float lo, float hi)
    {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
        return __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }

    template <int K>
    __device__ __forceinline__ static void level(float (&y)[R], int lane)
    {
        if constexpr (K < LEVELS) {
            if constexpr (WIDE && K == 0) {
                if constexpr (SPLIT > 0) {
                    constexpr int HALF = R / 2;
#pragma unroll
                    for (int i = 0; i < HALF; ++i)
                        y[i] = swap16_sum(y[i], y[i + HALF]);
                } else {
                    y[0] = swap16_sum(y[0], y[0]);
                }
            } else if constexpr (K < SPLIT) {
                constexpr int HALF = R >> (K + 1);
                const bool up = keeps_upper(lane, K);
#pragma unroll
                for (int i = 0; i < HALF; ++i) {
                    const float lo = y[i], hi = y[i + HALF];
                    const float send = pick(up, lo, hi);
                    y[i] = pick(up, hi, lo) + level_partner<K>(send);
                }
            } else {
#pragma unroll
                for (int i = 0; i < KEEP; ++i)
                    y[i] += level_partner<K>(y[i]);
            }
            level<K + 1>(y, lane);
        }
    }

    __device__ __forceinline__ static void run(float (&y)[R], int lane) { level<0>(y, lane); }
};

// One lane's share of one tile: `rows_per_group` consecutive state rows of one
// (request, head), split over the workgroup's waves (R row groups of RPI rows
// per wave). fetch() requests every operand the lane needs for token 0;
// step() waits for them, advances the state in registers by one token and
// emits that token's out; the state goes back to memory after the last token.
// finish() is the one-token case.
template <int N, int R, bool NT>
struct Work {
    static constexpr int VEC = N > 128 ? N / 128 : 1;  // 16-byte chunks per lane per row
    static constexpr int LPR = N / (4 * VEC);          // lanes per row
    static constexpr int RPI = 64 / LPR;               // rows per wave instruction
    static constexpr int ROWS_WAVE = RPI * R;
    static_assert(LPR >= 4 && LPR <= 32, "dstate");

    using RS = RowSums<LPR, R>;

    bool live;
    int b, h, grp, c, sub, wrow, p0, fr;
    const uint16_t *xh;  // x of this wave's first row, token 0 (uniform)
    uint16_t *oh;        // out of this wave's first row, token 0 (uniform)
    float *sp;
    int64_t jstep;
    f32x4 s[R][VEC];
    uint32_t dtbits;
    uint32_t dtlane, dtshift;  // LANEDT: the word holding the dt of token `lane`, its bit offset
    float bias, Ah, Dh;

    // One token's operands for this lane: its columns of B and C (bf16
    // pairs), the x of its rows and of the rows whose out it writes. The x
    // words hold the bf16 in the upper half (the fp32 value it stands for),
    // except those read by the lane's own 16-bit loads (XRAW, XORAW), which
    // hold it in the lower half until step() uses them: a value shifted where
    // it is loaded would make the wave wait for that load (and for the state
    // loads issued before it) before anything else, e.g. the discretisation
    // of the first tokens, could run.
    static constexpr bool XRAW = RPI != 2;
    static constexpr bool XORAW = XRAW || R >= 8;
    struct Ops {
        u32x2 Bw[VEC], Cw[VEC];
        uint32_t xbits[R];
        uint32_t xo[R >= 8 ? RS::KEEP : 1];  // R >= 8: the x of the out rows
    };
    Ops op;  // token 0's, requested by fetch()

    // This lane's columns of B and C for token t (8-byte vector loads at a
    // uniform row address plus the lane's 32-bit offset).
    __device__ __forceinline__ void load_bc(const Params &p, int t, Ops &o) const
    {
        const auto *const Bu = reinterpret_cast<const u32x2 *>(p.B + (b * p.B_b + t * p.B_t + grp * p.B_g));
        const auto *const Cu = reinterpret_cast<const u32x2 *>(p.C + (b * p.C_b + t * p.C_t + grp * p.C_g));
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            const uint32_t off = static_cast<uint32_t>(8 * c + 256 * v);  // bytes
            o.Bw[v] = *lane_at(Bu, off);
            o.Cw[v] = *lane_at(Cu, off);
        }
    }

    // dt of token t: the aligned 32-bit word that holds it.
    __device__ __forceinline__ void load_dt(const Params &p, int t)
    {
        const int64_t dte = b * p.dt_b + t * p.dt_t + h * p.dt_h + p.dt_off;
        const uint32_t dtw = load_ro(p.dt_words + (dte >> 1));
        dtbits = (dte & 1) ? (dtw >> 16) : (dtw & 0xffffu);
    }

    // x of this lane's rows wrow + sub + j*RPI for token t. With two rows per
    // instruction the wave's rows are R whole 32-bit words at a uniform
    // address (scalar loads); otherwise each lane reads its own values.
    __device__ __forceinline__ void load_x(const Params &p, int t, Ops &o) const
    {
        const uint16_t *xrow = xh + t * p.x_t;
        if constexpr (RPI == 2) {
            // one byte permute per row: this lane's half of the word into the
            // upper half (byte selectors 0-3 name the word's bytes, 0x0C a zero)
            const uint32_t *xw = reinterpret_cast<const uint32_t *>(xrow);
            const uint32_t sel = sub ? 0x03020C0Cu : 0x01000C0Cu;
#pragma unroll
            for (int j = 0; j < R; ++j)
                o.xbits[j] = __builtin_amdgcn_perm(0u, load_ro(xw + j), sel);
        } else {
#pragma unroll
            for (int j = 0; j < R; ++j)
                o.xbits[j] = *lane_at(xrow, 2u * (sub + j * RPI));
        }
        // the rows this lane's out values belong to: with 8 or more rows per
        // lane (the configurations of the instruction-bound K-token launches)
        // a lane's own load, which is cheaper than a select over its rows'
        // x values; with fewer, step() selects them (no extra load in a
        // memory-bound launch). The same value either way.
        if constexpr (R >= 8) {
#pragma unroll
            for (int i = 0; i < RS::KEEP; ++i)
                o.xo[i] = *lane_at(xrow, 2u * (sub + (fr + i) * RPI));
        }
    }

    // The x word of out row fr + i (see Ops). The selects go through an
    // opaque copy of each word: written plainly, the compiler turns the chain
    // into an array read at a run-time index and moves the operand set to
    // scratch memory.
    __device__ __forceinline__ uint32_t xout(const Ops &o, int i) const
    {
        if constexpr (R >= 8) {
            return o.xo[i];
        } else {
            uint32_t v = o.xbits[0];
#pragma unroll
            for (int j = 1; j < R; ++j) {
                uint32_t xj = o.xbits[j];
                asm("" : "+v"(xj));
                v = (fr + i == j) ? xj : v;
            }
            return v;
        }
    }

    // delta = softplus(dt + dt_bias) (or dt + dt_bias) and the decay
    // exp(A * delta) from a bf16 dt bit pattern (the fp32 softplus and exp
    // of internal.h: a few ulp each, NaN and infinities kept).
    __device__ __forceinline__ void discretize(const Params &p, uint32_t bits, float &delta, float &dA) const
    {
        const float u = __uint_as_float(bits << 16) + bias;
        delta = p.softplus ? softplus_f32(u) : u;
        dA = exp_f32(Ah * delta);
    }

    // graw: workgroup-order tile id (>= total_groups: nothing to do).
    // PRIO: the caller raised the wave's priority; it is lowered once the
    // state loads are issued. LANEDT: each lane also requests the word that
    // holds the dt of token min(lane, p.ntokens - 1) ahead of the state, so
    // that the tokens' discretisation can run while the state is in flight
    // (the bits are taken out of the word where they are used, so that
    // nothing here waits for the load).
    template <bool PRIO = false, bool LANEDT = false>
    __device__ __forceinline__ void fetch(const Params &p, int graw, int rows_group, int wave, int lane)
    {
        if (graw >= p.total_groups) {
            live = false;
            return;
        }
        const int g = p.xcd_remap ? xcd_order(graw, p.total_groups) : graw;
        // ptiles == 0: a wave covers a whole head (rows_per_wave == headdim)
        // and the group's waves take consecutive heads of one request;
        // otherwise the group's rows are tile t of one head
        const bool per_head = p.ptiles == 0;
        const int t = per_head ? 0 : g % p.ptiles;
        const int bh = per_head ? g * (rows_group / ROWS_WAVE) + wave : g / p.ptiles;
        // (uniform values that the divisions leave in vector registers:
        // moved to scalar ones once, so that every address built from them
        // is scalar arithmetic)
        h = __builtin_amdgcn_readfirstlane(bh % p.nheads);
        b = __builtin_amdgcn_readfirstlane(bh / p.nheads);
        grp = __builtin_amdgcn_readfirstlane(h / p.heads_per_group);
        c = lane % LPR;    // column chunk
        sub = lane / LPR;  // row within one instruction
        fr = RS::first(sub * LPR + c);
        wrow = __builtin_amdgcn_readfirstlane(per_head ? 0 : t * rows_group + wave * ROWS_WAVE);  // first row of this wave
        p0 = wrow + sub;
        xh = uniform_ptr(p.x + (b * p.x_b + h * p.x_h + wrow));
        oh = uniform_ptr(p.out + (b * p.o_b + h * p.o_h + wrow));

        // B and C do not depend on the slot: requested first (vector-memory
        // counters retire in order, so anything issued after the state stream
        // could only be used after it).
        load_bc(p, 0, op);

        const int64_t slot = p.idx64 ? load_ro(static_cast<const int64_t *>(p.idx) + b)
                                     : static_cast<int64_t>(load_ro(static_cast<const int32_t *>(p.idx) + b));
        live = slot >= 0 && slot < p.pool_slots;
        if (!live)
            return;  // padding entry: no state traffic, out rows untouched
        if constexpr (LANEDT) {
            const int tok = min(lane, p.ntokens - 1);
            const int64_t dte = b * p.dt_b + tok * p.dt_t + h * p.dt_h + p.dt_off;
            dtlane = p.dt_words[dte >> 1];
            dtshift = static_cast<uint32_t>(dte & 1) * 16u;
        }

        // State loads: all R * VEC dwordx4 of this lane are requested up front.
        sp = p.state + slot * p.s_slot + h * p.s_head + static_cast<int64_t>(p0) * p.s_row + 4 * c;
        jstep = static_cast<int64_t>(RPI) * p.s_row;
#pragma unroll
        for (int j = 0; j < R; ++j)
#pragma unroll
            for (int v = 0; v < VEC; ++v)
                s[j][v] = load4<NT>(sp + j * jstep + 128 * v);

        if constexpr (PRIO)
            __builtin_amdgcn_s_setprio(0);

        // Per-head parameters and token 0's dt and x through the scalar cache,
        // while the state is in flight.
        bias = p.dt_bias ? load_ro(p.dt_bias + h * p.dtb_h) : 0.0f;
        Ah = load_ro(p.A + h * p.A_h);
        Dh = p.D ? load_ro(p.D + h * p.D_h) : 0.0f;
        load_dt(p, 0);
        load_x(p, 0, op);
    }

    // Advance the state by token t (operands o) with its discretisation
    // (delta, dA); write the state back when LAST.
    template <bool LAST>
    __device__ __forceinline__ void step(const Params &p, int t, const Ops &o, float delta, float dA)
    {
        // delta * B[n] and C[n] of this lane's columns
        float dB[VEC][4], Cv[VEC][4];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            dB[v][0] = delta * __uint_as_float(o.Bw[v].x << 16);
            dB[v][1] = delta * __uint_as_float(o.Bw[v].x & 0xffff0000u);
            dB[v][2] = delta * __uint_as_float(o.Bw[v].y << 16);
            dB[v][3] = delta * __uint_as_float(o.Bw[v].y & 0xffff0000u);
            Cv[v][0] = __uint_as_float(o.Cw[v].x << 16);
            Cv[v][1] = __uint_as_float(o.Cw[v].x & 0xffff0000u);
            Cv[v][2] = __uint_as_float(o.Cw[v].y << 16);
            Cv[v][3] = __uint_as_float(o.Cw[v].y & 0xffff0000u);
        }

        // Update in registers (write back after the last token) and form each
        // lane's partial output.
        float y[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const float xj = __uint_as_float(XRAW ? o.xbits[j] << 16 : o.xbits[j]);
            float acc = 0.0f;
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                f32x4 &q = s[j][v];
                q.x = fmaf(q.x, dA, xj * dB[v][0]);
                q.y = fmaf(q.y, dA, xj * dB[v][1]);
                q.z = fmaf(q.z, dA, xj * dB[v][2]);
                q.w = fmaf(q.w, dA, xj * dB[v][3]);
                acc = (v == 0) ? q.x * Cv[v][0] : fmaf(q.x, Cv[v][0], acc);
                acc = fmaf(q.y, Cv[v][1], acc);
                acc = fmaf(q.z, Cv[v][2], acc);
                acc = fmaf(q.w, Cv[v][3], acc);
            }
            y[j] = acc;
            if constexpr (LAST) {
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    store4<NT>(sp + j * jstep + 128 * v, s[j][v]);
            }
        }

        // Row totals: this lane ends up with KEEP of them, rows fr + i.
        // When R < LPR several lanes of a row group hold each row; one of
        // them writes it.
        RS::run(y, sub * LPR + c);  // the wave lane
        uint16_t *const orow = oh + t * p.o_t;
        if (RS::writer(c)) {
#pragma unroll
            for (int i = 0; i < RS::KEEP; ++i) {
                const uint32_t xw = xout(o, i);
                const float xo = __uint_as_float(XORAW ? xw << 16 : xw);
                *lane_at(orow, 2u * (sub + (fr + i) * RPI)) = bf16_round(fmaf(Dh, xo, y[i]));
            }
        }
    }

    __device__ __forceinline__ void finish(const Params &p)
    {
        float delta, dA;
        discretize(p, dtbits, delta, dA);
        step<true>(p, 0, op, delta, dA);
    }
};

// One workgroup per tile, one token.
template <int N, int R, int W, bool NT>
__global__ void __launch_bounds__(64 * W) ssu_decode_kernel(const Params p)
{
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    Work<N, R, NT> w;
    w.fetch(p, static_cast<int>(blockIdx.x), Work<N, R, NT>::ROWS_WAVE * W, wave, lane);
    if (w.live)
        w.finish(p);
}

// One workgroup per tile, p.ntokens tokens: the state is read once, advanced
// token by token in registers with the same arithmetic as the one-token
// kernel, and written once; each token's out is written as it is formed. The
// operands of token t+1 are requested before token t is computed, into the
// other of two operand sets (the loop goes two tokens per trip, so the sets
// alternate without register copies), and the per-token discretisation is
// done 64 tokens at a time, one token per lane (the same fp32 operations as
// the one-token kernel, so the same bits), then read back with a uniform lane
// read; the first 64 tokens' dt are requested ahead of the state, so their
// discretisation overlaps the state's flight instead of following it.
template <int N, int R, int W, bool NT>
__global__ void __launch_bounds__(64 * W) ssu_decode_tokens_kernel(const Params p)
{
    using WK = Work<N, R, NT>;
    const int lane = static_cast<int>(threadIdx.x) & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    WK w;
    // Until its state is requested a wave takes issue slots before the waves
    // computing tokens on state that has arrived (fetch() drops the priority
    // after the state loads), so the state stream starts sooner.
    __builtin_amdgcn_s_setprio(2);
    w.template fetch<true, true>(p, static_cast<int>(blockIdx.x), WK::ROWS_WAVE * W, wave, lane);
    // (the tokens under the branch, not after an early return: the state's
    // and x's loads then stay unconsumed until their first use below)
    if (w.live) {
        const int K = p.ntokens;
        float lane_delta = 0.0f, lane_dA = 1.0f;
        // tokens 0 .. 63 from the dt words requested before the state (lanes
        // past the last token repeat it; their values are never read)
        w.discretize(p, (w.dtlane >> w.dtshift) & 0xffffu, lane_delta, lane_dA);
        // (delta, dA) of token t, discretising tokens t .. t+63 when t > 0 starts
        // a group of 64
        auto disc = [&](int t, float &delta, float &dA) {
            const int tl = t & 63;
            if (tl == 0 && t > 0 && t + lane < K) {
                const int64_t dte = w.b * p.dt_b + (t + lane) * p.dt_t + w.h * p.dt_h + p.dt_off;
                const uint32_t dtw = p.dt_words[dte >> 1];
                w.discretize(p, (dte & 1) ? (dtw >> 16) : (dtw & 0xffffu), lane_delta, lane_dA);
            }
            delta = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lane_delta), tl));
            dA = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lane_dA), tl));
        };
        typename WK::Ops o1;
        float delta, dA;
        int t = 0;
        for (; t + 2 < K; t += 2) {  // tokens t (operands w.op) and t+1 (o1)
            w.load_bc(p, t + 1, o1);
            w.load_x(p, t + 1, o1);
            disc(t, delta, dA);
            w.template step<false>(p, t, w.op, delta, dA);
            w.load_bc(p, t + 2, w.op);
            w.load_x(p, t + 2, w.op);
            disc(t + 1, delta, dA);
            w.template step<false>(p, t + 1, o1, delta, dA);
        }
        // one or two tokens left, the first with operands w.op
        if (t + 1 < K) {
            w.load_bc(p, t + 1, o1);
            w.load_x(p, t + 1, o1);
            disc(t, delta, dA);
            w.template step<false>(p, t, w.op, delta, dA);
            disc(t + 1, delta, dA);
            w.template step<true>(p, t + 1, o1, delta, dA);
        } else {
            disc(t, delta, dA);
            w.template step<true>(p, t, w.op, delta, dA);
        }
    }
}

// ------------------------------------------------------------------ tiles --

using LaunchFn = hipError_t (*)(const Params &, int grid, size_t lds_bytes, hipStream_t);

template <int N, int R, int W, bool NT>
hipError_t launch(const Params &p, int grid, size_t lds_bytes, hipStream_t stream)
{
    hipLaunchKernelGGL((ssu_decode_kernel<N, R, W, NT>), dim3(grid), dim3(64 * W), lds_bytes, stream, p);
    return hipGetLastError();
}

template <int N, int R, int W, bool NT>
hipError_t launch_tokens(const Params &p, int grid, size_t lds_bytes, hipStream_t stream)
{
    hipLaunchKernelGGL((ssu_decode_tokens_kernel<N, R, W, NT>), dim3(grid), dim3(64 * W), lds_bytes, stream, p);
    return hipGetLastError();
}

struct Tile {
    ssu_tile_desc d;
    LaunchFn fn;         // one token
    LaunchFn fn_tokens;  // several tokens
};

template <int N, int R, int W, bool NT>
void add_tile(std::vector<Tile> &v, int remap, int cap)
{
    constexpr int VEC = N > 128 ? N / 128 : 1;
    constexpr int RPI = 64 / (N / (4 * VEC));
    Tile t{};
    t.d.dstate = N;
    t.d.rows_per_wave = RPI * R;
    t.d.waves = W;
    t.d.rows_per_group = RPI * R * W;
    t.d.nontemporal = NT ? 1 : 0;
    t.d.xcd_remap = remap;
    t.d.groups_per_cu = cap;
    char capname[16] = "";
    if (cap > 0)
        std::snprintf(capname, sizeof capname, "_g%d", cap);
    std::snprintf(t.d.name, sizeof t.d.name, "n%d_r%d_w%d%s%s%s", N, RPI * R, W, NT ? "_nt" : "",
                  remap ? "_xcd" : "", capname);
    t.fn = &launch<N, R, W, NT>;
    t.fn_tokens = &launch_tokens<N, R, W, NT>;
    v.push_back(t);
}

// Every kernel in both workgroup orders, uncapped; non-temporal kernels also
// XCD-ordered with each residency cap in `caps` (workgroups per CU).
template <int N, int R, int W, bool NT>
void add_kernel(std::vector<Tile> &v, std::initializer_list<int> caps)
{
    add_tile<N, R, W, NT>(v, 1, 0);
    add_tile<N, R, W, NT>(v, 0, 0);
    if (NT)
        for (int cap : caps)
            add_tile<N, R, W, NT>(v, 1, cap);
}

template <bool NT>
void add_n128(std::vector<Tile> &v)
{
    const std::initializer_list<int> caps = {2, 3, 4, 5, 6, 7, 8, 10, 12, 16};
    // (the four-load one-wave kernel also at 14 and 20 groups per CU: the
    // caps of 2- and 3-token calls on large batches)
    const std::initializer_list<int> caps_r4w1 = {2, 3, 4, 5, 6, 7, 8, 10, 12, 14, 16, 20};
    add_kernel<128, 1, 1, NT>(v, caps);
    add_kernel<128, 1, 2, NT>(v, caps);
    add_kernel<128, 1, 4, NT>(v, caps);
    add_kernel<128, 1, 8, NT>(v, caps);
    add_kernel<128, 2, 1, NT>(v, caps);
    add_kernel<128, 2, 2, NT>(v, caps);
    add_kernel<128, 2, 4, NT>(v, caps);
    add_kernel<128, 2, 8, NT>(v, caps);
    add_kernel<128, 4, 1, NT>(v, caps_r4w1);
    add_kernel<128, 4, 2, NT>(v, caps);
    add_kernel<128, 4, 4, NT>(v, caps);
    add_kernel<128, 4, 8, NT>(v, caps);
    add_kernel<128, 8, 1, NT>(v, caps);
    add_kernel<128, 8, 2, NT>(v, caps);
    add_kernel<128, 8, 4, NT>(v, caps);
    add_kernel<128, 16, 1, NT>(v, caps);
    add_kernel<128, 16, 2, NT>(v, caps);
}

// Tiles for the other dstate values: non-temporal only (the measured winner
// for the state stream at N = 128).
template <int N>
void add_general(std::vector<Tile> &v)
{
    const std::initializer_list<int> caps = {6, 12};
    add_kernel<N, 1, 1, true>(v, caps);
    add_kernel<N, 1, 2, true>(v, caps);
    add_kernel<N, 1, 4, true>(v, caps);
    add_kernel<N, 2, 1, true>(v, caps);
    add_kernel<N, 2, 2, true>(v, caps);
    add_kernel<N, 2, 4, true>(v, caps);
    add_kernel<N, 4, 1, true>(v, caps);
    add_kernel<N, 4, 2, true>(v, caps);
    add_kernel<N, 4, 4, true>(v, caps);
    add_kernel<N, 8, 1, true>(v, caps);
    add_kernel<N, 8, 2, true>(v, caps);
    add_kernel<N, 8, 4, true>(v, caps);
}

const std::vector<Tile> &tiles()
{
    static const std::vector<Tile> table = [] {
        std::vector<Tile> v;
        add_n128<false>(v);
        add_n128<true>(v);
        add_general<16>(v);
        add_general<32>(v);
        add_general<64>(v);
        add_general<256>(v);
        return v;
    }();
    return table;
}

// Dynamic LDS that caps residency at `cap` workgroups per CU: the largest
// 512-byte multiple (the LDS allocation granule) not above lds_cu / cap and the
// per-workgroup limit. The kernel never touches this LDS; it only keeps more
// workgroups from fitting on a CU.
size_t lds_for_cap(int cap, int lds_cu, int lds_block)
{
    if (cap <= 0 || lds_cu <= 0)
        return 0;
    size_t b = (static_cast<size_t>(lds_cu) / cap) & ~static_cast<size_t>(511);
    if (lds_block > 0 && b > static_cast<size_t>(lds_block))
        b = static_cast<size_t>(lds_block) & ~static_cast<size_t>(511);
    return b;
}

int find_tile(int N, int rows_per_group, int waves, int nt, int remap, int cap)
{
    const auto &t = tiles();
    for (size_t i = 0; i < t.size(); ++i)
        if (t[i].d.dstate == N && t[i].d.rows_per_group == rows_per_group && t[i].d.waves == waves &&
            t[i].d.nontemporal == nt && t[i].d.xcd_remap == remap && t[i].d.groups_per_cu == cap)
            return static_cast<int>(i);
    return -1;
}

namespace {
thread_local char g_err[256] = "";
}  // namespace

ssu_status fail(ssu_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

DeviceLimits device_limits(int dev)
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int> lds_cu[kMaxDevices];
    static std::atomic<int> lds_block[kMaxDevices];
    if (dev < 0 || dev >= kMaxDevices)
        return {0, 0};
    int cu = lds_cu[dev].load(std::memory_order_acquire);
    int blk = lds_block[dev].load(std::memory_order_acquire);
    if (cu <= 0 || blk <= 0) {
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            hipDeviceGetAttribute(&blk, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
            return {0, 0};
        lds_cu[dev].store(cu, std::memory_order_release);
        lds_block[dev].store(blk, std::memory_order_release);
    }
    return {cu, blk};
}

}  // namespace ssu

// -------------------------------------------------------------- host ABI --

struct ssu_handle {
    ssu_config cfg;
    int32_t forced_tile;  // -1: table
};

namespace {

using ssu::DeviceLimits;
using ssu::device_limits;
using ssu::fail;

bool valid_dstate(int n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }

// A launch configuration fits H heads of headdim P if its rows per group
// divide P (a group covers part of one head), or if each of its waves covers
// exactly one head and its waves split the heads evenly (a group covers
// several whole heads of one request).
bool tile_fits(const ssu_tile_desc &d, int H, int P)
{
    if (P % d.rows_per_group == 0)
        return true;
    return d.rows_per_wave == P && d.rows_per_group % P == 0 && H % (d.rows_per_group / P) == 0;
}

// The launch configuration for `batch` requests, from tile sweeps on MI355X
// (every compiled configuration, H16 P64 N128, batches 8 to 512, cold state).
// Non-temporal access and XCD-ordered workgroups win everywhere. What matters
// next is how much state is in flight per CU: about 40-48 KiB is best; a full
// CU (32 waves x 2 KiB) congests the memory system, and fewer bytes leave it
// idle. So, by state bytes per call:
//   >= 32 MiB: one-wave groups, four dwordx4 loads per lane, at most 12
//              groups per CU (batch 512: 85.6 us against 88.5 us uncapped;
//              best or within 0.6% of best from batch 64 up);
//   smaller:   two loads per lane, the most waves (4, 2, 1) that still give
//              the chip 1024 workgroups, uncapped (batch 8: 3.18 us).
int select_tile(const ssu_config &c, int32_t batch, int32_t ntokens)
{
    using namespace ssu;
    const int64_t units = static_cast<int64_t>(batch) * c.nheads;  // (b, h) pairs
    const int P = c.headdim, N = c.dstate;
    const int vec = N > 128 ? N / 128 : 1;
    const int rpi = 64 / (N / (4 * vec));
    const int64_t state_bytes = units * P * N * 4;
    auto pick = [&](int loads_per_lane, int W, int cap) -> int {
        const int R = loads_per_lane / vec > 0 ? loads_per_lane / vec : 1;
        const int rows_group = rpi * R * W;
        if (rows_group > P || P % rows_group)
            return -1;
        return find_tile(N, rows_group, W, 1, 1, cap);
    };
    if (state_bytes >= (int64_t(32) << 20)) {
        // Several tokens per call make each workgroup's work longer and
        // ALU-heavier: full occupancy hides that better than the cap. From 8
        // tokens on (from 4 below 128 MiB of state), eight loads per lane win
        // (fewer waves repeating the per-token work; batch 512, 8 tokens:
        // 107.8 us against 120.0 us with four loads, 172.2 us with four loads
        // capped at 12), and from 16 tokens two-wave groups (batch 512:
        // 154.6 us against 156.8 us with one wave). At 4 tokens four loads
        // lead at batch 512 (96.6 against 98.6 us), eight at batch 128 (29.2
        // against 30.1 us). Between one token and four the best residency
        // rises with the work per wave: at batch 512 2 tokens take 91.0 us at
        // 14 groups per CU (12: 93.4, 16: 91.2, uncapped 92.4) and 3 tokens
        // 92.3 us at 20 (16: 93.5, uncapped 92.9); at batch 128 uncapped
        // leads from 2 tokens on. Shapes without such a cap run uncapped.
        const bool big = state_bytes >= (int64_t(128) << 20);
        const int loads = (ntokens >= 8 || (ntokens >= 4 && !big)) ? 8 : 4;
        const int waves = ntokens >= 16 ? 2 : 1;
        const int cap = ntokens == 1 ? 12 : !big ? 0 : ntokens == 2 ? 14 : ntokens == 3 ? 20 : 0;
        int id = pick(loads, waves, cap);
        if (id < 0 && ntokens > 1 && cap > 0)
            id = pick(loads, waves, 0);
        if (id < 0 && waves > 1)
            id = pick(loads, 1, 0);
        if (id >= 0)
            return id;
    }
    if (ntokens <= 1) {
        // One token below 32 MiB of state: about one wave per SIMD (1024 on
        // the chip), each streaming an equal share, i.e. as many loads per
        // lane as the call has MiB of state (a power of two, 2 to 16), in
        // two-wave groups from 8 loads per lane. From a sweep of every
        // configuration at H16 batch 1 to 64 and at H8 / H64 (us per call:
        // 4 MiB 3.39 with four loads against 3.75 with two; 8 MiB 4.79 with
        // eight in two-wave groups against 5.41; 16 MiB 7.01-7.16 with
        // sixteen against 8.14-8.28; 2 MiB and below two loads, within 1% of
        // the fastest). Where the shape has no such configuration, fewer
        // loads.
        int loads = 2;
        while (loads < 16 && (static_cast<int64_t>(loads) << 20) < state_bytes)
            loads *= 2;
        for (; loads >= 1; loads /= 2) {
            const int W = loads >= 8 ? 2 : 1;
            int id = pick(loads, W, 0);
            if (id < 0 && W > 1)
                id = pick(loads, 1, 0);
            if (id >= 0)
                return id;
        }
    }
    const int64_t target_groups = 1024;
    int fallback = -1;
    for (int loads : {2, 1}) {
        for (int W : {4, 2, 1}) {
            const int id = pick(loads, W, 0);
            if (id < 0)
                continue;
            const int rows_group = ssu::tiles()[id].d.rows_per_group;
            if (units * (P / rows_group) >= target_groups)
                return id;
            fallback = id;  // keep shrinking: smaller groups give more of them
        }
        if (fallback >= 0)
            return fallback;
    }
    return fallback;
}

ssu_status check_view(const ssu_view &v, const char *name, int32_t dtype, int rank, bool nullable)
{
    if (!v.ptr && !nullable)
        return fail(SSU_ERR_INVALID_ARGUMENT, "%s: null pointer", name);
    if (!v.ptr)
        return SSU_OK;
    if (v.dtype != dtype)
        return fail(SSU_ERR_INVALID_ARGUMENT, "%s: dtype tag %d, expected %d", name, v.dtype, dtype);
    if (v.reserved != 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "%s: reserved field must be 0", name);
    for (int i = 0; i < rank; ++i)
        if (v.stride[i] < 0)
            return fail(SSU_ERR_INVALID_ARGUMENT, "%s: negative stride[%d]", name, i);
    return SSU_OK;
}

#define SSU_TRY(expr)                    \
    do {                                 \
        const ssu_status s_ = (expr);    \
        if (s_ != SSU_OK)                \
            return s_;                   \
    } while (0)

}  // namespace

extern "C" {

int32_t ssu_abi_version(void) { return SSU_ABI_VERSION; }

const char *ssu_last_error(void) { return ssu::g_err; }

const char *ssu_status_string(ssu_status s)
{
    switch (s) {
    case SSU_OK: return "SSU_OK";
    case SSU_ERR_INVALID_ARGUMENT: return "SSU_ERR_INVALID_ARGUMENT";
    case SSU_ERR_UNSUPPORTED: return "SSU_ERR_UNSUPPORTED";
    case SSU_ERR_MISALIGNED: return "SSU_ERR_MISALIGNED";
    case SSU_ERR_HIP: return "SSU_ERR_HIP";
    case SSU_ERR_NO_MEMORY: return "SSU_ERR_NO_MEMORY";
    case SSU_ERR_BAD_INDEX: return "SSU_ERR_BAD_INDEX";
    }
    return "SSU_ERR_UNKNOWN";
}

int32_t ssu_tile_count(void) { return static_cast<int32_t>(ssu::tiles().size()); }

ssu_status ssu_tile_info(int32_t tile, ssu_tile_desc *out)
{
    if (!out)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_tile_info: null output");
    if (tile < 0 || tile >= ssu_tile_count())
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_tile_info: tile %d out of range", tile);
    *out = ssu::tiles()[tile].d;
    return SSU_OK;
}

ssu_status ssu_create(const ssu_config *cfg, ssu_handle **out)
{
    if (!cfg || !out)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_create: null argument");
    *out = nullptr;
    const ssu_config &c = *cfg;
    if (c.reserved != 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_create: reserved field must be 0");
    if (c.nheads < 1 || c.ngroups < 1 || c.nheads % c.ngroups != 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_create: need nheads >= 1 and ngroups dividing it (H=%d G=%d)",
                    c.nheads, c.ngroups);
    if (c.headdim < 1 || c.dstate < 1)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_create: headdim and dstate must be positive");
    if (!valid_dstate(c.dstate))
        return fail(SSU_ERR_UNSUPPORTED, "ssu_create: dstate %d not compiled (16, 32, 64, 128, 256)", c.dstate);
    if (c.headdim % 16 != 0 || c.headdim > 256)
        return fail(SSU_ERR_UNSUPPORTED, "ssu_create: headdim %d must be a multiple of 16 in [16, 256]",
                    c.headdim);
    if (c.dt_softplus != 0 && c.dt_softplus != 1)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_create: dt_softplus must be 0 or 1");
    if (c.device < -1)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_create: device must be >= -1");
    int32_t forced = c.tile;
    if (forced < -1 || forced >= ssu_tile_count())
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_create: tile %d out of range", forced);
    if (forced == -1) {
        if (const char *env = std::getenv("SSU_TILE")) {
            char *end = nullptr;
            const long v = std::strtol(env, &end, 10);
            if (end == env || *end != '\0' || v < -1 || v >= ssu_tile_count())
                return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_create: SSU_TILE=%s is not a tile index", env);
            forced = static_cast<int32_t>(v);
        }
    }
    if (forced >= 0 &&
        (ssu::tiles()[forced].d.dstate != c.dstate || !tile_fits(ssu::tiles()[forced].d, c.nheads, c.headdim)))
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_create: tile %s does not fit N=%d H=%d P=%d",
                    ssu::tiles()[forced].d.name, c.dstate, c.nheads, c.headdim);
    ssu_handle *h = new (std::nothrow) ssu_handle;
    if (!h)
        return fail(SSU_ERR_NO_MEMORY, "ssu_create: out of host memory");
    h->cfg = c;
    h->forced_tile = forced;
    *out = h;
    return SSU_OK;
}

void ssu_destroy(ssu_handle *h) { delete h; }

int32_t ssu_select_tile(const ssu_handle *h, int32_t batch)
{
    if (!h)
        return -1;
    if (h->forced_tile >= 0)
        return h->forced_tile;
    return select_tile(h->cfg, batch < 1 ? 1 : batch, 1);
}

int32_t ssu_select_tile_tokens(const ssu_handle *h, int32_t batch, int32_t ntokens)
{
    if (!h)
        return -1;
    if (h->forced_tile >= 0)
        return h->forced_tile;
    return select_tile(h->cfg, batch < 1 ? 1 : batch, ntokens < 1 ? 1 : ntokens);
}

}  // extern "C"

namespace {

// One call's operands in a single form: the per-token views (x, B, C, dt,
// out) carry four strides (request, token, head or group, innermost); a
// one-token call has token stride 0.
struct Operands {
    int32_t batch, ntokens;
    int64_t pool_slots;
    ssu_view state, idx, dt_bias, A, D;
    ssu_view x, B, C, dt, out;
};

// [request, head|group, inner] -> [request, token (stride 0), head|group, inner]
ssu_view with_token_axis(const ssu_view &v)
{
    ssu_view w = v;
    w.stride[3] = v.stride[2];
    w.stride[2] = v.stride[1];
    w.stride[1] = 0;
    return w;
}

// Restores the caller's current device on every return path.
struct DeviceGuard {
    int prev = -1;
    bool switched = false;
    ssu_status enter(int device)
    {
        if (device < 0)
            return SSU_OK;
        if (hipGetDevice(&prev) != hipSuccess)
            return fail(SSU_ERR_HIP, "hipGetDevice failed");
        if (prev != device) {
            if (hipSetDevice(device) != hipSuccess)
                return fail(SSU_ERR_HIP, "hipSetDevice(%d) failed", device);
            switched = true;
        }
        return SSU_OK;
    }
    ~DeviceGuard()
    {
        if (switched)
            (void)hipSetDevice(prev);
    }
};

ssu_status run(const ssu_handle *hd, const Operands &a, hipStream_t stream)
{
    const ssu_config &c = hd->cfg;
    SSU_TRY(check_view(a.state, "state", SSU_F32, 4, false));
    if (a.idx.ptr && a.idx.dtype == SSU_I64)
        SSU_TRY(check_view(a.idx, "idx", SSU_I64, 1, false));
    else
        SSU_TRY(check_view(a.idx, "idx", SSU_I32, 1, false));
    SSU_TRY(check_view(a.x, "x", SSU_BF16, 4, false));
    SSU_TRY(check_view(a.B, "B", SSU_BF16, 4, false));
    SSU_TRY(check_view(a.C, "C", SSU_BF16, 4, false));
    SSU_TRY(check_view(a.dt, "dt", SSU_BF16, 4, false));
    SSU_TRY(check_view(a.dt_bias, "dt_bias", SSU_F32, 2, true));
    SSU_TRY(check_view(a.A, "A", SSU_F32, 3, false));
    SSU_TRY(check_view(a.D, "D", SSU_F32, 2, true));
    SSU_TRY(check_view(a.out, "out", SSU_BF16, 4, false));

    if (a.state.stride[3] != 1)
        return fail(SSU_ERR_UNSUPPORTED, "state: dstate stride must be 1");
    if (a.idx.stride[0] != 1)
        return fail(SSU_ERR_UNSUPPORTED, "idx: stride must be 1");
    if (a.x.stride[3] != 1 || a.out.stride[3] != 1)
        return fail(SSU_ERR_UNSUPPORTED, "x/out: headdim stride must be 1");
    if (a.B.stride[3] != 1 || a.C.stride[3] != 1)
        return fail(SSU_ERR_UNSUPPORTED, "B/C: dstate stride must be 1");
    if (a.dt.stride[3] != 0)
        return fail(SSU_ERR_UNSUPPORTED, "dt: must be one value per (request, head) (headdim stride 0)");
    if (a.dt_bias.ptr && a.dt_bias.stride[1] != 0)
        return fail(SSU_ERR_UNSUPPORTED, "dt_bias: headdim stride must be 0");
    if (a.A.stride[1] != 0 || a.A.stride[2] != 0)
        return fail(SSU_ERR_UNSUPPORTED, "A: must be one value per head (headdim, dstate strides 0)");
    if (a.D.ptr && a.D.stride[1] != 0)
        return fail(SSU_ERR_UNSUPPORTED, "D: headdim stride must be 0");

    const uintptr_t sp = reinterpret_cast<uintptr_t>(a.state.ptr);
    if (sp % 16 || a.state.stride[0] % 4 || a.state.stride[1] % 4 || a.state.stride[2] % 4)
        return fail(SSU_ERR_MISALIGNED, "state: pointer and slot/head/row strides must be 16-byte multiples");
    const uintptr_t xp = reinterpret_cast<uintptr_t>(a.x.ptr);
    if (xp % 4 || a.x.stride[0] % 2 || a.x.stride[1] % 2 || a.x.stride[2] % 2)
        return fail(SSU_ERR_MISALIGNED, "x: pointer and request/token/head strides must be 4-byte multiples");
    for (const ssu_view *v : {&a.B, &a.C}) {
        const uintptr_t bp = reinterpret_cast<uintptr_t>(v->ptr);
        if (bp % 8 || v->stride[0] % 4 || v->stride[1] % 4 || v->stride[2] % 4)
            return fail(SSU_ERR_MISALIGNED, "B/C: pointer and request/token/group strides must be 8-byte multiples");
    }
    const uintptr_t dtp = reinterpret_cast<uintptr_t>(a.dt.ptr);
    if (dtp % 2)
        return fail(SSU_ERR_MISALIGNED, "dt: pointer must be 2-byte aligned");

    const int32_t tile = hd->forced_tile >= 0 ? hd->forced_tile : select_tile(c, a.batch, a.ntokens);
    if (tile < 0)
        return fail(SSU_ERR_UNSUPPORTED, "no launch configuration for N=%d P=%d", c.dstate, c.headdim);
    const ssu::Tile &T = ssu::tiles()[tile];
    // a group covers rows_per_group rows of one head, or (when its waves each
    // cover a whole head) rows_per_group / headdim heads of one request
    const bool per_head = T.d.rows_per_group > c.headdim;
    const int ptiles = per_head ? 0 : c.headdim / T.d.rows_per_group;
    const int64_t groups = per_head ? static_cast<int64_t>(a.batch) * c.nheads / (T.d.rows_per_group / c.headdim)
                                    : static_cast<int64_t>(a.batch) * c.nheads * ptiles;
    if (groups > 0x7fffffff)
        return fail(SSU_ERR_UNSUPPORTED, "batch * heads too large for one launch");

    ssu::Params p{};
    p.state = static_cast<float *>(const_cast<void *>(a.state.ptr));
    p.s_slot = a.state.stride[0];
    p.s_head = a.state.stride[1];
    p.s_row = a.state.stride[2];
    p.idx = a.idx.ptr;
    p.idx64 = a.idx.dtype == SSU_I64;
    p.pool_slots = a.pool_slots;
    p.x = static_cast<const uint16_t *>(a.x.ptr);
    p.x_b = a.x.stride[0];
    p.x_t = a.x.stride[1];
    p.x_h = a.x.stride[2];
    p.B = static_cast<const uint16_t *>(a.B.ptr);
    p.B_b = a.B.stride[0];
    p.B_t = a.B.stride[1];
    p.B_g = a.B.stride[2];
    p.C = static_cast<const uint16_t *>(a.C.ptr);
    p.C_b = a.C.stride[0];
    p.C_t = a.C.stride[1];
    p.C_g = a.C.stride[2];
    p.dt_words = reinterpret_cast<const uint32_t *>(dtp & ~uintptr_t(3));
    p.dt_off = (dtp & 2) ? 1 : 0;
    p.dt_b = a.dt.stride[0];
    p.dt_t = a.dt.stride[1];
    p.dt_h = a.dt.stride[2];
    p.dt_bias = static_cast<const float *>(a.dt_bias.ptr);
    p.dtb_h = a.dt_bias.stride[0];
    p.A = static_cast<const float *>(a.A.ptr);
    p.A_h = a.A.stride[0];
    p.D = static_cast<const float *>(a.D.ptr);
    p.D_h = a.D.stride[0];
    p.out = static_cast<uint16_t *>(const_cast<void *>(a.out.ptr));
    p.o_b = a.out.stride[0];
    p.o_t = a.out.stride[1];
    p.o_h = a.out.stride[2];
    p.nheads = c.nheads;
    p.heads_per_group = c.nheads / c.ngroups;
    p.ptiles = ptiles;
    p.softplus = c.dt_softplus;
    p.xcd_remap = T.d.xcd_remap;
    p.total_groups = static_cast<int32_t>(groups);
    p.ntokens = a.ntokens;

    DeviceGuard guard;
    SSU_TRY(guard.enter(c.device));
    size_t lds = 0;
    if (T.d.groups_per_cu > 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return fail(SSU_ERR_HIP, "hipGetDevice failed");
        const DeviceLimits lim = device_limits(dev);
        if (lim.lds_cu <= 0)
            return fail(SSU_ERR_HIP, "cannot query the LDS size of device %d", dev);
        lds = ssu::lds_for_cap(T.d.groups_per_cu, lim.lds_cu, lim.lds_block);
    }
    const ssu::LaunchFn fn = a.ntokens > 1 ? T.fn_tokens : T.fn;
    const hipError_t e = fn(p, static_cast<int>(groups), lds, stream);
    if (e != hipSuccess)
        return fail(SSU_ERR_HIP, "launch of %s failed: %s", T.d.name, hipGetErrorString(e));
    return SSU_OK;
}

}  // namespace

extern "C" {

ssu_status ssu_update(const ssu_handle *hd, const ssu_args *a, hipStream_t stream)
{
    if (!hd || !a)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_update: null handle or args");
    if (a->batch < 0 || a->pool_slots < 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_update: batch %d / pool_slots %lld negative", a->batch,
                    static_cast<long long>(a->pool_slots));
    if (a->reserved != 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_update: reserved field must be 0");
    if (a->batch == 0)
        return SSU_OK;
    Operands o{};
    o.batch = a->batch;
    o.ntokens = 1;
    o.pool_slots = a->pool_slots;
    o.state = a->state;
    o.idx = a->idx;
    o.dt_bias = a->dt_bias;
    o.A = a->A;
    o.D = a->D;
    o.x = with_token_axis(a->x);
    o.B = with_token_axis(a->B);
    o.C = with_token_axis(a->C);
    o.dt = with_token_axis(a->dt);
    o.out = with_token_axis(a->out);
    return run(hd, o, stream);
}

ssu_status ssu_update_tokens(const ssu_handle *hd, const ssu_tokens_args *a, hipStream_t stream)
{
    if (!hd || !a)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_update_tokens: null handle or args");
    if (a->batch < 0 || a->pool_slots < 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_update_tokens: batch %d / pool_slots %lld negative", a->batch,
                    static_cast<long long>(a->pool_slots));
    if (a->ntokens < 1 || a->ntokens > SSU_MAX_TOKENS)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_update_tokens: ntokens %d outside [1, %d]", a->ntokens,
                    SSU_MAX_TOKENS);
    if (a->batch == 0)
        return SSU_OK;
    Operands o{};
    o.batch = a->batch;
    o.ntokens = a->ntokens;
    o.pool_slots = a->pool_slots;
    o.state = a->state;
    o.idx = a->idx;
    o.dt_bias = a->dt_bias;
    o.A = a->A;
    o.D = a->D;
    o.x = a->x;
    o.B = a->B;
    o.C = a->C;
    o.dt = a->dt;
    o.out = a->out;
    return run(hd, o, stream);
}

ssu_status ssu_check_indices(const ssu_args *a, hipStream_t stream)
{
    if (!a)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_check_indices: null args");
    if (a->batch < 0 || a->pool_slots < 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_check_indices: negative size");
    if (a->batch == 0)
        return SSU_OK;
    const bool i64 = a->idx.dtype == SSU_I64;
    if (!a->idx.ptr || (!i64 && a->idx.dtype != SSU_I32) || a->idx.stride[0] != 1)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_check_indices: idx must be a contiguous i32/i64 view");
    // Memory in proportion to the batch, never to the pool: the in-range
    // (slot, position) pairs are sorted and neighbours compared.
    const size_t esz = i64 ? 8 : 4;
    std::vector<unsigned char> host;
    std::vector<std::pair<int64_t, int32_t>> live;
    try {
        host.resize(esz * static_cast<size_t>(a->batch));
        live.reserve(static_cast<size_t>(a->batch));
    } catch (const std::bad_alloc &) {
        return fail(SSU_ERR_NO_MEMORY, "ssu_check_indices: out of host memory for %d entries", a->batch);
    }
    if (hipMemcpyAsync(host.data(), a->idx.ptr, host.size(), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return fail(SSU_ERR_HIP, "ssu_check_indices: copy of idx failed");
    for (int32_t b = 0; b < a->batch; ++b) {
        int64_t s;
        if (i64) {
            std::memcpy(&s, host.data() + 8 * static_cast<size_t>(b), 8);
        } else {
            int32_t s32;
            std::memcpy(&s32, host.data() + 4 * static_cast<size_t>(b), 4);
            s = s32;
        }
        if (s >= 0 && s < a->pool_slots)
            live.emplace_back(s, b);
    }
    std::sort(live.begin(), live.end());
    for (size_t k = 1; k < live.size(); ++k)
        if (live[k].first == live[k - 1].first)
            return fail(SSU_ERR_BAD_INDEX, "idx[%d] = %lld repeats idx[%d]", live[k].second,
                        static_cast<long long>(live[k].first), live[k - 1].second);
    return SSU_OK;
}

}  // extern "C"
