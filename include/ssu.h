/*
 * ssu.h -- libssu: the Mamba2 decode-step selective_state_update on AMD
 * Instinct MI355X (gfx950), as a C ABI.
 *
 * The operation (one decode token for a batch of requests; sglang PR #41223,
 * "[Perf] Mamba2 selective_state_update up to 2x faster on B200 via 8x1 launch
 * config for dstate 128", sections "Summary" and "Kernel measurement"): for
 * every request b and head h, with g = h / (H/G) the head's group,
 *
 *     slot    = idx[b]
 *     delta   = softplus(dt[b,h] + dt_bias[h])        (or dt + dt_bias when
 *                                                      dt_softplus == 0)
 *     a       = exp(A[h] * delta)
 *     S[p,n]  = state[slot,h,p,n] * a + delta * x[b,h,p] * B[b,g,n]
 *     state[slot,h,p,n] = S[p,n]                       (in place, fp32)
 *     out[b,h,p] = bf16( sum_n S[p,n] * C[b,g,n] + D[h] * x[b,h,p] )
 *
 * The page states the problem this way: an fp32 state pool [pool, H, P, N]
 * addressed through random state_batch_indices, x/B/C as views into one packed
 * bf16 tensor, and dt, A, D, dt_bias holding one value per head (zero strides
 * over the other axes). The
 * arguments below mirror that statement: every operand is a strided view.
 *
 * Numerics: fp32 arithmetic throughout; the sum over n is taken in one fixed
 * order that does not depend on the launch configuration (tile), so every tile
 * gives bitwise-identical state and out, and repeated runs are bitwise
 * reproducible. out is rounded to bf16 to nearest, ties to even.
 *
 * Ownership and threading: the caller owns every device buffer and the stream.
 * ssu_update is asynchronous on the stream: buffers must stay alive until the
 * stream's work completes. The library keeps no pointer after a call returns.
 * A handle is immutable after ssu_create, so calls on one handle from several
 * threads or streams are safe. ssu_update allocates nothing, never
 * synchronises and never reads device memory, so it may be captured into a
 * HIP graph.
 *
 * Errors: every function reports through ssu_status; nothing throws across the
 * ABI. ssu_last_error() gives a one-line description of the calling thread's
 * most recent failure.
 */
#ifndef SSU_H
#define SSU_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSU_ABI_VERSION 1

typedef enum ssu_status {
    SSU_OK = 0,
    SSU_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, wrong dtype tag, bad config */
    SSU_ERR_UNSUPPORTED = 2,      /* shape or layout the library does not run (see ssu_update) */
    SSU_ERR_MISALIGNED = 3,       /* state or B/C address not aligned for vector access */
    SSU_ERR_HIP = 4,              /* a HIP runtime call failed (launch, device query, copy) */
    SSU_ERR_NO_MEMORY = 5,        /* host allocation failed */
    SSU_ERR_BAD_INDEX = 6         /* ssu_check_indices: duplicate in-range slot ids */
} ssu_status;

typedef enum ssu_dtype {
    SSU_F32 = 0,
    SSU_BF16 = 1,
    SSU_I32 = 2,
    SSU_I64 = 3,
    SSU_F16 = 4 /* IEEE binary16 (ssu_scan activations) */
} ssu_dtype;

/* Problem shape and options, fixed for the life of a handle. */
typedef struct ssu_config {
    int32_t nheads;      /* H >= 1 */
    int32_t headdim;     /* P: a multiple of 16, 16 <= P <= 256 */
    int32_t dstate;      /* N: 16, 32, 64, 128 or 256 */
    int32_t ngroups;     /* G >= 1, divides H; head h uses group h / (H/G) */
    int32_t dt_softplus; /* 1: delta = softplus(dt + dt_bias); 0: delta = dt + dt_bias */
    int32_t tile;        /* -1: launch configuration from the built-in table;
                            >= 0: always use tile #tile (for sweeps; see ssu_tile_info).
                            The environment variable SSU_TILE, read by ssu_create,
                            overrides a -1 here the same way. */
    int32_t device;      /* HIP device ordinal that launches run on (made
                            current for the call, then restored); -1: the
                            device current at each call */
    int32_t reserved;    /* must be 0 */
} ssu_config;

/* A strided view of device memory. Strides are in elements, outermost first;
 * unused trailing entries are ignored. */
typedef struct ssu_view {
    const void *ptr;
    int32_t dtype; /* ssu_dtype */
    int32_t reserved;
    int64_t stride[4];
} ssu_view;

/* One call's operands. Shapes are implied by the handle's config and `batch`;
 * the library cannot see buffer sizes, so the caller guarantees that every
 * view covers its shape.
 *
 *   state   [pool_slots, H, P, N] f32, read and written. stride[3] must be 1;
 *           the pointer and stride[0..2] must be 16-byte multiples.
 *   idx     [batch] i32 or i64 (state_batch_indices). stride[0] must be 1.
 *   x       [batch, H, P] bf16. stride[2] must be 1.
 *   B, C    [batch, G, N] bf16. stride[2] must be 1; the pointer and
 *           stride[0..1] must be 8-byte multiples.
 *   dt      [batch, H, P] bf16, one value per (request, head): stride[2] == 0.
 *   dt_bias [H, P] f32, stride[1] == 0. ptr may be NULL (no bias).
 *   A       [H, P, N] f32, stride[1] == stride[2] == 0.
 *   D       [H, P] f32, stride[1] == 0. ptr may be NULL (no skip term).
 *   out     [batch, H, P] bf16, written. stride[2] must be 1.
 *
 * x, B and C may be views into one packed tensor. Neither out nor the state
 * pool may overlap any input (the kernel reads inputs through the read-only
 * scalar cache), out must not overlap the state, and the state rows of
 * distinct requests must not overlap.
 *
 * dt is read as the aligned 32-bit words that hold its elements (the scalar
 * cache reads whole words), so reading the first or the last element of the
 * view may also read the 2 bytes beside it, just outside the view. An aligned
 * word never crosses a page, so such a read cannot fault wherever the element
 * itself is mapped, and the 2 extra bytes are never used; the caller need not
 * pad dt. A tool that tracks bytes (a sanitizer) may still report the read.
 */
typedef struct ssu_args {
    int32_t batch;      /* >= 0; 0 is a no-op */
    int32_t reserved;   /* must be 0 */
    int64_t pool_slots; /* number of slots in the state pool, >= 0 */
    ssu_view state, idx, x, B, C, dt, dt_bias, A, D, out;
} ssu_args;

/* Operands of a call that advances each request by `ntokens` tokens at once
 * (for example the draft tokens of speculative or multi-token-prediction
 * decoding). As ssu_args, but x, B, C, dt and out carry a token axis:
 *
 *   x    [batch, ntokens, H, P] bf16, stride[3] == 1
 *   B, C [batch, ntokens, G, N] bf16, stride[3] == 1
 *   dt   [batch, ntokens, H, P] bf16, stride[3] == 0
 *   out  [batch, ntokens, H, P] bf16, stride[3] == 1
 *
 * state, idx, dt_bias, A and D are as in ssu_args. Alignment rules extend to
 * the token stride (x: 4-byte multiples; B, C: 8-byte multiples). */
#define SSU_MAX_TOKENS 1024

typedef struct ssu_tokens_args {
    int32_t batch;      /* >= 0; 0 is a no-op */
    int32_t ntokens;    /* 1 .. SSU_MAX_TOKENS */
    int64_t pool_slots; /* number of slots in the state pool, >= 0 */
    ssu_view state, idx, x, B, C, dt, dt_bias, A, D, out;
} ssu_tokens_args;

typedef struct ssu_handle ssu_handle;

/* Description of one launch configuration. */
typedef struct ssu_tile_desc {
    int32_t dstate;          /* N this tile is compiled for */
    int32_t rows_per_wave;   /* state rows (p) each wave64 owns */
    int32_t waves;           /* waves per workgroup */
    int32_t rows_per_group;  /* rows_per_wave * waves */
    int32_t nontemporal;     /* 1: state loads/stores carry the non-temporal hint */
    int32_t xcd_remap;       /* 1: workgroups of neighbouring heads share an XCD */
    int32_t groups_per_cu;   /* residency cap: at most this many workgroups per CU
                                (enforced by reserving unused LDS); 0 = none */
    char name[48];
} ssu_tile_desc;

/* Validate `cfg` and create a handle. Does not touch the GPU.
 * Errors: SSU_ERR_INVALID_ARGUMENT (null, H/P/N/G out of range, G not dividing
 * H, tile index out of range), SSU_ERR_UNSUPPORTED (P or N the library has no
 * kernel for), SSU_ERR_NO_MEMORY. */
ssu_status ssu_create(const ssu_config *cfg, ssu_handle **out);

/* Enqueue one decode step on `stream` (NULL: the null stream).
 *
 * Preconditions the library cannot check without reading device memory (see
 * ssu_check_indices for a debug check): in-range entries of idx are distinct.
 * Entries outside [0, pool_slots) are padding: that request's state is neither
 * read nor written and its out rows are left untouched.
 *
 * Errors (nothing is launched): SSU_ERR_INVALID_ARGUMENT (null handle/args,
 * batch < 0, pool_slots < 0, null required pointer, wrong dtype tag, negative
 * stride, non-zero reserved field), SSU_ERR_UNSUPPORTED (an inner stride that
 * must be 1 is not, a broadcast stride that must be 0 is not),
 * SSU_ERR_MISALIGNED (state or B/C alignment), SSU_ERR_HIP (the launch
 * failed; the stream's state is the runtime's). batch == 0 returns SSU_OK
 * without launching and without reading any view. */
ssu_status ssu_update(const ssu_handle *h, const ssu_args *args, hipStream_t stream);

/* Enqueue `ntokens` decode steps per request in one launch: each request's
 * state is read once, advanced token by token (token t uses x, B, C, dt of
 * token t; out[:, t] is the output after token t) and written once. The
 * result is bitwise identical to `ntokens` successive ssu_update calls with
 * the per-token operands, at 1/ntokens of their state traffic. Same
 * preconditions, padding rule and errors as ssu_update, plus
 * SSU_ERR_INVALID_ARGUMENT for ntokens outside [1, SSU_MAX_TOKENS]. */
ssu_status ssu_update_tokens(const ssu_handle *h, const ssu_tokens_args *args, hipStream_t stream);

/* Release a handle. NULL is a no-op. */
void ssu_destroy(ssu_handle *h);

/* Debug check of idx, not for hot paths and not capturable: copies idx to the
 * host (synchronising `stream`) and returns SSU_ERR_BAD_INDEX if two in-range
 * entries are equal. Entries outside [0, pool_slots) are padding and allowed. */
ssu_status ssu_check_indices(const ssu_args *args, hipStream_t stream);

/* The launch configuration ssu_update would use for `batch` requests
 * (-1 if the handle's shape has none). */
int32_t ssu_select_tile(const ssu_handle *h, int32_t batch);

/* The launch configuration ssu_update_tokens would use for `batch` requests
 * of `ntokens` tokens (-1 if none). */
int32_t ssu_select_tile_tokens(const ssu_handle *h, int32_t batch, int32_t ntokens);

/* Number of compiled launch configurations, and their descriptions. */
int32_t ssu_tile_count(void);
ssu_status ssu_tile_info(int32_t tile, ssu_tile_desc *out);

/* Static string naming a status code. */
const char *ssu_status_string(ssu_status s);

/* The calling thread's most recent error description ("" if none). */
const char *ssu_last_error(void);

/* ---------------------------------------------------------- block copies --
 * Copy whole state blocks between slots, for prefix caching and multi-token
 * prediction in hybrid models (vLLM PR #48110, "[Perf][Hybrid] Vectorize
 * _copy_mamba_state_block to uint64 for temporal", section "Purpose"): for
 * every request r and every tensor k, block src_blocks[r] of tensor k is
 * copied to block dst_blocks[r] of tensor k.
 */

/* One state tensor (for example one layer's conv or temporal state). Block i
 * occupies bytes [base + i * block_stride, base + i * block_stride +
 * block_bytes). base, block_stride and block_bytes must be 16-byte multiples
 * (SSU_ERR_MISALIGNED otherwise: a guardrail, there is no narrow path). */
typedef struct ssu_block_tensor {
    void *base;
    int64_t block_stride; /* bytes, >= block_bytes unless nblocks <= 1 */
    int64_t block_bytes;  /* bytes copied per block (0: tensor skipped) */
    int64_t nblocks;      /* ids outside [0, nblocks) skip that request */
} ssu_block_tensor;

/* Enqueue the copies on `stream`. `tensors` is a host array read during the
 * call only; src_blocks and dst_blocks are device arrays [nreqs] int32.
 * src == dst is a no-op. Preconditions (not checked; the result would depend
 * on the order of the copies): destinations are distinct and no destination is
 * another request's source. tile = -1 uses the default launch configuration;
 * 0 .. ssu_copy_tile_count()-1 forces one (for sweeps). Asynchronous,
 * allocation-free and graph-capturable like ssu_update.
 * Errors: SSU_ERR_INVALID_ARGUMENT (negative sizes, null pointers, tile out of
 * range, overlapping blocks), SSU_ERR_MISALIGNED, SSU_ERR_UNSUPPORTED (more than
 * 2^31 workgroups in one launch), SSU_ERR_HIP. All of them but SSU_ERR_HIP are
 * found before anything is enqueued; more than 32 tensors take one launch per
 * 32, and SSU_ERR_HIP from a later launch leaves the earlier ones enqueued.
 * nreqs == 0 or ntensors == 0 is a no-op. */
ssu_status ssu_copy_blocks(const ssu_block_tensor *tensors, int32_t ntensors, const int32_t *src_blocks,
                           const int32_t *dst_blocks, int32_t nreqs, int32_t tile, hipStream_t stream);

/* Number of compiled copy configurations, and the name of one ("" if out of
 * range). */
int32_t ssu_copy_tile_count(void);
const char *ssu_copy_tile_name(int32_t tile);

/* ------------------------------------------------ selective scan (prefill) --
 * The selective scan over a whole sequence, as used to prefill a request
 * before decoding (COREY: Entropy-Guided Runtime Chunk Scheduling for
 * Selective Scan Kernels, Table 9, Table 17 and Table 18: selective_scan_fn
 * over dim channels with d_state states each, FP16 or BF16 activations, the
 * sequence cut into static chunks with one kernel call per chunk and the
 * state carried between calls). For every request b, channel d and token t in
 * order, with g = d / (dim / ngroups):
 *   Delta  = softplus(delta[b,d,t] + delta_bias[d])   (delta_softplus = 1)
 *          = delta[b,d,t] + delta_bias[d]             (delta_softplus = 0)
 *   h[n]   = h[n] * exp(A[d,n] * Delta) + (Delta * u[b,d,t]) * B[b,g,n,t]
 *   out[t] = sum_n h[n] * C[b,g,n,t] + D[d] * u[b,d,t]
 * h starts from state[b,d,:] and is written back there after the last token,
 * so a sequence may also be scanned piecewise over several calls. Arithmetic
 * is fp32; out is rounded to the activation type (nearest even).
 */
typedef struct ssu_scan_args {
    int32_t batch;          /* >= 0 (0: no-op) */
    int32_t dim;            /* channels, >= 1 */
    int32_t dstate;         /* states per channel, 1 .. 64 */
    int32_t ngroups;        /* B/C groups, divides dim */
    int64_t seqlen;         /* L >= 0 tokens (0: nothing to do) */
    int32_t delta_softplus; /* 1 or 0, see above */
    int32_t reserved;       /* must be 0 */
    ssu_view state;         /* [batch, dim, dstate] F32, read and written; stride[2] == 1 */
    ssu_view u;             /* [batch, dim, L] F16 or BF16; stride[2] == 1 */
    ssu_view delta;         /* [batch, dim, L], u's dtype; stride[2] == 1 */
    ssu_view B;             /* [batch, ngroups, dstate, L], u's dtype; stride[3] == 1 */
    ssu_view C;             /* [batch, ngroups, dstate, L], u's dtype; stride[3] == 1 */
    ssu_view A;             /* [dim, dstate] F32, finite */
    ssu_view D;             /* [dim] F32, contiguous; ptr may be NULL (no skip term) */
    ssu_view delta_bias;    /* [dim] F32, contiguous; ptr may be NULL (no bias) */
    ssu_view out;           /* [batch, dim, L], u's dtype, written; stride[2] == 1 */
} ssu_scan_args;

/* Enqueue the scan of `args` on `stream`, chunk after chunk of `chunk` tokens
 * (chunk = 0: the whole sequence), in order, the state carried between them
 * through `state`; a chunk is one kernel launch, or two when it ends in a
 * ragged or unaligned rest (its whole blocks, then the rest). Chunks whose
 * size is a multiple of 512 give bitwise the same results as one launch;
 * other chunk sizes agree within rounding. Every configuration with the same
 * token segment gives the same bits, so a request's results do not depend on
 * the batch it is scanned in. tile = -1 picks the launch configuration from
 * the chunk size and the number of channels; 0 .. ssu_scan_tile_count()-1
 * forces one.
 * Memory: the caller owns every buffer; the library allocates nothing and
 * keeps no pointer after the call. out and state must not overlap each other
 * or any input (the kernel reads inputs through the read-only cache).
 * Asynchronous and graph-capturable; nothing is checked on the device.
 * Errors (nothing is launched): SSU_ERR_INVALID_ARGUMENT (null pointers,
 * negative sizes or strides, wrong dtypes, non-zero reserved fields,
 * dim % ngroups != 0, tile out of range), SSU_ERR_UNSUPPORTED (non-contiguous
 * token or state axis, D or delta_bias, dstate > 64, batch * dim >= 2^31; a
 * forced staged or paired configuration when the channels of a group do not
 * split into its workgroups' 2, 4 or 8, or when B's or C's state stride is
 * 2^24 elements or more),
 * SSU_ERR_MISALIGNED (elements not aligned to their size), SSU_ERR_HIP
 * (launch failure; earlier chunks may have run). */
ssu_status ssu_scan(const ssu_scan_args *args, int64_t chunk, int32_t tile, hipStream_t stream);

/* Number of compiled scan configurations, and the name of one ("" if out of
 * range). */
int32_t ssu_scan_tile_count(void);
const char *ssu_scan_tile_name(int32_t tile);

/* The configuration ssu_scan(args, chunk, -1, ...) launches, from the tokens
 * one launch spans (chunk, or L if chunk is 0 or longer), the number of
 * channels (batch * dim), the channels of a group (dim / ngroups), dstate and
 * B's and C's state strides; only those fields of `args` are read (no
 * pointer is touched). Returns -1 if args is null or those sizes are invalid (negative
 * chunk, batch, seqlen or strides, dim or ngroups below 1, ngroups not
 * dividing dim). */
int32_t ssu_scan_select_tile(const ssu_scan_args *args, int64_t chunk);

/* SSU_ABI_VERSION of the built library. */
int32_t ssu_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SSU_H */
