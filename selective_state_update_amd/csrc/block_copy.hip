// block_copy.hip -- ssu_copy_blocks: copy SSM state blocks between slots on
// MI355X (gfx950).
//
// The copy serves prefix caching and multi-token prediction in hybrid models
// (vLLM PR #48110, "[Perf][Hybrid] Vectorize _copy_mamba_state_block to
// uint64 for temporal", section "Purpose"): for every request r and every
// state tensor k (the conv and temporal state of each linear-attention layer),
// block src[r] of tensor k is copied to block dst[r]. The page's point is that
// the copy is HBM-bound and needs wide transactions; here every lane moves
// 16-byte chunks (dwordx4), non-temporal, U of them in flight.
//
// Work split: each tensor's block is cut into chunks of U x 256 x 16 bytes;
// one 256-thread workgroup copies one chunk of one tensor for one request,
// U dwordx4 loads per lane issued before any store. Workgroup ids run over
// (request, chunk of tensor 0, chunk of tensor 1, ...); tensors are passed by
// value in the kernel arguments, up to kMaxTensors per launch.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <vector>

#include "internal.h"

namespace ssu {
namespace {

constexpr int kMaxTensors = 32;
constexpr int kThreads = 256;

struct TensorDesc {
    char *base;
    int64_t stride, bytes, nblocks;
};

struct CopyParams {
    TensorDesc t[kMaxTensors];
    int32_t first_chunk[kMaxTensors + 1];  // chunk index where tensor k starts, per request
    const int32_t *src;
    const int32_t *dst;
    int32_t ntensors, chunks_per_req, total, xcd_remap;
};

template <int U>
__global__ void __launch_bounds__(kThreads) ssu_copy_blocks_kernel(const CopyParams p)
{
    constexpr int64_t CHUNK = int64_t(U) * kThreads * 16;
    int g = static_cast<int>(blockIdx.x);
    if (p.xcd_remap)
        g = xcd_order(g, p.total);
    const int r = g / p.chunks_per_req;
    const int c = g - r * p.chunks_per_req;
    int k = 0;
    while (k + 1 < p.ntensors && c >= p.first_chunk[k + 1])
        ++k;
    const TensorDesc T = p.t[k];
    const int64_t s = load_ro(p.src + r);
    const int64_t d = load_ro(p.dst + r);
    if (s == d || s < 0 || s >= T.nblocks || d < 0 || d >= T.nblocks)
        return;  // no-op or skipped request
    const int64_t off = static_cast<int64_t>(c - p.first_chunk[k]) * CHUNK;
    const int64_t left = T.bytes - off;
    const float *sp = reinterpret_cast<const float *>(T.base + s * T.stride + off);
    float *dp = reinterpret_cast<float *>(T.base + d * T.stride + off);
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t o = (static_cast<int64_t>(u) * kThreads + threadIdx.x) * 16;
        if (o < left)
            v[u] = load4<true>(sp + o / 4);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t o = (static_cast<int64_t>(u) * kThreads + threadIdx.x) * 16;
        if (o < left)
            store4<true>(dp + o / 4, v[u]);
    }
}

using CopyFn = hipError_t (*)(const CopyParams &, int grid, size_t lds, hipStream_t);

template <int U>
hipError_t launch_copy(const CopyParams &p, int grid, size_t lds, hipStream_t stream)
{
    hipLaunchKernelGGL((ssu_copy_blocks_kernel<U>), dim3(grid), dim3(kThreads), lds, stream, p);
    return hipGetLastError();
}

struct CopyTile {
    int u, cap, remap;
    int64_t chunk;
    CopyFn fn;
    char name[32];
};

template <int U>
void add_copy_tiles(std::vector<CopyTile> &v)
{
    for (int remap : {1, 0})
        for (int cap : {0, 4, 6, 8}) {
            if (!remap && cap)
                continue;
            CopyTile t{};
            t.u = U;
            t.cap = cap;
            t.remap = remap;
            t.chunk = int64_t(U) * kThreads * 16;
            t.fn = &launch_copy<U>;
            if (cap)
                std::snprintf(t.name, sizeof t.name, "copy_u%d%s_g%d", U, remap ? "_xcd" : "", cap);
            else
                std::snprintf(t.name, sizeof t.name, "copy_u%d%s", U, remap ? "_xcd" : "");
            v.push_back(t);
        }
}

const std::vector<CopyTile> &copy_tiles()
{
    static const std::vector<CopyTile> table = [] {
        std::vector<CopyTile> v;
        add_copy_tiles<1>(v);
        add_copy_tiles<2>(v);
        add_copy_tiles<4>(v);
        add_copy_tiles<8>(v);
        return v;
    }();
    return table;
}

// Default copy configuration, from a sweep of every configuration on MI355X
// (24 x (2 MiB + 80 KiB) blocks per request, cold HBM): two dwordx4 per lane
// (8 KiB per workgroup), XCD-ordered, uncapped, is the fastest at 8, 32 and
// 128 requests (75.8%, 78.3%, 80.1% of peak); four per lane 71-77%, eight
// 47-49%, one 54-56%.
int default_copy_tile()
{
    const auto &t = copy_tiles();
    for (size_t i = 0; i < t.size(); ++i)
        if (t[i].u == 2 && t[i].remap == 1 && t[i].cap == 0)
            return static_cast<int>(i);
    return 0;
}

}  // namespace
}  // namespace ssu

extern "C" {

int32_t ssu_copy_tile_count(void) { return static_cast<int32_t>(ssu::copy_tiles().size()); }

const char *ssu_copy_tile_name(int32_t tile)
{
    if (tile < 0 || tile >= ssu_copy_tile_count())
        return "";
    return ssu::copy_tiles()[tile].name;
}

ssu_status ssu_copy_blocks(const ssu_block_tensor *tensors, int32_t ntensors, const int32_t *src_blocks,
                           const int32_t *dst_blocks, int32_t nreqs, int32_t tile, hipStream_t stream)
{
    using namespace ssu;
    if (ntensors < 0 || nreqs < 0)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_copy_blocks: negative ntensors %d / nreqs %d", ntensors, nreqs);
    if (tile < -1 || tile >= ssu_copy_tile_count())
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_copy_blocks: tile %d out of range", tile);
    if (ntensors == 0 || nreqs == 0)
        return SSU_OK;
    if (!tensors || !src_blocks || !dst_blocks)
        return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_copy_blocks: null tensors or block ids");
    for (int32_t k = 0; k < ntensors; ++k) {
        const ssu_block_tensor &t = tensors[k];
        if (t.block_bytes < 0 || t.nblocks < 0 || t.block_stride < 0)
            return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_copy_blocks: tensor %d: negative size", k);
        if (t.block_bytes == 0 || t.nblocks == 0)
            continue;
        if (!t.base)
            return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_copy_blocks: tensor %d: null base", k);
        if (reinterpret_cast<uintptr_t>(t.base) % 16 || t.block_stride % 16 || t.block_bytes % 16)
            return fail(SSU_ERR_MISALIGNED,
                        "ssu_copy_blocks: tensor %d: base, block stride and block bytes must be 16-byte multiples", k);
        if (t.nblocks > 1 && t.block_bytes > t.block_stride)
            return fail(SSU_ERR_INVALID_ARGUMENT, "ssu_copy_blocks: tensor %d: blocks overlap (bytes > stride)", k);
    }
    const CopyTile &T = copy_tiles()[tile >= 0 ? tile : default_copy_tile()];
    size_t lds = 0;
    if (T.cap > 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess)
            return fail(SSU_ERR_HIP, "hipGetDevice failed");
        const DeviceLimits lim = device_limits(dev);
        if (lim.lds_cu <= 0)
            return fail(SSU_ERR_HIP, "cannot query the LDS size of device %d", dev);
        lds = lds_for_cap(T.cap, lim.lds_cu, lim.lds_block);
    }
    // Launch over groups of up to kMaxTensors tensors. Every group's size is
    // checked before the first launch, so a size error enqueues nothing.
    auto group_chunks = [&](int32_t k0, CopyParams *p) -> int64_t {
        int64_t chunks = 0;
        int32_t n = 0;
        for (int32_t k = k0; k < ntensors && n < kMaxTensors; ++k, ++n) {
            const ssu_block_tensor &t = tensors[k];
            const int64_t bytes = (t.block_bytes > 0 && t.nblocks > 0) ? t.block_bytes : 0;
            if (p) {
                p->t[n].base = static_cast<char *>(t.base);
                p->t[n].stride = t.block_stride;
                p->t[n].bytes = bytes;
                p->t[n].nblocks = t.nblocks;
                p->first_chunk[n] = static_cast<int32_t>(chunks);
            }
            chunks += (bytes + T.chunk - 1) / T.chunk;
            if (chunks > 0x7fffffff)
                return -1;
        }
        if (p) {
            p->first_chunk[n] = static_cast<int32_t>(chunks);
            p->ntensors = n;
        }
        return chunks;
    };
    for (int32_t k0 = 0; k0 < ntensors; k0 += kMaxTensors) {
        const int64_t chunks = group_chunks(k0, nullptr);
        if (chunks < 0 || chunks * nreqs > 0x7fffffff)
            return fail(SSU_ERR_UNSUPPORTED, "ssu_copy_blocks: more than 2^31 workgroups in one launch");
    }
    for (int32_t k0 = 0; k0 < ntensors; k0 += kMaxTensors) {
        CopyParams p{};
        p.src = src_blocks;
        p.dst = dst_blocks;
        p.xcd_remap = T.remap;
        const int64_t chunks = group_chunks(k0, &p);
        if (chunks == 0)
            continue;
        const int64_t total = chunks * nreqs;
        p.chunks_per_req = static_cast<int32_t>(chunks);
        p.total = static_cast<int32_t>(total);
        const hipError_t e = T.fn(p, static_cast<int>(total), lds, stream);
        if (e != hipSuccess)
            return fail(SSU_ERR_HIP, "launch of %s failed: %s", T.name, hipGetErrorString(e));
    }
    return SSU_OK;
}

}  // extern "C"
