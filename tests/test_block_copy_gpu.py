"""ssu_copy_blocks on the GPU against the CPU oracle, bitwise."""
import numpy as np
import pytest

from . import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


def _tensors(rng, nblocks, shapes):
    """Host arrays (the oracle's copies) and device tensors of the same bits."""
    torch = gu.torch_mod()
    host, dev = [], []
    for shp, dt in shapes:
        a = rng.integers(0, 2 ** 16, size=(nblocks, *shp), dtype=np.uint16).view(dt)
        host.append(a.copy())
        dev.append(torch.from_numpy(a.view(np.int16).copy()).cuda())
    return host, dev


def _ids(rng, nblocks, nreqs):
    perm = rng.permutation(nblocks).astype(np.int32)
    return perm[:nreqs].copy(), perm[nreqs:2 * nreqs].copy()


def _check(ref, host, dev, src, dst, tile=-1):
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    ssu.copy_blocks(dev, torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda(), tile=tile)
    torch.cuda.synchronize()
    ref.copy_blocks(host, src, dst)
    for k, (h, d) in enumerate(zip(host, dev)):
        got = d.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, h.view(np.uint16)), f"tensor {k} differs"


# block shapes (in 16-bit units, so bytes = 2 * prod): small, exactly one
# chunk, several chunks with a ragged tail, 2 MiB
SHAPES = [((8,), np.uint16), ((4096, 2), np.uint16), ((3, 5000), np.uint16), ((1024, 1024), np.uint16),
          ((40, 1024), np.uint16)]


@pytest.mark.parametrize("nreqs", [1, 3, 17])
def test_copy_matches_oracle(ref, nreqs):
    rng = np.random.Generator(np.random.PCG64(40 + nreqs))
    host, dev = _tensors(rng, 2 * nreqs + 3, SHAPES)
    src, dst = _ids(rng, 2 * nreqs + 3, nreqs)
    _check(ref, host, dev, src, dst)


def test_copy_skip_noop_and_many_tensors(ref):
    rng = np.random.Generator(np.random.PCG64(50))
    shapes = [((8 * (k + 1),), np.uint16) for k in range(40)]  # 40 tensors: two launches
    host, dev = _tensors(rng, 12, shapes)
    src = np.array([1, -1, 5, 7, 11], dtype=np.int32)
    dst = np.array([2, 3, 5, 12, 0], dtype=np.int32)  # skip, no-op, out-of-range dst
    _check(ref, host, dev, src, dst)


def test_copy_strided_tensor(ref):
    """A layer's view of a larger cache: blocks not adjacent; bytes between
    blocks must not change."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    rng = np.random.Generator(np.random.PCG64(51))
    big = rng.standard_normal((10, 3, 256)).astype(np.float32)
    dbig = torch.from_numpy(big.copy()).cuda()
    view_h, view_d = big[:, 1], dbig[:, 1]
    src, dst = np.array([2, 7], dtype=np.int32), np.array([4, 9], dtype=np.int32)
    ssu.copy_blocks([view_d], torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    ref.copy_blocks([view_h], src, dst)
    assert np.array_equal(dbig.cpu().numpy(), big)


def test_copy_every_tile(ref):
    import selective_state_update_amd as ssu

    rng = np.random.Generator(np.random.PCG64(52))
    names = ssu.copy_tiles()
    assert names
    for tile in range(len(names)):
        host, dev = _tensors(rng, 9, SHAPES[:3])
        src, dst = _ids(rng, 9, 4)
        _check(ref, host, dev, src, dst, tile=tile)


def test_copy_page_layout_sample(ref):
    """The vLLM page's per-request layout (24 layers x (2 MiB fp32 temporal +
    80 KiB bf16 conv)) at 8 requests, checked in full."""
    rng = np.random.Generator(np.random.PCG64(53))
    shapes = [((64, 128, 128), np.uint16)] * 24 + [((40960,), np.uint16)] * 24  # 2 MiB and 80 KiB
    host, dev = _tensors(rng, 16, shapes)
    src, dst = _ids(rng, 16, 8)
    _check(ref, host, dev, src, dst)


def test_copy_hip_graph_replays(ref):
    """Copies captured in one HIP graph and replayed three times, the source
    blocks changed by eager work before each replay: every replay copies the
    current sources (checked against the oracle on the same host bits)."""
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    rng = np.random.Generator(np.random.PCG64(54))
    host, dev = _tensors(rng, 11, SHAPES[:3])
    src, dst = _ids(rng, 11, 4)
    s_d, d_d = torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda()
    src_rows = torch.from_numpy(src.astype(np.int64)).cuda()
    descs = ssu.block_tensors(dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ssu.copy_blocks(dev, s_d, d_d, descs=descs)  # warm-up, applied to the host copy too
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref.copy_blocks(host, src, dst)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ssu.copy_blocks(dev, s_d, d_d, descs=descs)
    torch.cuda.synchronize()
    for k in range(3):
        for h_, d_ in zip(host, dev):
            new = rng.integers(0, 2 ** 16, size=h_[src].shape, dtype=np.uint16)
            h_[src] = new
            d_[src_rows] = torch.from_numpy(new.view(np.int16)).cuda()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref.copy_blocks(host, src, dst)
        for j, (h_, d_) in enumerate(zip(host, dev)):
            assert np.array_equal(d_.cpu().numpy().view(np.uint16), h_.view(np.uint16)), f"replay {k} tensor {j}"
