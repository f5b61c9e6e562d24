"""The 920-point sweep: heads {8,16,32,64,128} x batch {1..64, then every 8 up
to 1024}, P=64, N=128 — the grid over which sglang PR #41223 ("Kernel
measurement", and the "Correctness Verification" table) checked that launch
configurations give bitwise-identical output and state.

At every point, in the launch configuration the library picks:
  * every request against the CPU oracle, state and out, at the points that
    move at most 256 MiB of state per call (batch x heads <= 8192: 528 of the
    920 points); three sampled requests (all heads) at the larger points;
  * untouched pool slots bitwise unchanged;
  * a rerun from the restored pool bitwise identical (determinism);
  * a run in a different launch configuration bitwise identical.
"""
import numpy as np
import pytest

import ssu_inputs as si

from . import gpu_util as gu

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BATCHES = sorted({bs for (_, bs) in si.sweep_points()})
# (request, head) units up to which every request is compared with the oracle
FULL_CHECK_UNITS = 8192


@pytest.fixture(autouse=True)
def _gpu():
    gu.require_gpu()


def _alt_tile(ssu, auto_id):
    """A configuration unlike the auto one: plain (temporal) access, 8 row
    pairs per wave, one wave per group."""
    for t in ssu.tiles():
        if t["dstate"] == 128 and t["name"] == "n128_r16_w1":
            assert t["id"] != auto_id
            return t["id"]
    raise AssertionError("reference tile missing")


@pytest.mark.parametrize("H", [8, 16, 32, 64, 128])
def test_sweep_heads(ref, H):
    import selective_state_update_amd as ssu

    torch = gu.torch_mod()
    h_auto = ssu.Handle(H, 64, 128, 1, True, -1)
    h_alt = None
    checked = full = 0
    for bs in BATCHES:
        seed = si.sweep_seed(H, bs)
        slots = 2 * bs
        p = si.make_problem(H=H, P=64, N=128, G=1, batch=bs, pool_slots=slots, seed=seed, host_pool=False)
        pool = torch.empty((slots, H, 64, 128), device="cuda")
        si.draw_pool_on_device(pool, seed)
        backup = pool.clone()
        dp = gu.DeviceProblem(p, pool=pool)
        idx_t = dp.idx.to(torch.int64)
        out = dp.run(h_auto)
        torch.cuda.synchronize()

        # every request (or three sampled ones at the larger points) against the oracle
        if bs * H <= FULL_CHECK_UNITS:
            sample = np.arange(bs)
            full += 1
        else:
            rng = np.random.Generator(np.random.PCG64(seed))
            sample = np.sort(rng.choice(bs, size=min(bs, 3), replace=False))
        sl = idx_t[torch.from_numpy(sample).cuda()]
        before = backup[sl].cpu().numpy()
        after = pool[sl].cpu().numpy()
        r = ref.run(before.copy(), np.arange(len(sample), dtype=np.int32), p.x[sample], p.B[sample],
                    p.C[sample], p.dt[sample], p.A, p.dt_bias, p.D)
        gu.assert_state(after, r["state"], f"H{H} bs{bs}")
        gu.assert_out(gu.bits(out)[sample], r, f"H{H} bs{bs}")

        # untouched slots
        mask = torch.ones(slots, dtype=torch.bool, device="cuda")
        mask[idx_t] = False
        assert torch.equal(pool[mask].view(torch.int32), backup[mask].view(torch.int32)), f"H{H} bs{bs}"

        # rerun and another launch configuration: bitwise
        first_state = pool[idx_t].clone()
        first_out = out.clone()
        if h_alt is None:
            h_alt = ssu.Handle(H, 64, 128, 1, True, _alt_tile(ssu, h_auto.selected_tile(bs)))
        for h in (h_auto, h_alt):
            pool.copy_(backup)
            o = dp.run(h, out=torch.empty_like(out))
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int16), first_out.view(torch.int16)), f"H{H} bs{bs} out"
            assert torch.equal(pool[idx_t].view(torch.int32), first_state.view(torch.int32)), f"H{H} bs{bs} state"
        checked += 1
        del pool, backup, dp, first_state
    torch.cuda.empty_cache()
    print(f"H{H}: {checked} points, every request against the oracle at {full} "
          f"(batch x heads <= {FULL_CHECK_UNITS}), three sampled requests at {checked - full}", flush=True)
    assert checked == len(BATCHES) == 184
    assert full == sum(1 for bs in BATCHES if bs * H <= FULL_CHECK_UNITS)
