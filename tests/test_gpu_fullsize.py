"""GPU path vs the oracle at the workloads' full sizes, in the launch configuration
the benchmark times (echo_layer_step, EMA prefetch on).

Every output of every step is compared, as in test_gpu_parity: scores within the
tolerance of echo_harness, and everything decided from them -- prefetch lists,
top-k, EMA state, misses, evictions, maps, priorities, free flags, the free list
and the GPU-pool bytes -- bit for bit, with the oracle fed the GPU's scores.
"""
import numpy as np
import pytest
import torch

from synth import get

from . import echo_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)


def _run(rig, steps, mode):
    for t in range(steps):
        out, o = rig.step_and_compare(mode)
        _say(f"  step {t}: status {out['status']}, selected {int(out['n_sel'].sum())}, "
             f"prefetched {int(out['n_pf'].sum())}, missed {int(out['n_miss'].sum())}, "
             f"evicted {int(o['n_evict'])}")
        assert out["status"] == 0


@pytest.mark.timeout(600)
def test_single_layer_full_size():
    # batch 8 x 65,536 tokens, 64 x 128 indexer, k = 2048, 200,000 slots, 2M host tokens
    _say("single_layer: 8 x 64K, EMA, 3 steps")
    rig = H.Rig(get("single_layer"), steps=3)
    _run(rig, 3, H.MODE_EMA)
    assert sum(int(out["n_pf"].sum()) for out, _ in rig.history[1:]) > 0  # prefetch ran
    rig.close()


@pytest.mark.timeout(900)
def test_capacity_one_layer_full_size():
    # one layer of the capacity workload as the benchmark runs it: batch 32, ctx
    # U[80K, 100K], 110,000 slots, 3.2M host tokens, prefetch cap ceil(ctx / 256); the
    # pool fills up over the first steps (65,536 cold misses, then about 10,000
    # prefetched rows a step) and the reserve for the next prefetch makes the fifth
    # step evict
    _say("capacity, layer 30: 32 x U[80K,100K], EMA, 5 steps")
    rig = H.Rig(get("capacity"), steps=5, layer=30)
    _run(rig, 5, H.MODE_EMA)
    assert sum(int(o["n_evict"]) for _, o in rig.history) > 0
    rig.close()


@pytest.mark.timeout(900)
def test_low_locality_full_size_and_lossless_ablation():
    # batch 16 x 100K, rho 0.5 (low locality): EMA prefetch against the oracle, then the
    # same steps with prefetch off select the same tokens and gather the same bytes
    wl = get("low_locality")
    steps = 3
    _say("low_locality: 16 x 100K, EMA, 3 steps")
    rig = H.Rig(wl, steps=steps)
    ema = []
    for t in range(steps):
        out, o = rig.step_and_compare(H.MODE_EMA)
        assert out["status"] == 0
        _say(f"  step {t}: prefetched {int(out['n_pf'].sum())}, missed {int(out['n_miss'].sum())}")
        ema.append((out["sel_tok"].copy(), out["n_sel"].copy(), rig.gathered()))
    assert sum(int(out["n_pf"].sum()) for out, _ in rig.history[1:]) > 0
    rig.close()
    _say("low_locality: same steps, prefetch off")
    rig = H.Rig(wl, steps=steps)
    for t in range(steps):
        rig.gpu_step(H.MODE_POS_INF)
        out = rig.ws.read(rig.B)
        assert out["status"] == 0
        sel, nsel, rows = ema[t]
        assert np.array_equal(out["n_sel"], nsel)
        for b in range(rig.B):
            n = int(nsel[b])
            assert np.array_equal(out["sel_tok"][b, :n], sel[b, :n]), (t, b)
        assert all(np.array_equal(x, y) for x, y in zip(rig.gathered(), rows)), t
    rig.close()


@pytest.mark.timeout(900)
def test_capacity_one_layer_full_size_paged():
    # the same layer with a page table: every 16-id page of the 3.2M-token host pool
    # moved to a random other page (K and latent rows move with it), so each request's
    # tokens lie on pages scattered over the whole pool
    _say("capacity, layer 30, page tables: 32 x U[80K,100K], EMA, 3 steps")
    rig = H.Rig(get("capacity"), steps=3, layer=30, paged=True)
    _run(rig, 3, H.MODE_EMA)
    assert sum(int(out["n_pf"].sum()) for out, _ in rig.history[1:]) > 0
    rig.close()
