"""Request release and admission (echo_release, echo_admit) against the oracle,
through the C ABI, in the middle of decoding.

After every call the status, the batch rows (host_base, ctx_len), the maps, the
priorities, the free flags, the thresholds and the ascending free list must equal
the oracle's; the decode steps around the calls are compared bit for bit as in
test_gpu_parity (selection, prefetch, misses, eviction, maps, GPU-pool bytes), so a
released request's slots are reused by the others and a re-admitted request starts
cold while every selected row the attention reads stays equal to the host copy.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
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


def _rig(ctx, steps, n_gpu, n_host, top_k=256, cap_div=64, rho=0.6):
    wl = get("single_layer").scaled(rho=rho, steps=steps)
    return H.Rig(wl, steps=steps, ctx=ctx, n_gpu=n_gpu, n_host=n_host, top_k=top_k,
                 cap_div=cap_div, max_ctx=max(ctx))


def _lossless(rig, out):
    rows = rig.gathered()
    for b in range(rig.B):
        n = int(out["n_sel"][b])
        hs = rig.host_ids(b, out["sel_tok"][b, :n])
        assert np.array_equal(rows[b], rig.orc_host[hs]), ("attention input", b)


@pytest.mark.parametrize("mode", [H.MODE_EMA, H.MODE_NEG_INF])
def test_release_and_readmit_mid_decode(mode):
    # three ragged requests, a pool small enough to evict: request 1 is cancelled
    # after three steps and admitted again (same host range) two steps later
    ctx = [3000, 1777, 2561]
    steps = 8
    _say(f"release/readmit, ctx {ctx}, mode {mode}")
    rig = _rig(ctx, steps, n_gpu=3 * 256 + 2 * 120, n_host=8000)
    base1 = int(rig.base[1])
    for t in range(steps):
        if t == 3:
            assert rig.release_and_compare([0, 1, 0]) == O.OK
            assert int(rig.ctx[1]) == 0
        if t == 5:
            assert rig.admit_and_compare(1, base1, 1777) == O.OK
        out, o = rig.step_and_compare(mode)
        _say(f"  step {t}: selected {list(out['n_sel'])}, missed {list(out['n_miss'])}, "
             f"prefetched {list(out['n_pf'])}, evicted {int(o['n_evict'])}")
        _lossless(rig, out)
        if t == 3:
            assert out["n_sel"][1] == 0
        if t == 5 and mode == H.MODE_EMA:  # cold: nothing resident, no estimate yet
            assert out["n_pf"][1] == 0 and out["n_miss"][1] == out["n_sel"][1] == 256
    rig.close()


def test_release_everything_then_admit_new_ranges():
    ctx = [2000, 1500]
    steps = 6
    _say("release everything, admit at new ranges")
    rig = _rig(ctx, steps, n_gpu=1200, n_host=8000)
    for _ in range(2):
        rig.step_and_compare(H.MODE_EMA)
    assert rig.release_and_compare([1, 1]) == O.OK
    st = rig.layer.state()
    assert (st["h2g"] == -1).all() and (st["free"] == 1).all() and st["nfree"] == 1200
    assert np.array_equal(st["idxbuf"], np.arange(1200))
    # the two requests swap places in the host pool (both ranges hold keys already)
    assert rig.admit_and_compare(0, 2000, 1500) == O.OK
    assert rig.admit_and_compare(1, 0, 2000) == O.OK
    for _ in range(3):
        out, _ = rig.step_and_compare(H.MODE_EMA)
        _lossless(rig, out)
    rig.close()


def test_release_without_commit_then_with_commit():
    # the non-last layers of a step release with commit = 0: maps and slots go,
    # the batch row stays for the next layer's call; the last call empties it
    ctx = [1000, 1200]
    _say("release without commit, then with")
    rig = _rig(ctx, 4, n_gpu=2048, n_host=4096)
    rig.step_and_compare(H.MODE_EMA)
    rig.step_and_compare(H.MODE_EMA)
    assert rig.release_and_compare([1, 0], commit=False) == O.OK
    assert list(rig.ctx) == ctx
    assert rig.release_and_compare([1, 0]) == O.OK
    assert list(rig.ctx) == [0, 1200]
    rig.step_and_compare(H.MODE_EMA)
    rig.close()


def test_admission_errors_change_nothing():
    ctx = [1000, 1200, 900]
    _say("admission errors")
    rig = _rig(ctx, 4, n_gpu=2048, n_host=4096)
    rig.step_and_compare(H.MODE_EMA)
    rig.step_and_compare(H.MODE_EMA)
    base = [int(x) for x in rig.base]
    # host-side checks: nothing enqueued
    for b, bs, n in ((3, 0, 10), (-1, 0, 10), (1, 0, rig.dims.max_ctx + 1), (1, -5, 10),
                     (1, 4090, 10)):
        assert rig.admit_and_compare(b, bs, n, expect_status=O.EINVAL) == O.EINVAL
    # the row is still in use
    assert rig.admit_and_compare(1, 3800, 10, expect_status=O.EDEVARG) == O.EDEVARG
    rig.ws.reset()
    # release row 1, then try to admit it over request 2's range
    assert rig.release_and_compare([0, 1, 0]) == O.OK
    assert rig.admit_and_compare(1, base[2] + 100, 50, expect_status=O.ECAPACITY) == \
        O.ECAPACITY
    rig.ws.reset()
    # request 2 emptied by hand, without a release: its tokens stay mapped
    rig.ctx[2] = 0
    rig.batch.ctx[2] = 0
    assert rig.admit_and_compare(1, base[2], 900, expect_status=O.EDEVARG) == O.EDEVARG
    rig.ws.reset()
    rig.ctx[2] = 900
    rig.batch.ctx[2] = 900
    # a free range between the requests' ranges is fine
    assert rig.admit_and_compare(1, base[1], 1200) == O.OK
    rig.step_and_compare(H.MODE_EMA)
    rig.close()


def test_release_rejects_a_range_that_does_not_fit():
    ctx = [1000, 1200]
    _say("release of a bad range")
    rig = _rig(ctx, 3, n_gpu=2048, n_host=4096)
    rig.step_and_compare(H.MODE_EMA)
    rig.ctx[1] = rig.dims.max_ctx + 1      # a corrupted batch row, on both sides
    rig.batch.ctx[1] = rig.dims.max_ctx + 1
    assert rig.release_and_compare([1, 1], expect_status=O.EDEVARG) == O.EDEVARG
    rig.ws.reset()
    rig.ctx[1] = 1200
    rig.batch.ctx[1] = 1200
    assert rig.release_and_compare([1, 1]) == O.OK
    rig.close()


@pytest.mark.timeout(600)
def test_release_at_scale_with_eviction_pressure():
    # eight requests of 20,000 tokens with k = 2048 and a pool that must evict;
    # half are cancelled, the others decode on and take over their slots
    ctx = [20000] * 8
    steps = 5
    _say("release at scale: 8 x 20,000, k = 2048")
    wl = get("single_layer").scaled(rho=0.5, steps=steps)
    rig = H.Rig(wl, steps=steps, ctx=ctx, n_gpu=8 * 2048 + 8 * 157 + 512, n_host=170000,
                max_ctx=20000)
    for t in range(steps):
        if t == 2:
            assert rig.release_and_compare([1, 0, 1, 0, 1, 0, 1, 0]) == O.OK
        if t == 4:
            assert rig.admit_and_compare(2, int(rig.base[2]), 20000) == O.OK
        out, o = rig.step_and_compare(H.MODE_EMA)
        _say(f"  step {t}: missed {int(out['n_miss'].sum())}, evicted {int(o['n_evict'])}")
        _lossless(rig, out)
    rig.close()


@pytest.mark.parametrize("mode", [H.MODE_EMA, H.MODE_NEG_INF])
def test_append_skips_released_row_until_readmitted(mode):
    # Request 1 (host ids 3008 ..) is cancelled at step 2.  The decode appends that
    # follow must leave its empty row alone (no token, no growth), and its stale base
    # must not block request 0, which grows into ids 3008 .. 3011 from step 4 on.
    # At step 5 request 1 is admitted again, at 3024 (clear of request 0's growth),
    # over 1761 tokens whose keys are already in place, and grows with the others.
    ctx = [3004, 1777, 2561]
    steps = 8
    _say(f"append around a released row, mode {mode}")
    wl = get("single_layer").scaled(rho=0.6, steps=steps)
    rig = H.Rig(wl, steps=steps, ctx=ctx, n_gpu=3 * 256 + 2 * 120, n_host=8000, top_k=256,
                cap_div=64, max_ctx=max(ctx) + steps)
    assert list(rig.base) == [0, 3008, 4800]
    for t in range(steps):
        if t == 2:
            assert rig.release_and_compare([0, 1, 0]) == O.OK
        if t == 5:
            assert int(rig.ctx[1]) == 0
            assert rig.admit_and_compare(1, 3024, 1761) == O.OK
        out, o = rig.step_and_compare(mode)
        _lossless(rig, out)
        assert rig.append_and_compare() == O.OK
        _say(f"  step {t}: ctx {list(rig.ctx)}, missed {list(out['n_miss'])}")
    assert list(rig.ctx) == [3004 + steps, 1761 + 3, 2561 + steps]
    rig.close()
