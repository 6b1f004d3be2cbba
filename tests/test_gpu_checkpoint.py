"""Checkpoint and resume of a layer's cache-management state.

The ECHO review ("Critical analysis / systemic flaws") leaves fault recovery open and
notes that the full host copy of the cache is not a persistence mechanism.  Between
calls a layer's state is in its own buffers (the five metadata arrays, the GPU pool,
the thresholds, the selection guard, the step counter and free-list length, and the
running totals); the workspace carries nothing across steps.  So a byte copy of
those buffers is a checkpoint: after some steps (checked against the oracle) the
state is copied, more steps run (also checked), and then the copy is written back,
into the same layer with a fresh workspace and into a second layer at other
addresses; the steps replayed from there must give bit-identical outputs, state,
pool bytes and totals.
"""
import numpy as np
import pytest
import torch

from kv_cache_offload_fp8_amd import abi
from kv_cache_offload_fp8_amd import runtime as R
from synth import get

from . import echo_harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _record(rig, layer, ws):
    """Everything a step leaves behind: outputs, scores, state buffers."""
    out = ws.read(rig.B)
    sc = ws.scores[: rig.B].cpu().numpy()
    snap = {n: t.cpu().numpy() for n, t in layer.snapshot().items()}
    return out, sc, snap


# per-request lists and their lengths: entries past the length are not outputs (they
# keep whatever an earlier step of that workspace left there)
_LISTS = {"sel_tok": "n_sel", "sel_slot": "n_sel", "pf_tok": "n_pf", "pf_slot": "n_pf",
          "miss_tok": "n_miss"}


def _assert_same(a, b, tag, ctx):
    out_a, sc_a, st_a = a
    out_b, sc_b, st_b = b
    for k, v in out_a.items():
        if k in _LISTS:
            for r, n in enumerate(out_a[_LISTS[k]]):
                assert np.array_equal(v[r, :n], out_b[k][r, :n]), (tag, k, r)
        else:
            assert np.array_equal(np.asarray(v), np.asarray(out_b[k])), (tag, k)
    for r, n in enumerate(ctx):
        assert np.array_equal(sc_a[r, :n].view(np.uint32), sc_b[r, :n].view(np.uint32)), \
            (tag, "scores", r)
    for k, v in st_a.items():
        assert np.array_equal(v, st_b[k]), (tag, k)


def _step(rig, layer, ws, mode):
    R.check(abi.echo_layer_step(rig.dims, layer.struct, rig.batch.struct, ws.ws, mode,
                                R.stream_handle()), "echo_layer_step")


@pytest.mark.parametrize("paged", [False, True])
def test_restored_state_replays_bit_for_bit(paged):
    wl = get("single_layer").scaled(rho=0.6, steps=8)
    ctx = [3000, 1777, 2561]
    print(f"checkpoint: 64x128 ragged {ctx}, paged {paged}", flush=True)
    rig = H.Rig(wl, steps=8, ctx=ctx, n_gpu=3 * 256 + 2 * 120, n_host=8000, top_k=256,
                cap_div=64, paged=paged, stride_extra=2)
    mode = H.MODE_EMA
    for _ in range(3):
        out, _ = rig.step_and_compare(mode)
        assert out["status"] == 0
    snap = rig.layer.snapshot()
    first = []
    for _ in range(3):
        out, _ = rig.step_and_compare(mode)
        assert out["status"] == 0
        first.append(_record(rig, rig.layer, rig.ws))
    assert sum(int(o["n_evict"]) for _, o in rig.history[3:]) > 0, "no eviction after the copy"

    # back into the same layer, with a fresh workspace
    rig.layer.restore(snap)
    ws2 = R.Workspace(rig.dims)
    ws2.reset()
    for i in range(3):
        _step(rig, rig.layer, ws2, mode)
        _assert_same(first[i], _record(rig, rig.layer, ws2), f"same layer, step {3 + i}",
                     rig.ctx)

    # into a second layer at other addresses (same K, host pool, queries and weights)
    other = R.Layer(rig.dims, rig.kidx, rig.host, rig.B)
    other.q.copy_(rig.layer.q)
    other.w.copy_(rig.layer.w)
    other.restore(snap)
    ws3 = R.Workspace(rig.dims)
    ws3.reset()
    for i in range(3):
        _step(rig, other, ws3, mode)
        _assert_same(first[i], _record(rig, other, ws3), f"other layer, step {3 + i}",
                     rig.ctx)
    del other
    rig.close()
