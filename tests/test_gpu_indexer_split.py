"""echo_indexer_begin + echo_indexer_score against echo_indexer_prefetch, through the
C ABI: the two halves enqueued one after the other must give the same scores (bit for
bit), the same prefetch lists and the same cache state as the single call."""
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


def _indexer(rig, mode, split):
    st = R.stream_handle()
    if split:
        R.check(abi.echo_indexer_begin(rig.dims, rig.layer.struct, rig.batch.struct, rig.ws.ws,
                                       mode, st), "echo_indexer_begin")
        R.check(abi.echo_indexer_score(rig.dims, rig.layer.struct, rig.batch.struct, rig.ws.ws,
                                       mode, st), "echo_indexer_score")
    else:
        R.check(abi.echo_indexer_prefetch(rig.dims, rig.layer.struct, rig.batch.struct,
                                          rig.ws.ws, mode, st), "echo_indexer_prefetch")
    torch.cuda.current_stream().synchronize()
    out = rig.ws.read(rig.B)
    return out, rig.gpu_scores(), rig.layer.state()


@pytest.mark.parametrize("mode", [H.MODE_POS_INF, H.MODE_EMA])
def test_begin_then_score_equals_prefetch(mode):
    print(f"indexer split, mode {mode}", flush=True)
    wl = get("single_layer").scaled(rho=0.7, steps=3)
    ctx = [3000, 1777, 2561]
    res = []
    for split in (False, True):
        rig = H.Rig(wl, steps=3, ctx=ctx, n_gpu=4096, n_host=8000, top_k=256, cap_div=64)
        rig.step_and_compare(H.MODE_EMA)     # one full step: thresholds set, cache warm
        res.append(_indexer(rig, mode, split))
        rig.close()
    (o0, s0, g0), (o1, s1, g1) = res
    assert o0["status"] == o1["status"] == 0
    assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32))
    for key in ("n_pf", "n_cand"):
        assert np.array_equal(o0[key], o1[key]), key
    for b in range(len(ctx)):
        n = int(o0["n_pf"][b])
        assert np.array_equal(o0["pf_tok"][b, :n], o1["pf_tok"][b, :n])
        assert np.array_equal(o0["pf_slot"][b, :n], o1["pf_slot"][b, :n])
    for key in ("h2g", "g2h", "prio", "free"):
        assert np.array_equal(g0[key], g1[key]), key
    if mode == H.MODE_EMA:
        assert int(o0["n_pf"].sum()) > 0
