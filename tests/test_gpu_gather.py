"""Attention input (echo_gather) against the attention input without offloading.

After every decode step, the rows the sparse attention would read from the GPU pool
(through sel_slot) must equal the oracle's gather of the same selected tokens
straight from the full host copy: the losslessness of the whole path, checked on
its output.  Stress: queries that change completely every step (rho = 0), pools so
small that every step evicts and recalls, and all three threshold modes.  Each step
is also compared with the oracle as in test_gpu_parity.
"""
import numpy as np
import pytest
import torch

from kv_cache_offload_fp8_amd import abi
from kv_cache_offload_fp8_amd import runtime as R
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


def _gather_and_compare(rig, o, tag):
    k, lat = rig.wl.top_k, rig.wl.latent
    out = torch.full((max(1, rig.B), k, lat), -1, dtype=torch.int16, device="cuda")
    R.check(abi.echo_gather(rig.dims, rig.layer.struct, rig.batch.struct, rig.ws.ws,
                            out.data_ptr(), R.stream_handle()), "echo_gather")
    torch.cuda.current_stream().synchronize()
    got = out[: rig.B].cpu().numpy().view(np.uint16)
    want = O.gather(rig.base, o["sel_tok"], o["n_sel"], rig.orc_host)
    assert np.array_equal(got, want), tag


@pytest.mark.parametrize("mode", [H.MODE_EMA, H.MODE_NEG_INF, H.MODE_POS_INF])
def test_attention_input_is_lossless_under_sudden_query_changes(mode):
    # rho = 0: every step's queries are new, so most selected tokens miss
    wl = get("single_layer").scaled(rho=0.0, steps=5)
    ctx = [3000, 1777, 2561]
    _say(f"gather, rho 0, ragged {ctx}, mode {mode}")
    rig = H.Rig(wl, steps=5, ctx=ctx, n_gpu=3 * 256 + 2 * 120, n_host=8000, top_k=256,
                cap_div=64)
    for t in range(5):
        out, o = rig.step_and_compare(mode)
        assert out["status"] == 0
        _gather_and_compare(rig, o, f"step {t}")
    assert sum(int(o["n_evict"]) for _, o in rig.history) > 0
    rig.close()


def test_attention_input_with_the_smallest_pool():
    # the pool holds exactly one step's selection: every step evicts everything older
    wl = get("tiny").scaled(rho=0.3, steps=6)
    _say("gather, tiny pool of k slots")
    rig = H.Rig(wl, steps=6, ctx=[4000], n_gpu=256, top_k=256, cap_div=10 ** 6)
    for t in range(6):
        out, o = rig.step_and_compare(H.MODE_EMA)
        assert out["status"] == 0
        _gather_and_compare(rig, o, f"step {t}")
    rig.close()


def test_attention_input_short_and_empty_contexts():
    # contexts shorter than k (every token selected) and an empty request
    wl = get("single_layer").scaled(rho=0.9, steps=3)
    ctx = [100, 0, 257, 1500]
    _say(f"gather, contexts {ctx}")
    rig = H.Rig(wl, steps=3, ctx=ctx, n_gpu=4096, n_host=4096, top_k=256, cap_div=64)
    for t in range(3):
        out, o = rig.step_and_compare(H.MODE_EMA)
        assert out["status"] == 0
        _gather_and_compare(rig, o, f"step {t}")
    rig.close()
