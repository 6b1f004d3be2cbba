"""Decode append and writeback (echo_append) against the oracle, through the C ABI.

Every decode step scores, selects and manages the cache as in test_gpu_parity (all
compared bit for bit with the oracle fed the GPU's scores); then each request's new
token is appended: its indexer key into the tiled K, its latent into the mapped host
pool, and the context grows.  After each append the device context lengths, the
whole tiled K and the host pool bytes must equal the oracle's, and the next step
scores the grown contexts (the new token's score is checked with the others).
"""
import numpy as np
import pytest
import torch

from kv_cache_offload_fp8_amd import abi
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


def test_tiny_decode_with_append():
    _say("tiny decode with append, EMA")
    steps = 8
    rig = H.Rig(get("tiny"), steps=steps, ctx=[3000], max_ctx=3000 + steps, room=steps)
    for _ in range(steps):
        rig.step_and_compare(H.MODE_EMA)
        assert rig.append_and_compare() == O.OK
    assert int(rig.ctx[0]) == 3000 + steps
    rig.close()


@pytest.mark.parametrize("mode", [H.MODE_EMA, H.MODE_NEG_INF])
def test_ragged_64x128_decode_with_append(mode):
    # three ragged requests with a pool small enough to evict; each grows by one
    # token per step (room for exactly the steps run)
    wl = get("single_layer").scaled(rho=0.6, steps=6)
    ctx = [3000, 1777, 2561]
    steps = 6
    _say(f"64x128 ragged {ctx} with append, mode {mode}")
    rig = H.Rig(wl, steps=steps, ctx=ctx, n_gpu=3 * 256 + 2 * 120, n_host=8000, top_k=256,
                cap_div=64, max_ctx=max(ctx) + steps, room=steps)
    for _ in range(steps):
        out, _ = rig.step_and_compare(mode)
        assert out["status"] == 0
        assert rig.append_and_compare() == O.OK
    assert np.array_equal(rig.ctx, np.array(ctx) + steps)
    rig.close()


def test_append_without_advance_and_out_of_room():
    # advance = 0 writes the same rows again and keeps the contexts; a request whose
    # next id is the next request's first row stops the call on the device with
    # ECHO_ECAPACITY, nothing written, and the status stays set
    wl = get("single_layer").scaled(rho=0.6, steps=4)
    ctx = [1000, 1200]
    rig = H.Rig(wl, steps=4, ctx=ctx, n_gpu=2048, n_host=4096, top_k=256, cap_div=64,
                max_ctx=1300, room=2)
    rig.step_and_compare(H.MODE_EMA)
    assert rig.append_and_compare(advance=False) == O.OK
    assert np.array_equal(rig.ctx, ctx)
    assert rig.append_and_compare() == O.OK
    assert rig.append_and_compare() == O.OK
    # request 0 now ends 16-aligned room later: fill it to the next request's base
    gap = int(rig.base[1]) - int(rig.base[0]) - int(rig.ctx[0])
    for _ in range(gap):
        assert rig.append_and_compare() == O.OK
    assert rig.append_and_compare(expect_status=abi.ECHO_ECAPACITY) == O.ECAPACITY
    rig.close()
