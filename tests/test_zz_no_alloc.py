"""echo_topk_noalloc, the top-k call for callers that cannot allocate, against
echo_topk through the C ABI.

Both calls get the same external scores (heavy ties, ragged contexts, contexts at
and around k, an empty request) and the same EMA thresholds; the selections,
counts, k-th scores, updated thresholds and status must be identical bit for bit,
and each selection must equal the oracle's top-k of the same scores.  Two calls
run in a row on the library's one static scratch array, the second with a smaller
batch, context and k (a different scratch layout over the first call's leftovers);
then dims too large for the array are refused with nothing enqueued, and a
device-side batch error is reported the same way by both calls.
"""
import numpy as np
import pytest
import torch

from kv_cache_offload_fp8_amd import abi
from kv_cache_offload_fp8_amd import runtime as R
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _say(msg):
    print(msg, flush=True)


def _scores(rng, ctx, n):
    sc = np.zeros((len(ctx), n), np.float32)
    for b, c in enumerate(ctx):
        kind = b % 3
        if kind == 0:
            sc[b, :c] = rng.integers(0, 40, c)            # heavy ties
        elif kind == 1:
            sc[b, :c] = rng.standard_normal(c) * 100
        else:
            sc[b, :c] = rng.random(c)
            sc[b, : c // 2] = 7.0                          # a long run of equal scores
    return sc


def _both(ctx, max_ctx, k, theta0, seed):
    """echo_topk (workspace) and echo_topk_noalloc (static scratch) on the same inputs;
    returns both results as numpy dicts."""
    B = len(ctx)
    rng = np.random.default_rng(seed)
    sc = _scores(rng, ctx, max_ctx)
    span = (max_ctx + 15) // 16 * 16
    dims = R.make_dims(4, 32, k, B * span, 4096, B, max_ctx)
    batch = R.Batch(np.arange(B) * span, ctx)
    dev = torch.from_numpy(sc).cuda()
    st = R.stream_handle()
    # the existing entry point
    ws = R.Workspace(dims)
    ws.reset()
    th_a = torch.tensor(theta0, dtype=torch.float32, device="cuda")
    R.check(abi.echo_topk(dims, dev.data_ptr(), max_ctx, batch.struct, ws.ws, th_a.data_ptr(),
                          st), "echo_topk")
    a = ws.read(B)
    # the variant that allocates nothing
    sel = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    kth = torch.zeros(B, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    th_b = torch.tensor(theta0, dtype=torch.float32, device="cuda")
    R.check(abi.echo_topk_noalloc(dims, dev.data_ptr(), max_ctx, batch.struct, sel.data_ptr(),
                                  nsel.data_ptr(), kth.data_ptr(), th_b.data_ptr(),
                                  status.data_ptr(), st), "echo_topk_noalloc")
    torch.cuda.current_stream().synchronize()
    b = dict(sel_tok=sel.cpu().numpy(), n_sel=nsel.cpu().numpy(), kth=kth.cpu().numpy(),
             status=int(status.item()))
    return sc, a, th_a.cpu().numpy(), b, th_b.cpu().numpy()


def _compare(ctx, max_ctx, k, theta0, seed):
    sc, a, th_a, b, th_b = _both(ctx, max_ctx, k, theta0, seed)
    assert a["status"] == b["status"] == 0
    assert np.array_equal(a["n_sel"], b["n_sel"])
    assert np.array_equal(a["kth"].view(np.uint32), b["kth"].view(np.uint32))
    assert np.array_equal(th_a.view(np.uint32), th_b.view(np.uint32))
    for i, c in enumerate(ctx):
        n = int(a["n_sel"][i])
        assert n == min(k, c)
        assert np.array_equal(a["sel_tok"][i, :n], b["sel_tok"][i, :n]), i
        if c:
            osel, okth = O.topk(sc[i, :c], k)
            assert np.array_equal(b["sel_tok"][i, :n], osel), i
            assert np.float32(b["kth"][i]) == np.float32(okth), i
    _say(f"  batch {len(ctx)}, max_ctx {max_ctx}, k {k}: identical, selected {b['n_sel'].tolist()}")


def test_noalloc_topk_matches_echo_topk_twice_then_refuses_oversize():
    inf = float("inf")
    # first call: six requests up to 9000 tokens, k = 2048 (contexts below, at and just
    # above k, and an empty one); EMA thresholds seeded and unseeded
    _compare([9000, 2048, 2049, 100, 0, 7777], 9000, 2048, [inf, 3.0, inf, inf, inf, 50.0], 1)
    # second call, smaller: two requests up to 3000 tokens, k = 256
    _compare([3000, 1500], 3000, 256, [inf, -1.0], 2)
    # dims whose scratch would not fit the static array (64 requests of 100,000 tokens
    # need about 52 MB): refused, nothing enqueued (real buffers all the same)
    dims = R.make_dims(4, 32, 2048, 64 * 100_000, 4096, 64, 100_000)
    sc = torch.zeros((1, 100_000), dtype=torch.float32, device="cuda")
    sel = torch.full((1, 2048), -7, dtype=torch.int32, device="cuda")
    nsel = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    kth = torch.zeros(1, dtype=torch.float32, device="cuda")
    status = torch.full((1,), 5, dtype=torch.int32, device="cuda")
    batch = R.Batch(np.zeros(1, np.int64), [10])
    rc = abi.echo_topk_noalloc(dims, sc.data_ptr(), 100_000, batch.struct, sel.data_ptr(),
                               nsel.data_ptr(), kth.data_ptr(), None, status.data_ptr(),
                               R.stream_handle())
    assert rc == abi.ECHO_ESCRATCH
    torch.cuda.current_stream().synchronize()
    assert int(status.item()) == 5 and int(nsel.item()) == -7


def test_noalloc_topk_reports_a_device_side_batch_error_like_echo_topk():
    k, max_ctx = 256, 1000
    dims = R.make_dims(4, 32, k, 4096, 4096, 2, max_ctx)
    bad = R.Batch([0, 100], [1000, 50])  # overlapping host ranges
    sc = torch.rand((2, max_ctx), device="cuda")
    ws = R.Workspace(dims)
    ws.reset()
    R.check(abi.echo_topk(dims, sc.data_ptr(), max_ctx, bad.struct, ws.ws, None,
                          R.stream_handle()), "echo_topk")
    sel = torch.zeros((2, k), dtype=torch.int32, device="cuda")
    nsel = torch.zeros(2, dtype=torch.int32, device="cuda")
    kth = torch.zeros(2, dtype=torch.float32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    R.check(abi.echo_topk_noalloc(dims, sc.data_ptr(), max_ctx, bad.struct, sel.data_ptr(),
                                  nsel.data_ptr(), kth.data_ptr(), None, status.data_ptr(),
                                  R.stream_handle()), "echo_topk_noalloc")
    torch.cuda.current_stream().synchronize()
    assert int(ws.status.item()) == int(status.item()) == abi.ECHO_EDEVARG
    # then a good batch: the sticky status keeps the call a no-op until cleared
    good = R.Batch([0, 1008], [1000, 50])
    R.check(abi.echo_topk_noalloc(dims, sc.data_ptr(), max_ctx, good.struct, sel.data_ptr(),
                                  nsel.data_ptr(), kth.data_ptr(), None, status.data_ptr(),
                                  R.stream_handle()), "echo_topk_noalloc")
    torch.cuda.current_stream().synchronize()
    assert int(status.item()) == abi.ECHO_EDEVARG and int(nsel.sum().item()) == 0
    status.zero_()
    R.check(abi.echo_topk_noalloc(dims, sc.data_ptr(), max_ctx, good.struct, sel.data_ptr(),
                                  nsel.data_ptr(), kth.data_ptr(), None, status.data_ptr(),
                                  R.stream_handle()), "echo_topk_noalloc")
    torch.cuda.current_stream().synchronize()
    assert int(status.item()) == 0 and nsel.cpu().tolist() == [256, 50]
    s0, _ = O.topk(sc[0].cpu().numpy(), k)
    assert np.array_equal(sel[0].cpu().numpy(), s0)
