"""Chunked-prefill selection (echo_prefill_score / _copy / _select) against the oracle,
through the C ABI.

Each chunk of queries is scored against one request's history on the GPU; the
scores are checked against the oracle's own (|rel| <= 2e-3 plus the cancellation
allowance), and the oracle, fed the GPU's scores, must then agree bit for bit on
everything decided from them: each query's boundary bucket and candidate count,
the union of candidates, each query's exact top-k and k-th score, the union of
selections, both install lists (host ids and slots), the maps, priorities, free
flags, free list, step counter and the GPU-pool bytes.  Later chunks pass the
previous chunk's k-th scores as the prediction, as the benchmark does.
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


def _run(rig, chunks, check_rows=None):
    for _ in range(chunks):
        o, g = rig.step_and_compare(check_rows=check_rows)
        _say(f"  chunk {rig.c - 1}: union {o['uni'].size}, candidates {o['cand'].size}, "
             f"early {o['pf_h'].size}, late {o['miss_h'].size}, "
             f"beta {np.unique(o['beta'])[:6]}")
    return o


@pytest.mark.parametrize("use_pred", [False, True])
def test_prefill_64x128_ragged(use_pred):
    # 40 queries (not a multiple of 16), a 3000-token history (not a multiple of 64)
    _say(f"prefill 64x128: N 3000, C 40, k 256, pred {use_pred}")
    wl = get("prefill").scaled(rho=0.9)
    rig = H.PrefillRig(wl, N=3000, C=40, chunks=3, n_gpu=4000, n_host=4096, top_k=256,
                       use_pred=use_pred)
    _run(rig, 3)
    rig.close()


@pytest.mark.parametrize("N,k,n_gpu,n_host", [(2999, 256, 4000, 4096), (1001, 64, 1500, 1024)])
def test_prefill_rows_off_16_byte_boundaries(N, k, n_gpu, n_host):
    # A history length that is not a multiple of 4: three score rows in four start
    # inside a 16-byte piece of the score buffer, and the coarse pass reads whole
    # pieces and must skip the neighbouring rows' floats.  19 queries leave a ragged
    # query block (the scoring kernel's stores for the missing queries are dropped)
    # and the last 64-token chunk is ragged too.
    _say(f"prefill 64x128: N {N}, C 19, k {k} (rows off 16-byte boundaries)")
    wl = get("prefill").scaled(rho=0.9)
    rig = H.PrefillRig(wl, N=N, C=19, chunks=2, n_gpu=n_gpu, n_host=n_host, top_k=k)
    _run(rig, 2)
    rig.close()


def test_prefill_single_query_chunks():
    # C = 1: one query block, so the scoring grid takes as many token splits as the
    # history allows and each workgroup has a single live wave (its second query and
    # the other seven waves' queries are missing); the coarse and exact passes run one
    # workgroup in all
    _say("prefill 64x128: N 1500, C 1, k 128")
    wl = get("prefill").scaled(rho=0.9)
    rig = H.PrefillRig(wl, N=1500, C=1, chunks=3, n_gpu=2000, n_host=2048, top_k=128)
    _run(rig, 3)
    rig.close()


def test_prefill_history_shorter_than_one_group():
    # N = 10: one partial 16-token group and one partial 64-token chunk; every
    # token split's range but the first is empty, and every token is selected
    _say("prefill 64x128: N 10, C 3, k 64")
    wl = get("prefill").scaled(rho=0.9)
    rig = H.PrefillRig(wl, N=10, C=3, chunks=2, n_gpu=256, n_host=256, top_k=64)
    o = _run(rig, 2)
    assert (o["beta"] == -1).all() and o["uni"].size == 10
    rig.close()


def test_prefill_4x32_small_heads():
    _say("prefill 4x32: N 1000, C 20, k 64")
    wl = get("tiny").scaled(rho=0.8)
    rig = H.PrefillRig(wl, N=1000, C=20, chunks=3, n_gpu=1500, n_host=1024, top_k=64)
    _run(rig, 3)
    rig.close()


@pytest.mark.parametrize("heads,dim", [(20, 64), (33, 96)])
def test_prefill_head_and_dim_shapes(heads, dim):
    _say(f"prefill {heads}x{dim}: N 1000, C 20, k 64")
    wl = get("tiny").scaled(heads=heads, head_dim=dim, rho=0.8)
    rig = H.PrefillRig(wl, N=1000, C=20, chunks=3, n_gpu=1500, n_host=1024, top_k=64)
    _run(rig, 3)
    rig.close()


def test_prefill_history_not_longer_than_k():
    _say("prefill: N 200 <= k 256")
    wl = get("prefill").scaled(rho=0.9)
    rig = H.PrefillRig(wl, N=200, C=17, chunks=2, n_gpu=512, n_host=1024, top_k=256)
    o = _run(rig, 2)
    assert (o["beta"] == -1).all() and o["uni"].size == 200
    rig.close()


def test_prefill_capacity_errors():
    wl = get("prefill").scaled(rho=0.9)
    # probe the sizes with a roomy pool
    probe = H.PrefillRig(wl, N=2000, C=24, chunks=1, n_gpu=3000, n_host=2048, top_k=128)
    o, _ = probe.step_and_compare()
    n_c, n_u = o["cand"].size, o["uni"].size
    probe.close()
    _say(f"prefill capacity: candidates {n_c}, union {n_u}")
    assert 0 < n_c < n_u
    # room for fewer than the candidates: nothing installed
    rig = H.PrefillRig(wl, N=2000, C=24, chunks=1, n_gpu=n_c - 1, n_host=2048, top_k=128)
    rig.step_and_compare(expect_status=O.ECAPACITY, fail_stage="early")
    rig.close()
    # room for the candidates only: they stay, the step counter does not move
    rig = H.PrefillRig(wl, N=2000, C=24, chunks=1, n_gpu=n_u - 1, n_host=2048, top_k=128)
    rig.step_and_compare(expect_status=O.ECAPACITY, fail_stage="late")
    rig.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("C", [256, 512])
def test_prefill_full_size(C):
    # 100K history, 64x128, k = 2048, 200K slots, 2M host tokens.  The scoring kernel
    # gives each workgroup 16 queries (8 waves of 2) over one token split, so rows 0-15
    # cover every wave and query position of a workgroup, at every token split of the
    # history; rows 16-17 and the rows around C/2 and at the end cross query-block
    # boundaries.  Those rows' scores are checked against the oracle's own, with the
    # top-k set clause; everything else bit for bit with the oracle fed the GPU's scores.
    _say(f"prefill full size: N 100,000, C {C}, 2 chunks")
    rig = H.PrefillRig(get("prefill"), N=100_000, C=C, chunks=2)
    rows = list(range(16)) + [16, 17, C // 2 - 1, C // 2, C - 2, C - 1]
    _run(rig, 2, check_rows=rows)
    _say(f"  max relative score error {H.STATS['max_rel']:.3g}, top-k set differences "
         f"{H.STATS['set_diffs']} over {H.STATS['set_checked']} rows")
    rig.close()


def test_prefill_graph_replay_matches_eager():
    # three chunks captured in one graph (fixed shapes and pointers; the later chunks
    # read the previous chunk's k-th scores as their prediction), replayed twice from
    # a fresh layer; every replay must leave what the eager calls leave
    wl = get("prefill").scaled(rho=0.9)
    kw = dict(N=3000, C=40, chunks=3, n_gpu=4000, n_host=4096, top_k=256)
    _say("prefill graph replay: N 3000, C 40, 3 chunks")
    eager = H.PrefillRig(wl, **kw)
    _run(eager, 3)
    graph = H.PrefillRig(wl, **kw)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for c in range(3):
                graph.gpu_chunk(c)
    torch.cuda.current_stream().wait_stream(s)
    ref = eager.layer.state()
    ref_pool = eager.layer.gpu_kv.clone()
    C, N = kw["C"], kw["N"]
    for rep in range(2):
        graph.layer.init()
        graph.pws.reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(graph.pws.status.item()) == 0
        st = graph.layer.state()
        for key in ("h2g", "g2h", "prio", "free", "idxbuf"):
            assert np.array_equal(st[key], ref[key]), (rep, key)
        assert st["t"] == ref["t"] == 3 and st["nfree"] == ref["nfree"]
        assert torch.equal(graph.layer.gpu_kv, ref_pool), rep
        assert torch.equal(graph.pws.scores(C, N), eager.pws.scores(C, N)), rep
        assert torch.equal(graph.pws.sel[:C], eager.pws.sel[:C]), rep
        assert torch.equal(graph.pws.counts, eager.pws.counts), rep
    graph.close()
    eager.close()
