"""GPU path vs the oracle, through the C ABI, on seeded inputs.

Scores: within 2e-3 relative of the oracle's fp64 scores (plus, at four heads or
fewer, the cancellation allowance of echo_harness.score_tolerance), and the GPU's
selected set may differ from the oracle's top-k of its own scores only on tokens
within that tolerance of the k-th score.  Everything decided
from the scores -- prefetch lists, top-k, EMA state, misses, evictions, slot maps,
priorities, free flags, the free list and the pool bytes -- bit-exact, with the
oracle fed the GPU's scores.
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


@pytest.mark.parametrize("mode", [H.MODE_EMA, H.MODE_NEG_INF, H.MODE_POS_INF])
def test_tiny_decode_bit_exact(mode):
    _say(f"tiny decode, mode {mode}")
    rig = H.Rig(get("tiny"), steps=8)
    for _ in range(8):
        rig.step_and_compare(mode)
    rig.close()


@pytest.mark.parametrize("mode", [H.MODE_EMA, H.MODE_NEG_INF])
def test_full_indexer_shape_ragged_with_eviction(mode):
    # 64 heads x 128, three ragged requests, k=256, a pool that forces eviction
    wl = get("single_layer").scaled(rho=0.6, steps=6)
    ctx = [3000, 1777, 2561]
    _say(f"64x128 ragged {ctx}, mode {mode}")
    # room for one step's selection plus two steps of prefetch (caps 47+28+41)
    rig = H.Rig(wl, steps=6, ctx=ctx, n_gpu=3 * 256 + 2 * 120, n_host=8000, top_k=256,
                cap_div=64)
    for _ in range(6):
        out, _ = rig.step_and_compare(mode)
        assert out["status"] == 0
    assert sum(int(o["n_evict"]) for _, o in rig.history) > 0
    rig.close()


def test_lossless_across_modes_on_gpu():
    wl = get("tiny").scaled(rho=0.7)
    outs = {}
    for mode in (H.MODE_EMA, H.MODE_NEG_INF, H.MODE_POS_INF):
        rig = H.Rig(wl, steps=6, n_gpu=600)
        seq = []
        for _ in range(6):
            rig.gpu_step(mode)
            o = rig.ws.read(rig.B)
            assert o["status"] == 0
            n = int(o["n_sel"][0])
            sel = o["sel_tok"][0, :n].copy()
            slots = torch.as_tensor(o["sel_slot"][0, :n].astype(np.int64), device="cuda")
            gathered = rig.layer.gpu_kv[slots].cpu().numpy().view(np.uint16)
            assert np.array_equal(gathered, rig.np_host[rig.base[0] + sel])
            seq.append((sel, gathered))
        outs[mode] = seq
        rig.close()
    for mode in (H.MODE_EMA, H.MODE_NEG_INF):
        for (s1, g1), (s2, g2) in zip(outs[mode], outs[H.MODE_POS_INF]):
            assert np.array_equal(s1, s2) and np.array_equal(g1, g2)


def test_graph_replay_matches_eager():
    wl = get("tiny")
    eager = H.Rig(wl, steps=6)
    graph = H.Rig(wl, steps=6)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            graph.gpu_step(H.MODE_EMA)
    torch.cuda.synchronize()
    # capture does not execute: both rigs are still at step 0
    for t in range(6):
        eager.gpu_step(H.MODE_EMA)
        g.replay()
        torch.cuda.synchronize()
        a, b = eager.layer.state(), graph.layer.state()
        for key in ("h2g", "g2h", "prio", "free", "theta", "idxbuf"):
            assert np.array_equal(a[key], b[key]), (t, key)
        assert a["t"] == b["t"] == t + 1
        oa, ob = eager.ws.read(eager.B), graph.ws.read(graph.B)
        assert np.array_equal(oa["sel_tok"], ob["sel_tok"])
        assert np.array_equal(eager.gpu_scores(), graph.gpu_scores())
        assert torch.equal(eager.layer.gpu_kv, graph.layer.gpu_kv)
    eager.close()
    graph.close()


@pytest.mark.parametrize("mode,n_gpu", [(H.MODE_EMA, 3 * 256 + 2 * 120),
                                         (H.MODE_NEG_INF, 1200)])
def test_eviction_boundary_in_the_clamped_oldest_bin(mode, n_gpu):
    # Two steps from t = 0 leave slots last used at steps 0 and 1.  The step counter
    # then jumps to 5002: every occupied slot is idle for 4096 steps or more, so the
    # eviction histogram puts them all in its clamped bin 0, and the boundary of the
    # eviction falls inside that bin.  The exact (priority, slot) select over the bin
    # must evict every priority-0 slot and the lowest-numbered priority-1 slots (the
    # two priorities interleave in slot order), as the oracle does.  The next steps
    # evict from bin 0 and from the fresh priorities.
    wl = get("single_layer").scaled(rho=0.6, steps=8)
    ctx = [3000, 1777, 2561]
    _say(f"clamped-age eviction: 64x128 ragged {ctx}, pool {n_gpu}, mode {mode}")
    rig = H.Rig(wl, steps=8, ctx=ctx, n_gpu=n_gpu, n_host=8000, top_k=256, cap_div=64)
    for _ in range(2):
        rig.step_and_compare(mode)
    rig.jump_to_step(5002)
    for t in range(5002, 5005):
        before = rig.orc.prio.copy()
        out, o = rig.step_and_compare(mode)
        assert out["status"] == 0
        ev = o["evicted"]
        prios = np.unique(before[ev]).tolist()
        _say(f"  step {t}: evicted {ev.size}, their priorities {prios}")
        if t == 5002:
            old = (before >= 0) & (before <= t - 4096)
            assert 0 < ev.size < int(old.sum()) and prios == [0, 1]
    rig.close()


@pytest.mark.parametrize("mode", [H.MODE_EMA, H.MODE_NEG_INF, H.MODE_POS_INF])
def test_separate_calls_match_the_oracle(mode):
    # echo_indexer_prefetch -> echo_topk -> echo_cache_alloc_evict -> echo_recall ->
    # echo_step_advance, one call each, step by step against the oracle (the same
    # results echo_layer_step gives in one call)
    wl = get("single_layer").scaled(rho=0.6, steps=6)
    ctx = [3000, 1777, 2561]
    _say(f"separate calls: 64x128 ragged {ctx}, mode {mode}")
    rig = H.Rig(wl, steps=6, ctx=ctx, n_gpu=3 * 256 + 2 * 120, n_host=8000, top_k=256,
                cap_div=64)
    rig.separate = True
    for _ in range(6):
        out, _ = rig.step_and_compare(mode)
        assert out["status"] == 0
    assert sum(int(o["n_evict"]) for _, o in rig.history) > 0
    assert sum(int(o["n_miss"].sum()) for _, o in rig.history) > 0
    if mode != H.MODE_POS_INF:
        assert sum(int(o["n_pf"].sum()) for _, o in rig.history) > 0
    rig.close()


@pytest.mark.parametrize("heads,dim", [(20, 64), (33, 96), (48, 128), (1, 32)])
def test_head_groups_and_dims(heads, dim):
    # the scoring kernel runs 1-4 groups of 16 heads (padded) over head dims of 32-128:
    # two and three groups, a group padded from one head, and every dim but the
    # tiny (4 x 32) and full (64 x 128) shapes other tests use
    wl = get("tiny").scaled(heads=heads, head_dim=dim, rho=0.7)
    ctx = [1500, 3001, 257]
    _say(f"{heads} heads x {dim}, ctx {ctx}")
    rig = H.Rig(wl, steps=4, ctx=ctx, n_gpu=3 * 256 + 2 * 120, n_host=8000, top_k=256,
                cap_div=64)
    for _ in range(4):
        out, _ = rig.step_and_compare(H.MODE_EMA)
        assert out["status"] == 0
    assert sum(int(o["n_evict"]) for _, o in rig.history) > 0
    rig.close()


def test_layers_share_one_workspace():
    # as in a decode step: three layers (their own K, queries, pools and metadata)
    # step in turn through one workspace, each against its own oracle layer
    wl = get("single_layer").scaled(rho=0.6, steps=4)
    ctx = [3000, 1777, 2561]
    _say(f"3 layers, one workspace, ctx {ctx}")
    rigs = [H.Rig(wl, steps=4, ctx=ctx, n_gpu=3 * 256 + 2 * 120, n_host=8000, top_k=256,
                  cap_div=64, layer=l) for l in range(3)]
    for r in rigs[1:]:
        r.ws = rigs[0].ws
    for _ in range(4):
        for r in rigs:
            out, _ = r.step_and_compare(H.MODE_EMA)
            assert out["status"] == 0
    for r in rigs:
        assert sum(int(o["n_evict"]) for _, o in r.history) > 0
        r.close()


def test_two_layer_graph_matches_eager():
    # the decode step as the benchmark runs it: several layers sharing one workspace,
    # captured in one graph; every replay equals the same calls made eagerly
    wl = get("tiny").scaled(rho=0.8)
    kw = dict(steps=5, ctx=[2000, 900], n_gpu=1600, n_host=4096, cap_div=32)
    eager = [H.Rig(wl, layer=l, **kw) for l in range(2)]
    graph = [H.Rig(wl, layer=l, **kw) for l in range(2)]
    eager[1].ws = eager[0].ws
    graph[1].ws = graph[0].ws
    _say("two layers, one workspace, graph against eager")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for r in graph:
                r.gpu_step(H.MODE_EMA)
    torch.cuda.synchronize()
    for t in range(5):
        for r in eager:
            r.gpu_step(H.MODE_EMA)
        g.replay()
        torch.cuda.synchronize()
        for re_, rg in zip(eager, graph):
            a, b = re_.layer.state(), rg.layer.state()
            for key in ("h2g", "g2h", "prio", "free", "theta", "idxbuf"):
                assert np.array_equal(a[key], b[key]), (t, key)
            assert a["t"] == b["t"] == t + 1
            assert torch.equal(re_.layer.gpu_kv, rg.layer.gpu_kv)
            assert torch.equal(re_.layer.stats, rg.layer.stats)  # running totals too
        oa, ob = eager[0].ws.read(2), graph[0].ws.read(2)  # the last layer's outputs
        assert oa["status"] == ob["status"] == 0
        for key in ("n_sel", "n_pf", "n_miss", "kth"):
            assert np.array_equal(oa[key], ob[key]), (t, key)
        for b in range(2):
            for key, n in (("sel_tok", "n_sel"), ("sel_slot", "n_sel"), ("pf_tok", "n_pf"),
                           ("pf_slot", "n_pf"), ("miss_tok", "n_miss")):
                m = int(oa[n][b])
                assert np.array_equal(oa[key][b, :m], ob[key][b, :m]), (t, key, b)
    for r in eager + graph:
        r.close()


@pytest.mark.parametrize("mode", [H.MODE_EMA, H.MODE_NEG_INF])
def test_largest_top_k_with_eviction(mode):
    # top_k = 4096, the largest the library takes, with contexts k - 1, k, k + 1 and
    # 9000, and a pool that holds one step's selection plus a little: later steps
    # evict
    wl = get("tiny").scaled(rho=0.7)
    ctx = [4095, 4096, 4097, 9000]
    _say(f"top_k 4096, ctx {ctx}, mode {mode}")
    rig = H.Rig(wl, steps=4, ctx=ctx, n_gpu=17_500, n_host=24_000, top_k=4096, cap_div=64)
    for _ in range(4):
        out, _ = rig.step_and_compare(mode)
        assert out["status"] == 0
        assert list(out["n_sel"][:4]) == [4095, 4096, 4096, 4096]
    assert sum(int(o["n_evict"]) for _, o in rig.history) > 0
    assert sum(int(o["n_pf"].sum()) for _, o in rig.history) > 0
    rig.close()


@pytest.mark.parametrize("n,k", [(5000, 256), (256, 256), (100, 256), (257, 256), (9000, 2048)])
def test_topk_external_scores_with_ties(n, k):
    rng = np.random.default_rng(n + k)
    B = 3
    sc = rng.integers(0, 40, size=(B, n)).astype(np.float32)  # heavy ties
    sc[1] = rng.standard_normal(n).astype(np.float32) * 100
    sc[2, : n // 2] = 7.0
    span = (n + 15) // 16 * 16
    dims = R.make_dims(4, 32, k, B * span, 4096, B, n)
    ws = R.Workspace(dims)
    ws.reset()
    batch = R.Batch(np.arange(B) * span, [n] * B)
    dev = torch.from_numpy(sc).cuda()
    theta = torch.full((B,), float("inf"), device="cuda")
    R.check(abi.echo_topk(dims, dev.data_ptr(), n, batch.struct, ws.ws, theta.data_ptr(),
                          R.stream_handle()), "echo_topk")
    o = ws.read(B)
    assert o["status"] == 0
    for b in range(B):
        sel, kth = O.topk(sc[b], k)
        m = sel.size
        assert o["n_sel"][b] == m
        assert np.array_equal(o["sel_tok"][b, :m], sel), b
        assert np.float32(o["kth"][b]) == np.float32(kth)
        if n >= k:
            assert theta[b].item() == np.float32(kth)


def test_capacity_error_matches_oracle():
    wl = get("tiny")
    rig = H.Rig(wl, steps=2, n_gpu=200)  # k=256 misses > 200 slots
    out, o = rig.step_and_compare(H.MODE_POS_INF, expect_status=abi.ECHO_ECAPACITY)
    assert out["status"] == abi.ECHO_ECAPACITY == o["status"]
    # the error is sticky: the next call changes nothing until the workspace is reset
    before = rig.layer.state()
    rig.gpu_step(H.MODE_POS_INF)
    after = rig.layer.state()
    for key in ("h2g", "g2h", "prio", "free"):
        assert np.array_equal(before[key], after[key])
    assert after["t"] == 0
    rig.close()


def test_device_side_batch_check():
    wl = get("tiny").scaled(n_host=8192)
    rig = H.Rig(wl, steps=1, ctx=[4096])
    bad = R.Batch([0, 100], [4096, 50], "cuda")  # overlapping host ranges
    dims = R.make_dims(wl.heads, wl.head_dim, wl.top_k, wl.n_host, wl.n_gpu, 2, 4096,
                       q_ring=1)
    ws = R.Workspace(dims)
    ws.reset()
    layer = R.Layer(dims, rig.kidx, rig.host, 2)
    layer.init()
    R.check(abi.echo_layer_step(dims, layer.struct, bad.struct, ws.ws, H.MODE_EMA,
                                R.stream_handle()), "launch")
    o = ws.read(2)
    assert o["status"] == abi.ECHO_EDEVARG
    st = layer.state()
    assert st["t"] == 0 and (st["h2g"] == -1).all() and (st["free"] == 1).all()
    rig.close()


def test_misaligned_host_base_is_rejected_on_device():
    wl = get("tiny").scaled(n_host=8192)
    rig = H.Rig(wl, steps=1, ctx=[4096])
    bad = R.Batch([8], [4000], "cuda")  # in range, no overlap, but not on a 16-row boundary
    ws = R.Workspace(rig.dims)
    ws.reset()
    R.check(abi.echo_layer_step(rig.dims, rig.layer.struct, bad.struct, ws.ws, H.MODE_EMA,
                                R.stream_handle()), "launch")
    o = ws.read(1)
    assert o["status"] == abi.ECHO_EDEVARG
    st = rig.layer.state()
    assert st["t"] == 0 and (st["h2g"] == -1).all() and (st["free"] == 1).all()
    rig.close()


@pytest.mark.parametrize("D", [32, 64, 96, 128])
def test_kindex_pack_layout(D):
    # the tiled layout is a fixed permutation inside each group of 16 rows
    n = 16 * 37
    rng = np.random.default_rng(D)
    rows = rng.integers(0, 256, size=(n, D), dtype=np.uint8)
    dims = R.make_dims(4, D, 256, n, 1024, 1, 4096)
    tiled = R.pack_kidx(dims, torch.from_numpy(rows).cuda()).cpu().numpy().reshape(-1)
    h = np.arange(n)[:, None]
    d = np.arange(D)[None, :]
    pos = 16 * D * (h // 16) + 8 * D * ((d % 32) // 16) + 256 * (d // 32) + 16 * (h % 16) + d % 16
    expect = np.empty(n * D, np.uint8)
    expect[pos.reshape(-1)] = rows.reshape(-1)
    assert np.array_equal(tiled, expect)
    assert np.unique(pos).size == n * D  # a permutation


def test_context_edge_cases():
    # an empty request, one shorter than k, one equal to k, one just above k
    wl = get("tiny").scaled(n_host=4 * 1024)
    ctx = [0, 100, 256, 257]
    rig = H.Rig(wl, steps=4, ctx=ctx, n_gpu=1024)
    for mode in (H.MODE_EMA, H.MODE_NEG_INF, H.MODE_EMA, H.MODE_EMA):
        rig.step_and_compare(mode)
    rig.close()


@pytest.mark.parametrize("mode", [H.MODE_EMA, H.MODE_NEG_INF])
def test_two_launch_step_when_the_fused_launch_does_not_fit(mode):
    # echo_layer_step runs selection and management in one launch only when its
    # workgroups (one per request, one per 4096 slots, the copy workgroups) fit one
    # per compute unit; 64 requests and 700,000 slots (171 slot tiles) do not, so the
    # step takes the two-launch path: top-k with its copy hand-off, then management.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n_gpu, B = 700_000, 64
    tiles = -(-n_gpu // 4096)
    copy_wgs = min(cus // 8, 64)  # the indexer's copy workgroups, as management launches them
    if B + tiles + copy_wgs <= cus:
        pytest.skip(f"{B + tiles + copy_wgs} workgroups fit {cus} compute units")
    rng = np.random.default_rng(5)
    ctx = [int(c) for c in rng.integers(300, 700, size=B)]
    wl = get("tiny").scaled(n_host=48_000, rho=0.9)
    _say(f"two-launch step: B={B}, n_gpu={n_gpu}, {cus} CUs, mode {mode}")
    rig = H.Rig(wl, steps=4, ctx=ctx, n_gpu=n_gpu)
    for _ in range(4):
        out, _ = rig.step_and_compare(mode)
        assert out["status"] == 0
    assert sum(int(o["n_pf"].sum()) for _, o in rig.history) > 0
    rig.close()
