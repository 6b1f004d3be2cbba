"""Pins of the CPU oracle against things other than itself.

Each test fixes one part of the oracle by an independent route: the library's
own fp8/bf16 decoders, exact rational arithmetic, a brute-force sort, closed
forms, the review page's worked metadata example, hand-derived state machines,
and invariants that must hold after every step.  None of them re-types the
oracle's C code.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- formats

def test_e4m3_decode_matches_torch_for_every_code():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy().astype(np.float64)
    got = np.array([O.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    # anchor points of the OCP E4M3FN format
    assert O.e4m3_value(0x7E) == 448.0 and O.e4m3_value(0xFE) == -448.0
    assert O.e4m3_value(0x01) == 2.0 ** -9 and O.e4m3_value(0x08) == 2.0 ** -6
    assert O.e4m3_value(0x38) == 1.0 and np.isnan(O.e4m3_value(0x7F))


def test_bf16_decode_matches_torch_for_every_code():
    codes = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    ref = codes.view(torch.bfloat16).to(torch.float32).numpy().astype(np.float64)
    lib = O.lib()
    got = np.array([lib.orc_bf16_value(c) for c in range(65536)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])


# ------------------------------------------------------------------ scores

def _f32_nearest_even(x: Fraction) -> np.float32:
    """Exact round-to-nearest-even of a rational to binary32 (finite range)."""
    f = np.float32(float(x))
    cands = {f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))}
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - x)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    out = best[1]
    return np.float32(0.0) if out == 0 else out


def _rand_case(H, D, n, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((H, D), generator=g).to(torch.bfloat16)
    w = torch.rand((H,), generator=g)
    k = torch.randn((n, D), generator=g).to(torch.float8_e4m3fn)
    return q, w, k


@pytest.mark.parametrize("H,D,n,seed", [(4, 32, 48, 0), (8, 16, 40, 1), (3, 5, 64, 2)])
def test_scores_equal_exact_rational_arithmetic(H, D, n, seed):
    q, w, k = _rand_case(H, D, n, seed)
    qf = [[Fraction(float(v)) for v in row] for row in q.float().tolist()]
    wf = [Fraction(float(v)) for v in w.tolist()]
    kf = [[Fraction(float(v)) for v in row] for row in k.float().tolist()]
    got = O.scores(q.view(torch.int16).numpy().view(np.uint16), w.numpy(),
                   k.view(torch.uint8).numpy())
    for s in range(n):
        exact = Fraction(0)
        for j in range(H):
            x = sum(qf[j][d] * kf[s][d] for d in range(D))
            exact += wf[j] * (x if x > 0 else 0)
        ref = _f32_nearest_even(exact)
        assert got[s].view(np.uint32) == np.float32(ref).view(np.uint32), (s, got[s], ref)


def _codes(q_vals, w_vals, k_vals):
    q = torch.tensor(q_vals, dtype=torch.float32).to(torch.bfloat16)
    k = torch.tensor(k_vals, dtype=torch.float32).to(torch.float8_e4m3fn)
    return (q.view(torch.int16).numpy().view(np.uint16), np.array(w_vals, np.float32),
            k.view(torch.uint8).numpy())


def test_scores_closed_forms():
    # one head, one dim: score = w * max(0, q*k)
    q, w, k = _codes([[1.5]], [0.25], [[2.0], [-2.0], [0.0], [448.0]])
    s = O.scores(q, w, k)
    assert s.tolist() == [0.75, 0.0, 0.0, 168.0]
    assert all(np.array(s, np.float32).view(np.uint32)[1:3] == 0)  # +0, never -0
    # ReLU is per head, before the weighted sum: heads (+3, -3) give w0*3, not 0
    q, w, k = _codes([[1.0, 1.0], [-1.0, -1.0]], [0.5, 0.75], [[1.0, 2.0]])
    assert O.scores(q, w, k).tolist() == [1.5]
    # a zero weight removes its head
    q, w, k = _codes([[1.0], [2.0]], [0.0, 1.0], [[4.0]])
    assert O.scores(q, w, k).tolist() == [8.0]


def test_scores_homogeneity_and_token_independence():
    q, w, k = _rand_case(6, 24, 50, 7)
    qc = q.view(torch.int16).numpy().view(np.uint16)
    kc = k.view(torch.uint8).numpy()
    base = O.scores(qc, w.numpy(), kc)
    q2 = (q.float() * 2).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.scores(q2, w.numpy(), kc), base * 2)      # relu(2x) = 2 relu(x)
    assert np.array_equal(O.scores(qc, (w * 4).numpy(), kc), base * 4)
    perm = np.random.default_rng(0).permutation(50)
    assert np.array_equal(O.scores(qc, w.numpy(), kc[perm]), base[perm])


# ------------------------------------------------------------------ top-k

def _brute_topk(sc, k):
    order = sorted(range(len(sc)), key=lambda i: (-float(sc[i]), i))[: min(k, len(sc))]
    return sorted(order), (float(sc[order[-1]]) if order else None)


@pytest.mark.parametrize("n,k,seed", [(0, 4, 0), (3, 8, 1), (8, 8, 2), (50, 7, 3),
                                      (300, 64, 4), (1000, 256, 5)])
def test_topk_equals_full_sort_with_ties(n, k, seed):
    rng = np.random.default_rng(seed)
    sc = rng.integers(0, 12, size=n).astype(np.float32)  # many ties
    sel, kth = O.topk(sc, k)
    ref, ref_kth = _brute_topk(sc, k)
    assert sel.tolist() == ref
    if ref:
        assert kth == ref_kth
        chosen = np.zeros(n, bool)
        chosen[sel] = True
        if (~chosen).any():
            assert sc[chosen].min() >= sc[~chosen].max()


def test_topk_lower_index_wins_ties():
    sel, kth = O.topk(np.array([5, 1, 5, 5, 1], np.float32), 2)
    assert sel.tolist() == [0, 2] and kth == 5.0


# -------------------------------------------------------------------- EMA

def test_ema_closed_form_at_half():
    s0, s1, s2 = 96.0, 40.0, 7.0
    th = O.ema_update(np.inf, s0)                    # first estimate seeds theta
    assert th == s0
    th = O.ema_update(th, s1)
    assert th == (s0 + s1) / 2
    th = O.ema_update(th, s2)
    assert th == (s0 + s1) / 4 + s2 / 2


def test_ema_is_fp32_and_weights_new_sample_by_alpha():
    th, s = np.float32(3.1), np.float32(1.7)
    a = np.float32(0.3)
    ref = np.float32(np.float32(a * s) + np.float32(np.float32(1) - a) * th)
    assert np.float32(O.ema_update(float(th), float(s), float(a))) == ref
    assert O.ema_update(float("-inf"), 5.0) == float("-inf")


# --------------------------------------------------------------- metadata

def test_metadata_matches_pages_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "metadata_example.json")))
    per_layer = O.meta_bytes(g["n_host"], g["n_gpu"])
    assert per_layer == g["bytes_per_layer_exact"]
    mb = g["mb"]
    tol = g["approx_rel_tolerance"]
    assert abs(per_layer / mb - g["approx_mb_per_layer"]) <= tol * g["approx_mb_per_layer"]
    model = per_layer * g["layers"] / mb
    assert abs(model - g["approx_mb_model"]) <= tol * g["approx_mb_model"]


def test_metadata_is_sum_of_structures():
    lay = O.OracleLayer(4, 8, 2, 4, n_host=1000, n_gpu=37, max_batch=1, keep_pool=False)
    idxbuf_bytes = 4 * 37  # the index buffer is scratch that the GPU side keeps per layer
    total = (lay.h2g.nbytes + lay.g2h.nbytes + lay.prio.nbytes + lay.free.nbytes + idxbuf_bytes)
    assert total == O.meta_bytes(1000, 37)


# ---------------------------------------------- hand-derived state machines

def _ext(ctx, winners, stride=None):
    """External scores: the listed tokens get descending high scores."""
    sc = np.zeros((1, stride or ctx), np.float32)
    for r, s in enumerate(winners):
        sc[0, s] = 100.0 - r
    return sc


def _tiny_layer(n_host, n_gpu, k, cap_div, latent=2):
    lay = O.OracleLayer(H=1, D=1, k=k, latent=latent, n_host=n_host, n_gpu=n_gpu, max_batch=1,
                        cap_div=cap_div)
    hostkv = (np.arange(n_host * latent, dtype=np.uint16) + 1).reshape(n_host, latent)
    return lay, hostkv


def _step(lay, hostkv, ctx, winners, mode):
    q = np.zeros((1, 1, 1), np.uint16)
    w = np.zeros((1, 1), np.float32)
    kidx = np.zeros((lay.cfg.n_host, 1), np.uint8)
    return lay.step([0], [ctx], q, w, kidx, hostkv, mode=mode, ext_scores=_ext(ctx, winners))


def test_lru_eviction_with_reserve_by_hand():
    # 8 host tokens, 4 slots, k=2, cap=min(2, ceil(8/8))=1 -> reserve R=1; no prefetch
    lay, hk = _tiny_layer(8, 4, 2, 8)
    P = O.MODE_POS_INF
    o = _step(lay, hk, 8, [1, 5], P)      # t=0: both miss -> slots 0,1
    assert o["sel_slot"][0].tolist() == [0, 1] and o["n_evict"] == 0
    o = _step(lay, hk, 8, [2, 5], P)      # t=1: 5 hits (slot 1 -> prio 1); 2 -> slot 2
    assert o["n_miss"].tolist() == [1] and o["sel_slot"][0].tolist() == [2, 1]
    assert o["n_evict"] == 0              # 1 miss + R=1 - 2 free = 0
    assert lay.prio.tolist() == [0, 1, 1, -1]
    o = _step(lay, hk, 8, [3, 6], P)      # t=2: 2 misses, 1 free -> evict 2 (LRU)
    assert o["evicted"].tolist() == [0, 1]   # (prio 0, slot 0) then (prio 1, slot 1)
    assert o["sel_slot"][0].tolist() == [0, 1]
    assert lay.h2g.tolist() == [-1, -1, 2, 0, -1, -1, 1, -1]
    assert lay.g2h.tolist() == [3, 6, 2, -1]
    o = _step(lay, hk, 8, [2, 3], P)      # t=3: all hit, nothing moves
    assert o["n_miss"].tolist() == [0] and o["n_evict"] == 0
    assert lay.prio.tolist() == [3, 2, 3, -1] and lay.t == 4
    for h in range(8):                    # pool rows equal their host rows
        if lay.h2g[h] >= 0:
            assert np.array_equal(lay.pool[lay.h2g[h]], hk[h])


def test_prefetch_cap_free_list_and_protection_by_hand():
    # cap = min(2, ceil(8/4)) = 2; threshold -inf: every non-resident token is a candidate
    lay, hk = _tiny_layer(8, 4, 2, 4)
    N = O.MODE_NEG_INF
    o = _step(lay, hk, 8, [1, 5], N)      # t=0: prefetch tokens 0,1 -> slots 0,1
    assert o["pf_tok"][0, :2].tolist() == [0, 1] and o["pf_slot"][0, :2].tolist() == [0, 1]
    assert o["n_cand"].tolist() == [8] and o["n_miss"].tolist() == [1]
    assert o["sel_slot"][0].tolist() == [1, 2] and o["n_evict"] == 0
    o = _step(lay, hk, 8, [0, 7], N)      # t=1: one free slot -> only token 2 prefetched
    assert o["n_pf"].tolist() == [1] and o["pf_tok"][0, 0] == 2 and o["pf_slot"][0, 0] == 3
    assert o["n_cand"].tolist() == [5]
    # E = slots 1 (token 1) and 2 (token 5), both prio 0; the prefetched token 2 is protected
    assert o["evicted"].tolist() == [1, 2]
    assert o["sel_slot"][0].tolist() == [0, 1]
    assert lay.h2g.tolist() == [0, -1, 3, -1, -1, -1, -1, 1]
    assert lay.prio.tolist() == [1, 1, -1, 1]


def test_prefetch_cap_rounds_up():
    # ctx 7, cap_div 4 -> cap = min(k=4, ceil(7/4)=2) = 2
    lay, hk = _tiny_layer(8, 8, 4, 4)
    o = _step(lay, hk, 7, [0, 1, 2, 3], O.MODE_NEG_INF)
    assert o["n_pf"].tolist() == [2] and o["pf_tok"][0, :2].tolist() == [0, 1]
    assert o["n_cand"].tolist() == [7]


def test_capacity_error_leaves_state_consistent():
    lay, hk = _tiny_layer(8, 1, 2, 8)
    o = _step(lay, hk, 8, [3, 4], O.MODE_POS_INF)
    assert o["status"] == O.ECAPACITY and lay.t == 0
    assert (lay.h2g == -1).all() and lay.free.tolist() == [1]


def test_ema_threshold_drives_prefetch_by_hand():
    lay, hk = _tiny_layer(8, 8, 2, 4)
    E = O.MODE_EMA
    sc0 = np.array([[1, 9, 3, 8, 2, 7, 0, 4]], np.float32)   # top-2: 9 (tok1), 8 (tok3)
    q = np.zeros((1, 1, 1), np.uint16)
    w = np.zeros((1, 1), np.float32)
    kidx = np.zeros((8, 1), np.uint8)
    o = lay.step([0], [8], q, w, kidx, hk, mode=E, ext_scores=sc0)
    assert o["n_pf"].tolist() == [0]      # theta=+inf before the first k-th score
    assert lay.theta[0] == 8.0 and o["kth"][0] == 8.0
    sc1 = np.array([[1, 9, 3, 8, 2, 7.5, 8.5, 8]], np.float32)
    o = lay.step([0], [8], q, w, kidx, hk, mode=E, ext_scores=sc1)
    # candidates: score strictly above 8 and not resident -> token 6 (8.5) only; token 7
    # sits exactly on the threshold and is not a candidate
    assert o["n_cand"].tolist() == [1] and o["pf_tok"][0, 0] == 6
    assert o["sel_tok"][0].tolist() == [1, 6] and o["n_miss"].tolist() == [0]
    assert lay.theta[0] == np.float32(0.5 * 8.0 + 0.5 * 8.5)


# ------------------------------------------ invariants and losslessness

def _check_invariants(lay, o, ctx, host_base, hk):
    h2g, g2h, prio, free = lay.h2g, lay.g2h, lay.prio, lay.free
    res = np.nonzero(h2g >= 0)[0]
    assert np.array_equal(g2h[h2g[res]], res)                         # mutual inverses
    occ = np.nonzero(g2h >= 0)[0]
    assert np.array_equal(h2g[g2h[occ]], occ)
    assert np.array_equal(free == 1, g2h == -1) and np.array_equal(free == 1, prio == -1)
    assert res.size + int(free.sum()) == g2h.size
    assert (prio < lay.t).all()                                       # prio <= t_step
    for b in range(len(ctx)):
        sel = o["sel_tok"][b, : o["n_sel"][b]]
        hs = host_base[b] + sel
        assert (h2g[hs] >= 0).all()                                   # selected resident
        assert np.array_equal(o["sel_slot"][b, : sel.size], h2g[hs])
        assert (prio[h2g[hs]] == lay.t - 1).all()                     # touched this step
        assert np.array_equal(lay.pool[h2g[hs]], hk[hs])              # bytes equal host
    for h in res:
        assert np.array_equal(lay.pool[h2g[h]], hk[h])


def _small_workload(seed=0, B=2, ctx=(700, 513), H=4, D=32, k=64, n_gpu=400, steps=6,
                    rho=0.9):
    rng = np.random.default_rng(seed)
    ctx = np.array(ctx, np.int32)
    host_base = np.concatenate([[0], np.cumsum(ctx)[:-1]]).astype(np.int32)
    n_host = int(ctx.sum()) + 17
    kid = torch.from_numpy(rng.standard_normal((n_host, D)).astype(np.float32))
    kidx = kid.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    hk = rng.integers(0, 65536, size=(n_host, 8)).astype(np.uint16)
    w = rng.random((B, H)).astype(np.float32)
    st = rng.standard_normal((B, H, D)).astype(np.float32)
    qs = []
    for _ in range(steps):
        qs.append(torch.from_numpy(st).to(torch.bfloat16).view(torch.int16).numpy()
                  .view(np.uint16))
        st = rho * st + np.sqrt(1 - rho * rho) * rng.standard_normal(st.shape).astype(np.float32)
    return dict(ctx=ctx, host_base=host_base, n_host=n_host, kidx=kidx, hk=hk, w=w, qs=qs,
                H=H, D=D, k=k, n_gpu=n_gpu)


def _run_modes(wk, mode):
    lay = O.OracleLayer(wk["H"], wk["D"], wk["k"], 8, wk["n_host"], wk["n_gpu"],
                        len(wk["ctx"]), cap_div=32)
    outs = []
    for q in wk["qs"]:
        o = lay.step(wk["host_base"], wk["ctx"], q, wk["w"], wk["kidx"], wk["hk"], mode=mode)
        assert o["status"] == O.OK
        _check_invariants(lay, o, wk["ctx"], wk["host_base"], wk["hk"])
        gathered = [lay.pool[o["sel_slot"][b, : o["n_sel"][b]]].copy()
                    for b in range(len(wk["ctx"]))]
        outs.append((o, gathered))
    return lay, outs


def test_lossless_across_threshold_modes_and_invariants():
    wk = _small_workload()
    runs = {m: _run_modes(wk, m) for m in (O.MODE_EMA, O.MODE_NEG_INF, O.MODE_POS_INF)}
    base = runs[O.MODE_POS_INF][1]
    for m in (O.MODE_EMA, O.MODE_NEG_INF):
        for (o, g), (ob, gb) in zip(runs[m][1], base):
            assert np.array_equal(o["sel_tok"], ob["sel_tok"])
            for x, y in zip(g, gb):
                assert np.array_equal(x, y)
    # the modes really differ in what they move
    pf = {m: sum(int(o["n_pf"].sum()) for o, _ in runs[m][1]) for m in runs}
    assert pf[O.MODE_POS_INF] == 0 and pf[O.MODE_NEG_INF] > pf[O.MODE_EMA] > 0
    miss = {m: sum(int(o["n_miss"].sum()) for o, _ in runs[m][1][1:]) for m in runs}
    assert miss[O.MODE_EMA] < miss[O.MODE_POS_INF]


def test_eviction_pressure_keeps_invariants():
    # a pool barely larger than one step's selection forces eviction every step
    wk = _small_workload(seed=3, n_gpu=2 * 64 + 2 * 22 + 5, rho=0.3, steps=8)
    for m in (O.MODE_EMA, O.MODE_NEG_INF, O.MODE_POS_INF):
        lay, outs = _run_modes(wk, m)
        assert sum(o["n_evict"] for o, _ in outs) > 0


def test_oracle_is_deterministic():
    wk = _small_workload(seed=5, steps=3)
    a = _run_modes(wk, O.MODE_EMA)[0].snapshot()
    b = _run_modes(wk, O.MODE_EMA)[0].snapshot()
    for key in a:
        assert np.array_equal(a[key], b[key])


def test_short_context_selects_everything_and_skips_ema():
    wk = _small_workload(seed=6, ctx=(40, 64), steps=2)
    lay, outs = _run_modes(wk, O.MODE_EMA)
    o = outs[0][0]
    assert o["n_sel"].tolist() == [40, 64]
    assert o["sel_tok"][0, :40].tolist() == list(range(40))
    assert np.isinf(lay.theta[0]) and lay.theta[1] == o["kth"][1]


# ---------------------------------------------------------------- decode append
# R10 (append and writeback): each request's new token lands at host id
# host_base + ctx, nothing else changes, and ctx grows by one; a request without
# room or whose id is mapped stops the whole call with nothing written.

def _append_case(B=3, D=8, latent=16, n_host=256, room=4, seed=0):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, 40, B).astype(np.int32)
    span = (ctx + room + 15) // 16 * 16
    base = np.concatenate([[0], np.cumsum(span)[:-1]]).astype(np.int32)
    kidx = rng.integers(0, 256, (n_host, D), dtype=np.uint8)
    host = rng.integers(0, 65536, (n_host, latent), dtype=np.uint16)
    k_new = rng.integers(0, 256, (B, D), dtype=np.uint8)
    lat_new = rng.integers(0, 65536, (B, latent), dtype=np.uint16)
    return ctx, base, kidx, host, k_new, lat_new


def test_append_writes_exactly_the_next_row_of_each_request():
    ctx, base, kidx, host, k_new, lat_new = _append_case()
    k0, h0, c0 = kidx.copy(), host.copy(), ctx.copy()
    h2g = np.full(kidx.shape[0], -1, np.int32)
    assert O.append(base, ctx, h2g, k_new, lat_new, kidx, host, max_ctx=64) == O.OK
    assert np.array_equal(ctx, c0 + 1)
    rows = base.astype(np.int64) + c0
    changed = np.nonzero((kidx != k0).any(1) | (host != h0).any(1))[0]
    assert set(changed.tolist()) <= set(rows.tolist())
    for b, h in enumerate(rows):
        assert np.array_equal(kidx[h], k_new[b]) and np.array_equal(host[h], lat_new[b])
    # without advance the same rows are written and ctx stays
    c1 = ctx.copy()
    assert O.append(base, ctx, h2g, k_new, lat_new, kidx, host, max_ctx=64,
                    advance=False) == O.OK
    assert np.array_equal(ctx, c1)
    for b in range(ctx.size):
        assert np.array_equal(kidx[int(base[b]) + int(c1[b])], k_new[b])


def test_append_checks_room_and_mapping_and_writes_nothing_on_error():
    ctx, base, kidx, host, k_new, lat_new = _append_case(room=0)
    h2g = np.full(kidx.shape[0], -1, np.int32)
    # request 0 ends exactly where request 1 starts: its next id is taken
    ctx[0] = base[1] - base[0]
    k0, h0, c0 = kidx.copy(), host.copy(), ctx.copy()
    assert O.append(base, ctx, h2g, k_new, lat_new, kidx, host, max_ctx=64) == O.ECAPACITY
    assert np.array_equal(kidx, k0) and np.array_equal(host, h0) and np.array_equal(ctx, c0)
    # room everywhere, but one target id already mapped to a slot
    ctx, base, kidx, host, k_new, lat_new = _append_case(room=8)
    h2g = np.full(kidx.shape[0], -1, np.int32)
    h2g[int(base[2]) + int(ctx[2])] = 5
    c0 = ctx.copy()
    assert O.append(base, ctx, h2g, k_new, lat_new, kidx, host, max_ctx=64) == O.EDEVARG
    assert np.array_equal(ctx, c0)
    # the context limit and the end of the host pool
    h2g[:] = -1
    ctx2 = ctx.copy()
    ctx2[1] = 20
    assert O.append(base, ctx2, h2g, k_new, lat_new, kidx, host, max_ctx=20) == O.ECAPACITY
    base3 = base.copy()
    base3[-1] = kidx.shape[0] - int(ctx[-1])
    assert O.append(base3, ctx.copy(), h2g, k_new, lat_new, kidx, host, max_ctx=64) == \
        O.ECAPACITY


def test_append_skips_empty_rows_and_their_stale_ranges():
    # Hand-derived.  Row 1 is empty (ctx 0, released) and its stale host_base 10 is
    # exactly request 0's next id; row 3 is empty with a stale base whose id is mapped.
    # Rows 0 and 2 take their tokens at ids 10 and 37; the empty rows take nothing,
    # block nothing and do not grow.
    D, latent, n_host = 4, 8, 64
    base = np.array([0, 10, 32, 20], np.int32)
    ctx = np.array([10, 0, 5, 0], np.int32)
    kidx = np.zeros((n_host, D), np.uint8)
    host = np.zeros((n_host, latent), np.uint16)
    k_new = (np.arange(4 * D, dtype=np.uint8).reshape(4, D) + 1)
    lat_new = (np.arange(4 * latent, dtype=np.uint16).reshape(4, latent) + 100)
    h2g = np.full(n_host, -1, np.int32)
    h2g[20] = 3
    assert O.append(base, ctx, h2g, k_new, lat_new, kidx, host, max_ctx=64) == O.OK
    assert ctx.tolist() == [11, 0, 6, 0]
    assert np.array_equal(kidx[10], k_new[0]) and np.array_equal(host[10], lat_new[0])
    assert np.array_equal(kidx[37], k_new[2]) and np.array_equal(host[37], lat_new[2])
    written = np.nonzero(kidx.any(1) | host.any(1))[0].tolist()
    assert written == [10, 37]
    # without advance: the same two rows again, contexts unchanged
    ctx2 = np.array([10, 0, 5, 0], np.int32)
    assert O.append(base, ctx2, h2g, k_new, lat_new, kidx, host, max_ctx=64,
                    advance=False) == O.OK
    assert ctx2.tolist() == [10, 0, 5, 0]


# ---------------------------------------------------------- attention input
# R11: rows that name themselves.  Host row h holds h's own bytes, so every
# gathered row must decode to host_base[b] + sel_tok[b][i]; rows past n_sel are 0.

def test_gather_reads_the_selected_host_rows_in_selection_order():
    rng = np.random.default_rng(3)
    B, k, latent, n_host = 3, 16, 8, 300
    host = np.zeros((n_host, latent), np.uint16)
    host[:, 0] = np.arange(n_host) & 0xFFFF
    host[:, 1] = np.arange(n_host) >> 16
    host[:, 2:] = 0xABCD
    base = np.array([0, 100, 220], np.int32)
    ctx = np.array([90, 110, 60], np.int32)
    n_sel = np.array([16, 9, 0], np.int32)
    sel = np.full((B, k), -1, np.int32)
    for b in range(B):
        sel[b, :n_sel[b]] = rng.choice(ctx[b], n_sel[b], replace=False)
    out = O.gather(base, sel, n_sel, host)
    assert out.shape == (B, k, latent)
    for b in range(B):
        for i in range(k):
            if i < n_sel[b]:
                h = int(out[b, i, 0]) | (int(out[b, i, 1]) << 16)
                assert h == base[b] + sel[b, i]
                assert (out[b, i, 2:] == 0xABCD).all()
            else:
                assert not out[b, i].any()


# ------------------------------------------------------------ request lifecycle
def _two_requests_all_tails_resident():
    """Two requests with external scores that select each request's first and last
    tokens (plus a few between), two steps: every selected token ends resident."""
    n_host, n_gpu, k, latent = 64, 24, 4, 2
    lay = O.OracleLayer(H=1, D=1, k=k, latent=latent, n_host=n_host, n_gpu=n_gpu, max_batch=2,
                        cap_div=64)
    hk = (np.arange(n_host * latent, dtype=np.uint16) + 1).reshape(n_host, latent)
    base = np.array([0, 20], np.int32)
    ctx = np.array([20, 30], np.int32)
    q = np.zeros((2, 1, 1), np.uint16)
    w = np.zeros((2, 1), np.float32)
    kidx = np.zeros((n_host, 1), np.uint8)
    for winners in (((0, 19, 5, 7), (0, 29, 11, 3)), ((19, 2, 4, 8), (29, 1, 12, 13))):
        sc = np.zeros((2, 30), np.float32)
        for b in range(2):
            for r, s in enumerate(winners[b]):
                sc[b, s] = 50.0 - r
        o = lay.step(base, ctx, q, w, kidx, hk, mode=O.MODE_POS_INF, ext_scores=sc)
        assert o["status"] == O.OK
    return lay, hk, base, ctx


def _state(lay):
    return [a.copy() for a in (lay.h2g, lay.g2h, lay.prio, lay.free, lay.theta)]


def test_release_gives_back_exactly_the_request_slots():
    lay, hk, base, ctx = _two_requests_all_tails_resident()
    lay.theta[:] = [1.5, 2.5]
    h2g, g2h, prio, free, theta = _state(lay)
    r0 = np.arange(base[1], base[1] + ctx[1])
    mine = h2g[r0][h2g[r0] >= 0]
    assert h2g[base[1]] >= 0 and h2g[base[1] + ctx[1] - 1] >= 0 and mine.size == 7
    c = ctx.copy()
    assert O.release(lay, base, c, [0, 1], max_ctx=64) == O.OK
    assert list(c) == [20, 0]
    assert (lay.h2g[r0] == -1).all()
    assert (lay.g2h[mine] == -1).all() and (lay.free[mine] == 1).all()
    assert (lay.prio[mine] == -1).all()
    assert lay.theta[1] == np.inf and lay.theta[0] == np.float32(1.5)
    keep = np.ones(lay.g2h.size, bool)
    keep[mine] = False
    other = np.setdiff1d(np.arange(lay.h2g.size), r0)
    assert np.array_equal(lay.h2g[other], h2g[other])
    for cur, old in ((lay.g2h, g2h), (lay.prio, prio), (lay.free, free)):
        assert np.array_equal(cur[keep], old[keep])
    # the invariants of the maps still hold
    res = np.nonzero(lay.h2g >= 0)[0]
    assert np.array_equal(lay.g2h[lay.h2g[res]], res)
    assert np.array_equal(lay.free == 1, lay.g2h == -1)
    assert np.array_equal(lay.free == 1, lay.prio == -1)
    assert res.size + int(lay.free.sum()) == lay.g2h.size


def test_release_of_every_request_returns_the_initial_state():
    lay, hk, base, ctx = _two_requests_all_tails_resident()
    c = ctx.copy()
    assert O.release(lay, base, c, [1, 1], max_ctx=64) == O.OK
    fresh = O.OracleLayer(H=1, D=1, k=4, latent=2, n_host=64, n_gpu=24, max_batch=2, cap_div=64)
    for cur, new in zip(_state(lay), _state(fresh)):
        assert np.array_equal(cur, new)
    assert list(c) == [0, 0]


def test_release_rejects_a_range_that_does_not_fit_and_changes_nothing():
    lay, hk, base, ctx = _two_requests_all_tails_resident()
    before = _state(lay)
    for bad_base, bad_ctx in (([0, 20], [20, 65]), ([0, -1], [20, 30]), ([0, 40], [20, 30]),
                              ([0, 20], [20, -2])):
        c = np.array(bad_ctx, np.int32)
        assert O.release(lay, np.array(bad_base, np.int32), c, [1, 1], max_ctx=64) == O.EDEVARG
        assert list(c) == bad_ctx
        for cur, old in zip(_state(lay), before):
            assert np.array_equal(cur, old)


def test_admit_checks_in_order_and_changes_nothing_on_error():
    lay, hk, base, ctx = _two_requests_all_tails_resident()
    b0, c0 = base.copy(), ctx.copy()
    c0[1] = 0                                   # row 1 emptied without a release:
    #                                             its tokens stay mapped (stale)
    cases = [(2, 50, 4, O.EINVAL), (-1, 50, 4, O.EINVAL), (1, 50, 65, O.EINVAL),
             (1, -1, 4, O.EINVAL), (1, 60, 5, O.EINVAL), (0, 50, 4, O.EDEVARG),
             (1, 15, 10, O.ECAPACITY), (1, 19, 1, O.ECAPACITY), (1, 20, 10, O.EDEVARG),
             (1, 48, 1, O.EDEVARG)]
    lay.h2g[48] = 3                             # a stale id outside every range
    before = _state(lay)
    for b, bs, n, want in cases:
        hb, cc = b0.copy(), c0.copy()
        assert O.admit(lay, hb, cc, b, bs, n, max_ctx=64) == want, (b, bs, n)
        assert np.array_equal(hb, b0) and np.array_equal(cc, c0)
        for cur, old in zip(_state(lay), before):
            assert np.array_equal(cur, old)
    # a free range after request 1's: admitted, threshold back to "no estimate"
    lay.theta[1] = 7.0
    hb, cc = b0.copy(), c0.copy()
    assert O.admit(lay, hb, cc, 1, 50, 10, max_ctx=64) == O.OK
    assert list(hb) == [0, 50] and list(cc) == [20, 10] and lay.theta[1] == np.inf
    # touching ranges do not overlap; an empty range fits anywhere that is free
    hb, cc = b0.copy(), c0.copy()
    assert O.admit(lay, hb, cc, 1, 20, 0, max_ctx=64) == O.OK and list(cc) == [20, 0]


def test_readmitted_request_starts_cold_and_stays_lossless():
    wk = _small_workload(seed=5, B=3, ctx=(700, 513, 300), n_gpu=600, steps=6)
    lay_ref, ref = _run_modes(wk, O.MODE_EMA)
    lay = O.OracleLayer(wk["H"], wk["D"], wk["k"], 8, wk["n_host"], wk["n_gpu"], 3, cap_div=32)
    ctx = wk["ctx"].copy()
    base = wk["host_base"].copy()
    for t, q in enumerate(wk["qs"]):
        if t == 3:
            assert O.release(lay, base, ctx, [0, 1, 0], max_ctx=700) == O.OK
            assert O.admit(lay, base, ctx, 1, int(wk["host_base"][1]), int(wk["ctx"][1]),
                           max_ctx=700) == O.OK
        o = lay.step(base, ctx, q, wk["w"], wk["kidx"], wk["hk"], mode=O.MODE_EMA)
        assert o["status"] == O.OK
        _check_invariants(lay, o, ctx, base, wk["hk"])
        ro, rows = ref[t]
        for b in range(3):                      # selection never depends on the cache
            n = int(o["n_sel"][b])
            assert n == ro["n_sel"][b]
            assert np.array_equal(o["sel_tok"][b, :n], ro["sel_tok"][b, :n])
            assert np.array_equal(lay.pool[o["sel_slot"][b, :n]], rows[b])
        if t == 3:                              # cold: no estimate, nothing resident
            assert o["n_pf"][1] == 0 and o["n_miss"][1] == o["n_sel"][1] == wk["k"]
            assert lay.theta[1] == o["kth"][1]


def test_lifecycle_without_commit_leaves_the_batch_row_to_the_last_layer():
    lay, hk, base, ctx = _two_requests_all_tails_resident()
    lay2, _, _, _ = _two_requests_all_tails_resident()
    c = ctx.copy()
    assert O.release(lay, base, c, [0, 1], max_ctx=64, commit=False) == O.OK
    assert list(c) == [20, 30] and (lay.h2g[20:50] == -1).all()
    assert O.release(lay2, base, c, [0, 1], max_ctx=64) == O.OK   # the last layer
    assert list(c) == [20, 0]
    for cur, new in zip(_state(lay), _state(lay2)):
        assert np.array_equal(cur, new)
    hb = base.copy()
    lay.theta[1] = 3.0
    assert O.admit(lay, hb, c, 1, 20, 30, max_ctx=64, commit=False) == O.OK
    assert list(hb) == [0, 20] and list(c) == [20, 0] and lay.theta[1] == np.inf
    assert O.admit(lay2, hb, c, 1, 24, 26, max_ctx=64) == O.OK
    assert list(hb) == [0, 24] and list(c) == [20, 26]


# ------------------------------------------------------------ chunked prefill
def test_f16_rounding_matches_numpy_including_ties_and_subnormals():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, size=60000, dtype=np.uint64).astype(np.uint32)
    vals = bits.view(np.float32)
    vals = vals[np.isfinite(vals)]
    # exact ties between neighbouring halves, normal and subnormal, both signs
    h = rng.integers(1, 0x7BFF, size=4000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    ties = ((lo + hi) / 2).astype(np.float32)
    extra = np.array([0.0, -0.0, 65504, 65519.99, 65520, 65536, 1e30, -1e30, 2**-24, 2**-25,
                      3 * 2**-26, 2**-14, 2**-15 * 1.5, 0.1, -7.5], np.float32)
    for v in np.concatenate([vals, ties, -ties, extra]):
        want = int(np.float32(v).astype(np.float16).view(np.uint16))
        assert O.f16_bits(float(v)) == want, (float(v), hex(want))


def test_f16_buckets_by_hand_and_monotone():
    # fp16 of 0..7: 0x0000 0x3C00 0x4000 0x4200 0x4400 0x4500 0x4600 0x4700; a non-negative
    # half u has key u | 0x8000, a negative one the complement
    by_hand = {0.0: 0x80, 1.0: 0xBC, 2.0: 0xC0, 3.0: 0xC2, 4.0: 0xC4, 5.0: 0xC5, 6.0: 0xC6,
               7.0: 0xC7, -1.0: 0x43, -0.0: 0x80, 255 * 2**-24: 0x80, 2**-16: 0x81,
               2**-14: 0x84}
    for x, b in by_hand.items():
        assert O.f16_bucket(O.f16_bits(x)) == b, x
    xs = np.sort(np.random.default_rng(2).standard_normal(3000).astype(np.float32) * 50)
    bk = [O.f16_bucket(O.f16_bits(float(x))) for x in xs]
    assert all(a <= b for a, b in zip(bk, bk[1:]))


def _prefill_layer(n_host, n_gpu, k, latent=2, H=1, D=1):
    lay = O.OracleLayer(H=H, D=D, k=k, latent=latent, n_host=n_host, n_gpu=n_gpu, max_batch=1)
    hk = (np.arange(n_host * latent, dtype=np.uint16) + 1).reshape(n_host, latent)
    return lay, hk


def _prefill_ext(lay, hk, scores, pred=None, hb=0):
    Cq, N = scores.shape
    q = np.zeros((Cq, lay.cfg.H, lay.cfg.D), np.uint16)
    w = np.zeros((Cq, lay.cfg.H), np.float32)
    kidx = np.zeros((lay.cfg.n_host, lay.cfg.D), np.uint8)
    return O.prefill_chunk(lay, hb, N, q, w, kidx, pred=pred, host_kv=hk,
                           ext_scores=np.asarray(scores, np.float32))


def test_prefill_coarse_candidates_by_hand():
    lay, hk = _prefill_layer(64, 32, k=2)
    perm = [3, 7, 0, 5, 1, 6, 2, 4]
    o = _prefill_ext(lay, hk, np.array([perm], np.float32))
    # buckets of 7 and 6 are 0xC7 and 0xC6: two tokens reach k = 2 at 0xC6
    assert o["beta"][0] == 0xC6 and list(o["cand"]) == [1] and list(o["uni"]) == [1, 5]
    lay, hk = _prefill_layer(64, 32, k=3)
    o = _prefill_ext(lay, hk, np.array([perm], np.float32))
    assert o["beta"][0] == 0xC5 and list(o["cand"]) == [1, 5]
    # 12 .. 13.5 share bucket 0xCA: with no prediction nothing is strictly above
    sc = np.array([[10, 10.5, 11, 11.5, 12, 12.5, 13, 13.5]], np.float32)
    lay, hk = _prefill_layer(64, 32, k=3)
    o = _prefill_ext(lay, hk, sc)
    assert o["beta"][0] == 0xCA and o["n_qcand"][0] == 0 and list(o["uni"]) == [5, 6, 7]
    assert list(o["miss_h"]) == [5, 6, 7] and o["pf_h"].size == 0
    # predicted k-th 12.5: differences 1, 0.5, 0 sit in buckets 0xBC, 0xB8, 0x80
    lay, hk = _prefill_layer(64, 32, k=3)
    o = _prefill_ext(lay, hk, sc, pred=np.array([12.5], np.float32))
    assert o["beta"][0] == 0x80 and list(o["cand"]) == [6, 7]
    assert list(o["pf_h"]) == [6, 7] and list(o["pf_g"]) == [0, 1]
    assert list(o["miss_h"]) == [5] and list(o["miss_g"]) == [2]


def _prefill_workload(seed=0, C=6, N=700, H=4, D=32, k=64, chunks=3, rho=0.9, n_gpu=1000):
    rng = np.random.default_rng(seed)
    n_host = N + 40
    hb = 16
    kid = torch.from_numpy(rng.standard_normal((n_host, D)).astype(np.float32))
    kidx = kid.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    hk = rng.integers(0, 65536, size=(n_host, 8)).astype(np.uint16)
    st = rng.standard_normal((H, D)).astype(np.float32)
    qs, ws = [], []
    for _ in range(chunks):
        rows = []
        for _ in range(C):  # AR(1) along the prompt positions
            rows.append(torch.from_numpy(st).to(torch.bfloat16).view(torch.int16).numpy()
                        .view(np.uint16))
            st = rho * st + np.sqrt(1 - rho * rho) * rng.standard_normal(st.shape) \
                .astype(np.float32)
        qs.append(np.stack(rows))
        ws.append(rng.random((C, H)).astype(np.float32))
    return dict(N=N, H=H, D=D, k=k, n_host=n_host, hb=hb, kidx=kidx, hk=hk, qs=qs, ws=ws,
                n_gpu=n_gpu)


def _prefill_run(wk, use_pred=True, n_gpu=None):
    lay = O.OracleLayer(wk["H"], wk["D"], wk["k"], 8, wk["n_host"], n_gpu or wk["n_gpu"], 1)
    outs, pred = [], None
    for q, w in zip(wk["qs"], wk["ws"]):
        before = dict(h2g=lay.h2g.copy(), free=lay.free.copy(), t=lay.t)
        o = O.prefill_chunk(lay, wk["hb"], wk["N"], q, w, wk["kidx"], pred=pred,
                            host_kv=wk["hk"])
        outs.append((o, before, dict(h2g=lay.h2g.copy(), prio=lay.prio.copy(), t=lay.t)))
        if o["status"] != O.OK:
            break
        pred = o["kth"].copy() if use_pred else None
    return lay, outs


def test_prefill_candidates_are_exact_top_k_members():
    # every token above a query's boundary bucket is one of its exact top-k (the
    # bucket of a rounded difference never decreases as the score grows)
    wk = _prefill_workload()
    for use_pred in (False, True):
        lay, outs = _prefill_run(wk, use_pred)
        pred = None
        for o, _, _ in outs:
            assert o["status"] == O.OK
            union = set()
            for i in range(o["kth"].size):
                sel = set(o["sel"][i, : o["n_sel"][i]].tolist())
                assert len(sel) == wk["k"]
                row = o["scores"][i]
                p = np.float32(0.0 if pred is None else pred[i])
                above = {s for s in range(wk["N"])
                         if O.f16_bucket(O.f16_bits(float(row[s] - p))) > o["beta"][i]}
                assert above <= sel and len(above) == o["n_qcand"][i] < wk["k"]
                union |= above
            assert sorted(union) == o["cand"].tolist()
            assert set(o["cand"].tolist()) <= set(o["uni"].tolist())
            pred = o["kth"].copy() if use_pred else None


def test_prefill_prediction_equal_to_the_kth_puts_the_boundary_at_zero():
    wk = _prefill_workload(seed=4)
    lay, outs = _prefill_run(wk, use_pred=False)
    o0 = outs[0][0]
    # the same chunk again on a fresh layer, predicted k-th = the exact k-th
    lay2 = O.OracleLayer(wk["H"], wk["D"], wk["k"], 8, wk["n_host"], wk["n_gpu"], 1)
    o1 = O.prefill_chunk(lay2, wk["hb"], wk["N"], wk["qs"][0], wk["ws"][0], wk["kidx"],
                         pred=o0["kth"], host_kv=wk["hk"])
    for i in range(o0["kth"].size):
        assert o1["beta"][i] == 0x80                       # difference 0 is bucket 0x80
        row = o0["scores"][i]
        sel = o0["sel"][i, : o0["n_sel"][i]]
        near = int(((row[sel] - o0["kth"][i]) < 2.0**-16).sum())
        assert o1["n_qcand"][i] == wk["k"] - near          # all but the ties near the k-th
        assert o1["n_qcand"][i] >= o0["n_qcand"][i]
    assert np.array_equal(o1["uni"], o0["uni"]) and o1["pf_h"].size >= o0["pf_h"].size


def test_prefill_state_after_each_chunk():
    wk = _prefill_workload(seed=7, chunks=4)
    lay, outs = _prefill_run(wk)
    hb = wk["hb"]
    for o, before, after in outs:
        assert o["status"] == O.OK
        t = before["t"]
        assert after["t"] == t + 1
        hu = hb + o["uni"]
        assert (after["h2g"][hu] >= 0).all()                       # the union is resident
        assert (after["prio"][after["h2g"][hu]] == t).all()         # and protected
        was = before["h2g"][hu] >= 0
        # the early transfer: exactly the candidates that were not resident, in order
        hc = hb + o["cand"]
        assert np.array_equal(o["pf_h"], hc[before["h2g"][hc] < 0])
        # then the rest of the union, in order
        rest = np.setdiff1d(hu[~was], o["pf_h"])
        assert np.array_equal(o["miss_h"], rest)
        # both take the lowest free slots, in that order
        free0 = np.nonzero(before["free"])[0]
        n = o["pf_h"].size + o["miss_h"].size
        assert np.array_equal(np.concatenate([o["pf_g"], o["miss_g"]]), free0[:n])
        assert np.array_equal(after["h2g"][o["pf_h"]], o["pf_g"])
    # maps are inverses and the pool holds the host rows of every resident token
    res = np.nonzero(lay.h2g >= 0)[0]
    assert np.array_equal(lay.g2h[lay.h2g[res]], res)
    assert np.array_equal(lay.free == 1, lay.g2h == -1)
    assert np.array_equal(lay.free == 1, lay.prio == -1)
    assert np.array_equal(lay.pool[lay.h2g[res]], wk["hk"][res])
    # later chunks reuse what earlier ones brought in
    assert outs[-1][0]["miss_h"].size + outs[-1][0]["pf_h"].size < outs[0][0]["uni"].size


def test_prefill_selection_does_not_depend_on_the_prediction():
    wk = _prefill_workload(seed=9, chunks=3)
    lay_a, a = _prefill_run(wk, use_pred=False)
    lay_b, b = _prefill_run(wk, use_pred=True)
    for (oa, _, _), (ob, _, _) in zip(a, b):
        assert np.array_equal(oa["uni"], ob["uni"]) and np.array_equal(oa["sel"], ob["sel"])
        assert np.array_equal(oa["kth"].view(np.uint32), ob["kth"].view(np.uint32))
    res = np.nonzero(lay_a.h2g >= 0)[0]
    assert np.array_equal(res, np.nonzero(lay_b.h2g >= 0)[0])
    assert np.array_equal(lay_a.pool[lay_a.h2g[res]], lay_b.pool[lay_b.h2g[res]])


def _same(lay, snap):
    for key, v in snap.items():
        cur = getattr(lay, key)
        assert (cur == v) if key == "t" else np.array_equal(cur, v), key


def test_prefill_capacity_errors_per_stage_and_short_history_takes_everything():
    wk = _prefill_workload(seed=3, chunks=1)
    probe = O.OracleLayer(wk["H"], wk["D"], wk["k"], 8, wk["n_host"], wk["n_gpu"], 1)
    full = O.prefill_chunk(probe, wk["hb"], wk["N"], wk["qs"][0], wk["ws"][0], wk["kidx"],
                           pred=None, host_kv=wk["hk"])
    n_c, n_u = full["cand"].size, full["uni"].size
    assert 0 < n_c < n_u
    # too few slots for the candidates: nothing changes
    lay = O.OracleLayer(wk["H"], wk["D"], wk["k"], 8, wk["n_host"], n_c - 1, 1)
    snap = lay.snapshot()
    o = O.prefill_chunk(lay, wk["hb"], wk["N"], wk["qs"][0], wk["ws"][0], wk["kidx"],
                        host_kv=wk["hk"])
    assert o["status"] == O.ECAPACITY and o["pf_h"].size == 0
    _same(lay, snap)
    # room for the candidates only: they stay installed, nothing else changes
    lay = O.OracleLayer(wk["H"], wk["D"], wk["k"], 8, wk["n_host"], n_u - 1, 1)
    o = O.prefill_chunk(lay, wk["hb"], wk["N"], wk["qs"][0], wk["ws"][0], wk["kidx"],
                        host_kv=wk["hk"])
    assert o["status"] == O.ECAPACITY and o["miss_h"].size == 0 and lay.t == 0
    assert np.array_equal(o["pf_h"], wk["hb"] + full["cand"])
    assert np.array_equal(o["pf_g"], np.arange(n_c))
    assert np.array_equal(np.nonzero(lay.h2g >= 0)[0], o["pf_h"])
    assert int(lay.free.sum()) == n_u - 1 - n_c
    # a history no longer than k: every token is selected and moves early
    lay = O.OracleLayer(wk["H"], wk["D"], 64, 8, wk["n_host"], 200, 1)
    o = O.prefill_chunk(lay, wk["hb"], 50, wk["qs"][0], wk["ws"][0], wk["kidx"],
                        host_kv=wk["hk"])
    assert o["status"] == O.OK and (o["beta"] == -1).all()
    assert list(o["uni"]) == list(range(50)) == list(o["cand"])
    assert np.array_equal(o["pf_h"], wk["hb"] + np.arange(50)) and o["miss_h"].size == 0


# ------------------------------------------------------------------ page tables
# R14: with a page table a request's token s is host id 16 * page[s // 16] + s % 16.
# Pinned by invariance (the method's results do not depend on where the pages lie;
# only the host ids in the maps move with the pages) and by hand-derived cases.

def _scatter_pages(wk, seed, spare=5):
    """The contiguous workload's requests moved to scattered pages: returns (pages
    [B, stride], kidx, hk, n_host, perm) where perm maps each contiguous host id of a
    request token to its paged host id."""
    rng = np.random.default_rng(seed)
    ctx, base = wk["ctx"], wk["host_base"]
    npages = [(int(c) + 15) // 16 for c in ctx]
    stride = max(npages) + 2
    total = sum(npages)
    phys = rng.permutation(total + spare)[:total]  # distinct pages anywhere in the pool
    n_host = 16 * (total + spare)
    pages = np.full((len(ctx), stride), -1, np.int32)
    kidx = np.zeros((n_host, wk["D"]), np.uint8)
    hk = np.zeros((n_host, wk["hk"].shape[1]), np.uint16)
    perm = {}
    i = 0
    for b, c in enumerate(ctx):
        for j in range(npages[b]):
            pages[b, j] = phys[i]
            i += 1
        for s in range(int(c)):
            h0 = int(base[b]) + s
            h1 = 16 * int(pages[b, s // 16]) + s % 16
            kidx[h1] = wk["kidx"][h0]
            hk[h1] = wk["hk"][h0]
            perm[h0] = h1
    return pages, kidx, hk, n_host, perm


@pytest.mark.parametrize("mode", [O.MODE_EMA, O.MODE_NEG_INF])
def test_scattered_pages_give_the_same_steps_with_moved_host_ids(mode):
    # a ragged batch under eviction pressure, run once with contiguous ranges and once
    # with every request's pages scattered over a larger pool in random order
    wk = _small_workload(ctx=(300, 177, 250), B=3, n_gpu=3 * 64 + 50, steps=6, rho=0.7)
    pages, kidx2, hk2, n_host2, perm = _scatter_pages(wk, seed=4)
    H, D, k = wk["H"], wk["D"], wk["k"]
    a = O.OracleLayer(H, D, k, 8, wk["n_host"], wk["n_gpu"], 3, cap_div=32)
    p = O.OracleLayer(H, D, k, 8, n_host2, wk["n_gpu"], 3, cap_div=32)
    ids = np.array(sorted(perm), np.int64)
    moved = np.array([perm[h] for h in ids], np.int64)
    for t, q in enumerate(wk["qs"]):
        oa = a.step(wk["host_base"], wk["ctx"], q, wk["w"], wk["kidx"], wk["hk"], mode=mode)
        op = p.step(None, wk["ctx"], q, wk["w"], kidx2, hk2, mode=mode, pages=pages)
        assert oa["status"] == op["status"] == O.OK
        for key in ("scores", "sel_tok", "sel_slot", "n_sel", "kth", "pf_tok", "pf_slot", "n_pf",
                    "n_cand", "miss_tok", "n_miss", "evicted"):
            assert np.array_equal(oa[key], op[key]), (t, key)
        assert oa["n_evict"] == op["n_evict"]
        assert np.array_equal(a.theta, p.theta) and a.t == p.t
        assert np.array_equal(a.prio, p.prio) and np.array_equal(a.free, p.free)
        assert np.array_equal(a.pool, p.pool), (t, "pool bytes")
        # the maps, with host ids carried along by the pages
        assert np.array_equal(p.h2g[moved], a.h2g[ids])
        others = np.setdiff1d(np.arange(n_host2), moved)
        assert (p.h2g[others] == -1).all()
        occ = a.g2h >= 0
        assert np.array_equal(p.g2h[~occ], a.g2h[~occ])
        assert np.array_equal(p.g2h[occ], [perm[int(h)] for h in a.g2h[occ]])
    assert sum(int(o) for o in [a.t]) == 6


def test_paged_append_writes_into_the_listed_page_by_hand():
    # request 0 holds pages [5, 2], request 1 pages [0, 7]; contexts 16 and 20:
    # request 0's token 16 opens its second page (id 16*2 + 0 = 32), request 1's
    # token 20 is id 16*7 + 4 = 116
    D, latent, n_host = 4, 8, 160
    pages = np.array([[5, 2, -1], [0, 7, -1]], np.int32)
    ctx = np.array([16, 20], np.int32)
    kidx = np.zeros((n_host, D), np.uint8)
    host = np.zeros((n_host, latent), np.uint16)
    k_new = np.array([[1, 2, 3, 4], [5, 6, 7, 8]], np.uint8)
    lat_new = (np.arange(2 * latent, dtype=np.uint16).reshape(2, latent) + 9)
    h2g = np.full(n_host, -1, np.int32)
    assert O.append(None, ctx, h2g, k_new, lat_new, kidx, host, max_ctx=48,
                    pages=pages) == O.OK
    assert ctx.tolist() == [17, 21]
    assert np.nonzero(kidx.any(1))[0].tolist() == [32, 116]
    assert np.array_equal(kidx[32], k_new[0]) and np.array_equal(host[116], lat_new[1])
    # no page listed for the next token (slot 2 holds -1), a page slot past the table,
    # a page past the pool, and a mapped id: each stops the call with nothing written
    k0, c0 = kidx.copy(), np.array([32, 21], np.int32)
    assert O.append(None, c0, h2g, k_new, lat_new, kidx, host, max_ctx=64,
                    pages=pages) == O.ECAPACITY
    c1 = np.array([48, 21], np.int32)
    assert O.append(None, c1, h2g, k_new, lat_new, kidx, host, max_ctx=64,
                    pages=pages) == O.ECAPACITY
    far = pages.copy()
    far[1, 1] = 10  # ids 160..175: past the pool
    assert O.append(None, np.array([17, 21], np.int32), h2g, k_new, lat_new, kidx, host,
                    max_ctx=64, pages=far) == O.ECAPACITY
    h2g[16 * 7 + 5] = 3
    assert O.append(None, np.array([17, 21], np.int32), h2g, k_new, lat_new, kidx, host,
                    max_ctx=64, pages=pages) == O.EDEVARG
    assert np.array_equal(kidx, k0) and c0.tolist() == [32, 21]


def test_paged_release_gives_back_the_slots_of_the_listed_pages_by_hand():
    # request 0: pages [3, 0], 20 tokens (ids 48..63 and 0..3); request 1: page [1],
    # 10 tokens (ids 16..25).  Slots: 48 -> 1, 50 -> 4, 2 -> 0 (request 0), 20 -> 2
    # (request 1), and id 5 -> 3 (page 0 but past request 0's 20 tokens)
    lay = O.OracleLayer(H=1, D=1, k=4, latent=2, n_host=80, n_gpu=6, max_batch=2)
    for h, g in ((48, 1), (50, 4), (2, 0), (20, 2), (5, 3)):
        lay.h2g[h], lay.g2h[g], lay.free[g], lay.prio[g] = g, h, 0, 7
    pages = np.array([[3, 0], [1, -1]], np.int32)
    ctx = np.array([20, 10], np.int32)
    lay.theta[:] = [4.0, 5.0]
    assert O.release(lay, None, ctx, [1, 0], max_ctx=32, pages=pages) == O.OK
    assert ctx.tolist() == [0, 10]
    assert lay.free.tolist() == [1, 1, 0, 0, 1, 1]
    assert lay.g2h.tolist() == [-1, -1, 20, 5, -1, -1]
    assert (lay.h2g[[48, 50, 2]] == -1).all() and lay.h2g[20] == 2 and lay.h2g[5] == 3
    assert lay.theta.tolist() == [np.inf, 5.0]
    # a page outside the pool: nothing changes
    bad = np.array([[3, 0], [9, -1]], np.int32)
    before = [x.copy() for x in (lay.h2g, lay.g2h, lay.free)]
    assert O.release(lay, None, np.array([0, 10], np.int32), [0, 1], max_ctx=32,
                     pages=bad) == O.EDEVARG
    for x, y in zip((lay.h2g, lay.g2h, lay.free), before):
        assert np.array_equal(x, y)


def test_paged_admission_checks_in_order_and_reuses_a_hole_by_hand():
    # a pool of 120 host ids: pages 0..6 are whole, page 7 would run past the pool;
    # request 0 lives on pages [6, 1]; row 1 is empty
    lay = O.OracleLayer(H=1, D=1, k=4, latent=2, n_host=120, n_gpu=4, max_batch=2)
    ctx = np.array([30, 0], np.int32)
    pages = np.array([[6, 1, -1], [-1, -1, -1]], np.int32)

    def admit(row1, n, expect):
        pg = pages.copy()
        pg[1] = row1
        c = ctx.copy()
        th = lay.theta.copy()
        assert O.admit(lay, None, c, 1, 0, n, max_ctx=48, pages=pg) == expect, (row1, n)
        if expect != O.OK:
            assert np.array_equal(c, ctx) and np.array_equal(lay.theta, th)
        return c

    admit([2, 3, 4], 49, O.EINVAL)                       # longer than max_ctx
    c = ctx.copy()
    c[1] = 5
    assert O.admit(lay, None, c, 1, 0, 10, max_ctx=48, pages=pages) == O.EDEVARG  # in use
    admit([2, 7, -1], 20, O.EDEVARG)                     # page 7 runs past the pool
    admit([2, -1, 3], 20, O.EDEVARG)                     # no page listed for token 16
    admit([2, 2, -1], 20, O.EDEVARG)                     # a page listed twice
    admit([2, 1, -1], 20, O.ECAPACITY)                   # page 1 is request 0's
    lay.h2g[16 * 3 + 2] = 0                              # token 18 (page 3) still mapped
    lay.g2h[0], lay.free[0], lay.prio[0] = 16 * 3 + 2, 0, 0
    admit([2, 3, -1], 20, O.EDEVARG)
    admit([2, 3, -1], 18, O.OK)                          # 18 tokens stop before that id
    # page 1 of request 0 is only its tokens 16..29: a third page of row 1 past its 20
    # tokens is not checked; pages 2 and 0 are a hole no live request uses
    lay.theta[1] = 3.0
    c = admit([2, 0, 1], 20, O.OK)
    assert c.tolist() == [30, 20] and lay.theta[1] == np.inf


def test_paged_gather_reads_the_rows_of_the_listed_pages():
    # host row h holds h itself, so each gathered row names the id it came from
    n_host, latent = 96, 4
    host = np.zeros((n_host, latent), np.uint16)
    host[:, 0] = np.arange(n_host)
    pages = np.array([[4, 0], [2, 5]], np.int32)
    sel = np.array([[0, 15, 16, 17], [3, 20, 0, 0]], np.int32)
    n_sel = np.array([4, 2], np.int32)
    out = O.gather(None, sel, n_sel, host, pages=pages)
    assert out[0, :, 0].tolist() == [64, 79, 0, 1]
    assert out[1, :2, 0].tolist() == [35, 84] and not out[1, 2:].any()
