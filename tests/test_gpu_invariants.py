"""echo_check_invariants through the C ABI: the device check of one layer's
cache-management state.

After every decode step of a ragged batch under eviction pressure the check must
count no violation, its resident and occupied counts must equal the state read
back, and the status must stay 0.  Then single entries of the state are corrupted
from the host, one kind at a time (a map entry, a free flag, a priority, the free
list, a reported slot): the report must equal the counts of a plain NumPy check of
the same definitions on the corrupted state, and the status must become
ECHO_ECORRUPT.  With the entry restored and the workspace reset the check is clean
again.
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


def _say(msg):
    print(msg, flush=True)


def numpy_counts(st, n_sel, sel_tok, sel_slot, host_ids, ctx, check_sel=True):
    """The invariants of echo_check_invariants, counted on state read back;
    host_ids(b, s) gives the host id of request b's token s."""
    h2g, g2h, prio, free = st["h2g"], st["g2h"], st["prio"], st["free"].astype(np.int64)
    n_host, n_gpu, t = h2g.size, g2h.size, st["t"]
    c = np.zeros(abi.ECHO_INV_WORDS, np.int64)
    res = h2g >= 0
    c[abi.ECHO_INV_RESIDENT] = res.sum()
    hs = np.nonzero(res)[0]
    gs = h2g[hs]
    bad_h = (gs >= n_gpu) | (g2h[np.minimum(gs, n_gpu - 1)] != hs)
    c[abi.ECHO_INV_H2G] = bad_h.sum() + (h2g < -1).sum()
    ok_free = ((free == 1) & (g2h == -1) & (prio == -1)) | ((free == 0) & (g2h >= 0) & (prio >= 0))
    c[abi.ECHO_INV_FREE] = (~ok_free).sum()
    occ = free == 0
    c[abi.ECHO_INV_OCCUPIED] = occ.sum()
    c[abi.ECHO_INV_PRIO] = (occ & ((prio < 0) | (prio >= t))).sum()
    ms = np.nonzero(g2h >= 0)[0]
    hm = g2h[ms]
    bad_g = (hm >= n_host) | (h2g[np.minimum(hm, n_host - 1)] != ms)
    c[abi.ECHO_INV_G2H] = bad_g.sum() + (g2h < -1).sum()
    nfree = int(np.clip(st["nfree"], 0, n_gpu))
    lst = st["idxbuf"][:nfree]
    inr = (lst >= 0) & (lst < n_gpu)
    ok = inr.copy()
    ok[inr] &= free[lst[inr]] == 1
    ok[1:] &= lst[:-1] < lst[1:]
    c[abi.ECHO_INV_FREE_LIST] = (~ok).sum() + int(st["nfree"] != n_gpu - occ.sum())
    if check_sel:
        for b in range(len(ctx)):
            n = int(np.clip(n_sel[b], 0, sel_tok.shape[1]))
            for i in range(n):
                s = int(sel_tok[b, i])
                good = 0 <= s < ctx[b]
                h = int(host_ids(b, [s])[0]) if good else -1
                good = good and 0 <= h < n_host
                if good:
                    g = int(h2g[h])
                    good = 0 <= g < n_gpu and g == sel_slot[b, i] and prio[g] == t - 1
                c[abi.ECHO_INV_SELECTED] += 0 if good else 1
    return c


def _check(rig, report, with_batch=True):
    R.check(abi.echo_check_invariants(rig.dims, rig.layer.struct,
                                      rig.batch.struct if with_batch else None, rig.ws.ws,
                                      report.data_ptr(), R.stream_handle()),
            "echo_check_invariants")
    torch.cuda.current_stream().synchronize()
    return report.cpu().numpy().astype(np.int64), int(rig.ws.status.item())


def _expected(rig):
    torch.cuda.current_stream().synchronize()
    out = rig.ws.read(rig.B)
    return numpy_counts(rig.layer.state(), out["n_sel"], out["sel_tok"], out["sel_slot"],
                        rig.host_ids, rig.ctx)


def test_clean_state_after_every_step_and_each_corruption_is_reported():
    wl = get("single_layer").scaled(rho=0.6, steps=6)
    ctx = [3000, 1777, 2561]
    _say(f"invariant check: 64x128 ragged {ctx}, pool with eviction")
    rig = H.Rig(wl, steps=6, ctx=ctx, n_gpu=3 * 256 + 2 * 120, n_host=8000, top_k=256,
                cap_div=64)
    report = torch.full((abi.ECHO_INV_WORDS,), -1, dtype=torch.int32, device="cuda")
    for t in range(4):
        rig.step_and_compare(H.MODE_EMA)
        got, status = _check(rig, report)
        want = _expected(rig)
        assert status == 0, abi.echo_status_string(status)
        assert np.array_equal(got, want), (t, got, want)
        assert got[:abi.ECHO_INV_RESIDENT].sum() == 0
        assert got[abi.ECHO_INV_RESIDENT] == got[abi.ECHO_INV_OCCUPIED] > 0
    # without a batch the selection is not looked at
    got, status = _check(rig, report, with_batch=False)
    assert status == 0 and got[abi.ECHO_INV_SELECTED] == 0
    _say(f"  clean: resident {got[abi.ECHO_INV_RESIDENT]}, occupied {got[abi.ECHO_INV_OCCUPIED]}")

    L = rig.layer
    st = L.state()
    occ = np.nonzero(st["free"] == 0)[0]
    g0, g1 = int(occ[3]), int(occ[10])
    h0 = int(st["g2h"][g0])
    out = rig.ws.read(rig.B)

    def corrupt(tensor, idx, value, kind):
        old = tensor[idx].clone()
        tensor[idx] = value
        got, status = _check(rig, report)
        want = _expected(rig)
        assert np.array_equal(got, want), (kind, got, want)
        assert status == abi.ECHO_ECORRUPT, (kind, status)
        _say(f"  {kind}: report {got.tolist()}")
        tensor[idx] = old
        rig.ws.reset()
        got, status = _check(rig, report)
        assert status == 0 and got[:abi.ECHO_INV_RESIDENT].sum() == 0, (kind, "restored", got)
        return want

    w = corrupt(L.h2g, h0, g1, "h2g points at another occupied slot")
    assert w[abi.ECHO_INV_H2G] >= 1 and w[abi.ECHO_INV_G2H] >= 1
    w = corrupt(L.free, g0, 1, "free flag set on an occupied slot")
    assert w[abi.ECHO_INV_FREE] == 1 and w[abi.ECHO_INV_FREE_LIST] >= 1
    w = corrupt(L.prio, g0, int(st["t"]), "priority in the future")
    assert w[abi.ECHO_INV_PRIO] == 1
    nfree = st["nfree"]
    assert nfree >= 2
    w = corrupt(L.idxbuf, 0, int(st["idxbuf"][1]), "free list not ascending")
    assert w[abi.ECHO_INV_FREE_LIST] >= 1
    w = corrupt(rig.ws.sel_slot[0], 0, int(out["sel_slot"][0, 1]), "reported slot wrong")
    assert w[abi.ECHO_INV_SELECTED] == 1
    rig.close()
