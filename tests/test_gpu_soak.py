"""A longer decode run with the whole request lifecycle mixed in, against the oracle.

Five ragged requests decode for 24 steps on a pool small enough to evict every step.
After every step each request's new token is appended (tiled K in HBM, latent in the
host pool, the context grows); at steps 3, 9 and 15 one live request, drawn from a
seeded generator, is released, and three steps later it is admitted again over a
shorter prefix of its old host range, cold.  Every step, append, release and
admission is compared with the oracle as in the other GPU tests (selection, prefetch,
misses, eviction, maps, free list, pool bytes, thresholds), and every selected row the
attention would read must equal the host copy.  The paged run does the same with every
request on 16-id pages scattered over the pool: appends open unused pages, and a
released request comes back on a shuffled subset of its own old pages.
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


def _lossless(rig, out):
    rows = rig.gathered()
    for b in range(rig.B):
        n = int(out["n_sel"][b])
        hs = rig.host_ids(b, out["sel_tok"][b, :n])
        assert np.array_equal(rows[b], rig.orc_host[hs]), ("attention input", b)


@pytest.mark.parametrize("mode", [H.MODE_EMA, H.MODE_NEG_INF])
def test_decode_with_appends_releases_and_readmissions(mode):
    steps = 24
    ctx = [2500, 1777, 3000, 900, 2222]
    print(f"soak: {len(ctx)} requests {ctx}, {steps} steps, mode {mode}", flush=True)
    wl = get("single_layer").scaled(rho=0.6, steps=steps)
    # room: each request's host range has space for every token it can append
    rig = H.Rig(wl, steps=steps, ctx=ctx, n_gpu=5 * 256 + 400, n_host=16_000, top_k=256,
                cap_div=64, max_ctx=max(ctx) + steps, room=steps)
    base0 = [int(x) for x in rig.base]
    rng = np.random.default_rng(11)
    released = {}  # row -> step it was released at
    events = 0
    for t in range(steps):
        live = [b for b in range(rig.B) if int(rig.ctx[b]) > 0]
        if t in (3, 9, 15) and len(live) > 2:
            b = int(rng.choice(live))
            mask = np.zeros(rig.B, np.int32)
            mask[b] = 1
            assert rig.release_and_compare(mask) == O.OK
            assert int(rig.ctx[b]) == 0
            released[b] = t
            events += 1
        for b, t_rel in list(released.items()):
            if t - t_rel == 3:
                # a shorter prefix of the old range: clear of every live request's
                # growth, and room left for this one's own appends
                length = int(rng.integers(200, ctx[b]))
                assert rig.admit_and_compare(b, base0[b], length) == O.OK
                assert int(rig.ctx[b]) == length
                del released[b]
                events += 1
        out, o = rig.step_and_compare(mode)
        assert out["status"] == 0
        _lossless(rig, out)
        assert rig.append_and_compare() == O.OK
        if t % 4 == 3:
            print(f"  step {t}: ctx {list(rig.ctx)}, missed {list(out['n_miss'])}, "
                  f"evicted {int(o['n_evict'])}", flush=True)
    assert events == 6
    assert sum(int(o["n_evict"]) for _, o in rig.history) > 0
    rig.close()


def _free_pages(rig):
    """Pool pages no request's row lists, in a fixed scrambled order."""
    used = set(int(p) for p in rig.pages.ravel() if p >= 0)
    free = [p for p in range(rig.wl.n_host // 16) if p not in used]
    return [int(p) for p in np.random.default_rng(11).permutation(free)]


def test_paged_decode_with_appends_releases_and_readmissions():
    # The same run on page tables: every request's tokens on 16-id pages scattered over
    # the pool; appends open new pages from the pool's unused ones, and a released
    # request comes back on a shuffled subset of its own old pages (the holes).
    steps = 24
    ctx = [2500, 1777, 3000, 900, 2222]
    print(f"paged soak: {len(ctx)} requests {ctx}, {steps} steps", flush=True)
    wl = get("single_layer").scaled(rho=0.6, steps=steps)
    rig = H.Rig(wl, steps=steps, ctx=ctx, n_gpu=5 * 256 + 400, n_host=16_000, top_k=256,
                cap_div=64, max_ctx=max(ctx) + steps, paged=True, stride_extra=4)
    fresh = iter(_free_pages(rig))
    rng = np.random.default_rng(12)
    released = {}  # row -> (step, its old pages)
    events = 0
    for t in range(steps):
        live = [b for b in range(rig.B) if int(rig.ctx[b]) > 0]
        if t in (3, 9, 15) and len(live) > 2:
            b = int(rng.choice(live))
            old = [int(p) for p in rig.pages[b] if p >= 0]
            mask = np.zeros(rig.B, np.int32)
            mask[b] = 1
            assert rig.release_and_compare(mask) == O.OK
            released[b] = (t, old)
            events += 1
        for b, (t_rel, old) in list(released.items()):
            if t - t_rel == 3:
                k = int(rng.integers(13, len(old)))
                pages = [int(p) for p in rng.permutation(old)[:k]]
                length = 16 * k - int(rng.integers(1, 16))
                rig.set_pages(b, pages)
                assert rig.admit_and_compare(b, 0, length) == O.OK
                assert int(rig.ctx[b]) == length
                del released[b]
                events += 1
        out, o = rig.step_and_compare(H.MODE_EMA)
        assert out["status"] == 0
        _lossless(rig, out)
        assert rig.append_and_compare(new_pages=fresh) == O.OK
    assert events == 6
    assert sum(int(o["n_evict"]) for _, o in rig.history) > 0
    rig.close()
