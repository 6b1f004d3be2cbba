"""Shared test rig: one layer on the GPU through the C ABI, the oracle beside it.

The GPU side runs echo_layer_step (or the individual calls); the oracle runs the
same step on the same seeded inputs, fed the GPU's scores so that every later
decision (prefetch, top-k, eviction, allocation) can be compared bit for bit.
The GPU scores themselves are compared with the oracle's own fp64 scores within
the score tolerance.
"""
from __future__ import annotations

import numpy as np
import torch

from kv_cache_offload_fp8_amd import abi
from kv_cache_offload_fp8_amd import runtime as R
from oracle import oracle as O
from synth import make_inputs
from synth.gen import gen_append, gen_prefill_qw

MODE_EMA, MODE_NEG_INF, MODE_POS_INF = abi.ECHO_THETA_EMA, abi.ECHO_THETA_NEG_INF, \
    abi.ECHO_THETA_POS_INF
assert (MODE_EMA, MODE_NEG_INF, MODE_POS_INF) == (O.MODE_EMA, O.MODE_NEG_INF, O.MODE_POS_INF)

# Score tolerance: |gpu - oracle| <= 2e-3 |oracle|.  Shapes with at most SMALL_HEADS
# heads also get a cancellation allowance proportional to the magnitude of the summed
# terms, sum_j |w_j| sum_d |q_jd k_d|: with so few heads a score can be one head's
# near-zero dot product, and the indexer's fp8 MFMA adds neighbouring products in a
# window about 2^-15 below the largest of them (448 - 448 + 2^-6 returns 0 on gfx950),
# so its error there is bounded by a small multiple of 2^-15 times that magnitude;
# 2^-14 leaves a factor of two (measured worst case 2^-15.8 at 4 heads x 32).  With
# more heads every score is a weighted sum of many ReLU terms and the plain relative
# bound is asserted.
SCORE_RTOL = 2e-3
SCORE_ATOL_REL = 2.0 ** -14
SMALL_HEADS = 4

# Largest relative score error at the shapes held to the plain relative bound, and
# top-k set differences seen so far (printed at the end of a test run).
STATS = dict(max_rel=0.0, set_diffs=0, set_checked=0)


def _magnitude(q_codes, w, krows) -> np.ndarray:
    qf = np.abs(torch.from_numpy(q_codes.view(np.int16)).view(torch.bfloat16).float()
                .numpy().astype(np.float64))
    kf = np.abs(torch.from_numpy(krows).view(torch.float8_e4m3fn).float().numpy()
                .astype(np.float64))
    return (kf @ qf.T) @ np.abs(w.astype(np.float64))


def score_allowance(q_codes: np.ndarray, w: np.ndarray, krows: np.ndarray) -> np.ndarray:
    """Per-token cancellation allowance: SCORE_ATOL_REL times the magnitude of the
    summed terms for shapes with at most SMALL_HEADS heads, zero otherwise."""
    if q_codes.shape[0] > SMALL_HEADS:
        return np.zeros(krows.shape[0])
    return SCORE_ATOL_REL * _magnitude(q_codes, w, krows)


def score_tolerance(q_codes: np.ndarray, w: np.ndarray, krows: np.ndarray,
                    ref: np.ndarray) -> np.ndarray:
    """Per-token allowed |gpu - oracle|: 2e-3 relative, plus the cancellation allowance
    at small head counts."""
    return SCORE_RTOL * np.abs(ref.astype(np.float64)) + score_allowance(q_codes, w, krows)


def assert_scores_close(gpu: np.ndarray, q_codes, w, krows, ctx_note="", with_allowance=False):
    """GPU scores against the oracle's own fp64 scores.  Returns the oracle's scores, or
    (scores, allowance) with ``with_allowance``."""
    ref = O.scores(q_codes, w, krows)
    allow = score_allowance(q_codes, w, krows)
    tol = SCORE_RTOL * np.abs(ref.astype(np.float64)) + allow
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, (f"{ctx_note}: {bad.size} scores out of tolerance, first at {bad[:5]}: "
                           f"gpu={gpu[bad[:5]]} ref={ref[bad[:5]]}")
    nz = ref != 0
    if nz.any() and q_codes.shape[0] > SMALL_HEADS:
        STATS["max_rel"] = max(STATS["max_rel"],
                               float((err[nz] / np.abs(ref[nz].astype(np.float64))).max()))
    return (ref, allow) if with_allowance else ref


def assert_topk_set_clause(gpu_sel: np.ndarray, ref: np.ndarray, allow: np.ndarray, k: int,
                           ctx_note="") -> int:
    """The GPU's selected set against the oracle's top-k of its own fp64 scores: they may
    differ only on tokens whose oracle score lies within the score tolerance of the
    oracle's k-th score (2e-3 of it, plus the cancellation allowances of the token and of
    the k-th token at small head counts).  Returns the number of tokens that differ."""
    osel, okth = O.topk(ref, k)
    assert gpu_sel.size == osel.size, (ctx_note, "selected count", gpu_sel.size, osel.size)
    diff = np.setxor1d(gpu_sel.astype(np.int64), osel.astype(np.int64))
    STATS["set_checked"] += 1
    if diff.size:
        kth_tok = int(osel[np.argmin(ref[osel])]) if osel.size else 0
        lim = SCORE_RTOL * abs(okth) + allow[diff] + allow[kth_tok]
        far = np.abs(ref[diff].astype(np.float64) - okth) > lim
        assert not far.any(), (f"{ctx_note}: top-k sets differ on tokens {diff[far][:5]} whose "
                               f"oracle scores {ref[diff[far][:5]]} are not within the tolerance "
                               f"of the k-th score {okth}")
        STATS["set_diffs"] += int(diff.size)
    return int(diff.size)


def tile_kidx(rows: np.ndarray) -> np.ndarray:
    """Row-major indexer K [n, D] (n a multiple of 16) in the tiled layout of
    include/echo.h: byte d of host id h at 16*D*(h/16) + 8*D*((d%32)/16) +
    256*(d/32) + 16*(h%16) + d%16."""
    n, D = rows.shape
    h = np.arange(n)[:, None]
    d = np.arange(D)[None, :]
    off = 16 * D * (h // 16) + 8 * D * ((d % 32) // 16) + 256 * (d // 32) + 16 * (h % 16) + d % 16
    out = np.empty(n * D, np.uint8)
    out[off.ravel()] = rows.ravel()
    return out.reshape(n, D)


def scatter_pages(base, ctx, room, n_host, seed, stride_extra=0):
    """A page table for requests laid out at host_base (each owning ceil((ctx + room) / 16)
    pages): every page of the pool moved to a random other page.  Returns (pages
    [B, stride] (-1 past each request's pages), perm: old page -> new page)."""
    npool = n_host // 16
    perm = np.random.default_rng(seed).permutation(npool).astype(np.int64)
    span = (np.asarray(ctx, np.int64) + room + 15) // 16
    stride = int(span.max() if span.size else 1) + stride_extra
    pages = np.full((len(ctx), max(1, stride)), -1, np.int32)
    for b in range(len(ctx)):
        first = int(base[b]) // 16
        pages[b, : span[b]] = perm[first: first + span[b]]
    return pages, perm


class Rig:
    def __init__(self, wl, steps, device="cuda", ctx=None, n_gpu=None, n_host=None, seed=0,
                 keep_pool=True, max_ctx=None, layer=0, cap_div=None, top_k=None, room=0,
                 paged=False, page_seed=7, stride_extra=0):
        """paged: the requests' pages scattered over the host pool in random order, with
        a page table on both sides (the oracle's R14); stride_extra: spare page-table
        entries per request."""
        if n_gpu is not None or n_host is not None or cap_div is not None or top_k is not None:
            wl = wl.scaled(n_gpu=n_gpu or wl.n_gpu, n_host=n_host or wl.n_host,
                           cap_div=cap_div or wl.cap_div, top_k=top_k or wl.top_k)
        self.wl = wl
        self.separate = False  # True: gpu_step makes the five separate calls
        self.inp = make_inputs(wl, layer=layer, device="cpu", seed=seed, steps=steps, ctx=ctx,
                               room=room)
        self.layer_id = layer
        self.seed = seed
        self.ctx = self.inp.ctx
        self.base = self.inp.host_base
        self.B = int(self.ctx.size)
        self.steps = steps
        mc = int(max_ctx or max(1, int(self.ctx.max()) if self.B else 1))
        self.dims = R.make_dims(wl.heads, wl.head_dim, wl.top_k, wl.n_host, wl.n_gpu,
                                max(1, self.B), mc, wl.latent, wl.alpha, wl.cap_div, steps)
        self.host = R.HostPool(wl.n_host, wl.latent)
        self.pages = None
        kid = self.inp.np_kidx()
        lat = self.inp.np_latents()
        if paged:
            # every host page moved to its image under a random permutation of the pool
            self.pages, perm = scatter_pages(self.base, self.ctx, room, wl.n_host, page_seed,
                                             stride_extra)
            self.page_perm = perm
            src = (np.arange(wl.n_host) // 16).astype(np.int64)
            dst = 16 * perm[src] + np.arange(wl.n_host) % 16
            kid2 = np.empty_like(kid)
            kid2[dst] = kid
            lat2 = np.empty_like(lat)
            lat2[dst] = lat
            kid, lat = kid2, lat2
        self.host.np[:] = lat
        self.kidx_rows = torch.from_numpy(kid).to(device)  # row-major, as the oracle reads it
        self.kidx = R.pack_kidx(self.dims, self.kidx_rows)
        self.layer = R.Layer(self.dims, self.kidx, self.host, self.B, device)
        if self.B:
            self.layer.q.copy_(self.inp.q.to(device))
            self.layer.w.copy_(self.inp.w.to(device))
        self.layer.init()
        self.batch = R.Batch(self.base, self.ctx, device, pages=self.pages)
        self.ws = R.Workspace(self.dims, device)
        self.ws.reset()
        self.orc = O.OracleLayer(wl.heads, wl.head_dim, wl.top_k, wl.latent, wl.n_host, wl.n_gpu,
                                 max(1, self.B), wl.cap_div, wl.alpha, keep_pool=keep_pool)
        self.np_kidx = kid
        # the oracle's own copy of the host pool: bytes the GPU writes there are
        # compared with it, not read back by the oracle
        self.orc_host = self.host.np.copy()
        self.np_host = self.orc_host
        self.np_w = self.inp.np_w()
        self.t = 0
        self.history = []
        # the running totals echo_layer_step keeps (echo_layer_t.stats), as the
        # oracle's outputs add up; compared while every step so far ended cleanly
        self.exp_stats = np.zeros(abi.ECHO_STAT_WORDS, np.int64)
        self.stats_valid = True

    def host_ids(self, b, toks):
        """Host ids of request b's tokens `toks` (through the page table if any)."""
        toks = np.asarray(toks, np.int64)
        if self.pages is None:
            return int(self.base[b]) + toks
        return 16 * self.pages[b, toks // 16].astype(np.int64) + toks % 16

    def set_pages(self, b, row):
        """Write page-table row b on both sides (the caller's page allocation)."""
        row = np.asarray(row, np.int32)
        self.pages[b, :] = -1
        self.pages[b, : row.size] = row
        torch.cuda.current_stream().synchronize()
        self.batch.pages[b] = torch.as_tensor(self.pages[b], device=self.batch.pages.device)
        torch.cuda.current_stream().synchronize()

    # ------------------------------------------------------------ GPU calls
    def gpu_step(self, mode):
        if self.separate:
            self.gpu_step_separate(mode)
            return
        R.check(abi.echo_layer_step(self.dims, self.layer.struct, self.batch.struct, self.ws.ws,
                                    mode, R.stream_handle()), "echo_layer_step")

    def gpu_step_separate(self, mode):
        """The same step as the five calls echo_layer_step fuses: indexer + prefetch,
        top-k (with the EMA update in mode EMA), protect/evict/allocate, recall, and
        the step-counter advance."""
        s = R.stream_handle()
        L, Bt, W = self.layer.struct, self.batch.struct, self.ws.ws
        R.check(abi.echo_indexer_prefetch(self.dims, L, Bt, W, mode, s), "echo_indexer_prefetch")
        theta = self.layer.theta.data_ptr() if mode == MODE_EMA else None
        R.check(abi.echo_topk(self.dims, self.ws.scores.data_ptr(), self.dims.max_ctx, Bt, W,
                              theta, s), "echo_topk")
        R.check(abi.echo_cache_alloc_evict(self.dims, L, Bt, W, s), "echo_cache_alloc_evict")
        R.check(abi.echo_recall(self.dims, L, W, s), "echo_recall")
        R.check(abi.echo_step_advance(L, W, s), "echo_step_advance")

    def gpu_scores(self) -> np.ndarray:
        torch.cuda.current_stream().synchronize()
        return self.ws.scores[: self.B].cpu().numpy()

    # --------------------------------------------------------- comparison
    def step_and_compare(self, mode, check_scores=True, check_pool=True, expect_status=0):
        t = self.t
        q_t = self.inp.np_q(t % self.steps)
        self.gpu_step(mode)
        out = self.ws.read(self.B)
        sc = self.gpu_scores()
        st = self.layer.state()
        if check_scores:
            for b in range(self.B):
                n = int(self.ctx[b])
                if n:
                    note = f"step {t} request {b}"
                    rows = self.np_kidx[self.host_ids(b, np.arange(n))]
                    ref, allow = assert_scores_close(sc[b, :n], q_t[b], self.np_w[b], rows, note,
                                                     with_allowance=True)
                    if out["status"] == 0:
                        assert_topk_set_clause(out["sel_tok"][b, :int(out["n_sel"][b])], ref,
                                               allow, self.wl.top_k, note)
        o = self.orc.step(self.base, self.ctx, q_t, self.np_w, self.np_kidx, self.np_host,
                          mode=mode, ext_scores=sc, pages=self.pages)
        self.compare(out, st, o, t, check_pool)
        assert out["status"] == expect_status, (f"step {t}: status {out['status']}",
                                                abi.echo_status_string(int(out["status"])))
        if o["status"] != O.OK:
            self.stats_valid = False
        if not self.separate and self.stats_valid:
            self.compare_stats(o, t)
        self.history.append((out, o))
        if o["status"] == O.OK:
            self.t += 1
        return out, o

    def compare_stats(self, o, t):
        e = self.exp_stats
        e[abi.ECHO_STAT_STEPS] += 1
        e[abi.ECHO_STAT_SELECTED] += int(o["n_sel"].sum())
        e[abi.ECHO_STAT_MISSED] += int(o["n_miss"].sum())
        e[abi.ECHO_STAT_PREFETCHED] += int(o["n_pf"].sum())
        e[abi.ECHO_STAT_CANDIDATES] += int(o["n_cand"].sum())
        e[abi.ECHO_STAT_EVICTED] += int(o["n_evict"])
        for b in range(self.B):
            pf = o["pf_tok"][b, : int(o["n_pf"][b])]
            sel = o["sel_tok"][b, : int(o["n_sel"][b])]
            e[abi.ECHO_STAT_PF_SELECTED] += int(np.intersect1d(pf, sel).size)
        got = self.layer.stats.cpu().numpy()
        assert np.array_equal(got, e), (f"step {t}", "running totals", got, e)

    def compare(self, out, st, o, t, check_pool=True):
        tag = f"step {t}"
        assert out["status"] == o["status"], (tag, out["status"], o["status"])
        B, k = self.B, self.wl.top_k
        for b in range(B):
            n = int(o["n_sel"][b])
            assert out["n_sel"][b] == n, (tag, "n_sel", b, out["n_sel"][b], n)
            assert np.array_equal(out["sel_tok"][b, :n], o["sel_tok"][b, :n]), (tag, "sel_tok", b)
            assert np.array_equal(np.float32(out["kth"][b]).view(np.uint32),
                                  np.float32(o["kth"][b]).view(np.uint32)) or \
                (np.isnan(out["kth"][b]) and np.isnan(o["kth"][b])), (tag, "kth", b)
            npf = int(o["n_pf"][b])
            assert out["n_pf"][b] == npf, (tag, "n_pf", b, out["n_pf"][b], npf)
            assert out["n_cand"][b] == o["n_cand"][b], (tag, "n_cand", b, "gpu", out["n_cand"],
                                                         "oracle", o["n_cand"])
            assert np.array_equal(out["pf_tok"][b, :npf], o["pf_tok"][b, :npf]), (tag, "pf_tok")
            assert np.array_equal(out["pf_slot"][b, :npf], o["pf_slot"][b, :npf]), (tag, "pf_slot")
            nm = int(o["n_miss"][b])
            assert out["n_miss"][b] == nm, (tag, "n_miss", b, out["n_miss"][b], nm)
            assert np.array_equal(out["miss_tok"][b, :nm], o["miss_tok"][b, :nm]), (tag, "miss")
            if o["status"] == O.OK:
                assert np.array_equal(out["sel_slot"][b, :n], o["sel_slot"][b, :n]), \
                    (tag, "sel_slot", b)
        assert np.array_equal(st["theta"][:B], self.orc.theta[:B]), (tag, "theta")
        assert np.array_equal(st["h2g"], self.orc.h2g), (tag, "h2g")
        assert np.array_equal(st["g2h"], self.orc.g2h), (tag, "g2h")
        assert np.array_equal(st["prio"], self.orc.prio), (tag, "prio")
        assert np.array_equal(st["free"], self.orc.free), (tag, "free")
        assert st["t"] == self.orc.t, (tag, "t", st["t"], self.orc.t)
        if o["status"] == O.OK:
            assert out["counters"][abi.ECHO_CNT_EVICT] == o["n_evict"], (tag, "n_evict")
            assert out["counters"][abi.ECHO_CNT_MISS] == int(o["n_miss"].sum())
            # the index buffer holds the ascending free list
            nfree = st["nfree"]
            assert nfree == int(self.orc.free.sum()), (tag, "nfree")
            assert np.array_equal(st["idxbuf"][:nfree], np.nonzero(self.orc.free)[0]), \
                (tag, "idxbuf")
        if check_pool and self.orc.pool is not None:
            torch.cuda.current_stream().synchronize()
            gp = self.layer.gpu_kv.cpu().numpy().view(np.uint16)
            assert np.array_equal(gp, self.orc.pool), (tag, "pool bytes")

    def jump_to_step(self, t):
        """Set the layer's step counter to t on both sides (as if t - self.t steps had
        passed without touching this layer), so that slots last used before
        t - 4096 fall into the eviction histogram's clamped oldest bin."""
        torch.cuda.current_stream().synchronize()
        self.layer.ctl[abi.ECHO_CTL_STEP] = int(t)
        # the totals carry on: the jump skips no step of this layer's own
        torch.cuda.current_stream().synchronize()
        self.orc.t = int(t)
        self.t = int(t)

    # ------------------------------------------------------------ decode append
    def append_and_compare(self, advance=True, expect_status=0, new_pages=None):
        """echo_append of this step's new tokens against the oracle's append: device
        context lengths, the whole tiled indexer K (against the oracle's rows tiled
        here, independently of the library) and the host pool bytes.  With a page
        table, new_pages (an iterator of free host pages) gives every request whose
        next token opens a page that page first."""
        if self.pages is not None and new_pages is not None:
            for b in range(self.B):
                c = int(self.ctx[b])
                if c and c % 16 == 0 and c // 16 < self.pages.shape[1]:
                    row = self.pages[b].copy()
                    row[c // 16] = next(new_pages)
                    self.set_pages(b, row[row >= 0])
        k_new, lat_new = gen_append(self.wl, self.layer_id, self.B, self.t, self.seed)
        kd = torch.as_tensor(k_new, device="cuda")
        ld = torch.as_tensor(lat_new, device="cuda")
        R.check(abi.echo_append(self.dims, self.layer.struct, self.batch.struct, kd.data_ptr(),
                                ld.data_ptr(), self.ws.ws, int(advance), R.stream_handle()),
                "echo_append")
        torch.cuda.current_stream().synchronize()
        rc = O.append(self.base, self.ctx, self.orc.h2g, k_new, lat_new.view(np.uint16),
                      self.np_kidx, self.orc_host, self.dims.max_ctx, advance, pages=self.pages)
        st = int(self.ws.status.item())
        assert st == rc == expect_status, ("append status", st, rc, expect_status)
        assert np.array_equal(self.batch.ctx.cpu().numpy(), self.ctx), "ctx_len"
        assert np.array_equal(self.layer.kidx.cpu().numpy(), tile_kidx(self.np_kidx)), \
            "tiled indexer K"
        assert np.array_equal(self.host.np, self.orc_host), "host pool bytes"
        return rc

    # ------------------------------------------------------------ request lifecycle
    def release_and_compare(self, mask, commit=True, expect_status=0):
        """echo_release of the masked requests against the oracle's release: status,
        batch rows, maps, priorities, free flags, thresholds and the free list."""
        mask = np.asarray(mask, np.int32)
        m = torch.as_tensor(mask, device="cuda")
        R.check(abi.echo_release(self.dims, self.layer.struct, self.batch.struct, m.data_ptr(),
                                 int(commit), self.ws.ws, R.stream_handle()), "echo_release")
        rc = O.release(self.orc, self.base, self.ctx, mask, self.dims.max_ctx, commit,
                       pages=self.pages)
        self._compare_lifecycle(rc, expect_status, "release")
        return rc

    def admit_and_compare(self, b, base, length, commit=True, expect_status=0):
        """echo_admit of row b against the oracle's admission (a host-side rejection
        must be the oracle's EINVAL, with nothing enqueued)."""
        ret = abi.echo_admit(self.dims, self.layer.struct, self.batch.struct, int(b), int(base),
                             int(length), int(commit), self.ws.ws, R.stream_handle())
        rc = O.admit(self.orc, self.base, self.ctx, b, base, length, self.dims.max_ctx, commit,
                     pages=self.pages)
        if ret != abi.ECHO_OK:
            assert ret == rc == expect_status == O.EINVAL, ("admit", ret, rc, expect_status)
            return rc
        self._compare_lifecycle(rc, expect_status, "admit")
        return rc

    def _compare_lifecycle(self, rc, expect_status, tag):
        torch.cuda.current_stream().synchronize()
        st = int(self.ws.status.item())
        assert st == rc == expect_status, (tag, "status", st, rc, expect_status)
        assert np.array_equal(self.batch.ctx.cpu().numpy(), self.ctx), (tag, "ctx_len")
        if self.pages is None:
            assert np.array_equal(self.batch.host_base.cpu().numpy(), self.base), \
                (tag, "host_base")
        g = self.layer.state()
        for name in ("h2g", "g2h", "prio", "free"):
            assert np.array_equal(g[name], getattr(self.orc, name)), (tag, name)
        assert np.array_equal(g["theta"][: self.B], self.orc.theta[: self.B]), (tag, "theta")
        nfree = int(self.orc.free.sum())
        assert g["nfree"] == nfree, (tag, "nfree", g["nfree"], nfree)
        assert np.array_equal(g["idxbuf"][:nfree], np.nonzero(self.orc.free)[0]), (tag, "idxbuf")

    def gathered(self):
        """GPU-pool rows of every request's selected tokens, in selection order (what the
        sparse attention of the step would read)."""
        torch.cuda.current_stream().synchronize()
        n_sel = self.ws.n_sel[: self.B].cpu().numpy()
        slots = self.ws.sel_slot[: self.B].cpu().numpy()
        rows = []
        for b in range(self.B):
            g = torch.as_tensor(slots[b, : int(n_sel[b])].astype(np.int64), device="cuda")
            rows.append(self.layer.gpu_kv[g].cpu().numpy().view(np.uint16))
        return rows

    def hit_rates(self):
        hr = []
        for out, _ in self.history:
            sel = int(out["n_sel"].sum())
            hr.append(1.0 - int(out["n_miss"].sum()) / sel if sel else 1.0)
        return hr

    def close(self):
        torch.cuda.synchronize()
        self.host.close()


class PrefillRig:
    """One request's history of N tokens (host ids 0 .. N-1) on a fresh layer, chunks of C
    prefill queries run through echo_prefill_score / _copy / _select and compared with
    the oracle's prefill chunk, which is fed the GPU's scores."""

    def __init__(self, wl, N, C, chunks, n_gpu=None, n_host=None, top_k=None, seed=0,
                 layer=0, device="cuda", use_pred=True):
        wl = wl.scaled(n_gpu=n_gpu or wl.n_gpu, n_host=n_host or wl.n_host,
                       top_k=top_k or wl.top_k)
        self.wl, self.N, self.C, self.chunks, self.use_pred = wl, N, C, chunks, use_pred
        self.inp = make_inputs(wl, layer=layer, device="cpu", seed=seed, steps=1, ctx=[N])
        self.hb = int(self.inp.host_base[0])
        self.dims = R.make_dims(wl.heads, wl.head_dim, wl.top_k, wl.n_host, wl.n_gpu, 1, N,
                                wl.latent, wl.alpha, wl.cap_div, 1)
        self.host = R.HostPool(wl.n_host, wl.latent)
        self.host.np[:] = self.inp.np_latents()
        self.kidx = R.pack_kidx(self.dims, self.inp.kidx.to(device))
        self.layer = R.Layer(self.dims, self.kidx, self.host, 1, device)
        self.layer.init()
        self.pws = R.PrefillWorkspace(self.dims, C, device)
        q, w = gen_prefill_qw(wl, layer, C, chunks, "cpu", seed)
        self.q_np = q.view(torch.int16).numpy().view(np.uint16)
        self.w_np = w.numpy()
        self.q_dev, self.w_dev = q.to(device), w.to(device)
        self.np_kidx = self.inp.np_kidx()
        self.orc_host = self.host.np.copy()
        self.orc = O.OracleLayer(wl.heads, wl.head_dim, wl.top_k, wl.latent, wl.n_host, wl.n_gpu,
                                 1)
        self.pred = None  # the oracle's view of the prediction the GPU used
        self.c = 0

    def chunk(self, c):
        pred = self.pws.kth.data_ptr() if (self.use_pred and c > 0) else None
        return abi.echo_prefill_chunk_t(self.C, self.hb, self.N, self.q_dev[c].data_ptr(),
                                        self.w_dev[c].data_ptr(), pred)

    def gpu_chunk(self, c):
        st = R.stream_handle()
        ch = self.chunk(c)
        R.check(abi.echo_prefill_score(self.dims, self.layer.struct, ch, self.pws.ws, st),
                "echo_prefill_score")
        R.check(abi.echo_prefill_early(self.dims, self.layer.struct, ch, self.pws.ws, st),
                "echo_prefill_early")
        R.check(abi.echo_prefill_copy(self.dims, self.layer.struct, self.pws.ws, 0, st),
                "echo_prefill_copy")
        R.check(abi.echo_prefill_select(self.dims, self.layer.struct, ch, self.pws.ws, st),
                "echo_prefill_select")
        R.check(abi.echo_prefill_copy(self.dims, self.layer.struct, self.pws.ws, 1, st),
                "echo_prefill_copy")

    def step_and_compare(self, check_rows=None, expect_status=0, fail_stage=None):
        """One chunk on both sides.  check_rows: the query rows whose scores are checked
        against the oracle's own (None: all).  fail_stage: "early" or "late" when a
        capacity error is expected in that stage."""
        c = self.c
        C, N, k = self.C, self.N, self.wl.top_k
        pred_used = self.pws.kth[:C].cpu().numpy().copy() if (self.use_pred and c > 0) \
            else None
        self.gpu_chunk(c)
        torch.cuda.current_stream().synchronize()
        P = self.pws
        status = int(P.status.item())
        sc = P.scores(C, N).cpu().numpy()
        rows = range(C) if check_rows is None else check_rows
        refs = {}
        for i in rows:
            refs[i] = assert_scores_close(sc[i], self.q_np[c, i], self.w_np[c, i],
                                          self.np_kidx[self.hb:self.hb + N],
                                          f"chunk {c} query {i}", with_allowance=True)
        o = O.prefill_chunk(self.orc, self.hb, N, self.q_np[c], self.w_np[c], self.np_kidx,
                            pred=pred_used, host_kv=self.orc_host, ext_scores=sc)
        tag = f"chunk {c}"
        assert status == o["status"] == expect_status, (tag, "status", status, o["status"])
        cnt = P.counts.cpu().numpy()
        assert np.array_equal(P.beta[:C].cpu().numpy(), o["beta"]), (tag, "beta")
        assert np.array_equal(P.n_qcand[:C].cpu().numpy(), o["n_qcand"]), (tag, "n_qcand")
        assert cnt[abi.ECHO_PF_CNT_CAND] == o["cand"].size, (tag, "n_cand")
        assert np.array_equal(P.cand[: o["cand"].size].cpu().numpy(), o["cand"]), (tag, "cand")
        if status == 0 or fail_stage == "late":
            n_pf = o["pf_h"].size
            assert cnt[abi.ECHO_PF_CNT_EARLY] == n_pf, (tag, "n_early")
            assert np.array_equal(P.pf_h[:n_pf].cpu().numpy(), o["pf_h"]), (tag, "pf_h")
            assert np.array_equal(P.pf_g[:n_pf].cpu().numpy(), o["pf_g"]), (tag, "pf_g")
        if status == 0:
            assert np.array_equal(P.n_sel[:C].cpu().numpy(), o["n_sel"]), (tag, "n_sel")
            gsel = P.sel[:C].cpu().numpy()
            for i in range(C):
                n = int(o["n_sel"][i])
                assert np.array_equal(gsel[i, :n], o["sel"][i, :n]), (tag, "sel", i)
            for i, (ref, allow) in refs.items():
                assert_topk_set_clause(gsel[i, :int(o["n_sel"][i])], ref, allow, k,
                                       f"{tag} query {i}")
            assert np.array_equal(P.kth[:C].cpu().numpy().view(np.uint32),
                                  o["kth"].view(np.uint32)), (tag, "kth")
            assert cnt[abi.ECHO_PF_CNT_UNION] == o["uni"].size, (tag, "n_union")
            assert np.array_equal(P.uni[: o["uni"].size].cpu().numpy(), o["uni"]), (tag, "uni")
            nm = o["miss_h"].size
            assert cnt[abi.ECHO_PF_CNT_LATE] == nm, (tag, "n_late")
            assert np.array_equal(P.miss_h[:nm].cpu().numpy(), o["miss_h"]), (tag, "miss_h")
            assert np.array_equal(P.miss_g[:nm].cpu().numpy(), o["miss_g"]), (tag, "miss_g")
        st = self.layer.state()
        for name in ("h2g", "g2h", "prio", "free"):
            assert np.array_equal(st[name], getattr(self.orc, name)), (tag, name)
        assert st["t"] == self.orc.t, (tag, "t", st["t"], self.orc.t)
        if status == 0:
            nfree = int(self.orc.free.sum())
            assert st["nfree"] == nfree, (tag, "nfree")
            assert np.array_equal(st["idxbuf"][:nfree], np.nonzero(self.orc.free)[0]), \
                (tag, "idxbuf")
        gp = self.layer.gpu_kv.cpu().numpy().view(np.uint16)
        assert np.array_equal(gp, self.orc.pool), (tag, "pool bytes")
        if status == 0:
            self.c += 1
        return o, dict(status=status, counts=cnt)

    def close(self):
        torch.cuda.synchronize()
        self.host.close()
