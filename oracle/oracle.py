"""ctypes wrapper around the CPU oracle (``echo_oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark use this module; the product path never imports it.  It
shares no code with the GPU library.  Every function cites, in the C source, the
passage of the ECHO review page it follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "echo_oracle.c")
LIB = os.path.join(HERE, "libecho_oracle.so")

MODE_EMA, MODE_NEG_INF, MODE_POS_INF = 0, 1, 2
OK, EINVAL, ECAPACITY, EDEVARG = 0, -1, -4, -6


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C99 + OpenMP, no FMA contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        cmd = ["gcc", "-std=gnu99", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
               "-shared", SRC, "-o", LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def lib() -> C.CDLL:
    """Load the oracle.  ECHO_ORACLE_LIB may name another build of the same source (the
    planted-mistake tests use it to check that the pins notice a wrong oracle)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ECHO_ORACLE_LIB") or build()
        _lib = C.CDLL(path)
        _lib.orc_e4m3_value.restype = C.c_double
        _lib.orc_e4m3_value.argtypes = [C.c_uint8]
        _lib.orc_bf16_value.restype = C.c_double
        _lib.orc_bf16_value.argtypes = [C.c_uint16]
        _lib.orc_set_threads.restype = C.c_int
        _lib.orc_set_threads.argtypes = [C.c_int]
        _lib.orc_meta_bytes.restype = C.c_int64
        _lib.orc_meta_bytes.argtypes = [C.c_int64, C.c_int64]
        _lib.orc_scores.restype = None
        _lib.orc_scores.argtypes = [C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_int64, C.c_void_p]
        _lib.orc_topk.restype = C.c_int
        _lib.orc_topk.argtypes = [C.c_void_p, C.c_int64, C.c_int, C.c_void_p, C.c_void_p]
        _lib.orc_ema_update.restype = C.c_float
        _lib.orc_ema_update.argtypes = [C.c_float, C.c_float, C.c_float]
        _lib.orc_append.restype = C.c_int
        _lib.orc_append.argtypes = [C.c_int, C.c_int, C.c_int, C.c_int64, C.c_int32,
                                    C.POINTER(TokMap), C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_void_p, C.c_void_p, C.c_void_p, C.c_int]
        _lib.orc_gather.restype = None
        _lib.orc_release.restype = C.c_int
        _lib.orc_release.argtypes = [C.c_int, C.c_int64, C.c_int32, C.POINTER(TokMap)] + \
            [C.c_void_p] * 7 + [C.c_int]
        _lib.orc_admit.restype = C.c_int
        _lib.orc_admit.argtypes = [C.c_int, C.c_int64, C.c_int32, C.POINTER(TokMap)] + \
            [C.c_void_p] * 3 + [C.c_int, C.c_int32, C.c_int32, C.c_int]
        _lib.orc_f16_bits.restype = C.c_uint16
        _lib.orc_f16_bits.argtypes = [C.c_float]
        _lib.orc_f16_bucket.restype = C.c_int
        _lib.orc_f16_bucket.argtypes = [C.c_uint16]
        _lib.orc_prefill_chunk.restype = C.c_int
        _lib.orc_prefill_chunk.argtypes = [C.POINTER(Cfg), C.POINTER(State), C.c_int, C.c_int32,
                                           C.c_int64] + [C.c_void_p] * 6 + \
            [C.POINTER(PrefillOut)]
        _lib.orc_gather.argtypes = [C.c_int, C.c_int, C.c_int, C.POINTER(TokMap), C.c_void_p,
                                    C.c_void_p, C.c_void_p, C.c_void_p]
        _lib.orc_layer_step.restype = C.c_int
        _lib.orc_layer_step.argtypes = [C.POINTER(Cfg), C.POINTER(State), C.c_int,
                                        C.POINTER(TokMap), C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_void_p, C.c_void_p, C.c_int, C.c_void_p,
                                        C.c_int64, C.POINTER(Out)]
    return _lib


class TokMap(C.Structure):
    """Where each request's tokens live: host_base (contiguous ranges) or a page table
    [B][page_stride] of 16-id host pages (R14 in the C source)."""
    _fields_ = [("host_base", C.c_void_p), ("pages", C.c_void_p), ("page_stride", C.c_int32)]


def _tokmap(host_base, pages):
    """(TokMap, arrays it points into).  pages: int32 [B, page_stride] or None."""
    if pages is not None:
        pages = np.ascontiguousarray(pages, np.int32)
        assert pages.ndim == 2
        return TokMap(None, pages.ctypes.data, pages.shape[1]), (pages,)
    assert host_base.dtype == np.int32 and host_base.flags["C_CONTIGUOUS"]
    return TokMap(host_base.ctypes.data, None, 0), (host_base,)


def page_host_ids(pages, ctx):
    """Host ids of each request's tokens under a page table: list of int64 arrays."""
    out = []
    for b, n in enumerate(np.asarray(ctx)):
        s = np.arange(int(n), dtype=np.int64)
        out.append(16 * pages[b, s // 16].astype(np.int64) + s % 16)
    return out


class Cfg(C.Structure):
    _fields_ = [("H", C.c_int32), ("D", C.c_int32), ("k", C.c_int32), ("latent", C.c_int32),
                ("n_host", C.c_int64), ("n_gpu", C.c_int32), ("cap_div", C.c_int32),
                ("alpha", C.c_float)]


class State(C.Structure):
    _fields_ = [("h2g", C.c_void_p), ("g2h", C.c_void_p), ("prio", C.c_void_p),
                ("freef", C.c_void_p), ("theta", C.c_void_p), ("t", C.c_int32),
                ("pool", C.c_void_p)]


class PrefillOut(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("scores", "sel", "n_sel", "kth", "beta", "n_qcand",
                                          "cand", "uni", "pf_h", "pf_g", "miss_h", "miss_g")] + \
        [(n, C.c_int32) for n in ("n_cand", "n_uni", "n_pf", "n_miss")]


class Out(C.Structure):
    _fields_ = [("scores", C.c_void_p), ("sel_tok", C.c_void_p), ("sel_slot", C.c_void_p),
                ("n_sel", C.c_void_p), ("kth", C.c_void_p), ("pf_tok", C.c_void_p),
                ("pf_slot", C.c_void_p), ("n_pf", C.c_void_p), ("n_cand", C.c_void_p),
                ("miss_tok", C.c_void_p), ("n_miss", C.c_void_p), ("evicted", C.c_void_p),
                ("n_evict", C.c_int32), ("n_free_start", C.c_int32), ("status", C.c_int32)]


def _p(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle buffers must be contiguous"
    return a.ctypes.data


def set_threads(n: int) -> int:
    """OpenMP threads of the oracle's scoring loop; returns the previous maximum."""
    return lib().orc_set_threads(int(n))


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(int(code))


def bf16_value(code: int) -> float:
    return lib().orc_bf16_value(int(code))


def meta_bytes(n_host: int, n_gpu: int) -> int:
    return lib().orc_meta_bytes(int(n_host), int(n_gpu))


def scores(q: np.ndarray, w: np.ndarray, krows: np.ndarray) -> np.ndarray:
    """q: uint16 bf16 codes [H, D]; w: float32 [H]; krows: uint8 e4m3 [ctx, D]."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    krows = np.ascontiguousarray(krows, dtype=np.uint8)
    H, D = q.shape
    assert krows.ndim == 2 and krows.shape[1] == D and w.shape == (H,)
    out = np.empty(krows.shape[0], np.float32)
    lib().orc_scores(H, D, _p(q), _p(w), _p(krows), krows.shape[0], _p(out))
    return out


def topk(sc: np.ndarray, k: int) -> tuple[np.ndarray, float]:
    sc = np.ascontiguousarray(sc, dtype=np.float32)
    sel = np.empty(max(1, min(k, sc.size)), np.int32)
    kth = np.zeros(1, np.float32)
    m = lib().orc_topk(_p(sc), sc.size, int(k), _p(sel), _p(kth))
    return sel[:m].copy(), float(kth[0])


def append(host_base, ctx, h2g, k_new, lat_new, kidx, host_kv, max_ctx: int,
           advance: bool = True, pages=None) -> int:
    """Decode append (orc_append): writes each request's new token into kidx (uint8
    [n_host, D]) and host_kv (uint16 [n_host, latent] or None) at its next host id
    (host_base + ctx, or through the page table ``pages``), then grows ctx (int32, in
    place) if ``advance``.  Returns OK or the error code."""
    host_base = np.ascontiguousarray(host_base if host_base is not None else [0], np.int32)
    assert ctx.dtype == np.int32 and ctx.flags["C_CONTIGUOUS"]
    h2g = np.ascontiguousarray(h2g, np.int32)
    k_new = np.ascontiguousarray(k_new, np.uint8)
    lat_new = np.ascontiguousarray(lat_new, np.uint16)
    B = int(ctx.size)
    D = kidx.shape[1]
    latent = lat_new.shape[1] if lat_new.ndim == 2 else 0
    assert k_new.shape == (B, D) and kidx.flags["C_CONTIGUOUS"]
    if host_kv is not None:
        assert host_kv.flags["C_CONTIGUOUS"] and host_kv.shape[1] == latent
    tm, _keep = _tokmap(host_base, pages)
    return lib().orc_append(B, D, latent, kidx.shape[0], int(max_ctx), C.byref(tm), _p(ctx),
                            _p(h2g), _p(k_new), _p(lat_new), _p(kidx),
                            _p(host_kv) if host_kv is not None else None, int(bool(advance)))


def gather(host_base, sel_tok, n_sel, host_kv, pages=None) -> np.ndarray:
    """Attention input without offloading (orc_gather): uint16 [B, k, latent], the host
    latents of each request's selected tokens in selection order, zero past n_sel."""
    host_base = np.ascontiguousarray(host_base if host_base is not None else [0], np.int32)
    sel_tok = np.ascontiguousarray(sel_tok, np.int32)
    n_sel = np.ascontiguousarray(n_sel, np.int32)
    host_kv = np.ascontiguousarray(host_kv, np.uint16)
    B, k = sel_tok.shape
    latent = host_kv.shape[1]
    out = np.empty((B, k, latent), np.uint16)
    tm, _keep = _tokmap(host_base, pages)
    lib().orc_gather(B, k, latent, C.byref(tm), _p(sel_tok), _p(n_sel), _p(host_kv), _p(out))
    return out


def release(layer, host_base, ctx, mask, max_ctx: int, commit: bool = True, pages=None) -> int:
    """Request cancellation (orc_release) on an OracleLayer's state: the masked
    requests' slots and map rows are given back, theta resets, and with ``commit`` ctx
    (int32, in place) becomes 0.  Returns OK or the error code."""
    host_base = np.ascontiguousarray(host_base if host_base is not None else [0], np.int32)
    assert ctx.dtype == np.int32 and ctx.flags["C_CONTIGUOUS"]
    mask = np.ascontiguousarray(mask, np.int32)
    B = int(ctx.size)
    assert (pages is not None or host_base.size == B) and mask.size == B and \
        layer.theta.size >= B
    tm, _keep = _tokmap(host_base, pages)
    return lib().orc_release(B, layer.cfg.n_host, int(max_ctx), C.byref(tm), _p(ctx),
                             _p(mask), _p(layer.h2g), _p(layer.g2h), _p(layer.prio),
                             _p(layer.free), _p(layer.theta), int(bool(commit)))


def admit(layer, host_base, ctx, b: int, base: int, length: int, max_ctx: int,
          commit: bool = True, pages=None) -> int:
    """Request admission (orc_admit) into batch row b: if the checks pass theta[b]
    resets and, with ``commit``, ctx[b] = length and (without a page table) host_base[b]
    = base (int32 arrays, in place).  With ``pages`` the caller has written row b of the
    page table.  Returns OK or the error code."""
    if host_base is None:
        host_base = np.zeros(1, np.int32)
    assert ctx.dtype == np.int32 and ctx.flags["C_CONTIGUOUS"]
    B = int(ctx.size)
    tm, _keep = _tokmap(host_base, pages)
    return lib().orc_admit(B, layer.cfg.n_host, int(max_ctx), C.byref(tm), _p(ctx),
                           _p(layer.h2g), _p(layer.theta), int(b), int(base), int(length),
                           int(bool(commit)))


def f16_bits(x: float) -> int:
    return lib().orc_f16_bits(float(x))


def f16_bucket(u: int) -> int:
    return lib().orc_f16_bucket(int(u))


def prefill_chunk(layer, hb: int, N: int, q, w, kidx, pred=None, host_kv=None,
                  ext_scores=None) -> dict:
    """One chunked-prefill step (orc_prefill_chunk) on an OracleLayer's state.  q: uint16
    [C, H, D]; w: float32 [C, H]; kidx: uint8 [n_host, D]; pred: float32 [C] or None;
    ext_scores: float32 [C, N] or None.  Returns the outputs (lists trimmed)."""
    cfg = layer.cfg
    q = np.ascontiguousarray(q, np.uint16)
    w = np.ascontiguousarray(w, np.float32)
    kidx = np.ascontiguousarray(kidx, np.uint8)
    Cq = q.shape[0]
    assert q.shape == (Cq, cfg.H, cfg.D) and w.shape == (Cq, cfg.H)
    assert kidx.shape == (cfg.n_host, cfg.D) and 0 <= hb and hb + N <= cfg.n_host
    k = cfg.k
    o = dict(scores=np.zeros((Cq, max(N, 1)), np.float32), sel=np.full((Cq, k), -1, np.int32),
             n_sel=np.zeros(Cq, np.int32), kth=np.zeros(Cq, np.float32),
             beta=np.zeros(Cq, np.int32), n_qcand=np.zeros(Cq, np.int32))
    for n in ("cand", "uni", "pf_h", "pf_g", "miss_h", "miss_g"):
        o[n] = np.full(max(N, 1), -1, np.int32)
    out = PrefillOut(*[_p(o[n]) for n in ("scores", "sel", "n_sel", "kth", "beta", "n_qcand",
                                           "cand", "uni", "pf_h", "pf_g", "miss_h", "miss_g")],
                     0, 0, 0, 0)
    if pred is not None:
        pred = np.ascontiguousarray(pred, np.float32)
        assert pred.shape == (Cq,)
    if ext_scores is not None:
        ext_scores = np.ascontiguousarray(ext_scores, np.float32)
        assert ext_scores.shape == (Cq, N)
    if host_kv is not None:
        host_kv = np.ascontiguousarray(host_kv, np.uint16)
    theta = np.ascontiguousarray(layer.theta)
    st = State(_p(layer.h2g), _p(layer.g2h), _p(layer.prio), _p(layer.free), _p(theta), layer.t,
               _p(layer.pool) if layer.pool is not None else None)
    rc = lib().orc_prefill_chunk(C.byref(cfg), C.byref(st), Cq, int(hb), int(N), _p(q), _p(w),
                                 _p(kidx), _p(pred) if pred is not None else None,
                                 _p(host_kv) if host_kv is not None else None,
                                 _p(ext_scores) if ext_scores is not None else None,
                                 C.byref(out))
    layer.t = st.t
    o["scores"] = o["scores"][:, :N]
    o["cand"] = o["cand"][: out.n_cand]
    o["uni"] = o["uni"][: out.n_uni]
    o["pf_h"], o["pf_g"] = o["pf_h"][: out.n_pf], o["pf_g"][: out.n_pf]
    o["miss_h"], o["miss_g"] = o["miss_h"][: out.n_miss], o["miss_g"][: out.n_miss]
    o["status"] = rc
    return o


def ema_update(theta: float, s_k: float, alpha: float = 0.5) -> float:
    return lib().orc_ema_update(theta, s_k, alpha)


class OracleLayer:
    """State of one layer (maps, priorities, free flags, EMA, pool) plus the step."""

    def __init__(self, H, D, k, latent, n_host, n_gpu, max_batch, cap_div=128, alpha=0.5,
                 keep_pool=True):
        self.cfg = Cfg(H, D, k, latent, n_host, n_gpu, cap_div, alpha)
        self.h2g = np.full(n_host, -1, np.int32)
        self.g2h = np.full(n_gpu, -1, np.int32)
        self.prio = np.full(n_gpu, -1, np.int32)
        self.free = np.ones(n_gpu, np.uint8)
        self.theta = np.full(max_batch, np.inf, np.float32)
        self.pool = np.zeros((n_gpu, latent), np.uint16) if keep_pool else None
        self.t = 0
        self.max_batch = max_batch

    def step(self, host_base, ctx, q, w, kidx, host_kv, mode=MODE_EMA, ext_scores=None,
             pages=None):
        """One decode step.  q: uint16 [B, H, D]; w: float32 [B, H]; kidx: uint8 [n_host, D];
        host_kv: uint16 [n_host, latent] or None; ext_scores: float32 [B, >= max ctx] or None;
        pages: int32 [B, page_stride] page table, or None for host_base ranges.
        Returns a dict of outputs (numpy arrays, trimmed to their counts)."""
        cfg = self.cfg
        k = cfg.k
        host_base = np.ascontiguousarray(host_base if host_base is not None else
                                         np.zeros(len(ctx), np.int32), np.int32)
        ctx = np.ascontiguousarray(ctx, np.int32)
        B = int(ctx.size)
        stride = max(1, int(ctx.max()) if B else 1)
        if ext_scores is not None:
            ext_scores = np.ascontiguousarray(ext_scores, np.float32)
            stride = ext_scores.shape[1]
        q = np.ascontiguousarray(q, np.uint16)
        w = np.ascontiguousarray(w, np.float32)
        kidx = np.ascontiguousarray(kidx, np.uint8)
        assert q.shape == (B, cfg.H, cfg.D) and w.shape == (B, cfg.H)
        assert kidx.shape == (cfg.n_host, cfg.D)
        if B and pages is None:
            assert int((host_base.astype(np.int64) + ctx).max()) <= cfg.n_host
        if B and pages is not None:
            assert all(int(h.max()) < cfg.n_host for h in page_host_ids(pages, ctx) if h.size)
        if host_kv is not None:
            host_kv = np.ascontiguousarray(host_kv, np.uint16)
            assert host_kv.shape == (cfg.n_host, cfg.latent)
        o = dict(scores=np.zeros((B, stride), np.float32),
                 sel_tok=np.full((B, k), -1, np.int32), sel_slot=np.full((B, k), -1, np.int32),
                 n_sel=np.zeros(B, np.int32), kth=np.zeros(B, np.float32),
                 pf_tok=np.full((B, k), -1, np.int32), pf_slot=np.full((B, k), -1, np.int32),
                 n_pf=np.zeros(B, np.int32), n_cand=np.zeros(B, np.int32),
                 miss_tok=np.full((B, k), -1, np.int32), n_miss=np.zeros(B, np.int32),
                 evicted=np.full(max(1, cfg.n_gpu), -1, np.int32))
        out = Out(*[_p(o[n]) for n in ("scores", "sel_tok", "sel_slot", "n_sel", "kth", "pf_tok",
                                        "pf_slot", "n_pf", "n_cand", "miss_tok", "n_miss",
                                        "evicted")], 0, 0, 0)
        theta = np.ascontiguousarray(self.theta)
        st = State(_p(self.h2g), _p(self.g2h), _p(self.prio), _p(self.free), _p(theta), self.t,
                   _p(self.pool) if self.pool is not None else None)
        tm, _keep = _tokmap(host_base, pages)
        rc = lib().orc_layer_step(C.byref(cfg), C.byref(st), B, C.byref(tm), _p(ctx), _p(q),
                                  _p(w), _p(kidx),
                                  _p(host_kv) if host_kv is not None else None, int(mode),
                                  _p(ext_scores) if ext_scores is not None else None,
                                  stride, C.byref(out))
        self.theta = theta
        self.t = st.t
        o["status"] = rc
        o["n_evict"] = out.n_evict
        o["n_free_start"] = out.n_free_start
        o["evicted"] = o["evicted"][: out.n_evict]
        return o

    def snapshot(self):
        return dict(h2g=self.h2g.copy(), g2h=self.g2h.copy(), prio=self.prio.copy(),
                    free=self.free.copy(), theta=self.theta.copy(), t=self.t,
                    pool=None if self.pool is None else self.pool.copy())
