"""ctypes binding of the C ABI in include/echo.h -- argument marshalling only.

Every function keeps the C name and returns the C status code; all work happens in
the HIP kernels of libecho.so.  There is no fallback: if the library is missing or
fails to load, the first call raises.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libecho.so")

ECHO_OK, ECHO_EINVAL, ECHO_EHIP, ECHO_EUNSUPPORTED = 0, -1, -2, -3
ECHO_ECAPACITY, ECHO_ETIMEOUT, ECHO_EDEVARG, ECHO_ECORRUPT, ECHO_ESCRATCH = -4, -5, -6, -7, -8
ECHO_THETA_EMA, ECHO_THETA_NEG_INF, ECHO_THETA_POS_INF = 0, 1, 2
(ECHO_CNT_MISS, ECHO_CNT_EVICT, ECHO_CNT_FREE, ECHO_CNT_EVICTABLE, ECHO_CNT_FREE_END,
 ECHO_CNT_PREFETCH, ECHO_CNT_SHORTCUT) = range(7)
ECHO_NCOUNTERS = 16
ECHO_CTL_STEP, ECHO_CTL_NFREE, ECHO_CTL_WORDS = 0, 1, 4
(ECHO_STAT_STEPS, ECHO_STAT_SELECTED, ECHO_STAT_MISSED, ECHO_STAT_PREFETCHED,
 ECHO_STAT_PF_SELECTED, ECHO_STAT_CANDIDATES, ECHO_STAT_EVICTED) = range(7)
ECHO_STAT_WORDS = 8
(ECHO_INV_H2G, ECHO_INV_G2H, ECHO_INV_FREE, ECHO_INV_PRIO, ECHO_INV_FREE_LIST, ECHO_INV_SELECTED,
 ECHO_INV_RESIDENT, ECHO_INV_OCCUPIED) = range(8)
ECHO_INV_WORDS = 8

EXPORTS = ("echo_meta_bytes", "echo_ws_bytes", "echo_ws_bind", "echo_meta_init",
           "echo_ws_reset", "echo_kindex_pack", "echo_indexer_prefetch", "echo_topk",
           "echo_cache_alloc_evict", "echo_recall", "echo_step_advance", "echo_layer_step",
           "echo_indexer_begin", "echo_indexer_score", "echo_append", "echo_gather", "echo_release", "echo_admit", "echo_prefill_ws_bytes",
           "echo_prefill_ws_bind", "echo_prefill_ws_reset", "echo_prefill_score",
           "echo_prefill_early",
           "echo_prefill_select", "echo_prefill_copy", "echo_check_invariants",
           "echo_topk_noalloc", "echo_status_string")

P = C.c_void_p


class echo_dims_t(C.Structure):
    _fields_ = [("n_heads", C.c_int32), ("head_dim", C.c_int32), ("top_k", C.c_int32),
                ("latent_dim", C.c_int32), ("n_host", C.c_int64), ("n_gpu", C.c_int32),
                ("max_batch", C.c_int32), ("max_ctx", C.c_int32), ("ema_alpha", C.c_float),
                ("prefetch_cap_div", C.c_int32), ("q_ring", C.c_int32)]


class echo_layer_meta_t(C.Structure):
    _fields_ = [("h2g", P), ("g2h", P), ("prio", P), ("idxbuf", P), ("free_flags", P)]


class echo_layer_t(C.Structure):
    _fields_ = [("meta", echo_layer_meta_t), ("k_index", P), ("gpu_kv", P), ("host_kv", P),
                ("q", P), ("w", P), ("theta", P), ("guard", P), ("ctl", P), ("stats", P)]


class echo_batch_t(C.Structure):
    _fields_ = [("batch", C.c_int32), ("host_base", P), ("ctx_len", P), ("page_table", P),
                ("page_stride", C.c_int32)]


class echo_ws_t(C.Structure):
    _fields_ = [("scores", P), ("sel_tok", P), ("sel_slot", P), ("n_sel", P), ("kth", P),
                ("pf_tok", P), ("pf_slot", P), ("n_pf", P), ("n_cand", P), ("miss_tok", P),
                ("n_miss", P), ("recall_h", P), ("recall_g", P), ("counters", P),
                ("status", P), ("internal", P), ("internal_bytes", C.c_size_t)]


class echo_prefill_chunk_t(C.Structure):
    _fields_ = [("queries", C.c_int32), ("host_base", C.c_int32), ("hist_len", C.c_int32),
                ("q", P), ("w", P), ("pred", P)]


class echo_prefill_ws_t(C.Structure):
    _fields_ = [("max_chunk", C.c_int32)] + \
        [(n, P) for n in ("scores", "sel", "n_sel", "kth", "beta", "n_qcand", "cand", "uni",
                          "pf_h", "pf_g", "miss_h", "miss_g", "counts", "status",
                          "internal")] + [("internal_bytes", C.c_size_t)]


ECHO_PF_CNT_CAND, ECHO_PF_CNT_UNION, ECHO_PF_CNT_EARLY, ECHO_PF_CNT_LATE = 0, 1, 2, 3
ECHO_PF_NCOUNTS = 8

_lib = None


def lib() -> C.CDLL:
    """Load libecho.so (built by __graft_entry__.build / kv_cache_offload_fp8_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m kv_cache_offload_fp8_amd.build` (no CPU fallback)")
        L = C.CDLL(LIB_PATH)
        dp, lp, bp, wp = (C.POINTER(echo_dims_t), C.POINTER(echo_layer_t),
                          C.POINTER(echo_batch_t), C.POINTER(echo_ws_t))
        sigs = {
            "echo_meta_bytes": (C.c_int64, [C.c_int64, C.c_int64]),
            "echo_ws_bytes": (C.c_size_t, [dp]),
            "echo_ws_bind": (C.c_int, [dp, P, C.c_size_t, wp]),
            "echo_meta_init": (C.c_int, [dp, lp, P]),
            "echo_ws_reset": (C.c_int, [dp, wp, P]),
            "echo_kindex_pack": (C.c_int, [dp, P, P, C.c_int64, P]),
            "echo_indexer_prefetch": (C.c_int, [dp, lp, bp, wp, C.c_int, P]),
            "echo_indexer_begin": (C.c_int, [dp, lp, bp, wp, C.c_int, P]),
            "echo_indexer_score": (C.c_int, [dp, lp, bp, wp, C.c_int, P]),
            "echo_topk": (C.c_int, [dp, P, C.c_int64, bp, wp, P, P]),
            "echo_cache_alloc_evict": (C.c_int, [dp, lp, bp, wp, P]),
            "echo_recall": (C.c_int, [dp, lp, wp, P]),
            "echo_step_advance": (C.c_int, [lp, wp, P]),
            "echo_layer_step": (C.c_int, [dp, lp, bp, wp, C.c_int, P]),
            "echo_append": (C.c_int, [dp, lp, bp, P, P, wp, C.c_int, P]),
            "echo_gather": (C.c_int, [dp, lp, bp, wp, P, P]),
            "echo_release": (C.c_int, [dp, lp, bp, P, C.c_int, wp, P]),
            "echo_admit": (C.c_int, [dp, lp, bp, C.c_int32, C.c_int32, C.c_int32, C.c_int, wp,
                                     P]),
            "echo_prefill_ws_bytes": (C.c_size_t, [dp, C.c_int32]),
            "echo_prefill_ws_bind": (C.c_int, [dp, C.c_int32, P, C.c_size_t,
                                               C.POINTER(echo_prefill_ws_t)]),
            "echo_prefill_ws_reset": (C.c_int, [dp, C.POINTER(echo_prefill_ws_t), P]),
            "echo_prefill_score": (C.c_int, [dp, lp, C.POINTER(echo_prefill_chunk_t),
                                             C.POINTER(echo_prefill_ws_t), P]),
            "echo_prefill_early": (C.c_int, [dp, lp, C.POINTER(echo_prefill_chunk_t),
                                             C.POINTER(echo_prefill_ws_t), P]),
            "echo_prefill_select": (C.c_int, [dp, lp, C.POINTER(echo_prefill_chunk_t),
                                              C.POINTER(echo_prefill_ws_t), P]),
            "echo_prefill_copy": (C.c_int, [dp, lp, C.POINTER(echo_prefill_ws_t), C.c_int, P]),
            "echo_check_invariants": (C.c_int, [dp, lp, bp, wp, P, P]),
            "echo_topk_noalloc": (C.c_int, [dp, P, C.c_int64, bp, P, P, P, P, P, P]),
            "echo_status_string": (C.c_char_p, [C.c_int]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ref(x):
    return None if x is None else C.byref(x)


def echo_meta_bytes(n_host: int, n_gpu: int) -> int:
    return lib().echo_meta_bytes(n_host, n_gpu)


def echo_ws_bytes(dims: echo_dims_t) -> int:
    return lib().echo_ws_bytes(C.byref(dims))


def echo_ws_bind(dims, base: int, nbytes: int, ws: echo_ws_t) -> int:
    return lib().echo_ws_bind(C.byref(dims), base, nbytes, C.byref(ws))


def echo_meta_init(dims, layer, stream: int) -> int:
    return lib().echo_meta_init(C.byref(dims), _ref(layer), stream)


def echo_ws_reset(dims, ws, stream: int) -> int:
    return lib().echo_ws_reset(C.byref(dims), _ref(ws), stream)


def echo_kindex_pack(dims, rows: int, tiled: int, n_rows: int, stream: int) -> int:
    return lib().echo_kindex_pack(C.byref(dims), rows, tiled, n_rows, stream)


def echo_indexer_prefetch(dims, layer, batch, ws, theta_mode: int, stream: int) -> int:
    return lib().echo_indexer_prefetch(C.byref(dims), _ref(layer), _ref(batch), _ref(ws),
                                       theta_mode, stream)


def echo_indexer_begin(dims, layer, batch, ws, theta_mode: int, stream: int) -> int:
    return lib().echo_indexer_begin(C.byref(dims), _ref(layer), _ref(batch), _ref(ws),
                                    theta_mode, stream)


def echo_indexer_score(dims, layer, batch, ws, theta_mode: int, stream: int) -> int:
    return lib().echo_indexer_score(C.byref(dims), _ref(layer), _ref(batch), _ref(ws),
                                    theta_mode, stream)


def echo_topk(dims, scores: int, score_stride: int, batch, ws, theta, stream: int) -> int:
    return lib().echo_topk(C.byref(dims), scores, score_stride, _ref(batch), _ref(ws), theta,
                           stream)


def echo_topk_noalloc(dims, scores: int, score_stride: int, batch, sel_tok: int, n_sel: int,
                      kth: int, theta, status: int, stream: int) -> int:
    """All pointers are device addresses; theta may be None."""
    return lib().echo_topk_noalloc(C.byref(dims), scores, score_stride, _ref(batch), sel_tok,
                                   n_sel, kth, theta, status, stream)


def echo_cache_alloc_evict(dims, layer, batch, ws, stream: int) -> int:
    return lib().echo_cache_alloc_evict(C.byref(dims), _ref(layer), _ref(batch), _ref(ws), stream)


def echo_recall(dims, layer, ws, stream: int) -> int:
    return lib().echo_recall(C.byref(dims), _ref(layer), _ref(ws), stream)


def echo_step_advance(layer, ws, stream: int) -> int:
    return lib().echo_step_advance(_ref(layer), _ref(ws), stream)


def echo_layer_step(dims, layer, batch, ws, theta_mode: int, stream: int) -> int:
    return lib().echo_layer_step(C.byref(dims), _ref(layer), _ref(batch), _ref(ws), theta_mode,
                                 stream)


def echo_append(dims, layer, batch, k_new: int, latent_new: int, ws, advance: int,
                stream: int) -> int:
    """k_new, latent_new: device pointers; batch.ctx_len is updated in place when
    advance != 0."""
    return lib().echo_append(C.byref(dims), _ref(layer), _ref(batch), k_new, latent_new,
                             _ref(ws), advance, stream)


def echo_gather(dims, layer, batch, ws, out: int, stream: int) -> int:
    """out: device pointer to [batch][k][latent] bf16 (16-byte aligned)."""
    return lib().echo_gather(C.byref(dims), _ref(layer), _ref(batch), _ref(ws), out, stream)


def echo_release(dims, layer, batch, mask: int, commit: int, ws, stream: int) -> int:
    """mask: device int32 pointer; with commit, batch.ctx_len of the released requests
    becomes 0."""
    return lib().echo_release(C.byref(dims), _ref(layer), _ref(batch), mask, commit, _ref(ws),
                              stream)


def echo_admit(dims, layer, batch, b: int, base: int, length: int, commit: int, ws,
               stream: int) -> int:
    """With commit, row b of the batch takes (base, length), or length tokens on the pages
    of its page-table row."""
    return lib().echo_admit(C.byref(dims), _ref(layer), _ref(batch), b, base, length, commit,
                            _ref(ws), stream)


def echo_prefill_ws_bytes(dims, max_chunk: int) -> int:
    return lib().echo_prefill_ws_bytes(C.byref(dims), max_chunk)


def echo_prefill_ws_bind(dims, max_chunk: int, base: int, nbytes: int, pws) -> int:
    return lib().echo_prefill_ws_bind(C.byref(dims), max_chunk, base, nbytes, C.byref(pws))


def echo_prefill_ws_reset(dims, pws, stream: int) -> int:
    return lib().echo_prefill_ws_reset(C.byref(dims), C.byref(pws), stream)


def echo_prefill_score(dims, layer, chunk, pws, stream: int) -> int:
    return lib().echo_prefill_score(C.byref(dims), _ref(layer), C.byref(chunk), C.byref(pws),
                                    stream)


def echo_prefill_early(dims, layer, chunk, pws, stream: int) -> int:
    return lib().echo_prefill_early(C.byref(dims), _ref(layer), C.byref(chunk), C.byref(pws),
                                    stream)


def echo_prefill_select(dims, layer, chunk, pws, stream: int) -> int:
    return lib().echo_prefill_select(C.byref(dims), _ref(layer), C.byref(chunk), C.byref(pws),
                                     stream)


def echo_prefill_copy(dims, layer, pws, which: int, stream: int) -> int:
    """which: 0 = the early installs, 1 = the later ones."""
    return lib().echo_prefill_copy(C.byref(dims), _ref(layer), C.byref(pws), which, stream)


def echo_check_invariants(dims, layer, batch, ws, report: int, stream: int) -> int:
    """report: device pointer to int32 [ECHO_INV_WORDS]; batch may be None."""
    return lib().echo_check_invariants(C.byref(dims), _ref(layer), _ref(batch), _ref(ws),
                                       report, stream)


def echo_status_string(code: int) -> str:
    return lib().echo_status_string(code).decode()
