"""The C-ABI library loads, exports every declared symbol, and its host-side logic
(sizes, workspace carving, argument checks) works without a GPU."""
import ctypes as C
import os
import re

import pytest

from kv_cache_offload_fp8_amd import abi
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    if not os.path.exists(abi.LIB_PATH):
        pytest.skip("libecho.so not built (run __graft_entry__.build())")
    return abi.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "echo.h")).read()
    return sorted(set(re.findall(r"^\S[^;(]*?\b(echo_\w+)\(", src, re.M)))


def test_every_declared_symbol_is_exported():
    lib = _lib_or_skip()
    names = _declared()
    assert len(names) >= 12
    assert set(names) == set(abi.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None


def test_meta_bytes_matches_oracle_and_page_example():
    _lib_or_skip()
    for nh, ng in [(2_000_000, 200_000), (4096, 1024), (3_200_000, 110_000), (0, 0)]:
        assert abi.echo_meta_bytes(nh, ng) == O.meta_bytes(nh, ng)
    assert abi.echo_meta_bytes(2_000_000, 200_000) == 10_600_000
    assert abi.echo_meta_bytes(-1, 5) == -1


def _dims(**kw):
    d = dict(n_heads=64, head_dim=128, top_k=2048, latent_dim=576, n_host=2_000_000,
             n_gpu=200_000, max_batch=8, max_ctx=65536, ema_alpha=0.5, prefetch_cap_div=128,
             q_ring=1)
    d.update(kw)
    return abi.echo_dims_t(**d)


def test_workspace_size_and_bind():
    _lib_or_skip()
    d = _dims()
    n = abi.echo_ws_bytes(d)
    assert n > 8 * 65536 * 4  # at least the score buffer
    ws = abi.echo_ws_t()
    base = 1 << 40  # any 256-aligned address: bind only does arithmetic
    assert abi.echo_ws_bind(d, base, n, ws) == abi.ECHO_OK
    ptrs = [getattr(ws, f) for f, _ in abi.echo_ws_t._fields_ if f != "internal_bytes"]
    assert all(base <= p < base + n for p in ptrs)
    assert len(set(ptrs)) == len(ptrs)
    assert all(p % 256 == 0 for p in ptrs)
    assert ws.internal + ws.internal_bytes <= base + n
    assert ws.scores == base
    assert abi.echo_ws_bind(d, base, n - 1, ws) == abi.ECHO_EINVAL
    assert abi.echo_ws_bind(d, base + 8, n, ws) == abi.ECHO_EINVAL


@pytest.mark.parametrize("kw,code", [
    (dict(n_heads=0), abi.ECHO_EINVAL), (dict(top_k=0), abi.ECHO_EINVAL),
    (dict(ema_alpha=0.0), abi.ECHO_EINVAL), (dict(ema_alpha=1.5), abi.ECHO_EINVAL),
    (dict(n_host=1 << 31), abi.ECHO_EINVAL), (dict(q_ring=0), abi.ECHO_EINVAL),
    (dict(n_host=2_000_008 + 4), abi.ECHO_EINVAL),
    (dict(n_heads=65), abi.ECHO_EUNSUPPORTED), (dict(head_dim=256), abi.ECHO_EUNSUPPORTED),
    (dict(head_dim=48), abi.ECHO_EUNSUPPORTED), (dict(top_k=4097), abi.ECHO_EUNSUPPORTED),
    (dict(max_batch=65), abi.ECHO_EUNSUPPORTED), (dict(latent_dim=575), abi.ECHO_EUNSUPPORTED),
])
def test_dims_are_checked(kw, code):
    _lib_or_skip()
    d = _dims(**kw)
    assert abi.echo_ws_bytes(d) == 0
    assert abi.echo_ws_bind(d, 1 << 40, 1 << 40, abi.echo_ws_t()) == code


def test_null_arguments_are_rejected_before_any_launch():
    _lib_or_skip()
    d = _dims()
    ws = abi.echo_ws_t()
    layer = abi.echo_layer_t()
    batch = abi.echo_batch_t(1, None, None)  # batch of one with null arrays
    assert abi.echo_layer_step(d, layer, batch, ws, 0, 0) == abi.ECHO_EINVAL
    assert abi.echo_layer_step(d, None, None, None, 0, 0) == abi.ECHO_EINVAL
    assert abi.echo_indexer_prefetch(d, None, None, None, 0, 0) == abi.ECHO_EINVAL
    assert abi.echo_layer_step(d, layer, batch, ws, 7, 0) == abi.ECHO_EINVAL
    assert abi.echo_topk(d, None, 65536, batch, ws, None, 0) == abi.ECHO_EINVAL
    assert abi.echo_cache_alloc_evict(d, None, batch, ws, 0) == abi.ECHO_EINVAL
    assert abi.echo_recall(d, None, ws, 0) == abi.ECHO_EINVAL
    assert abi.echo_step_advance(None, None, 0) == abi.ECHO_EINVAL
    assert abi.echo_meta_init(d, None, 0) == abi.ECHO_EINVAL
    assert abi.echo_ws_reset(d, None, 0) == abi.ECHO_EINVAL
    too_big = abi.echo_batch_t(9, 1, 1)  # batch above max_batch
    assert abi.echo_topk(d, 1, 65536, too_big, ws, None, 0) == abi.ECHO_EINVAL
    # K layout: null, a row count that is not a whole number of 16-row groups,
    # overlapping buffers, misaligned buffers
    assert abi.echo_kindex_pack(d, None, 1 << 30, 16, 0) == abi.ECHO_EINVAL
    assert abi.echo_kindex_pack(d, 1 << 30, None, 16, 0) == abi.ECHO_EINVAL
    assert abi.echo_kindex_pack(d, 1 << 30, 1 << 31, 15, 0) == abi.ECHO_EINVAL
    assert abi.echo_kindex_pack(d, 1 << 30, (1 << 30) + 1024, 16, 0) == abi.ECHO_EINVAL
    assert abi.echo_kindex_pack(d, (1 << 30) + 8, 1 << 31, 16, 0) == abi.ECHO_EINVAL


def test_status_strings():
    _lib_or_skip()
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
        s = abi.echo_status_string(code)
        assert s and s != "unknown status"
    assert abi.echo_status_string(42) == "unknown status"


def test_binding_has_no_compute_fallback():
    src = open(os.path.join(ROOT, "kv_cache_offload_fp8_amd", "abi.py")).read()
    src += open(os.path.join(ROOT, "kv_cache_offload_fp8_amd", "runtime.py")).read()
    assert "oracle" not in src


def test_newer_entry_points_check_arguments_before_any_launch():
    _lib_or_skip()
    d = _dims()
    ws = abi.echo_ws_t()
    layer = abi.echo_layer_t()
    batch = abi.echo_batch_t(1, None, None)
    for fn in (abi.echo_indexer_begin, abi.echo_indexer_score):
        assert fn(d, None, None, None, 0, 0) == abi.ECHO_EINVAL
        assert fn(d, layer, batch, ws, 7, 0) == abi.ECHO_EINVAL
    assert abi.echo_gather(d, None, batch, ws, 1 << 30, 0) == abi.ECHO_EINVAL
    b1 = abi.echo_batch_t(1, 1 << 30, 1 << 30, None, 0)
    assert abi.echo_append(d, None, b1, 1, 1 << 30, ws, 1, 0) == abi.ECHO_EINVAL
    assert abi.echo_release(d, None, b1, 1, 1, ws, 0) == abi.ECHO_EINVAL
    assert abi.echo_release(d, layer, b1, None, 1, ws, 0) == abi.ECHO_EINVAL
    assert abi.echo_admit(d, None, b1, 0, 0, 16, 1, ws, 0) == abi.ECHO_EINVAL
    # a page table needs a stride of at least one entry; without one, host_base is needed
    for bad in (abi.echo_batch_t(1, None, 1 << 30, 1 << 30, 0),
                abi.echo_batch_t(1, None, 1 << 30, None, 0)):
        assert abi.echo_layer_step(d, layer, bad, ws, 0, 0) == abi.ECHO_EINVAL
    pws = abi.echo_prefill_ws_t()
    chunk = abi.echo_prefill_chunk_t(4, 0, 1000, 1 << 30, 1 << 30, None)
    for fn in (abi.echo_prefill_score, abi.echo_prefill_early, abi.echo_prefill_select):
        assert fn(d, layer, chunk, pws, 0) == abi.ECHO_EINVAL
    assert abi.echo_prefill_copy(d, layer, pws, 0, 0) == abi.ECHO_EINVAL
    assert abi.echo_prefill_ws_reset(d, pws, 0) == abi.ECHO_EINVAL
    # the top-k call without a workspace: null outputs or status, a short stride
    b1 = abi.echo_batch_t(1, 1 << 30, 1 << 30)
    for args in ((None, 65536, b1, 1, 1, 1, None, 1), (1, 65536, b1, None, 1, 1, None, 1),
                 (1, 65536, b1, 1, 1, 1, None, None), (1, 100, b1, 1, 1, 1, None, 1)):
        assert abi.echo_topk_noalloc(d, *args, 0) == abi.ECHO_EINVAL
    # dims whose scratch exceeds the 32 MiB static array are refused before any launch
    big = _dims(max_batch=64, max_ctx=100_000, n_host=6_400_000)
    assert abi.echo_topk_noalloc(big, 1, 100_000, b1, 1, 1, 1, None, 1, 0) == abi.ECHO_ESCRATCH
    fits = _dims(max_batch=32, max_ctx=100_000, n_host=3_200_000)
    assert abi.echo_topk_noalloc(fits, None, 100_000, b1, 1, 1, 1, None, 1, 0) == \
        abi.ECHO_EINVAL
    # the invariant check: null layer, workspace or report, a batch above max_batch
    assert abi.echo_check_invariants(d, None, None, ws, 1 << 30, 0) == abi.ECHO_EINVAL
    assert abi.echo_check_invariants(d, layer, None, ws, 1 << 30, 0) == abi.ECHO_EINVAL
    assert abi.echo_check_invariants(d, layer, abi.echo_batch_t(9, 1, 1), ws, 1 << 30, 0) == \
        abi.ECHO_EINVAL


def test_prefill_workspace_size_and_bind():
    _lib_or_skip()
    d = _dims()
    assert abi.echo_prefill_ws_bytes(d, 0) == 0
    assert abi.echo_prefill_ws_bytes(d, 4097) == 0
    n = abi.echo_prefill_ws_bytes(d, 64)
    m = abi.echo_prefill_ws_bytes(d, 128)
    # the score rows grow with the chunk: at least max_ctx floats per extra query
    assert n > 64 * d.max_ctx * 4 and m - n >= 64 * d.max_ctx * 4
    pws = abi.echo_prefill_ws_t()
    base = 1 << 32
    assert abi.echo_prefill_ws_bind(d, 64, base + 16, n, pws) == abi.ECHO_EINVAL  # misaligned
    assert abi.echo_prefill_ws_bind(d, 64, base, n - 1, pws) == abi.ECHO_EINVAL   # too small
    assert abi.echo_prefill_ws_bind(d, 64, base, n, pws) == abi.ECHO_OK
    ptrs = [getattr(pws, f) for f in ("scores", "sel", "n_sel", "kth", "beta", "n_qcand", "cand",
                                      "uni", "pf_h", "pf_g", "miss_h", "miss_g", "counts",
                                      "status", "internal")]
    assert all(p % 256 == 0 and base <= p < base + n for p in ptrs)
    assert len(set(ptrs)) == len(ptrs) and ptrs == sorted(ptrs)
    assert pws.max_chunk == 64 and pws.internal + pws.internal_bytes == base + n


def test_bench_refuses_more_than_one_gpu():
    # one process per GPU, each with its own requests: the benchmark measures one GPU
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
