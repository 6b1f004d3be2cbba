"""Buffers for the C ABI: device tensors from PyTorch, the host pool from hipHostMalloc.

This module only allocates memory and fills the ABI structs; every step of the
path runs in libecho.so.  Device memory comes from torch (caching allocator,
256-byte aligned); the host KV pool is pinned, mapped host memory allocated with
the HIP runtime so that the recall and prefetch kernels can read it directly.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import torch

from . import abi

_hip = None


def hip() -> C.CDLL:
    global _hip
    if _hip is None:
        _hip = C.CDLL("libamdhip64.so")
        _hip.hipHostMalloc.restype = C.c_int
        _hip.hipHostMalloc.argtypes = [C.POINTER(C.c_void_p), C.c_size_t, C.c_uint]
        _hip.hipHostFree.restype = C.c_int
        _hip.hipHostFree.argtypes = [C.c_void_p]
        _hip.hipHostGetDevicePointer.restype = C.c_int
        _hip.hipHostGetDevicePointer.argtypes = [C.POINTER(C.c_void_p), C.c_void_p, C.c_uint]
    return _hip


HIP_HOST_MALLOC_MAPPED = 0x2
HIP_HOST_MALLOC_COHERENT = 0x40000000


class HostPool:
    """Pinned, mapped, fine-grained host memory holding [rows, latent] bf16 latents."""

    def __init__(self, rows: int, latent: int):
        self.rows, self.latent = rows, latent
        self.nbytes = max(1, rows * latent * 2)
        p = C.c_void_p()
        rc = hip().hipHostMalloc(C.byref(p), self.nbytes,
                                 HIP_HOST_MALLOC_MAPPED | HIP_HOST_MALLOC_COHERENT)
        if rc != 0 or not p.value:
            raise RuntimeError(f"hipHostMalloc({self.nbytes}) failed with {rc}")
        self.host_ptr = p.value
        d = C.c_void_p()
        rc = hip().hipHostGetDevicePointer(C.byref(d), p, 0)
        if rc != 0:
            raise RuntimeError(f"hipHostGetDevicePointer failed with {rc}")
        self.dev_ptr = d.value
        buf = (C.c_uint16 * (rows * latent)).from_address(self.host_ptr)
        self.np = np.ctypeslib.as_array(buf).reshape(rows, latent)  # uint16 bf16 codes
        self.tensor = torch.from_numpy(self.np.view(np.int16))          # CPU view, same memory

    def close(self):
        if self.host_ptr:
            self.np = None
            self.tensor = None
            hip().hipHostFree(C.c_void_p(self.host_ptr))
            self.host_ptr = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def make_dims(n_heads, head_dim, top_k, n_host, n_gpu, max_batch, max_ctx, latent_dim=576,
              ema_alpha=0.5, prefetch_cap_div=128, q_ring=1) -> abi.echo_dims_t:
    return abi.echo_dims_t(n_heads, head_dim, top_k, latent_dim, n_host, n_gpu, max_batch,
                           max_ctx, ema_alpha, prefetch_cap_div, q_ring)


def dims_for(wl, max_ctx=None, q_ring=1) -> abi.echo_dims_t:
    ctx = wl.contexts()
    return make_dims(wl.heads, wl.head_dim, wl.top_k, wl.n_host, wl.n_gpu, wl.batch,
                     int(max_ctx or ctx.max()), wl.latent, wl.alpha, wl.cap_div, q_ring)


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


def check(rc: int, what: str = "") -> None:
    if rc != abi.ECHO_OK:
        raise RuntimeError(f"{what}: {abi.echo_status_string(rc)} ({rc})")


class Workspace:
    """One device buffer carved by echo_ws_bind, with typed views of the outputs."""

    def __init__(self, dims: abi.echo_dims_t, device="cuda"):
        self.dims = dims
        n = abi.echo_ws_bytes(dims)
        if n == 0:
            raise ValueError("invalid dims for the workspace")
        self.buf = torch.zeros(n, dtype=torch.uint8, device=device)
        self.ws = abi.echo_ws_t()
        check(abi.echo_ws_bind(dims, _ptr(self.buf), n, self.ws), "echo_ws_bind")
        B, Cx, K = dims.max_batch, dims.max_ctx, dims.top_k
        base = _ptr(self.buf)

        def view(field, dtype, shape):
            off = getattr(self.ws, field) - base
            cnt = int(np.prod(shape))
            itemsize = torch.empty((), dtype=dtype).element_size()
            return self.buf[off:off + cnt * itemsize].view(dtype).view(*shape)

        self.scores = view("scores", torch.float32, (B, Cx))
        self.sel_tok = view("sel_tok", torch.int32, (B, K))
        self.sel_slot = view("sel_slot", torch.int32, (B, K))
        self.n_sel = view("n_sel", torch.int32, (B,))
        self.kth = view("kth", torch.float32, (B,))
        self.pf_tok = view("pf_tok", torch.int32, (B, K))
        self.pf_slot = view("pf_slot", torch.int32, (B, K))
        self.n_pf = view("n_pf", torch.int32, (B,))
        self.n_cand = view("n_cand", torch.int32, (B,))
        self.miss_tok = view("miss_tok", torch.int32, (B, K))
        self.n_miss = view("n_miss", torch.int32, (B,))
        self.recall_h = view("recall_h", torch.int32, (B * K,))
        self.recall_g = view("recall_g", torch.int32, (B * K,))
        self.counters = view("counters", torch.int32, (abi.ECHO_NCOUNTERS,))
        self.status = view("status", torch.int32, (1,))

    def reset(self):
        check(abi.echo_ws_reset(self.dims, self.ws, stream_handle()), "echo_ws_reset")

    def read(self, B: int) -> dict:
        """Copy the step's outputs to numpy (synchronizes the current stream)."""
        torch.cuda.current_stream().synchronize()
        o = dict(status=int(self.status.item()), counters=self.counters.cpu().numpy(),
                 n_sel=self.n_sel[:B].cpu().numpy(), kth=self.kth[:B].cpu().numpy(),
                 n_pf=self.n_pf[:B].cpu().numpy(), n_cand=self.n_cand[:B].cpu().numpy(),
                 n_miss=self.n_miss[:B].cpu().numpy())
        for name in ("sel_tok", "sel_slot", "pf_tok", "pf_slot", "miss_tok"):
            o[name] = getattr(self, name)[:B].cpu().numpy()
        n = int(o["counters"][abi.ECHO_CNT_MISS])
        o["recall_h"] = self.recall_h[:n].cpu().numpy()
        o["recall_g"] = self.recall_g[:n].cpu().numpy()
        return o


class PrefillWorkspace:
    """One device buffer carved by echo_prefill_ws_bind, with typed views."""

    def __init__(self, dims: abi.echo_dims_t, max_chunk: int, device="cuda"):
        self.dims = dims
        n = abi.echo_prefill_ws_bytes(dims, max_chunk)
        if n == 0:
            raise ValueError("invalid dims or chunk size for the prefill workspace")
        self.buf = torch.zeros(n, dtype=torch.uint8, device=device)
        self.ws = abi.echo_prefill_ws_t()
        check(abi.echo_prefill_ws_bind(dims, max_chunk, _ptr(self.buf), n, self.ws),
              "echo_prefill_ws_bind")
        base = _ptr(self.buf)
        Cq, Nx, K = max_chunk, dims.max_ctx, dims.top_k

        def view(field, dtype, count):
            off = getattr(self.ws, field) - base
            itemsize = torch.empty((), dtype=dtype).element_size()
            return self.buf[off:off + count * itemsize].view(dtype)

        self.scores_flat = view("scores", torch.float32, Cq * Nx)
        self.sel = view("sel", torch.int32, Cq * K).view(Cq, K)
        for name, dt in (("n_sel", torch.int32), ("kth", torch.float32), ("beta", torch.int32),
                         ("n_qcand", torch.int32)):
            setattr(self, name, view(name, dt, Cq))
        for name in ("cand", "uni", "pf_h", "pf_g", "miss_h", "miss_g"):
            setattr(self, name, view(name, torch.int32, Nx))
        self.counts = view("counts", torch.int32, abi.ECHO_PF_NCOUNTS)
        self.status = view("status", torch.int32, 1)
        self.reset()

    def reset(self):
        check(abi.echo_prefill_ws_reset(self.dims, self.ws, stream_handle()),
              "echo_prefill_ws_reset")

    def scores(self, C: int, N: int) -> torch.Tensor:
        return self.scores_flat[: C * N].view(C, N)


class Batch:
    """Device batch rows: contiguous host ranges (host_base), or a page table
    [B, page_stride] of 16-id host pages (pages; host_base is then not used)."""

    def __init__(self, host_base, ctx, device="cuda", pages=None):
        self.ctx = torch.as_tensor(np.asarray(ctx, np.int32), device=device)
        self.B = int(self.ctx.numel())
        self.host_base = torch.as_tensor(np.asarray(host_base if host_base is not None else
                                                    np.zeros(self.B), np.int32), device=device)
        self.pages = None
        stride = 0
        if pages is not None:
            self.pages = torch.as_tensor(np.ascontiguousarray(pages, np.int32), device=device)
            stride = int(self.pages.shape[1])
        self.struct = abi.echo_batch_t(
            self.B, _ptr(self.host_base) if self.B and pages is None else None,
            _ptr(self.ctx) if self.B else None,
            _ptr(self.pages) if self.pages is not None else None, stride)


def pack_kidx(dims: abi.echo_dims_t, rows: torch.Tensor, out: torch.Tensor = None) -> torch.Tensor:
    """Indexer K rows (uint8 fp8 codes [n, D], row-major, on the device) in the tiled
    layout the scoring kernel reads (echo_kindex_pack); n must be a multiple of 16."""
    assert rows.dtype == torch.uint8 and rows.dim() == 2 and rows.is_contiguous()
    if out is None:
        out = torch.empty_like(rows)
    assert out.shape == rows.shape and out.dtype == torch.uint8 and out.is_contiguous()
    check(abi.echo_kindex_pack(dims, rows.data_ptr(), out.data_ptr(), rows.shape[0],
                               stream_handle()), "echo_kindex_pack")
    return out


class Layer:
    """Tensors of one layer.  `kidx` (uint8 [n_host, D] in the tiled layout of
    pack_kidx) and the host pool are shared or owned by the caller; the metadata, GPU
    pool, queries, weights and EMA state are allocated here."""

    def __init__(self, dims: abi.echo_dims_t, kidx: torch.Tensor, host: HostPool, batch: int,
                 device="cuda"):
        self.dims = dims
        G, NH = dims.n_gpu, dims.n_host
        assert kidx.dtype == torch.uint8 and tuple(kidx.shape) == (NH, dims.head_dim)
        assert host.rows >= NH and host.latent == dims.latent_dim
        self.h2g = torch.empty(NH, dtype=torch.int32, device=device)
        self.g2h = torch.empty(G, dtype=torch.int32, device=device)
        self.prio = torch.empty(G, dtype=torch.int32, device=device)
        self.idxbuf = torch.empty(G, dtype=torch.int32, device=device)
        self.free = torch.empty(G, dtype=torch.uint8, device=device)
        self.gpu_kv = torch.zeros((G, dims.latent_dim), dtype=torch.int16, device=device)
        self.q = torch.zeros((dims.q_ring, max(1, batch), dims.n_heads, dims.head_dim),
                             dtype=torch.bfloat16, device=device)
        self.w = torch.zeros((max(1, batch), dims.n_heads), dtype=torch.float32, device=device)
        self.theta = torch.empty(dims.max_batch, dtype=torch.float32, device=device)
        self.guard = torch.empty(dims.max_batch, dtype=torch.float32, device=device)
        self.ctl = torch.zeros(abi.ECHO_CTL_WORDS, dtype=torch.int32, device=device)
        self.stats = torch.zeros(abi.ECHO_STAT_WORDS, dtype=torch.int64, device=device)
        self.kidx = kidx
        self.host = host
        meta = abi.echo_layer_meta_t(_ptr(self.h2g), _ptr(self.g2h), _ptr(self.prio),
                                     _ptr(self.idxbuf), _ptr(self.free))
        self.struct = abi.echo_layer_t(meta, _ptr(kidx), _ptr(self.gpu_kv), host.dev_ptr,
                                       _ptr(self.q), _ptr(self.w), _ptr(self.theta),
                                       _ptr(self.guard), _ptr(self.ctl), _ptr(self.stats))

    def meta_bytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.h2g, self.g2h, self.prio, self.idxbuf, self.free))

    def init(self):
        check(abi.echo_meta_init(self.dims, self.struct, stream_handle()), "echo_meta_init")

    # Between calls the layer's whole cache-management state is in these buffers (the
    # workspace carries nothing from one step to the next): a copy of their bytes is a
    # checkpoint, and written back -- here or into another Layer of the same dims -- the
    # following steps give bit-identical results.
    STATE = ("h2g", "g2h", "prio", "idxbuf", "free", "gpu_kv", "theta", "guard", "ctl",
             "stats")

    def snapshot(self) -> dict:
        """Device copies of the layer's state buffers (stream-ordered)."""
        return {n: getattr(self, n).clone() for n in self.STATE}

    def restore(self, snap: dict) -> None:
        """Write a snapshot back (stream-ordered); shapes must match."""
        for n in self.STATE:
            dst = getattr(self, n)
            assert snap[n].shape == dst.shape and snap[n].dtype == dst.dtype, n
            dst.copy_(snap[n])

    def state(self) -> dict:
        torch.cuda.current_stream().synchronize()
        return dict(h2g=self.h2g.cpu().numpy(), g2h=self.g2h.cpu().numpy(),
                    prio=self.prio.cpu().numpy(), free=self.free.cpu().numpy(),
                    theta=self.theta.cpu().numpy(), t=int(self.ctl[0].item()),
                    nfree=int(self.ctl[1].item()), idxbuf=self.idxbuf.cpu().numpy())
