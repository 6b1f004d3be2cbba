"""Seeded generators for the decode workloads.

Recipe (seed 0 unless stated; every tensor has its own substream, keyed by
(workload, layer, request, tensor) through numpy's SeedSequence):
  * indexer K     ~ N(0, 1), rounded to fp8 E4M3FN (nearest-even), one row per
                    host token; rows no request owns stay zero;
  * MLA latents   ~ N(0, 1), rounded to bf16, 576 per host token;
  * head weights  ~ U[0, 1) fp32, fixed per (layer, request);
  * queries       q_0 ~ N(0, 1); q_t = rho * q_{t-1} + sqrt(1 - rho^2) * eps_t,
                    state kept in fp32, emitted as bf16 at every step;
  * host layout   request b owns host ids host_base[b] .. host_base[b]+ctx[b]-1,
                    host_base[b] = sum of the earlier contexts.
  * prefill       one request's history as above; the chunk queries follow the
                    AR(1) recipe along the prompt positions, head weights
                    U[0, 1) per position.
Generation runs with torch on the requested device: the same seed gives the same
tensor on the same device type (CPU and GPU streams differ from each other).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .configs import Workload

T_K, T_LAT, T_W, T_Q0, T_QN, T_APPEND, T_PQ, T_PW = 1, 2, 3, 4, 5, 6, 7, 8


def seed_for(wl: Workload, seed: int, *key: int) -> int:
    ss = np.random.SeedSequence(seed, spawn_key=(wl.cfg_id,) + tuple(int(x) for x in key))
    return int(ss.generate_state(1, np.uint64)[0])


def _gen(device, s: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(s)
    return g


def host_layout(ctx: np.ndarray, room: int = 0) -> np.ndarray:
    """First host id of each request: requests packed back to back, each starting on a
    16-row boundary (the tiled indexer-K layout groups host ids by 16), with ``room``
    free rows after each context for tokens appended later."""
    ctx = np.asarray(ctx, np.int64)
    span = (ctx + room + 15) // 16 * 16
    base = np.zeros(ctx.size, np.int64)
    if ctx.size > 1:
        base[1:] = np.cumsum(span)[:-1]
    assert base.size == 0 or base[-1] + ctx[-1] < 2**31
    return base.astype(np.int32)


def gen_kidx(wl: Workload, layer: int, ctx, host_base, device, seed=0, out=None) -> torch.Tensor:
    """uint8 fp8-E4M3FN codes [n_host, D]."""
    if out is None:
        out = torch.zeros((wl.n_host, wl.head_dim), dtype=torch.uint8, device=device)
    for b in range(ctx.size):
        n = int(ctx[b])
        if n == 0:
            continue
        g = _gen(device, seed_for(wl, seed, layer, b, T_K))
        x = torch.randn((n, wl.head_dim), generator=g, device=device, dtype=torch.float32)
        h0 = int(host_base[b])
        out[h0:h0 + n] = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def gen_latents(wl: Workload, layer: int, ctx, host_base, device, seed=0, out=None,
                rows=None) -> torch.Tensor:
    """bf16 latents as int16 codes [n_host, latent] (rows no request owns are zero).
    ``rows`` may restrict generation to the first ``rows`` tokens of each request
    (used by bounded samples); the default generates every owned row."""
    if out is None:
        out = torch.zeros((wl.n_host, wl.latent), dtype=torch.int16, device=device)
    for b in range(ctx.size):
        n = int(ctx[b]) if rows is None else min(int(ctx[b]), rows)
        if n == 0:
            continue
        g = _gen(device, seed_for(wl, seed, layer, b, T_LAT))
        x = torch.randn((n, wl.latent), generator=g, device=device, dtype=torch.float32)
        h0 = int(host_base[b])
        out[h0:h0 + n] = x.to(torch.bfloat16).view(torch.int16)
    return out


def gen_w(wl: Workload, layer: int, batch: int, device, seed=0) -> torch.Tensor:
    """fp32 head weights [B, H]."""
    out = torch.empty((batch, wl.heads), dtype=torch.float32, device=device)
    for b in range(batch):
        g = _gen(device, seed_for(wl, seed, layer, b, T_W))
        out[b] = torch.rand((wl.heads,), generator=g, device=device, dtype=torch.float32)
    return out


def gen_q(wl: Workload, layer: int, batch: int, steps: int, device, seed=0) -> torch.Tensor:
    """bf16 queries [steps, B, H, D] following the AR(1) recipe."""
    out = torch.empty((steps, batch, wl.heads, wl.head_dim), dtype=torch.bfloat16, device=device)
    c = float(np.sqrt(max(0.0, 1.0 - wl.rho * wl.rho)))
    for b in range(batch):
        g0 = _gen(device, seed_for(wl, seed, layer, b, T_Q0))
        gn = _gen(device, seed_for(wl, seed, layer, b, T_QN))
        st = torch.randn((wl.heads, wl.head_dim), generator=g0, device=device,
                         dtype=torch.float32)
        for t in range(steps):
            if t > 0:
                eps = torch.randn((wl.heads, wl.head_dim), generator=gn, device=device,
                                  dtype=torch.float32)
                st = wl.rho * st + c * eps
            out[t, b] = st.to(torch.bfloat16)
    return out


def gen_prefill_qw(wl: Workload, layer: int, chunk: int, chunks: int, device, seed=0):
    """Prefill queries and weights for ``chunks`` chunks of ``chunk`` prompt positions:
    bf16 q [chunks, C, H, D] following the AR(1) recipe along the prompt positions
    (coefficient wl.rho) and fp32 w [chunks, C, H] ~ U[0, 1) per position."""
    n = chunk * chunks
    gq = _gen(device, seed_for(wl, seed, layer, 0, T_PQ))
    gw = _gen(device, seed_for(wl, seed, layer, 0, T_PW))
    c = float(np.sqrt(max(0.0, 1.0 - wl.rho * wl.rho)))
    eps = torch.randn((n, wl.heads, wl.head_dim), generator=gq, device=device,
                      dtype=torch.float32)
    q = torch.empty((n, wl.heads, wl.head_dim), dtype=torch.bfloat16, device=device)
    st = eps[0]
    q[0] = st.to(torch.bfloat16)
    for i in range(1, n):
        st = wl.rho * st + c * eps[i]
        q[i] = st.to(torch.bfloat16)
    w = torch.rand((n, wl.heads), generator=gw, device=device, dtype=torch.float32)
    return (q.view(chunks, chunk, wl.heads, wl.head_dim),
            w.view(chunks, chunk, wl.heads))


@dataclass
class Inputs:
    wl: Workload
    layer: int
    ctx: np.ndarray          # int32 [B]
    host_base: np.ndarray    # int32 [B]
    kidx: torch.Tensor       # uint8 [n_host, D]
    latents: torch.Tensor    # int16 (bf16 codes) [n_host, latent]
    w: torch.Tensor          # fp32 [B, H]
    q: torch.Tensor          # bf16 [steps, B, H, D]

    # numpy views for the oracle (copies from the device when needed)
    def np_kidx(self) -> np.ndarray:
        return self.kidx.cpu().numpy()

    def np_latents(self) -> np.ndarray:
        return self.latents.cpu().numpy().view(np.uint16)

    def np_w(self) -> np.ndarray:
        return self.w.cpu().numpy()

    def np_q(self, t: int) -> np.ndarray:
        return self.q[t].cpu().view(torch.int16).numpy().view(np.uint16)


def gen_append(wl: Workload, layer: int, batch: int, step: int, seed=0):
    """The new token of each request at decode step ``step``: uint8 fp8-E4M3FN key codes
    [B, D] and bf16 latent codes as int16 [B, latent], N(0,1) like the history."""
    k = np.zeros((batch, wl.head_dim), np.uint8)
    lat = np.zeros((batch, wl.latent), np.int16)
    for b in range(batch):
        g = _gen("cpu", seed_for(wl, seed, layer, b, T_APPEND, step))
        x = torch.randn((wl.head_dim,), generator=g, dtype=torch.float32)
        y = torch.randn((wl.latent,), generator=g, dtype=torch.float32)
        k[b] = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        lat[b] = y.to(torch.bfloat16).view(torch.int16).numpy()
    return k, lat


def make_inputs(wl: Workload, layer: int = 0, device="cpu", seed: int = 0, steps=None,
                ctx=None, with_latents=True, room: int = 0) -> Inputs:
    ctx = wl.contexts(seed) if ctx is None else np.asarray(ctx, np.int32)
    base = host_layout(ctx, room)
    assert ctx.size == 0 or int(base[-1]) + int(ctx[-1]) <= wl.n_host, "host pool too small"
    steps = wl.steps if steps is None else steps
    kidx = gen_kidx(wl, layer, ctx, base, device, seed)
    lat = (gen_latents(wl, layer, ctx, base, device, seed) if with_latents else
           torch.zeros((wl.n_host, wl.latent), dtype=torch.int16, device=device))
    w = gen_w(wl, layer, ctx.size, device, seed)
    q = gen_q(wl, layer, ctx.size, steps, device, seed)
    return Inputs(wl, layer, ctx, base, kidx, lat, w, q)
