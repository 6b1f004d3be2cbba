"""Decode-step benchmark of the ECHO offload hot path on one MI355X.

Default workload: capacity-constrained decode -- batch 32, contexts uniform in
[80,000, 100,000], 61 layers run one after another in one hipGraph per decode
step, indexer 64 heads x 128 (bf16 q, fp8-E4M3 K), top-k 2048, GPU pool 110,000
slots per layer, host pool 3,200,000 tokens x 576 bf16, query AR(1) rho 0.98.
A "step" is one decode step: every layer runs indexer + prefetch, exact top-k,
protect/evict/alloc and recall for the whole batch.  The metric is layer-steps/s
(layers x steps / elapsed).  Inputs are seeded synthetic tensors resident in HBM
(and in pinned host memory for the host pool) before the timed region starts.

Also reported: the scoring kernel's HBM roofline (algorithmic bytes: 128 B of K
read + 4 B of score written per scored token; measured with prefetch off, where
the same kernel only scores), the layer step against its host-link floor (every
prefetched or missed row crosses the link once), the recall host-link rate, the
measured pinned host-link peaks, the GPU-cache hit rate and a CPU baseline of the
oracle on a bounded sample of one layer-step.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload capacity]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0  # dense fp8 MFMA
BYTES_PER_SCORED_TOKEN = 128 + 4


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=16)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--workload", default="capacity")
    p.add_argument("--layers", type=int, default=None, help="override the layer count")
    p.add_argument("--host-pools", type=int, default=4,
                   help="distinct pinned host pools; layers share them round-robin")
    p.add_argument("--breakdown-steps", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-requests", type=int, default=32)
    p.add_argument("--cpu-sample-steps", type=int, default=12,
                   help="decode steps of layer 0 the CPU oracle runs (about 1 s each)")
    p.add_argument("--mode", default="ema", choices=["ema", "neg_inf", "pos_inf"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cap-div", type=int, default=None,
                   help="override the prefetch cap divisor (cap = min(k, ceil(ctx/div)))")
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the chunked-prefill measurement")
    p.add_argument("--prefill-chunks", type=int, default=4)
    p.add_argument("--prefill-only", action="store_true",
                   help="run only the chunked-prefill measurement and print its JSON object")
    p.add_argument("--pmc-calibrate", action="store_true",
                   help="end with a 256 MiB device-to-device copy whose FETCH_SIZE / WRITE_SIZE "
                        "counters scale the indexer's")
    p.add_argument("--headline-only", action="store_true",
                   help="only the timed decode steps of the workload (for kernel traces of the "
                        "step as it runs)")
    p.add_argument("--no-paged", action="store_true",
                   help="skip the decode step with page tables")
    p.add_argument("--no-ablation", action="store_true",
                   help="skip the threshold-mode ablation and the prefetch-cap sweep")
    p.add_argument("--no-other-workloads", action="store_true",
                   help="skip the low-locality and single-layer decode workloads")
    p.add_argument("--cap-sweep", default="128,192,384",
                   help="prefetch cap divisors measured beside the workload's own")
    return p.parse_args()


# the sources the scoring kernel and its launch are built from
SCORE_SOURCES = ("kv_cache_offload_fp8_amd/csrc/k_index.hip", "kv_cache_offload_fp8_amd/csrc/copy.h",
                 "kv_cache_offload_fp8_amd/csrc/kernels.h", "kv_cache_offload_fp8_amd/csrc/common.h",
                 "include/echo.h")


def source_digest() -> str:
    """sha1 over the scoring kernel's sources: the stored HBM-traffic figures hold only
    while it matches."""
    import hashlib
    h = hashlib.sha1()
    for f in SCORE_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def stored_traffic():
    """Bytes per launch of the scoring kernel from the committed counter summary
    (profiles/k_score_capacity_traffic.txt), or None if it is missing or the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "k_score_capacity_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha1") != source_digest():
        return None
    try:
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def stored_step_kernel(total_tok):
    """The scoring kernel as the decode step runs it (k_score<4,true>: prefetch on, its
    copy handed over to the next kernel), from the committed kernel-trace summary
    (profiles/k_score_in_step_capacity.txt), or None if it is missing or the scoring
    kernel's sources changed since the trace was taken."""
    path = os.path.join(ROOT, "profiles", "k_score_in_step_capacity.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha1") != source_digest():
        return None
    try:
        ms = float(kv["avg_launch_us"]) / 1e3
        n = int(kv["launches"])
    except (KeyError, ValueError):
        return None
    gbps = total_tok * BYTES_PER_SCORED_TOKEN / (ms * 1e-3) / 1e9
    return {"kernel": "k_score<4,true> inside the captured decode step (EMA prefetch on, host "
                      "reads of the prefetch copy in flight on other compute units)",
            "avg_launch_ms": round(ms, 5), "launches": n, "hbm_gbps": round(gbps, 1),
            "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "source": "profiles/k_score_in_step_capacity.txt (rocprofv3 kernel trace of "
                      "bench.py --headline-only)"}


def replay_median_ms(graph, n, warm=40):
    """Median duration of n replays of `graph`, each timed with events on the current
    stream after the previous one has finished, after `warm` untimed replays: the GPU
    reaches its sustained speed only after some tens of milliseconds of load (after 5
    warm-up replays the scoring kernel still measured 1-4% slower than after 40, and
    the first replays after idle or link-bound work 3-8% slower)."""
    import torch
    for _ in range(warm):
        graph.replay()
    times = []
    for _ in range(n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    return 0.5 * (times[(n - 1) // 2] + times[n // 2])


class Decode:
    """One decode workload on the device: its layers (tiled indexer K, queries,
    weights, metadata and GPU pool), pinned host pools shared round-robin by the
    layers, the batch and one workspace shared by every layer."""

    def __init__(self, wl, args, dev, L, npools, q_ring, room=0, keep_rows0=False):
        import torch

        from kv_cache_offload_fp8_amd import runtime as R
        from synth import gen as G

        self.wl, self.L, self.dev = wl, L, dev
        self.ctx = wl.contexts(args.seed)
        self.base = G.host_layout(self.ctx, room=room)
        self.B = int(self.ctx.size)
        self.total_tok = int(self.ctx.sum())
        self.q_ring = q_ring
        self.dims = self.make_dims(wl.cap_div)
        t0 = time.time()
        self.pools = []
        for i in range(max(1, min(npools, L))):
            hp = R.HostPool(wl.n_host, wl.latent)
            lat = G.gen_latents(wl, i, self.ctx, self.base, dev, args.seed,
                                out=torch.empty((wl.n_host, wl.latent), dtype=torch.int16,
                                                device=dev))
            hp.tensor.copy_(lat)
            del lat
            self.pools.append(hp)
        self.layers = []
        rows = torch.empty((wl.n_host, wl.head_dim), dtype=torch.uint8, device=dev)
        self.rows0 = None
        for l in range(L):
            rows.zero_()
            G.gen_kidx(wl, l, self.ctx, self.base, dev, args.seed, out=rows)
            if l == 0 and keep_rows0:
                self.rows0 = rows.clone()
            kidx = R.pack_kidx(self.dims, rows, torch.empty_like(rows))
            lay = R.Layer(self.dims, kidx, self.pools[l % len(self.pools)], self.B, dev)
            lay.q.copy_(G.gen_q(wl, l, self.B, q_ring, dev, args.seed))
            lay.w.copy_(G.gen_w(wl, l, self.B, dev, args.seed))
            lay.init()
            self.layers.append(lay)
        del rows
        self.batch = R.Batch(self.base, self.ctx, dev)
        self.ws = R.Workspace(self.dims, dev)
        self.ws.reset()
        torch.cuda.synchronize()
        log(f"[bench] {wl.name}: B={self.B} ctx {self.ctx.min()}..{self.ctx.max()} (sum "
            f"{self.total_tok}) L={L} n_gpu={wl.n_gpu} n_host={wl.n_host}: {len(self.pools)} "
            f"host pools, {L} layers ready ({time.time() - t0:.1f}s)")

    def make_dims(self, cap_div):
        from kv_cache_offload_fp8_amd import runtime as R
        wl = self.wl
        return R.make_dims(wl.heads, wl.head_dim, wl.top_k, wl.n_host, wl.n_gpu, self.B,
                           int(self.ctx.max()) + 1, wl.latent, wl.alpha, cap_div, self.q_ring)

    def paged_batch(self, seed):
        """The same requests on 16-id host pages scattered over the whole pool: every page
        the contiguous layout uses is replaced by a page drawn without replacement from a
        seeded permutation of all the pool's pages.  The data stay where they are (every
        token's K and latent are i.i.d. draws, so the scores keep their distribution); only
        the addressing of every kernel changes."""
        from kv_cache_offload_fp8_amd import runtime as R
        npages = self.wl.n_host // 16
        span = (self.ctx.astype(np.int64) + 15) // 16
        stride = int(span.max())
        perm = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(0x9A6E,))) \
            .permutation(npages).astype(np.int32)
        pages = np.full((self.B, stride), -1, np.int32)
        off = 0
        for b in range(self.B):
            pages[b, : span[b]] = perm[off: off + span[b]]
            off += int(span[b])
        return R.Batch(None, self.ctx, self.dev, pages=pages)

    def reinit(self):
        import torch
        for lay in self.layers:
            lay.init()
        self.ws.reset()
        torch.cuda.synchronize()

    def capture(self, mode, dims, stream):
        """One decode step (every layer's echo_layer_step) captured in one hipGraph."""
        import torch

        from kv_cache_offload_fp8_amd import abi
        from kv_cache_offload_fp8_amd import runtime as R
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for lay in self.layers:
                    R.check(abi.echo_layer_step(dims, lay.struct, self.batch.struct, self.ws.ws,
                                                mode, stream.cuda_stream), "echo_layer_step")
        torch.cuda.synchronize()
        return g

    def stats(self):
        import torch
        return torch.stack([lay.stats for lay in self.layers]).cpu().numpy().astype(np.int64)

    def status(self, what):
        from kv_cache_offload_fp8_amd import abi
        st = int(self.ws.status.item())
        if st != 0:
            raise SystemExit(f"device status after {what}: {abi.echo_status_string(st)}")

    def run(self, mode, steps, warmup, stream, cap_div=None, init=True):
        """Capture a decode step, replay it `warmup` times untimed, then time `steps`
        replays between synchronizations.  Returns the timing and the layers' running
        totals over the timed replays."""
        import torch
        dims = self.dims if cap_div is None else self.make_dims(cap_div)
        if init:
            self.reinit()
        g = self.capture(mode, dims, stream)
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        self.status("warmup")
        s0 = self.stats()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ev0.record()
        for _ in range(steps):
            g.replay()
        ev1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        gpu_ms = ev0.elapsed_time(ev1)
        elapsed = max(wall, gpu_ms / 1e3)
        self.status("timed steps")
        delta = self.stats() - s0
        del g
        return dict(elapsed=elapsed, ms_per_step=elapsed * 1e3 / steps,
                    layer_steps_per_s=steps * self.L / elapsed,
                    us_per_layer_step=elapsed * 1e6 / (steps * self.L), stats=delta, steps=steps)

    def close(self):
        for hp in self.pools:
            hp.close()
        self.pools = []
        self.layers = []


def totals_summary(delta, steps, row_bytes, link_peak=None, us_per_layer_step=None):
    """Per-layer-step figures from the layers' running totals over timed replays."""
    from kv_cache_offload_fp8_amd import abi
    L = delta.shape[0]
    tot = delta.sum(0)
    ls = max(1, int(tot[abi.ECHO_STAT_STEPS]))
    sel = max(1, int(tot[abi.ECHO_STAT_SELECTED]))
    pf = int(tot[abi.ECHO_STAT_PREFETCHED])
    per_layer_hit = 1.0 - delta[:, abi.ECHO_STAT_MISSED] / np.maximum(
        1, delta[:, abi.ECHO_STAT_SELECTED])
    worst = np.argsort(per_layer_hit)[:3]
    tot = [int(x) for x in tot]
    out = {
        "layer_steps_counted": ls,
        "hit_rate": round(1.0 - tot[abi.ECHO_STAT_MISSED] / sel, 5),
        "selected_per_layer_step": round(sel / ls, 1),
        "misses_per_layer_step": round(tot[abi.ECHO_STAT_MISSED] / ls, 1),
        "prefetched_per_layer_step": round(pf / ls, 1),
        "prefetch_candidates_per_layer_step": round(tot[abi.ECHO_STAT_CANDIDATES] / ls, 1),
        "prefetch_selected_same_step_frac": round(tot[abi.ECHO_STAT_PF_SELECTED] / max(1, pf), 4),
        "evicted_per_layer_step": round(tot[abi.ECHO_STAT_EVICTED] / ls, 1),
        "link_mb_per_layer_step": round((pf + tot[abi.ECHO_STAT_MISSED]) * row_bytes / ls / 1e6,
                                        3),
    }
    if L > 1:
        out["per_layer_hit_rate_min"] = round(float(per_layer_hit.min()), 5)
        out["lowest_hit_layers"] = [[int(l), round(float(per_layer_hit[l]), 4)] for l in worst]
    if link_peak and us_per_layer_step:
        link_us = (pf + tot[abi.ECHO_STAT_MISSED]) * row_bytes / ls / (link_peak * 1e3)
        out["link_floor_us"] = round(float(link_us), 2)
        out["link_floor_frac"] = round(float(link_us / us_per_layer_step), 4)
    assert steps * L == ls, (steps, L, ls)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the decode hot "
              "path shards by request, one independent copy per GPU, and this benchmark "
              "measures the single-GPU share.", file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_offload_fp8_amd import abi
    from kv_cache_offload_fp8_amd import runtime as R
    from synth import get

    torch.cuda.set_device(0)
    dev = "cuda"
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_measure(args, dev)}), flush=True)
        return
    wl = get(args.workload)
    if args.cap_div:
        wl = wl.scaled(cap_div=args.cap_div)
    L = args.layers or wl.layers
    mode_of = {"ema": abi.ECHO_THETA_EMA, "neg_inf": abi.ECHO_THETA_NEG_INF,
               "pos_inf": abi.ECHO_THETA_POS_INF}
    mode = mode_of[args.mode]
    q_ring = args.warmup + args.steps + args.breakdown_steps
    # one free row per request: the append measurement writes there
    D = Decode(wl, args, dev, L, args.host_pools, q_ring, room=1,
               keep_rows0=not args.no_cpu_baseline)
    dims, layers, batch, ws, B = D.dims, D.layers, D.batch, D.ws, D.B
    ctx, base, total_tok = D.ctx, D.base, D.total_tok
    log(f"[bench] meta/layer {layers[0].meta_bytes()} B = echo_meta_bytes "
        f"{abi.echo_meta_bytes(wl.n_host, wl.n_gpu)}")
    cs = torch.cuda.Stream()
    row = wl.latent * 2

    # -------------------------------------------------------- timed region
    head = D.run(mode, args.steps, args.warmup, cs, init=False)
    ms_per_step = head["ms_per_step"]
    layer_steps_per_s = head["layer_steps_per_s"]
    shortcut_last = int(ws.counters[abi.ECHO_CNT_SHORTCUT].item())
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step, "
        f"{layer_steps_per_s:.1f} layer-steps/s")
    timed = totals_summary(head["stats"], args.steps, row)
    log(f"[bench] timed replays: {timed}")
    if args.headline_only:
        print(json.dumps({"metric": "decode layer-steps/s", "value": round(layer_steps_per_s, 3),
                          "unit": "layer-steps/s", "steps": args.steps,
                          "ms_per_step": round(ms_per_step, 4), "timed_replays": timed}),
              flush=True)
        D.close()
        return

    # ------------------------------------------- per-phase breakdown (eager)
    # The same layer steps as the five separate calls, with events between them;
    # each layer's threshold before the step, its k-th scores, prefetch list and
    # selection are kept for the threshold and prefetch-usefulness figures.
    s = torch.cuda.current_stream()
    sh = s.cuda_stream
    nph = 4
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)]
           for _ in range(args.breakdown_steps * L)]
    miss_rows = []
    keep = []  # per (step, layer): theta before, kth, n_pf, pf_tok, n_sel, sel_tok
    i = 0
    for _ in range(args.breakdown_steps):
        for lay in layers:
            e = evs[i]
            theta_before = lay.theta[:B].clone()
            e[0].record(s)
            R.check(abi.echo_indexer_prefetch(dims, lay.struct, batch.struct, ws.ws, mode, sh),
                    "indexer")
            e[1].record(s)
            R.check(abi.echo_topk(dims, ws.ws.scores, dims.max_ctx, batch.struct, ws.ws,
                                  lay.struct.theta if mode == abi.ECHO_THETA_EMA else None, sh),
                    "topk")
            e[2].record(s)
            R.check(abi.echo_cache_alloc_evict(dims, lay.struct, batch.struct, ws.ws, sh),
                    "alloc_evict")
            e[3].record(s)
            R.check(abi.echo_recall(dims, lay.struct, ws.ws, sh), "recall")
            e[4].record(s)
            R.check(abi.echo_step_advance(lay.struct, ws.ws, sh), "advance")
            miss_rows.append(ws.counters[abi.ECHO_CNT_MISS].clone())
            keep.append((theta_before, ws.kth[:B].clone(), ws.n_pf[:B].clone(),
                         ws.pf_tok[:B].clone(), ws.n_sel[:B].clone(), ws.sel_tok[:B].clone()))
            i += 1
    torch.cuda.synchronize()
    D.status("breakdown")
    ph = np.array([[evs[j][p].elapsed_time(evs[j][p + 1]) for p in range(nph)]
                   for j in range(len(evs))])  # ms
    misses = np.array([int(x) for x in miss_rows])
    idx_ms = float(ph[:, 0].mean())
    idx_bytes = total_tok * BYTES_PER_SCORED_TOKEN
    idx_gbps = idx_bytes / (idx_ms * 1e-3) / 1e9
    recall_ms = ph[:, 3]
    recall_eager_gbps = float((misses * row).sum() / (recall_ms.sum() * 1e-3) / 1e9)
    thr = threshold_and_usefulness(keep, L, args.breakdown_steps, wl.top_k, ctx)
    log(f"[bench] phases (ms, mean over {len(evs)} layer-steps): indexer {idx_ms:.4f} "
        f"topk {ph[:, 1].mean():.4f} alloc/evict {ph[:, 2].mean():.4f} "
        f"recall {recall_ms.mean():.4f}; threshold and usefulness {thr}")
    # Recall rate as the step runs it, back to back in a graph: the last layer's
    # miss list (still in the workspace) recalled `nrc` times into its pool (the
    # same rows to the same slots each time), timed with events around one replay.
    nrc = 32
    rc_rows, rc_ms = recall_in_graph(D, layers[-1], nrc, cs)
    recall_gbps = rc_rows * row / (rc_ms * 1e-3) / 1e9
    log(f"[bench] recall in a graph: {rc_rows} rows in {rc_ms * 1e3:.1f} us per launch = "
        f"{recall_gbps:.1f} GB/s (eager, event per call: {recall_eager_gbps:.1f} GB/s)")

    # ------------------------------------- indexer with prefetch off (scoring only)
    # Threshold +inf: the same kernel scores every token but prefetches nothing and
    # changes no cache state, so this isolates the HBM-bound scoring stream.
    nso = min(L, 16)
    nrep = 10
    # back to back in a graph, as the step runs its kernels: nso calls (layers
    # 0..nso-1) per replay.  Each of nrep replays is timed on its own with events on
    # the stream it is replayed on, after the previous one has finished, and the
    # median is taken.  (Replays launched back to back vary between replays by about
    # 10%: the scoring graph runs once per layer-step in the decode step, between
    # link-bound kernels, not back to back with itself.)
    gso = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(gso, stream=cs):
            for j in range(nso):
                R.check(abi.echo_indexer_prefetch(dims, layers[j].struct, batch.struct, ws.ws,
                                                  abi.ECHO_THETA_POS_INF, cs.cuda_stream),
                        "indexer")
    gso.replay()
    torch.cuda.synchronize()
    so_ms = replay_median_ms(gso, nrep) / nso
    del gso
    so_gbps = total_tok * BYTES_PER_SCORED_TOKEN / (so_ms * 1e-3) / 1e9
    log(f"[bench] indexer, prefetch off: {so_ms:.4f} ms = {so_gbps:.0f} GB/s "
        f"({so_gbps / HBM_PEAK_GBPS:.1%} of HBM peak; {nso} calls back to back in a graph, "
        f"median of {nrep} replays)")
    # the scoring kernel alone: the same graph with only the prologue of every call
    # (echo_indexer_begin), timed the same way; the difference per call is the
    # scoring kernel's launch duration in the graph
    gbg = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(gbg, stream=cs):
            for j in range(nso):
                R.check(abi.echo_indexer_begin(dims, layers[j].struct, batch.struct, ws.ws,
                                               abi.ECHO_THETA_POS_INF, cs.cuda_stream), "begin")
    gbg.replay()
    torch.cuda.synchronize()
    begin_ms = replay_median_ms(gbg, nrep) / nso
    del gbg
    ks_ms = so_ms - begin_ms
    ks_gbps = total_tok * BYTES_PER_SCORED_TOKEN / (ks_ms * 1e-3) / 1e9
    log(f"[bench] scoring kernel (k_score, prefetch off): {ks_ms:.4f} ms per launch = "
        f"{ks_gbps:.0f} GB/s ({ks_gbps / HBM_PEAK_GBPS:.1%} of HBM peak): {so_ms:.4f} ms per "
        f"call less {begin_ms:.4f} ms per prologue, both the median of {nrep} replays of {nso} calls")

    if args.pmc_calibrate:  # a plain copy of known size for the HBM-traffic counters
        cal_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        cal_dst = torch.empty_like(cal_src)
        cal_dst.copy_(cal_src)
        torch.cuda.synchronize()
        del cal_src, cal_dst

    # ------------------------------------------------------ host-link peaks
    memcpy_gbps, zc_gbps = link_peaks(D, sh)
    link_peak = max(memcpy_gbps, zc_gbps)
    log(f"[bench] host link: hipMemcpy H2D {memcpy_gbps:.1f} GB/s, zero-copy recall kernel "
        f"{zc_gbps:.1f} GB/s")

    # layer-step floor: every prefetched and missed row of the timed replays crosses
    # the host link once
    step_ms = ms_per_step / L
    timed = totals_summary(head["stats"], args.steps, row, link_peak, step_ms * 1e3)
    link_bytes = timed["link_mb_per_layer_step"] * 1e6
    link_floor_ms = link_bytes / (link_peak * 1e9) * 1e3
    traffic = stored_traffic()
    in_step = stored_step_kernel(total_tok)
    log(f"[bench] layer step {step_ms * 1e3:.1f} us; host-link floor "
        f"{link_floor_ms * 1e3:.1f} us ({link_floor_ms / step_ms:.1%})")

    # ----------------------------------------------- attention input (gather)
    # The last layer-step's selections (still in the workspace) gathered from layer
    # 0's pool into the dense [B][k][latent] attention input, 16 calls back to back in
    # a graph.  HBM-bound: each selected row is read once and every output row written.
    n_sel_tot = int(ws.n_sel[:B].sum().item())
    gout = torch.empty((B, wl.top_k, wl.latent), dtype=torch.int16, device=dev)
    ngr = 16
    ggr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(ggr, stream=cs):
            for _ in range(ngr):
                R.check(abi.echo_gather(dims, layers[0].struct, batch.struct, ws.ws,
                                        gout.data_ptr(), cs.cuda_stream), "gather")
    ggr.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    ggr.replay()
    g1.record()
    torch.cuda.synchronize()
    gather_ms = g0.elapsed_time(g1) / ngr
    del ggr, gout
    gather_bytes = (n_sel_tot + B * wl.top_k) * row
    gather_gbps = gather_bytes / (gather_ms * 1e-3) / 1e9
    log(f"[bench] attention-input gather: {gather_ms * 1e3:.1f} us for {n_sel_tot} rows = "
        f"{gather_gbps:.0f} GB/s ({gather_gbps / HBM_PEAK_GBPS:.1%} of HBM peak)")

    # ----------------------------------------------- decode append (writeback)
    # One step's new tokens appended to every layer, back to back in a graph, without
    # advancing the contexts (each replay writes the same rows): the per-layer cost
    # of keeping the indexer K on the GPU and backing each token up to the host pool.
    k_new = torch.randint(0, 120, (B, wl.head_dim), dtype=torch.uint8, device=dev)
    lat_new = torch.zeros((B, wl.latent), dtype=torch.int16, device=dev)
    gap = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(gap, stream=cs):
            for lay in layers:
                R.check(abi.echo_append(dims, lay.struct, batch.struct, k_new.data_ptr(),
                                        lat_new.data_ptr(), ws.ws, 0, cs.cuda_stream), "append")
    gap.replay()
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    gap.replay()
    a1.record()
    torch.cuda.synchronize()
    D.status("append")
    append_ms = a0.elapsed_time(a1) / L
    del gap
    log(f"[bench] append: {append_ms * 1e3:.1f} us per layer ({B} tokens: {B * wl.head_dim} B "
        f"of indexer K in HBM, {B * row} B of latents to the host pool)")

    # ----------------------------------------------- request release and admission
    # Request 0 cancelled on every layer (its slots and map rows given back, the free
    # list rebuilt), then admitted again into its own range; each call once per layer,
    # eagerly (a second release would find nothing to free), with commit on the last.
    mask = torch.zeros(B, dtype=torch.int32, device=dev)
    mask[0] = 1
    resident0 = int((layers[-1].h2g[int(base[0]):int(base[0]) + int(ctx[0])] >= 0).sum().item())
    torch.cuda.synchronize()
    r0, r1, r2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    r0.record(cs)
    for i, lay in enumerate(layers):
        R.check(abi.echo_release(dims, lay.struct, batch.struct, mask.data_ptr(),
                                 int(i == L - 1), ws.ws, cs.cuda_stream), "release")
    r1.record(cs)
    for i, lay in enumerate(layers):
        R.check(abi.echo_admit(dims, lay.struct, batch.struct, 0, int(base[0]), int(ctx[0]),
                               int(i == L - 1), ws.ws, cs.cuda_stream), "admit")
    r2.record(cs)
    torch.cuda.synchronize()
    D.status("release/admit")
    release_ms = r0.elapsed_time(r1) / L
    admit_ms = r1.elapsed_time(r2) / L
    log(f"[bench] release of one request ({int(ctx[0])} tokens, {resident0} resident on the "
        f"last layer): {release_ms * 1e3:.1f} us per layer; admission {admit_ms * 1e3:.1f} us "
        "per layer")

    # ------------------------------------------------------- CPU baselines
    cpu = cpu1 = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, ctx, base, layers[0], D.rows0, args, dims, threads=0)
        cpu1 = cpu_baseline(wl, ctx, base, layers[0], D.rows0, args, dims, threads=1)

    # --------------------------------- threshold ablation and prefetch-cap sweep
    ablation = sweep = None
    if not args.no_ablation:
        ablation = {args.mode: dict(layer_steps_per_s=round(layer_steps_per_s, 2),
                                    us_per_layer_step=round(step_ms * 1e3, 2), **timed)}
        for m in ("ema", "pos_inf", "neg_inf"):
            if m == args.mode:
                continue
            r = D.run(mode_of[m], args.steps, args.warmup, cs)
            ablation[m] = dict(layer_steps_per_s=round(r["layer_steps_per_s"], 2),
                               us_per_layer_step=round(r["us_per_layer_step"], 2),
                               **totals_summary(r["stats"], args.steps, row, link_peak,
                                                r["us_per_layer_step"]))
            log(f"[bench] {wl.name}, threshold {m}: {r['layer_steps_per_s']:.1f} layer-steps/s")
        ablation["ema_speedup_vs_pos_inf"] = round(
            ablation["ema"]["layer_steps_per_s"] / ablation["pos_inf"]["layer_steps_per_s"], 4)
        sweep = {str(wl.cap_div): dict(layer_steps_per_s=round(layer_steps_per_s, 2), **timed)}
        for cd in [int(x) for x in args.cap_sweep.split(",") if x.strip()]:
            if cd == wl.cap_div:
                continue
            r = D.run(mode, args.steps, args.warmup, cs, cap_div=cd)
            sweep[str(cd)] = dict(layer_steps_per_s=round(r["layer_steps_per_s"], 2),
                                  **totals_summary(r["stats"], args.steps, row, link_peak,
                                                   r["us_per_layer_step"]))
            log(f"[bench] {wl.name}, cap divisor {cd}: {r['layer_steps_per_s']:.1f} "
                f"layer-steps/s, {sweep[str(cd)]}")
    # -------------------------------- the same decode step with page tables
    paged = None
    if not args.no_paged:
        contiguous = D.batch
        D.batch = D.paged_batch(args.seed)
        r = D.run(mode, args.steps, args.warmup, cs)
        D.batch = contiguous
        paged = dict(layer_steps_per_s=round(r["layer_steps_per_s"], 2),
                     us_per_layer_step=round(r["us_per_layer_step"], 2),
                     vs_contiguous=round(r["layer_steps_per_s"] / layer_steps_per_s, 4),
                     **totals_summary(r["stats"], args.steps, row, link_peak,
                                      r["us_per_layer_step"]),
                     how="every request's 16-id pages scattered over the whole host pool "
                         "through a page table (echo_batch_t.page_table); the same data, "
                         "steps and timing as the headline")
        log(f"[bench] {wl.name} with page tables: {r['layer_steps_per_s']:.1f} layer-steps/s "
            f"({paged['vs_contiguous']:.3f} of contiguous)")
    D.close()
    del D, layers, ws, batch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    # ------------------------------------------------- the other decode workloads
    others = None
    if not args.no_other_workloads:
        others = {}
        for name in ("low_locality", "single_layer"):
            others[name] = other_workload(get(name), args, dev, cs, mode_of, link_peak)

    # ------------------------------------------------------- chunked prefill
    prefill = None if args.no_prefill else prefill_measure(args, dev)

    out = {
        "metric": "decode layer-steps/s @100K ctx; indexer HBM GB/s % peak; recall host-link GB/s",
        "value": round(layer_steps_per_s, 3),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8 MFMA (bf16 q split into two e4m3 terms) with fp32 accumulate; int32 "
                 "management",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: batch {B}, ctx U[{wl.ctx_lo},{wl.ctx_hi}], "
                               f"{L} layers in one hipGraph per step, indexer {wl.heads}x"
                               f"{wl.head_dim}, top-k {wl.top_k}, GPU pool {wl.n_gpu}/layer, "
                               f"host pool {wl.n_host} x {wl.latent} bf16, rho {wl.rho}",
                   "global_batch": B, "seq_len": int(ctx.max()), "layers": L,
                   "threshold_mode": args.mode, "prefetch_cap_div": wl.cap_div},
        "roofline": {"kernel": "lightning-indexer scoring kernel k_score<4,false> (prefetch "
                               f"off): a graph of {nso} echo_indexer_prefetch calls less a "
                               f"graph of their {nso} prologues, each the median of {nrep} "
                               "replays timed one at a time with events on the replay stream, "
                               "after 40 untimed replays",
                     "bound": "hbm", "achieved": round(ks_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(ks_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "bytes_per_launch": idx_bytes,
                     "avg_launch_ms": round(ks_ms, 5)},
        "scoring_in_step": in_step,
        "indexer_call": {"what": "echo_indexer_prefetch with prefetch off = k_begin + "
                                 f"k_score<4,false>, per call over {nso} calls back to back "
                                 f"in a graph, median of {nrep} replays",
                         "ms": round(so_ms, 5), "prologue_ms": round(begin_ms, 5),
                         "hbm_gbps": round(so_gbps, 1),
                         "frac_of_hbm_peak": round(so_gbps / HBM_PEAK_GBPS, 4)},
        "layer_step_link_roofline": {
            "bound": "host link", "link_bytes_per_layer_step": int(link_bytes),
            "floor_ms": round(link_floor_ms, 5), "measured_ms": round(step_ms, 5),
            "frac": round(link_floor_ms / step_ms, 4), "link_peak_gbps": round(link_peak, 2),
            "achieved_gbps": round(link_bytes / (step_ms * 1e-3) / 1e9, 2),
            "rows_from": "the layers' running totals over the timed replays"},
        "timed_replays": timed,
        "threshold_and_prefetch_usefulness": thr,
        "indexer_ema_standalone": {"avg_launch_ms": round(idx_ms, 5),
                                   "hbm_gbps": round(idx_gbps, 1),
                                   "note": "echo_indexer_prefetch alone also copies every "
                                           "prefetched row before it returns"},
        "indexer_hbm_gbps": round(so_gbps, 1),
        "recall_host_link_gbps": round(recall_gbps, 2),
        "recall_frac_of_link_peak": round(recall_gbps / link_peak, 4),
        "recall_measure": {"rows": rc_rows, "launch_ms": round(rc_ms, 5),
                           "how": f"echo_recall of the last layer-step's miss list, {nrc} "
                                  "launches back to back in a graph",
                           "eager_event_per_call_gbps": round(recall_eager_gbps, 2)},
        "host_link_peak_gbps": {"hipMemcpy_h2d": round(memcpy_gbps, 2),
                                "zero_copy_recall_kernel": round(zc_gbps, 2)},
        "phase_ms": {"indexer": round(idx_ms, 5), "topk": round(float(ph[:, 1].mean()), 5),
                     "alloc_evict": round(float(ph[:, 2].mean()), 5),
                     "recall": round(float(recall_ms.mean()), 5),
                     "how": "the five separate calls, eager, events between them"},
        "attention_input_gather": {"ms_per_layer": round(gather_ms, 5), "rows": n_sel_tot,
                                   "bytes": gather_bytes, "hbm_gbps": round(gather_gbps, 1),
                                   "frac_of_hbm_peak": round(gather_gbps / HBM_PEAK_GBPS, 4),
                                   "how": f"echo_gather, {ngr} calls back to back in a graph"},
        "append": {"ms_per_layer": round(append_ms, 5), "tokens": B,
                   "host_bytes": B * row, "hbm_bytes": B * wl.head_dim,
                   "how": f"echo_append on all {L} layers back to back in a graph, contexts "
                          "not advanced"},
        "lifecycle": {"release_ms_per_layer": round(release_ms, 5),
                      "admit_ms_per_layer": round(admit_ms, 5), "request_tokens": int(ctx[0]),
                      "resident_last_layer": resident0,
                      "how": f"echo_release then echo_admit of request 0 on all {L} layers, "
                             "eager, events on the launch stream"},
        "threshold_ablation": ablation,
        "prefetch_cap_sweep": sweep,
        "paged_step": paged,
        "other_workloads": others,
        "prefill": prefill,
        "hit_rate": timed["hit_rate"],
        "topk_shortcut_requests_last_layer": f"{shortcut_last}/{B}",
        "misses_per_layer_step": timed["misses_per_layer_step"],
        "prefetched_per_layer_step": timed["prefetched_per_layer_step"],
        "cpu_baseline": cpu,
        "cpu_baseline_single_thread": cpu1,
    }
    print(json.dumps(out), flush=True)


def threshold_and_usefulness(keep, L, steps, k, ctx):
    """From the eager breakdown steps: how far each layer's EMA threshold was from the
    step's k-th score, and what became of the prefetched tokens -- selected by the same
    step, by the next step only, or by neither."""
    th_err, same, nxt, pf_total, pf_checked = [], 0, 0, 0, 0
    per_layer = np.zeros(L)
    full = np.asarray(ctx) >= k
    for j, (th, kth, npf, pft, nsel, selt) in enumerate(keep):
        th, kth = th.cpu().numpy(), kth.cpu().numpy()
        ok = full & np.isfinite(th) & (np.abs(kth) > 0)
        if ok.any():
            e = np.abs(th[ok] - kth[ok]) / np.abs(kth[ok])
            th_err.append(float(e.mean()))
            per_layer[j % L] += float(e.mean()) / steps
        if j + L >= len(keep):
            continue  # no next step to look at
        npf, pft = npf.cpu().numpy(), pft.cpu().numpy()
        nsel, selt = nsel.cpu().numpy(), selt.cpu().numpy()
        nsel2, selt2 = keep[j + L][4].cpu().numpy(), keep[j + L][5].cpu().numpy()
        for b in range(npf.size):
            p = pft[b, : int(npf[b])]
            if p.size == 0:
                continue
            s1 = np.isin(p, selt[b, : int(nsel[b])])
            s2 = np.isin(p[~s1], selt2[b, : int(nsel2[b])])
            same += int(s1.sum())
            nxt += int(s2.sum())
            pf_checked += p.size
        pf_total += int(npf.sum())
    return {
        "threshold_rel_err_vs_kth_mean": round(float(np.mean(th_err)), 5) if th_err else None,
        "threshold_rel_err_layers_0_30_60": [round(float(per_layer[l]), 5)
                                             for l in (0, L // 2, L - 1) if l < L],
        "prefetched_checked": pf_checked,
        "selected_same_step_frac": round(same / max(1, pf_checked), 4),
        "selected_next_step_only_frac": round(nxt / max(1, pf_checked), 4),
        "selected_within_two_steps_frac": round((same + nxt) / max(1, pf_checked), 4),
        "how": "eager breakdown steps: |theta before the step - the step's k-th score| / k-th "
               "score, over requests with ctx >= k; each prefetched token of a step looked up "
               "in that step's selection and the next step's"}


def recall_in_graph(D, lay, nrc, cs):
    """The workspace's recall list (the last layer-step's misses) recalled `nrc` times
    back to back in a graph; returns (rows, ms per launch)."""
    import torch

    from kv_cache_offload_fp8_amd import abi
    from kv_cache_offload_fp8_amd import runtime as R
    rows = int(D.ws.counters[abi.ECHO_CNT_MISS].item())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for _ in range(nrc):
                R.check(abi.echo_recall(D.dims, lay.struct, D.ws.ws, cs.cuda_stream), "recall")
    g.replay()
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    g.replay()
    r1.record()
    torch.cuda.synchronize()
    return rows, r0.elapsed_time(r1) / nrc


def link_peaks(D, sh):
    """Pinned host -> device: hipMemcpy and the zero-copy recall kernel, in GB/s."""
    import torch

    from kv_cache_offload_fp8_amd import abi
    from kv_cache_offload_fp8_amd import runtime as R
    wl = D.wl
    row = wl.latent * 2
    n_rows = min(wl.n_host, 65536)
    dst = torch.empty((n_rows, wl.latent), dtype=torch.int16, device=D.dev)
    src = D.pools[0].tensor[:n_rows]
    for _ in range(2):
        dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    memcpy_gbps = 5 * n_rows * row / (e0.elapsed_time(e1) * 1e-3) / 1e9
    # zero-copy: echo_recall over a synthetic recall list of nz rows into layer 0's pool
    ws = D.ws
    nz = min(n_rows, D.B * wl.top_k, wl.n_gpu)
    ws.recall_h[:nz] = torch.arange(nz, dtype=torch.int32, device=D.dev)
    ws.recall_g[:nz] = torch.arange(nz, dtype=torch.int32, device=D.dev)
    ws.counters[abi.ECHO_CNT_MISS] = nz
    R.check(abi.echo_recall(D.dims, D.layers[0].struct, ws.ws, sh), "recall")
    e0.record()
    for _ in range(5):
        R.check(abi.echo_recall(D.dims, D.layers[0].struct, ws.ws, sh), "recall")
    e1.record()
    torch.cuda.synchronize()
    zc_gbps = 5 * nz * row / (e0.elapsed_time(e1) * 1e-3) / 1e9
    return memcpy_gbps, zc_gbps


def other_workload(wl, args, dev, cs, mode_of, link_peak):
    """One of the other decode workloads of the same path (one layer): EMA against
    prefetch off (threshold +inf) and -inf, each from a fresh layer, with the recall
    rate of one layer-step's misses in a graph."""
    import torch
    q_ring = args.warmup + args.steps
    D = Decode(wl, args, dev, 1, 1, q_ring)
    row = wl.latent * 2
    out = {"workload": f"{wl.name}: batch {D.B}, ctx {wl.ctx_lo}"
                       + (f"..{wl.ctx_hi}" if wl.ctx_hi != wl.ctx_lo else "")
                       + f", 1 layer, indexer {wl.heads}x{wl.head_dim}, top-k {wl.top_k}, "
                         f"GPU pool {wl.n_gpu}, host pool {wl.n_host}, rho {wl.rho}"}
    for m in ("ema", "pos_inf", "neg_inf"):
        r = D.run(mode_of[m], args.steps, args.warmup, cs)
        res = dict(layer_steps_per_s=round(r["layer_steps_per_s"], 2),
                   us_per_layer_step=round(r["us_per_layer_step"], 2),
                   **totals_summary(r["stats"], args.steps, row, link_peak,
                                    r["us_per_layer_step"]))
        nrc = 32
        rows, ms = recall_in_graph(D, D.layers[0], nrc, cs)
        if rows:
            res["recall_rows"] = rows
            res["recall_gbps"] = round(rows * row / (ms * 1e-3) / 1e9, 2)
            res["recall_frac_of_link_peak"] = round(res["recall_gbps"] / link_peak, 4)
        out[m] = res
        log(f"[bench] {wl.name}, threshold {m}: {res}")
    out["ema_speedup_vs_pos_inf"] = round(out["ema"]["layer_steps_per_s"] /
                                          out["pos_inf"]["layer_steps_per_s"], 4)
    D.close()
    torch.cuda.synchronize()
    return out


def prefill_measure(args, dev):
    """Chunked prefill on the prefill workload (one request, 100,000-token history,
    64 x 128 indexer, top-2048 per query, 200,000 GPU slots, 2M host tokens), for each
    query-chunk size: the chunk pipeline with the copies on a second stream (the early
    candidates' copy overlaps the exact selection and the next chunk's scoring) against
    the same calls run one after another on one stream, from a cold GPU pool; and the
    scoring call's fp8 MFMA rate (algorithmic 2*C*N*H*D flop per chunk)."""
    import torch

    from kv_cache_offload_fp8_amd import abi
    from kv_cache_offload_fp8_amd import runtime as R
    from synth import gen as G
    from synth import get
    from synth.configs import PREFILL_CHUNKS

    wl = get("prefill")
    N, chunks = wl.ctx_lo, max(2, args.prefill_chunks)
    dims = R.make_dims(wl.heads, wl.head_dim, wl.top_k, wl.n_host, wl.n_gpu, 1, N, wl.latent,
                       wl.alpha, wl.cap_div, 1)
    ctx = np.array([N], np.int32)
    base = G.host_layout(ctx)
    host = R.HostPool(wl.n_host, wl.latent)
    lat = G.gen_latents(wl, 0, ctx, base, dev, args.seed,
                        out=torch.empty((wl.n_host, wl.latent), dtype=torch.int16, device=dev))
    host.tensor.copy_(lat)
    del lat
    rows = G.gen_kidx(wl, 0, ctx, base, dev, args.seed)
    kidx = R.pack_kidx(dims, rows, torch.empty_like(rows))
    del rows
    layer = R.Layer(dims, kidx, host, 1, dev)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    out = {"workload": f"prefill: 1 request, history {N}, 64x128, k {wl.top_k}, "
                       f"{wl.n_gpu} GPU slots, {wl.n_host} host tokens, {chunks} chunks",
           "chunks": {}}
    for C in PREFILL_CHUNKS:
        q, w = G.gen_prefill_qw(wl, 0, C, chunks, dev, args.seed)
        pws = R.PrefillWorkspace(dims, C, dev)
        structs = [abi.echo_prefill_chunk_t(C, int(base[0]), N, q[c].data_ptr(), w[c].data_ptr(),
                                            pws.kth.data_ptr() if c else None)
                   for c in range(chunks)]

        def call(fn, c, st):
            R.check(fn(dims, layer.struct, structs[c], pws.ws, st.cuda_stream), fn.__name__)

        def copy(which, st):
            R.check(abi.echo_prefill_copy(dims, layer.struct, pws.ws, which, st.cuda_stream),
                    "echo_prefill_copy")

        def fresh():
            torch.cuda.synchronize()
            layer.init()
            pws.reset()
            torch.cuda.synchronize()

        def run(overlap, stats=None):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            ea = eb = None
            e0.record(s1)
            for c in range(chunks):
                call(abi.echo_prefill_score, c, s1)
                if overlap and ea is not None:
                    s1.wait_event(ea)
                call(abi.echo_prefill_early, c, s1)
                if overlap:
                    ev = torch.cuda.Event()
                    ev.record(s1)
                    s2.wait_event(ev)
                    copy(0, s2)
                    ea = torch.cuda.Event()
                    ea.record(s2)
                    if eb is not None:
                        s1.wait_event(eb)
                call(abi.echo_prefill_select, c, s1)
                if overlap:
                    ev = torch.cuda.Event()
                    ev.record(s1)
                    s2.wait_event(ev)
                    copy(1, s2)
                    eb = torch.cuda.Event()
                    eb.record(s2)
                else:
                    copy(0, s1)
                    copy(1, s1)
                if stats is not None:
                    torch.cuda.synchronize()
                    cnt = pws.counts.cpu().numpy()
                    stats.append([int(cnt[abi.ECHO_PF_CNT_UNION]), int(cnt[abi.ECHO_PF_CNT_CAND]),
                                  int(cnt[abi.ECHO_PF_CNT_EARLY]), int(cnt[abi.ECHO_PF_CNT_LATE])])
            if overlap:
                s1.wait_event(eb)
            e1.record(s1)
            torch.cuda.synchronize()
            st = int(pws.status.item())
            if st != 0:
                raise SystemExit(f"prefill status {abi.echo_status_string(st)}")
            return e0.elapsed_time(e1)

        stats = []
        fresh()
        run(True, stats)          # untimed: counts per chunk
        fresh()
        run(True)                 # warm the code paths
        times = {}
        for overlap in (True, False):
            fresh()
            times[overlap] = run(overlap)
        # the scoring call alone (stage, MFMA scores, coarse pass, candidate list)
        fresh()
        es, ee = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 4
        es.record(s1)
        for _ in range(reps):
            call(abi.echo_prefill_score, 1, s1)
        ee.record(s1)
        torch.cuda.synchronize()
        score_ms = es.elapsed_time(ee) / reps
        flop = 2.0 * C * N * wl.heads * wl.head_dim
        tflops = flop / (score_ms * 1e-3) / 1e12
        rows_moved = sum(x[2] + x[3] for x in stats)
        out["chunks"][str(C)] = {
            "ms_per_chunk_overlapped": round(times[True] / chunks, 4),
            "ms_per_chunk_serial": round(times[False] / chunks, 4),
            "overlap_speedup": round(times[False] / times[True], 4),
            "score_call_ms": round(score_ms, 4),
            "score_call_tflops_algorithmic": round(tflops, 1),
            "score_call_frac_of_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
            "rows_over_host_link": rows_moved,
            "per_chunk_union_cand_early_late": stats}
        log(f"[bench] prefill C={C}: {times[True] / chunks:.3f} ms/chunk with the copies "
            f"overlapped, {times[False] / chunks:.3f} serial ({times[False] / times[True]:.3f}x); "
            f"scoring call {score_ms:.3f} ms = {tflops:.0f} TFLOP/s algorithmic "
            f"({tflops / FP8_PEAK_TFLOPS:.1%} of fp8 peak); union/cand/early/late {stats}")
        del pws, q, w
    host.close()
    return out


def cpu_baseline(wl, ctx, base, lay0, rows0, args, dims, threads=0):
    """The oracle, as it stands, on a bounded sample: layer 0 of the same workload,
    the first `--cpu-sample-requests` requests, `--cpu-sample-steps` decode steps in
    EMA mode (its own scores), on every host thread (threads=0) or on `threads`.
    Reported as layer-steps/s, scaled by the share of the layer-step's scored tokens
    the sample covers.  One thread takes a smaller sample (8 requests, 6 steps: about
    10 s of CPU time)."""
    import torch

    from oracle import oracle as O
    from synth import gen as G

    nb = max(1, min(args.cpu_sample_requests, ctx.size))
    steps = max(1, min(args.cpu_sample_steps, lay0.q.shape[0]))
    if threads == 1:
        nb, steps = min(nb, 8), min(steps, 6)
    sctx = ctx[:nb].astype(np.int32)
    sbase = G.host_layout(sctx)
    n = int(sctx.sum())
    n_rows = (int(sbase[-1]) + int(sctx[-1]) + 15) // 16 * 16
    kid = np.zeros((n_rows, wl.head_dim), np.uint8)
    for b in range(nb):
        kid[sbase[b]:sbase[b] + sctx[b]] = rows0[int(base[b]):int(base[b]) + int(sctx[b])].cpu() \
            .numpy()
    qs = lay0.q[:steps, :nb].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    w0 = lay0.w[:nb].cpu().numpy()
    orc = O.OracleLayer(wl.heads, wl.head_dim, wl.top_k, wl.latent, n_rows, wl.n_gpu, nb,
                        wl.cap_div, wl.alpha, keep_pool=False)
    prev = O.set_threads(threads) if threads else None
    used = threads or int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    t0 = time.perf_counter()
    for t in range(steps):
        o = orc.step(sbase, sctx, qs[t], w0, kid, None, mode=O.MODE_EMA)
        assert o["status"] == O.OK
    dt = time.perf_counter() - t0
    if prev:
        O.set_threads(prev)
    threads = used
    frac = n / float(ctx.sum())
    per_layer_step = dt / steps / frac
    log(f"[bench] cpu oracle: {steps} steps x {nb} requests ({n} tokens each) in {dt:.2f}s on "
        f"{threads} threads -> {per_layer_step:.2f}s per full layer-step")
    return {"value": round(1.0 / per_layer_step, 6), "unit": "layer-steps/s", "cores": threads,
            "kind": "oracle",
            "sample": f"layer 0, decode steps 0..{steps - 1} in EMA mode, {nb} of {ctx.size} "
                      f"requests ({n} scored tokens per step, {frac:.1%} of the layer-step's "
                      f"tokens), {dt:.1f} s of CPU time; scaled by tokens"}


if __name__ == "__main__":
    main()
