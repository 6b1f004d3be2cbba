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


def replay_median_ms(graph, n):
    """Median duration of n replays of `graph`, each timed with events on the current
    stream after the previous one has finished."""
    import torch
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
    from synth import gen as G

    torch.cuda.set_device(0)
    dev = "cuda"
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_measure(args, dev)}), flush=True)
        return
    wl = get(args.workload)
    if args.cap_div:
        wl = wl.scaled(cap_div=args.cap_div)
    L = args.layers or wl.layers
    mode = {"ema": abi.ECHO_THETA_EMA, "neg_inf": abi.ECHO_THETA_NEG_INF,
            "pos_inf": abi.ECHO_THETA_POS_INF}[args.mode]
    ctx = wl.contexts(args.seed)
    base = G.host_layout(ctx, room=1)  # one free row per request: the append measurement
    B = int(ctx.size)
    total_tok = int(ctx.sum())
    q_ring = args.warmup + args.steps + args.breakdown_steps
    dims = R.make_dims(wl.heads, wl.head_dim, wl.top_k, wl.n_host, wl.n_gpu, B,
                       int(ctx.max()) + 1, wl.latent, wl.alpha, wl.cap_div, q_ring)
    log(f"[bench] workload {wl.name}: B={B} ctx {ctx.min()}..{ctx.max()} (sum {total_tok}) "
        f"L={L} n_gpu={wl.n_gpu} n_host={wl.n_host} q_ring={q_ring}")

    # ---------------------------------------------------------------- setup
    t0 = time.time()
    npools = max(1, min(args.host_pools, L))
    pools = []
    for i in range(npools):
        hp = R.HostPool(wl.n_host, wl.latent)
        lat = G.gen_latents(wl, i, ctx, base, dev, args.seed,
                            out=torch.empty((wl.n_host, wl.latent), dtype=torch.int16,
                                            device=dev))
        hp.tensor.copy_(lat)
        del lat
        pools.append(hp)
    log(f"[bench] {npools} host pools of {wl.n_host * wl.latent * 2 / 1e9:.2f} GB ready "
        f"({time.time() - t0:.1f}s)")
    layers = []
    rows = torch.empty((wl.n_host, wl.head_dim), dtype=torch.uint8, device=dev)
    rows0 = None  # layer 0's row-major K, for the CPU baseline
    for l in range(L):
        rows.zero_()
        G.gen_kidx(wl, l, ctx, base, dev, args.seed, out=rows)
        if l == 0:
            rows0 = rows.clone()
        kidx = R.pack_kidx(dims, rows, torch.empty_like(rows))
        lay = R.Layer(dims, kidx, pools[l % npools], B, dev)
        lay.q.copy_(G.gen_q(wl, l, B, q_ring, dev, args.seed))
        lay.w.copy_(G.gen_w(wl, l, B, dev, args.seed))
        lay.init()
        layers.append(lay)
    del rows
    batch = R.Batch(base, ctx, dev)
    ws = R.Workspace(dims, dev)
    ws.reset()
    torch.cuda.synchronize()
    log(f"[bench] {L} layers ready ({time.time() - t0:.1f}s); meta/layer "
        f"{layers[0].meta_bytes()} B = echo_meta_bytes {abi.echo_meta_bytes(wl.n_host, wl.n_gpu)}")

    def one_step(stream):
        for lay in layers:
            R.check(abi.echo_layer_step(dims, lay.struct, batch.struct, ws.ws, mode, stream),
                    "echo_layer_step")

    # ------------------------------------------------------- graph capture
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            one_step(cs.cuda_stream)
    torch.cuda.synchronize()
    log("[bench] captured one decode step "
        f"({L} layers) in a graph; warmup {args.warmup}")
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    st = int(ws.status.item())
    if st != 0:
        raise SystemExit(f"device status after warmup: {abi.echo_status_string(st)}")

    # -------------------------------------------------------- timed region
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = ev0.elapsed_time(ev1)
    elapsed = max(wall, gpu_ms / 1e3)
    st = int(ws.status.item())
    if st != 0:
        raise SystemExit(f"device status after timed steps: {abi.echo_status_string(st)}")
    shortcut_last = int(ws.counters[abi.ECHO_CNT_SHORTCUT].item())
    ms_per_step = elapsed * 1e3 / args.steps
    layer_steps_per_s = args.steps * L / elapsed
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step, "
        f"{layer_steps_per_s:.1f} layer-steps/s")

    # ------------------------------------------- per-phase breakdown (eager)
    s = torch.cuda.current_stream()
    sh = s.cuda_stream
    nph = 4
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)]
           for _ in range(args.breakdown_steps * L)]
    miss_rows, sel_rows, pf_rows, sc_rows = [], [], [], []
    i = 0
    for _ in range(args.breakdown_steps):
        for lay in layers:
            e = evs[i]
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
            c = ws.counters.clone()
            miss_rows.append(c[abi.ECHO_CNT_MISS])
            pf_rows.append(c[abi.ECHO_CNT_PREFETCH])
            sc_rows.append(c[abi.ECHO_CNT_SHORTCUT])
            sel_rows.append(ws.n_sel[:B].sum())
            i += 1
    torch.cuda.synchronize()
    st = int(ws.status.item())
    if st != 0:
        raise SystemExit(f"device status after breakdown: {abi.echo_status_string(st)}")
    ph = np.array([[evs[j][p].elapsed_time(evs[j][p + 1]) for p in range(nph)]
                   for j in range(len(evs))])  # ms
    misses = np.array([int(x) for x in miss_rows])
    prefetched = np.array([int(x) for x in pf_rows])
    selected = np.array([int(x) for x in sel_rows])
    idx_ms = float(ph[:, 0].mean())
    idx_bytes = total_tok * BYTES_PER_SCORED_TOKEN
    idx_gbps = idx_bytes / (idx_ms * 1e-3) / 1e9
    row = wl.latent * 2
    recall_ms = ph[:, 3]
    recall_eager_gbps = float((misses * row).sum() / (recall_ms.sum() * 1e-3) / 1e9)
    # Recall rate as the step runs it, back to back in a graph: the last layer's
    # miss list (still in the workspace) recalled `nrc` times into its pool (the
    # same rows to the same slots each time), timed with events around one replay.
    nrc = 32
    rc_rows = int(ws.counters[abi.ECHO_CNT_MISS].item())
    grc = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(grc, stream=cs):
            for _ in range(nrc):
                R.check(abi.echo_recall(dims, layers[-1].struct, ws.ws, cs.cuda_stream),
                        "recall")
    grc.replay()
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record()
    grc.replay()
    r1.record()
    torch.cuda.synchronize()
    rc_ms = r0.elapsed_time(r1) / nrc
    recall_gbps = rc_rows * row / (rc_ms * 1e-3) / 1e9
    del grc
    hit = float(1.0 - misses.sum() / max(1, selected.sum()))
    log(f"[bench] phases (ms, mean over {len(evs)} layer-steps): indexer {idx_ms:.4f} "
        f"topk {ph[:, 1].mean():.4f} alloc/evict {ph[:, 2].mean():.4f} "
        f"recall {recall_ms.mean():.4f}; hit rate {hit:.4f}; misses/layer-step "
        f"{misses.mean():.0f}; prefetched/layer-step {prefetched.mean():.0f}")
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
    n_rows = min(wl.n_host, 65536)
    big = pools[0]
    dst = torch.empty((n_rows, wl.latent), dtype=torch.int16, device=dev)
    src = big.tensor[:n_rows]
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
    # zero-copy: echo_recall over a synthetic recall list of n_rows rows into layer 0's pool
    nz = min(n_rows, B * wl.top_k, wl.n_gpu)
    ws.recall_h[:nz] = torch.arange(nz, dtype=torch.int32, device=dev)
    ws.recall_g[:nz] = torch.arange(nz, dtype=torch.int32, device=dev)
    ws.counters[abi.ECHO_CNT_MISS] = nz
    R.check(abi.echo_recall(dims, layers[0].struct, ws.ws, sh), "recall")
    e0.record()
    for _ in range(5):
        R.check(abi.echo_recall(dims, layers[0].struct, ws.ws, sh), "recall")
    e1.record()
    torch.cuda.synchronize()
    zc_gbps = 5 * nz * row / (e0.elapsed_time(e1) * 1e-3) / 1e9
    link_peak = max(memcpy_gbps, zc_gbps)
    log(f"[bench] host link: hipMemcpy H2D {memcpy_gbps:.1f} GB/s, zero-copy recall kernel "
        f"{zc_gbps:.1f} GB/s over {nz} rows")

    # layer-step floor: every prefetched and missed row crosses the host link once
    step_ms = ms_per_step / L
    link_bytes = (float(prefetched.mean()) + float(misses.mean())) * row
    link_floor_ms = link_bytes / (link_peak * 1e9) * 1e3
    traffic = stored_traffic()
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
                R.check(abi.echo_append(dims, lay.struct, batch.host_base.data_ptr(),
                                        batch.ctx.data_ptr(), B, k_new.data_ptr(),
                                        lat_new.data_ptr(), ws.ws, 0, cs.cuda_stream), "append")
    gap.replay()
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record()
    gap.replay()
    a1.record()
    torch.cuda.synchronize()
    st = int(ws.status.item())
    if st != 0:
        raise SystemExit(f"device status after append: {abi.echo_status_string(st)}")
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
        R.check(abi.echo_release(dims, lay.struct, batch.host_base.data_ptr(),
                                 batch.ctx.data_ptr(), B, mask.data_ptr(), int(i == L - 1),
                                 ws.ws, cs.cuda_stream), "release")
    r1.record(cs)
    for i, lay in enumerate(layers):
        R.check(abi.echo_admit(dims, lay.struct, batch.host_base.data_ptr(),
                               batch.ctx.data_ptr(), B, 0, int(base[0]), int(ctx[0]),
                               int(i == L - 1), ws.ws, cs.cuda_stream), "admit")
    r2.record(cs)
    torch.cuda.synchronize()
    st = int(ws.status.item())
    if st != 0:
        raise SystemExit(f"device status after release/admit: {abi.echo_status_string(st)}")
    release_ms = r0.elapsed_time(r1) / L
    admit_ms = r1.elapsed_time(r2) / L
    log(f"[bench] release of one request ({int(ctx[0])} tokens, {resident0} resident on the "
        f"last layer): {release_ms * 1e3:.1f} us per layer; admission {admit_ms * 1e3:.1f} us "
        "per layer")

    # ------------------------------------------------------- chunked prefill
    prefill = None if args.no_prefill else prefill_measure(args, dev)

    # ------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, ctx, base, layers[0], rows0, args, dims)

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
                   "threshold_mode": args.mode},
        "roofline": {"kernel": "lightning-indexer scoring kernel k_score<4,false> (prefetch "
                               f"off): a graph of {nso} echo_indexer_prefetch calls less a "
                               f"graph of their {nso} prologues, each the median of {nrep} "
                               "replays timed one at a time with events on the replay stream",
                     "bound": "hbm", "achieved": round(ks_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(ks_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "bytes_per_launch": idx_bytes,
                     "avg_launch_ms": round(ks_ms, 5)},
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
            "achieved_gbps": round(link_bytes / (step_ms * 1e-3) / 1e9, 2)},
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
                     "recall": round(float(recall_ms.mean()), 5)},
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
        "prefill": prefill,
        "hit_rate": round(hit, 5),
        "topk_shortcut_requests_last_layer": f"{shortcut_last}/{B}",
        "misses_per_layer_step": round(float(misses.mean()), 1),
        "prefetched_per_layer_step": round(float(prefetched.mean()), 1),
        "cpu_baseline": cpu,
    }
    for hp in pools:
        hp.close()
    print(json.dumps(out), flush=True)


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


def cpu_baseline(wl, ctx, base, lay0, rows0, args, dims):
    """The oracle, as it stands, on a bounded sample: layer 0 of the same workload,
    the first `--cpu-sample-requests` requests, `--cpu-sample-steps` decode steps in
    EMA mode (its own scores).  Reported as layer-steps/s, scaled by the share of the
    layer-step's scored tokens the sample covers."""
    import torch

    from oracle import oracle as O
    from synth import gen as G

    nb = max(1, min(args.cpu_sample_requests, ctx.size))
    steps = max(1, min(args.cpu_sample_steps, lay0.q.shape[0]))
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
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    t0 = time.perf_counter()
    for t in range(steps):
        o = orc.step(sbase, sctx, qs[t], w0, kid, None, mode=O.MODE_EMA)
        assert o["status"] == O.OK
    dt = time.perf_counter() - t0
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
