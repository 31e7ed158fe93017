#!/usr/bin/env python3
"""Benchmark of the FP4 sparse-indexer hot path on one MI355X.

A step is one decode step of the indexer over 21 layers at batch 8 x context 131072 (64
index heads x 128, index_topk 2048): the decode schedule is published once, then every
layer writes its 8 new keys and quantizes its queries with the fused writer (key LayerNorm,
RoPE on keys and query heads, MXFP4 write, weights_mqa: indexer_fp4_norm_rope_quant_and_cache),
scores all keys (indexer_fp4_score_decode) and selects the top-k (indexer_topk); --fused-write
runs the writer's work inside the scorer instead (indexer_fp4_write_and_score_decode, one
launch). Each layer
has its own key cache (21 x 78 MB), so the scan streams from HBM instead of the 256 MB
last-level cache. The pages' indexer has 21 layers ("Score a DSA sparse indexer in FP4",
PR description: 21 layers x 5.8 us of grid overhead a step).

Steps run as replays of a HIP graph captured from the library calls (the calls are
capturable: fixed grids, lengths read on the device, no host reads or allocations), as a
serving engine would run them. Printed: one JSON line with the throughput (keys scored per
second over whole steps), the roofline of the step's scoring kernel (algorithmic bytes per
launch over its mean launch time: HIP events around replays of a graph holding the step's 21
scoring launches), the same figures per layer for the long decode workloads (16 x 131072 and
8 x 262144, 8 layers each), the prefill path's time per layer and FP4 MFMA roofline (4
requests of 3420..4213 tokens, 512-token chunks; and the same requests as a stream of steps
of at most 512 tokens in all), and the CPU oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MXFP4
ROPE_DIM = 64                  # rotated leading elements of each 128-element key / query head
WEIGHT_SCALE = (128 * 64) ** -0.5  # softmax scale 128^-1/2 times heads^-1/2
METRIC = "indexer keys scored/sec + µs/layer decode & prefill; % HBM / MFMA roofline"


def kernel_source_hash(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_attention_indexer_fp4_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_scorer_bytes(n_keys: int, n_pages: int, rows: int, heads: int) -> int:
    """Algorithmic HBM bytes of one decode-scorer launch: every key's 64 packed + 4 scale
    bytes read once and its fp32 logit written once; one block-table entry per page; per
    row the quantized query (64 + 4 bytes per head), its fp32 head weights and its length."""
    return n_keys * (64 + 4 + 4) + n_pages * 4 + rows * (heads * (64 + 4) + heads * 4 + 4)


def decode_write_score_bytes(n_keys: int, n_pages: int, rows: int, heads: int) -> int:
    """Algorithmic HBM bytes of one write-and-score launch: the scorer's keys, table entries,
    logits and lengths as above, and per row the writer's inputs instead of the quantized
    query: the bf16 query heads, the fp32 weights, the bf16 new key, its position, slot and
    rotary table row, and the new key's 68 cache bytes written."""
    return (n_keys * (64 + 4 + 4) + n_pages * 4 +
            rows * (heads * 256 + heads * 4 + 4 + 256 + 8 + 8 + 4 * ROPE_DIM + 68))


def build_decode(torch, ifp4, W, layers, units, seed, fp8=False, workload="decode_b8_128k", contexts=None):
    """The layers of a decode workload of equal contexts (the named workload's, or `contexts`
    with its heads and top-k); with fp8, every layer also gets MXFP8 planes of the same keys
    and queries (the FP8 comparator)."""
    dev = torch.device("cuda:0")
    case_ctx = W.DECODE_CONFIGS[workload]
    ctx = np.array(case_ctx["ctx"] if contexts is None else contexts, np.int32)
    H, k = case_ctx["heads"], case_ctx["topk"]
    B = ctx.shape[0]
    rng = np.random.default_rng(seed)
    # one shuffled block table shared by the layers (each layer has its own cache buffers)
    pages_per = (ctx + 63) // 64
    need = int(pages_per.sum())
    n_pages = need + need // 10
    perm = rng.permutation(n_pages).astype(np.int32)
    bt = perm[:need].reshape(B, -1)
    bt_t = torch.from_numpy(bt).to(dev)
    slots_all = (bt.astype(np.int64)[:, :, None] * 64 + np.arange(64)).reshape(B, -1)
    slots_all_t = torch.from_numpy(slots_all.reshape(-1).copy()).to(dev)
    new_slots = torch.from_numpy(slots_all[np.arange(B), ctx - 1].copy()).to(dev)
    gen = torch.Generator(device=dev)
    L = []
    for layer in range(layers):
        gen.manual_seed(seed * 1000 + layer)
        kp = torch.empty((n_pages, 64, 64), dtype=torch.uint8, device=dev)
        ks = torch.empty((n_pages, 4, 64), dtype=torch.uint8, device=dev)
        keys = torch.randn((B * int(ctx[0]), 128), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        ifp4.indexer_fp4_quant_and_cache(keys, slots_all_t, kp, ks)
        extra = {}
        if fp8:
            extra["kp8"] = torch.empty((n_pages, 64, 128), dtype=torch.uint8, device=dev)
            extra["ks8"] = torch.empty((n_pages, 4, 64), dtype=torch.uint8, device=dev)
            ifp4.indexer_fp8_quant_and_cache(keys, slots_all_t, extra["kp8"], extra["ks8"])
        del keys
        q = torch.randn((B, H, 128), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        if fp8:
            extra["qp8"] = torch.empty((B, H, 128), dtype=torch.uint8, device=dev)
            extra["qs8"] = torch.empty((B, H, 4), dtype=torch.uint8, device=dev)
            ifp4.indexer_fp8_quant_and_cache(None, None, extra["kp8"], extra["ks8"], q, extra["qp8"], extra["qs8"])
        w = torch.rand((B, H), generator=gen, device=dev, dtype=torch.float32)
        knew = torch.randn((B, 128), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
        gamma = torch.rand(128, generator=gen, device=dev, dtype=torch.float32) + 0.5
        beta = (torch.rand(128, generator=gen, device=dev, dtype=torch.float32) - 0.5) * 0.4
        L.append(dict(kp=kp, ks=ks, q=q, w=w, knew=knew, gamma=gamma, beta=beta, **extra,
                      wm=torch.empty((B, H), dtype=torch.float32, device=dev),
                      qp=torch.empty((B, H, 64), dtype=torch.uint8, device=dev),
                      qs=torch.empty((B, H, 4), dtype=torch.uint8, device=dev)))
    ld = bt.shape[1] * 64
    shared = dict(
        ctx=torch.from_numpy(ctx).to(dev), bt=bt_t, new_slots=new_slots,
        # rotary table over the context and the new tokens' positions
        cos_sin=torch.from_numpy(W.rope_table(int(ctx.max()), ROPE_DIM)).to(dev),
        positions=torch.from_numpy((ctx - 1).astype(np.int64)).to(dev),
        sched=torch.empty(ifp4.indexer_fp4_decode_sched_bytes(B, 1, units), dtype=torch.uint8, device=dev),
        row_len=torch.empty(B, dtype=torch.int32, device=dev),
        logits=torch.empty((B, ld), dtype=torch.float32, device=dev),
        top=torch.empty((B, k), dtype=torch.int32, device=dev),
        ws=torch.zeros(max(ifp4.indexer_topk_workspace_bytes(B, ld, k), 1), dtype=torch.uint8, device=dev),
        # first-digit histograms: filled by each layer's scorer, consumed and re-zeroed by its top-k
        hist=ifp4.row_histogram(B, dev),
        hist_scorer=ifp4.row_histogram(B, dev),  # the scorer-only graph's (never read)
    )
    torch.cuda.synchronize()
    meta = dict(B=B, H=H, k=k, ctx=int(ctx[0]), n_keys=int(ctx.astype(np.int64).sum()), n_pages_read=need,
                ld=ld, units=units, separate_writer=True)
    return L, shared, meta


def decode_step(ifp4, L, S, meta):
    """One decode step over all layers: schedule once, then per layer write + score (one launch,
    or two with separate_writer) and select."""
    units, ld, k = meta["units"], meta["ld"], meta["k"]
    ifp4.indexer_fp4_decode_schedule(S["ctx"], 1, units, S["sched"], S["row_len"])
    for lay in L:
        if meta["separate_writer"]:
            write_decode(ifp4, lay, S)
            ifp4.indexer_fp4_score_decode(lay["qp"], lay["qs"], lay["wm"], lay["kp"], lay["ks"], S["bt"], 1,
                                          S["sched"], units, S["row_len"], S["logits"], S["hist"])
        else:
            write_and_score(ifp4, lay, S, meta, S["hist"])
        ifp4.indexer_topk(S["logits"], S["row_len"], ld, k, S["top"], S["ws"], S["hist"])


def write_and_score(ifp4, lay, S, meta, hist):
    """A layer's fused write and its scores in one launch."""
    ifp4.indexer_fp4_write_and_score_decode(
        lay["knew"], S["new_slots"], lay["kp"], lay["ks"], lay["q"], lay["w"], S["bt"], S["sched"], meta["units"],
        S["row_len"], S["logits"], positions=S["positions"], cos_sin=S["cos_sin"], rope_dim=ROPE_DIM,
        k_norm_weight=lay["gamma"], k_norm_bias=lay["beta"], eps=1e-6, weight_scale=WEIGHT_SCALE, row_hist=hist)


def write_decode(ifp4, lay, S):
    """The layer's fused write: the new keys normalized, rotated and cached, the query heads
    rotated and quantized, the head weights scaled (softmax scale times heads^-1/2)."""
    ifp4.indexer_fp4_norm_rope_quant_and_cache(
        lay["knew"], S["new_slots"], lay["kp"], lay["ks"], positions=S["positions"], cos_sin=S["cos_sin"],
        rope_dim=ROPE_DIM, k_norm_weight=lay["gamma"], k_norm_bias=lay["beta"], eps=1e-6, q=lay["q"],
        q_packed=lay["qp"], q_scale=lay["qs"], weights=lay["w"], weight_scale=WEIGHT_SCALE, weights_mqa=lay["wm"])


def decode_scorers(ifp4, L, S, meta, plain=False):
    """The step's 21 scoring launches alone (one per layer cache), histogram included: the
    kernel the step runs (write-and-score), or with plain the scorer on quantized rows."""
    for lay in L:
        if plain or meta["separate_writer"]:
            ifp4.indexer_fp4_score_decode(lay["qp"], lay["qs"], lay["wm"], lay["kp"], lay["ks"], S["bt"], 1,
                                          S["sched"], meta["units"], S["row_len"], S["logits"], S["hist_scorer"])
        else:
            write_and_score(ifp4, lay, S, meta, S["hist_scorer"])


def capture(torch, fn):
    """Capture fn() into a HIP graph (after one run on the capture side stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def timed_replays(torch, g, reps):
    """Milliseconds per replay, HIP events on the replay stream, synchronized on both sides."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def scoring_bytes(meta):
    """Algorithmic bytes of the kernel decode_scorers times."""
    f = decode_scorer_bytes if meta["separate_writer"] else decode_write_score_bytes
    return f(meta["n_keys"], meta["n_pages_read"], meta["B"], meta["H"])


def bench_decode(torch, ifp4, W, args):
    L, S, meta = build_decode(torch, ifp4, W, args.layers, args.units, args.seed)
    meta["separate_writer"] = not args.fused_write
    for lay in L:  # the quantized rows the plain scorer reads
        write_decode(ifp4, lay, S)
    for _ in range(args.warmup):
        decode_step(ifp4, L, S, meta)
    torch.cuda.synchronize()
    if ifp4.sched_error(S["sched"]) != 0:
        raise RuntimeError(f"device error flags {ifp4.sched_error(S['sched'])}")
    step_graph = capture(torch, lambda: decode_step(ifp4, L, S, meta))
    for _ in range(args.warmup):
        step_graph.replay()
    wall0 = time.perf_counter()
    ms_per_step = timed_replays(torch, step_graph, args.steps)
    wall = time.perf_counter() - wall0
    # the dominant kernel alone: 21 scoring launches per replay, averaged over the replays
    scorer_graph = capture(torch, lambda: decode_scorers(ifp4, L, S, meta))
    scorer_graph.replay()
    scorer_us = 1e3 * timed_replays(torch, scorer_graph, args.steps) / args.layers
    plain_scorer_us = scorer_us
    if not meta["separate_writer"]:  # the scorer on quantized rows, beside the writing one
        plain_scorer_graph = capture(torch, lambda: decode_scorers(ifp4, L, S, meta, plain=True))
        plain_scorer_graph.replay()
        plain_scorer_us = 1e3 * timed_replays(torch, plain_scorer_graph, args.steps) / args.layers
    # the step's other per-layer kernel: the fused writer (and the plain writer beside it)
    writer_graph = capture(torch, lambda: [write_decode(ifp4, lay, S) for lay in L])
    writer_us = 1e3 * timed_replays(torch, writer_graph, args.steps) / args.layers
    plain_graph = capture(torch, lambda: [ifp4.indexer_fp4_quant_and_cache(
        lay["knew"], S["new_slots"], lay["kp"], lay["ks"], lay["q"], lay["qp"], lay["qs"]) for lay in L])
    plain_us = 1e3 * timed_replays(torch, plain_graph, args.steps) / args.layers
    for lay in L:  # leave the fused write's outputs in place
        write_decode(ifp4, lay, S)
    keys_per_step = meta["n_keys"] * args.layers
    alg_bytes = scoring_bytes(meta)
    achieved = alg_bytes / (scorer_us * 1e-6) / 1e9
    plain_bytes = decode_scorer_bytes(meta["n_keys"], meta["n_pages_read"], meta["B"], meta["H"])
    return dict(meta=meta, ms_per_step=ms_per_step, wall_s=wall, keys_per_s=keys_per_step / (ms_per_step * 1e-3),
                scorer_us=scorer_us, alg_bytes=alg_bytes, achieved_gbs=achieved,
                plain_scorer={"us": round(plain_scorer_us, 3), "alg_bytes_per_launch": plain_bytes,
                              "frac": round(plain_bytes / (plain_scorer_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)},
                writer={"fused_us_per_layer": round(writer_us, 3), "plain_us_per_layer": round(plain_us, 3),
                        "tokens": meta["B"], "heads": meta["H"], "rope_dim": ROPE_DIM})


SWEEP_WORKLOADS = ("decode_b16_128k", "decode_b8_256k")


def bench_decode_sweep(torch, ifp4, W, args, layers=8):
    """The long decode workloads, 16 x 131072 and 8 x 262144 (64 heads, top-2048): whole
    steps (schedule, then per layer fused write + score + top-k) and the scorer alone, per
    layer. A layer's cache holds 2^21 keys (143 MB), so 8 layers stream from HBM."""
    out = {}
    for name in SWEEP_WORKLOADS:
        L, S, meta = build_decode(torch, ifp4, W, layers, args.units, args.seed, workload=name)
        meta["separate_writer"] = not args.fused_write
        for _ in range(args.warmup):
            decode_step(ifp4, L, S, meta)
        torch.cuda.synchronize()
        if ifp4.sched_error(S["sched"]) != 0:
            raise RuntimeError(f"{name}: device error flags {ifp4.sched_error(S['sched'])}")
        step_graph = capture(torch, lambda: decode_step(ifp4, L, S, meta))
        for _ in range(args.warmup):
            step_graph.replay()
        step_ms = timed_replays(torch, step_graph, args.steps)
        scorer_graph = capture(torch, lambda: decode_scorers(ifp4, L, S, meta))
        scorer_graph.replay()
        scorer_us = 1e3 * timed_replays(torch, scorer_graph, args.steps) / layers
        alg = scoring_bytes(meta)
        gbs = alg / (scorer_us * 1e-6) / 1e9
        out[name] = {"batch": meta["B"], "context": meta["ctx"], "layers": layers,
                     "us_per_layer": round(1e3 * step_ms / layers, 3),
                     "keys_per_s": round(meta["n_keys"] * layers / (step_ms * 1e-3), 1),
                     "scorer_us": round(scorer_us, 3), "scorer_gbs": round(gbs, 1),
                     "scorer_frac": round(gbs / PEAK_HBM_GBS, 4), "alg_bytes_per_launch": alg}
        del step_graph, scorer_graph, L, S
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


SIZE_CONTEXTS = (32768, 65536, 131072, 262144)  # 8 rows each: 2^18 .. 2^21 keys a launch


def bench_scorer_sizes(torch, ifp4, W, args, layers=21):
    """The decode scorer alone at 2^18, 2^19, 2^20 and 2^21 keys a launch (8 rows of 32768 to
    262144 keys, 64 heads, 21 layer caches so every launch streams from HBM), with and without
    the top-k's first-digit histogram. A least-squares line of time against keys splits a
    launch into its fixed part and its per-key part."""
    rows = []
    for c in SIZE_CONTEXTS:
        L, S, meta = build_decode(torch, ifp4, W, layers, args.units, args.seed, contexts=[c] * 8)
        for _ in range(max(1, args.warmup)):
            decode_step(ifp4, L, S, meta)
        torch.cuda.synchronize()
        row = {"keys": meta["n_keys"], "context": c, "alg_bytes_per_launch": scoring_bytes(meta)}
        for hist in (True, False):
            def scorers():
                for lay in L:
                    ifp4.indexer_fp4_score_decode(lay["qp"], lay["qs"], lay["wm"], lay["kp"], lay["ks"], S["bt"], 1,
                                                  S["sched"], meta["units"], S["row_len"], S["logits"],
                                                  S["hist_scorer"] if hist else None)
            g = capture(torch, scorers)
            g.replay()
            us = 1e3 * timed_replays(torch, g, args.steps) / layers
            row["us_hist" if hist else "us_plain"] = round(us, 3)
            del g
        row["frac_hist"] = round(row["alg_bytes_per_launch"] / (row["us_hist"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)
        rows.append(row)
        print(f"bench: scorer at {row['keys']} keys: {row['us_hist']:.2f} us with the histogram, "
              f"{row['us_plain']:.2f} us without", file=sys.stderr, flush=True)
        del L, S
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    fit = {}
    x = np.array([r["keys"] for r in rows], np.float64)
    for key in ("us_hist", "us_plain"):
        y = np.array([r[key] for r in rows], np.float64)
        slope, icpt = np.polyfit(x, y, 1)
        fit[key] = {"fixed_us": round(float(icpt), 3), "us_per_2e20_keys": round(float(slope) * 2 ** 20, 3)}
    return {"rows": 8, "heads": 64, "layers": layers, "sizes": rows, "fit": fit}


PROBE_MODES = ("two MFMA waves a SIMD", "two VALU waves a SIMD", "one MFMA and one VALU wave a SIMD",
               "two waves a SIMD doing both", "one MFMA wave a SIMD", "one VALU wave a SIMD")


def mfma_valu_probe(torch, iters=4096, blocks=256):
    """The scorers' instruction mix alone (libindexer_fp4_probe.so, one 8-wave workgroup per CU):
    per mode the launch time and the shader clocks per iteration of the MFMA role (waves 0-3)
    and the other role (waves 4-7). An iteration is 16 FP4 MFMAs 16x16x128 and/or the page
    epilogue's 128 VALU operations."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_indexer_fp4_amd", "libindexer_fp4_probe.so"))
    lib.indexer_fp4_probe_mfma_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.indexer_fp4_probe_mfma_valu.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    g = torch.Generator().manual_seed(5)
    inp = torch.randint(0, 2 ** 31 - 1, (4096,), generator=g, dtype=torch.int32).to(dev)
    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    cyc = torch.zeros(blocks * 16, dtype=torch.int64, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = []
    for mode, name in enumerate(PROBE_MODES):
        for rep in range(2):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rc = lib.indexer_fp4_probe_mfma_valu(mode, iters, blocks, inp.data_ptr(), out.data_ptr(), cyc.data_ptr(),
                                                 stream)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"mfma/valu probe mode {mode}: error {rc}")
        c = cyc.view(blocks, 8, 2).cpu().numpy().astype(np.float64)
        clk = c[:, :, 0] / iters
        wall_us = c[:, :, 1] / 100.0  # 100 MHz
        mhz = float(np.median(c[:, :4, 0] / (c[:, :4, 1] * 10.0)) * 1e3)
        res.append({"mode": mode, "waves": name, "launch_us": round(e0.elapsed_time(e1) * 1e3, 1),
                    "clk_per_iter_waves_0_3": round(float(clk[:, :4].mean()), 1),
                    "clk_per_iter_waves_4_7": round(float(clk[:, 4:].mean()), 1),
                    "wave_us_0_3": round(float(wall_us[:, :4].mean()), 1),
                    "wave_us_4_7": round(float(wall_us[:, 4:].mean()), 1), "clock_mhz": round(mhz)})
        print(f"bench: probe mode {mode} ({name}): {res[-1]['launch_us']} us, clk/iter {res[-1]['clk_per_iter_waves_0_3']}"
              f" / {res[-1]['clk_per_iter_waves_4_7']}, {res[-1]['clock_mhz']} MHz", file=sys.stderr, flush=True)
    return {"iters": iters, "blocks": blocks, "modes": res}


def bench_decode_latency(torch, ifp4, W, args, layers=21):
    """Batch 1 at context 4096 (64 heads, top-2048): a latency-bound step. Whole steps
    (schedule, then per layer fused write + score + top-k) and the scorer alone, per layer, at
    the pages' two grid sizes: 512 units and 4096 ("Score a DSA sparse indexer in FP4", PR
    description, Decode grid floor: 2.99 against 8.75 us per layer). Empty units exit before
    any load, so the larger grid should cost only its extra dispatch."""
    out = {}
    for units in (512, 4096):
        L, S, meta = build_decode(torch, ifp4, W, layers, units, args.seed, workload="decode_b1_4k")
        meta["separate_writer"] = not args.fused_write
        for _ in range(args.warmup):
            decode_step(ifp4, L, S, meta)
        torch.cuda.synchronize()
        if ifp4.sched_error(S["sched"]) != 0:
            raise RuntimeError(f"decode_b1_4k: device error flags {ifp4.sched_error(S['sched'])}")
        step_graph = capture(torch, lambda: decode_step(ifp4, L, S, meta))
        for _ in range(args.warmup):
            step_graph.replay()
        step_ms = timed_replays(torch, step_graph, args.steps)
        scorer_graph = capture(torch, lambda: decode_scorers(ifp4, L, S, meta))
        scorer_graph.replay()
        scorer_us = 1e3 * timed_replays(torch, scorer_graph, args.steps) / layers
        out[f"units_{units}"] = {"us_per_layer": round(1e3 * step_ms / layers, 3), "scorer_us": round(scorer_us, 3)}
        del step_graph, scorer_graph, L, S
        torch.cuda.synchronize()
    return {"workload": "decode_b1_4k", "batch": 1, "context": 4096, "heads": 64, "index_topk": 2048,
            "layers": layers, **out}


def bench_prefill(torch, ifp4, W, args, workload="prefill_4req"):
    dev = torch.device("cuda:0")
    layers = args.layers
    case = W.prefill_config(workload, seed=args.seed)
    units = args.prefill_units
    kp = torch.zeros((case.n_pages, 64, 64), dtype=torch.uint8, device=dev)
    ks = torch.zeros((case.n_pages, 4, 64), dtype=torch.uint8, device=dev)
    ld = case.block_table.shape[1] * 64
    steps = []
    pairs = 0
    for st in case.steps:
        NP, R = st.n_rows_padded, len(st.req_ids)
        keys, slots = W.step_keys(case, st)
        bt = W.step_block_table(case, st)
        rl = np.zeros(NP, np.int64)
        for i in range(R):
            n = int(st.cu_rows[i + 1] - st.cu_rows[i])
            rl[st.cu_rows[i]:st.cu_rows[i + 1]] = st.start_pos[i] + np.arange(n) + 1
        pairs += int(rl.sum())
        steps.append(dict(
            NP=NP, R=R,
            keys=torch.from_numpy(keys.view(np.int16)).view(torch.bfloat16).to(dev),
            slots=torch.from_numpy(slots).to(dev),
            q=torch.from_numpy(st.q.view(np.int16)).view(torch.bfloat16).to(dev),
            w=torch.from_numpy(st.w).to(dev),
            cu=torch.from_numpy(st.cu_rows).to(dev), sp=torch.from_numpy(st.start_pos).to(dev),
            bt=torch.from_numpy(bt).to(dev),
            qp=torch.empty((NP, case.heads, 64), dtype=torch.uint8, device=dev),
            qs=torch.empty((NP, case.heads, 4), dtype=torch.uint8, device=dev),
            sched=torch.empty(ifp4.indexer_fp4_prefill_sched_bytes(R, NP, units, bt.shape[1]), dtype=torch.uint8,
                              device=dev),
            row_len=torch.empty(NP, dtype=torch.int32, device=dev),
            logits=torch.empty((NP, ld), dtype=torch.float32, device=dev),
            top=torch.empty((NP, case.topk), dtype=torch.int32, device=dev)))

    def schedules():
        # published once a step and shared by every layer of the step
        for s in steps:
            ifp4.indexer_fp4_prefill_schedule(s["cu"], s["sp"], s["NP"], units, s["bt"], kp.shape[0], s["sched"],
                                              s["row_len"])

    def run():
        # one layer: per step the chunk's key/query write, the scorer and the top-k
        for s in steps:
            ifp4.indexer_fp4_quant_and_cache(s["keys"], s["slots"], kp, ks, s["q"], s["qp"], s["qs"])
            ifp4.indexer_fp4_score_prefill(s["qp"], s["qs"], s["w"], kp, ks, s["R"], s["bt"].shape[1], s["sched"],
                                           units, s["NP"], s["logits"])
            ifp4.indexer_topk(s["logits"], s["row_len"], ld, case.topk, s["top"])

    def scorers():
        for s in steps:
            ifp4.indexer_fp4_score_prefill(s["qp"], s["qs"], s["w"], kp, ks, s["R"], s["bt"].shape[1], s["sched"],
                                           units, s["NP"], s["logits"])

    def writers():
        for s in steps:
            ifp4.indexer_fp4_quant_and_cache(s["keys"], s["slots"], kp, ks, s["q"], s["qp"], s["qs"])

    def topks():
        for s in steps:
            ifp4.indexer_topk(s["logits"], s["row_len"], ld, case.topk, s["top"])

    for _ in range(max(1, args.warmup)):
        schedules()
        run()
    torch.cuda.synchronize()
    reps = max(1, args.prefill_reps)
    sched_graph = capture(torch, schedules)
    sched_us = 1e3 * timed_replays(torch, sched_graph, reps)
    layer_graph = capture(torch, run)
    layer_us = 1e3 * timed_replays(torch, layer_graph, reps) + sched_us / layers
    scorer_graph = capture(torch, scorers)
    scorer_us = 1e3 * timed_replays(torch, scorer_graph, reps)
    writer_us = 1e3 * timed_replays(torch, capture(torch, writers), reps)
    topk_us = 1e3 * timed_replays(torch, capture(torch, topks), reps)
    flops = 16384 * pairs
    tflops = flops / (scorer_us * 1e-6) / 1e12
    return dict(workload=workload, lengths=[int(x) for x in case.lengths], chunk=case.chunk,
                steps=len(steps), causal_pairs=pairs, us_per_layer=round(layer_us, 2),
                schedule_us_per_pass=round(sched_us, 2), layers_sharing_schedule=layers,
                scorer_us_per_layer=round(scorer_us, 2), writer_us_per_layer=round(writer_us, 2),
                topk_us_per_layer=round(topk_us, 2), keys_scored_per_s=pairs / (layer_us * 1e-6),
                scorer_keys_per_s=round(pairs / (scorer_us * 1e-6), 1),
                roofline={"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_FP4_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP4_TFLOPS, 4)})


def bench_fp8_comparator(torch, ifp4, W, args):
    """The pages' FP4-vs-FP8 scorer comparison on this hardware: the same decode workload's
    keys and queries in MXFP8 planes, scored by the same scorer template; the step's 21 scorer
    launches per replay for each format (no histogram, so only the scan differs)."""
    L, S, meta = build_decode(torch, ifp4, W, args.layers, args.units, args.seed, fp8=True)
    for lay in L:  # the FP4 queries and the scaled weights (the FP8 query planes hold the same queries unrotated)
        write_decode(ifp4, lay, S)
    ifp4.indexer_fp4_decode_schedule(S["ctx"], 1, meta["units"], S["sched"], S["row_len"])

    def scorers(fp8):
        fn = ifp4.indexer_fp8_score_decode if fp8 else ifp4.indexer_fp4_score_decode
        for lay in L:
            fn(lay["qp8"] if fp8 else lay["qp"], lay["qs8"] if fp8 else lay["qs"], lay["wm"],
               lay["kp8"] if fp8 else lay["kp"], lay["ks8"] if fp8 else lay["ks"], S["bt"], 1, S["sched"],
               meta["units"], S["row_len"], S["logits"])

    us = {}
    for name, fp8 in (("fp4", False), ("fp8", True)):
        scorers(fp8)
        g = capture(torch, lambda: scorers(fp8))
        g.replay()
        us[name] = 1e3 * timed_replays(torch, g, args.steps) / args.layers
        del g
    torch.cuda.synchronize()
    if ifp4.sched_error(S["sched"]) != 0:
        raise RuntimeError("fp8 comparator: device error flags")
    n_keys, pages, B, H = meta["n_keys"], meta["n_pages_read"], meta["B"], meta["H"]
    b4 = decode_scorer_bytes(n_keys, pages, B, H)
    b8 = b4 + n_keys * 64 + B * H * 64  # 64 more code bytes per key and per query head
    del L, S
    torch.cuda.empty_cache()
    return {"format": "MXFP8 (E4M3, e8m0 per 32)", "workload": "decode_b8_128k",
            "fp4_scorer_us": round(us["fp4"], 3), "fp8_scorer_us": round(us["fp8"], 3),
            "fp4_minus_fp8_us": round(us["fp4"] - us["fp8"], 3),
            "time_ratio_fp4_over_fp8": round(us["fp4"] / us["fp8"], 4),
            "cache_bytes_per_key": {"fp4": 68, "fp8": 132}, "byte_ratio_alg": round(b4 / b8, 4),
            "fp8_achieved_gbs": round(b8 / (us["fp8"] * 1e-6) / 1e9, 1),
            "fp8_frac": round(b8 / (us["fp8"] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


def bench_dcp_merge(torch, ifp4, args, shards=4, rows=8, k=2048):
    """Merge of `shards` local top-k candidate lists per row (context-parallel decode on one
    GPU's share; the exchange itself is not timed): one launch per layer."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(args.seed)
    sc = torch.randn((rows, shards * k), generator=g, device=dev, dtype=torch.float32)
    ix = torch.randperm(rows * shards * k * 2, generator=g, device=dev)[: rows * shards * k].view(rows, -1).int()
    out = torch.empty((rows, k), dtype=torch.int32, device=dev)
    ifp4.indexer_topk_merge(sc, ix, k, out)
    graph = capture(torch, lambda: [ifp4.indexer_topk_merge(sc, ix, k, out) for _ in range(args.layers)])
    us = 1e3 * timed_replays(torch, graph, args.steps) / args.layers
    return {"shards": shards, "rows": rows, "candidates_per_row": shards * k, "k": k, "us_per_layer": round(us, 3)}


def cpu_baseline(W, seconds: float):
    """The oracle on the decode workload's first sequences: score every key (fp64) and run
    the full-sort top-k, repeated until `seconds` of work; returns keys scored per second."""
    import oracle

    case = W.decode_config("decode_b8_128k", seed=0)
    kp = np.zeros((case.n_pages, 64, 64), np.uint8)
    ks = np.zeros((case.n_pages, 4, 64), np.uint8)
    oracle.quant_and_cache(case.keys, case.slots, kp, ks)
    qp, qs = oracle.quant_q(case.q)
    rs, rl = oracle.decode_geometry(case.ctx)
    done_keys, t0 = 0, time.perf_counter()
    reps = 0
    while True:
        s, _ = oracle.score(qp, qs, case.w, rs, rl, kp, ks, case.block_table)
        oracle.topk(s, rl, case.topk)
        done_keys += int(rl.sum())
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(done_keys / dt, 1), "unit": "keys/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} pass(es) of fp64 score + full-sort top-k over one layer of the 8 x 131072 decode "
                      f"workload ({int(rl.sum())} keys each), cache already written; {dt:.1f} s on {threads} "
                      f"threads of {model}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=21)
    ap.add_argument("--units", type=int, default=None)
    ap.add_argument("--prefill-units", type=int, default=None)
    ap.add_argument("--prefill-reps", type=int, default=10)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 comparator")
    ap.add_argument("--no-sweep", action="store_true", help="skip the long decode workloads")
    ap.add_argument("--no-latency", action="store_true", help="skip the batch-1, 4096-context decode leg")
    ap.add_argument("--mfma-valu-probe", action="store_true",
                    help="run only the MFMA/VALU instruction-mix probe and print its JSON line")
    ap.add_argument("--scorer-sizes", action="store_true",
                    help="also time the decode scorer alone at 2^18 .. 2^21 keys a launch (fixed and per-key parts)")
    ap.add_argument("--fused-write", action="store_true",
                    help="decode steps run the writer's work inside the scorer (one launch a layer)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 256 MiB device-to-device copy, a kernel of known traffic "
                         "for scaling hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (this build has no "
              f"multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import torch

    import sparse_attention_indexer_fp4_amd as ifp4
    import workloads as W

    if args.mfma_valu_probe:
        print(json.dumps({"probe": "mfma_valu", **mfma_valu_probe(torch)}), flush=True)
        return
    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("bench: copy calibration kernel: 268435456 bytes read, 268435456 written", file=sys.stderr, flush=True)
        del src, dst
    args.units = args.units or ifp4.DECODE_UNITS
    args.prefill_units = args.prefill_units or ifp4.PREFILL_UNITS
    print(f"bench: decode 8 x 131072, {args.layers} layers, steps={args.steps} warmup={args.warmup}",
          file=sys.stderr, flush=True)
    d = bench_decode(torch, ifp4, W, args)
    print(f"bench: decode {d['ms_per_step']:.3f} ms/step, scoring kernel {d['scorer_us']:.2f} us "
          f"({d['achieved_gbs']:.0f} GB/s), plain scorer {d['plain_scorer']['us']:.2f} us, writer "
          f"{d['writer']['fused_us_per_layer']:.2f} us", file=sys.stderr, flush=True)
    pre = pre_mbt = None
    sweep = None
    if not args.no_sweep:
        sweep = bench_decode_sweep(torch, ifp4, W, args)
        for name, r in sweep.items():
            print(f"bench: {name} {r['us_per_layer']:.2f} us/layer, scorer {r['scorer_us']:.2f} us "
                  f"({r['scorer_gbs']:.0f} GB/s)", file=sys.stderr, flush=True)
    lat = None
    if not args.no_latency:
        lat = bench_decode_latency(torch, ifp4, W, args)
        print(f"bench: decode_b1_4k {lat['units_512']['us_per_layer']:.2f} / {lat['units_4096']['us_per_layer']:.2f} "
              f"us/layer at 512 / 4096 units, scorer {lat['units_512']['scorer_us']:.2f} / "
              f"{lat['units_4096']['scorer_us']:.2f} us", file=sys.stderr, flush=True)
    sizes = None
    if args.scorer_sizes:
        sizes = bench_scorer_sizes(torch, ifp4, W, args)
        f = sizes["fit"]
        print(f"bench: scorer fit: {f['us_hist']['fixed_us']:.2f} us fixed + {f['us_hist']['us_per_2e20_keys']:.2f} us "
              f"per 2^20 keys with the histogram, {f['us_plain']['fixed_us']:.2f} + "
              f"{f['us_plain']['us_per_2e20_keys']:.2f} without", file=sys.stderr, flush=True)
    dcp = bench_dcp_merge(torch, ifp4, args)
    fp8 = None
    if not args.no_fp8:
        fp8 = bench_fp8_comparator(torch, ifp4, W, args)
        print(f"bench: fp8 comparator {fp8['fp4_scorer_us']:.2f} vs {fp8['fp8_scorer_us']:.2f} us", file=sys.stderr,
              flush=True)
    if not args.no_prefill:
        pre = bench_prefill(torch, ifp4, W, args)
        pre_mbt = bench_prefill(torch, ifp4, W, args, "prefill_4req_mbt512")
        for nm, r in (("prefill", pre), ("prefill, 512-token step budget", pre_mbt)):
            print(f"bench: {nm}: {r['steps']} steps, {r['us_per_layer']:.1f} us/layer, scorer "
                  f"{r['scorer_us_per_layer']:.1f} us, writer {r['writer_us_per_layer']:.1f} us, top-k "
                  f"{r['topk_us_per_layer']:.1f} us", file=sys.stderr, flush=True)

    # HBM traffic of the scorer from rocprofv3 counters, valid only for the kernel they were taken on
    traffic = None
    tf = os.path.join(ROOT, "profiles", "decode_scorer_traffic.json")
    if os.path.exists(tf):
        with open(tf) as f:
            rec = json.load(f)
        if rec.get("kernel_hash") == kernel_source_hash(["score_decode.hip", "score_common.h", "common.h"]):
            traffic = rec.get("bytes_per_launch")
    cpu = None
    if rank == 0 and not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(W, args.cpu_seconds)

    m = d["meta"]
    line = {
        "metric": METRIC,
        "value": round(d["keys_per_s"], 1),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(d["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "decode_b8_128k", "batch": m["B"], "context": m["ctx"], "heads": m["H"],
                   "head_dim": 128, "index_topk": m["k"], "layers": args.layers, "page": 64,
                   "units": m["units"]},
        "decode_us_per_layer": round(1e3 * d["ms_per_step"] / args.layers, 3),
        "decode_scorer_keys_per_s": round(d["meta"]["n_keys"] / (d["scorer_us"] * 1e-6), 1),
        "roofline": {"bound": "hbm", "achieved": round(d["achieved_gbs"], 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(d["achieved_gbs"] / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "kernel": "write_and_score_decode" if args.fused_write else "score_decode",
                     "launch_us_mean": round(d["scorer_us"], 3), "alg_bytes_per_launch": d["alg_bytes"]},
        "plain_scorer": d["plain_scorer"],
        "cpu_baseline": cpu,
        "writer": d["writer"],
        "decode_latency": lat,
        "decode_long": sweep,
        "scorer_sizes": sizes,
        "prefill": pre,
        "prefill_mbt512": pre_mbt,
        "dcp_merge": dcp,
        "fp8_comparator": fp8,
    }
    if rank == 0:
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
