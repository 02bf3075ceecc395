#!/usr/bin/env python3
"""Decode-step benchmark: top-k sparse decode attention, DSA sparse MLA at
64K context (batch 16, 64x128 bf16 indexer, page 64, top-k 2048, 128 heads
over a 576-wide latent row), on one MI355X.

One step = one sd_sparse_decode call over the whole batch: score every
cached token, select the top 2048 per request, attend over them.  Inputs are
seeded synthetic tensors of that shape, resident in HBM before timing; the
pools are replicated and the replicas rotated step by step so the scored
indexer keys (268 MB per replica) do not sit in the 256 MB last-level cache.

Prints one JSON line.  Algorithmic bytes per step = indexer K bytes scored
+ selected latent rows gathered.  The roofline entry is for the dominant
kernel (the MFMA indexer scorer), timed with HIP events on its own stream;
a second entry covers the gather phase (attention + combine over the
selected rows), and both are also put against a plain device copy's
bandwidth measured in the same run.  Per-step times come from an event
between every two steps.  The CPU baseline is the oracle on a sample of
the same workload, on every host core this process may use and on one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse decode steps/s + achieved HBM GB/s, DSA-MLA 64K ctx top-k 2048"
PEAK_HBM_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
SCORER_SOURCE = os.path.join(ROOT, "top_sparse_decode_amd", "csrc", "score.hip")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--replicas", type=int, default=3, help="input replicas rotated per step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-requests", type=int, default=16, help="requests in the oracle sample")
    p.add_argument("--cpu-repeats", type=int, default=20, help="passes of the oracle over the sample")
    p.add_argument("--cpu-single-requests", type=int, default=16,
                   help="requests in the single-threaded oracle sample")
    p.add_argument("--workload", choices=["dsa_mla", "triattention", "blocks", "gqa", "dsa_mixed"],
                   default="dsa_mla",
                   help="dsa_mla: the fused decode step (default); triattention: one eviction-time "
                        "selection (normalize, reduce, top-k) over 36 layers x 32 requests x 8 KV heads "
                        "x 4096 tokens, keeping 2048; blocks: sparse MLA attention at 64K over 128 "
                        "selected 16-token blocks per request; gqa: the fused step on the Qwen3-8B-shaped "
                        "GQA workload (32 requests, 32 query / 8 KV heads x 128, 8192 tokens, top-k 2048 "
                        "per KV head, exact scores); dsa_mixed: the fused step on the mixed-length DSA MLA "
                        "workload (64 requests, kv_len uniform in [4096, 131072], shared fragmented page pool)")
    p.add_argument("--tri-mode", choices=["union", "per_head", "per_layer_perhead"], default="union")
    p.add_argument("--next-n", type=int, default=1,
                   help="query tokens per request (multi-query decode: a token and its drafts)")
    p.add_argument("--index-dtype", choices=["bf16", "fp8"], default="bf16",
                   help="indexer K cache: bf16, or FP8 E4M3 codes with one float32 scale per row")
    p.add_argument("--hint", action="store_true",
                   help="feed each step the previous step's selection as its top-k hint (written back "
                        "by the selection itself)")
    p.add_argument("--copy-bytes", type=int, default=0,
                   help="also run a plain device copy of this many bytes (3 launches) before the "
                        "steps: the reference kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE")
    return p.parse_args()


def per_step_stats(ms):
    """Median, 10% trimmed mean, min and max of per-step times (ms in, us out)."""
    v = sorted(ms)
    n = len(v)
    cut = n // 10
    core = v[cut:n - cut] if n - 2 * cut > 0 else v
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"median_us": round(med * 1e3, 2), "trimmed_mean_10_us": round(sum(core) / len(core) * 1e3, 2),
            "min_us": round(v[0] * 1e3, 2), "max_us": round(v[-1] * 1e3, 2), "n": n}


def scorer_traffic(kernel_hash: str, fp8: bool):
    """HBM bytes per scorer launch from the committed rocprofv3 counter
    summary, or None when it is missing or was taken on another version of
    the scorer source."""
    path = os.path.join(PROFILES, "score_dsa_fp8_traffic.json" if fp8 else "score_dsa_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("source_sha256") != kernel_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def bench_triattention(args, api, torch, dev):
    """One TriAttention eviction-time selection: the stacked per-layer score
    rows of a 36-layer, 8-KV-head model for 32 requests at 4096 tokens
    (budget 2048 + window 2048), normalized, reduced by mode, top 2048 kept.
    The rows are seeded synthetic scores (per-row location and spread drawn
    once, then N(0,1) tokens), generated on the device."""
    layers, B, G, S, k = 36, 32, 8, 4096, 2048
    gen = torch.Generator(device=dev)
    gen.manual_seed(2048)
    loc = torch.rand((layers, B, G, 1), generator=gen, device=dev) * 100 - 50
    spread = torch.exp(torch.rand((layers, B, G, 1), generator=gen, device=dev) * 4 - 2)
    scores = [torch.randn((layers, B, G, S), generator=gen, device=dev) * spread + loc
              for _ in range(max(1, args.replicas))]
    kv = torch.full((B,), S, dtype=torch.int32, device=dev)
    out_rows = {"per_layer_perhead": layers * B * G, "per_head": B * G, "union": B}[args.tri_mode]
    idx = torch.empty((out_rows, k), dtype=torch.int32, device=dev)
    ws = torch.empty(api.triattention_select_workspace_size(layers, B, G, S, args.tri_mode, k),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        api.triattention_select(scores[i % len(scores)], kv, args.tri_mode, k, idx, None, None, ws,
                                stream=stream)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    score_bytes = layers * B * G * S * 4
    gbps = score_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "TriAttention selections/s (normalize + reduce + top-k)",
        "value": round(1000.0 / ms, 2), "unit": "selections/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 scores, f64 statistics", "data": "synthetic (seeded per-row "
        "location U(-50,50), spread exp(U(-2,2)), N(0,1) tokens, generated on the device)",
        "config": {"workload": f"triattention {args.tri_mode}: 36 layers x 32 requests x 8 KV heads x "
                               f"4096 tokens, keep 2048", "layers": layers, "batch": B, "kv_heads": G,
                   "kv_len": S, "topk": k, "mode": args.tri_mode, "input_replicas": len(scores)},
        "roofline": {"kernel": "whole call (tri_stats, tri_reduce, selection)", "bound": "hbm",
                     "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                     "bytes_per_launch": score_bytes},
    }
    print(json.dumps(result), flush=True)


def bench_blocks(args, api, torch, dev, synth, np):
    """Sparse MLA attention over block-granular selections: the 64K-context DSA-MLA
    latent cache (16 requests, 64K tokens), 128 distinct random 16-token
    blocks per request (2048 tokens), against the same tokens given as a
    token list."""
    w = synth.make_workload(4)
    step = api.prepare(w, precision=api.EXACT, device=dev)
    kb, bs = 128, 16
    rs = np.random.default_rng(16)
    B = w.batch
    blocks = np.stack([np.sort(rs.permutation(int(L) // bs)[:kb]) for L in w.kv_lens]).astype(np.int32)[:, None, :]
    d_blk = torch.from_numpy(blocks).to(dev)
    tok = torch.from_numpy((blocks[..., None] * bs + np.arange(bs)).reshape(B, 1, kb * bs).astype(np.int32)).to(dev)
    Hq = w.q.shape[1]
    nb = api.sparse_decode_attn_blocks_workspace_size(step.args.pages, Hq, step.args.k, w.v_dim, kb, bs)
    nt = api.sparse_decode_attn_workspace_size(step.args.pages, Hq, step.args.k, w.v_dim, kb * bs)
    wsb = torch.empty(nb, dtype=torch.uint8, device=dev)
    wst = torch.empty(nt, dtype=torch.uint8, device=dev)
    out = torch.empty_like(step.out)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps
    ms_b = timed(lambda: api.sparse_decode_attn_blocks(step.args.pages, step.q, Hq, step.args.k, step.args.v,
                                                       w.v_dim, d_blk, kb, bs, w.softmax_scale, out, wsb,
                                                       stream=stream))
    ms_t = timed(lambda: api.sparse_decode_attn(step.args.pages, step.q, Hq, step.args.k, step.args.v, w.v_dim,
                                                tok, kb * bs, w.softmax_scale, out, wst, stream=stream))
    gathered = B * kb * bs * w.k.shape[-1] * 2
    gbps = gathered / (ms_b * 1e-3) / 1e9
    print(json.dumps({
        "metric": "block-granular sparse MLA attention calls/s",
        "value": round(1000.0 / ms_b, 2), "unit": "calls/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_b, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (64K-context DSA-MLA latent pool, seeded random blocks)",
        "config": {"workload": "sparse MLA 128 heads x 576/512 over 128 blocks of 16 tokens per request, "
                               "16 requests at 64K", "batch": B, "k_blocks": kb, "block_size": bs},
        "token_list_ms": round(ms_t, 5),
        "roofline": {"kernel": "whole call (block expansion, attention, combine)", "bound": "hbm",
                     "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(gbps / PEAK_HBM_GBPS, 4), "traffic": None, "bytes_per_launch": gathered},
    }), flush=True)


def bench_gqa(args, api, torch, dev, synth):
    """The fused step on the Qwen3-8B-shaped GQA workload: 32 requests, 32
    query heads over 8 KV heads of 128 dims, 8192 tokens in 64-token pages,
    score = mean over the 4 query heads of a KV head, top 2048 per KV head,
    softmax attention per query head over the selected K/V rows.  Scores are
    computed in the exact order (the vector scorer: one lane per token); the
    roofline entry is that scorer alone."""
    say("[bench] generating gqa workload (B32, 32q/8kv x 128, L8192) ...")
    w = synth.make_workload(3)
    step = api.prepare(w, precision=api.EXACT, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    B, Hq = w.q.shape[0], w.q.shape[1]
    Hkv, D = w.k.shape[1], w.k.shape[-1]
    L = int(w.kv_lens[0])

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps
    ms = timed(lambda: step.run(stream))
    sc = torch.empty((B, Hkv, w.max_kv_len), dtype=torch.float32, device=dev)
    bound = torch.zeros((B, Hkv), dtype=torch.float32, device=dev)
    ms_sc = timed(lambda: api.sparse_score_paged(step.args.pages, step.args.score_k, step.score_q, Hq, None,
                                                 api.MODES[w.mode], w.head_scale, api.EXACT, sc, bound, stream))
    k_scored = B * Hkv * L * D * 2
    gathered = B * Hkv * w.topk * D * 2 * 2  # selected K and V rows
    alg = k_scored + gathered
    sc_gbps = k_scored / (ms_sc * 1e-3) / 1e9
    print(json.dumps({
        "metric": "sparse decode steps/s, Qwen3-8B-shaped GQA 8K ctx top-k 2048 per KV head",
        "value": round(1000.0 / ms, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) K/V with log-uniform "
        "per-channel scales, one replica: 537 MB of K per step exceeds the last-level cache)",
        "config": {"workload": "gqa: 32 requests, 32 query heads over 8 KV heads x 128, kv_len 8192, page 64, "
                               "score = mean over a KV head's 4 query heads, top-k 2048 per KV head, exact "
                               "scores", "batch": B, "kv_len": L, "page_size": w.page_size, "topk": w.topk},
        "algorithmic_bytes_per_step": alg,
        "step_gbps": round(alg / (ms * 1e-3) / 1e9, 1),
        "step_frac_of_hbm_peak": round(alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "roofline": {"kernel": "score_exact_kernel (GROUP_MEAN, bf16)", "bound": "hbm",
                     "achieved": round(sc_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(sc_gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                     "avg_launch_us": round(ms_sc * 1e3, 2), "bytes_per_launch": k_scored},
    }), flush=True)


def bench_mixed(args, api, torch, dev, synth):
    """The fused step on the mixed-length DSA sparse-MLA workload: 64
    requests with kv_len uniform in [4096, 131072] over one fragmented page
    pool (about 4M cached tokens), the 64K-context DSA-MLA indexer and latent cache,
    top-k 2048.  One replica (7 GB of pools: nothing stays in the last-level
    cache between steps).  The roofline entry is the fast indexer scorer."""
    say("[bench] generating dsa_mixed workload (B64, L ~ U[4096, 131072]) ...")
    t0 = time.time()
    w = synth.make_workload(5)
    say(f"[bench] generated in {time.time() - t0:.1f}s")
    step = api.prepare(w, precision=api.FAST, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    B = w.batch
    lens = [int(x) for x in w.kv_lens]

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps
    ms = timed(lambda: step.run(stream))
    sc = torch.empty((B, 1, w.max_kv_len), dtype=torch.float32, device=dev)
    bound = torch.zeros((B, 1), dtype=torch.float32, device=dev)
    ms_sc = timed(lambda: api.sparse_score_paged(step.args.pages, step.args.score_k, step.score_q,
                                                 w.score_q.shape[1], step.head_weights, api.RELU_WEIGHTED, 1.0,
                                                 api.FAST, sc, bound, stream))
    k_scored = sum(lens) * w.score_k.shape[-1] * 2
    gathered = sum(min(L, w.topk) for L in lens) * w.k.shape[-1] * 2
    alg = k_scored + gathered
    sc_gbps = k_scored / (ms_sc * 1e-3) / 1e9
    print(json.dumps({
        "metric": "sparse decode steps/s + achieved HBM GB/s, DSA-MLA mixed lengths 4K-128K top-k 2048",
        "value": round(1000.0 / ms, 2), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) pools, 1% of tokens with a "
        "+4 sigma key bias, one shared fragmented page pool, one replica)",
        "config": {"workload": "dsa_mixed: 64 requests, kv_len uniform in [4096, 131072], page 64, indexer 64 "
                               "heads x 128 bf16 (ReLU-weighted), top-k 2048, sparse MLA 128 heads over "
                               "576-dim latent rows", "batch": B, "tokens": sum(lens), "max_kv_len": w.max_kv_len,
                   "page_size": w.page_size, "topk": w.topk},
        "algorithmic_bytes_per_step": alg,
        "step_gbps": round(alg / (ms * 1e-3) / 1e9, 1),
        "step_frac_of_hbm_peak": round(alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "roofline": {"kernel": "score_dsa_kernel (fast indexer scorer)", "bound": "hbm",
                     "achieved": round(sc_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(sc_gbps / PEAK_HBM_GBPS, 4), "traffic": None,
                     "avg_launch_us": round(ms_sc * 1e3, 2), "bytes_per_launch": k_scored},
    }), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by "
              "request across GPUs with no exchange between them.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from top_sparse_decode_amd import api, synth

    torch.cuda.set_device(0)
    dev = "cuda:0"
    if args.workload == "triattention":
        return bench_triattention(args, api, torch, dev)
    if args.workload == "blocks":
        return bench_blocks(args, api, torch, dev, synth, np)
    if args.workload == "gqa":
        return bench_gqa(args, api, torch, dev, synth)
    if args.workload == "dsa_mixed":
        return bench_mixed(args, api, torch, dev, synth)
    fp8 = args.index_dtype == "fp8"
    say(f"[bench] generating dsa_mla workload (B16, L65536, {args.index_dtype} indexer) ...")
    t0 = time.time()
    w = synth.make_workload(4, index_dtype=args.index_dtype, next_n=args.next_n)
    say(f"[bench] generated in {time.time() - t0:.1f}s; uploading {args.replicas} replicas")
    steps = [api.prepare(w, precision=api.FAST, device=dev, hint=args.hint) for _ in range(max(1, args.replicas))]
    torch.cuda.synchronize()

    B, L, P = w.batch, int(w.kv_lens[0]), w.page_size
    # bytes of indexer K read (fp8: the codes and one float32 scale per row)
    k_scored = B * L * (w.score_k.shape[-1] + 4 if fp8 else w.score_k.shape[-1] * 2)
    # selected latent rows (V is inside them), per query token
    k_gathered = B * args.next_n * w.topk * w.k.shape[-1] * 2
    alg_bytes = k_scored + k_gathered

    stream = torch.cuda.current_stream()
    if args.copy_bytes > 0:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        say(f"[bench] copy reference: 3 x {n * 4} bytes")
        del src, dst
    for i in range(args.warmup):
        steps[i % len(steps)].run(stream)
    torch.cuda.synchronize()

    # ---- timed region: K whole steps, an event between every two
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(args.steps):
        steps[i % len(steps)].run(stream)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    ms_total = ev[0].elapsed_time(ev[-1])
    ms_step = ms_total / args.steps
    steps_per_s = 1000.0 / ms_step
    per_step = per_step_stats([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    say(f"[bench] {args.steps} steps: {ms_step * 1e3:.1f} us/step (median {per_step['median_us']} us)")

    # ---- warm figure: the same step on one replica, its pools partly in the
    # last-level cache between steps
    def timed_region(fn, n):
        for i in range(min(args.warmup, 5)):
            fn(i)
        torch.cuda.synchronize()
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for i in range(n):
            fn(i)
        a1.record(stream)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) / n
    warm_ms = timed_region(lambda i: steps[0].run(stream), args.steps)

    # ---- gather phase alone: attention + combine over each replica's
    # selection (rotated like the steps)
    Hq = w.q.shape[1]
    attn_ws = torch.empty(api.sparse_decode_attn_workspace_size(steps[0].args.pages, Hq, steps[0].args.k,
                                                                w.v_dim, w.topk * args.next_n),
                          dtype=torch.uint8, device=dev)
    attn_out = torch.empty_like(steps[0].out)

    def attend(i):
        s = steps[i % len(steps)]
        api.sparse_decode_attn(s.args.pages, s.q, Hq, s.args.k, s.args.v, w.v_dim, s.indices,
                               w.topk * args.next_n, w.softmax_scale, attn_out, attn_ws, stream=stream)
    attn_ms = timed_region(attend, args.steps) if args.next_n == 1 else None

    # ---- plain device copy (read + write) of 1 GiB: the bandwidth a simple
    # streaming kernel reaches on this device, measured here
    cp_src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cp_dst = torch.empty_like(cp_src)
    copy_ms = timed_region(lambda i: cp_dst.copy_(cp_src), 10)
    copy_gbps = 2 * cp_src.numel() * 4 / (copy_ms * 1e-3) / 1e9
    del cp_src, cp_dst

    # ---- dominant kernel: the MFMA indexer scorer alone (the call launches
    # that one kernel: its bound output is max-accumulated into a buffer
    # zeroed once), back to back over the rotated replicas, HIP events on
    # the launch stream around the whole run
    groups, hi = 1, w.score_q.shape[1]
    sc = torch.empty((B, groups, w.max_kv_len), dtype=torch.float32, device=dev)
    bound = torch.zeros((B, groups), dtype=torch.float32, device=dev)

    def score(i):
        s = steps[i % len(steps)]
        api.sparse_score_paged(s.args.pages, s.args.score_k, s.score_q, hi, s.head_weights,
                               api.RELU_WEIGHTED, 1.0, api.FAST, sc, bound, stream)
    for i in range(min(args.warmup, 5)):
        score(i)
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for i in range(args.steps):
        score(i)
    s1.record(stream)
    torch.cuda.synchronize()
    score_ms = s0.elapsed_time(s1) / args.steps
    score_gbps = k_scored / (score_ms * 1e-3) / 1e9
    src_hash = hashlib.sha256(open(SCORER_SOURCE, "rb").read()).hexdigest()
    gather_gbps = k_gathered / (attn_ms * 1e-3) / 1e9 if attn_ms else None

    result = {
        "metric": METRIC,
        "value": round(steps_per_s, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16" if fp8 else "bf16",
        "data": "synthetic (seeded N(0,1) bf16 pools, U(0,1) head weights"
                + (", indexer keys quantized to FP8 E4M3 per row)" if fp8 else ")"),
        "config": {
            "workload": "dsa_mla: batch 16, one decode query each, kv_len 65536, page 64, "
                        + ("indexer 64 heads x 128 fp8 e4m3 keys with a float32 scale per row"
                           if fp8 else "indexer 64 heads x 128 bf16")
                        + " (ReLU-weighted), top-k 2048, sparse MLA "
                        "128 heads over 576-dim latent rows (V = first 512), scale 1/sqrt(192)",
            "batch": B, "kv_len": L, "page_size": P, "topk": w.topk,
            "precision": "fast scores + exact band re-score (indices exact)",
            "input_replicas": args.replicas,
            "next_n": args.next_n,
            "topk_hint": "previous step's selection, written back in place" if args.hint else None,
        },
        "algorithmic_bytes_per_step": alg_bytes,
        "step_gbps": round(alg_bytes / (ms_step * 1e-3) / 1e9, 1),
        "step_frac_of_hbm_peak": round(alg_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
        "per_step": per_step,
        "warm": {"what": "the same step on one replica (pools partly in the 256 MB last-level cache)",
                 "steps_per_s": round(1000.0 / warm_ms, 2), "ms_per_step": round(warm_ms, 5)},
        "stream_copy_gbps": round(copy_gbps, 1),
        "roofline_gather": None if attn_ms is None else {
            "kernel": "attn_mla_kernel + attn_mla_combine_kernel (selected latent rows)",
            "bound": "hbm",
            "achieved": round(gather_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(gather_gbps / PEAK_HBM_GBPS, 4),
            "frac_of_stream_copy": round(gather_gbps / copy_gbps, 4),
            "avg_call_us": round(attn_ms * 1e3, 2),
            "bytes_per_launch": k_gathered,
        },
        "roofline": {
            "kernel": "score_dsa_fp8_kernel<4, 8, 3, 16>" if fp8 else "score_dsa_kernel<4, 4, 4, 32>",
            "bound": "hbm",
            "achieved": round(score_gbps, 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(score_gbps / PEAK_HBM_GBPS, 4),
            "frac_of_stream_copy": round(score_gbps / copy_gbps, 4),
            "traffic": scorer_traffic(src_hash, fp8),
            "avg_launch_us": round(score_ms * 1e3, 2),
            "bytes_per_launch": k_scored,
        },
    }

    # ---- CPU baseline: the oracle on a bounded sample, plus a parity check
    if not args.no_cpu_baseline:
        import oracle
        n = max(1, min(args.cpu_requests, B))
        reqs = list(range(n))
        import dataclasses

        nq = args.next_n
        rows = [b * nq + j for b in reqs for j in range(nq)]   # the requests' query rows
        ws = dataclasses.replace(w, block_table=w.block_table[reqs], kv_lens=w.kv_lens[reqs],
                                 score_q=w.score_q[rows], head_weights=w.head_weights[rows],
                                 q=w.q[rows])
        reps = max(1, args.cpu_repeats)
        cores = len(os.sched_getaffinity(0))
        used = oracle.set_threads(cores)
        say(f"[bench] oracle on {n} request(s) x {reps}, {used} threads ...")
        t0 = time.perf_counter()
        for _ in range(reps):
            ref = oracle.sparse_decode(ws)
        cpu_s = time.perf_counter() - t0
        per_step_s = cpu_s / (n * reps) * B
        # the same oracle on one thread, over fewer requests
        n1 = max(1, min(args.cpu_single_requests, n))
        ws1 = dataclasses.replace(ws, block_table=ws.block_table[:n1], kv_lens=ws.kv_lens[:n1],
                                  score_q=ws.score_q[:n1 * nq], head_weights=ws.head_weights[:n1 * nq],
                                  q=ws.q[:n1 * nq])
        oracle.set_threads(1)
        say(f"[bench] oracle on {n1} request(s), 1 thread ...")
        t1 = time.perf_counter()
        oracle.sparse_decode(ws1)
        cpu1_s = time.perf_counter() - t1
        oracle.set_threads(used)
        result["cpu_baseline"] = {
            "value": round(1.0 / per_step_s, 5),
            "unit": "steps/s",
            "cores": used,
            "kind": "oracle",
            "sample": f"{reps} pass(es) over {n} of {B} requests of the same workload (score all "
                      f"65536 tokens, full sort, float64 attention), {cpu_s:.1f}s on {used} threads "
                      f"(OpenMP over rows; every host core this process may use), scaled to one step",
            "single_thread": {"value": round(1.0 / (cpu1_s / n1 * B), 5), "unit": "steps/s", "cores": 1,
                              "sample": f"{n1} of {B} requests, {cpu1_s:.1f}s, scaled to one step"},
        }
        s0 = steps[(args.steps - 1) % len(steps)]
        idx = s0.indices.cpu().numpy()[rows]
        got = s0.out.float().cpu().numpy()[rows].astype(np.float64)
        err = np.linalg.norm(got - ref["out"], axis=-1) / np.linalg.norm(ref["out"], axis=-1)
        result["parity_sample"] = {"requests": reqs,
                                   "indices_equal": bool(np.array_equal(idx, ref["indices"])),
                                   "max_row_rel_l2": float(err.max())}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
