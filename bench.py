"""Benchmark: global K=V attention prefill at 32K (TFLOP/s) and global K=V decode
(KV GB/s), each against the MI355X roofline, with the float64 oracle timed on
the host as a reported baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints one JSON line.  A step is one pass of the hot path over the workload:
one gemma_attn_prefill call (RoPE table + key/value prep + attention) on the
32K global-layer prefill.  Reported beside it: the global decode (one
gemma_attn_decode call on 16 sequences with lengths drawn from [4096, 131072],
and kv_append on its own), the local-layer prefill (B=4, S=32K, window 1024)
one decode step of a 6-layer stack (5 local + 1 global layer, B=32, 64K
context, kv_append then decode per layer), the global decode with two new
tokens per sequence (multi-token decode) and the last 4K positions of the 32K
global prompt as a chunk against the 28K cached ones (chunked prefill).
Inputs are seeded synthetic tensors already resident in HBM when timing starts.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

MI355X_BF16_DENSE_TFLOPS = 2500.0   # published dense bf16 MFMA peak
MI355X_HBM_GBS = 8000.0             # published HBM3E bandwidth

# HBM bytes per launch of each kernel from rocprofv3 --pmc FETCH_SIZE and then
# --pmc WRITE_SIZE on this benchmark, scaled by what the same counters read for
# a plain 256 MiB device copy (FETCH_SIZE x 2, WRITE_SIZE x 1), together with a
# digest of the kernel's code (comments and layout ignored) at the time.  Reported only while the sources
# still match; after any change to them the figure is stale and reads null.
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "global_gqa_rope_amd", "csrc")
MEASURED_TRAFFIC = {
    "prefill_attn": {"sources": ("prefill.hip", "common.h", "kernels.h"), "digest": "7316aabfd60968e3",
                     "bytes": 7968733504},
    "local_prefill_attn": {"sources": ("prefill.hip", "common.h", "kernels.h"), "digest": "7316aabfd60968e3",
                           "bytes": 8566853963},
    "chunk_prefill_attn": {"sources": ("prefill.hip", "common.h", "kernels.h"), "digest": "7316aabfd60968e3",
                           "bytes": 1592819541},
    "decode_splitk": {"sources": ("decode.hip", "common.h", "kernels.h"), "digest": "d34ee62a58bc973d",
                      "bytes": 4289380021},
    "multi_decode_splitk": {"sources": ("decode.hip", "common.h", "kernels.h"), "digest": "d34ee62a58bc973d",
                            "bytes": 4312982825},
    "prerotated_decode_splitk": {"sources": ("decode.hip", "common.h", "kernels.h"), "digest": "d34ee62a58bc973d",
                                 "bytes": 5355693905},
    "int8_decode_splitk": {"sources": ("decode.hip", "common.h", "kernels.h"), "digest": "d34ee62a58bc973d",
                           "bytes": 2173660475},
}


def measured_traffic(kernel):
    """Counter-measured HBM bytes per launch of `kernel`, or None if its sources changed since."""
    return MEASURED_TRAFFIC[kernel]["bytes"] if source_digest(kernel) == MEASURED_TRAFFIC[kernel]["digest"] else None


def source_digest(kernel):
    """SHA-256 prefix of the kernel's sources with // comments and whitespace removed."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in MEASURED_TRAFFIC[kernel]["sources"]:
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            code = re.sub(r"//[^\n]*", "", f.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-local", action="store_true", help="skip the local-layer prefill leg")
    ap.add_argument("--no-stack", action="store_true", help="skip the 6-layer stack decode leg")
    ap.add_argument("--no-verify", action="store_true", help="skip the 6-layer two-token verification leg")
    ap.add_argument("--no-multi", action="store_true", help="skip the multi-token decode leg")
    ap.add_argument("--no-int8", action="store_true", help="skip the int8-cache decode leg")
    ap.add_argument("--no-prerotated", action="store_true", help="skip the pre-rotated-cache decode leg")
    ap.add_argument("--no-chunk", action="store_true", help="skip the chunked prefill leg")
    ap.add_argument("--no-long", action="store_true", help="skip the 256K-context decode leg")
    ap.add_argument("--no-estack", action="store_true",
                    help="skip the 4:1 stack decode leg of the smaller models' layer types")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle sample")
    ap.add_argument("--no-calibrate", action="store_true",
                    help="skip the measured-peak probes (an MFMA chain on random bf16 operands, a streaming read)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy, the reference for HBM byte counters")
    ap.add_argument("--only", default=None,
                    help="comma list of legs to run after the global prefill (decode, multi, prerotated, int8, "
                         "chunk, local, stack, verify, long, estack); the others are skipped (for per-leg "
                         "profiles)")
    args = ap.parse_args()
    if args.only is not None:
        legs = {x for x in args.only.split(",") if x}
        known = {"decode", "multi", "prerotated", "int8", "chunk", "local", "stack", "verify", "long", "estack"}
        if not legs <= known:
            ap.error(f"--only: unknown legs {sorted(legs - known)}")
        for leg in known - legs:
            setattr(args, "no_" + leg, True)
    return args


def graph_of(fn, torch):
    """fn captured into a CUDA (HIP) graph after two warm-up calls on a side stream,
    or None if capture fails.  fn must launch only kernels (no allocation, no sync)."""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g
    except Exception as e:  # noqa: BLE001
        print(f"graph capture failed: {e}", file=sys.stderr)
        return None


def timed(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def bench_prefill(args, torch, api, W):
    wl = W.CONFIGS["global_prefill_32k"]
    shape, S = wl.layer, wl.seq_len
    dev = torch.device("cuda", 0)
    x = wl.draw(dev)
    lay = api.Layer.from_shape(shape, torch.bfloat16)
    kc = torch.empty((1, shape.n_kv_heads, S, shape.head_dim), dtype=torch.bfloat16, device=dev)
    out = torch.empty_like(x["q"])
    ws = api.workspace(api.gemma_attn_prefill_workspace_size(lay, 1, S), dev)

    def step():
        api.gemma_attn_prefill(lay, x["q"], x["k"], None, x["g_q"], x["g_k"], kc, None, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    api.profile_reset()
    api.profile_enable(True)
    sec = timed(step, args.steps, 0, torch)
    api.profile_enable(False)
    attn_ms, n_attn = api.profile_read("prefill_attn")
    prep_ms, n_prep = api.profile_read("prefill_prep")
    api.profile_reset()
    flops = wl.flops()
    return {
        "sec": sec, "flops": flops, "attn_ms": attn_ms / max(n_attn, 1), "prep_ms": prep_ms / max(n_prep, 1),
        "n_attn": n_attn, "wl": wl, "x": x,
    }


def bench_decode(args, torch, api, W):
    wl = W.CONFIGS["global_decode"]
    shape = wl.layer
    dev = torch.device("cuda", 0)
    lens = wl.lengths()
    B, cap, D = wl.batch, wl.cache_cap(), shape.head_dim
    kc = W.normal((B, shape.n_kv_heads, cap, D), wl.seed, "k_cache", torch.bfloat16, dev)
    q = W.normal((B, shape.n_q_heads, D), wl.seed, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, wl.seed, "g_q", False, torch.bfloat16, dev)
    lay = api.Layer.from_shape(shape, torch.bfloat16)
    seq = lens.to(dev)
    maxlen = int(lens.max())
    out = torch.empty_like(q)
    ws = api.workspace(api.gemma_attn_decode_workspace_size(lay, B, maxlen), dev)

    def step():
        api.gemma_attn_decode(lay, q, g_q, kc, None, seq, maxlen, out, ws)

    steps = args.decode_steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the whole call timed without per-launch events (they add ~0.015 ms to a
    # decode call), then a second timed loop for the kernels' own durations
    sec = timed(step, steps, 0, torch)
    api.profile_reset()
    api.profile_enable(True)
    timed(step, steps, 0, torch)
    api.profile_enable(False)
    split_ms, n_split = api.profile_read("decode_splitk")
    merge_ms, n_merge = api.profile_read("decode_merge")
    api.profile_reset()
    # kv_append of the step's new token, timed on its own
    kn = W.normal((B, shape.n_kv_heads, D), wl.seed, "k_new", torch.bfloat16, dev)
    g_k = W.gains(D, wl.seed, "g_k", False, torch.bfloat16, dev)
    pos = (lens - 1).to(dev)
    api.profile_enable(True)
    for _ in range(steps):
        api.kv_append(lay, kn, None, g_k, pos, kc, None)
    torch.cuda.synchronize()
    api.profile_enable(False)
    append_ms, n_append = api.profile_read("kv_append")
    api.profile_reset()
    nbytes = wl.kv_bytes(lens)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_decode(wl, lens, kc, q, g_q, args.cpu_seconds / 3, torch)
    del kc
    torch.cuda.empty_cache()
    return {"sec": sec, "bytes": nbytes, "split_ms": split_ms / max(n_split, 1),
            "merge_ms": merge_ms / max(n_merge, 1), "append_ms": append_ms / max(n_append, 1), "lens": lens,
            "cpu": cpu}


def bench_long_decode(args, torch, api, W):
    """Global K=V decode at the pages' longest context: B=4, every sequence at 262144 keys."""
    wl = W.CONFIGS["long_decode"]
    shape = wl.layer
    dev = torch.device("cuda", 0)
    lens = wl.lengths()
    B, cap, D = wl.batch, wl.cache_cap(), shape.head_dim
    kc = W.normal((B, shape.n_kv_heads, cap, D), wl.seed, "k_cache", torch.bfloat16, dev)
    q = W.normal((B, shape.n_q_heads, D), wl.seed, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, wl.seed, "g_q", False, torch.bfloat16, dev)
    lay = api.Layer.from_shape(shape, torch.bfloat16)
    seq = lens.to(dev)
    maxlen = int(lens.max())
    out = torch.empty_like(q)
    ws = api.workspace(api.gemma_attn_decode_workspace_size(lay, B, maxlen), dev)

    def step():
        api.gemma_attn_decode(lay, q, g_q, kc, None, seq, maxlen, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the whole call timed without per-launch events (they add ~0.015 ms to a
    # decode call), then a second timed loop for the kernels' own durations
    sec = timed(step, args.decode_steps, 0, torch)
    api.profile_reset()
    api.profile_enable(True)
    timed(step, args.decode_steps, 0, torch)
    api.profile_enable(False)
    split_ms, n_split = api.profile_read("decode_splitk")
    api.profile_reset()
    nbytes = wl.kv_bytes(lens)
    del kc
    torch.cuda.empty_cache()
    split_ms /= max(n_split, 1)
    return {
        "workload": "global K=V layer decode at 256K context: B=4, 262144 cached keys per sequence, 32q/4kv, d=512",
        "value": round(nbytes / sec / 1e9, 1), "unit": "GB/s", "ms_per_step": round(sec * 1e3, 4),
        "tokens_per_s": round(B / sec, 1), "kv_bytes": nbytes,
        "roofline": {"kernel": "decode_kernel<bf16,512,8,K=V>", "bound": "hbm",
                     "achieved": round(nbytes / (split_ms * 1e-3) / 1e9, 1), "peak": MI355X_HBM_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (split_ms * 1e-3) / 1e9 / MI355X_HBM_GBS, 4), "traffic": None,
                     "avg_ms": round(split_ms, 4)},
    }


def bench_local_prefill(args, torch, api, W):
    """Local (sliding-window) layer prefill: B=4, S=32K, 32q/16kv, d=256, W=1024."""
    wl = W.CONFIGS["local_prefill_32k"]
    shape, S, B = wl.layer, wl.seq_len, wl.batch
    dev = torch.device("cuda", 0)
    x = wl.draw(dev)
    lay = api.Layer.from_shape(shape, torch.bfloat16)
    kc = torch.empty((B, shape.n_kv_heads, shape.window, shape.head_dim), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    out = torch.empty_like(x["q"])
    ws = api.workspace(api.gemma_attn_prefill_workspace_size(lay, B, S), dev)

    def step():
        api.gemma_attn_prefill(lay, x["q"], x["k"], x["v"], x["g_q"], x["g_k"], kc, vc, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    api.profile_reset()
    api.profile_enable(True)
    sec = timed(step, args.steps, 0, torch)
    api.profile_enable(False)
    attn_ms, n_attn = api.profile_read("prefill_attn")
    api.profile_reset()
    flops = wl.flops()
    attn_ms /= max(n_attn, 1)
    del x, kc, vc, out, ws
    torch.cuda.empty_cache()
    attn = flops / (attn_ms * 1e-3) / 1e12
    return {
        "workload": "local layer prefill: B=4, S=32768, 32 query heads / 16 KV heads, d=256, window 1024, "
                    "RoPE theta=1e4, QKNorm",
        "value": round(flops / sec / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(sec * 1e3, 3),
        "flops_per_step": flops,
        "roofline": {"kernel": "prefill_attn_kernel<bf16,256,2>", "bound": "mfma", "achieved": round(attn, 2),
                     "peak": MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn / MI355X_BF16_DENSE_TFLOPS, 4),
                     "traffic": measured_traffic("local_prefill_attn"), "avg_ms": round(attn_ms, 4)},
    }


def bench_prefill_chunk(args, torch, api, W, start=28672):
    """The last 4K positions of the 32K global prompt as a chunk against the 28K cached ones."""
    wl = W.CONFIGS["global_prefill_32k"]
    shape, S = wl.layer, wl.seq_len
    dev = torch.device("cuda", 0)
    x = wl.draw(dev)
    lay = api.Layer.from_shape(shape, torch.bfloat16)
    kc = torch.empty((1, shape.n_kv_heads, S, shape.head_dim), dtype=torch.bfloat16, device=dev)
    api.gemma_attn_prefill(lay, x["q"][:, :start].contiguous(), x["k"][:, :start].contiguous(), None, x["g_q"],
                           x["g_k"], kc)
    q, k = x["q"][:, start:].contiguous(), x["k"][:, start:].contiguous()
    out = torch.empty_like(q)
    ws = api.workspace(api.gemma_attn_prefill_chunk_workspace_size(lay, 1, start, S - start), dev)

    def step():
        api.gemma_attn_prefill_chunk(lay, start, q, k, x["g_q"], x["g_k"], kc, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    api.profile_reset()
    api.profile_enable(True)
    sec = timed(step, args.steps, 0, torch)
    api.profile_enable(False)
    attn_ms, n_attn = api.profile_read("prefill_attn")
    prep_ms, n_prep = api.profile_read("prefill_prep")
    api.profile_reset()
    del x, kc, q, k, out, ws
    torch.cuda.empty_cache()
    flops = 4.0 * shape.n_q_heads * shape.head_dim * sum(range(start + 1, S + 1))
    attn_ms /= max(n_attn, 1)
    attn = flops / (attn_ms * 1e-3) / 1e12
    return {
        "workload": "global K=V layer, positions 28672..32767 of a 32K prompt as one chunk against the 28672 "
                    "cached positions (chunked prefill), 32q/4kv, d=512",
        "value": round(flops / sec / 1e12, 2), "unit": "TFLOP/s", "ms_per_step": round(sec * 1e3, 3),
        "flops_per_step": flops, "prep_avg_ms": round(prep_ms / max(n_prep, 1), 4),
        "roofline": {"kernel": "prefill_attn_kernel<bf16,512,8>", "bound": "mfma", "achieved": round(attn, 2),
                     "peak": MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn / MI355X_BF16_DENSE_TFLOPS, 4),
                     "traffic": measured_traffic("chunk_prefill_attn"),
                     "avg_ms": round(attn_ms, 4)},
    }


def bench_multi_decode(args, torch, api, W, q_len=2):
    """Global K=V decode workload (B=16, contexts up to 128K) with q_len new tokens per sequence."""
    wl = W.CONFIGS["global_decode"]
    shape = wl.layer
    dev = torch.device("cuda", 0)
    lens = wl.lengths()
    B, cap, D = wl.batch, wl.cache_cap(), shape.head_dim
    kc = W.normal((B, shape.n_kv_heads, cap, D), wl.seed, "k_cache", torch.bfloat16, dev)
    q = W.normal((B, q_len, shape.n_q_heads, D), wl.seed, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, wl.seed, "g_q", False, torch.bfloat16, dev)
    lay = api.Layer.from_shape(shape, torch.bfloat16)
    seq = lens.to(dev)
    maxlen = int(lens.max())
    out = torch.empty_like(q)
    ws = api.workspace(api.gemma_attn_decode_multi_workspace_size(lay, B, q_len, maxlen), dev)

    def step():
        api.gemma_attn_decode_multi(lay, q, g_q, kc, None, seq, maxlen, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the whole call timed without per-launch events (they add ~0.015 ms to a
    # decode call), then a second timed loop for the kernels' own durations
    sec = timed(step, args.decode_steps, 0, torch)
    api.profile_reset()
    api.profile_enable(True)
    timed(step, args.decode_steps, 0, torch)
    api.profile_enable(False)
    split_ms, n_split = api.profile_read("decode_splitk")
    api.profile_reset()
    nbytes = wl.kv_bytes(lens)
    del kc
    torch.cuda.empty_cache()
    gbs = nbytes / sec / 1e9
    split_ms /= max(n_split, 1)
    return {
        "workload": f"global K=V layer, {q_len} new tokens per sequence (multi-token decode): B=16, "
                    "context ~ U[4096,131072] (seed 0), 32q/4kv, d=512",
        "q_len": q_len, "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(sec * 1e3, 4),
        "tokens_per_s": round(B * q_len / sec, 1), "kv_bytes": nbytes,
        "roofline": {"kernel": "decode_kernel<bf16,512,8,K=V>", "bound": "hbm",
                     "achieved": round(nbytes / (split_ms * 1e-3) / 1e9, 1), "peak": MI355X_HBM_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (split_ms * 1e-3) / 1e9 / MI355X_HBM_GBS, 4),
                     "traffic": measured_traffic("multi_decode_splitk") if q_len == 2 else None,
                     "avg_ms": round(split_ms, 4), "launches_per_call": round(n_split / max(args.decode_steps, 1), 2)},
    }


def bench_int8_decode(args, torch, api, W):
    """The global decode workload on an int8 K=V cache (codes + one fp32 scale per row)."""
    from dataclasses import replace
    wl = W.CONFIGS["global_decode"]
    shape = wl.layer
    dev = torch.device("cuda", 0)
    lens = wl.lengths()
    B, cap, D = wl.batch, wl.cache_cap(), shape.head_dim
    lay = replace(api.Layer.from_shape(shape, torch.bfloat16), cache_format=1)
    cache = api.new_cache(lay, B, cap, dev)
    for b in range(B):
        c, sc = W.int8_rows((1, shape.n_kv_heads, cap, D), 71 + b, dev)
        cache.codes()[b:b + 1].copy_(c)
        cache.scales()[b:b + 1].copy_(sc)
        del c, sc
    q = W.normal((B, shape.n_q_heads, D), wl.seed, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, wl.seed, "g_q", False, torch.bfloat16, dev)
    seq = lens.to(dev)
    maxlen = int(lens.max())
    out = torch.empty_like(q)
    ws = api.workspace(api.gemma_attn_decode_workspace_size(lay, B, maxlen), dev)

    def step():
        api.gemma_attn_decode(lay, q, g_q, cache, None, seq, maxlen, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the whole call timed without per-launch events (they add ~0.015 ms to a
    # decode call), then a second timed loop for the kernels' own durations
    sec = timed(step, args.decode_steps, 0, torch)
    api.profile_reset()
    api.profile_enable(True)
    timed(step, args.decode_steps, 0, torch)
    api.profile_enable(False)
    split_ms, n_split = api.profile_read("decode_splitk")
    api.profile_reset()
    kn = W.normal((B, shape.n_kv_heads, D), wl.seed, "k_new", torch.bfloat16, dev)
    g_k = W.gains(D, wl.seed, "g_k", False, torch.bfloat16, dev)
    pos = (lens - 1).to(dev)
    api.profile_enable(True)
    for _ in range(args.decode_steps):
        api.kv_append(lay, kn, None, g_k, pos, cache, None)
    torch.cuda.synchronize()
    api.profile_enable(False)
    append_ms, n_append = api.profile_read("kv_append")
    api.profile_reset()
    rows = int(lens.sum()) * shape.n_kv_heads
    nbytes = rows * (D + 4)          # each cached row's codes and scale, once
    del cache
    torch.cuda.empty_cache()
    split_ms /= max(n_split, 1)
    return {
        "workload": "global K=V layer decode on an int8 cache (codes + fp32 row scale): B=16, "
                    "context ~ U[4096,131072] (seed 0), 32q/4kv, d=512",
        "value": round(nbytes / sec / 1e9, 1), "unit": "GB/s", "ms_per_step": round(sec * 1e3, 4),
        "tokens_per_s": round(B / sec, 1), "kv_bytes": nbytes,
        "roofline": {"kernel": "decode_kernel<bf16,512,8,K=V,int8>", "bound": "hbm",
                     "achieved": round(nbytes / (split_ms * 1e-3) / 1e9, 1), "peak": MI355X_HBM_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (split_ms * 1e-3) / 1e9 / MI355X_HBM_GBS, 4),
                     "traffic": measured_traffic("int8_decode_splitk"),
                     "avg_ms": round(split_ms, 4)},
        "kv_append_avg_ms": round(append_ms / max(n_append, 1), 4),
    }


def bench_prerotated_decode(args, torch, api, W):
    """The global decode workload on a pre-rotated ("1.25 d") K=V cache: rows plus rotated heads."""
    from dataclasses import replace
    wl = W.CONFIGS["global_decode"]
    shape = wl.layer
    dev = torch.device("cuda", 0)
    lens = wl.lengths()
    B, cap, D = wl.batch, wl.cache_cap(), shape.head_dim
    lay = replace(api.Layer.from_shape(shape, torch.bfloat16), cache_format=2)
    cache = api.new_cache(lay, B, cap, dev)
    for b in range(B):
        cache.rows()[b:b + 1].copy_(W.normal((1, shape.n_kv_heads, cap, D), wl.seed + b, "k_cache",
                                             torch.bfloat16, dev))
        cache.heads()[b:b + 1].copy_(W.normal((1, shape.n_kv_heads, cap, cache.head_width), wl.seed + b, "k_new",
                                              torch.bfloat16, dev))
    q = W.normal((B, shape.n_q_heads, D), wl.seed, "q_dec", torch.bfloat16, dev)
    g_q = W.gains(D, wl.seed, "g_q", False, torch.bfloat16, dev)
    seq = lens.to(dev)
    maxlen = int(lens.max())
    out = torch.empty_like(q)
    ws = api.workspace(api.gemma_attn_decode_workspace_size(lay, B, maxlen), dev)

    def step():
        api.gemma_attn_decode(lay, q, g_q, cache, None, seq, maxlen, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the whole call timed without per-launch events (they add ~0.015 ms to a
    # decode call), then a second timed loop for the kernels' own durations
    sec = timed(step, args.decode_steps, 0, torch)
    api.profile_reset()
    api.profile_enable(True)
    timed(step, args.decode_steps, 0, torch)
    api.profile_enable(False)
    split_ms, n_split = api.profile_read("decode_splitk")
    api.profile_reset()
    rows = int(lens.sum()) * shape.n_kv_heads
    nbytes = rows * (D + cache.head_width) * 2     # each cached row and its head, once
    del cache
    torch.cuda.empty_cache()
    split_ms /= max(n_split, 1)
    return {
        "workload": "global K=V layer decode on a pre-rotated cache (rows + rotated 128-dim heads, 1.25 d "
                    "per row): B=16, context ~ U[4096,131072] (seed 0), 32q/4kv, d=512",
        "value": round(nbytes / sec / 1e9, 1), "unit": "GB/s", "ms_per_step": round(sec * 1e3, 4),
        "tokens_per_s": round(B / sec, 1), "kv_bytes": nbytes,
        "roofline": {"kernel": "decode_kernel<bf16,512,8,K=V,pre-rotated>", "bound": "hbm",
                     "achieved": round(nbytes / (split_ms * 1e-3) / 1e9, 1), "peak": MI355X_HBM_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (split_ms * 1e-3) / 1e9 / MI355X_HBM_GBS, 4),
                     "traffic": measured_traffic("prerotated_decode_splitk"), "avg_ms": round(split_ms, 4)},
    }


def bench_stack_decode(args, torch, api, W, local="stack_decode_local", glob="stack_decode_global", n_local=5,
                       workload=None):
    """One decode step of a stack of n_local local layers and one global layer, each layer kv_append then
    decode."""
    wl_l, wl_g = W.CONFIGS[local], W.CONFIGS[glob]
    dev = torch.device("cuda", 0)
    B = wl_l.batch
    layers = []
    for i, wl in enumerate([wl_l] * n_local + [wl_g]):
        shape = wl.layer
        D, Hkv = shape.head_dim, shape.n_kv_heads
        seed = wl.seed + i
        cap = wl.cache_cap()
        kc = W.normal((B, Hkv, cap, D), seed, "k_cache", torch.bfloat16, dev)
        vc = None if shape.kv_shared else W.normal((B, Hkv, cap, D), seed, "v_cache", torch.bfloat16, dev)
        lens = wl.lengths()
        lay = api.Layer.from_shape(shape, torch.bfloat16)
        layers.append({
            "lay": lay, "kc": kc, "vc": vc, "seq": lens.to(dev), "pos": (lens - 1).to(dev), "max": int(lens.max()),
            "q": W.normal((B, shape.n_q_heads, D), seed, "q_dec", torch.bfloat16, dev),
            "kn": W.normal((B, Hkv, D), seed, "k_new", torch.bfloat16, dev),
            "vn": None if shape.kv_shared else W.normal((B, Hkv, D), seed, "v_new", torch.bfloat16, dev),
            "g_q": W.gains(D, seed, "g_q", False, torch.bfloat16, dev),
            "g_k": W.gains(D, seed, "g_k", False, torch.bfloat16, dev),
            "out": torch.empty((B, shape.n_q_heads, D), dtype=torch.bfloat16, device=dev),
            "ws": api.workspace(api.gemma_attn_decode_workspace_size(lay, B, int(lens.max())), dev),
            "bytes": wl.kv_bytes(lens),
        })

    def step():
        for L in layers:
            api.kv_append(L["lay"], L["kn"], L["vn"], L["g_k"], L["pos"], L["kc"], L["vc"])
            api.gemma_attn_decode(L["lay"], L["q"], L["g_q"], L["kc"], L["vc"], L["seq"], L["max"], L["out"],
                                  L["ws"])

    steps = max(args.decode_steps // 2, 8)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sec = timed(step, steps, 0, torch)
    g = graph_of(step, torch)
    graph_sec = timed(g.replay, steps, 2, torch) if g is not None else None
    del g
    nbytes = sum(L["bytes"] for L in layers)
    del layers
    torch.cuda.empty_cache()
    gbs = nbytes / sec / 1e9
    return {
        "workload": workload or ("6-layer decode step: 5 local (32q/16kv, d=256, W=1024) + 1 global K=V (32q/4kv, "
                                 "d=512), B=32, context 65536, kv_append then decode per layer (graph_ms_per_step: "
                                 "the same step replayed as one HIP graph)"),
        "ms_per_step": round(sec * 1e3, 4),
        "graph_ms_per_step": None if graph_sec is None else round(graph_sec * 1e3, 4),
        "tokens_per_s": round(B / sec, 1), "kv_bytes": nbytes,
        "value": round(gbs, 1), "unit": "GB/s", "steps": steps,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": MI355X_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / MI355X_HBM_GBS, 4)},
    }


def calibrate(torch, api):
    """Rates this GPU reaches on the two bounding resources: chains of 32x32x16
    bf16 MFMAs on random operands (4 per SIMD, 4 chains each), and a streaming
    read of 4 GiB in 16-byte loads.  Best of 5 runs, timed with events on the
    stream the probes run on."""
    import ctypes
    from global_gqa_rope_amd import _lib
    lib = _lib.load()
    dev = torch.device("cuda", 0)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream()
    ops = torch.randn(1 << 20, device=dev).to(torch.bfloat16)          # 131072 random 16-byte pieces
    n_wgs, iters = 4 * cus, 4096
    sink = torch.empty(n_wgs * 256, dtype=torch.float32, device=dev)

    def run_mfma():
        _lib.check(lib.gemma_attn_calibrate_mfma(ops.data_ptr(), ops.numel() // 8, iters, n_wgs, sink.data_ptr(),
                                                 stream.cuda_stream))

    buf = torch.randn((4 << 30) // 4, device=dev)                      # 4 GiB of random floats
    sinku = torch.empty(8 * cus, dtype=torch.int32, device=dev)

    def run_stream():
        _lib.check(lib.gemma_attn_calibrate_stream(buf.data_ptr(), buf.numel() * 4, 8 * cus, sinku.data_ptr(),
                                                   stream.cuda_stream))

    def best_ms(fn):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        return min(times)

    mfma_ms = best_ms(run_mfma)
    flops = n_wgs * 4 * 4 * iters * 32768.0
    stream_ms = best_ms(run_stream)
    nbytes = buf.numel() * 4
    del ops, sink, buf, sinku
    torch.cuda.empty_cache()
    tf = flops / (mfma_ms * 1e-3) / 1e12
    gbs = nbytes / (stream_ms * 1e-3) / 1e9
    return {
        "mfma_bf16": {"value": round(tf, 1), "unit": "TFLOP/s", "frac_of_published": round(tf / MI355X_BF16_DENSE_TFLOPS, 4),
                      "probe": f"{n_wgs} workgroups x 4 waves, 4 independent chains of {iters} 32x32x16 bf16 MFMAs "
                               "per wave on random N(0,1) operands"},
        "hbm_read": {"value": round(gbs, 1), "unit": "GB/s", "frac_of_published": round(gbs / MI355X_HBM_GBS, 4),
                     "probe": f"{8 * cus} workgroups read 4 GiB once, each a contiguous chunk in 16-byte loads, 8 in flight "
                              "per lane"},
    }


def with_measured_peak(roof, cal):
    """Adds the fraction of the measured peak to a roofline object."""
    if cal is None or roof is None:
        return
    key = "mfma_bf16" if roof.get("bound") == "mfma" else "hbm_read"
    roof["measured_peak"] = cal[key]["value"]
    roof["frac_of_measured_peak"] = round(roof["achieved"] / cal[key]["value"], 4)


def host_info():
    """The host the oracle runs on: core counts, CPU model and the BLAS threads numpy uses."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = None
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"nproc": os.cpu_count(), "affinity": affinity, "cpu_model": model, "blas_threads": blas}


def cpu_baseline_decode(wl, lens, kc, q, g_q, budget_s, torch):
    """The oracle's decode on whole sequences of the same B=16 decode workload
    (every KV head of a sequence, all its cached positions), as GB/s of cache."""
    import oracle as O
    shape = wl.layer
    ol = O.OracleLayer(shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.window, shape.kv_shared,
                       shape.rope_theta, shape.rope_fraction, shape.norm_eps)
    g64 = g_q.to("cpu", torch.float64).numpy()
    order = np.argsort(lens.numpy())          # shortest sequences first, so the budget covers several
    done, nbytes, elapsed = [], 0, 0.0
    for b in order:
        if elapsed >= budget_s:
            break
        L = int(lens[b])
        kb = kc[b:b + 1, :, :L].to("cpu", torch.float64).numpy()
        qb = q[b:b + 1].to("cpu", torch.float64).numpy()
        t0 = time.perf_counter()
        O.decode_from_cache(ol, qb, g64, kb, None, np.array([L]))
        elapsed += time.perf_counter() - t0
        done.append(L)
        nbytes += L * shape.n_kv_heads * shape.head_dim * 2
    return {"value": nbytes / elapsed / 1e9, "unit": "GB/s", "kind": "oracle",
            "sample": f"{len(done)} whole sequences of the B=16 global decode (lengths {min(done)}..{max(done)}, "
                      f"all 4 KV heads), float64 numpy, {elapsed:.1f} s timed (the host copy and cast excluded); "
                      "GB/s counts the bf16 cache bytes the step reads"}


def bench_stack_verify(args, torch, api, W, q_len=2):
    """One verification step of the 6-layer stack (5 local + 1 global): each
    layer appends q_len drafted tokens per sequence, then checks them in one
    gemma_attn_decode_multi call (local rings of W + q_len - 1 slots)."""
    wl_l, wl_g = W.CONFIGS["stack_decode_local"], W.CONFIGS["stack_decode_global"]
    dev = torch.device("cuda", 0)
    B = wl_l.batch
    layers = []
    for i, wl in enumerate([wl_l] * 5 + [wl_g]):
        shape = wl.layer
        D, Hkv = shape.head_dim, shape.n_kv_heads
        seed = wl.seed + i
        cap = shape.window + q_len - 1 if shape.window else wl.ctx_hi + q_len
        kc = W.normal((B, Hkv, cap, D), seed, "k_cache", torch.bfloat16, dev)
        vc = None if shape.kv_shared else W.normal((B, Hkv, cap, D), seed, "v_cache", torch.bfloat16, dev)
        lens = wl.lengths() + (q_len - 1)          # context + q_len new tokens
        lay = api.Layer.from_shape(shape, torch.bfloat16)
        n_keys = [min(int(n), cap) if shape.window else int(n) for n in lens]
        layers.append({
            "lay": lay, "kc": kc, "vc": vc, "seq": lens.to(dev), "max": int(lens.max()),
            "pos": [(lens - q_len + j).to(dev) for j in range(q_len)],
            "q": W.normal((B, q_len, shape.n_q_heads, D), seed, "q_dec", torch.bfloat16, dev),
            "kn": W.normal((q_len, B, Hkv, D), seed, "k_new", torch.bfloat16, dev),
            "vn": None if shape.kv_shared else W.normal((q_len, B, Hkv, D), seed, "v_new", torch.bfloat16, dev),
            "g_q": W.gains(D, seed, "g_q", False, torch.bfloat16, dev),
            "g_k": W.gains(D, seed, "g_k", False, torch.bfloat16, dev),
            "out": torch.empty((B, q_len, shape.n_q_heads, D), dtype=torch.bfloat16, device=dev),
            "ws": api.workspace(api.gemma_attn_decode_multi_workspace_size(lay, B, q_len, int(lens.max())), dev),
            "bytes": sum(n_keys) * Hkv * D * 2 * (1 if shape.kv_shared else 2),
        })

    def step():
        for L in layers:
            for j in range(q_len):
                api.kv_append(L["lay"], L["kn"][j], None if L["vn"] is None else L["vn"][j], L["g_k"], L["pos"][j],
                              L["kc"], L["vc"])
            api.gemma_attn_decode_multi(L["lay"], L["q"], L["g_q"], L["kc"], L["vc"], L["seq"], L["max"],
                                        L["out"], L["ws"])

    steps = max(args.decode_steps // 2, 8)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    sec = timed(step, steps, 0, torch)
    g = graph_of(step, torch)
    graph_sec = timed(g.replay, steps, 2, torch) if g is not None else None
    del g
    nbytes = sum(L["bytes"] for L in layers)
    del layers
    torch.cuda.empty_cache()
    gbs = nbytes / sec / 1e9
    return {
        "workload": f"6-layer verification step of {q_len} drafted tokens per sequence: 5 local (32q/16kv, d=256, "
                    f"W=1024, ring of {1024 + q_len - 1} slots) + 1 global K=V (32q/4kv, d=512), B=32, context "
                    "65536, per layer kv_append of each token then one multi-token decode (graph_ms_per_step: replayed "
                    "as one HIP graph)",
        "q_len": q_len, "ms_per_step": round(sec * 1e3, 4),
        "graph_ms_per_step": None if graph_sec is None else round(graph_sec * 1e3, 4),
        "tokens_per_s": round(B * q_len / sec, 1),
        "kv_bytes": nbytes, "value": round(gbs, 1), "unit": "GB/s", "steps": steps,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": MI355X_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / MI355X_HBM_GBS, 4)},
    }


def cpu_baseline(pre, budget_s, torch):
    """The oracle as it stands, on a bounded sample of the same prefill."""
    import oracle as O
    host = host_info()
    cores = host["blas_threads"] or host["nproc"] or 1
    wl, x = pre["wl"], pre["x"]
    shape = wl.layer
    ol = O.OracleLayer(shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.window, shape.kv_shared,
                       shape.rope_theta, shape.rope_fraction, shape.norm_eps)
    S = wl.seq_len
    rng = np.random.default_rng(0)
    k64 = x["k"].to("cpu", torch.float64).numpy()
    g_q = x["g_q"].to("cpu", torch.float64).numpy()
    g_k = x["g_k"].to("cpu", torch.float64).numpy()
    done_rows, flops, elapsed = 0, 0.0, 0.0
    t0 = time.perf_counter()
    while elapsed < budget_s and done_rows < 256:
        rows = np.sort(rng.integers(0, S, size=4))
        q_rows = x["q"][:, torch.as_tensor(rows, device=x["q"].device)].to("cpu", torch.float64).numpy()
        hi = int(rows.max()) + 1
        O.prefill(ol, q_rows, k64[:, :hi], None, g_q, g_k, rows=rows, q_at_rows=True)
        done_rows += len(rows)
        flops += 4.0 * shape.n_q_heads * shape.head_dim * float(np.sum(rows + 1))
        elapsed = time.perf_counter() - t0
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done_rows} random query rows of the same 32K global prefill (all 32 heads), "
                      f"float64 numpy, {elapsed:.1f} s incl. key norm/rotation per call",
            "host": host}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build runs on a single "
              "MI355X and has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    from global_gqa_rope_amd import api
    from global_gqa_rope_amd import workloads as W

    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cpu_dec = None
    pre = bench_prefill(args, torch, api, W)
    tflops = pre["flops"] / pre["sec"] / 1e12
    attn_tflops = pre["flops"] / (pre["attn_ms"] * 1e-3) / 1e12
    line = {
        "metric": "global K=V attn prefill TFLOP/s @32K; decode KV GB/s (% of MI355X roofline)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["sec"] * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k, QKNorm gains N(1,0.1))",
        "config": {"workload": "global K=V layer prefill: B=1, S=32768, 32 query heads / 4 K=V heads, "
                               "d=512, causal, p-RoPE p=0.25 theta=1e6, QKNorm",
                   "batch": 1, "seq_len": 32768, "flops_per_step": pre["flops"]},
        "roofline": {"kernel": "prefill_attn_kernel<bf16,512,8>", "bound": "mfma",
                     "achieved": round(attn_tflops, 2), "peak": MI355X_BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / MI355X_BF16_DENSE_TFLOPS, 4),
                     "traffic": measured_traffic("prefill_attn"),
                     "avg_ms": round(pre["attn_ms"], 4), "prep_avg_ms": round(pre["prep_ms"], 4)},
    }
    if not args.no_decode:
        dec = bench_decode(args, torch, api, W)
        gbs = dec["bytes"] / dec["sec"] / 1e9
        split_gbs = dec["bytes"] / (dec["split_ms"] * 1e-3) / 1e9
        line["decode"] = {
            "workload": "global K=V layer decode: B=16, context ~ U[4096,131072] (seed 0), 32q/4kv, d=512",
            "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(dec["sec"] * 1e3, 4),
            "kv_bytes": dec["bytes"],
            "roofline": {"kernel": "decode_kernel<bf16,512,8,K=V>", "bound": "hbm",
                         "achieved": round(split_gbs, 1), "peak": MI355X_HBM_GBS, "unit": "GB/s",
                         "frac": round(split_gbs / MI355X_HBM_GBS, 4),
                         "traffic": measured_traffic("decode_splitk"),
                         "avg_ms": round(dec["split_ms"], 4), "merge_avg_ms": round(dec["merge_ms"], 4)},
            "kv_append_avg_ms": round(dec["append_ms"], 4),
        }
        cpu_dec = dec["cpu"]
    if not args.no_multi:
        line["multi_token_decode"] = bench_multi_decode(args, torch, api, W)
        # a 4-token draft on the G = 8 layer: 32 query columns, two column groups in one launch
        line["multi_token_decode_4"] = bench_multi_decode(args, torch, api, W, q_len=4)
    if not args.no_prerotated:
        line["prerotated_decode"] = bench_prerotated_decode(args, torch, api, W)
        if "decode" in line:
            line["prerotated_decode"]["speedup_vs_kv_shared_cache"] = round(
                line["decode"]["ms_per_step"] / line["prerotated_decode"]["ms_per_step"], 3)
    if not args.no_int8:
        line["int8_decode"] = bench_int8_decode(args, torch, api, W)
        if "decode" in line:
            line["int8_decode"]["speedup_vs_bf16_cache"] = round(
                line["decode"]["ms_per_step"] / line["int8_decode"]["ms_per_step"], 3)
    if not args.no_chunk:
        line["prefill_chunk"] = bench_prefill_chunk(args, torch, api, W)
    if not args.no_local:
        line["local_prefill"] = bench_local_prefill(args, torch, api, W)
    if not args.no_stack:
        line["stack_decode"] = bench_stack_decode(args, torch, api, W)
    if not args.no_verify:
        line["stack_verify"] = bench_stack_verify(args, torch, api, W)
    if not args.no_long:
        line["long_decode"] = bench_long_decode(args, torch, api, W)
    if not args.no_estack:
        line["e_stack_decode"] = bench_stack_decode(
            args, torch, api, W, "e_stack_local", "e_stack_global", 4,
            "5-layer decode step of the smaller models' layer types, 4:1: 4 local (8q/2kv, d=256, W=512) + 1 global "
            "with a separate V cache (8q/2kv, d=512, keys stored rotated), B=32, context 65536, kv_append then "
            "decode per layer (graph_ms_per_step: the same step replayed as one HIP graph)")
    if not args.no_calibrate:
        cal = calibrate(torch, api)
        line["calibration"] = cal
        with_measured_peak(line["roofline"], cal)
        for k, v in line.items():
            if isinstance(v, dict) and isinstance(v.get("roofline"), dict):
                with_measured_peak(v["roofline"], cal)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(pre, args.cpu_seconds, torch)
        if not args.no_decode and cpu_dec is not None:
            line["cpu_baseline"]["decode"] = cpu_dec
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
