"""Benchmark: absorbed MLA decode over a paged latent cache on one MI355X.

A step is one pass of the whole hot path for one layer: mla_absorb_q ->
mla_decode_paged -> stage 2 + up-projection (mla_combine_up_proj, one pass;
--separate-stage2 runs mla_combine_splits and mla_up_proj instead). The default workload is
B=16 sequences of 65536 cached tokens with 60 layers of latent cache resident
(72.5 GB); step k uses layer k mod 60, so every step reads its 1.2 GB of cache
from HBM (it cannot be served by the 256 MB last-level cache).

Prints one JSON line (rank 0):
  value            whole-step throughput, algorithmic TFLOP/s
  roofline         the dominant kernel (mla_decode_paged) against HBM
  cpu_baseline     the fp64 CPU oracle on a bounded sample of the workload
plus effective KV GB/s, per-kernel times and, under next_rows, the cache
append and query rotation, the step as one launch (mla_decode_step) against
the four kernels it fuses, the same step over the 8-bit cache
(mla_decode_paged_fp8) and over the 4-bit cache (mla_decode_paged_mxfp4), and
for chunks of s_q > 1 the decompressed branch.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
FLOP_PER_PAIR = 128 * 2 * (576 + 512)  # all heads, one (query, key) pair: QK over 576 + PV over 512
KV_BYTES_PER_TOKEN = 576 * 2
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_paged_long_hbm_traffic.json")
TRAFFIC_FILES = {
    "bf16": TRAFFIC_FILE,
    "fp8": os.path.join(ROOT, "profiles", "decode_paged_fp8_long_hbm_traffic.json"),
    "mxfp4": os.path.join(ROOT, "profiles", "decode_paged_mxfp4_long_hbm_traffic.json"),
}
FORMAT_HEADERS = {"bf16": (), "fp8": ("fp8_cache.hpp",), "mxfp4": ("mxfp4_cache.hpp",)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    # the board's power controller overshoots during the first ~15 ms of
    # sustained load (decode slows by up to 40%, then recovers); 100 warmup
    # steps (~30 ms) start the timed region in the settled state
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="long", choices=["single", "uniform", "ragged", "long", "prefill"])
    p.add_argument("--layers", type=int, default=0, help="resident cache layers (0: workload default)")
    p.add_argument("--splits", type=int, default=0, help="num_splits (0: library recommendation)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--separate-stage2", action="store_true",
                   help="run mla_combine_splits and mla_up_proj as two kernels instead of mla_combine_up_proj")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle time for the baseline")
    p.add_argument("--no-fp8", action="store_true", help="skip the 8-bit cache leg")
    p.add_argument("--no-mxfp4", action="store_true", help="skip the 4-bit cache leg")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only copy 1 GiB device to device three times (the known-size reference for "
                        "rocprofv3 FETCH_SIZE / WRITE_SIZE) and exit")
    return p.parse_args()


def visible_pairs(seqlens, s_q):
    """(query, key) pairs the causal rule admits: query i sees L - s_q + i + 1 keys."""
    tot = 0
    for L in seqlens:
        for i in range(s_q):
            tot += max(L - s_q + i + 1, 0)
    return tot


def kernel_source_digest(fmt="bf16"):
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_body.hpp", "mla_device.hpp", "decode.hpp") + FORMAT_HEADERS[fmt]:
        with open(os.path.join(ROOT, "mla_latent_kv_06_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, splits, fmt="bf16"):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source and launch configuration."""
    try:
        with open(TRAFFIC_FILES[fmt]) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("kernel_digest") != kernel_source_digest(fmt) or t.get("workload") != workload
            or t.get("splits") != splits):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inp_cpu, q_abs_cpu, target_s):
    """fp64 oracle (absorbed path) on whole sequences of the workload until ~target_s."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    kvb = O.bf16_bits(inp_cpu["kv_cache"])
    bt = inp_cpu["block_table"].numpy()
    sl = inp_cpu["seqlens"].numpy()
    qa = O.as_f64(q_abs_cpu)
    qr = O.as_f64(inp_cpu["q_r"])
    s_q = qa.shape[1]
    scale = 1.0 / math.sqrt(192)
    t0 = time.perf_counter()
    done, flop = 0, 0.0
    while time.perf_counter() - t0 < target_s:
        b = done % qa.shape[0]
        O.decode_absorbed(qa[b:b + 1], qr[b:b + 1], kvb, bt[b:b + 1], sl[b:b + 1], scale)
        flop += visible_pairs([int(sl[b])], s_q) * FLOP_PER_PAIR
        done += 1
    dt = time.perf_counter() - t0
    return {
        "value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
        "sample": f"fp64 numpy absorbed path (gather, scores, softmax, P.c_KV) over {done} whole sequences "
                  f"(cycling through the {qa.shape[0]} of layer 0), all 128 heads, {dt:.1f} s; "
                  f"host logical CPUs {os.cpu_count()}, "
                  f"affinity {len(os.sched_getaffinity(0))}",
        "seconds": dt,
    }


def time_next_rows(M, torch, kv, tables, seqlens, lens, B, s_q, layers, reps=200):
    """The step before the path at this workload: writing the chunk's tokens
    into the cache (c_KV copied, k_R rotated) and rotating the queries' RoPE
    parts. Both are launch-bound at decode sizes, so `reps` launches are
    captured in one HIP graph and the replay is timed with HIP events: the
    per-launch time is the GPU's, without Python dispatch in between."""
    dev = kv.device
    T = B * s_q
    g = torch.Generator(device=dev).manual_seed(77)
    c_new = torch.randn((B, s_q, 512), device=dev, generator=g).to(torch.bfloat16)
    kr_new = torch.randn((B, s_q, 64), device=dev, generator=g).to(torch.bfloat16)
    q_rot = torch.randn((B, s_q, 128, 64), device=dev, generator=g).to(torch.bfloat16)
    rope = M.mla_rope_table(max(lens) + 1, device=dev)
    # per token: append reads 1024 + 128 input bytes and 32 (cos, sin) pairs,
    # writes a 1152-byte row; the query rotation reads and writes 128 heads x
    # 64 bf16 and reads the same 32 pairs
    cases = [("mla_append_latent", lambda k: M.mla_append_latent(kv[k % layers], tables[k % layers], seqlens,
                                                                 c_new, kr_new, rope), T * (1024 + 128 + 256 + 1152)),
             ("mla_rope_q", lambda k: M.mla_rope_q(q_rot, seqlens, rope), T * (2 * 128 * 64 * 2 + 256))]
    res = {}
    for name, fn, nbytes in cases:
        for k in range(10):
            fn(k)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(reps):
                fn(k)
        graph.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us_per_launch": round(us, 2), "bytes_per_launch": nbytes, "achieved_gbps": round(gbs, 1),
                     "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "timing": f"HIP graph of {reps} launches"}
        del graph
    return res


def time_decompressed_branch(M, torch, kv, tables, seqlens, lens, q_c, q_r, w_uk, w_uv, s_q, layers, reps=5):
    """The decompressed branch (per-head K/V, then causal MHA) at this
    workload, timed per kernel with HIP events, with its algorithmic FLOP
    and bytes. The absorbed step above is the comparison the dispatch rule
    makes."""
    B = len(lens)
    max_len = -(-max(lens) // 64) * 64
    shape = (B, 128, max_len, 128)
    k_nope = torch.empty(shape, dtype=torch.bfloat16, device=kv.device)
    v = torch.empty(shape, dtype=torch.float16, device=kv.device)
    out = torch.empty((B, s_q, 128, 128), dtype=torch.bfloat16, device=kv.device)
    lse = torch.empty((B, s_q, 128), dtype=torch.float32, device=kv.device)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for k in range(2 + reps):
        layer = k % layers
        e = ev[k - 2] if k >= 2 else None
        if e: e[0].record(stream)
        M.mla_decompress_kv(kv[layer], tables[layer], seqlens, w_uk, w_uv, max_len, k_nope=k_nope, v=v)
        if e: e[1].record(stream)
        M.mla_prefill_mha(q_c, q_r, k_nope, v, kv[layer], tables[layer], seqlens, out=out, lse=lse)
        if e: e[2].record(stream)
    torch.cuda.synchronize()
    t_dec = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    t_mha = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
    tokens = sum(lens)
    flop_dec = 2.0 * tokens * 512 * (2 * 128 * 128)
    pairs = visible_pairs(lens, s_q)
    flop_mha = 2.0 * pairs * 128 * (192 + 128)
    bytes_dec = tokens * (1024 + 2 * 128 * 128 * 2) + 2 * 128 * 128 * 512 * 2
    del k_nope, v
    return {
        "mla_decompress_kv": {"ms": round(t_dec, 4), "flop": flop_dec, "tflops": round(flop_dec / (t_dec * 1e-3) / 1e12, 1),
                              "mfma_frac": round(flop_dec / (t_dec * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                              "bytes": bytes_dec, "gbps": round(bytes_dec / (t_dec * 1e-3) / 1e9, 1)},
        "mla_prefill_mha": {"ms": round(t_mha, 4), "flop": flop_mha, "tflops": round(flop_mha / (t_mha * 1e-3) / 1e12, 1),
                            "mfma_frac": round(flop_mha / (t_mha * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "branch_ms": round(t_dec + t_mha, 4),
    }


QUANT_FORMATS = {
    # page bytes, bytes per token, what the cache holds
    "fp8": (41216, 512 + 64 * 2 + 4, "c_KV in E4M3 with a power-of-two scale per token, k_R in bf16"),
    "mxfp4": (25600, 256 + 64 * 2 + 16, "c_KV in MXFP4 (E2M1 with an E8M0 scale per 32 dims), k_R in bf16"),
}


def time_quantized_cache(M, torch, fmt, kv, tables, seqlens, lens, q_c, q_r, w_uk, w_uv, S, layers, steps, warmup,
                         flop_step, flop_attn, q_bytes, olat_bytes, workload):
    """The same step over a quantized cache: every resident layer converted once
    (mla_quantize_cache_<fmt>), then absorb -> mla_decode_paged_<fmt> ->
    mla_combine_up_proj, rotating through the layers as the main loop does."""
    page_bytes, per_token, what = QUANT_FORMATS[fmt]
    quantize = getattr(M, f"mla_quantize_cache_{fmt}")
    scan = getattr(M, f"mla_decode_paged_{fmt}")
    B, s_q = q_c.shape[0], q_c.shape[1]
    T = B * s_q
    dev = q_c.device
    kv8 = torch.empty((layers, kv.shape[1], page_bytes), dtype=torch.uint8, device=dev)
    for l in range(layers):
        quantize(kv[l], kv8[l])
    torch.cuda.synchronize()
    q_abs = torch.empty((B, s_q, 128, 512), dtype=torch.bfloat16, device=dev)
    o_part = torch.empty((B, s_q, 128, S, 512), dtype=torch.float32, device=dev)
    lse_part = torch.empty((B, s_q, 128, S), dtype=torch.float32, device=dev)
    out = torch.empty((T, 128, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, s_q, 128), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(k, e=None):
        layer = k % layers
        if e: e[0].record(stream)
        M.mla_absorb_q(q_c, w_uk, q_abs)
        if e: e[1].record(stream)
        scan(q_abs, q_r, kv8[layer], tables[layer], seqlens, S, o_part=o_part, lse_part=lse_part)
        if e: e[2].record(stream)
        M.mla_combine_up_proj(o_part, lse_part, w_uv, out, lse)
        if e: e[3].record(stream)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(warmup + k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for k in range(steps):
        step(warmup + k, ev[k])
    torch.cuda.synchronize()
    per = [sum(ev[k][j].elapsed_time(ev[k][j + 1]) for k in range(steps)) / steps for j in range(3)]
    ms_step = wall / steps * 1e3
    kv_bytes = sum(lens) * per_token
    dec_bytes = kv_bytes + q_bytes + olat_bytes
    dec_ms = per[1]
    del kv8
    return {
        "cache": f"{what}: {per_token} bytes per token instead of {KV_BYTES_PER_TOKEN}",
        "ms_per_step": round(ms_step, 4),
        "value_tflops": round(flop_step / (ms_step * 1e-3) / 1e12, 2),
        "kernels_ms": {"mla_absorb_q": round(per[0], 4), f"mla_decode_paged_{fmt}": round(dec_ms, 4),
                       "mla_combine_up_proj": round(per[2], 4)},
        "decode_roofline": {"bound": "hbm", "achieved": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                            "traffic": measured_traffic(workload, S, fmt),
                            "algorithmic_bytes_per_launch": dec_bytes,
                            "decode_tflops": round(flop_attn / (dec_ms * 1e-3) / 1e12, 1),
                            "mfma_frac": round(flop_attn / (dec_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
    }


def time_one_launch_step(M, torch, kv, tables, seqlens, q_c, q_r, w_uk, w_uv, S, layers, steps, warmup):
    """mla_decode_step (one cooperative launch) against the four kernels it
    fuses (mla_absorb_q, mla_decode_paged, mla_combine_splits, mla_up_proj),
    same buffers, same layer rotation; wall-clock per step."""
    B, s_q = q_c.shape[0], q_c.shape[1]
    dev = q_c.device
    buf = dict(q_abs=torch.empty((B, s_q, 128, 512), dtype=torch.bfloat16, device=dev),
               o_part=torch.empty((B, s_q, 128, S, 512), dtype=torch.float32, device=dev),
               lse_part=torch.empty((B, s_q, 128, S), dtype=torch.float32, device=dev),
               o_lat=torch.empty((B, s_q, 128, 512), dtype=torch.float32, device=dev),
               lse=torch.empty((B, s_q, 128), dtype=torch.float32, device=dev),
               out=torch.empty((B, s_q, 128, 128), dtype=torch.bfloat16, device=dev))
    def fused(k):
        l = k % layers
        M.mla_decode_step(q_c, q_r, kv[l], tables[l], seqlens, w_uk, w_uv, S, buffers=buf)

    def four(k):
        l = k % layers
        M.mla_absorb_q(q_c, w_uk, buf["q_abs"])
        M.mla_decode_paged(buf["q_abs"], q_r, kv[l], tables[l], seqlens, S, o_part=buf["o_part"],
                           lse_part=buf["lse_part"])
        M.mla_combine_splits(buf["o_part"], buf["lse_part"], buf["o_lat"], buf["lse"])
        M.mla_up_proj(buf["o_lat"], w_uv, buf["out"])

    res = {}
    for name, fn in (("four_kernels_ms", four), ("one_launch_ms", fused)):
        for k in range(warmup):
            fn(k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            fn(warmup + k)
        torch.cuda.synchronize()
        res[name] = round((time.perf_counter() - t0) / steps * 1e3, 4)
    res["speedup"] = round(res["four_kernels_ms"] / res["one_launch_ms"], 3)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the split-KV decode is measured on one "
              "MI355X and multi-GPU sharding is not built", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n // 4, dtype=torch.float32, device="cuda")
        a.fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(f"[bench] copied {n} bytes three times", file=sys.stderr, flush=True)
        return
    import mla_latent_kv_06_amd as M
    from mla_inputs import CONFIGS, make_inputs, make_structure, make_cache_on_device

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs resident in HBM before timing
    inp = make_inputs(cfg, seed=42, with_cache=False)
    st0 = make_structure(cfg, seed=42)
    layer_bytes = st0.num_pages * 64 * 576 * 2
    layers = args.layers or max(cfg.layers, math.ceil(2 * 2**30 / layer_bytes))
    print(f"[bench] workload={cfg.name} B={cfg.B} s_q={cfg.s_q} layers={layers} "
          f"cache={layers * layer_bytes / 1e9:.1f} GB", file=sys.stderr, flush=True)
    kv = make_cache_on_device(st0.num_pages, layers, seed=1234, device=dev)
    tables = torch.stack([make_structure(cfg, seed=42 + l).block_table for l in range(layers)]).to(dev)
    seqlens = st0.seqlens.to(dev)
    q_c, q_r = inp.q_c.to(dev), inp.q_r.to(dev)
    w_uk, w_uv = inp.w_uk.to(dev), inp.w_uv.to(dev)
    lens = [int(x) for x in st0.seqlens]
    S = args.splits or M.mla_plan_splits(lens, tables.shape[2], cfg.s_q)
    B, s_q = cfg.B, cfg.s_q
    T = B * s_q

    # preallocated outputs: the timed loop allocates nothing
    q_abs = torch.empty((B, s_q, 128, 512), dtype=torch.bfloat16, device=dev)
    o_part = torch.empty((B, s_q, 128, S, 512), dtype=torch.float32, device=dev)
    lse_part = torch.empty((B, s_q, 128, S), dtype=torch.float32, device=dev)
    o_lat = torch.empty((B, s_q, 128, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((B, s_q, 128), dtype=torch.float32, device=dev)
    out = torch.empty((B, s_q, 128, 128), dtype=torch.bfloat16, device=dev)

    stream = torch.cuda.current_stream()
    sep = args.separate_stage2
    nev = 5 if sep else 4
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    out_rows = out.view(T, 128, 128)

    def step(k, ev=None):
        layer = k % layers
        if ev: ev[0].record(stream)
        M.mla_absorb_q(q_c, w_uk, q_abs)
        if ev: ev[1].record(stream)
        M.mla_decode_paged(q_abs, q_r, kv[layer], tables[layer], seqlens, S, o_part=o_part, lse_part=lse_part)
        if ev: ev[2].record(stream)
        if sep:
            M.mla_combine_splits(o_part, lse_part, o_lat, lse)
            if ev: ev[3].record(stream)
            M.mla_up_proj(o_lat, w_uv, out)
        else:
            # stage 2 and the up-projection in one pass (o_lat stays on chip)
            M.mla_combine_up_proj(o_part, lse_part, w_uv, out_rows, lse)
        if ev: ev[nev - 1].record(stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; timing {args.steps} steps (splits={S})", file=sys.stderr, flush=True)

    # wall-clock over exactly K steps (no events inside, so nothing is added between kernels)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(args.warmup + k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # the same K steps again with HIP events around each kernel (same stream)
    for k in range(args.steps):
        step(args.warmup + k, events[k])
    torch.cuda.synchronize()
    per = [[events[k][j].elapsed_time(events[k][j + 1]) for k in range(args.steps)] for j in range(nev - 1)]
    avg = [sum(x) / len(x) for x in per]
    names = (["mla_absorb_q", "mla_decode_paged", "mla_combine_splits", "mla_up_proj"] if sep else
             ["mla_absorb_q", "mla_decode_paged", "mla_combine_up_proj"])

    # the same steps launched from a HIP graph (one captured step per resident
    # layer, replayed): the step without host launch overhead, as a serving
    # loop that captures it would run it
    n_cap = min(layers, 64)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(n_cap):
            step(k)
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-args.steps // n_cap))
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) / (reps * n_cap) * 1e3
    del graph

    pairs = visible_pairs(lens, s_q)
    flop_attn = pairs * FLOP_PER_PAIR
    flop_proj = 2 * (2 * T * 128 * 128 * 512)
    flop_step = flop_attn + flop_proj
    kv_bytes = sum(lens) * KV_BYTES_PER_TOKEN
    q_bytes = T * 128 * 576 * 2
    olat_bytes = T * 128 * (512 + 1) * 4
    decode_bytes = kv_bytes + q_bytes + olat_bytes        # algorithmic bytes of the attention itself
    step_bytes = decode_bytes + 2 * (128 * 128 * 512 * 2) + T * 128 * 128 * 2 * 2
    ms_step = wall / args.steps * 1e3
    dec_ms = avg[1]
    achieved_gbs = decode_bytes / (dec_ms * 1e-3) / 1e9
    t_roof = max(flop_step / (MFMA_BF16_PEAK_TFLOPS * 1e12), step_bytes / (HBM_PEAK_GBS * 1e9))
    traffic = measured_traffic(cfg.name, S)

    result = {
        "metric": "MLA decode TFLOP/s + effective KV GB/s, B=16 ctx 64K, % of MI355X roofline",
        "value": round(flop_step / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 cache and activations, N(0,1/512) weights)",
        "config": {"workload": f"{cfg.name}: {cfg.notes}", "B": B, "s_q": s_q, "ctx": max(lens),
                   "heads": 128, "d_c": 512, "d_R": 64, "page": 64, "num_splits": S,
                   "resident_layers": layers, "cache_gb": round(layers * layer_bytes / 1e9, 2)},
        "kv_gbps": round(kv_bytes / (ms_step * 1e-3) / 1e9, 1),
        "graph_ms_per_step": round(graph_ms, 4),
        "step_roofline_frac": round(t_roof / (ms_step * 1e-3), 4),
        "kernels_ms": {n: round(a, 4) for n, a in zip(names, avg)},
        "roofline": {
            "kernel": "mla_decode_paged",
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": decode_bytes,
            "decode_tflops": round(flop_attn / (dec_ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flop_attn / (dec_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        },
    }
    # cache append + query rotation, timed after the step (they write into the
    # cache rows the step has already read)
    result["next_rows"] = time_next_rows(M, torch, kv, tables, seqlens, lens, B, s_q, layers)
    print("[bench] one-launch step against the four kernels it fuses", file=sys.stderr, flush=True)
    result["next_rows"]["one_launch_step"] = time_one_launch_step(
        M, torch, kv, tables, seqlens, q_c, q_r, w_uk, w_uv, S, layers, args.steps, args.warmup)
    for fmt, bits in (("fp8", 8), ("mxfp4", 4)):
        if getattr(args, f"no_{fmt}"):
            continue
        print(f"[bench] {bits}-bit cache: convert the resident layers, time the same steps", file=sys.stderr,
              flush=True)
        result["next_rows"][f"{fmt}_cache"] = time_quantized_cache(
            M, torch, fmt, kv, tables, seqlens, lens, q_c, q_r, w_uk, w_uv, S, layers, args.steps, args.warmup,
            flop_step, flop_attn, q_bytes, olat_bytes, cfg.name)
    if s_q > 1:
        # the decompressed branch the dispatch rule would take above 256 new
        # tokens, timed at this chunk length for comparison with the step
        result["next_rows"]["decompressed_branch"] = time_decompressed_branch(
            M, torch, kv, tables, seqlens, lens, q_c, q_r, w_uk, w_uv, s_q, layers)
        result["next_rows"]["decompressed_branch"]["absorbed_step_ms"] = round(ms_step, 4)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle on host cores)", file=sys.stderr, flush=True)
        layer0 = {"kv_cache": kv[0].cpu(), "block_table": tables[0].cpu(), "seqlens": st0.seqlens,
                  "q_r": inp.q_r}
        M.mla_absorb_q(q_c, w_uk, q_abs)
        torch.cuda.synchronize()
        result["cpu_baseline"] = cpu_baseline(layer0, q_abs.cpu(), args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
