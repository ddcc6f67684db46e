"""Benchmark: absorbed MLA decode over a paged latent cache on one MI355X.

A step is one pass of the whole hot path for one layer: mla_absorb_q ->
mla_decode_paged -> stage 2 fused with the up-projection (mla_combine_up_proj;
--separate-stage2 runs mla_combine_splits and mla_up_proj instead). The
headline workload (--workload, default "long") is B=16 sequences of 65536
cached tokens with 60 layers of latent cache resident (72.5 GB); step k uses
layer k mod 60, so every step reads its 1.2 GB of cache from HBM. The other
four workloads are measured the same way, each rotating through enough
resident layers (>= 2 GiB) that no step is served by the 256 MB last-level
cache.

Order of the run: every workload's inputs are built first; then the
workloads are measured back to back, the two short ones first, then the
prefill chunk, the ragged batch and the headline last, so that the few warmup
steps of the long scans do not start from an idle board (this board's power
controller runs the first ~40 launches of sustained load up to 1.5x slower);
then the headline's next rows; then the CPU baseline.

Prints one JSON line:
  value         whole-step throughput of the headline workload, algorithmic TFLOP/s
  roofline      mla_decode_paged on the headline workload against the roof its
                arithmetic intensity selects (HBM below the ridge, bf16 MFMA above)
  configs       every workload: decode and step times (mean, median, min of the timed
                steps), intensity, binding roof, fraction; `warm` (the workloads whose
                layer fits the 256 MB last-level cache): the scan alone on one layer at
                every launch, labelled as warm (--no-warm skips it)
  cpu_baseline  the fp64 CPU oracle on a bounded sample of every workload
  next_rows     for the headline: cache append and query rotation, the scan over the
                8-bit and 4-bit caches, the decompressed branch (chunks with s_q > 1)
  ceilings      the streaming-read rate and the sustained dense bf16 MFMA rate this
                board reaches with nothing else to do, and the headline decode's
                fractions of them (beside its fractions of the published peaks)
Per-kernel times come from HIP events recorded around each launch inside the K
timed steps, on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
RIDGE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # 312.5 FLOP per byte
LLC_BYTES = 256 * 10**6              # MI355X last-level (Infinity) cache, bytes
FLOP_PER_PAIR = 128 * 2 * (576 + 512)  # all heads, one (query, key) pair: QK over 576 + PV over 512
KV_BYTES_PER_TOKEN = 576 * 2
# measurement order: the two short workloads are latency-bound and never reach
# the board's power limit; the MFMA-heavy prefill step then runs the power
# controller through its settling transient before the ragged and long scans
WORKLOAD_ORDER = ("single", "uniform", "prefill", "ragged", "long")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
FORMAT_HEADERS = {"bf16": (), "fp8": ("fp8_cache.hpp",), "mxfp4": ("mxfp4_cache.hpp",)}
QUANT_FORMATS = {
    # page bytes, bytes per token, what the cache holds
    "fp8": (41216, 512 + 64 * 2 + 4, "c_KV in E4M3 with a power-of-two scale per token, k_R in bf16"),
    "mxfp4": (25600, 256 + 64 * 2 + 16, "c_KV in MXFP4 (E2M1 with an E8M0 scale per 32 dims), k_R in bf16"),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--workload", default="long", choices=list(WORKLOAD_ORDER),
                   help="the headline workload (the JSON line's value and roofline)")
    p.add_argument("--configs", default="all", choices=["all", "headline"],
                   help="measure every workload (default) or the headline only")
    p.add_argument("--layers", type=int, default=0, help="resident cache layers of the headline (0: default)")
    p.add_argument("--splits", type=int, default=0, help="num_splits of the headline (0: mla_plan_splits)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--separate-stage2", action="store_true",
                   help="run mla_combine_splits and mla_up_proj as two kernels instead of mla_combine_up_proj")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle time for the baseline")
    p.add_argument("--no-next", action="store_true", help="skip the next rows (append, quantized caches, ...)")
    p.add_argument("--no-fp8", action="store_true", help="skip the 8-bit cache leg")
    p.add_argument("--no-mxfp4", action="store_true", help="skip the 4-bit cache leg")
    p.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay of the step")
    p.add_argument("--no-warm", action="store_true",
                   help="skip the warm-cache scan timing (the counter runs average over every dispatch)")
    p.add_argument("--no-ceilings", action="store_true",
                   help="skip the achievable streaming-read and sustained MFMA measurements")
    p.add_argument("--one-launch", action="store_true",
                   help="also time mla_decode_step (one cooperative launch) against the four kernels")
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


def roof(flop, nbytes, seconds, peak_dtype="bf16"):
    """The roof a kernel's arithmetic intensity selects, and its fraction.
    Below the ridge (312.5 FLOP/byte) it is HBM bandwidth, above it the dense
    bf16 MFMA rate; both fractions are given."""
    intensity = flop / nbytes
    gbs = nbytes / seconds / 1e9
    tfs = flop / seconds / 1e12
    hbm, mfma = gbs / HBM_PEAK_GBS, tfs / MFMA_BF16_PEAK_TFLOPS
    if intensity > RIDGE:
        r = {"bound": "mfma", "achieved": round(tfs, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": round(mfma, 4), "peak_dtype": peak_dtype}
    else:
        r = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(hbm, 4)}
    r.update({"intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": RIDGE,
              "hbm_frac": round(hbm, 4), "mfma_frac": round(mfma, 4), "tflops": round(tfs, 1), "gbps": round(gbs, 1)})
    return r


def kernel_source_digest(fmt="bf16"):
    import hashlib
    h = hashlib.sha256()
    for f in ("decode.hip", "decode_body.hpp", "mla_device.hpp", "decode.hpp") + FORMAT_HEADERS[fmt]:
        with open(os.path.join(ROOT, "mla_latent_kv_06_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, splits, fmt="bf16"):
    """HBM bytes (read + written) per decode launch from the committed rocprofv3
    counter runs, if they were taken on the current kernel source and launch
    configuration; None otherwise."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(f"{fmt}/{workload}")
    except (OSError, ValueError):
        return None
    if not t or t.get("kernel_digest") != kernel_source_digest(fmt) or t.get("splits") != splits:
        return None
    return t.get("hbm_bytes_per_launch")


class Workload:
    """One workload's inputs resident on the device, its preallocated outputs
    and the algorithmic work of one step."""

    def __init__(self, M, torch, name, dev, layers=0, splits=0, separate=False):
        from mla_inputs import CONFIGS, make_cache_on_device, make_inputs, make_structure
        self.M, self.torch, self.name, self.separate = M, torch, name, separate
        cfg = self.cfg = CONFIGS[name]
        inp = make_inputs(cfg, seed=42, with_cache=False)
        st0 = make_structure(cfg, seed=42)
        self.layer_bytes = st0.num_pages * 64 * 576 * 2
        self.layers = layers or max(cfg.layers, math.ceil(2 * 2**30 / self.layer_bytes))
        self.kv = make_cache_on_device(st0.num_pages, self.layers, seed=1234, device=dev)
        # every layer holds the same sequences (lengths of seed 42) at another
        # physical page layout; each table is checked against its cache
        tabs = [make_structure(cfg, seed=42, layout_seed=42 + l).block_table for l in range(self.layers)]
        for t in tabs:
            M.mla_validate_block_table(t, st0.seqlens, st0.num_pages)
        self.tables = torch.stack(tabs).to(dev)
        self.seqlens = st0.seqlens.to(dev)
        self.seqlens_cpu = st0.seqlens
        self.inp_cpu = inp
        self.q_c, self.q_r = inp.q_c.to(dev), inp.q_r.to(dev)
        self.w_uk, self.w_uv = inp.w_uk.to(dev), inp.w_uv.to(dev)
        self.lens = [int(x) for x in st0.seqlens]
        self.B, self.s_q = cfg.B, cfg.s_q
        T = self.T = self.B * self.s_q
        self.S = splits or M.mla_plan_splits(self.lens, self.tables.shape[2], self.s_q)
        B, s_q, S = self.B, self.s_q, self.S
        self.q_abs = torch.empty((B, s_q, 128, 512), dtype=torch.bfloat16, device=dev)
        self.o_part = torch.empty((B, s_q, 128, S, 512), dtype=torch.float32, device=dev)
        self.lse_part = torch.empty((B, s_q, 128, S), dtype=torch.float32, device=dev)
        self.o_lat = torch.empty((B, s_q, 128, 512), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, s_q, 128), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, 128, 128), dtype=torch.bfloat16, device=dev)
        # algorithmic work (the FLOP convention of the K3 study: 2 (Lq + Lv) per
        # visible pair and head; bytes: cache rows, queries, fp32 o_lat and LSE)
        self.pairs = visible_pairs(self.lens, s_q)
        self.flop_attn = self.pairs * FLOP_PER_PAIR
        self.flop_proj = 2 * (2 * T * 128 * 128 * 512)
        self.flop_step = self.flop_attn + self.flop_proj
        self.kv_bytes = sum(self.lens) * KV_BYTES_PER_TOKEN
        self.q_bytes = T * 128 * 576 * 2
        self.olat_bytes = T * 128 * (512 + 1) * 4
        self.decode_bytes = self.kv_bytes + self.q_bytes + self.olat_bytes
        self.step_bytes = self.decode_bytes + 2 * (128 * 128 * 512 * 2) + T * 128 * 128 * 2 * 2
        self.names = (["mla_absorb_q", "mla_decode_paged", "mla_combine_splits", "mla_up_proj"] if separate else
                      ["mla_absorb_q", "mla_decode_paged", "mla_combine_up_proj"])

    def step(self, k, ev=None):
        M, layer = self.M, k % self.layers
        stream = self.torch.cuda.current_stream()
        if ev: ev[0].record(stream)
        M.mla_absorb_q(self.q_c, self.w_uk, self.q_abs)
        if ev: ev[1].record(stream)
        M.mla_decode_paged(self.q_abs, self.q_r, self.kv[layer], self.tables[layer], self.seqlens, self.S,
                           o_part=self.o_part, lse_part=self.lse_part)
        if ev: ev[2].record(stream)
        if self.separate:
            M.mla_combine_splits(self.o_part, self.lse_part, self.o_lat, self.lse)
            if ev: ev[3].record(stream)
            M.mla_up_proj(self.o_lat.view(self.T, 128, 512), self.w_uv, self.out)
        else:
            M.mla_combine_up_proj(self.o_part, self.lse_part, self.w_uv, self.out, self.lse)
        if ev: ev[len(self.names)].record(stream)

    def measure(self, warmup, steps):
        """W untimed steps, then exactly K timed steps bracketed by synchronisations,
        with HIP events around every kernel of every timed step."""
        torch = self.torch
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(self.names) + 1)] for _ in range(steps)]
        for k in range(warmup):
            self.step(k)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            self.step(warmup + k, ev[k])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = [[e[j].elapsed_time(e[j + 1]) for e in ev] for j in range(len(self.names))]
        self.kernel_ms = {n: sum(x) / len(x) for n, x in zip(self.names, per)}
        self.kernel_min_ms = {n: min(x) for n, x in zip(self.names, per)}
        self.kernel_median_ms = {n: statistics.median(x) for n, x in zip(self.names, per)}
        self.ms_step = wall / steps * 1e3
        return self

    def warm_decode(self, steps):
        """The scan alone, on layer 0 at every launch (after 5 untimed ones), HIP events
        between consecutive launches: the warm figure, taken where a layer's cache fits
        the 256 MB last-level cache (single, uniform, prefill) and is served from there."""
        torch, M = self.torch, self.M
        stream = torch.cuda.current_stream()

        def launch():
            M.mla_decode_paged(self.q_abs, self.q_r, self.kv[0], self.tables[0], self.seqlens, self.S,
                               o_part=self.o_part, lse_part=self.lse_part)
        for _ in range(5):
            launch()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for k in range(steps):
            launch()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        t = [ev[k].elapsed_time(ev[k + 1]) * 1e3 for k in range(steps)]
        self.warm = {"decode_median_us": round(statistics.median(t), 2), "decode_min_us": round(min(t), 2),
                     "cache": f"warm: layer 0 ({self.layer_bytes / 1e6:.0f} MB of cache) at every launch, "
                              f"inside the 256 MB last-level cache"}
        return self

    def graph_ms(self, steps):
        """The same step launched from a HIP graph (one captured step per resident
        layer, at most 64, replayed): the step without host launch overhead."""
        torch = self.torch
        n_cap = min(self.layers, 64)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(n_cap):
                self.step(k)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, -(-steps // n_cap))
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / (reps * n_cap) * 1e3
        del graph
        return ms

    def summary(self):
        dec_s = self.kernel_ms["mla_decode_paged"] * 1e-3
        r = roof(self.flop_attn, self.decode_bytes, dec_s)
        r.update({
            "decode_us": round(self.kernel_ms["mla_decode_paged"] * 1e3, 2),
            "decode_min_us": round(self.kernel_min_ms["mla_decode_paged"] * 1e3, 2),
            "decode_median_us": round(self.kernel_median_ms["mla_decode_paged"] * 1e3, 2),
            "step_us": round(self.ms_step * 1e3, 2),
            "graph_step_us": None if math.isnan(self.graph_step_ms) else round(self.graph_step_ms * 1e3, 2),
            "kernels_us": {n: round(v * 1e3, 2) for n, v in self.kernel_ms.items()},
            "num_splits": self.S, "B": self.B, "s_q": self.s_q, "max_ctx": max(self.lens),
            "tokens": sum(self.lens), "visible_pairs": self.pairs,
            "flop_per_launch": self.flop_attn, "algorithmic_bytes_per_launch": self.decode_bytes,
            "roofline_time_us": round(max(self.flop_attn / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                                          self.decode_bytes / (HBM_PEAK_GBS * 1e9)) * 1e6, 2),
            "step_tflops": round(self.flop_step / (self.ms_step * 1e-3) / 1e12, 2),
            "kv_gbps_decode": round(self.kv_bytes / dec_s / 1e9, 1),
            "resident_layers": self.layers,
            "cache": f"cold: step k reads layer k mod {self.layers} ({self.layers * self.layer_bytes / 1e9:.1f} GB)",
            "traffic": measured_traffic(self.name, self.S),
            "warm": getattr(self, "warm", None),
            "projections": self.projection_roofs(),
        })
        return r

    def projection_roofs(self):
        """The absorb and the up-projection against their own roofs: each is
        2 T H 128 512 FLOP over a 16 MiB weight. Absorb bytes: W_UK, bf16 q_c in,
        bf16 q_abs out; up-projection bytes: W_UV, fp32 o_lat in, bf16 out. The
        fused stage 2 also merges the splits, so its time covers both steps (its
        o_lat never reaches HBM, its partials are the scan's overhead)."""
        T, w = self.T, 128 * 128 * 512 * 2
        flop = 2 * T * 128 * 128 * 512
        out = {}
        for name, kern, nbytes in (("absorb", "mla_absorb_q", w + T * 128 * 128 * 2 + T * 128 * 512 * 2),
                                   ("up_proj", "mla_up_proj" if self.separate else "mla_combine_up_proj",
                                    w + T * 128 * 512 * 4 + T * 128 * 128 * 2)):
            sec = self.kernel_ms[kern] * 1e-3
            r = roof(flop, nbytes, sec)
            out[name] = {"kernel": kern, "us": round(sec * 1e6, 2), "bound": r["bound"], "frac": r["frac"],
                         "algorithmic_bytes": nbytes, "flop": flop,
                         "roofline_time_us": round(max(flop / (MFMA_BF16_PEAK_TFLOPS * 1e12),
                                                       nbytes / (HBM_PEAK_GBS * 1e9)) * 1e6, 2)}
        return out


def time_next_rows(M, torch, wl, reps=200):
    """The step before the path at this workload: writing the chunk's tokens
    into the cache (c_KV copied, k_R rotated) and rotating the queries' RoPE
    parts. Both are launch-bound at decode sizes, so `reps` launches are
    captured in one HIP graph and the replay is timed with HIP events: the
    per-launch time is the GPU's, without Python dispatch in between."""
    dev, kv, tables, seqlens, lens, B, s_q, layers = (wl.kv.device, wl.kv, wl.tables, wl.seqlens, wl.lens, wl.B,
                                                      wl.s_q, wl.layers)
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


def time_decompressed_branch(M, torch, wl, reps=5):
    """The decompressed branch (per-head K/V, then causal MHA) at this
    workload, timed per kernel with HIP events, with its algorithmic FLOP
    and bytes. The absorbed step is the comparison the dispatch rule makes."""
    kv, tables, seqlens, lens, s_q, layers = wl.kv, wl.tables, wl.seqlens, wl.lens, wl.s_q, wl.layers
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
        M.mla_decompress_kv(kv[layer], tables[layer], seqlens, wl.w_uk, wl.w_uv, max_len, k_nope=k_nope, v=v)
        if e: e[1].record(stream)
        M.mla_prefill_mha(wl.q_c, wl.q_r, k_nope, v, kv[layer], tables[layer], seqlens, out=out, lse=lse)
        if e: e[2].record(stream)
    torch.cuda.synchronize()
    t_dec = sum(e[0].elapsed_time(e[1]) for e in ev) / reps
    t_mha = sum(e[1].elapsed_time(e[2]) for e in ev) / reps
    tokens = sum(lens)
    flop_dec = 2.0 * tokens * 512 * (2 * 128 * 128)
    flop_mha = 2.0 * visible_pairs(lens, s_q) * 128 * (192 + 128)
    bytes_dec = tokens * (1024 + 2 * 128 * 128 * 2) + 2 * 128 * 128 * 512 * 2
    del k_nope, v
    return {
        "mla_decompress_kv": dict(ms=round(t_dec, 4), flop=flop_dec, bytes=bytes_dec,
                                  roofline=roof(flop_dec, bytes_dec, t_dec * 1e-3)),
        "mla_prefill_mha": dict(ms=round(t_mha, 4), flop=flop_mha,
                                mfma_frac=round(flop_mha / (t_mha * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)),
        "branch_ms": round(t_dec + t_mha, 4),
    }


def time_quantized_cache(M, torch, fmt, wl, steps, warmup):
    """The same step over a quantized cache: every resident layer converted once
    (mla_quantize_cache_<fmt>), then absorb -> mla_decode_paged_<fmt> ->
    mla_combine_up_proj, rotating through the layers as the main loop does,
    HIP events around every kernel of the timed steps."""
    page_bytes, per_token, what = QUANT_FORMATS[fmt]
    quantize = getattr(M, f"mla_quantize_cache_{fmt}")
    scan = getattr(M, f"mla_decode_paged_{fmt}")
    dev = wl.q_c.device
    kvq = torch.empty((wl.layers, wl.kv.shape[1], page_bytes), dtype=torch.uint8, device=dev)
    for l in range(wl.layers):
        quantize(wl.kv[l], kvq[l])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]

    def step(k, e=None):
        layer = k % wl.layers
        if e: e[0].record(stream)
        M.mla_absorb_q(wl.q_c, wl.w_uk, wl.q_abs)
        if e: e[1].record(stream)
        scan(wl.q_abs, wl.q_r, kvq[layer], wl.tables[layer], wl.seqlens, wl.S, o_part=wl.o_part,
             lse_part=wl.lse_part)
        if e: e[2].record(stream)
        M.mla_combine_up_proj(wl.o_part, wl.lse_part, wl.w_uv, wl.out, wl.lse)
        if e: e[3].record(stream)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(warmup + k, ev[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [sum(e[j].elapsed_time(e[j + 1]) for e in ev) / steps for j in range(3)]
    ms_step = wall / steps * 1e3
    dec_bytes = sum(wl.lens) * per_token + wl.q_bytes + wl.olat_bytes
    dec_ms = per[1]
    del kvq
    r = roof(wl.flop_attn, dec_bytes, dec_ms * 1e-3)
    r.update({"algorithmic_bytes_per_launch": dec_bytes, "traffic": measured_traffic(wl.name, wl.S, fmt),
              "note": "the bf16 peak: the scan does the bf16 scan's arithmetic (the query as two E4M3 terms "
                      "reproduces its bf16 value; V is dequantized to bf16)"})
    return {
        "cache": f"{what}: {per_token} bytes per token instead of {KV_BYTES_PER_TOKEN}",
        "ms_per_step": round(ms_step, 4),
        "value_tflops": round(wl.flop_step / (ms_step * 1e-3) / 1e12, 2),
        "kernels_ms": {"mla_absorb_q": round(per[0], 4), f"mla_decode_paged_{fmt}": round(dec_ms, 4),
                       "mla_combine_up_proj": round(per[2], 4)},
        "decode_roofline": r,
    }


def time_one_launch_step(M, torch, wl, steps, warmup):
    """mla_decode_step (one cooperative launch) against the four kernels it
    fuses, same buffers, same layer rotation; wall-clock per step."""
    def fused(k):
        l = k % wl.layers
        M.mla_decode_step(wl.q_c, wl.q_r, wl.kv[l], wl.tables[l], wl.seqlens, wl.w_uk, wl.w_uv, wl.S,
                          buffers=dict(q_abs=wl.q_abs, o_part=wl.o_part, lse_part=wl.lse_part, o_lat=wl.o_lat,
                                       lse=wl.lse, out=wl.out.view(wl.B, wl.s_q, 128, 128)))

    def four(k):
        l = k % wl.layers
        M.mla_absorb_q(wl.q_c, wl.w_uk, wl.q_abs)
        M.mla_decode_paged(wl.q_abs, wl.q_r, wl.kv[l], wl.tables[l], wl.seqlens, wl.S, o_part=wl.o_part,
                           lse_part=wl.lse_part)
        M.mla_combine_splits(wl.o_part, wl.lse_part, wl.o_lat, wl.lse)
        M.mla_up_proj(wl.o_lat.view(wl.T, 128, 512), wl.w_uv, wl.out)

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


def time_ceilings(M, torch, wl, reads=10, mfma_launches=20, mfma_iters=100_000):
    """What this board achieves with nothing else to do, for setting the decode's
    fractions of the published peaks beside it: the streaming-read rate (one
    non-temporal read of up to 4 GiB of the resident cache per launch) and the
    sustained dense bf16 matrix rate (the register-only MFMA loop, after as many
    warmup launches as timed ones so the board's power controller has settled).
    HIP events on the stream the kernels run on, around all timed launches."""
    stream = torch.cuda.current_stream()
    flat = wl.kv.view(-1)
    n = min(flat.numel(), (4 << 30) // 2) // 8 * 8  # bf16 elements, whole 16-byte chunks
    buf = flat[:n]
    sink = torch.empty(M.BENCH_SINK_FLOATS, dtype=torch.float32, device=buf.device)

    def per_launch(fn, launches, warmup):
        for _ in range(warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / launches

    nbytes = n * 2
    s_read = per_launch(lambda: M.mla_bench_stream_read(buf, sink), reads, 3)
    flop = 256 * 4 * 4 * mfma_iters * 32768
    s_mfma = per_launch(lambda: M.mla_bench_mfma(mfma_iters, sink), mfma_launches, mfma_launches)
    gbps, tfs = nbytes / s_read / 1e9, flop / s_mfma / 1e12
    return {
        "stream_read": {"gbps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBS, 4),
                        "bytes_per_launch": nbytes, "us_per_launch": round(s_read * 1e6, 1), "launches": reads,
                        "kernel": "mla_bench_stream_read (non-temporal 16-byte loads, 2048 x 256 threads)"},
        "mfma_bf16": {"tflops": round(tfs, 1), "frac_of_peak": round(tfs / MFMA_BF16_PEAK_TFLOPS, 4),
                      "flop_per_launch": flop, "us_per_launch": round(s_mfma * 1e6, 1), "launches": mfma_launches,
                      "kernel": "mla_bench_mfma (v_mfma_f32_32x32x16_bf16, 256 x 4 waves, register operands)"},
    }


def _cpu_facts():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        blas = int(os.environ.get("OMP_NUM_THREADS", "1"))
    affinity = len(os.sched_getaffinity(0))
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "affinity": affinity, "blas_threads": int(blas),
            "threads_used": int(min(blas, affinity))}


def cpu_baseline(M, torch, workloads, headline, target_s):
    """The fp64 oracle (test infrastructure, not the product path) on the host
    cores, on a bounded sample of every workload: the absorbed path (gather,
    scores, softmax, P.c_KV on the GPU's own q_abs) on whole sequences (query
    rows for the chunked workload), and the naive path (decompressed per-head
    K and V, then attention and the output) on the single and uniform ones."""
    import oracle as O
    facts = _cpu_facts()
    scale = 1.0 / math.sqrt(192)
    share = {"single": 0.05, "uniform": 0.1, "ragged": 0.15, "prefill": 0.2, "long": 0.3}
    per = {}
    for name, wl in workloads.items():
        budget = target_s * share.get(name, 0.2)
        M.mla_absorb_q(wl.q_c, wl.w_uk, wl.q_abs)
        torch.cuda.synchronize()
        qa = O.as_f64(wl.q_abs.cpu())
        qr = O.as_f64(wl.inp_cpu.q_r)
        kvb = O.bf16_bits(wl.kv[0].cpu())
        bt = wl.tables[0].cpu().numpy()
        sl = wl.seqlens_cpu.numpy()
        t0, done, pairs = time.perf_counter(), 0, 0
        if wl.s_q == 1:
            while time.perf_counter() - t0 < budget and done < wl.B:
                b = done
                O.decode_absorbed(qa[b:b + 1], qr[b:b + 1], kvb, bt[b:b + 1], sl[b:b + 1], scale)
                pairs += visible_pairs([int(sl[b])], 1)
                done += 1
            what = f"absorbed path, {done} of {wl.B} whole sequences, all 128 heads"
        else:   # query rows of the first sequence, one by one (the chunk's causal rows)
            L = int(sl[0])
            while time.perf_counter() - t0 < budget and done < wl.s_q:
                i = done
                O.decode_absorbed(qa[0:1, i:i + 1], qr[0:1, i:i + 1], kvb, bt[0:1],
                                  [L - wl.s_q + i + 1], scale)
                pairs += L - wl.s_q + i + 1
                done += 1
            what = f"absorbed path, {done} of {wl.s_q} query rows of sequence 0, all 128 heads"
        dt = time.perf_counter() - t0
        entry = {"absorbed": {"seconds": round(dt, 3), "visible_pairs": pairs,
                              "tflops": round(pairs * FLOP_PER_PAIR / dt / 1e12, 4), "sample": what}}
        if name in ("single", "uniform"):
            qc = O.as_f64(wl.inp_cpu.q_c)
            wuk, wuv = O.as_f64(wl.inp_cpu.w_uk), O.as_f64(wl.inp_cpu.w_uv)
            t0, done, flop = time.perf_counter(), 0, 0.0
            while (done == 0 or time.perf_counter() - t0 < budget) and done < wl.B:
                b = done
                O.decode_naive(qc[b:b + 1], qr[b:b + 1], kvb, bt[b:b + 1], sl[b:b + 1], wuk, wuv, scale)
                L = int(sl[b])
                # per head: K and V decompression (2 L 512 128 each), scores and P.V
                # (2 L (128 + 64) and 2 L 128), per query
                flop += 128 * (2 * 2 * L * 512 * 128 + 2 * L * (192 + 128))
                done += 1
            dt = time.perf_counter() - t0
            entry["naive"] = {"seconds": round(dt, 3), "tflops": round(flop / dt / 1e12, 4),
                              "sample": f"naive path, {done} of {wl.B} whole sequences, all 128 heads"}
        per[name] = entry
    head = per[headline]["absorbed"]
    return {
        "value": head["tflops"], "unit": "TFLOP/s", "cores": facts["threads_used"], "kind": "oracle",
        "sample": f"{head['sample']} of the {headline} workload (layer 0), {head['seconds']} s; "
                  f"CPU {facts['cpu_model']}, {facts['logical_cpus']} logical CPUs, affinity {facts['affinity']}, "
                  f"BLAS threads {facts['blas_threads']}",
        "host": facts,
        "configs": per,
    }


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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    head = args.workload
    names = [n for n in WORKLOAD_ORDER if n != head] if args.configs == "all" else []
    names.append(head)

    # ---- every workload's inputs resident in HBM before any timing
    wls = {}
    for n in names:
        is_head = n == head
        wls[n] = Workload(M, torch, n, dev, layers=args.layers if is_head else 0,
                          splits=args.splits if is_head else 0, separate=args.separate_stage2)
        w = wls[n]
        print(f"[bench] {n}: B={w.B} s_q={w.s_q} layers={w.layers} cache={w.layers * w.layer_bytes / 1e9:.1f} GB "
              f"splits={w.S}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()

    # ---- measurements, back to back, the headline last
    for n in names:
        wls[n].measure(args.warmup, args.steps)
        print(f"[bench] {n}: decode {wls[n].kernel_ms['mla_decode_paged'] * 1e3:.1f} us, "
              f"step {wls[n].ms_step * 1e3:.1f} us", file=sys.stderr, flush=True)
    for n in names:
        wls[n].graph_step_ms = float("nan") if args.no_graph else wls[n].graph_ms(args.steps)
    if not args.no_warm:
        for n in names:
            if wls[n].layer_bytes <= LLC_BYTES:  # larger layers stream from HBM anyway
                wls[n].warm_decode(args.steps)

    wl = wls[head]
    dec_s = wl.kernel_ms["mla_decode_paged"] * 1e-3
    r = roof(wl.flop_attn, wl.decode_bytes, dec_s)
    roofline = {"kernel": "mla_decode_paged", "bound": r["bound"], "achieved": r["achieved"], "peak": r["peak"],
                "unit": r["unit"], "frac": r["frac"], "traffic": measured_traffic(head, wl.S),
                "algorithmic_bytes_per_launch": wl.decode_bytes, "algorithmic_flop_per_launch": wl.flop_attn,
                "intensity_flop_per_byte": r["intensity_flop_per_byte"], "ridge_flop_per_byte": RIDGE,
                "decode_tflops": r["tflops"], "mfma_frac": r["mfma_frac"], "hbm_frac": r["hbm_frac"],
                "timing": f"HIP events around each launch inside the {args.steps} timed steps"}
    t_roof = max(wl.flop_step / (MFMA_BF16_PEAK_TFLOPS * 1e12), wl.step_bytes / (HBM_PEAK_GBS * 1e9))
    result = {
        "metric": "MLA decode TFLOP/s + effective KV GB/s, B=16 ctx 64K, % of MI355X roofline",
        "value": round(wl.flop_step / (wl.ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wl.ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 cache and activations, N(0,1/512) weights)",
        "config": {"workload": f"{wl.cfg.name}: {wl.cfg.notes}", "B": wl.B, "s_q": wl.s_q, "ctx": max(wl.lens),
                   "heads": 128, "d_c": 512, "d_R": 64, "page": 64, "num_splits": wl.S,
                   "resident_layers": wl.layers, "cache_gb": round(wl.layers * wl.layer_bytes / 1e9, 2)},
        "kv_gbps": round(wl.kv_bytes / (wl.ms_step * 1e-3) / 1e9, 1),
        "graph_ms_per_step": None if math.isnan(wl.graph_step_ms) else round(wl.graph_step_ms, 4),
        "step_roofline_frac": round(t_roof / (wl.ms_step * 1e-3), 4),
        "kernels_ms": {n: round(a, 4) for n, a in wl.kernel_ms.items()},
        "roofline": roofline,
        "configs": {n: wls[n].summary() for n in names},
    }
    # the headline's own order of runs: other workloads first (see the module docstring)
    result["configs_order"] = names

    if not args.no_next:
        nxt = result["next_rows"] = {}
        # cache append + query rotation, timed after the step (they write into the
        # cache rows the step has already read)
        nxt.update(time_next_rows(M, torch, wl))
        for fmt, bits in (("fp8", 8), ("mxfp4", 4)):
            if getattr(args, f"no_{fmt}"):
                continue
            print(f"[bench] {bits}-bit cache: convert the resident layers, time the same steps", file=sys.stderr,
                  flush=True)
            nxt[f"{fmt}_cache"] = time_quantized_cache(M, torch, fmt, wl, args.steps, args.warmup)
        if wl.s_q > 1:
            # the decompressed branch the dispatch rule would take above 256 new
            # tokens, timed at this chunk length for comparison with the step
            nxt["decompressed_branch"] = time_decompressed_branch(M, torch, wl)
            nxt["decompressed_branch"]["absorbed_step_ms"] = round(wl.ms_step, 4)
        if args.one_launch:
            print("[bench] one-launch step against the four kernels it fuses", file=sys.stderr, flush=True)
            nxt["one_launch_step"] = time_one_launch_step(M, torch, wl, args.steps, args.warmup)
    if not args.no_ceilings:
        print("[bench] ceilings: streaming read and dense bf16 MFMA on this board", file=sys.stderr, flush=True)
        c = result["ceilings"] = time_ceilings(M, torch, wl)
        c["headline_decode"] = {"gbps_frac_of_stream_read": round(r["gbps"] / c["stream_read"]["gbps"], 4),
                                "tflops_frac_of_sustained_mfma": round(r["tflops"] / c["mfma_bf16"]["tflops"], 4)}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle on host cores)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(M, torch, wls, head, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
