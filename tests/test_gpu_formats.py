"""The three cache formats against each other and on the ragged and chunked
workloads.

A bf16 cache whose c_KV values are E2M1 magnitudes times one power of two per
token is held exactly by all three formats (E2M1 values are E4M3 values, and a
per-token power of two is a valid scale for both the 8-bit cache and every
32-dim block of the 4-bit one). The library's quantizers must then be lossless,
and the three scans compute the same attention. The two quantized scans hold
the query in the same two E4M3 terms and multiply exactly, so they agree with
each other to fp32 summation order; both differ from the bf16 scan by the query
bits those terms drop (values under 2^-13 of their 32-dim block's largest),
which with N(0, 1) queries moves a score by ~1e-4 and the L1-relative output
by ~2e-5 (measured), far below the parity bar.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from mla_inputs import make_inputs, random_fp8_pages, random_mxfp4_pages
from tests._bars import assert_bar, assert_lse

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 1.0 / math.sqrt(192)


@pytest.fixture(scope="module")
def M():
    import mla_latent_kv_06_amd as mod
    return mod


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _grid_cache(pool, seed):
    """bf16 cache [pool, 64, 576]: c_KV = E2M1 value * 2^k_token, k_R ~ N(0, 1)."""
    g = torch.Generator().manual_seed(seed)
    mags = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=torch.float64)
    codes = torch.randint(0, 16, (pool, 64, 512), generator=g)
    vals = mags[codes & 7] * torch.where(codes >= 8, -1.0, 1.0).double()
    vals[..., 0] = 6.0                                # every token's largest value is 6: one scale per row
    k = torch.randint(-6, 0, (pool, 64, 1), generator=g).double()
    kv = torch.empty((pool, 64, 576), dtype=torch.float64)
    kv[..., :512] = vals * torch.exp2(k)
    kv[..., 512:] = torch.randn((pool, 64, 64), generator=g, dtype=torch.float64)
    out = kv.to(torch.bfloat16)
    assert torch.equal(out[..., :512].double(), kv[..., :512])
    return out


def test_three_formats_agree_on_values_all_of_them_hold(M):
    lens = [1, 63, 64, 65, 700, 2049, 4096, 333]
    g = torch.Generator().manual_seed(5)
    need = [-(-L // 64) for L in lens]
    pool = sum(need) + 3
    order = torch.randperm(pool, generator=g)
    bt = torch.full((len(lens), max(need) + 1), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[off:off + n].to(torch.int32)
        off += n
    kv = _grid_cache(pool, seed=6)
    q_abs = torch.randn((len(lens), 1, 128, 512), generator=g).to(torch.bfloat16).to(DEV)
    q_r = torch.randn((len(lens), 1, 128, 64), generator=g).to(torch.bfloat16).to(DEV)
    bt_d, sl = bt.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV)
    kv_d = kv.to(DEV)
    _say(f"three formats: lens={lens}")
    kv8 = M.mla_quantize_cache_fp8(kv_d)
    kv4 = M.mla_quantize_cache_mxfp4(kv_d)
    torch.cuda.synchronize()
    stored = O.as_f64(kv)
    assert np.array_equal(O.dequantize_fp8_pages(kv8.cpu().numpy()), stored), "8-bit cache not lossless"
    assert np.array_equal(O.dequantize_mxfp4_pages(kv4.cpu().numpy()), stored), "4-bit cache not lossless"
    res = {}
    for name, scan, cache in (("bf16", M.mla_decode_paged, kv_d), ("fp8", M.mla_decode_paged_fp8, kv8),
                              ("mxfp4", M.mla_decode_paged_mxfp4, kv4)):
        o_part, lse_part = scan(q_abs, q_r, cache, bt_d, sl, 5, SCALE)
        res[name] = [t.cpu().double().numpy() for t in M.mla_combine_splits(o_part, lse_part)]
    torch.cuda.synchronize()
    ref_o, ref_l = O.decode_absorbed(O.as_f64(q_abs.cpu()), O.as_f64(q_r.cpu()), stored, bt.numpy(),
                                     np.array(lens), SCALE)
    for name, (o, l) in res.items():
        assert_bar(o, ref_o, f"{name} o_lat")
        assert_lse(l, ref_l, f"{name} lse")
    base_o, base_l = res["bf16"]
    for name in ("fp8", "mxfp4"):
        o, l = res[name]
        rel = np.abs(o - base_o).sum() / np.abs(base_o).sum()
        _say(f"{name} vs bf16 scan: l1-rel {rel:.2e}, max |dlse| {np.abs(l - base_l).max():.2e}")
        assert rel < 1e-4, f"{name} differs from the bf16 scan by {rel:.2e} (L1-relative)"
        assert np.abs(l - base_l).max() < 2e-4, f"{name} lse differs from the bf16 scan"
    o8, l8 = res["fp8"]
    o4, l4 = res["mxfp4"]
    rel = np.abs(o4 - o8).sum() / np.abs(o8).sum()
    _say(f"mxfp4 vs fp8 scan: l1-rel {rel:.2e}, max |dlse| {np.abs(l4 - l8).max():.2e}")
    assert rel < 1e-6 and np.abs(l4 - l8).max() < 1e-6, "the two quantized scans disagree"


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_quantized_scans_on_the_ragged_workload_sampled(M, fmt):
    """B = 64 sequences of U[1, 32768] tokens in a shared shuffled pool, with -1
    tails in the block table, over a seeded cache of the format, in the
    launch configuration the split heuristic picks; rows the oracle computes
    one by one."""
    inp = make_inputs("ragged", with_cache=False)
    P = int(inp.block_table.max()) + 1
    pages = (random_fp8_pages(P, seed=91) if fmt == "fp8" else random_mxfp4_pages(P, seed=92))
    cache = O.PagedFp8Cache(pages.numpy()) if fmt == "fp8" else O.PagedMxfp4Cache(pages.numpy())
    d = {k: getattr(inp, k).to(DEV) for k in ("q_c", "q_r", "w_uk", "w_uv", "block_table", "seqlens")}
    S = M.mla_recommended_splits(inp.cfg.B, 1, int(inp.seqlens.max()))
    _say(f"{fmt} ragged: pages={P} splits={S}")
    r = M.decode_layer(d["q_c"], d["q_r"], pages.to(DEV), d["block_table"], d["seqlens"], d["w_uk"], d["w_uv"],
                       num_splits=S)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    picks = [(b, 0, int(h)) for b in range(0, inp.cfg.B, 2) for h in rng.choice(128, 2, replace=False)]
    ro, rl = O.decode_rows(O.as_f64(r["q_abs"].cpu()), O.as_f64(inp.q_r), cache, inp.block_table.numpy(),
                           inp.seqlens.numpy(), SCALE, picks)
    o_lat, lse = r["o_lat"].cpu(), r["lse"].cpu()
    assert_bar(np.stack([o_lat[b, i, h].double().numpy() for b, i, h in picks]), ro, f"{fmt} ragged o_lat rows")
    assert_lse(np.array([float(lse[b, i, h]) for b, i, h in picks]), rl, f"{fmt} ragged lse rows")


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_quantized_scans_on_a_causal_chunk(M, fmt):
    """s_q = 64 new tokens per sequence over 1000- and 3000-token caches
    (query i sees keys up to L - 64 + i), every row against the oracle."""
    g = torch.Generator().manual_seed(44)
    lens, s_q = [1000, 3000], 64
    need = [-(-L // 64) for L in lens]
    pool = sum(need) + 2
    order = torch.randperm(pool, generator=g)
    bt = torch.full((2, max(need)), -1, dtype=torch.int32)
    bt[0, :need[0]] = order[:need[0]].to(torch.int32)
    bt[1, :need[1]] = order[need[0]:need[0] + need[1]].to(torch.int32)
    pages = random_fp8_pages(pool, seed=45) if fmt == "fp8" else random_mxfp4_pages(pool, seed=46)
    cache = O.PagedFp8Cache(pages.numpy()) if fmt == "fp8" else O.PagedMxfp4Cache(pages.numpy())
    q_abs = (torch.randn((2, s_q, 128, 512), generator=g) * 0.3).to(torch.bfloat16)
    q_r = torch.randn((2, s_q, 128, 64), generator=g).to(torch.bfloat16)
    scan = M.mla_decode_paged_fp8 if fmt == "fp8" else M.mla_decode_paged_mxfp4
    _say(f"{fmt} causal chunk: lens={lens} s_q={s_q}")
    o_part, lse_part = scan(q_abs.to(DEV), q_r.to(DEV), pages.to(DEV), bt.to(DEV),
                            torch.tensor(lens, dtype=torch.int32, device=DEV), 4, SCALE)
    o_lat, lse = M.mla_combine_splits(o_part, lse_part)
    torch.cuda.synchronize()
    ref_o, ref_l = O.decode_absorbed(O.as_f64(q_abs), O.as_f64(q_r), cache, bt.numpy(), np.array(lens), SCALE)
    assert_bar(o_lat.cpu().numpy(), ref_o, f"{fmt} chunk o_lat")
    assert_lse(lse.cpu().numpy(), ref_l, f"{fmt} chunk lse")


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_decode_layer_replays_in_a_graph(M, fmt):
    """The whole layer (absorb -> scan -> merge -> up-projection) captured in
    one HIP graph over each cache format and replayed three times with new
    queries copied in between (eager work and synchronisations between the
    replays): every replay equals the eager call on the same queries, bit for
    bit (the kernels' results do not depend on how they were launched)."""
    lens = [700, 64, 1500]
    g = torch.Generator().manual_seed(70)
    need = [-(-L // 64) for L in lens]
    pool = sum(need) + 2
    order = torch.randperm(pool, generator=g)
    bt = torch.full((len(lens), max(need)), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[off:off + n].to(torch.int32)
        off += n
    kv = torch.randn((pool, 64, 576), generator=g).to(torch.bfloat16).to(DEV)
    cache = {"bf16": lambda: kv, "fp8": lambda: M.mla_quantize_cache_fp8(kv),
             "mxfp4": lambda: M.mla_quantize_cache_mxfp4(kv)}[fmt]()
    w_uk = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16).to(DEV)
    w_uv = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16).to(DEV)
    btd, sld = bt.to(DEV), torch.tensor(lens, dtype=torch.int32, device=DEV)
    qs = [(torch.randn((3, 1, 128, 128), generator=g).to(torch.bfloat16).to(DEV),
           torch.randn((3, 1, 128, 64), generator=g).to(torch.bfloat16).to(DEV)) for _ in range(3)]
    _say(f"decode layer in a HIP graph, cache={fmt}")
    q_c, q_r = qs[0][0].clone(), qs[0][1].clone()
    M.decode_layer(q_c, q_r, cache, btd, sld, w_uk, w_uv, num_splits=4)   # warm the allocator outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        r = M.decode_layer(q_c, q_r, cache, btd, sld, w_uk, w_uv, num_splits=4)
    for rep, (qc, qr) in enumerate(qs):
        q_c.copy_(qc)
        q_r.copy_(qr)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = M.decode_layer(qc, qr, cache, btd, sld, w_uk, w_uv, num_splits=4)
        torch.cuda.synchronize()
        assert torch.equal(r["out"].view(torch.int16), ref["out"].view(torch.int16)), f"replay {rep}: out"
        assert torch.equal(r["lse"], ref["lse"]), f"replay {rep}: lse"
        assert torch.equal(r["o_lat"], ref["o_lat"]), f"replay {rep}: o_lat"
    del graph
