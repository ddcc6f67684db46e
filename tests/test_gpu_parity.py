"""GPU parity of every C-ABI entry point against the fp64 oracle.

Each function is judged on exactly the inputs it received (the GPU's own bf16
q_abs for the decode, its own fp32 o_lat for the up-projection), so a bar
measures that function's own error. Large workloads are checked on sampled
rows that the oracle computes one by one. Integer work (the paged gather) and
placement invariance are bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from mla_inputs import CONFIGS, Config, make_inputs, make_structure
from tests._plan import header_pieces, row_pages
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


def _to(inp):
    d = {k: getattr(inp, k).to(DEV) for k in ("q_c", "q_r", "w_uk", "kv_cache", "w_uv", "block_table", "seqlens")}
    return d


def _random_case(seqlens, s_q, seed, pool_extra=5, nan_tail=False):
    """Small random inputs with real dims, arbitrary lengths and a permuted pool."""
    g = torch.Generator().manual_seed(seed)
    need = [-(-int(L) // 64) for L in seqlens]
    pool = sum(need) + pool_extra
    order = torch.randperm(pool, generator=g)
    maxp = max(max(need), 1) + 1
    bt = torch.full((len(seqlens), maxp), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[off:off + n].to(torch.int32)
        off += n
    B = len(seqlens)
    q_abs = torch.randn((B, s_q, 128, 512), generator=g).to(torch.bfloat16)
    q_r = torch.randn((B, s_q, 128, 64), generator=g).to(torch.bfloat16)
    kv = torch.randn((pool, 64, 576), generator=g).to(torch.bfloat16)
    if nan_tail:
        for b, L in enumerate(seqlens):
            if L % 64:
                kv[int(bt[b, L // 64]), L % 64:, :] = float("nan")
    return q_abs, q_r, kv, bt, torch.tensor(seqlens, dtype=torch.int32)


def _decode_check(M, q_abs, q_r, kv, bt, sl, num_splits, what, check_parts=True):
    _say(f"{what}: B={q_abs.shape[0]} s_q={q_abs.shape[1]} lens={sl.tolist()[:6]} splits={num_splits}")
    o_part, lse_part = M.mla_decode_paged(q_abs.to(DEV), q_r.to(DEV), kv.to(DEV), bt.to(DEV), sl.to(DEV),
                                          num_splits, SCALE)
    o_lat, lse = M.mla_combine_splits(o_part, lse_part)
    torch.cuda.synchronize()
    kvb = O.bf16_bits(kv)
    ref_o, ref_l = O.decode_absorbed(O.as_f64(q_abs), O.as_f64(q_r), kvb, bt.numpy(), sl.numpy(), SCALE)
    assert_bar(o_lat.cpu().numpy(), ref_o, f"{what} o_lat")
    assert_lse(lse.cpu().numpy(), ref_l, f"{what} lse")
    if check_parts:
        rp_o, rp_l = O.decode_split(O.as_f64(q_abs), O.as_f64(q_r), kvb, bt.numpy(), sl.numpy(), SCALE,
                                    header_pieces(row_pages(sl.tolist(), q_abs.shape[1]), num_splits), num_splits)
        assert_lse(lse_part.cpu().numpy(), rp_l, f"{what} lse_part")
        # rows of empty splits are not written: compare the others only
        live = np.isfinite(rp_l)
        assert_bar(o_part.cpu().numpy()[live], rp_o[live], f"{what} o_part")
    return o_lat, lse


# ---------------------------------------------------------------------------
# paged gather: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", ["single", "uniform"])
def test_gather_bit_exact(M, cfg):
    inp = make_inputs(cfg)
    max_len = int(inp.seqlens.max()) + 17
    _say(f"gather {cfg} max_len={max_len}")
    out = M.mla_debug_gather(inp.kv_cache.to(DEV), inp.block_table.to(DEV), inp.seqlens.to(DEV), max_len)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy()
    bits = O.bf16_bits(inp.kv_cache)
    for b in range(inp.cfg.B):
        L = int(inp.seqlens[b])
        ref = np.zeros((max_len, 576), np.uint16)
        ref[:L] = bits[inp.block_table[b, :(L + 63) // 64].numpy().astype(np.int64)].reshape(-1, 576)[:L]
        assert np.array_equal(got[b].view(np.uint16), ref), f"sequence {b}"


def test_gather_ragged_lengths_bit_exact(M):
    lens = [0, 1, 63, 64, 65, 127, 129, 300]
    _, _, kv, bt, sl = _random_case(lens, 1, seed=5)
    out = M.mla_debug_gather(kv.to(DEV), bt.to(DEV), sl.to(DEV), 320)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    bits = O.bf16_bits(kv)
    for b, L in enumerate(lens):
        ref = np.zeros((320, 576), np.uint16)
        if L:
            ref[:L] = bits[bt[b, :(L + 63) // 64].numpy().astype(np.int64)].reshape(-1, 576)[:L]
        assert np.array_equal(got[b], ref), f"L={L}"


# ---------------------------------------------------------------------------
# absorb and up-projection
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 16, 45, 128, 129, 300, 1024])
def test_absorb_parity(M, T):
    """Token counts on and around the 128-token blocks the absorb splits a chunk into."""
    g = torch.Generator().manual_seed(100 + T)
    q_c = torch.randn((T, 128, 128), generator=g).to(torch.bfloat16)
    w_uk = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    _say(f"absorb T={T}")
    q_abs = M.mla_absorb_q(q_c.to(DEV), w_uk.to(DEV))
    torch.cuda.synchronize()
    ref = O.absorb(O.as_f64(q_c), O.as_f64(w_uk))
    assert_bar(O.as_f64(q_abs.cpu()), ref, f"absorb T={T}")


@pytest.mark.parametrize("T", [1, 16, 45, 1024])
def test_up_proj_parity(M, T):
    g = torch.Generator().manual_seed(200 + T)
    o_lat = torch.randn((T, 128, 512), generator=g, dtype=torch.float32)
    w_uv = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    _say(f"up_proj T={T}")
    out = M.mla_up_proj(o_lat.to(DEV), w_uv.to(DEV))
    torch.cuda.synchronize()
    ref = O.up_proj(o_lat.double().numpy(), O.as_f64(w_uv))
    assert_bar(O.as_f64(out.cpu()), ref, f"up_proj T={T}")


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("S", [1, 3, 16, 70])
def test_combine_parity(M, S):
    g = torch.Generator().manual_seed(300 + S)
    B, s_q = 3, 2
    o_part = torch.randn((B, s_q, 128, S, 512), generator=g)
    lse_part = torch.randn((B, s_q, 128, S), generator=g) * 5
    if S > 1:
        lse_part[0, 0, :, -1] = float("-inf")   # an empty split
    lse_part[2, 1, 5, :] = float("-inf")        # a row with no keys at all
    # the partial rows of empty splits are never written by the scan and must
    # never be read: NaN there for the GPU, zeros for the oracle
    ref_part = torch.where(torch.isneginf(lse_part)[..., None], torch.zeros(()), o_part)
    o_part[torch.isneginf(lse_part)] = float("nan")
    _say(f"combine S={S}")
    o_lat, lse = M.mla_combine_splits(o_part.to(DEV), lse_part.to(DEV))
    torch.cuda.synchronize()
    ref_o, ref_l = O.combine(ref_part.double().numpy(), lse_part.double().numpy())
    assert_bar(o_lat.cpu().numpy(), ref_o, f"combine S={S}")
    assert_lse(lse.cpu().numpy(), ref_l, f"combine S={S}")


@pytest.mark.parametrize("B,s_q,S", [(1, 1, 1), (16, 1, 17), (3, 15, 3), (2, 512, 2), (2, 1, 70), (1, 1, 130), (3, 11, 5),
                                     (1, 1, 32), (3, 1, 7), (1, 4, 9), (5, 1, 3), (9, 1, 4), (2, 13, 6),
                                     (37, 16, 1), (1, 1000, 2), (3, 12, 20), (1, 1000, 1), (5, 13, 1)])
def test_combine_up_proj_parity(M, B, s_q, S):
    """Merge + up-projection in one pass against the oracle's combine then up_proj.
    Row counts 1 to 9 and 26 take every way the merge deals a tile's rows to its
    waves (8, 4, 2 or 1 waves per row, ranges crossing a block of 64 splits);
    the rest cover the 16-row tiles with few splits (loads of 4 splits in flight)
    and with many (36 rows, 20 splits), ragged last tiles, workgroups looping
    over several tiles of a head (1000 rows, 2 splits) and the one-split kernel
    that streams the partials (592, 1000 and 65 rows)."""
    g = torch.Generator().manual_seed(400 + B + s_q + S)
    o_part = torch.randn((B, s_q, 128, S, 512), generator=g)
    lse_part = torch.randn((B, s_q, 128, S), generator=g) * 5
    w_uv = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    if S > 1:
        lse_part[0, 0, :, -1] = float("-inf")
    lse_part[-1, -1, 7, :] = float("-inf")
    ref_part = torch.where(torch.isneginf(lse_part)[..., None], torch.zeros(()), o_part)
    o_part[torch.isneginf(lse_part)] = float("nan")
    _say(f"combine+up_proj B={B} s_q={s_q} S={S}")
    out, lse = M.mla_combine_up_proj(o_part.to(DEV), lse_part.to(DEV), w_uv.to(DEV))
    torch.cuda.synchronize()
    ref_o, ref_l = O.combine(ref_part.double().numpy(), lse_part.double().numpy())
    ref_out = O.up_proj(ref_o.reshape(B * s_q, 128, 512), O.as_f64(w_uv))
    assert_bar(O.as_f64(out.cpu()), ref_out, f"combine+up_proj B={B} s_q={s_q} S={S}")
    assert_lse(lse.cpu().numpy(), ref_l, f"combine+up_proj lse B={B} s_q={s_q} S={S}")
    assert (O.as_f64(out.cpu())[-1, 7] == 0).all(), "a row with no keys must project to zero"


# ---------------------------------------------------------------------------
# decode (+ combine): workloads, edge lengths, causal chunks, split plans
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("num_splits", [1, 2, 7, 32])
def test_decode_single_config(M, num_splits):
    inp = make_inputs("single")
    d = _to(inp)
    q_abs = M.mla_absorb_q(d["q_c"], d["w_uk"]).cpu()
    _decode_check(M, q_abs, inp.q_r, inp.kv_cache, inp.block_table, inp.seqlens, num_splits, "single")


def test_decode_uniform_config(M):
    inp = make_inputs("uniform")
    d = _to(inp)
    S = M.mla_recommended_splits(16, 1, 4096)
    q_abs = M.mla_absorb_q(d["q_c"], d["w_uk"]).cpu()
    _decode_check(M, q_abs, inp.q_r, inp.kv_cache, inp.block_table, inp.seqlens, S, "uniform")


@pytest.mark.parametrize("lens,s_q,S", [
    ([1, 31, 32, 33, 63], 1, 1),
    ([64, 65, 127, 129, 2047], 1, 3),
    ([5, 300, 1000], 1, 17),      # more splits than pages of short rows: empty splits
    ([300, 77], 2, 2),
    ([100, 400], 37, 3),          # causal chunk
    ([700, 300], 512, 2),         # a long chunk: deep row search, the first 212 rows of sequence 1 see no key
])
def test_decode_edge_lengths(M, lens, s_q, S):
    q_abs, q_r, kv, bt, sl = _random_case(lens, s_q, seed=sum(lens) + s_q)
    _decode_check(M, q_abs, q_r, kv, bt, sl, S, f"edge lens={lens} s_q={s_q}")


@pytest.mark.parametrize("B,s_q,S", [(150, 1, 1), (150, 1, 3), (130, 1, 7), (70, 3, 2), (200, 1, 256)])
def test_decode_many_sequences(M, B, s_q, S):
    """More than 64 sequences: the split plan reads the lengths in several blocks
    of 64 (wave-wide sums, maximum and scan per block) and its row search walks
    past the first block. Lengths 0..300 with zeros and one-token rows mixed in;
    every row and every partial slot against the oracle."""
    g = torch.Generator().manual_seed(1000 + B + s_q + S)
    lens = torch.randint(0, 301, (B,), generator=g)
    lens[::17] = 0
    lens[5::19] = 1
    q_abs, q_r, kv, bt, sl = _random_case(lens.tolist(), s_q, seed=2000 + B + S)
    S = min(S, bt.shape[1])
    _decode_check(M, q_abs, q_r, kv, bt, sl, S, f"{B} sequences s_q={s_q}")


def test_decode_zero_length_rows(M):
    q_abs, q_r, kv, bt, sl = _random_case([0, 70], 1, seed=9)
    o_lat, lse = _decode_check(M, q_abs, q_r, kv, bt, sl, 2, "zero length", check_parts=True)
    assert (o_lat[0].cpu() == 0).all() and torch.isneginf(lse[0].cpu()).all()


def test_decode_ragged_plan_leaves_empty_splits_unwritten_and_unread(M):
    """Balanced plan on a ragged batch: rows use only the slots of their pieces; the
    unused ones get lse = -inf, their o_part rows are never written (a NaN fill
    survives) and the combine never reads them."""
    lens = [5000, 1000, 64, 30, 2047]
    q_abs, q_r, kv, bt, sl = _random_case(lens, 1, seed=15)
    S = 8
    B = len(lens)
    o_part = torch.full((B, 1, 128, S, 512), float("nan"), dtype=torch.float32, device=DEV)
    lse_part = torch.empty((B, 1, 128, S), dtype=torch.float32, device=DEV)
    M.mla_decode_paged(q_abs.to(DEV), q_r.to(DEV), kv.to(DEV), bt.to(DEV), sl.to(DEV), S, SCALE,
                       o_part=o_part, lse_part=lse_part)
    o_lat, lse = M.mla_combine_splits(o_part, lse_part)
    torch.cuda.synchronize()
    kvb = O.bf16_bits(kv)
    ref_o, ref_l = O.decode_absorbed(O.as_f64(q_abs), O.as_f64(q_r), kvb, bt.numpy(), sl.numpy(), SCALE)
    assert_bar(o_lat.cpu().numpy(), ref_o, "ragged plan o_lat")
    assert_lse(lse.cpu().numpy(), ref_l, "ragged plan lse")
    plan = header_pieces(row_pages(sl.tolist(), 1), S)
    rp_o, rp_l = O.decode_split(O.as_f64(q_abs), O.as_f64(q_r), kvb, bt.numpy(), sl.numpy(), SCALE, plan, S)
    assert_lse(lse_part.cpu().numpy(), rp_l, "ragged plan lse_part")
    live = np.isfinite(rp_l)
    used = live.reshape(B, 128, S)[:, 0, :].sum(1).tolist()
    assert used == [len(p) for p in plan], used
    assert min(used) < S
    op = o_part.cpu().numpy()
    assert_bar(op[live], rp_o[live], "ragged plan o_part")
    assert np.isnan(op[~live]).all(), "an empty split's partial rows were written"


def test_decode_nan_in_unused_tail_rows(M):
    q_abs, q_r, kv, bt, sl = _random_case([100, 33, 130], 1, seed=10, nan_tail=True)
    _decode_check(M, q_abs, q_r, kv, bt, sl, 2, "NaN past the end")


def test_decode_score_jump_triggers_exact_rescan(M):
    """A key scoring 2^208 above the first tile's reference forces the rescan path."""
    L, tstar = 2048, 1500
    g = torch.Generator().manual_seed(11)
    kv = torch.randn((32, 64, 576), generator=g).to(torch.bfloat16)
    kv[..., 512:] = 0
    kv.view(-1, 576)[tstar, 512] = 1.0
    q_abs = torch.zeros((1, 1, 128, 512), dtype=torch.bfloat16)
    q_r = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16)
    q_r[..., 0] = 2000.0
    bt = torch.arange(32, dtype=torch.int32)[None]
    sl = torch.tensor([L], dtype=torch.int32)
    o_lat, lse = _decode_check(M, q_abs, q_r, kv, bt, sl, 1, "rescan one-hot")
    row = kv.view(-1, 576)[tstar, :512].float()
    # Every other weight underflows to 0, so the output is the row divided by
    # the dominant weight's own fp32 value 2^e: the kernel forms x*c - m in one
    # fma, leaving |e| <= half an ulp of 208 (2^-17) and a relative error
    # below 1e-5. Without the rescan the dominant weight overflows (inf/NaN).
    got = o_lat[0, 0].cpu()
    assert torch.isfinite(got).all()
    rel = ((got - row) / row.abs().clamp_min(1e-30)).abs().max().item()
    assert rel <= 1e-5, f"one-hot row reproduced to {rel:.2e} relative"


def test_decode_rising_scores_within_headroom(M):
    """Scores that climb by ~40 (log2) over the sequence stay on the single-pass path."""
    L = 1024
    g = torch.Generator().manual_seed(12)
    kv = torch.randn((16, 64, 576), generator=g).to(torch.bfloat16)
    ramp = torch.linspace(0, 1, L)
    kv.view(-1, 576)[:L, 512] = ramp.to(torch.bfloat16)
    kv.view(-1, 576)[:L, 513:] = 0
    q_abs = (torch.randn((1, 1, 128, 512), generator=g) * 0.1).to(torch.bfloat16)
    q_r = torch.zeros((1, 1, 128, 64), dtype=torch.bfloat16)
    q_r[..., 0] = 384.0
    bt = torch.randperm(16, generator=g).to(torch.int32)[None]
    _decode_check(M, q_abs, q_r, kv, bt, torch.tensor([L], dtype=torch.int32), 1, "rising scores")


# ---------------------------------------------------------------------------
# bit-exact invariances
# ---------------------------------------------------------------------------

def test_debug_checks_switch_reports_a_bad_table(M, monkeypatch):
    """MLA_DEBUG_CHECKS=1: the scan validates the device block table on the
    host before launching and reports a bad entry instead of clamping it; with
    a good table it changes nothing (same partials, bit for bit)."""
    q_abs, q_r, kv, bt, sl = _random_case([300, 130], 1, seed=93)
    dev = [x.to(DEV) for x in (q_abs, q_r, kv, sl)]
    run = lambda t: M.mla_decode_paged(dev[0], dev[1], dev[2], t.to(DEV), dev[3], 2, SCALE)
    ref_o, ref_l = run(bt)
    torch.cuda.synchronize()
    monkeypatch.setenv("MLA_DEBUG_CHECKS", "1")
    got_o, got_l = run(bt)
    torch.cuda.synchronize()
    live = torch.isfinite(ref_l)
    assert torch.equal(got_l.cpu(), ref_l.cpu()) and torch.equal(got_o[live].cpu(), ref_o[live].cpu())
    bad = bt.clone()
    bad[1, 2] = kv.shape[0] + 4
    with pytest.raises(M.MlaError) as e:
        run(bad)
    assert e.value.status == 2 and "MLA_DEBUG_CHECKS" in str(e.value) and "block_table[1, 2]" in str(e.value)
    monkeypatch.setenv("MLA_DEBUG_CHECKS", "0")
    run(bad)  # switched off: clamped, no error
    torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_out_of_range_table_entries_are_clamped_into_the_pool(M, fmt):
    """Table entries outside [0, num_pages) break the interface's contract; the
    scan clamps them (below 0 -> page 0, from num_pages on -> the last page)
    so that no entry addresses memory outside the pool. Both page lookups, for
    a piece's first two tiles and the steady loop's one-tile-ahead prefetch,
    clamp alike: a table with such entries gives bit for bit the result of its
    clamped copy (pieces of ~32 tiles, so the steady loop runs)."""
    lens = [700, 1500, 64, 2100]
    q_abs, q_r, kv, bt, sl = _random_case(lens, 1, seed=91)
    P = kv.shape[0]
    bad = bt.clone()
    kinds = [-7, P + 3, 2**31 - 1]
    k = 0
    for b, L in enumerate(lens):
        for p in range(0, -(-L // 64), 3):  # every third live page of each row
            bad[b, p] = kinds[k % 3]
            k += 1
    clamped = bad.clamp(0, P - 1)
    kv_d = kv.to(DEV)
    if fmt == "fp8":
        kv_d, fn = M.mla_quantize_cache_fp8(kv_d), M.mla_decode_paged_fp8
    elif fmt == "mxfp4":
        kv_d, fn = M.mla_quantize_cache_mxfp4(kv_d), M.mla_decode_paged_mxfp4
    else:
        fn = M.mla_decode_paged
    _say(f"out-of-range entries ({fmt}): pool {P} pages, {k} entries replaced, splits 3")
    outs = []
    for t in (bad, clamped):
        o_part, lse_part = fn(q_abs.to(DEV), q_r.to(DEV), kv_d, t.to(DEV), sl.to(DEV), 3, SCALE)
        torch.cuda.synchronize()
        outs.append((o_part.cpu(), lse_part.cpu()))
    (o1, l1), (o2, l2) = outs
    live = torch.isfinite(l2)
    assert bool(live.any())
    assert torch.equal(l1, l2)
    assert torch.equal(o1[live], o2[live])


def test_page_placement_neighbour_values_and_rerun_bit_exact(M):
    q_abs, q_r, kv, bt, sl = _random_case([700, 64, 1500], 1, seed=13)
    S = 4
    o1, l1 = M.mla_decode_paged(q_abs.to(DEV), q_r.to(DEV), kv.to(DEV), bt.to(DEV), sl.to(DEV), S, SCALE)
    # same logical rows at other physical pages
    perm = torch.randperm(kv.shape[0], generator=torch.Generator().manual_seed(1))
    inv = torch.argsort(perm)
    kv2 = kv[perm]
    bt2 = torch.where(bt >= 0, inv[bt.clamp(min=0).long()].to(torch.int32), bt)
    o2, l2 = M.mla_decode_paged(q_abs.to(DEV), q_r.to(DEV), kv2.to(DEV), bt2.to(DEV), sl.to(DEV), S, SCALE)
    # other queries for the neighbours (same lengths, so the same split plan)
    g = torch.Generator().manual_seed(2)
    q_abs3, q_r3 = q_abs.clone(), q_r.clone()
    q_abs3[:2] = (torch.randn(q_abs3[:2].shape, generator=g) * 0.05).to(torch.bfloat16)
    q_r3[:2] = torch.randn(q_r3[:2].shape, generator=g).to(torch.bfloat16)
    o3, l3 = M.mla_decode_paged(q_abs3.to(DEV), q_r3.to(DEV), kv.to(DEV), bt.to(DEV), sl.to(DEV), S, SCALE)
    # sequence 2 alone: the plan depends on the batch's lengths, so only the
    # combined result is compared, to the numerical bar
    o5, l5 = M.mla_decode_paged(q_abs[2:].contiguous().to(DEV), q_r[2:].contiguous().to(DEV), kv.to(DEV),
                                bt[2:].contiguous().to(DEV), sl[2:].contiguous().to(DEV), S, SCALE)
    # and a rerun: deterministic
    o4, l4 = M.mla_decode_paged(q_abs.to(DEV), q_r.to(DEV), kv.to(DEV), bt.to(DEV), sl.to(DEV), S, SCALE)
    torch.cuda.synchronize()

    def same(oa, la, ob, lb):
        # the partial rows of empty splits (lse = -inf) are not written
        live = torch.isfinite(la)
        return torch.equal(la, lb) and torch.equal(oa[live], ob[live])
    assert same(o1, l1, o2, l2), "physical placement changed the result"
    assert same(o1[2:], l1[2:], o3[2:], l3[2:]), "the neighbours' values changed the result"
    assert same(o1, l1, o4, l4), "rerun is not bit-identical"
    c1, cl1 = M.mla_combine_splits(o1, l1)
    c5, cl5 = M.mla_combine_splits(o5, l5)
    torch.cuda.synchronize()
    assert_bar(c5.cpu().numpy(), c1[2:].cpu().numpy().astype(np.float64), "alone vs in batch")
    assert_lse(cl5.cpu().numpy(), cl1[2:].cpu().numpy(), "alone vs in batch lse")


# ---------------------------------------------------------------------------
# whole chain on the teardown page's size: vs the naive (path A) oracle
# ---------------------------------------------------------------------------

def test_chain_single_vs_naive(M):
    inp = make_inputs("single")
    d = _to(inp)
    _say("chain single: absorb -> decode -> combine -> up_proj vs naive path")
    r = M.decode_layer(d["q_c"], d["q_r"], d["kv_cache"], d["block_table"], d["seqlens"], d["w_uk"], d["w_uv"],
                       num_splits=4)
    torch.cuda.synchronize()
    f = {k: O.as_f64(getattr(inp, k)) for k in ("q_c", "q_r", "w_uk", "w_uv")}
    ref_out, ref_lse = O.decode_naive(f["q_c"], f["q_r"], O.bf16_bits(inp.kv_cache), inp.block_table.numpy(),
                                      inp.seqlens.numpy(), f["w_uk"], f["w_uv"], SCALE)
    # per-function bars on each function's own inputs
    assert_bar(O.as_f64(r["q_abs"].cpu()), O.absorb(f["q_c"], f["w_uk"]), "chain absorb")
    assert_bar(O.as_f64(r["out"].cpu()), O.up_proj(r["o_lat"].cpu().double().numpy(), f["w_uv"]), "chain up_proj")
    # end to end: the bf16 rounding of q_abs and P compounds; max bar holds, mean reported
    mx, l1 = assert_bar(O.as_f64(r["out"].cpu()), ref_out, "chain end-to-end", l1_rel=5e-3)
    assert_lse(r["lse"].cpu().numpy(), ref_lse, "chain lse")


# ---------------------------------------------------------------------------
# full-size workloads, every output row, in the launch configuration the bench uses
# ---------------------------------------------------------------------------

def _full_check(M, inp, what, num_splits=None):
    """decode_layer at the workload's full size; every (b, i, h) row of o_lat
    and lse against the fp64 oracle (decode_absorbed on the GPU's own q_abs),
    absorb on the whole tensor and the up-projection on its own o_lat."""
    d = _to(inp)
    B, s_q = inp.cfg.B, inp.cfg.s_q
    S = num_splits or M.mla_plan_splits(inp.seqlens.tolist(), inp.block_table.shape[1], s_q)
    _say(f"{what}: B={B} s_q={s_q} pages={inp.kv_cache.shape[0]} splits={S} (all rows)")
    r = M.decode_layer(d["q_c"], d["q_r"], d["kv_cache"], d["block_table"], d["seqlens"], d["w_uk"], d["w_uv"],
                       num_splits=S)
    torch.cuda.synchronize()
    q_abs = r["q_abs"].cpu()
    ref_o, ref_l = O.decode_absorbed(O.as_f64(q_abs), O.as_f64(inp.q_r), O.bf16_bits(inp.kv_cache),
                                     inp.block_table.numpy(), inp.seqlens.numpy(), SCALE)
    assert_bar(r["o_lat"].cpu().double().numpy(), ref_o, f"{what} o_lat (all rows)")
    assert_lse(r["lse"].cpu().numpy(), ref_l, f"{what} lse (all rows)")
    assert_bar(O.as_f64(q_abs), O.absorb(O.as_f64(inp.q_c), O.as_f64(inp.w_uk)), f"{what} absorb")
    w_uv = O.as_f64(inp.w_uv)
    o_lat = r["o_lat"].cpu().double().numpy().reshape(B * s_q, 128, 512)
    assert_bar(O.as_f64(r["out"].cpu()).reshape(B * s_q, 128, 128), O.up_proj(o_lat, w_uv), f"{what} up_proj")
    # the bench's stage 2 (merge fused with the up-projection) on the same partials,
    # against the oracle's merge of those partials (unwritten empty slots zeroed)
    out2, lse2 = M.mla_combine_up_proj(r["o_part"], r["lse_part"], d["w_uv"])
    torch.cuda.synchronize()
    out2 = O.as_f64(out2.cpu()).reshape(B, s_q, 128, 128)
    lp = r["lse_part"].cpu().double().numpy()
    ref_out2, ref_lse2 = [], []
    for b in range(B):
        op = r["o_part"][b].cpu().double().numpy()
        op[np.isneginf(lp[b])] = 0.0
        mo, ml = O.combine(op, lp[b])
        ref_out2.append(O.up_proj(mo, w_uv))
        ref_lse2.append(ml)
    assert_bar(out2, np.stack(ref_out2), f"{what} combine_up_proj")
    assert_lse(lse2.cpu().numpy(), np.stack(ref_lse2), f"{what} combine_up_proj lse")


def test_ragged_config_full(M):
    _full_check(M, make_inputs("ragged"), "ragged")


def test_long_config_full(M):
    _full_check(M, make_inputs("long"), "long 64K")


def test_prefill_config_full(M):
    _full_check(M, make_inputs("prefill"), "prefill 256 over 16K")


# ---------------------------------------------------------------------------
# pools larger than 2^31 bytes: page offsets need 64 bits
# ---------------------------------------------------------------------------

def _top_pool(page_bytes, num_pages, pages_cpu, seed):
    """A device pool of num_pages pages of page_bytes bytes, all 0xFF (NaN in
    bf16, NaN scales in the quantized layouts) except for the given pages,
    which land at the top ids in a seeded order. Returns the pool and the
    physical id of each given page."""
    n = pages_cpu.shape[0]
    assert num_pages * page_bytes > 2**31 and n < num_pages
    pool = torch.full((num_pages, page_bytes), 0xFF, dtype=torch.uint8, device=DEV)
    ids = num_pages - n + torch.randperm(n, generator=torch.Generator().manual_seed(seed))
    assert int(ids.max()) == num_pages - 1
    pool[ids.to(DEV)] = pages_cpu.reshape(n, page_bytes).to(DEV)
    return pool, ids


def _large_case(lens, seed):
    need = [-(-L // 64) for L in lens]
    n = sum(need)
    g = torch.Generator().manual_seed(seed)
    local = torch.full((len(lens), max(need) + 3), -1, dtype=torch.int32)
    off = 0
    for b, k in enumerate(need):
        local[b, :k] = torch.arange(off, off + k, dtype=torch.int32)
        off += k
    q_abs = (torch.randn((len(lens), 1, 128, 512), generator=g) * 0.05).to(torch.bfloat16)
    q_r = torch.randn((len(lens), 1, 128, 64), generator=g).to(torch.bfloat16)
    return n, local, q_abs, q_r, torch.tensor(lens, dtype=torch.int32)


def _remap(local, ids):
    return torch.where(local >= 0, ids[local.clamp(min=0).long()].to(torch.int32), local)


LARGE_LENS = [1, 4000, 9000, 64 * 30]


def test_large_bf16_pool_gather_and_decode(M):
    """A 2.21 GB bf16 pool (30000 pages; page ids >= 29128 start past 2^31
    bytes) whose sequences live in its top pages: the gather is bit-exact and
    the decode meets the bar against the oracle on the same rows."""
    n, local, q_abs, q_r, sl = _large_case(LARGE_LENS, 31)
    pages = torch.randn((n, 64, 576), generator=torch.Generator().manual_seed(32)).to(torch.bfloat16)
    pool_u8, ids = _top_pool(73728, 30000, pages.view(torch.uint8), 33)
    assert int(ids.min()) * 73728 > 2**31
    pool = pool_u8.view(torch.bfloat16).view(30000, 64, 576)
    bt = _remap(local, ids)
    _say(f"large bf16 pool: 30000 pages, ids {int(ids.min())}..{int(ids.max())}, lens={LARGE_LENS}")
    out = M.mla_debug_gather(pool, bt.to(DEV), sl.to(DEV), max(LARGE_LENS))
    o_part, lse_part = M.mla_decode_paged(q_abs.to(DEV), q_r.to(DEV), pool, bt.to(DEV), sl.to(DEV), 5, SCALE)
    o_lat, lse = M.mla_combine_splits(o_part, lse_part)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    bits = O.bf16_bits(pages)
    for b, L in enumerate(LARGE_LENS):
        ref = np.zeros((max(LARGE_LENS), 576), np.uint16)
        ref[:L] = bits[local[b, :-(-L // 64)].numpy().astype(np.int64)].reshape(-1, 576)[:L]
        assert np.array_equal(got[b], ref), f"gather, sequence {b}"
    ref_o, ref_l = O.decode_absorbed(O.as_f64(q_abs), O.as_f64(q_r), bits, local.numpy(), sl.numpy(), SCALE)
    assert_bar(o_lat.cpu().numpy(), ref_o, "large bf16 pool o_lat")
    assert_lse(lse.cpu().numpy(), ref_l, "large bf16 pool lse")
    del pool, pool_u8
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", ["fp8", "mxfp4"])
def test_large_quantized_pool_decode(M, fmt):
    """The 8-bit (53000 pages of 41216 bytes; ids >= 52104 start past 2^31)
    and 4-bit (85000 pages of 25600 bytes; ids >= 83887) caches, sequences in
    the top pages, against the oracle over the stored values."""
    from mla_inputs import random_fp8_pages, random_mxfp4_pages
    n, local, q_abs, q_r, sl = _large_case(LARGE_LENS, 41)
    if fmt == "fp8":
        pages, num_pages, page_bytes, scan, cache_cls = (random_fp8_pages(n, 42), 53000, 41216,
                                                         M.mla_decode_paged_fp8, O.PagedFp8Cache)
    else:
        pages, num_pages, page_bytes, scan, cache_cls = (random_mxfp4_pages(n, 42), 85000, 25600,
                                                         M.mla_decode_paged_mxfp4, O.PagedMxfp4Cache)
    pool, ids = _top_pool(page_bytes, num_pages, pages, 43)
    assert int(ids.min()) * page_bytes > 2**31
    bt = _remap(local, ids)
    _say(f"large {fmt} pool: {num_pages} pages, ids {int(ids.min())}..{int(ids.max())}, lens={LARGE_LENS}")
    o_part, lse_part = scan(q_abs.to(DEV), q_r.to(DEV), pool, bt.to(DEV), sl.to(DEV), 5, SCALE)
    o_lat, lse = M.mla_combine_splits(o_part, lse_part)
    torch.cuda.synchronize()
    cache = cache_cls(pages.numpy())
    ref_o, ref_l = O.decode_absorbed(O.as_f64(q_abs), O.as_f64(q_r), cache, local.numpy(), sl.numpy(), SCALE)
    assert_bar(o_lat.cpu().numpy(), ref_o, f"large {fmt} pool o_lat")
    assert_lse(lse.cpu().numpy(), ref_l, f"large {fmt} pool lse")
    del pool
    torch.cuda.empty_cache()
