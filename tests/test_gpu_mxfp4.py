"""GPU parity of the 4-bit (MXFP4) latent cache against the fp64 oracle.

The conversion and the append are byte work and must match the oracle's
quantizer bit for bit (a rotated k_R keeps the bf16 append's rounding bound).
The 4-bit decode scan is judged against the oracle's attention over the stored
values (E2M1 code times its block's scale) with the bar of the bf16 scan: it
multiplies the codes exactly (block-scaled E2M1 x E4M3 MFMAs for QK, with the
query as two E4M3 terms that reproduce it up to 2^-13 of each block's largest
value; exact bf16 dequantization of V for PV), so its own error is the bf16
scan's.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from mla_inputs import make_inputs, random_mxfp4_pages
from tests._plan import header_pieces, row_pages
from tests._bars import assert_bar, assert_lse

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SCALE = 1.0 / math.sqrt(192)
PB = 25600
ROPE0, SCALE0 = 16384, 24576


@pytest.fixture(scope="module")
def M():
    import mla_latent_kv_06_amd as mod
    return mod


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def _table(lens, g, extra=4):
    need = [-(-int(L) // 64) for L in lens]
    pool = sum(need) + extra
    order = torch.randperm(pool, generator=g)
    bt = torch.full((len(lens), max(max(need), 1) + 1), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[off:off + n].to(torch.int32)
        off += n
    return bt, pool


def _fp4_case(lens, s_q, seed):
    """Queries, a bf16 cache ~ N(0, 1) packed to 4 bits by the oracle, a permuted table."""
    g = torch.Generator().manual_seed(seed)
    bt, pool = _table(lens, g)
    B = len(lens)
    q_abs = torch.randn((B, s_q, 128, 512), generator=g).to(torch.bfloat16)
    q_r = torch.randn((B, s_q, 128, 64), generator=g).to(torch.bfloat16)
    kv = torch.randn((pool, 64, 576), generator=g).to(torch.bfloat16)
    pages = torch.from_numpy(O.pack_mxfp4_cache(O.bf16_bits(kv)))
    return q_abs, q_r, pages, bt, torch.tensor(lens, dtype=torch.int32)


def _decode4_check(M, q_abs, q_r, pages, bt, sl, S, what, check_parts=True):
    _say(f"{what}: B={q_abs.shape[0]} s_q={q_abs.shape[1]} lens={sl.tolist()[:6]} splits={S}")
    o_part, lse_part = M.mla_decode_paged_mxfp4(q_abs.to(DEV), q_r.to(DEV), pages.to(DEV), bt.to(DEV), sl.to(DEV),
                                                S, SCALE)
    o_lat, lse = M.mla_combine_splits(o_part, lse_part)
    torch.cuda.synchronize()
    cache = O.PagedMxfp4Cache(pages.numpy())
    ref_o, ref_l = O.decode_absorbed(O.as_f64(q_abs), O.as_f64(q_r), cache, bt.numpy(), sl.numpy(), SCALE)
    assert_bar(o_lat.cpu().numpy(), ref_o, f"{what} o_lat")
    assert_lse(lse.cpu().numpy(), ref_l, f"{what} lse")
    if check_parts:
        rp_o, rp_l = O.decode_split(O.as_f64(q_abs), O.as_f64(q_r), cache, bt.numpy(), sl.numpy(), SCALE,
                                    header_pieces(row_pages(sl.tolist(), q_abs.shape[1]), S), S)
        assert_lse(lse_part.cpu().numpy(), rp_l, f"{what} lse_part")
        live = np.isfinite(rp_l)
        assert_bar(o_part.cpu().numpy()[live], rp_o[live], f"{what} o_part")
    return o_lat, lse


# ---------------------------------------------------------------------------
# conversion and append: bit-exact
# ---------------------------------------------------------------------------

def _special_cache(seed=3, pool=24):
    """Gaussian rows at many magnitudes plus blocks the scale rule and the
    rounding treat specially."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn((pool, 64, 576), generator=g) * torch.exp(torch.empty((pool, 64, 1)).uniform_(-30, 30, generator=g))
    kv = x.to(torch.bfloat16)
    rows = kv.view(-1, 576)
    rows[0, :512] = 0                                            # all zero: scales 2^-126
    rows[1, :512] = -0.0                                         # negative zeros keep their sign
    rows[2, :512] = torch.randn(512, generator=g).to(torch.bfloat16) * 1e-39   # bf16 subnormals
    rows[3, :512] = 0.5
    rows[3, 7] = 6.0 * 2.0 ** -3                                 # block 0 max exactly 6 * 2^k: k = -3
    rows[4, :512] = torch.randn(512, generator=g).to(torch.bfloat16) * 3e37  # near the top of bf16
    # every E2M1 rounding midpoint, both signs, in blocks whose largest value is 6 (k = 0)
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=torch.float64)
    t = torch.arange(512)
    ties = mids[t % 7] * torch.where((t // 7) % 2 == 1, -1.0, 1.0).double()
    ties[t % 32 == 31] = 6.0
    rows[5, :512] = ties.to(torch.bfloat16)
    assert torch.equal(rows[5, :512].double(), ties)
    # blocks mixing one value with others 2^-10 .. 2^-30 smaller (they round to 0)
    rows[6, :512] = torch.randn(512, generator=g).to(torch.bfloat16) * 2.0 ** -20
    rows[6, ::32] = 3.0
    return kv


def test_quantize_cache_mxfp4_bit_exact(M):
    kv = _special_cache()
    _say(f"quantize mxfp4 cache pages={kv.shape[0]}")
    out = M.mla_quantize_cache_mxfp4(kv.to(DEV))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = O.pack_mxfp4_cache(O.bf16_bits(kv))
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:3].tolist()}"


def test_quantize_mxfp4_full_cache_sampled_pages(M):
    """The whole 16384-page cache of the 64K-context workload, sampled pages
    compared with the oracle byte for byte."""
    inp = make_inputs("long")
    P = inp.kv_cache.shape[0]
    _say(f"quantize mxfp4 full cache pages={P}")
    out = M.mla_quantize_cache_mxfp4(inp.kv_cache.to(DEV))
    torch.cuda.synchronize()
    rng = np.random.default_rng(4)
    pick = np.concatenate([[0, P - 1], rng.choice(P, 30, replace=False)])
    got = out[torch.from_numpy(pick).to(DEV)].cpu().numpy()
    ref = O.pack_mxfp4_cache(O.bf16_bits(inp.kv_cache[torch.from_numpy(pick)]))
    assert np.array_equal(got, ref)


def _rotation_ok(got, ref, x):
    a = np.abs(np.asarray(x, np.float64))
    pair = np.repeat(a[..., 0::2] + a[..., 1::2], 2, axis=-1)
    return np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * pair


@pytest.mark.parametrize("lens,s_q", [([2, 70, 200], 3), ([65536, 1, 4097], 1), ([1000, 1300], 300)])
def test_append_mxfp4_matches_oracle(M, lens, s_q):
    g = torch.Generator().manual_seed(sum(lens) + s_q + 1)
    B = len(lens)
    width = max(-(-L // 64) for L in lens)
    targets = sorted({(b, p // 64) for b, L in enumerate(lens) for p in range(max(L - s_q, 0), L)})
    pool = len(targets) + 3
    ids = torch.randperm(pool, generator=g)
    bt = torch.randint(0, pool, (B, width), generator=g, dtype=torch.int32)
    for k, (b, lp) in enumerate(targets):
        bt[b, lp] = int(ids[k])
    base = torch.from_numpy(O.pack_mxfp4_cache(O.bf16_bits(
        torch.randn((pool, 64, 576), generator=g).to(torch.bfloat16))))
    c_new = torch.randn((B, s_q, 512), generator=g).to(torch.bfloat16)
    kr_new = torch.randn((B, s_q, 64), generator=g).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32)
    _say(f"append mxfp4 lens={lens} s_q={s_q}")
    rope = M.mla_rope_table(max(lens) + 1)
    kv = base.to(DEV)
    M.mla_append_latent_mxfp4(kv, bt.to(DEV), sl.to(DEV), c_new.to(DEV), kr_new.to(DEV), rope)
    torch.cuda.synchronize()
    got = kv.cpu().numpy()
    exp = base.numpy().copy()
    touched = np.zeros_like(exp, dtype=bool)
    pos = O.chunk_positions(lens, s_q)
    codes, k = O.quantize_latent_mxfp4(O.as_f64(c_new))
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    rot_x, rot_ref, rot_at = [], [], []
    for b in range(B):
        for i in range(s_q):
            p = int(pos[b, i])
            if p < 0:
                continue
            pg, r = int(bt[b, p // 64]), p % 64
            exp[pg, r * 256:(r + 1) * 256] = packed[b, i]
            exp[pg, SCALE0 + 16 * r:SCALE0 + 16 * (r + 1)] = (k[b, i] + 127).astype(np.uint8)
            touched[pg, ROPE0 + 128 * r:ROPE0 + 128 * (r + 1)] = True
            rot_x.append(O.as_f64(kr_new[b, i]))
            rot_ref.append(O.rope_rotate(O.as_f64(kr_new[b, i]), p))
            rot_at.append((pg, r))
    assert np.array_equal(got[~touched], exp[~touched]), "codes, scales or untouched bytes differ"
    gr = np.stack([O.bf16_bits_to_f64(got[pg, ROPE0 + 128 * r:ROPE0 + 128 * (r + 1)].copy().view("<u2"))
                   for pg, r in rot_at])
    assert _rotation_ok(gr, np.stack(rot_ref), np.stack(rot_x)).all(), "k_R rotation above its rounding bound"


# ---------------------------------------------------------------------------
# decode over the 4-bit cache
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("lens,s_q,S", [
    ([1, 31, 32, 33, 63], 1, 1),
    ([64, 65, 127, 129, 2047], 1, 3),
    ([5, 300, 1000], 1, 17),
    ([300, 77], 2, 2),
    ([100, 400], 37, 3),
])
def test_decode_mxfp4_edge_lengths(M, lens, s_q, S):
    q_abs, q_r, pages, bt, sl = _fp4_case(lens, s_q, seed=sum(lens) + s_q + 5)
    _decode4_check(M, q_abs, q_r, pages, bt, sl, S, f"mxfp4 lens={lens} s_q={s_q}")


def test_decode_mxfp4_zero_length_rows(M):
    q_abs, q_r, pages, bt, sl = _fp4_case([0, 70], 1, seed=19)
    o_lat, lse = _decode4_check(M, q_abs, q_r, pages, bt, sl, 2, "mxfp4 zero length")
    assert (o_lat[0].cpu() == 0).all() and torch.isneginf(lse[0].cpu()).all()


def test_decode_mxfp4_garbage_past_the_end(M):
    """Rows past a sequence's end hold the largest codes, NaN scale bytes
    (0xFF) and NaN k_R; none of it may reach the result."""
    lens = [100, 33, 130]
    q_abs, q_r, pages, bt, sl = _fp4_case(lens, 1, seed=20)
    for b, L in enumerate(lens):
        if L % 64:
            pg, r0 = int(bt[b, L // 64]), L % 64
            pages[pg, r0 * 256:64 * 256] = 0x77
            pages[pg, ROPE0 + r0 * 128:SCALE0] = 0xFF
            pages[pg, SCALE0 + 16 * r0:] = 0xFF
    _decode4_check(M, q_abs, q_r, pages, bt, sl, 2, "mxfp4 garbage past the end", check_parts=False)


def test_decode_mxfp4_uniform_config_full(M):
    """B = 16 at 4096 tokens, the bf16 cache of that workload quantized by the
    library and checked byte for byte first, then the whole decode layer."""
    inp = make_inputs("uniform")
    d = {k: getattr(inp, k).to(DEV) for k in ("q_c", "q_r", "w_uk", "kv_cache", "w_uv", "block_table", "seqlens")}
    _say("mxfp4 uniform config: quantize + decode layer")
    pages = M.mla_quantize_cache_mxfp4(d["kv_cache"])
    torch.cuda.synchronize()
    ref_pages = O.pack_mxfp4_cache(O.bf16_bits(inp.kv_cache))
    assert np.array_equal(pages.cpu().numpy(), ref_pages)
    S = M.mla_recommended_splits(16, 1, 4096)
    r = M.decode_layer(d["q_c"], d["q_r"], pages, d["block_table"], d["seqlens"], d["w_uk"], d["w_uv"], num_splits=S)
    torch.cuda.synchronize()
    ref_o, ref_l = O.decode_absorbed(O.as_f64(r["q_abs"].cpu()), O.as_f64(inp.q_r), O.PagedMxfp4Cache(ref_pages),
                                     inp.block_table.numpy(), inp.seqlens.numpy(), SCALE)
    assert_bar(r["o_lat"].cpu().numpy(), ref_o, "mxfp4 uniform o_lat")
    assert_lse(r["lse"].cpu().numpy(), ref_l, "mxfp4 uniform lse")


def test_decode_mxfp4_long_config_full(M):
    """The 64K-context workload (B = 16) over a seeded 4-bit cache, in the
    launch configuration of the benchmark: every (b, h) row of o_lat and lse
    against the oracle over the stored values."""
    inp = make_inputs("long", with_cache=False)
    P = int(inp.block_table.max()) + 1
    pages = random_mxfp4_pages(P, seed=78)
    d = {k: getattr(inp, k).to(DEV) for k in ("q_c", "q_r", "w_uk", "w_uv", "block_table", "seqlens")}
    S = M.mla_plan_splits(inp.seqlens.tolist(), inp.block_table.shape[1], 1)
    _say(f"mxfp4 long config: pages={P} splits={S} (all rows)")
    r = M.decode_layer(d["q_c"], d["q_r"], pages.to(DEV), d["block_table"], d["seqlens"], d["w_uk"], d["w_uv"],
                       num_splits=S)
    torch.cuda.synchronize()
    ro, rl = O.decode_absorbed(O.as_f64(r["q_abs"].cpu()), O.as_f64(inp.q_r), O.PagedMxfp4Cache(pages.numpy()),
                               inp.block_table.numpy(), inp.seqlens.numpy(), SCALE)
    assert_bar(r["o_lat"].cpu().numpy(), ro, "mxfp4 long o_lat (all rows)")
    assert_lse(r["lse"].cpu().numpy(), rl, "mxfp4 long lse (all rows)")


def test_decode_mxfp4_query_with_wide_range_inside_blocks(M):
    """Blocks of the query that mix one large value with values 10^4 to 2^20
    times smaller, and blocks of zeros, still meet the bar."""
    lens = [900, 257]
    q_abs, q_r, pages, bt, sl = _fp4_case(lens, 1, seed=33)
    g = torch.Generator().manual_seed(34)
    q = torch.randn((2, 1, 128, 512), generator=g) * 0.01
    q[..., ::32] = 100.0 * torch.sign(torch.randn((2, 1, 128, 16), generator=g))
    q[..., 5::32] *= 2.0 ** -20 / 0.01
    q[:, :, :64, 64:128] = 0.0
    q_abs = (q * 0.02).to(torch.bfloat16)
    _decode4_check(M, q_abs, q_r, pages, bt, sl, 3, "mxfp4 wide-range query")


def test_decode_layer_dispatches_on_the_cache_format(M):
    """decode_layer over the 4-bit cache runs the 4-bit scan; the decompressed
    branch refuses it (it reads bf16 rows)."""
    q_abs, q_r, pages, bt, sl = _fp4_case([200, 64], 1, seed=40)
    assert M.is_mxfp4_cache(pages) and not M.is_fp8_cache(pages)
    g = torch.Generator().manual_seed(41)
    q_c = torch.randn((2, 1, 128, 128), generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16).to(DEV)
    r = M.decode_layer(q_c, q_r.to(DEV), pages.to(DEV), bt.to(DEV), sl.to(DEV), w, w, num_splits=2)
    o_part, lse_part = M.mla_decode_paged_mxfp4(r["q_abs"], q_r.to(DEV), pages.to(DEV), bt.to(DEV), sl.to(DEV), 2,
                                                SCALE)
    torch.cuda.synchronize()
    assert torch.equal(lse_part, r["lse_part"])
    live = torch.isfinite(lse_part)          # empty split slots (LSE -inf) leave o_part unwritten
    assert torch.equal(o_part[live], r["o_part"][live])
    with pytest.raises(ValueError):
        M.attention_layer(q_c, q_r.to(DEV), pages.to(DEV), bt.to(DEV), sl.to(DEV), w, w, max_len=200, absorbed=False)
