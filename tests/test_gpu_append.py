"""GPU parity of the step before the decode path: the latent-cache append
(c_KV copied, k_R rotated, written through the block table) and the RoPE
rotation of the queries, against the fp64 oracle, and the append followed by
the decode against the oracle's own append and decode.

Bars: cache rows the append must not touch and the copied c_KV values are
bit-exact; a rotated value may differ from the fp64 rotation by its bf16
rounding (2^-8 relative: bf16 keeps 8 significant bits) plus the fp32
arithmetic on the pair
(2^-20 of |x0| + |x1|), and the standard floating-point bar is reported too.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
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


def _append_case(lens, s_q, seed, width=None):
    """Random cache and chunk; the logical pages the chunk writes get distinct
    physical pages, every other block-table entry an arbitrary valid page."""
    g = torch.Generator().manual_seed(seed)
    B = len(lens)
    width = width or max(max(-(-L // 64) for L in lens), 1)
    targets = sorted({(b, p // 64) for b, L in enumerate(lens) for p in range(max(L - s_q, 0), L)
                      if p // 64 < width})
    pool = len(targets) + 3
    ids = torch.randperm(pool, generator=g)
    bt = torch.randint(0, pool, (B, width), generator=g, dtype=torch.int32)
    for k, (b, lp) in enumerate(targets):
        bt[b, lp] = int(ids[k])
    cache = torch.randn((pool, 64, 576), generator=g).to(torch.bfloat16)
    c_new = torch.randn((B, s_q, 512), generator=g).to(torch.bfloat16)
    kr_new = torch.randn((B, s_q, 64), generator=g).to(torch.bfloat16)
    return cache, bt, torch.tensor(lens, dtype=torch.int32), c_new, kr_new


def _pair_bound(x):
    """|x0| + |x1| of each value's pair, repeated for both members."""
    a = np.abs(np.asarray(x, np.float64))
    s = a[..., 0::2] + a[..., 1::2]
    return np.repeat(s, 2, axis=-1)


def _check_rotation(got, ref, x, what):
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -20 * _pair_bound(x)
    worst = float((err - bound).max()) if err.size else 0.0
    print(f"  {what}: worst excess over the rounding bound {worst:.2e}", flush=True)
    assert (err <= bound).all(), f"{what}: rotation error above its rounding bound"
    if err.size:
        assert_bar(got, ref, what)


def _run_append(M, cache, bt, sl, c_new, kr_new, max_pos):
    rope = M.mla_rope_table(max_pos)
    kv = cache.to(DEV)
    M.mla_append_latent(kv, bt.to(DEV), sl.to(DEV), c_new.to(DEV), kr_new.to(DEV), rope)
    torch.cuda.synchronize()
    return kv.cpu()


def _compare_append(out, cache, ref, written, what):
    mask = np.zeros(cache.shape[:2], bool)
    for pg, r in written:
        mask[pg, r] = True
    bits_out, bits_in = O.bf16_bits(out), O.bf16_bits(cache)
    assert (bits_out[~mask] == bits_in[~mask]).all(), f"{what}: rows outside the chunk changed"
    got = O.as_f64(out)[mask]
    exp = ref[mask]
    assert np.array_equal(got[:, :512], exp[:, :512]), f"{what}: c_KV not copied bit for bit"
    return got, exp, mask


@pytest.mark.parametrize("lens,s_q,width", [
    ([2, 70, 200], 3, None),         # a sequence shorter than the chunk; page crossings
    ([65536, 1, 4097], 1, None),     # decode: large position, position 0, page boundary
    ([1000, 1300], 300, None),       # a chunk spanning several pages
    ([130], 4, 2),                   # positions past the block table are not written
])
def test_append_latent_parity(M, lens, s_q, width):
    cache, bt, sl, c_new, kr_new = _append_case(lens, s_q, seed=sum(lens) + s_q, width=width)
    _say(f"append lens={lens} s_q={s_q} width={bt.shape[1]}")
    out = _run_append(M, cache, bt, sl, c_new, kr_new, max_pos=max(lens) + 1)
    ref, written = O.append_latent(O.as_f64(cache), bt.numpy(), sl.numpy(), O.as_f64(c_new), O.as_f64(kr_new))
    got, exp, mask = _compare_append(out, cache, ref, written, "append")
    # the unrotated inputs in the same (page, row) order as the mask
    x = np.zeros(ref.shape[:2] + (64,))
    pos = O.chunk_positions(sl.numpy(), s_q)
    for b in range(len(lens)):
        for i in range(s_q):
            p = int(pos[b, i])
            if 0 <= p < bt.shape[1] * 64:
                x[int(bt[b, p // 64]), p % 64] = O.as_f64(kr_new[b, i])
    _check_rotation(got[:, 512:], exp[:, 512:], x[mask], "append k_R")


def test_append_stops_at_the_rotation_table(M):
    """Tokens at positions >= max_pos have no table row and are not written."""
    lens, s_q, max_pos = [150], 80, 100             # positions 70..149
    cache, bt, sl, c_new, kr_new = _append_case(lens, s_q, seed=11)
    _say("append past the rotation table")
    out = _run_append(M, cache, bt, sl, c_new, kr_new, max_pos=max_pos)
    # the oracle for the tokens that have a table row: positions 70..99 = a
    # 30-token chunk ending at L = 100
    ref, written = O.append_latent(O.as_f64(cache), bt.numpy(), np.array([100]), O.as_f64(c_new[:, :30]),
                                   O.as_f64(kr_new[:, :30]))
    assert len(written) == 30
    got, exp, mask = _compare_append(out, cache, ref, written, "append capped")
    x = np.zeros(ref.shape[:2] + (64,))
    for i in range(30):
        p = 70 + i
        x[int(bt[0, p // 64]), p % 64] = O.as_f64(kr_new[0, i])
    _check_rotation(got[:, 512:], exp[:, 512:], x[mask], "append capped k_R")


@pytest.mark.parametrize("lens,s_q", [([2, 70, 65536], 3), ([1, 4097], 1), ([700], 256)])
def test_rope_q_parity(M, lens, s_q):
    g = torch.Generator().manual_seed(7 + s_q)
    B = len(lens)
    q = torch.randn((B, s_q, 128, 64), generator=g).to(torch.bfloat16)
    sl = torch.tensor(lens, dtype=torch.int32)
    _say(f"rope_q lens={lens} s_q={s_q}")
    rope = M.mla_rope_table(max(lens) + 1)
    qd = q.to(DEV)
    M.mla_rope_q(qd, sl.to(DEV), rope)
    torch.cuda.synchronize()
    got = O.as_f64(qd.cpu())
    x = O.as_f64(q)
    pos = O.chunk_positions(lens, s_q)
    live = pos >= 0
    assert (O.bf16_bits(qd.cpu())[~live] == O.bf16_bits(q)[~live]).all(), "rows without a position changed"
    ref = O.rope_rotate(x, pos[:, :, None])
    _check_rotation(got[live], ref[live], x[live], "rope_q")


def test_append_then_decode_matches_oracle(M):
    """Cache append and query rotation feeding the decode, against the oracle
    doing the same from the same raw inputs (fp64 throughout)."""
    lens, s_q = [300, 77, 129], 2
    cache, bt, sl, c_new, kr_new = _append_case(lens, s_q, seed=5)
    g = torch.Generator().manual_seed(6)
    q_abs = torch.randn((len(lens), s_q, 128, 512), generator=g).to(torch.bfloat16)
    q_r = torch.randn((len(lens), s_q, 128, 64), generator=g).to(torch.bfloat16)
    _say("append -> rope_q -> decode -> combine")
    rope = M.mla_rope_table(512)
    kv, btd, sld = cache.to(DEV), bt.to(DEV), sl.to(DEV)
    M.mla_append_latent(kv, btd, sld, c_new.to(DEV), kr_new.to(DEV), rope)
    qr = M.mla_rope_q(q_r.to(DEV), sld, rope)
    o_part, lse_part = M.mla_decode_paged(q_abs.to(DEV), qr, kv, btd, sld, 3, SCALE)
    o_lat, lse = M.mla_combine_splits(o_part, lse_part)
    torch.cuda.synchronize()
    ref_cache, _ = O.append_latent(O.as_f64(cache), bt.numpy(), sl.numpy(), O.as_f64(c_new), O.as_f64(kr_new))
    ref_qr = O.rope_rotate(O.as_f64(q_r), O.chunk_positions(lens, s_q)[:, :, None])
    ref_o, ref_l = O.decode_absorbed(O.as_f64(q_abs), ref_qr, ref_cache, bt.numpy(), sl.numpy(), SCALE)
    # the GPU's k_R and q_R carry one bf16 rounding each that the fp64 chain does not
    assert_bar(o_lat.cpu().numpy(), ref_o, "append+decode o_lat", l1_rel=5e-3)
    assert_lse(lse.cpu().numpy(), ref_l, "append+decode lse", tol=5e-3)


def test_append_and_rope_q_replay_in_a_graph(M):
    """Captured in a HIP graph and replayed three times, with eager work and
    synchronisations between the replays, every replay gives the eager result."""
    lens, s_q = [300, 77], 2
    cache, bt, sl, c_new, kr_new = _append_case(lens, s_q, seed=21)
    g = torch.Generator().manual_seed(22)
    q0 = torch.randn((len(lens), s_q, 128, 64), generator=g).to(torch.bfloat16)
    _say("append + rope_q in a HIP graph")
    rope = M.mla_rope_table(512)
    btd, sld, cd, kd = bt.to(DEV), sl.to(DEV), c_new.to(DEV), kr_new.to(DEV)
    kv_e, q_e = cache.to(DEV), q0.to(DEV)
    M.mla_append_latent(kv_e, btd, sld, cd, kd, rope)
    M.mla_rope_q(q_e, sld, rope)
    torch.cuda.synchronize()
    kv_g, q_g = cache.to(DEV), q0.to(DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        M.mla_append_latent(kv_g, btd, sld, cd, kd, rope)
        M.mla_rope_q(q_g, sld, rope)
    for rep in range(3):
        kv_g.copy_(cache.to(DEV))
        q_g.copy_(q0.to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(kv_g.cpu().view(torch.int16), kv_e.cpu().view(torch.int16)), f"replay {rep}: cache"
        assert torch.equal(q_g.cpu().view(torch.int16), q_e.cpu().view(torch.int16)), f"replay {rep}: q_r"
