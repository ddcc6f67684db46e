"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these re-types an oracle formula: each check is a closed form, a
brute-force loop in plain Python floats, a value printed on the pages, or an
identity between two independently written paths (naive vs absorbed).
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
from mla_inputs import make_inputs, tiny_inputs, CONFIGS, make_structure

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# storage arithmetic printed on the teardown page (sections 1 and 3)
# --------------------------------------------------------------------------

def test_storage_arithmetic_matches_teardown_page():
    g = _golden("teardown_storage.json")
    d_c, d_r = g["latent_kv_dim"], g["rope_dim"]
    assert O.latent_row_elems(d_c, d_r) == g["elements_per_token_layer"]
    assert O.latent_row_bytes(d_c, d_r) / 1024 == g["bf16_kb_per_token_layer"]
    mha = O.mha_kv_bytes_per_token_layer(g["heads"], g["head_dim_content"])
    assert mha / 1024 == g["mha_kb_per_token_layer"]
    assert round(100 * (1 - O.latent_row_bytes(d_c, d_r) / mha), 2) == g["compression_percent"]
    assert 16 * O.latent_row_bytes(d_c, d_r) / 1024 == g["page16_kb"]
    assert 64 * O.latent_row_bytes(d_c, d_r) / 1024 == pytest.approx(g["page64_kb_approx"], rel=0.01)
    assert O.default_scale(g["head_dim_content"], g["rope_dim"]) == 1.0 / math.sqrt(g["softmax_scale_denominator_sqrt_of"])


def test_k3_byte_count_per_token():
    g = _golden("k3_mla_bytes.json")
    per_tok = g["mla_layers"] * O.latent_row_bytes()
    assert per_tok / 1024 == pytest.approx(g["kib_per_token_all_layers"], abs=0.05)
    # "1M context" read as 2^20 tokens: 28.99 GB vs the printed 28.96 GB (0.1%)
    assert per_tok * 2**20 / 1e9 == pytest.approx(g["gb_per_step_at_1M"], rel=2e-3)
    bw = g["gb_per_step_at_1M"] / (g["scan_ms_at_1M"] * 1e-3) / 1e3
    assert bw == pytest.approx(g["scan_tb_per_s"], abs=0.01)
    assert 100 * bw / g["peak_tb_per_s"] == pytest.approx(g["scan_fraction_of_peak_percent"], abs=0.05)


# --------------------------------------------------------------------------
# bf16 decoding: against IEEE bit patterns and torch's own conversion
# --------------------------------------------------------------------------

def test_bf16_decoding():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x4049, 0x0000, 0x8000], dtype=np.uint16)
    v = O.bf16_bits_to_f64(bits)
    assert v[0] == 1.0 and v[1] == -2.0
    assert v[2] == np.inf and v[3] == -np.inf
    assert v[4] == 2.0 ** -133
    assert v[5] == 3.140625
    assert v[6] == 0.0 and np.signbit(v[7])
    x = torch.randn(4096, dtype=torch.float32).to(torch.bfloat16)
    assert np.array_equal(O.as_f64(x), x.to(torch.float64).numpy())


# --------------------------------------------------------------------------
# brute force in plain Python floats (tiny dims, several pages, ragged, causal)
# --------------------------------------------------------------------------

def _brute_naive(inp, scale):
    """Path A written as explicit loops over Python floats."""
    q_c, q_r = inp["q_c"].tolist(), inp["q_r"].tolist()
    w_uk, w_uv = inp["w_uk"].tolist(), inp["w_uv"].tolist()
    kv, bt, seqlens = inp["kv_cache"].tolist(), inp["block_table"].tolist(), inp["seqlens"].tolist()
    B, s_q, Hn, d_hc = inp["q_c"].shape
    d_c = inp["w_uk"].shape[2]
    page = inp["kv_cache"].shape[1]
    out = [[[None] * Hn for _ in range(s_q)] for _ in range(B)]
    lse = [[[None] * Hn for _ in range(s_q)] for _ in range(B)]
    for b in range(B):
        L = seqlens[b]
        rows = []
        for t in range(L):
            rows.append(kv[bt[b][t // page]][t % page])
        for i in range(s_q):
            last = L - s_q + i  # last visible key index
            for h in range(Hn):
                scores, vals = [], []
                for t in range(last + 1):
                    row = rows[t]
                    k = [sum(row[c] * w_uk[h][d][c] for c in range(d_c)) for d in range(d_hc)]
                    v = [sum(row[c] * w_uv[h][d][c] for c in range(d_c)) for d in range(d_hc)]
                    s = sum(q_c[b][i][h][d] * k[d] for d in range(d_hc))
                    s += sum(q_r[b][i][h][j] * row[d_c + j] for j in range(len(q_r[b][i][h])))
                    scores.append(s * scale)
                    vals.append(v)
                mx = max(scores)
                ex = [math.exp(s - mx) for s in scores]
                tot = sum(ex)
                out[b][i][h] = [sum(ex[t] * vals[t][d] for t in range(len(ex))) / tot for d in range(d_hc)]
                lse[b][i][h] = mx + math.log(tot)
    return np.array(out), np.array(lse)


def _brute_absorbed(inp, q_abs, scale):
    """o_lat and lse over the latent rows, as explicit loops."""
    q_r = inp["q_r"].tolist()
    kv, bt, seqlens = inp["kv_cache"].tolist(), inp["block_table"].tolist(), inp["seqlens"].tolist()
    qa = np.asarray(q_abs).tolist()
    B, s_q, Hn, d_c = np.asarray(q_abs).shape
    page = inp["kv_cache"].shape[1]
    o = np.zeros((B, s_q, Hn, d_c))
    l = np.zeros((B, s_q, Hn))
    for b in range(B):
        L = seqlens[b]
        for i in range(s_q):
            n = L - s_q + i + 1
            for h in range(Hn):
                sc = []
                for t in range(n):
                    row = kv[bt[b][t // page]][t % page]
                    s = sum(qa[b][i][h][c] * row[c] for c in range(d_c))
                    s += sum(q_r[b][i][h][j] * row[d_c + j] for j in range(len(row) - d_c))
                    sc.append(s * scale)
                mx = max(sc)
                ex = [math.exp(s - mx) for s in sc]
                tot = sum(ex)
                for c in range(d_c):
                    o[b, i, h, c] = sum(ex[t] * kv[bt[b][t // page]][t % page][c] for t in range(n)) / tot
                l[b, i, h] = mx + math.log(tot)
    return o, l


@pytest.mark.parametrize("seqlens,s_q", [([7, 10], 3), ([4, 1, 9], 1), ([13], 5)])
def test_brute_force_tiny(seqlens, s_q):
    inp = tiny_inputs(B=len(seqlens), s_q=s_q, seqlens=seqlens, h=2, d_hc=3, d_c=5, d_r=2, page=4)
    n = {k: v.numpy() for k, v in inp.items()}
    scale = 1.0 / math.sqrt(3 + 2)
    ref_out, ref_lse = _brute_naive(inp, scale)
    out_a, lse_a = O.decode_naive(n["q_c"], n["q_r"], n["kv_cache"], n["block_table"], n["seqlens"],
                                  n["w_uk"], n["w_uv"], scale)
    np.testing.assert_allclose(out_a, ref_out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_a, ref_lse, rtol=1e-12, atol=1e-13)
    q_abs = O.absorb(n["q_c"], n["w_uk"])
    o_lat, lse_b = O.decode_absorbed(q_abs, n["q_r"], n["kv_cache"], n["block_table"], n["seqlens"], scale)
    ref_o, ref_l = _brute_absorbed(inp, q_abs, scale)
    np.testing.assert_allclose(o_lat, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse_b, ref_l, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(O.up_proj(o_lat, n["w_uv"]), ref_out, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse_b, ref_lse, rtol=1e-12, atol=1e-13)


def test_absorb_brute_force():
    g = np.random.default_rng(3)
    q = g.standard_normal((2, 3, 4, 5))
    w = g.standard_normal((4, 5, 6))
    ref = np.zeros((2, 3, 4, 6))
    for a in range(2):
        for b in range(3):
            for h in range(4):
                for c in range(6):
                    ref[a, b, h, c] = sum(q[a, b, h, d] * w[h, d, c] for d in range(5))
    np.testing.assert_allclose(O.absorb(q, w), ref, rtol=1e-13, atol=1e-14)


def test_up_proj_brute_force():
    g = np.random.default_rng(4)
    o = g.standard_normal((3, 4, 7))
    w = g.standard_normal((4, 5, 7))
    ref = np.zeros((3, 4, 5))
    for t in range(3):
        for h in range(4):
            for d in range(5):
                ref[t, h, d] = sum(o[t, h, c] * w[h, d, c] for c in range(7))
    np.testing.assert_allclose(O.up_proj(o, w), ref, rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# the teardown page's equivalence (section 4) at real dims, in fp64
# --------------------------------------------------------------------------

def test_naive_equals_absorbed_real_dims():
    inp = make_inputs("single")
    f = {k: O.as_f64(getattr(inp, k)) for k in ("q_c", "q_r", "w_uk", "kv_cache", "w_uv")}
    bt, L = inp.block_table.numpy(), inp.seqlens.numpy()
    scale = O.default_scale()
    out_a, lse_a = O.decode_naive(f["q_c"], f["q_r"], f["kv_cache"], bt, L, f["w_uk"], f["w_uv"], scale)
    q_abs = O.absorb(f["q_c"], f["w_uk"])
    o_lat, lse_b = O.decode_absorbed(q_abs, f["q_r"], f["kv_cache"], bt, L, scale)
    out_b = O.up_proj(o_lat, f["w_uv"])
    assert np.abs(out_a - out_b).max() <= 1e-11 * np.abs(out_a).max()
    assert np.abs(lse_a - lse_b).max() <= 1e-11


def test_score_variance_with_documented_weight_scale():
    """W ~ N(0, 1/512) with unit inputs makes the scaled score variance 1."""
    inp = make_inputs("single")
    q_abs = O.absorb(O.as_f64(inp.q_c), O.as_f64(inp.w_uk))
    kv = O.as_f64(inp.kv_cache).reshape(-1, 576)
    s = O.scores_absorbed(q_abs[0, 0], O.as_f64(inp.q_r)[0, 0], kv[:, :512], kv[:, 512:], O.default_scale())
    assert 0.9 < s.std() < 1.1


# --------------------------------------------------------------------------
# softmax and closed forms
# --------------------------------------------------------------------------

def test_softmax_rows_sum_to_one():
    g = np.random.default_rng(5)
    s = g.standard_normal((64, 1000)) * 7
    P, m, l = O.softmax_rows(s)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-12)
    assert (P >= 0).all()
    np.testing.assert_array_equal(m, s.max(-1))


def _single_row_inputs(L, seed=11):
    g = torch.Generator().manual_seed(seed)
    kv = torch.randn((-(-L // 64), 64, 576), generator=g).to(torch.bfloat16)
    return O.as_f64(kv), np.arange(kv.shape[0])[None].astype(np.int32)


def test_closed_form_single_key():
    kv, bt = _single_row_inputs(1)
    g = np.random.default_rng(6)
    qa, qr = g.standard_normal((1, 1, 128, 512)), g.standard_normal((1, 1, 128, 64))
    o, lse = O.decode_absorbed(qa, qr, kv, bt, [1], O.default_scale())
    assert np.array_equal(o[0, 0], np.broadcast_to(kv[0, 0, :512], (128, 512)))
    s0 = (qa[0, 0] @ kv[0, 0, :512] + qr[0, 0] @ kv[0, 0, 512:]) * O.default_scale()
    np.testing.assert_allclose(lse[0, 0], s0, rtol=1e-14, atol=1e-14)


def test_closed_form_zero_query_is_mean():
    L = 300
    kv, bt = _single_row_inputs(L)
    qa, qr = np.zeros((1, 1, 4, 512)), np.zeros((1, 1, 4, 64))
    o, lse = O.decode_absorbed(qa, qr, kv, bt, [L], O.default_scale())
    mean = kv.reshape(-1, 576)[:L, :512].mean(0)
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(mean, (4, 512)), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse[0, 0], math.log(L), rtol=1e-14)


def test_closed_form_one_hot_selects_row():
    L, tstar = 200, 137
    kv, bt = _single_row_inputs(L)
    kv = kv.copy()
    kv[..., 512:] = 0.0
    kv.reshape(-1, 576)[tstar, 512] = 1.0
    qa = np.zeros((1, 1, 2, 512))
    qr = np.zeros((1, 1, 2, 64))
    qr[..., 0] = 2000.0
    o, lse = O.decode_absorbed(qa, qr, kv, bt, [L], O.default_scale())
    row = kv.reshape(-1, 576)[tstar, :512]
    np.testing.assert_allclose(o[0, 0], np.broadcast_to(row, (2, 512)), rtol=1e-15, atol=1e-50)
    np.testing.assert_allclose(lse[0, 0], 2000.0 * O.default_scale(), rtol=1e-14)


def test_empty_range_convention():
    kv, bt = _single_row_inputs(64)
    o, lse = O.decode_absorbed(np.ones((1, 1, 3, 512)), np.ones((1, 1, 3, 64)), kv, bt, [0], 0.1)
    assert (o == 0).all() and np.isneginf(lse).all()


# --------------------------------------------------------------------------
# paged gather
# --------------------------------------------------------------------------

def test_gather_matches_token_loop_and_rejects_bad_ids():
    st = make_structure(CONFIGS["ragged"], seed=5)
    pool = st.num_pages
    kv = np.arange(pool * 64 * 3, dtype=np.float64).reshape(pool, 64, 3)
    for b in (0, 17, 63):
        L = int(st.seqlens[b])
        rows = O.gather_rows(kv, st.block_table[b].numpy(), L)
        bt = st.block_table[b].tolist()
        ref = np.array([kv[bt[t // 64], t % 64] for t in range(L)])
        assert np.array_equal(rows, ref)
    bad = st.block_table[0].numpy().copy()
    bad[0] = pool
    with pytest.raises(ValueError):
        O.gather_rows(kv, bad, 10)


def test_page_permutation_invariance():
    inp = tiny_inputs(B=2, s_q=2, seqlens=[150, 70], h=3, d_hc=4, d_c=8, d_r=2, page=16, seed=9)
    n = {k: v.numpy() for k, v in inp.items()}
    qa = O.absorb(n["q_c"], n["w_uk"])
    o1, l1 = O.decode_absorbed(qa, n["q_r"], n["kv_cache"], n["block_table"], n["seqlens"], 0.3)
    perm = np.random.default_rng(1).permutation(n["kv_cache"].shape[0])
    inv = np.argsort(perm)
    kv2 = n["kv_cache"][perm]          # new physical page p holds old page perm[p]
    bt2 = np.where(n["block_table"] >= 0, inv[np.maximum(n["block_table"], 0)], -1)
    o2, l2 = O.decode_absorbed(qa, n["q_r"], kv2, bt2, n["seqlens"], 0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# --------------------------------------------------------------------------
# split scan + combine
# --------------------------------------------------------------------------

def _random_pieces(row_pages, num_splits, rng):
    """An arbitrary page-aligned partition of every row into at most num_splits
    pieces (cut points drawn at random, empty pieces allowed, slots shuffled)."""
    out = []
    for n in row_pages:
        k = int(rng.integers(1, num_splits + 1))
        cuts = np.sort(rng.integers(0, n + 1, size=k - 1)) if k > 1 else np.array([], int)
        edges = [0] + [int(c) for c in cuts] + [int(n)]
        slots = rng.permutation(num_splits)[:k]
        out.append([(int(s_), edges[j], edges[j + 1]) for j, s_ in enumerate(slots)])
    return out


@pytest.mark.parametrize("num_splits", [1, 2, 7, 20])
def test_split_invariance(num_splits):
    """Any page-aligned partition merges to the unsplit result (K3 study,
    "Inside the blocks": stage 2 reduces the per-split partials exactly)."""
    inp = tiny_inputs(B=3, s_q=2, seqlens=[300, 64, 129], h=4, d_hc=8, d_c=32, d_r=8, page=16, seed=12)
    n = {k: v.numpy() for k, v in inp.items()}
    qa = O.absorb(n["q_c"], n["w_uk"])
    ref_o, ref_l = O.decode_absorbed(qa, n["q_r"], n["kv_cache"], n["block_table"], n["seqlens"], 0.25)
    rows = [-(-max(int(L) - 2 + i + 1, 0) // 16) for L in n["seqlens"] for i in range(2)]
    rng = np.random.default_rng(num_splits)
    for _ in range(3):
        pieces = _random_pieces(rows, num_splits, rng)
        op, lp = O.decode_split(qa, n["q_r"], n["kv_cache"], n["block_table"], n["seqlens"], 0.25, pieces,
                                num_splits)
        o, l = O.combine(op, lp)
        np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l, ref_l, rtol=1e-13, atol=1e-13)


def test_split_piece_is_the_attention_over_its_range():
    """One piece's partial is the plain softmax attention over its own keys:
    brute force over the tokens of pages [1, 3) of a row."""
    inp = tiny_inputs(B=1, s_q=1, seqlens=[70], h=2, d_hc=4, d_c=8, d_r=2, page=16, seed=21)
    n = {k: v.numpy() for k, v in inp.items()}
    qa = O.absorb(n["q_c"], n["w_uk"])
    op, lp = O.decode_split(qa, n["q_r"], n["kv_cache"], n["block_table"], n["seqlens"], 0.5, [[(1, 1, 3)]], 3)
    rows = O.gather_rows(n["kv_cache"], n["block_table"][0], 70)
    for h in range(2):
        s = [0.5 * (sum(qa[0, 0, h, c] * rows[t, c] for c in range(8)) +
                    sum(n["q_r"][0, 0, h, d] * rows[t, 8 + d] for d in range(2))) for t in range(16, 48)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        ref = [sum(w[k] * rows[16 + k, c] for k in range(32)) / sum(w) for c in range(8)]
        np.testing.assert_allclose(op[0, 0, h, 1], ref, rtol=1e-12, atol=1e-14)
        assert lp[0, 0, h, 1] == pytest.approx(m + math.log(sum(w)), abs=1e-12)
        assert np.isneginf(lp[0, 0, h, [0, 2]]).all() and not op[0, 0, h, [0, 2]].any()


def test_combine_closed_forms():
    g = np.random.default_rng(8)
    o = g.standard_normal((5, 3, 16))
    # one split: identity
    oc, lc = O.combine(o[:, :1], np.array([[0.7]] * 5))
    np.testing.assert_array_equal(oc, o[:, 0])
    np.testing.assert_allclose(lc, 0.7)
    # equal lse over 3 splits: average, lse + ln 3
    oc, lc = O.combine(o, np.full((5, 3), -1.5))
    np.testing.assert_allclose(oc, o.mean(1), rtol=1e-14)
    np.testing.assert_allclose(lc, -1.5 + math.log(3), rtol=1e-14)
    # an empty split is ignored; all-empty gives zero / -inf
    lp = np.array([[0.2, -np.inf, 0.2]] * 5)
    oc, lc = O.combine(o, lp)
    np.testing.assert_allclose(oc, (o[:, 0] + o[:, 2]) / 2, rtol=1e-14)
    oc, lc = O.combine(o, np.full((5, 3), -np.inf))
    assert (oc == 0).all() and np.isneginf(lc).all()


def test_causal_chunk_reduces_to_single_queries():
    inp = tiny_inputs(B=2, s_q=4, seqlens=[40, 9], h=2, d_hc=4, d_c=8, d_r=2, page=8, seed=21)
    n = {k: v.numpy() for k, v in inp.items()}
    qa = O.absorb(n["q_c"], n["w_uk"])
    o, l = O.decode_absorbed(qa, n["q_r"], n["kv_cache"], n["block_table"], n["seqlens"], 0.5)
    for b in range(2):
        for i in range(4):
            Lv = int(n["seqlens"][b]) - 4 + i + 1
            o1, l1 = O.decode_absorbed(qa[b:b + 1, i:i + 1], n["q_r"][b:b + 1, i:i + 1], n["kv_cache"],
                                       n["block_table"][b:b + 1], [Lv], 0.5)
            assert np.array_equal(o1[0, 0], o[b, i]) and np.array_equal(l1[0, 0], l[b, i])


def test_decode_rows_matches_full():
    inp = tiny_inputs(B=2, s_q=3, seqlens=[100, 33], h=4, d_hc=4, d_c=16, d_r=4, page=8, seed=2)
    n = {k: v.numpy() for k, v in inp.items()}
    qa = O.absorb(n["q_c"], n["w_uk"])
    o, l = O.decode_absorbed(qa, n["q_r"], n["kv_cache"], n["block_table"], n["seqlens"], 0.4)
    picks = [(0, 0, 1), (1, 2, 3), (0, 2, 0)]
    ro, rl = O.decode_rows(qa, n["q_r"], n["kv_cache"], n["block_table"], n["seqlens"], 0.4, picks)
    for k, (b, i, h) in enumerate(picks):
        # one-row and many-row BLAS products round differently in the last ulp
        np.testing.assert_allclose(ro[k], o[b, i, h], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(rl[k], l[b, i, h], rtol=1e-14)


def test_gather_of_bf16_bits_decodes_exactly():
    g = torch.Generator().manual_seed(3)
    kv = torch.randn((5, 64, 576), generator=g).to(torch.bfloat16)
    bt = np.array([3, 0, 4], dtype=np.int32)
    rows_bits = O.gather_rows(O.bf16_bits(kv), bt, 150)
    rows_f64 = O.gather_rows(O.as_f64(kv), bt, 150)
    assert rows_bits.dtype == np.float64 and np.array_equal(rows_bits, rows_f64)
    ref = kv.to(torch.float64)[[3, 0, 4]].reshape(-1, 576)[:150].numpy()
    assert np.array_equal(rows_bits, ref)


# --------------------------------------------------------------------------
# RoPE and the cache append (teardown page, sections 3 and 4; the frequency,
# pair-layout and position readings are stated in the oracle)
# --------------------------------------------------------------------------

def _rope_by_complex(x, p, base=10000.0):
    """Textbook form of the rotation: each pair (x[2j], x[2j+1]) as a complex
    number multiplied by e^(i p base^(-j/(d/2)))."""
    d = len(x)
    out = []
    for j in range(d // 2):
        z = complex(float(x[2 * j]), float(x[2 * j + 1])) * cmath.exp(1j * p * base ** (-j / (d // 2)))
        out += [z.real, z.imag]
    return np.array(out)


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(1).normal(size=(5, 64))
    assert np.array_equal(O.rope_rotate(x, 0), x)


@pytest.mark.parametrize("p", [1, 7, 1000, 65535])
def test_rope_is_complex_multiplication(p):
    x = np.random.default_rng(p).normal(size=64)
    # the angle p*theta carries an fp64 rounding of ~1e-16 * p radians
    np.testing.assert_allclose(O.rope_rotate(x, p), _rope_by_complex(x, p), rtol=0, atol=1e-14 * max(p, 100))


def test_rope_exact_one_radian_angles():
    # pair 0 turns by p; pair 16 by p/100; pair 31 by p * 10000^(-31/32)
    for j, p in [(0, 1), (16, 100), (31, 10000.0 ** (31 / 32))]:
        e = np.zeros(64)
        e[2 * j] = 1.0
        y = O.rope_rotate(e, p)
        assert y[2 * j] == pytest.approx(math.cos(1.0), abs=1e-12)
        assert y[2 * j + 1] == pytest.approx(math.sin(1.0), abs=1e-12)
        assert np.count_nonzero(np.abs(y) > 1e-15) == 2


@pytest.mark.parametrize("p", [3, 4097, 65535])
def test_rope_is_a_proper_rotation(p):
    M = np.stack([O.rope_rotate(e, p) for e in np.eye(64)], axis=1)
    np.testing.assert_allclose(M.T @ M, np.eye(64), atol=1e-12)
    assert np.linalg.det(M) == pytest.approx(1.0, abs=1e-9)


def test_rope_composes_and_scores_depend_on_offset_only():
    rng = np.random.default_rng(5)
    q, k = rng.normal(size=64), rng.normal(size=64)
    for m, n in [(0, 0), (5, 3), (1000, 17), (40000, 39999), (12, 300)]:
        np.testing.assert_allclose(O.rope_rotate(O.rope_rotate(q, n), m), O.rope_rotate(q, m + n), atol=1e-9)
        lhs = O.rope_rotate(q, m) @ O.rope_rotate(k, n)
        assert lhs == pytest.approx(O.rope_rotate(q, m - n) @ k, abs=1e-9)


def test_chunk_positions_follow_causal_rule():
    L, s_q = [5, 64, 300], 4
    pos = O.chunk_positions(L, s_q)
    for b, Lb in enumerate(L):
        for i in range(s_q):
            # a new token sees itself as its last key
            assert pos[b, i] + 1 == O.visible_len(Lb, s_q, i)


def _tiny_append_case(seed=3, page=4, P=9, B=3, s_q=3, d_c=5, d_r=4):
    rng = np.random.default_rng(seed)
    cache = rng.normal(size=(P, page, d_c + d_r))
    seqlens = np.array([2, 7, 11])                    # sequence 0 is shorter than the chunk
    perm = rng.permutation(P)
    bt = np.full((B, 3), -1, np.int64)
    bt[0, :1], bt[1, :2], bt[2, :3] = perm[:1], perm[1:3], perm[3:6]
    c_new = rng.normal(size=(B, s_q, d_c))
    kr_new = rng.normal(size=(B, s_q, d_r))
    return cache, bt, seqlens, c_new, kr_new, page, d_c


def test_append_matches_token_loop():
    cache, bt, L, c_new, kr_new, page, d_c = _tiny_append_case()
    out, written = O.append_latent(cache, bt, L, c_new, kr_new)
    expect = cache.copy()
    n_written = 0
    for b in range(3):
        for i in range(3):
            p = int(L[b]) - 3 + i
            if p < 0:
                continue
            row = expect[bt[b][p // page], p % page]
            row[:d_c] = c_new[b, i]
            row[d_c:] = _rope_by_complex(kr_new[b, i], p)
            n_written += 1
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-12)
    assert len(written) == n_written == 8            # one token of sequence 0 has no slot


def test_append_then_gather_returns_the_chunk():
    cache, bt, L, c_new, kr_new, page, d_c = _tiny_append_case(seed=9)
    out, _ = O.append_latent(cache, bt, L, c_new, kr_new)
    for b in (1, 2):
        before = O.gather_rows(cache, bt[b], int(L[b]))
        after = O.gather_rows(out, bt[b], int(L[b]))
        np.testing.assert_array_equal(after[:-3], before[:-3])
        np.testing.assert_array_equal(after[-3:, :d_c], c_new[b])
        for i in range(3):
            np.testing.assert_allclose(after[-3 + i, d_c:], _rope_by_complex(kr_new[b, i], int(L[b]) - 3 + i),
                                       atol=1e-12)


# --------------------------------------------------------------------------
# decompressed branch and the dispatch threshold (teardown page, sections 3-4)
# --------------------------------------------------------------------------

def test_dispatch_threshold_matches_teardown_page():
    g = _golden("teardown_dispatch.json")
    assert O.PREFILL_ABSORPTION_THRESHOLD == g["kPrefillThresh"] == g["prefill_absorption_threshold"]
    assert O.uses_absorption(1) and O.uses_absorption(g["kPrefillThresh"])
    assert not O.uses_absorption(g["kPrefillThresh"] + 1)
    assert O.uses_absorption(512, threshold=512) and not O.uses_absorption(129, threshold=128)


def test_decompress_kv_brute_force():
    rng = np.random.default_rng(8)
    Hn, d_hc, d_c, d_r, page = 2, 3, 5, 2, 4
    kv = rng.normal(size=(6, page, d_c + d_r))
    bt = np.array([[4, 1, 0], [2, 5, 3]])
    L = [9, 5]
    w_uk, w_uv = rng.normal(size=(Hn, d_hc, d_c)), rng.normal(size=(Hn, d_hc, d_c))
    K, V = O.decompress_kv(kv, bt, L, w_uk, w_uv, max_len=10)
    for b in range(2):
        for t in range(10):
            row = kv[bt[b][t // page], t % page] if t < L[b] else None
            for h in range(Hn):
                for d in range(d_hc):
                    kk = sum(float(row[c]) * float(w_uk[h, d, c]) for c in range(d_c)) if row is not None else 0.0
                    vv = sum(float(row[c]) * float(w_uv[h, d, c]) for c in range(d_c)) if row is not None else 0.0
                    assert K[b, h, t, d] == pytest.approx(kk, abs=1e-12)
                    assert V[b, h, t, d] == pytest.approx(vv, abs=1e-12)
    R = O.rope_keys(kv, bt, L, 10, d_c=d_c)
    assert np.array_equal(R[1, :5], np.stack([kv[bt[1][t // page], t % page, d_c:] for t in range(5)]))
    assert (R[1, 5:] == 0).all()


def test_attend_mha_brute_force():
    rng = np.random.default_rng(9)
    B, s_q, Hn, d, d_r, n_max = 2, 3, 2, 4, 2, 7
    L = [7, 2]                                   # the second sequence is shorter than the chunk
    q_c, q_r = rng.normal(size=(B, s_q, Hn, d)), rng.normal(size=(B, s_q, Hn, d_r))
    K, V = rng.normal(size=(B, Hn, n_max, d)), rng.normal(size=(B, Hn, n_max, d))
    R = rng.normal(size=(B, n_max, d_r))
    out, lse = O.attend_mha(q_c, q_r, K, V, R, L, 0.3)
    for b in range(B):
        for i in range(s_q):
            n = L[b] - s_q + i + 1
            for h in range(Hn):
                if n <= 0:
                    assert lse[b, i, h] == -math.inf and (out[b, i, h] == 0).all()
                    continue
                s = [0.3 * (sum(q_c[b, i, h, k] * K[b, h, t, k] for k in range(d))
                            + sum(q_r[b, i, h, k] * R[b, t, k] for k in range(d_r))) for t in range(n)]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = sum(w)
                for k in range(d):
                    assert out[b, i, h, k] == pytest.approx(sum(w[t] * V[b, h, t, k] for t in range(n)) / tot,
                                                            abs=1e-12)
                assert lse[b, i, h] == pytest.approx(m + math.log(tot), abs=1e-12)


def test_decompressed_branch_equals_naive_and_absorbed_paths():
    """Both stages together reproduce path A (decode_naive), itself pinned to
    the absorbed path, at real dimensions and a causal chunk."""
    inp = tiny_inputs(B=2, s_q=4, seqlens=[70, 9], h=4, d_hc=128, d_c=512, d_r=64, page=64, seed=3)
    f = {k: O.as_f64(inp[k]) for k in ("q_c", "q_r", "w_uk", "w_uv")}
    kvb = O.as_f64(inp["kv_cache"])
    bt, sl = inp["block_table"].numpy(), inp["seqlens"].numpy()
    K, V = O.decompress_kv(kvb, bt, sl, f["w_uk"], f["w_uv"], max_len=70)
    R = O.rope_keys(kvb, bt, sl, 70)
    out, lse = O.attend_mha(f["q_c"], f["q_r"], K, V, R, sl, O.default_scale())
    ref_out, ref_lse = O.decode_naive(f["q_c"], f["q_r"], kvb, bt, sl, f["w_uk"], f["w_uv"], O.default_scale())
    np.testing.assert_allclose(out, ref_out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)
    qa = O.absorb(f["q_c"], f["w_uk"])
    o_lat, lse_b = O.decode_absorbed(qa, f["q_r"], kvb, bt, sl, O.default_scale())
    np.testing.assert_allclose(out, O.up_proj(o_lat, f["w_uv"]), rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse, lse_b, rtol=0, atol=1e-11)


# --------------------------------------------------------------------------
# 8-bit latent cache (FP8 E4M3 codes, one power-of-two scale per token)
# --------------------------------------------------------------------------
# The E4M3 value table and round-to-nearest-even are pinned to torch's own
# float8_e4m3fn type (an independent implementation of the OCP format), the
# scale rule to a brute-force search, the page layout to byte offsets worked
# out by hand, and the 8-bit decode to the definition "attention over the
# stored values".

def _torch_e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def test_e4m3_values_match_torch_float8_and_format_landmarks():
    got = O.e4m3_value(np.arange(256))
    ref = _torch_e4m3_table()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin]))
    # landmarks of the format: largest finite, smallest normal and subnormal, one
    assert got[0x7E] == 448.0 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x38] == 1.0
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    assert np.all(np.diff(got[:0x7F]) > 0)          # codes 0x00..0x7E increase strictly


def _all_bf16_within(limit):
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        v = (bits << 16).view(np.float32).astype(np.float64)
    return v[np.isfinite(v) & (np.abs(v) <= limit)]


def test_e4m3_encode_matches_torch_cast_on_every_bf16_value_and_midpoint():
    """Every value the quantizer can meet (a bf16 value times a power of two,
    at most 448 in magnitude) has at most 8 significant bits; all of them, and
    the exact midpoints between neighbouring E4M3 values (the ties), round as
    torch's cast to float8_e4m3fn does, sign of zero included."""
    table = _torch_e4m3_table()
    pos = np.unique(table[(~np.isnan(table)) & (table >= 0)])
    mids = (pos[:-1] + pos[1:]) / 2
    v = np.concatenate([_all_bf16_within(448.0), mids, -mids, [0.0, -0.0]])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(v), ref)


def test_e4m3_encode_is_nearest_with_ties_to_even_by_brute_force():
    table = _torch_e4m3_table()
    codes = [c for c in range(256) if not math.isnan(table[c])]
    rng = np.random.default_rng(8)
    vals = list(rng.uniform(-448, 448, 300)) + list(rng.uniform(-2 ** -5, 2 ** -5, 300)) + [2.5 * 2 ** -9, 9.5 * 2 ** -9]
    enc = O.e4m3_encode(np.array(vals))
    for v, c in zip(vals, enc):
        best = min(abs(v - table[k]) for k in codes)
        assert abs(v - table[c]) == best
        ties = [k for k in codes if abs(v - table[k]) == best and (k & 0x80) == (0x80 if v < 0 else 0)]
        if len(ties) > 1:
            assert c % 2 == 0, f"tie at {v} not rounded to the even mantissa"
    with pytest.raises(ValueError):
        O.e4m3_encode(np.array([448.5]))


def test_fp8_scale_exponent_is_the_smallest_that_fits_by_search():
    rng = np.random.default_rng(9)
    amax = np.concatenate([np.exp(rng.uniform(-80, 80, 200)), [448.0, 449.0, 448.0 * 2 ** -20, 224.0, 1.0,
                                                               np.nextafter(448.0, 0), 2.0 ** -140, 3e38]])
    got = O.fp8_scale_exponent(amax)
    for a, k in zip(amax, got):
        want = next(j for j in range(-300, 300) if a <= 448.0 * 2.0 ** j)
        assert k == min(max(want, -126), 127), (a, k, want)
    assert O.fp8_scale_exponent(np.array([0.0]))[0] == -126


def test_quantize_latent_fp8_error_bound_and_no_saturation():
    rng = np.random.default_rng(10)
    c = torch.from_numpy(rng.standard_normal((64, 512)) * np.exp(rng.uniform(-20, 20, (64, 1)))).to(torch.bfloat16)
    x = O.as_f64(c)
    codes, k = O.quantize_latent_fp8(x)
    back = O.dequantize_latent_fp8(codes, k)
    s = np.ldexp(1.0, k)[:, None]
    normal = np.abs(x) >= 2.0 ** -6 * s
    # half a spacing of E4M3: 2^-4 relative in the normal range, 2^-10 * s below it
    assert np.all(np.abs(back - x)[normal] <= 2.0 ** -4 * np.abs(x)[normal])
    assert np.all(np.abs(back - x)[~normal] <= (2.0 ** -10 * s + 0 * x)[~normal])
    amax_codes = np.abs(O.e4m3_value(codes)).max(axis=1)
    assert np.all(amax_codes <= 448.0)
    assert np.all(np.abs(x).max(axis=1) / s[:, 0] > 224.0)   # a smaller scale would overflow
    assert np.array_equal(np.signbit(O.e4m3_value(codes)), np.signbit(x))


def test_fp8_page_layout_by_hand():
    P, page, d_c, d_r = 2, 64, 512, 64
    kv = torch.zeros((P, page, d_c + d_r), dtype=torch.bfloat16)
    kv[1, 5, 7] = 3.0
    kv[1, 5, 100] = -0.5
    kv[1, 5, d_c + 3] = 1.25
    pages = O.pack_fp8_cache(O.bf16_bits(kv))
    assert pages.shape == (P, 64 * 512 + 64 * 128 + 64 * 4) == (P, 41216)
    # token (page 1, row 5): max |c| = 3 -> smallest 2^k with 3 <= 448 * 2^k is 2^-7
    assert pages[1, 5 * 512 + 7] == 0x7C                  # 3 / 2^-7 = 384 = 1.5 * 2^8: 0.1111.100
    assert pages[1, 5 * 512 + 100] == 0xE8               # -0.5 / 2^-7 = -64 = -2^6: 1.1101.000
    assert pages[1, 32768 + 5 * 128 + 6] == 0xA0 and pages[1, 32768 + 5 * 128 + 7] == 0x3F   # bf16 1.25, LE
    assert pages[1, 40960 + 5 * 4: 40960 + 5 * 4 + 4].view("<f4")[0] == 2.0 ** -7
    assert pages[0, 40960: 40960 + 4].view("<f4")[0] == 2.0 ** -126   # zero row
    assert not pages[0, :32768].any()


def test_fp8_cache_decode_is_attention_over_stored_values():
    inp = tiny_inputs(B=3, s_q=2, seqlens=[70, 9, 130], h=4, d_hc=128, d_c=512, d_r=64, page=64, seed=21)
    kv16 = inp["kv_cache"].to(torch.bfloat16)
    pages = O.pack_fp8_cache(O.bf16_bits(kv16))
    cache8 = O.PagedFp8Cache(pages)
    stored = O.dequantize_fp8_pages(pages)
    bt, sl = inp["block_table"].numpy(), inp["seqlens"].numpy()
    qa = O.absorb(O.as_f64(inp["q_c"]), O.as_f64(inp["w_uk"]))
    qr = O.as_f64(inp["q_r"])
    o8, l8 = O.decode_absorbed(qa, qr, cache8, bt, sl, O.default_scale())
    o_ref, l_ref = O.decode_absorbed(qa, qr, stored, bt, sl, O.default_scale())
    assert np.array_equal(o8, o_ref) and np.array_equal(l8, l_ref)
    # k_R is stored exactly; c_KV within half an E4M3 spacing of the bf16 cache
    kvb = O.as_f64(kv16)
    assert np.array_equal(stored[..., 512:], kvb[..., 512:])
    assert np.all(np.abs(stored[..., :512] - kvb[..., :512]) <= 2.0 ** -4 * np.abs(kvb[..., :512]) + 2.0 ** -12)
    # and the attention result stays close to the bf16 cache's
    o16, l16 = O.decode_absorbed(qa, qr, kvb, bt, sl, O.default_scale())
    assert np.abs(o8 - o16).max() < 0.05 * np.abs(o16).max()


# --------------------------------------------------------------------------
# 4-bit latent cache (OCP MXFP4: E2M1 codes, one E8M0 scale per 32 dims)
# --------------------------------------------------------------------------
# torch has an E2M1 storage type but no conversion for it, so the value table
# is pinned to the magnitudes the OCP microscaling format lists for E2M1,
# rounding to a brute-force nearest search with the ties worked out by hand,
# the block scale rule to a search, the page layout to byte offsets worked
# out by hand, and the 4-bit decode to the definition "attention over the
# stored values".

OCP_E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # codes 0..7; bit 3 is the sign


def test_e2m1_values_match_the_ocp_table():
    v = O.e2m1_value(np.arange(16))
    assert v[:8].tolist() == OCP_E2M1_MAGNITUDES
    assert (-v[8:]).tolist() == OCP_E2M1_MAGNITUDES
    assert np.signbit(v[8])                       # code 0x8 is -0
    assert O.E2M1_MAX == 6.0


def test_e2m1_encode_is_nearest_with_ties_to_even_by_brute_force():
    grid = np.arange(-6 * 64, 6 * 64 + 1) / 64.0      # every multiple of 1/64 in [-6, 6]
    codes = O.e2m1_encode(grid)
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}   # to the even code
    for x, c in zip(grid, codes):
        a = abs(x)
        if a in ties:
            want = ties[a]
        else:
            dist = [abs(a - m) for m in OCP_E2M1_MAGNITUDES]
            want = dist.index(min(dist))
        assert (int(c) & 7) == want, (x, c)
        assert (int(c) >> 3) == (1 if np.signbit(x) else 0)
    assert O.e2m1_encode([-0.1])[0] == 0x8          # a negative value that rounds to zero keeps its sign
    with pytest.raises(ValueError):
        O.e2m1_encode([6.01])


def test_mx_scale_exponent_is_the_smallest_that_fits_by_search():
    rng = np.random.default_rng(5)
    amax = np.concatenate([
        np.exp2(rng.uniform(-120, 120, 400)),
        6.0 * np.exp2(np.arange(-20, 21)),                       # exactly 6 * 2^k
        np.nextafter(6.0 * np.exp2(np.arange(-20, 21)), np.inf),  # just above
        [0.0, 2.0 ** -140, 3.0e38]])
    k = O.mx_scale_exponent(amax)
    for a, kk in zip(amax, k):
        if a == 0:
            assert kk == -126
            continue
        want = next(j for j in range(-140, 140) if a <= 6.0 * 2.0 ** j)
        assert kk == min(max(want, -126), 127), (a, kk, want)


def test_quantize_latent_mxfp4_error_bound_and_no_saturation():
    rng = np.random.default_rng(6)
    c = rng.standard_normal((40, 512)) * np.exp2(rng.integers(-20, 20, (40, 1)))
    c[3, 64:96] = 0.0                                   # one zero block
    codes, k = O.quantize_latent_mxfp4(c)
    assert codes.shape == (40, 512) and k.shape == (40, 16)
    q = O.dequantize_latent_mxfp4(codes, k)
    blocks = np.abs(c).reshape(40, 16, 32)
    scaled_max = blocks.max(axis=-1) / np.exp2(k)
    nz = blocks.max(axis=-1) > 0
    assert np.all(scaled_max[nz] <= 6.0) and np.all(scaled_max[nz] > 3.0)   # smallest k: no clip, no waste
    assert k[3, 2] == -126 and not np.any(q[3, 64:96])
    # within half an E2M1 spacing (0.5 below 2, 1 below 4, 2 above) of the value
    a = np.abs(c) / np.repeat(np.exp2(k), 32, axis=1)
    half = np.where(a < 2, 0.25, np.where(a < 4, 0.5, 1.0)) * np.repeat(np.exp2(k), 32, axis=1)
    assert np.all(np.abs(q - c) <= half)
    # values on the grid come back exactly
    exact = np.repeat(np.exp2(k), 32, axis=1) * O.e2m1_value(codes)
    assert np.array_equal(O.dequantize_latent_mxfp4(*O.quantize_latent_mxfp4(exact)), exact)


def test_mxfp4_page_layout_by_hand():
    P, page, d_c, d_r = 2, 64, 512, 64
    kv = torch.zeros((P, page, d_c + d_r), dtype=torch.bfloat16)
    kv[1, 5, 0] = 1.0
    kv[1, 5, 1] = -6.0        # block 0: max 6 -> k = 0
    kv[1, 5, 40] = 0.75       # block 1: max 0.75 = 6 * 2^-3 -> k = -3
    kv[1, 5, 41] = -0.1       # bf16 -0.10009765625 * 8 = -0.80078 -> -1.0
    kv[1, 5, d_c + 3] = 1.25
    pages = O.pack_mxfp4_cache(O.bf16_bits(kv))
    assert pages.shape == (P, 64 * 256 + 64 * 128 + 64 * 16) == (P, 25600)
    row = 5 * 256
    assert pages[1, row + 0] == 0xF2                     # dim 0: 1.0 = 0.01.0 (low), dim 1: -6 = 1.11.1 (high)
    assert pages[1, row + 20] == 0xA7                    # dim 40: 6 = 0.11.1, dim 41: -1.0 = 1.01.0
    assert not pages[1, row + 1: row + 20].any() and not pages[1, row + 21: row + 256].any()
    assert pages[1, 16384 + 5 * 128 + 6] == 0xA0 and pages[1, 16384 + 5 * 128 + 7] == 0x3F   # bf16 1.25, LE
    sc = pages[1, 24576 + 5 * 16: 24576 + 6 * 16]
    assert sc[0] == 127 and sc[1] == 124 and np.all(sc[2:] == 1)          # E8M0 k + 127; zero blocks 2^-126
    assert np.all(pages[0, 24576:] == 1) and not pages[0, :24576].any()   # zero page


def test_mxfp4_cache_decode_is_attention_over_stored_values():
    inp = tiny_inputs(B=3, s_q=2, seqlens=[70, 9, 130], h=4, d_hc=128, d_c=512, d_r=64, page=64, seed=22)
    kv16 = inp["kv_cache"].to(torch.bfloat16)
    pages = O.pack_mxfp4_cache(O.bf16_bits(kv16))
    cache4 = O.PagedMxfp4Cache(pages)
    stored = O.dequantize_mxfp4_pages(pages)
    assert np.array_equal(np.asarray(cache4), stored)
    bt, sl = inp["block_table"].numpy(), inp["seqlens"].numpy()
    qa = O.absorb(O.as_f64(inp["q_c"]), O.as_f64(inp["w_uk"]))
    qr = O.as_f64(inp["q_r"])
    o4, l4 = O.decode_absorbed(qa, qr, cache4, bt, sl, O.default_scale())
    o_ref, l_ref = O.decode_absorbed(qa, qr, stored, bt, sl, O.default_scale())
    assert np.array_equal(o4, o_ref) and np.array_equal(l4, l_ref)
    # the split oracle reads the 4-bit cache the same way
    rows = [-(-max(int(L) - 2 + i + 1, 0) // 64) for L in sl for i in range(2)]
    pieces = _random_pieces(rows, 3, np.random.default_rng(4))
    os_, ls_ = O.decode_split(qa, qr, cache4, bt, sl, O.default_scale(), pieces, 3)
    oc, lc = O.combine(os_, ls_)
    assert np.allclose(oc, o_ref, rtol=0, atol=1e-12) and np.allclose(lc, l_ref, rtol=0, atol=1e-12)
    # k_R is stored exactly; c_KV within half the coarsest E2M1 spacing of its block
    kvb = O.as_f64(kv16)
    assert np.array_equal(stored[..., 512:], kvb[..., 512:])
    blk_max = np.abs(kvb[..., :512]).reshape(kvb.shape[0], 64, 16, 32).max(axis=-1)
    # (half the top spacing is 2^k, and 2^k < max|block| / 3 by the scale rule)
    assert np.all(np.abs(stored[..., :512] - kvb[..., :512]) < np.repeat(blk_max, 32, axis=-1) / 3.0 + 1e-300)
