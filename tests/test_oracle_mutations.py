"""Planted mistakes in the oracle (CPU only) must each be caught by a pin.

Every mutant replaces one oracle function with a plausible wrong version
(a dropped term, an off-by-one, a wrong weight) for the duration of one test,
then re-runs the pins that should notice and expects at least one to fail.
"""
import numpy as np
import pytest

import oracle as O
import oracle.mla_oracle as M
import tests.test_oracle as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(M, name, fn)
    monkeypatch.setattr(O, name, fn)


def _expect_fail(*checks):
    failed = 0
    for chk in checks:
        try:
            chk()
        except (AssertionError, ValueError, IndexError):
            failed += 1
    assert failed > 0, "no pin noticed the planted mistake"


def test_dropped_rope_term_is_caught(monkeypatch):
    _patch(monkeypatch, "scores_absorbed", lambda qa, qr, C, R, scale: (qa @ C.T) * scale)
    _expect_fail(pins.test_naive_equals_absorbed_real_dims,
                 lambda: pins.test_brute_force_tiny([7, 10], 3))


def test_wrong_scale_is_caught(monkeypatch):
    real = M.scores_absorbed
    _patch(monkeypatch, "scores_absorbed", lambda qa, qr, C, R, scale: real(qa, qr, C, R, scale) * 1.01)
    _expect_fail(pins.test_closed_form_one_hot_selects_row,
                 lambda: pins.test_brute_force_tiny([4, 1, 9], 1))


def test_causal_off_by_one_is_caught(monkeypatch):
    _patch(monkeypatch, "visible_len", lambda L, s_q, i: int(L) - int(s_q) + int(i))
    _expect_fail(lambda: pins.test_brute_force_tiny([7, 10], 3))


def test_split_losing_last_page_is_caught(monkeypatch):
    real = M.decode_split

    def lossy(q_abs, q_r, kv, bt, sl, scale, pieces, num_splits):
        # every piece that ends a row stops one page short
        short = [[(s_, a, e - 1 if e - 1 > a and e == max(x[2] for x in row) else e) for s_, a, e in row]
                 for row in pieces]
        return real(q_abs, q_r, kv, bt, sl, scale, short, num_splits)
    _patch(monkeypatch, "decode_split", lossy)
    _expect_fail(lambda: pins.test_split_invariance(2))


def test_gather_ignoring_block_table_is_caught(monkeypatch):
    def naive_gather(kv, bt_row, n):
        kv = np.asarray(kv)
        return kv.reshape(-1, kv.shape[2])[:n]
    _patch(monkeypatch, "gather_rows", naive_gather)
    _expect_fail(pins.test_gather_matches_token_loop_and_rejects_bad_ids,
                 pins.test_page_permutation_invariance,
                 lambda: pins.test_brute_force_tiny([7, 10], 3))


def test_combine_without_lse_weights_is_caught(monkeypatch):
    def plain_mean(o_part, lse_part):
        o_part = np.asarray(o_part, np.float64)
        return o_part.mean(axis=-2), np.asarray(lse_part).max(axis=-1)
    _patch(monkeypatch, "combine", plain_mean)
    _expect_fail(pins.test_combine_closed_forms, lambda: pins.test_split_invariance(7))


def test_transposed_up_proj_is_caught(monkeypatch):
    def wrong(o_lat, w_uv):
        w = np.asarray(w_uv, np.float64)
        # contracts the right index but reads heads in reverse order
        return np.einsum("...hc,hdc->...hd", np.asarray(o_lat, np.float64), w[::-1])
    _patch(monkeypatch, "up_proj", wrong)
    _expect_fail(pins.test_up_proj_brute_force, lambda: pins.test_brute_force_tiny([4, 1, 9], 1))


def test_softmax_without_max_subtraction_bias_is_caught(monkeypatch):
    def biased(s):
        m = s.max(axis=-1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=-1, keepdims=True) + 1e-3
        return e / l, m[..., 0], l[..., 0]
    _patch(monkeypatch, "softmax_rows", biased)
    _expect_fail(pins.test_softmax_rows_sum_to_one, pins.test_closed_form_zero_query_is_mean)


def test_rope_half_split_pairing_is_caught(monkeypatch):
    def half_split(x, positions, base=M.ROPE_BASE):
        x = np.asarray(x, np.float64)
        d = x.shape[-1]
        a = M.rope_angles(np.broadcast_to(np.asarray(positions), x.shape[:-1]), d, base)
        c, s = np.cos(a), np.sin(a)
        lo, hi = x[..., : d // 2], x[..., d // 2:]
        return np.concatenate([lo * c - hi * s, lo * s + hi * c], axis=-1)
    _patch(monkeypatch, "rope_rotate", half_split)
    _expect_fail(lambda: pins.test_rope_is_complex_multiplication(7), pins.test_rope_exact_one_radian_angles)


def test_rope_frequency_exponent_is_caught(monkeypatch):
    real_angles = M.rope_angles

    def wrong(positions, d_r=64, base=M.ROPE_BASE):   # base^(-j/d) instead of base^(-2j/d)
        return real_angles(positions, 2 * d_r, base)[..., : d_r // 2]
    _patch(monkeypatch, "rope_angles", wrong)
    _expect_fail(pins.test_rope_exact_one_radian_angles, lambda: pins.test_rope_is_complex_multiplication(7))


def test_rope_reflection_is_caught(monkeypatch):
    def reflect(x, positions, base=M.ROPE_BASE):
        x = np.asarray(x, np.float64)
        a = M.rope_angles(np.broadcast_to(np.asarray(positions), x.shape[:-1]), x.shape[-1], base)
        c, s = np.cos(a), np.sin(a)
        y = np.empty_like(x)
        y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
        y[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c      # wrong sign: not a rotation
        return y
    _patch(monkeypatch, "rope_rotate", reflect)
    _expect_fail(lambda: pins.test_rope_is_a_proper_rotation(3),
                 pins.test_rope_composes_and_scores_depend_on_offset_only)


def test_append_off_by_one_position_is_caught(monkeypatch):
    monkeypatch.setattr(M, "chunk_positions",
                        lambda L, s_q: np.asarray(L, np.int64)[:, None] - s_q + 1 + np.arange(s_q)[None, :])
    _expect_fail(pins.test_append_matches_token_loop, pins.test_append_then_gather_returns_the_chunk)


def test_append_without_rotation_is_caught(monkeypatch):
    monkeypatch.setattr(M, "rope_rotate", lambda x, positions, base=M.ROPE_BASE: np.asarray(x, np.float64))
    _expect_fail(pins.test_append_matches_token_loop, pins.test_append_then_gather_returns_the_chunk)


def test_decompress_swapping_weights_is_caught(monkeypatch):
    real = M.decompress_kv
    _patch(monkeypatch, "decompress_kv",
           lambda kv, bt, L, w_uk, w_uv, max_len: real(kv, bt, L, w_uv, w_uk, max_len))
    _expect_fail(pins.test_decompress_kv_brute_force, pins.test_decompressed_branch_equals_naive_and_absorbed_paths)


def test_mha_without_rope_term_is_caught(monkeypatch):
    real = M.attend_mha
    _patch(monkeypatch, "attend_mha",
           lambda q_c, q_r, K, V, R, L, scale: real(q_c, np.zeros_like(np.asarray(q_r, np.float64)), K, V, R, L, scale))
    _expect_fail(pins.test_attend_mha_brute_force, pins.test_decompressed_branch_equals_naive_and_absorbed_paths)


def test_dispatch_strict_threshold_is_caught(monkeypatch):
    _patch(monkeypatch, "uses_absorption", lambda s_q, threshold=M.PREFILL_ABSORPTION_THRESHOLD: int(s_q) < threshold)
    _expect_fail(pins.test_dispatch_threshold_matches_teardown_page)


def test_e4m3_round_half_away_from_zero_is_caught(monkeypatch):
    real = M.e4m3_encode

    def half_up(v):
        v = np.asarray(v, np.float64)
        a = np.abs(v)
        _, x = np.frexp(a)
        E = np.maximum(x - 1, -6)
        ulp = np.ldexp(1.0, E - 3)
        return real(np.copysign(np.floor(a / ulp + 0.5) * ulp, v))   # ties away from zero
    _patch(monkeypatch, "e4m3_encode", half_up)
    _expect_fail(pins.test_e4m3_encode_matches_torch_cast_on_every_bf16_value_and_midpoint,
                 pins.test_e4m3_encode_is_nearest_with_ties_to_even_by_brute_force)


def test_e4m3_unsigned_zero_is_caught(monkeypatch):
    real = M.e4m3_encode

    def no_neg_zero(v):
        c = real(v)
        return np.where(c == 0x80, 0, c).astype(np.uint8)
    _patch(monkeypatch, "e4m3_encode", no_neg_zero)
    _expect_fail(pins.test_e4m3_encode_matches_torch_cast_on_every_bf16_value_and_midpoint,
                 pins.test_quantize_latent_fp8_error_bound_and_no_saturation)


def test_e4m3_subnormal_scale_is_caught(monkeypatch):
    real = M.e4m3_value

    def wrong(codes):
        c = np.asarray(codes).astype(np.int64)
        v = real(c)
        return np.where(((c >> 3) & 15) == 0, v / 2, v)   # subnormals m/8 * 2^-7
    _patch(monkeypatch, "e4m3_value", wrong)
    _expect_fail(pins.test_e4m3_values_match_torch_float8_and_format_landmarks)


def test_fp8_scale_off_by_one_is_caught(monkeypatch):
    real = M.fp8_scale_exponent
    _patch(monkeypatch, "fp8_scale_exponent", lambda a: real(a) + 1)
    _expect_fail(pins.test_fp8_scale_exponent_is_the_smallest_that_fits_by_search,
                 pins.test_quantize_latent_fp8_error_bound_and_no_saturation)


def test_fp8_scale_saturating_rule_is_caught(monkeypatch):
    # the MX rule 2^(floor(log2 amax) - 8), which clips amax in (448, 512) * 2^k
    def mx_rule(a):
        a = np.asarray(a, np.float64)
        _, x = np.frexp(a)
        return np.where(a == 0, -126, np.clip(x - 9, -126, 127)).astype(np.int64)
    _patch(monkeypatch, "fp8_scale_exponent", mx_rule)
    _expect_fail(pins.test_fp8_scale_exponent_is_the_smallest_that_fits_by_search)


def test_fp8_page_with_swapped_rope_and_scale_is_caught(monkeypatch):
    real = M.pack_fp8_cache

    def swapped(kv_bits, d_c=512, chunk_pages=256):
        out = real(kv_bits, d_c, chunk_pages)
        page = np.asarray(kv_bits).shape[1]
        o_rope, o_scale = page * d_c, page * d_c + page * 128
        fixed = out.copy()
        fixed[:, o_rope:o_rope + page * 4] = out[:, o_scale:]
        fixed[:, o_rope + page * 4:] = out[:, o_rope:o_scale]
        return fixed
    _patch(monkeypatch, "pack_fp8_cache", swapped)
    _expect_fail(pins.test_fp8_page_layout_by_hand)


def test_e2m1_ties_away_from_zero_is_caught(monkeypatch):
    real = M.e2m1_encode

    def half_up(v):
        v = np.asarray(v, np.float64)
        c = real(v)
        a = np.abs(v)
        tie_down = np.isin(a, [0.25, 1.25, 2.5, 5.0])       # ties that went to the smaller even code
        return np.where(tie_down, c + 1, c).astype(np.uint8)
    _patch(monkeypatch, "e2m1_encode", half_up)
    _expect_fail(pins.test_e2m1_encode_is_nearest_with_ties_to_even_by_brute_force)


def test_e2m1_subnormal_value_is_caught(monkeypatch):
    real = M.e2m1_value

    def wrong(codes):
        c = np.asarray(codes).astype(np.int64)
        v = real(c)
        return np.where((c & 7) == 1, v / 2, v)             # 0.25 instead of 0.5
    _patch(monkeypatch, "e2m1_value", wrong)
    _expect_fail(pins.test_e2m1_values_match_the_ocp_table)


def test_mx_scale_ocp_floor_rule_is_caught(monkeypatch):
    # k = floor(log2 amax) - 2, which clips amax in (6, 8) * 2^k
    def floor_rule(a):
        a = np.asarray(a, np.float64)
        _, x = np.frexp(a)
        return np.where(a == 0, -126, np.clip(x - 3, -126, 127)).astype(np.int64)
    _patch(monkeypatch, "mx_scale_exponent", floor_rule)
    _expect_fail(pins.test_mx_scale_exponent_is_the_smallest_that_fits_by_search,
                 pins.test_quantize_latent_mxfp4_error_bound_and_no_saturation)


def test_mxfp4_nibble_order_is_caught(monkeypatch):
    real = M.pack_mxfp4_cache

    def swapped(kv_bits, d_c=512, chunk_pages=256):
        out = real(kv_bits, d_c, chunk_pages)
        page = np.asarray(kv_bits).shape[1]
        n = page * d_c // 2
        out[:, :n] = (out[:, :n] >> 4) | (out[:, :n] << 4)
        return out
    _patch(monkeypatch, "pack_mxfp4_cache", swapped)
    _expect_fail(pins.test_mxfp4_page_layout_by_hand)


def test_mxfp4_one_scale_per_token_is_caught(monkeypatch):
    def per_token(c):
        c = np.asarray(c, np.float64)
        k1 = M.mx_scale_exponent(np.abs(c).max(axis=-1))
        k = np.repeat(k1[..., None], c.shape[-1] // M.MX_BLOCK, axis=-1)
        return M.e2m1_encode(np.ldexp(c, -k1[..., None])), k
    _patch(monkeypatch, "quantize_latent_mxfp4", per_token)
    _expect_fail(pins.test_mxfp4_page_layout_by_hand,
                 pins.test_quantize_latent_mxfp4_error_bound_and_no_saturation)
