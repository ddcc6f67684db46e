"""fp64 reference for absorbed MLA decode (test infrastructure only).

Notation (MLA operator-teardown page, sections 1, 3, 4):
  H heads, d_hc = 128 content dims per head, d_c = 512 latent dims,
  d_R = 64 decoupled-RoPE dims, page = 64 tokens.
  A cache row holds c_KV (d_c values) followed by k_R (d_R values).
  Path A (naive): K_h = c_KV . W_UK[h]^T, score = q_c . K_h + q_R . k_R.
  Path B (absorbed): q_abs[h] = q_c[h] . W_UK[h], score = q_abs . c_KV + q_R . k_R.
  Both scores are multiplied by 1/sqrt(d_hc + d_R).

Readings taken where the pages are silent (each also listed in the design notes):
  * W_UV has the layout of W_UK, [H, d_hc, d_c]; out[h, d] = sum_c o_lat[h, c] W_UV[h, d, c].
  * q_R and k_R arrive already rotated; no rotation happens here.
  * with s_q new tokens per sequence, query i (0-based) sees cache tokens
    t <= L_b - s_q + i (the chunk's own latents are already in the cache).
  * LSE is the natural log of the sum of exp(scaled score).
  * an empty key range yields o = 0 and LSE = -inf.
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# bf16 decoding and storage arithmetic
# --------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the top 16 bits of an IEEE float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def bf16_bits(x) -> np.ndarray:
    """Zero-copy uint16 view of a CPU torch bf16 tensor (its bit patterns)."""
    if str(getattr(x, "dtype", "")) != "torch.bfloat16":
        raise TypeError(f"bf16_bits takes a bfloat16 tensor, got {getattr(x, 'dtype', type(x))}")
    return x.detach().cpu().contiguous().view(__import__("torch").int16).numpy().view(np.uint16)


def as_f64(x) -> np.ndarray:
    """Exact float64 copy of a torch tensor or numpy array (bf16 via its bits)."""
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        x = x.detach().cpu()
        if x.dtype == torch.bfloat16:
            return bf16_bits_to_f64(x.contiguous().view(torch.int16).numpy().view(np.uint16))
        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def latent_row_elems(d_c: int = 512, d_r: int = 64) -> int:
    """Values stored per token and layer: the latent plus the shared RoPE key."""
    return d_c + d_r


def latent_row_bytes(d_c: int = 512, d_r: int = 64, elem_bytes: int = 2) -> int:
    return latent_row_elems(d_c, d_r) * elem_bytes


def mha_kv_bytes_per_token_layer(h: int = 128, d_head: int = 128, elem_bytes: int = 2) -> int:
    """Uncompressed multi-head K and V for one token and layer."""
    return 2 * h * d_head * elem_bytes


def default_scale(d_hc: int = 128, d_r: int = 64) -> float:
    """Softmax scale 1/sqrt(d_hc + d_R) (teardown page, section 4 script)."""
    return 1.0 / math.sqrt(d_hc + d_r)


# --------------------------------------------------------------------------
# paged gather
# --------------------------------------------------------------------------


def gather_rows(kv_cache: np.ndarray, block_table_row: np.ndarray, n_tokens: int) -> np.ndarray:
    """Logical rows 0..n_tokens-1 of one sequence.

    Token t lives in physical page block_table_row[t // page] at row t % page.
    Only the entries the sequence needs are read; they must be valid page ids.
    A uint16 cache is taken as bf16 bit patterns and decoded exactly after the
    gather (so a large cache never has to exist in float64); a quantized
    cache (PagedFp8Cache, PagedMxfp4Cache) is dequantized after the gather in
    the same way.
    """
    fp8 = isinstance(kv_cache, PagedQuantCache)
    kv = kv_cache if fp8 else np.asarray(kv_cache)
    page = kv.shape[1]
    n_pages = -(-int(n_tokens) // page)
    ids = np.asarray(block_table_row[:n_pages], dtype=np.int64)
    if n_pages and (ids.min() < 0 or ids.max() >= kv.shape[0]):
        raise ValueError("block table entry out of range")
    if fp8:   # a quantized cache is dequantized after the gather
        return kv.rows_of_pages(ids).reshape(n_pages * page, kv.shape[2])[:n_tokens]
    rows = kv[ids].reshape(n_pages * page, kv.shape[2])[:n_tokens]
    if rows.dtype == np.uint16:
        return bf16_bits_to_f64(rows)
    return rows


# --------------------------------------------------------------------------
# absorbed path (path B)
# --------------------------------------------------------------------------


def absorb(q_c: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q_abs[..., h, c] = sum_d q_c[..., h, d] * W_UK[h, d, c] (one matmul per head)."""
    q = np.asarray(q_c, np.float64)
    w = np.asarray(w_uk, np.float64)
    lead = q.shape[:-2]
    qh = q.reshape(-1, q.shape[-2], q.shape[-1]).transpose(1, 0, 2)   # [H, T, d]
    out = np.matmul(qh, w)                                             # [H, T, c]
    return out.transpose(1, 0, 2).reshape(lead + (w.shape[0], w.shape[2]))


def visible_len(L_b: int, s_q: int, i: int) -> int:
    """Keys visible to query i of an s_q-token chunk whose latents end the cache."""
    return int(L_b) - int(s_q) + int(i) + 1


def scores_absorbed(qa: np.ndarray, qr: np.ndarray, C: np.ndarray, R: np.ndarray,
                    scale: float) -> np.ndarray:
    """[H, L] scaled scores (q_abs . c_KV + q_R . k_R) * scale."""
    return (qa @ C.T + qr @ R.T) * scale


def softmax_rows(s: np.ndarray):
    """Row softmax with max subtraction; returns (P, m, l) with P = exp(s-m)/l."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    return e / l, m[..., 0], l[..., 0]


def attend_absorbed(qa: np.ndarray, qr: np.ndarray, C: np.ndarray, R: np.ndarray, scale: float):
    """One query token, all heads: (o_lat [H, d_c], lse [H]) over keys C, R."""
    Hn, d_c = qa.shape
    if C.shape[0] == 0:
        return np.zeros((Hn, d_c)), np.full((Hn,), -np.inf)
    s = scores_absorbed(qa, qr, C, R, scale)
    P, m, l = softmax_rows(s)
    return P @ C, m + np.log(l)


def _split_row(row: np.ndarray, d_c: int):
    return row[:, :d_c], row[:, d_c:]


def decode_absorbed(q_abs, q_r, kv_cache, block_table, seqlens, scale: float):
    """Latent attention output o_lat [B, s_q, H, d_c] and lse [B, s_q, H]."""
    q_abs = np.asarray(q_abs, np.float64)
    q_r = np.asarray(q_r, np.float64)
    B, s_q, Hn, d_c = q_abs.shape
    o = np.zeros((B, s_q, Hn, d_c))
    lse = np.zeros((B, s_q, Hn))
    for b in range(B):
        L = int(seqlens[b])
        rows = gather_rows(kv_cache, block_table[b], max(L, 0))
        C, R = _split_row(np.asarray(rows, np.float64), d_c)
        for i in range(s_q):
            n = max(visible_len(L, s_q, i), 0)
            o[b, i], lse[b, i] = attend_absorbed(q_abs[b, i], q_r[b, i], C[:n], R[:n], scale)
    return o, lse


# --------------------------------------------------------------------------
# naive path (path A): decompress per-head keys and values
# --------------------------------------------------------------------------


def decode_naive(q_c, q_r, kv_cache, block_table, seqlens, w_uk, w_uv, scale: float):
    """Final output out [B, s_q, H, d_hc] and lse [B, s_q, H] without absorption.

    K_h[t, d] = sum_c c_KV[t, c] W_UK[h, d, c];  V_h[t, d] = sum_c c_KV[t, c] W_UV[h, d, c].
    """
    q_c = np.asarray(q_c, np.float64)
    q_r = np.asarray(q_r, np.float64)
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    B, s_q, Hn, d_hc = q_c.shape
    d_c = w_uk.shape[2]
    out = np.zeros((B, s_q, Hn, w_uv.shape[1]))
    lse = np.zeros((B, s_q, Hn))
    for b in range(B):
        L = int(seqlens[b])
        rows = np.asarray(gather_rows(kv_cache, block_table[b], max(L, 0)), np.float64)
        C, R = _split_row(rows, d_c)
        for h in range(Hn):
            K = C @ w_uk[h].T          # [L, d_hc]
            V = C @ w_uv[h].T          # [L, d_hc]
            for i in range(s_q):
                n = max(visible_len(L, s_q, i), 0)
                if n == 0:
                    out[b, i, h] = 0.0
                    lse[b, i, h] = -np.inf
                    continue
                s = (K[:n] @ q_c[b, i, h] + R[:n] @ q_r[b, i, h]) * scale
                m = s.max()
                e = np.exp(s - m)
                l = e.sum()
                out[b, i, h] = (e @ V[:n]) / l
                lse[b, i, h] = m + np.log(l)
    return out, lse


# --------------------------------------------------------------------------
# up-projection
# --------------------------------------------------------------------------


def up_proj(o_lat, w_uv) -> np.ndarray:
    """out[..., h, d] = sum_c o_lat[..., h, c] * W_UV[h, d, c] (one matmul per head)."""
    o = np.asarray(o_lat, np.float64)
    w = np.asarray(w_uv, np.float64)
    lead = o.shape[:-2]
    oh = o.reshape(-1, o.shape[-2], o.shape[-1]).transpose(1, 0, 2)   # [H, T, c]
    out = np.matmul(oh, w.transpose(0, 2, 1))                          # [H, T, d]
    return out.transpose(1, 0, 2).reshape(lead + (w.shape[0], w.shape[1]))


# --------------------------------------------------------------------------
# split scan + log-sum-exp combine (stage 1 / stage 2)
# --------------------------------------------------------------------------


def decode_split(q_abs, q_r, kv_cache, block_table, seqlens, scale: float, pieces, num_splits: int):
    """Partials of a given split: stage 1 of the K3 study's "Inside the blocks"
    (each split scans a page range of one row and keeps its own normalised
    output and log-sum-exp).

    pieces[r] for row r = b * s_q + i lists that row's splits as
    (slot, first page, end page): pages [first, end) of the row's visible keys
    go to partial slot `slot`. The caller chooses the partition (any set of
    disjoint page ranges; the combined result does not depend on it). Returns
    o_part [B, s_q, H, S, d_c] (zero for an unused slot) and lse_part
    [B, s_q, H, S] (-inf for an unused slot or an empty range).
    """
    q_abs = np.asarray(q_abs, np.float64)
    q_r = np.asarray(q_r, np.float64)
    B, s_q, Hn, d_c = q_abs.shape
    page = (kv_cache.shape if isinstance(kv_cache, PagedQuantCache) else np.asarray(kv_cache).shape)[1]
    if len(pieces) != B * s_q:
        raise ValueError("one list of pieces per query row")
    o = np.zeros((B, s_q, Hn, num_splits, d_c))
    lse = np.full((B, s_q, Hn, num_splits), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        rows = np.asarray(gather_rows(kv_cache, block_table[b], max(L, 0)), np.float64)
        C, R = _split_row(rows, d_c)
        for i in range(s_q):
            n = max(visible_len(L, s_q, i), 0)
            for s, p0, p1 in pieces[b * s_q + i]:
                if not (0 <= s < num_splits and 0 <= p0 <= p1):
                    raise ValueError(f"bad piece {(s, p0, p1)}")
                t0, t1 = p0 * page, min(p1 * page, n)
                o[b, i, :, s], lse[b, i, :, s] = attend_absorbed(
                    q_abs[b, i], q_r[b, i], C[t0:t1], R[t0:t1], scale)
    return o, lse


def combine(o_part, lse_part):
    """Merge normalised split outputs by their log-sum-exp weights.

    LSE = M + ln sum_s exp(lse_s - M), M = max_s lse_s;  o = sum_s exp(lse_s - LSE) o_s.
    Rows whose splits are all empty give o = 0, LSE = -inf.
    """
    o_part = np.asarray(o_part, np.float64)
    lse_part = np.asarray(lse_part, np.float64)
    M = lse_part.max(axis=-1)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    w = np.where(np.isfinite(lse_part), np.exp(lse_part - Ms[..., None]), 0.0)
    tot = w.sum(axis=-1)
    LSE = np.where(finite, Ms + np.log(np.where(finite, tot, 1.0)), -np.inf)
    wn = np.where(finite[..., None], w / np.where(finite, tot, 1.0)[..., None], 0.0)
    o = np.einsum("...s,...sc->...c", wn, o_part)
    return o, LSE


# --------------------------------------------------------------------------
# sampled rows for large workloads
# --------------------------------------------------------------------------


def decode_rows(q_abs, q_r, kv_cache, block_table, seqlens, scale: float, picks):
    """o_lat and lse for selected (b, i, h) rows only; picks is a list of triples.

    Gathers each needed sequence once; cost is linear in the rows requested.
    """
    q_abs = np.asarray(q_abs)
    q_r = np.asarray(q_r)
    s_q = q_abs.shape[1]
    d_c = q_abs.shape[-1]
    out_o = np.zeros((len(picks), d_c))
    out_l = np.zeros((len(picks),))
    by_b: dict[int, list[int]] = {}
    for k, (b, _, _) in enumerate(picks):
        by_b.setdefault(int(b), []).append(k)
    for b, ks in by_b.items():
        L = int(seqlens[b])
        rows = np.asarray(gather_rows(kv_cache, block_table[b], max(L, 0)), np.float64)
        C, R = _split_row(rows, d_c)
        for k in ks:
            _, i, h = picks[k]
            n = max(visible_len(L, s_q, int(i)), 0)
            qa = np.asarray(q_abs[b, i, h], np.float64)[None]
            qr = np.asarray(q_r[b, i, h], np.float64)[None]
            o, l = attend_absorbed(qa, qr, C[:n], R[:n], scale)
            out_o[k], out_l[k] = o[0], l[0]
    return out_o, out_l


# --------------------------------------------------------------------------
# cache append with the decoupled RoPE key (the step before the path)
# --------------------------------------------------------------------------
# The teardown page fixes the precision of the rotation (the plugin computes
# RoPE in fp32, section 3; the cure for a phase error is a table generated in
# fp32 and fp32 multiply-adds in the kernel, section 4) but not its
# frequencies or pair layout. Readings taken here:
#   * pair j of a d_R-vector is (x[2j], x[2j+1]), j = 0 .. d_R/2 - 1;
#   * its frequency is theta_j = base^(-2j / d_R), base a parameter (10000);
#   * at position p the pair turns by the angle p * theta_j, counter-clockwise
#     in the (x[2j], x[2j+1]) plane;
#   * token i of an s_q-token chunk of sequence b sits at position
#     L_b - s_q + i (L_b counts the chunk), the position the causal reading
#     above gives it; a chunk token with a negative position has no slot.

ROPE_BASE = 10000.0


def rope_angles(positions, d_r: int = 64, base: float = ROPE_BASE) -> np.ndarray:
    """[..., d_r/2] angles p * theta_j for positions of any shape, float64."""
    j = np.arange(d_r // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * j / d_r)
    return np.asarray(positions, np.float64)[..., None] * theta


def rope_rotate(x, positions, base: float = ROPE_BASE) -> np.ndarray:
    """Rotate the last axis (d_R values) of x by RoPE at positions.

    positions broadcasts against x.shape[:-1].
    """
    x = np.asarray(x, np.float64)
    a = rope_angles(np.broadcast_to(np.asarray(positions), x.shape[:-1]), x.shape[-1], base)
    c, s = np.cos(a), np.sin(a)
    xe, xo = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = xe * c - xo * s
    y[..., 1::2] = xe * s + xo * c
    return y


def chunk_positions(seqlens, s_q: int) -> np.ndarray:
    """[B, s_q] positions L_b - s_q + i of each sequence's new tokens."""
    L = np.asarray(seqlens, np.int64)
    return L[:, None] - int(s_q) + np.arange(int(s_q), dtype=np.int64)[None, :]


def append_latent(kv_cache, block_table, seqlens, c_new, kr_new, base: float = ROPE_BASE):
    """Cache after writing one chunk of new tokens.

    kv_cache [P, page, d_c + d_R] (float64 values, copied, not modified);
    c_new [B, s_q, d_c] and kr_new [B, s_q, d_R] (k_R before rotation).
    Token (b, i) goes to logical row p = L_b - s_q + i of sequence b, i.e.
    physical page block_table[b, p // page], row p % page: its c_KV unchanged,
    its k_R rotated by position p. Tokens with p < 0 or past the block table
    are not written. Returns (new cache, list of the (page, row) written).
    """
    cache = np.array(kv_cache, dtype=np.float64, copy=True)
    bt = np.asarray(block_table, np.int64)
    page = cache.shape[1]
    c_new = np.asarray(c_new, np.float64)
    kr_new = np.asarray(kr_new, np.float64)
    d_c = c_new.shape[-1]
    pos = chunk_positions(seqlens, c_new.shape[1])
    written = []
    for b in range(pos.shape[0]):
        for i in range(pos.shape[1]):
            p = int(pos[b, i])
            if p < 0 or p // page >= bt.shape[1]:
                continue
            pg = int(bt[b, p // page])
            if pg < 0 or pg >= cache.shape[0]:
                raise ValueError("block table entry out of range")
            cache[pg, p % page, :d_c] = c_new[b, i]
            cache[pg, p % page, d_c:] = rope_rotate(kr_new[b, i], p, base)
            written.append((pg, p % page))
    return cache, written


# --------------------------------------------------------------------------
# decompressed branch for long chunks, and the dispatch between the two
# --------------------------------------------------------------------------
# The teardown page keeps the absorbed form for chunks of up to
# kPrefillThresh = 256 new tokens (section 3: the constant and the plugin's
# prefill_absorption_threshold) and decompresses the latent cache per head
# for longer chunks (path A of section 4, split into its two stages here:
# per-head keys and values, then causal attention over them).

PREFILL_ABSORPTION_THRESHOLD = 256


def uses_absorption(s_q: int, threshold: int = PREFILL_ABSORPTION_THRESHOLD) -> bool:
    """Whether an s_q-token chunk takes the absorbed path (s_q <= threshold)."""
    return int(s_q) <= int(threshold)


def decompress_kv(kv_cache, block_table, seqlens, w_uk, w_uv, max_len: int):
    """Per-head keys and values of every cached token.

    Returns K, V [B, H, max_len, d_hc]: K[b, h, t] = W_UK[h] . c_KV[t] and
    V[b, h, t] = W_UV[h] . c_KV[t] for t < L_b, zero after.
    """
    w_uk = np.asarray(w_uk, np.float64)
    w_uv = np.asarray(w_uv, np.float64)
    Hn, d_hc, d_c = w_uk.shape
    B = len(seqlens)
    K = np.zeros((B, Hn, max_len, d_hc))
    V = np.zeros((B, Hn, max_len, d_hc))
    for b in range(B):
        L = min(int(seqlens[b]), max_len)
        C = np.asarray(gather_rows(kv_cache, block_table[b], max(L, 0)), np.float64)[:, :d_c]
        K[b, :, :L] = np.einsum("tc,hdc->htd", C, w_uk)
        V[b, :, :L] = np.einsum("tc,hdc->htd", C, w_uv)
    return K, V


def rope_keys(kv_cache, block_table, seqlens, max_len: int, d_c: int = 512):
    """k_R of every cached token, [B, max_len, d_R] (zero past L_b)."""
    d_r = (kv_cache.shape if isinstance(kv_cache, PagedQuantCache) else np.asarray(kv_cache).shape)[2] - d_c
    B = len(seqlens)
    R = np.zeros((B, max_len, d_r))
    for b in range(B):
        L = min(int(seqlens[b]), max_len)
        R[b, :L] = np.asarray(gather_rows(kv_cache, block_table[b], max(L, 0)), np.float64)[:, d_c:]
    return R


def attend_mha(q_c, q_r, K, V, R, seqlens, scale: float):
    """Causal multi-head attention over decompressed keys and values.

    q_c [B, s_q, H, d_hc], q_r [B, s_q, H, d_R]; K, V [B, H, max_len, d_hc];
    R [B, max_len, d_R] (the shared RoPE keys). Query i of sequence b sees
    keys t < visible_len(L_b, s_q, i) with score (q_c . K + q_r . k_R) * scale.
    Returns out [B, s_q, H, d_hc] and lse [B, s_q, H] (0 and -inf for a
    query with no visible key).
    """
    q_c = np.asarray(q_c, np.float64)
    q_r = np.asarray(q_r, np.float64)
    B, s_q, Hn, d_hc = q_c.shape
    out = np.zeros((B, s_q, Hn, V.shape[-1]))
    lse = np.full((B, s_q, Hn), -np.inf)
    for b in range(B):
        L = int(seqlens[b])
        for i in range(s_q):
            n = min(max(visible_len(L, s_q, i), 0), K.shape[2])
            if n == 0:
                continue
            for h in range(Hn):
                s = (K[b, h, :n] @ q_c[b, i, h] + R[b, :n] @ q_r[b, i, h]) * scale
                p, m, l = softmax_rows(s[None])
                out[b, i, h] = p[0] @ V[b, h, :n]
                lse[b, i, h] = m[0] + np.log(l[0])
    return out, lse


# --------------------------------------------------------------------------
# 8-bit latent cache: c_KV in FP8 E4M3 with one power-of-two scale per token
# --------------------------------------------------------------------------
# The teardown page reads a 4-bit (NVFP4) latent cache with 16-byte vector
# loads whose page base and dimension offset must be 16-byte aligned
# (section 5, the misaligned-address failure), and gives neither the element
# format nor the scaling. Readings taken here, for an 8-bit cache:
#   * c_KV is stored in OCP FP8 E4M3: sign, 4 exponent bits with bias 7 and
#     3 mantissa bits; exponent 0 holds the subnormals m/8 * 2^-6; there are
#     no infinities, S.1111.111 is NaN and the largest finite value is 448;
#   * k_R keeps its bf16 bits (the rotated key is stored exactly);
#   * each token's c_KV shares one scale 2^k: the smallest power of two with
#     max|c_KV| <= 448 * 2^k, k clamped to [-126, 127] (-126 for a zero row),
#     so no element ever saturates;
#   * an element's code is c / 2^k rounded to the nearest E4M3 value, ties to
#     the even mantissa, with the sign bit of c (a negative value that rounds
#     to zero is stored as -0);
#   * the stored value of a code is its E4M3 value times 2^k;
#   * a page of 64 tokens is three arrays, each starting on a 16-byte
#     boundary: 64 x 512 codes, then 64 x 64 bf16 k_R, then 64 float32
#     scales (41216 bytes).

FP8_MAX = 448.0
FP8_SCALE_EXP_MIN = -126
FP8_SCALE_EXP_MAX = 127


def e4m3_value(codes) -> np.ndarray:
    """Exact float64 value of E4M3 codes (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.ldexp(1.0, e - 10))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def _e4m3_table() -> np.ndarray:
    """e4m3_value of every code 0..255, indexed by the code."""
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        _E4M3_TABLE = e4m3_value(np.arange(256))
    return _E4M3_TABLE


_E4M3_TABLE = None


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of exact values with |v| <= 448, ties to even, sign kept."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    if not np.all(a <= FP8_MAX):
        raise ValueError("E4M3 encode: value outside [-448, 448] or NaN")
    _, x = np.frexp(a)                      # a = f * 2^x, f in [0.5, 1); x = 0 for a = 0
    E = np.maximum(x - 1, -6)               # binade of a; below 2^-6 the subnormal spacing
    q = np.round(np.ldexp(a, 3 - E))        # a in units of the binade's spacing 2^(E-3); ties to even
    up = q >= 16                            # rounded up into the next binade
    E = np.where(up, E + 1, E)
    q = np.where(up, 8, q).astype(np.int64)
    normal = q >= 8
    e_field = np.where(normal, E + 7, 0)
    m_field = np.where(normal, q - 8, q)
    return ((np.signbit(v).astype(np.int64) << 7) | (e_field << 3) | m_field).astype(np.uint8)


def fp8_scale_exponent(amax) -> np.ndarray:
    """k of a token's scale: the smallest integer with amax <= 448 * 2^k, clamped."""
    a = np.asarray(amax, np.float64)
    f, x = np.frexp(a)                      # 448 * 2^k = 0.875 * 2^(k + 9)
    k = x - 9 + (f > 0.875)
    k = np.clip(k, FP8_SCALE_EXP_MIN, FP8_SCALE_EXP_MAX)
    return np.where(a == 0, FP8_SCALE_EXP_MIN, k).astype(np.int64)


def quantize_latent_fp8(c):
    """(codes uint8 [..., d_c], k int64 [...]) of latent rows c [..., d_c]."""
    c = np.asarray(c, np.float64)
    k = fp8_scale_exponent(np.abs(c).max(axis=-1))
    return e4m3_encode(np.ldexp(c, -k[..., None])), k


def dequantize_latent_fp8(codes, k) -> np.ndarray:
    """Stored values: E4M3 value of each code times 2^k of its token."""
    return np.ldexp(e4m3_value(codes), np.asarray(k, np.int64)[..., None])


def fp8_page_bytes(page: int = 64, d_c: int = 512, d_r: int = 64) -> int:
    """Bytes of one page of the 8-bit cache: codes, bf16 k_R and float32 scales."""
    return page * d_c + page * d_r * 2 + page * 4


def pack_fp8_cache(kv_bits, d_c: int = 512, chunk_pages: int = 256) -> np.ndarray:
    """8-bit pages [P, fp8_page_bytes] of a bf16 cache given as bit patterns [P, page, d_c + d_R]."""
    kv_bits = np.asarray(kv_bits)
    if kv_bits.dtype != np.uint16:
        raise ValueError("pack_fp8_cache takes the bf16 bit patterns (uint16)")
    P, page, row = kv_bits.shape
    d_r = row - d_c
    out = np.zeros((P, fp8_page_bytes(page, d_c, d_r)), np.uint8)
    o_rope, o_scale = page * d_c, page * d_c + page * d_r * 2
    for p0 in range(0, P, chunk_pages):
        blk = kv_bits[p0:p0 + chunk_pages]
        n = blk.shape[0]
        codes, k = quantize_latent_fp8(bf16_bits_to_f64(blk[..., :d_c]))
        out[p0:p0 + n, :o_rope] = codes.reshape(n, page * d_c)
        out[p0:p0 + n, o_rope:o_scale] = np.ascontiguousarray(blk[..., d_c:]).view(np.uint8).reshape(n, -1)
        scale = np.ldexp(1.0, k).astype("<f4")
        out[p0:p0 + n, o_scale:] = scale.view(np.uint8).reshape(n, -1)
    return out


def unpack_fp8_pages(pages, page: int = 64, d_c: int = 512, d_r: int = 64):
    """(codes [n, page, d_c] uint8, k_R bits [n, page, d_R] uint16, scales [n, page] float32)."""
    pages = np.ascontiguousarray(pages, np.uint8)
    n = pages.shape[0]
    if pages.shape[1] != fp8_page_bytes(page, d_c, d_r):
        raise ValueError("page size does not match the 8-bit layout")
    o_rope, o_scale = page * d_c, page * d_c + page * d_r * 2
    codes = pages[:, :o_rope].reshape(n, page, d_c)
    rope = pages[:, o_rope:o_scale].copy().view("<u2").reshape(n, page, d_r)
    scale = pages[:, o_scale:].copy().view("<f4").reshape(n, page)
    return codes, rope, scale


def dequantize_fp8_pages(pages, page: int = 64, d_c: int = 512, d_r: int = 64) -> np.ndarray:
    """float64 rows [n, page, d_c + d_R] stored by 8-bit pages. Codes are looked
    up in the table of e4m3_value over all 256 codes (the same values, without
    evaluating the format's formula once per element of a large cache)."""
    codes, rope, scale = unpack_fp8_pages(pages, page, d_c, d_r)
    c = np.take(_e4m3_table(), codes.astype(np.intp)) * scale.astype(np.float64)[..., None]
    return np.concatenate([c, bf16_bits_to_f64(rope)], axis=-1)


class PagedQuantCache:
    """A quantized paged cache (uint8 pages [P, page_bytes]) as the decode
    oracles read it: gather_rows dequantizes only the pages a sequence uses,
    and np.asarray gives the whole cache in float64 (small caches only).
    Subclasses name the page size and the dequantization of a page."""

    page_bytes = None   # (page, d_c, d_r) -> bytes of one page
    dequantize = None   # (pages, page, d_c, d_r) -> float64 rows [n, page, d_c + d_r]

    def __init__(self, pages, page: int = 64, d_c: int = 512, d_r: int = 64):
        self.pages = np.asarray(pages, np.uint8)
        self.page, self.d_c, self.d_r = page, d_c, d_r
        nbytes = type(self).page_bytes(page, d_c, d_r)
        if self.pages.ndim != 2 or self.pages.shape[1] != nbytes:
            raise ValueError(f"expected uint8 pages [P, {nbytes}]")
        self.shape = (self.pages.shape[0], page, d_c + d_r)

    def rows_of_pages(self, ids) -> np.ndarray:
        return type(self).dequantize(self.pages[np.asarray(ids, np.int64)], self.page, self.d_c, self.d_r)

    def __array__(self, dtype=None, copy=None):
        out = type(self).dequantize(self.pages, self.page, self.d_c, self.d_r)
        return out if dtype is None else out.astype(dtype)


class PagedFp8Cache(PagedQuantCache):
    """The 8-bit cache: pages [P, fp8_page_bytes]."""
    page_bytes = staticmethod(fp8_page_bytes)
    dequantize = staticmethod(dequantize_fp8_pages)


# --------------------------------------------------------------------------
# 4-bit latent cache: c_KV in MXFP4 (E2M1 elements, one E8M0 scale per 32)
# --------------------------------------------------------------------------
# The NVFP4 gather of the teardown page (section 5) names a 4-bit latent
# cache; MI355X's matrix cores read the OCP microscaling form of one (MXFP4)
# directly. Readings taken here:
#   * an element is OCP E2M1: sign, 2 exponent bits with bias 1, 1 mantissa
#     bit; exponent 0 holds 0 and the subnormal 0.5; the magnitudes are
#     0, 0.5, 1, 1.5, 2, 3, 4, 6; there are no infinities or NaN;
#   * each block of 32 consecutive c_KV dims of a token (16 blocks per row)
#     shares one scale 2^k, stored as the E8M0 byte k + 127, with k the
#     smallest integer such that max|block| <= 6 * 2^k, clamped to
#     [-126, 127] (-126 for a zero block): no element saturates (the OCP
#     rule k = floor(log2 max|block|) - 2 would clip values above 6 * 2^k);
#   * an element's code is c / 2^k rounded to the nearest E2M1 value, ties
#     to the even mantissa, with the sign bit of c (a negative value that
#     rounds to zero is stored as -0);
#   * two elements per byte, the even dim in the low nibble;
#   * k_R keeps its bf16 bits;
#   * a page of 64 tokens is three arrays, each starting on a 16-byte
#     boundary: 64 x 256 code bytes, then 64 x 64 bf16 k_R, then 64 x 16
#     scale bytes (25600 bytes).

E2M1_MAX = 6.0
MX_BLOCK = 32
MX_SCALE_EXP_MIN = -126
MX_SCALE_EXP_MAX = 127


def e2m1_value(codes) -> np.ndarray:
    """Exact float64 value of E2M1 codes (4-bit, 0..15)."""
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(c & 8, -mag, mag)


def e2m1_encode(v) -> np.ndarray:
    """Nearest E2M1 code of exact values with |v| <= 6, ties to the even code, sign kept."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    if not np.all(a <= E2M1_MAX):
        raise ValueError("E2M1 encode: value outside [-6, 6] or NaN")
    mags = e2m1_value(np.arange(8))                       # the 8 magnitudes, in code order
    d = np.abs(a[..., None] - mags)
    near = d == d.min(axis=-1, keepdims=True)             # one code, or two adjacent ones on a tie
    even = near & (np.arange(8) % 2 == 0)
    code = np.where(even.any(axis=-1), even.argmax(axis=-1), near.argmax(axis=-1))
    return ((np.signbit(v).astype(np.int64) << 3) | code).astype(np.uint8)


def mx_scale_exponent(amax) -> np.ndarray:
    """k of a block's scale: the smallest integer with amax <= 6 * 2^k, clamped."""
    a = np.asarray(amax, np.float64)
    f, x = np.frexp(a)                      # 6 * 2^k = 0.75 * 2^(k + 3)
    k = x - 3 + (f > 0.75)
    k = np.clip(k, MX_SCALE_EXP_MIN, MX_SCALE_EXP_MAX)
    return np.where(a == 0, MX_SCALE_EXP_MIN, k).astype(np.int64)


def quantize_latent_mxfp4(c):
    """(codes uint8 [..., d_c], one E2M1 code per element; k int64 [..., d_c / 32])."""
    c = np.asarray(c, np.float64)
    blocks = c.reshape(c.shape[:-1] + (c.shape[-1] // MX_BLOCK, MX_BLOCK))
    k = mx_scale_exponent(np.abs(blocks).max(axis=-1))
    codes = e2m1_encode(np.ldexp(blocks, -k[..., None]))
    return codes.reshape(c.shape), k


def dequantize_latent_mxfp4(codes, k) -> np.ndarray:
    """Stored values: E2M1 value of each code times 2^k of its block."""
    codes = np.asarray(codes)
    k = np.asarray(k, np.int64)
    v = np.take(e2m1_value(np.arange(16)), np.asarray(codes).astype(np.intp))
    v = v.reshape(codes.shape[:-1] + (k.shape[-1], MX_BLOCK))
    # 2^k of each block times its values: exact in float64 (E2M1 values have two
    # significant bits and 2^k, |k| <= 127, is a float64 power of two)
    return (v * np.ldexp(1.0, k)[..., None]).reshape(codes.shape)


def mxfp4_page_bytes(page: int = 64, d_c: int = 512, d_r: int = 64) -> int:
    """Bytes of one page of the 4-bit cache: packed codes, bf16 k_R and E8M0 scales."""
    return page * d_c // 2 + page * d_r * 2 + page * d_c // MX_BLOCK


def pack_mxfp4_cache(kv_bits, d_c: int = 512, chunk_pages: int = 256) -> np.ndarray:
    """4-bit pages [P, mxfp4_page_bytes] of a bf16 cache given as bit patterns [P, page, d_c + d_R]."""
    kv_bits = np.asarray(kv_bits)
    if kv_bits.dtype != np.uint16:
        raise ValueError("pack_mxfp4_cache takes the bf16 bit patterns (uint16)")
    P, page, row = kv_bits.shape
    d_r = row - d_c
    out = np.zeros((P, mxfp4_page_bytes(page, d_c, d_r)), np.uint8)
    o_rope = page * d_c // 2
    o_scale = o_rope + page * d_r * 2
    for p0 in range(0, P, chunk_pages):
        blk = kv_bits[p0:p0 + chunk_pages]
        n = blk.shape[0]
        codes, k = quantize_latent_mxfp4(bf16_bits_to_f64(blk[..., :d_c]))
        packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
        out[p0:p0 + n, :o_rope] = packed.reshape(n, -1)
        out[p0:p0 + n, o_rope:o_scale] = np.ascontiguousarray(blk[..., d_c:]).view(np.uint8).reshape(n, -1)
        out[p0:p0 + n, o_scale:] = (k + 127).astype(np.uint8).reshape(n, -1)
    return out


def unpack_mxfp4_pages(pages, page: int = 64, d_c: int = 512, d_r: int = 64):
    """(codes [n, page, d_c] uint8 one per element, k_R bits [n, page, d_R] uint16,
    scale exponents k [n, page, d_c / 32] int64)."""
    pages = np.ascontiguousarray(pages, np.uint8)
    n = pages.shape[0]
    if pages.shape[1] != mxfp4_page_bytes(page, d_c, d_r):
        raise ValueError("page size does not match the 4-bit layout")
    o_rope = page * d_c // 2
    o_scale = o_rope + page * d_r * 2
    packed = pages[:, :o_rope].reshape(n, page, d_c // 2)
    codes = np.empty((n, page, d_c), np.uint8)
    codes[..., 0::2] = packed & 15
    codes[..., 1::2] = packed >> 4
    rope = pages[:, o_rope:o_scale].copy().view("<u2").reshape(n, page, d_r)
    k = pages[:, o_scale:].reshape(n, page, d_c // MX_BLOCK).astype(np.int64) - 127
    return codes, rope, k


def dequantize_mxfp4_pages(pages, page: int = 64, d_c: int = 512, d_r: int = 64) -> np.ndarray:
    """float64 rows [n, page, d_c + d_R] stored by 4-bit pages."""
    codes, rope, k = unpack_mxfp4_pages(pages, page, d_c, d_r)
    return np.concatenate([dequantize_latent_mxfp4(codes, k), bf16_bits_to_f64(rope)], axis=-1)


class PagedMxfp4Cache(PagedQuantCache):
    """The 4-bit cache: pages [P, mxfp4_page_bytes]."""
    page_bytes = staticmethod(mxfp4_page_bytes)
    dequantize = staticmethod(dequantize_mxfp4_pages)
