"""Seeded synthetic inputs for absorbed MLA decode over a paged latent cache.

This module only *generates data*: tensor shapes, value distributions, page
placement and sequence lengths. It contains no attention arithmetic, so both
the fp64 oracle tests and the GPU tests (and the benchmark) can draw the same
inputs from it without sharing any of the method's computation.

Shapes follow the MLA operator-teardown page (jh158.com "DeepSeek MLA source
teardown", section 3 constants and section 4 absorption check): 128 heads,
content head dim 128, latent dim 512, decoupled RoPE dim 64, page size 64.

Recipe (one reading of the pages, stated once here):
  * values: float32 ``torch.randn`` rounded to bfloat16 (round-to-nearest-even);
    activations and cache rows ~ N(0, 1); W_UK and W_UV ~ N(0, variance 1/512).
  * draw order on the tensor generator (seeded ``seed``): q_c, q_R, W_UK,
    c_KV, k_R, W_UV -- the order of the teardown page's section-4 script,
    with W_UV appended.
  * structure (sequence lengths, page placement) comes from a second CPU
    generator seeded ``seed ^ 0x5EED`` so that the pool size can depend on the
    drawn lengths before any tensor is drawn.
  * the physical page pool is permuted; sequence b owns the next
    ``ceil(L_b/64)`` pool pages in permuted order; unused block-table tail
    entries are -1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

H = 128          # attention heads
D_HC = 128       # per-head content (nope) dim of q_c / W_UK rows
D_C = 512        # latent dim of c_KV
D_R = 64         # decoupled RoPE dim
ROW = D_C + D_R  # 576 bf16 values stored per token and layer
PAGE = 64        # tokens per page

STRUCT_SEED_XOR = 0x5EED


@dataclass(frozen=True)
class Config:
    """One synthetic workload."""
    name: str
    B: int
    s_q: int
    seqlen_rule: str            # "fixed" | "uniform"
    ctx: int = 0                # fixed context length (tokens in cache incl. chunk)
    max_ctx: int = 0            # upper bound for "uniform" lengths
    pool_pages: int = 0         # physical pages in the pool (0: exactly what is needed)
    identity_table: bool = False
    max_pages: int = 0          # block-table width (0: ceil(max length / 64))
    layers: int = 1             # resident cache layers (bench rotates through them)
    notes: str = ""


CONFIGS: dict[str, Config] = {
    # the teardown page's absorption check size: one query, S = 2048
    "single": Config("single", B=1, s_q=1, seqlen_rule="fixed", ctx=2048,
                     identity_table=True,
                     notes="B=1 ctx 2048, 32 pages, identity block table"),
    "uniform": Config("uniform", B=16, s_q=1, seqlen_rule="fixed", ctx=4096,
                      pool_pages=1024,
                      notes="B=16 ctx 4096, pages from a permuted 1024-page pool"),
    "ragged": Config("ragged", B=64, s_q=1, seqlen_rule="uniform", max_ctx=32768,
                     max_pages=512,
                     notes="B=64, L_b ~ U[1, 32768], shuffled shared pool, -1 tails"),
    "long": Config("long", B=16, s_q=1, seqlen_rule="fixed", ctx=65536, layers=60,
                   notes="B=16 ctx 65536, 16384 pages per layer, 60 layers resident"),
    "prefill": Config("prefill", B=4, s_q=256, seqlen_rule="fixed", ctx=16384 + 256,
                      pool_pages=1040,
                      notes="B=4, 256-token causal chunk over a 16384-token prefix"),
}


@dataclass
class Structure:
    seqlens: torch.Tensor       # [B] int32, tokens in cache per sequence (incl. chunk)
    block_table: torch.Tensor   # [B, max_pages] int32, -1 for unused entries
    num_pages: int              # physical pages per layer


@dataclass
class Inputs:
    cfg: Config
    seqlens: torch.Tensor       # [B] int32
    block_table: torch.Tensor   # [B, max_pages] int32
    q_c: torch.Tensor           # [B, s_q, H, 128] bf16
    q_r: torch.Tensor           # [B, s_q, H, 64] bf16
    w_uk: torch.Tensor          # [H, 128, 512] bf16
    kv_cache: torch.Tensor      # [num_pages, 64, 576] bf16 (c_KV cols 0..511, k_R 512..575)
    w_uv: torch.Tensor          # [H, 128, 512] bf16
    extra: dict = field(default_factory=dict)


def pages_for(n_tokens: int) -> int:
    """Pages a sequence of ``n_tokens`` occupies (input construction only)."""
    return -(-int(n_tokens) // PAGE)


def make_structure(cfg: Config, seed: int = 42, layout_seed: int | None = None) -> Structure:
    """Sequence lengths drawn from ``seed``; the physical page layout from the
    same generator, or, with another ``layout_seed``, from a generator of its
    own (the lengths stay those of ``seed``: several layers of one batch)."""
    g = torch.Generator().manual_seed(seed ^ STRUCT_SEED_XOR)
    if cfg.seqlen_rule == "fixed":
        seqlens = torch.full((cfg.B,), cfg.ctx, dtype=torch.int32)
    elif cfg.seqlen_rule == "uniform":
        seqlens = torch.randint(1, cfg.max_ctx + 1, (cfg.B,), generator=g, dtype=torch.int64).to(torch.int32)
    else:
        raise ValueError(cfg.seqlen_rule)
    if layout_seed is not None and layout_seed != seed:
        g = torch.Generator().manual_seed(layout_seed ^ STRUCT_SEED_XOR)
    need = [pages_for(int(L)) for L in seqlens]
    total = sum(need)
    pool = cfg.pool_pages or total
    if pool < total:
        raise ValueError(f"pool of {pool} pages cannot hold {total}")
    max_pages = cfg.max_pages or max(need)
    if cfg.identity_table:
        order = torch.arange(pool, dtype=torch.int64)
    else:
        order = torch.randperm(pool, generator=g)
    bt = torch.full((cfg.B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[off:off + n].to(torch.int32)
        off += n
    return Structure(seqlens=seqlens, block_table=bt, num_pages=pool)


def _randn_bf16(shape, g, scale: float = 1.0) -> torch.Tensor:
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(torch.bfloat16)


def make_inputs(cfg: Config | str, seed: int = 42, with_cache: bool = True) -> Inputs:
    """All inputs of one layer on the CPU, in the documented draw order."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    st = make_structure(cfg, seed)
    g = torch.Generator().manual_seed(seed)
    w_scale = 1.0 / math.sqrt(D_C)
    q_c = _randn_bf16((cfg.B, cfg.s_q, H, D_HC), g)
    q_r = _randn_bf16((cfg.B, cfg.s_q, H, D_R), g)
    w_uk = _randn_bf16((H, D_HC, D_C), g, w_scale)
    rows = st.num_pages * PAGE
    if with_cache:
        c_kv = _randn_bf16((rows, D_C), g)
        k_r = _randn_bf16((rows, D_R), g)
        kv = torch.cat([c_kv, k_r], dim=1).view(st.num_pages, PAGE, ROW)
        del c_kv, k_r
    else:
        kv = torch.empty((0, PAGE, ROW), dtype=torch.bfloat16)
    w_uv = _randn_bf16((H, D_HC, D_C), g, w_scale)
    return Inputs(cfg, st.seqlens, st.block_table, q_c, q_r, w_uk, kv, w_uv)


def make_cache_on_device(num_pages: int, layers: int, seed: int, device) -> torch.Tensor:
    """[layers, num_pages, 64, 576] bf16 ~ N(0,1) drawn directly on ``device``.

    Used where the cache is too large to draw on the host (60 resident layers of
    the 64K-context workload); the values come from torch's device generator
    seeded with ``seed``.
    """
    g = torch.Generator(device=device).manual_seed(seed)
    out = torch.empty((layers, num_pages, PAGE, ROW), dtype=torch.bfloat16, device=device)
    chunk = 1024  # pages per draw (~75 MB of float32 at a time)
    for l in range(layers):
        for p0 in range(0, num_pages, chunk):
            p1 = min(num_pages, p0 + chunk)
            out[l, p0:p1].copy_(torch.randn((p1 - p0, PAGE, ROW), generator=g, device=device,
                                            dtype=torch.float32))
    return out


FP8_PAGE_BYTES = PAGE * D_C + PAGE * D_R * 2 + PAGE * 4   # 41216: codes, bf16 k_R, float32 scales


def random_fp8_pages(num_pages: int, seed: int, k_lo: int = -10, k_hi: int = -6) -> torch.Tensor:
    """uint8 [num_pages, 41216] in the 8-bit cache layout, filled with seeded
    data (no quantization happens here): E4M3 codes uniform over all bytes
    with the two NaN codes 0x7F / 0xFF replaced by 0x7E / 0xFE, k_R ~ N(0, 1)
    rounded to bf16, and per-token scales 2^k, k uniform in [k_lo, k_hi],
    stored as float32 bit patterns (k + 127) << 23."""
    g = torch.Generator().manual_seed(seed)
    out = torch.empty((num_pages, FP8_PAGE_BYTES), dtype=torch.uint8)
    codes = out[:, :PAGE * D_C]
    codes.copy_(torch.randint(0, 256, (num_pages, PAGE * D_C), generator=g, dtype=torch.uint8))
    codes[(codes & 0x7F) == 0x7F] -= 1
    rope = _randn_bf16((num_pages, PAGE * D_R), g)
    out[:, PAGE * D_C:PAGE * D_C + PAGE * D_R * 2] = rope.view(torch.uint8).view(num_pages, -1)
    k = torch.randint(k_lo, k_hi + 1, (num_pages, PAGE), generator=g, dtype=torch.int32)
    out[:, PAGE * D_C + PAGE * D_R * 2:] = ((k + 127) << 23).view(torch.uint8).view(num_pages, -1)
    return out


MXFP4_PAGE_BYTES = PAGE * D_C // 2 + PAGE * D_R * 2 + PAGE * D_C // 32   # 25600: codes, bf16 k_R, E8M0 scales


def random_mxfp4_pages(num_pages: int, seed: int, k_lo: int = -3, k_hi: int = -1) -> torch.Tensor:
    """uint8 [num_pages, 25600] in the 4-bit cache layout, filled with seeded
    data (no quantization happens here): packed E2M1 codes uniform over all
    bytes (every nibble is a number), k_R ~ N(0, 1) rounded to bf16, and one
    E8M0 scale byte k + 127 per token and 32-dim block, k uniform in
    [k_lo, k_hi]."""
    g = torch.Generator().manual_seed(seed)
    out = torch.empty((num_pages, MXFP4_PAGE_BYTES), dtype=torch.uint8)
    n_codes = PAGE * D_C // 2
    out[:, :n_codes] = torch.randint(0, 256, (num_pages, n_codes), generator=g, dtype=torch.uint8)
    rope = _randn_bf16((num_pages, PAGE * D_R), g)
    out[:, n_codes:n_codes + PAGE * D_R * 2] = rope.view(torch.uint8).view(num_pages, -1)
    k = torch.randint(k_lo, k_hi + 1, (num_pages, PAGE * D_C // 32), generator=g, dtype=torch.int32)
    out[:, n_codes + PAGE * D_R * 2:] = (k + 127).to(torch.uint8)
    return out


def tiny_inputs(B: int, s_q: int, seqlens, h: int, d_hc: int, d_c: int, d_r: int,
                page: int, seed: int = 7, pool_extra: int = 3):
    """Small float64 inputs of arbitrary dims for brute-force oracle checks.

    Returns a dict of numpy-free torch float64 tensors plus a permuted block
    table. Used only on the CPU.
    """
    g = torch.Generator().manual_seed(seed)
    need = [-(-int(L) // page) for L in seqlens]
    pool = sum(need) + pool_extra
    order = torch.randperm(pool, generator=g)
    maxp = max(max(need), 1)
    bt = torch.full((B, maxp), -1, dtype=torch.int64)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[off:off + n]
        off += n
    return dict(
        q_c=torch.randn((B, s_q, h, d_hc), generator=g, dtype=torch.float64),
        q_r=torch.randn((B, s_q, h, d_r), generator=g, dtype=torch.float64),
        w_uk=torch.randn((h, d_hc, d_c), generator=g, dtype=torch.float64) / math.sqrt(d_c),
        kv_cache=torch.randn((pool, page, d_c + d_r), generator=g, dtype=torch.float64),
        w_uv=torch.randn((h, d_hc, d_c), generator=g, dtype=torch.float64) / math.sqrt(d_c),
        block_table=bt,
        seqlens=torch.tensor(list(seqlens), dtype=torch.int64),
    )
