"""Absorbed MLA decode over a paged latent cache on MI355X (gfx950).

Python binding of libmla (include/mla.h). Each function has the name of the
C entry point it calls; it only checks and marshals arguments (dtype, shape,
device, contiguity, the current torch stream) and allocates outputs through
torch when none are given. All computation runs in the HIP kernels.

Shapes (H = 128 heads, content dim 128, latent 512, RoPE 64, page 64):
  q_c      bf16 [B, s_q, H, 128]          w_uk, w_uv  bf16 [H, 128, 512]
  q_abs    bf16 [B, s_q, H, 512]          q_r         bf16 [B, s_q, H, 64]
  kv_cache bf16 [num_pages, 64, 576]      block_table int32 [B, max_pages]
  seqlens  int32 [B] (tokens in cache incl. the s_q new ones)
  o_part   fp32 [B, s_q, H, S, 512]       lse_part    fp32 [B, s_q, H, S]
  o_lat    fp32 [B, s_q, H, 512]          lse         fp32 [B, s_q, H]
  out      bf16 [B, s_q, H, 128]
  c_new    bf16 [B, s_q, 512]             kr_new      bf16 [B, s_q, 64]
  rope     fp32 [max_pos, 32, 2] (cos, sin of p * 10000^(-2j/64) by default)
"""
from __future__ import annotations

import math

import torch

from . import _lib

H, D_HC, D_C, D_R, ROW, PAGE = 128, 128, 512, 64, 576, 64
DEFAULT_SCALE = 1.0 / math.sqrt(D_HC + D_R)

STATUS_NAMES = {0: "MLA_OK", 1: "MLA_ERR_NULL", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_ALIGN",
                4: "MLA_ERR_WORKSPACE", 5: "MLA_ERR_HIP"}


class MlaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = _lib.LIB.mla_status_string(status).decode()
        detail = _lib.LIB.mla_last_error().decode()
        super().__init__(f"{where}: {name}: {detail}")


def _check(status: int, where: str):
    if status != 0:
        raise MlaError(status, where)


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def num_cus(device=None) -> int:
    return torch.cuda.get_device_properties(device or torch.cuda.current_device()).multi_processor_count


def mla_recommended_splits(B: int, s_q: int, max_len: int, cus: int | None = None) -> int:
    return int(_lib.LIB.mla_recommended_splits(int(B), int(s_q), int(max_len), int(cus or num_cus())))


def mla_plan_splits(seqlens, max_pages: int, s_q: int = 1, cus: int | None = None) -> int:
    """Split count for host-known lengths (a sequence of ints or a CPU int tensor)."""
    lens = torch.as_tensor(seqlens, dtype=torch.int32, device="cpu").contiguous()
    if lens.dim() != 1 or lens.numel() < 1:
        raise ValueError("seqlens must be a non-empty 1-D sequence of lengths")
    return int(_lib.LIB.mla_plan_splits(lens.data_ptr(), int(lens.numel()), int(s_q), int(max_pages),
                                        int(cus or num_cus())))


def mla_validate_block_table(block_table, seqlens, num_pages: int):
    """Host check of a block table against the paged calls' contract (the C
    function of the same name): returns None when every length lies in
    [0, max_pages * 64] and every entry a decode reads lies in [0, num_pages);
    otherwise raises MlaError naming the first bad (sequence, page). Tensors
    on a GPU are copied to the host first."""
    bt = torch.as_tensor(block_table).to(device="cpu", dtype=torch.int32).contiguous()
    lens = torch.as_tensor(seqlens).to(device="cpu", dtype=torch.int32).contiguous()
    if bt.dim() != 2 or lens.dim() != 1 or bt.shape[0] != lens.numel():
        raise ValueError("block_table must be [B, max_pages] and seqlens [B]")
    import ctypes
    bad_seq, bad_page = ctypes.c_int(-1), ctypes.c_int(-1)
    st = _lib.LIB.mla_validate_block_table(bt.data_ptr(), int(bt.shape[1]), lens.data_ptr(), int(lens.numel()),
                                           int(num_pages), ctypes.addressof(bad_seq), ctypes.addressof(bad_page))
    _check(st, "mla_validate_block_table")


def mla_decode_workspace_bytes(B: int, s_q: int, num_splits: int, heads: int = H) -> int:
    return int(_lib.LIB.mla_decode_workspace_bytes(int(B), int(s_q), int(heads), int(num_splits)))


def mla_absorb_q(q_c: torch.Tensor, w_uk: torch.Tensor, q_abs: torch.Tensor | None = None, stream=None):
    """q_abs[..., h, :] = q_c[..., h, :] @ W_UK[h]; q_c [..., H, 128] -> q_abs [..., H, 512]."""
    lead = tuple(q_c.shape[:-2])
    T = math.prod(lead) if lead else 1
    _need(q_c, "q_c", torch.bfloat16, lead + (H, D_HC))
    _need(w_uk, "w_uk", torch.bfloat16, (H, D_HC, D_C))
    if q_abs is None:
        q_abs = torch.empty(lead + (H, D_C), dtype=torch.bfloat16, device=q_c.device)
    _need(q_abs, "q_abs", torch.bfloat16, lead + (H, D_C))
    _check(_lib.LIB.mla_absorb_q(_ptr(q_c), _ptr(w_uk), _ptr(q_abs), T, H, _stream(stream)), "mla_absorb_q")
    return q_abs


def mla_decode_paged(q_abs, q_r, kv_cache, block_table, seqlens, num_splits: int,
                     softmax_scale: float = DEFAULT_SCALE, o_part=None, lse_part=None, stream=None):
    """Split scan; returns (o_part [B,s_q,H,S,512] fp32, lse_part [B,s_q,H,S] fp32)."""
    B, s_q = q_abs.shape[0], q_abs.shape[1]
    _need(q_abs, "q_abs", torch.bfloat16, (B, s_q, H, D_C))
    _need(q_r, "q_r", torch.bfloat16, (B, s_q, H, D_R))
    if kv_cache.dim() != 3 or kv_cache.shape[1:] != (PAGE, ROW):
        raise ValueError(f"kv_cache must be [num_pages, 64, 576], got {tuple(kv_cache.shape)}")
    _need(kv_cache, "kv_cache", torch.bfloat16)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B, max_pages], got {tuple(block_table.shape)}")
    _need(block_table, "block_table", torch.int32)
    _need(seqlens, "seqlens", torch.int32, (B,))
    S = int(num_splits)
    if o_part is None:
        o_part = torch.empty((B, s_q, H, S, D_C), dtype=torch.float32, device=q_abs.device)
    if lse_part is None:
        lse_part = torch.empty((B, s_q, H, S), dtype=torch.float32, device=q_abs.device)
    _need(o_part, "o_part", torch.float32, (B, s_q, H, S, D_C))
    _need(lse_part, "lse_part", torch.float32, (B, s_q, H, S))
    _check(_lib.LIB.mla_decode_paged(
        _ptr(q_abs), _ptr(q_r), _ptr(kv_cache), kv_cache.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), B, s_q, H, float(softmax_scale), S, _ptr(o_part), _ptr(lse_part), _stream(stream)),
        "mla_decode_paged")
    return o_part, lse_part


FP8_PAGE_BYTES = 41216  # MLA_FP8_PAGE_BYTES: 64 x 512 E4M3 codes, 64 x 64 bf16 k_R, 64 fp32 scales


MXFP4_PAGE_BYTES = 25600  # MLA_MXFP4_PAGE_BYTES: 64 x 256 E2M1 code bytes, 64 x 64 bf16 k_R, 64 x 16 E8M0 scales


def is_fp8_cache(kv_cache) -> bool:
    """Whether kv_cache is the 8-bit layout (uint8 [num_pages, 41216])."""
    return kv_cache.dtype == torch.uint8 and kv_cache.dim() == 2 and kv_cache.shape[1] == FP8_PAGE_BYTES


def is_mxfp4_cache(kv_cache) -> bool:
    """Whether kv_cache is the 4-bit layout (uint8 [num_pages, 25600])."""
    return kv_cache.dtype == torch.uint8 and kv_cache.dim() == 2 and kv_cache.shape[1] == MXFP4_PAGE_BYTES


def _need_paged_bytes(kv, name, page_bytes):
    if kv.dim() != 2 or kv.shape[1] != page_bytes:
        raise ValueError(f"{name} must be [num_pages, {page_bytes}] uint8, got {tuple(kv.shape)}")
    _need(kv, name, torch.uint8)


def _need_fp8_cache(kv_fp8, name="kv_fp8"):
    _need_paged_bytes(kv_fp8, name, FP8_PAGE_BYTES)


def _need_mxfp4_cache(kv_fp4, name="kv_fp4"):
    _need_paged_bytes(kv_fp4, name, MXFP4_PAGE_BYTES)


def mla_decode_paged_fp8(q_abs, q_r, kv_fp8, block_table, seqlens, num_splits: int,
                         softmax_scale: float = DEFAULT_SCALE, o_part=None, lse_part=None, stream=None):
    """mla_decode_paged over the 8-bit cache (uint8 [num_pages, 41216]); same outputs."""
    _need_fp8_cache(kv_fp8)
    return _decode_quantized("mla_decode_paged_fp8", q_abs, q_r, kv_fp8, block_table, seqlens, num_splits,
                             softmax_scale, o_part, lse_part, stream)


def mla_decode_paged_mxfp4(q_abs, q_r, kv_fp4, block_table, seqlens, num_splits: int,
                           softmax_scale: float = DEFAULT_SCALE, o_part=None, lse_part=None, stream=None):
    """mla_decode_paged over the 4-bit cache (uint8 [num_pages, 25600]); same outputs."""
    _need_mxfp4_cache(kv_fp4)
    return _decode_quantized("mla_decode_paged_mxfp4", q_abs, q_r, kv_fp4, block_table, seqlens, num_splits,
                             softmax_scale, o_part, lse_part, stream)


def _decode_quantized(fn, q_abs, q_r, kv, block_table, seqlens, num_splits, softmax_scale, o_part, lse_part,
                      stream):
    B, s_q = q_abs.shape[0], q_abs.shape[1]
    _need(q_abs, "q_abs", torch.bfloat16, (B, s_q, H, D_C))
    _need(q_r, "q_r", torch.bfloat16, (B, s_q, H, D_R))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B, max_pages], got {tuple(block_table.shape)}")
    _need(block_table, "block_table", torch.int32)
    _need(seqlens, "seqlens", torch.int32, (B,))
    S = int(num_splits)
    if o_part is None:
        o_part = torch.empty((B, s_q, H, S, D_C), dtype=torch.float32, device=q_abs.device)
    if lse_part is None:
        lse_part = torch.empty((B, s_q, H, S), dtype=torch.float32, device=q_abs.device)
    _need(o_part, "o_part", torch.float32, (B, s_q, H, S, D_C))
    _need(lse_part, "lse_part", torch.float32, (B, s_q, H, S))
    _check(getattr(_lib.LIB, fn)(
        _ptr(q_abs), _ptr(q_r), _ptr(kv), kv.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), B, s_q, H, float(softmax_scale), S, _ptr(o_part), _ptr(lse_part), _stream(stream)), fn)
    return o_part, lse_part


def _quantize_cache(fn, page_bytes, kv_cache, out, stream):
    if kv_cache.dim() != 3 or kv_cache.shape[1:] != (PAGE, ROW):
        raise ValueError(f"kv_cache must be [num_pages, 64, 576], got {tuple(kv_cache.shape)}")
    _need(kv_cache, "kv_cache", torch.bfloat16)
    P = kv_cache.shape[0]
    if out is None:
        out = torch.empty((P, page_bytes), dtype=torch.uint8, device=kv_cache.device)
    _need(out, "out", torch.uint8, (P, page_bytes))
    _check(getattr(_lib.LIB, fn)(_ptr(kv_cache), P, _ptr(out), _stream(stream)), fn)
    return out


def mla_quantize_cache_fp8(kv_cache, out=None, stream=None):
    """bf16 cache [P, 64, 576] -> 8-bit cache uint8 [P, 41216], page for page."""
    return _quantize_cache("mla_quantize_cache_fp8", FP8_PAGE_BYTES, kv_cache, out, stream)


def mla_quantize_cache_mxfp4(kv_cache, out=None, stream=None):
    """bf16 cache [P, 64, 576] -> 4-bit cache uint8 [P, 25600], page for page."""
    return _quantize_cache("mla_quantize_cache_mxfp4", MXFP4_PAGE_BYTES, kv_cache, out, stream)


def mla_combine_splits(o_part, lse_part, o_lat=None, lse=None, stream=None):
    """LSE-weighted merge; returns (o_lat [B,s_q,H,512] fp32, lse [B,s_q,H] fp32)."""
    B, s_q, _, S = lse_part.shape
    _need(o_part, "o_part", torch.float32, (B, s_q, H, S, D_C))
    _need(lse_part, "lse_part", torch.float32, (B, s_q, H, S))
    if o_lat is None:
        o_lat = torch.empty((B, s_q, H, D_C), dtype=torch.float32, device=o_part.device)
    if lse is None:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=o_part.device)
    _need(o_lat, "o_lat", torch.float32, (B, s_q, H, D_C))
    _need(lse, "lse", torch.float32, (B, s_q, H))
    _check(_lib.LIB.mla_combine_splits(_ptr(o_part), _ptr(lse_part), B, s_q, H, S, _ptr(o_lat), _ptr(lse),
                                       _stream(stream)), "mla_combine_splits")
    return o_lat, lse


def mla_combine_up_proj(o_part, lse_part, w_uv, out=None, lse=None, stream=None):
    """Merge + up-projection in one pass; returns (out [B*s_q, H, 128] bf16, lse [B, s_q, H] fp32)."""
    B, s_q, _, S = lse_part.shape
    _need(o_part, "o_part", torch.float32, (B, s_q, H, S, D_C))
    _need(lse_part, "lse_part", torch.float32, (B, s_q, H, S))
    _need(w_uv, "w_uv", torch.bfloat16, (H, D_HC, D_C))
    if out is None:
        out = torch.empty((B * s_q, H, D_HC), dtype=torch.bfloat16, device=o_part.device)
    if lse is None:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=o_part.device)
    _need(out, "out", torch.bfloat16, (B * s_q, H, D_HC))
    _need(lse, "lse", torch.float32, (B, s_q, H))
    _check(_lib.LIB.mla_combine_up_proj(_ptr(o_part), _ptr(lse_part), _ptr(w_uv), B, s_q, H, S, _ptr(out), _ptr(lse),
                                        _stream(stream)), "mla_combine_up_proj")
    return out, lse


def mla_up_proj(o_lat, w_uv, out=None, stream=None):
    """out[..., h, :] = W_UV[h] @ o_lat[..., h, :]; o_lat [..., H, 512] fp32 -> out [..., H, 128] bf16."""
    lead = tuple(o_lat.shape[:-2])
    T = math.prod(lead) if lead else 1
    _need(o_lat, "o_lat", torch.float32, lead + (H, D_C))
    _need(w_uv, "w_uv", torch.bfloat16, (H, D_HC, D_C))
    if out is None:
        out = torch.empty(lead + (H, D_HC), dtype=torch.bfloat16, device=o_lat.device)
    _need(out, "out", torch.bfloat16, lead + (H, D_HC))
    _check(_lib.LIB.mla_up_proj(_ptr(o_lat), _ptr(w_uv), _ptr(out), T, H, _stream(stream)), "mla_up_proj")
    return out


BENCH_SINK_FLOATS = 4096


def _bench_sink(device):
    return torch.empty(BENCH_SINK_FLOATS, dtype=torch.float32, device=device)


def mla_bench_stream_read(buf, sink=None, stream=None):
    """Enqueue one streaming read of every byte of the device tensor buf
    (contiguous, a whole number of 16-byte chunks); returns the bytes read."""
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    sink = _bench_sink(buf.device) if sink is None else sink
    _check(_lib.LIB.mla_bench_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "mla_bench_stream_read")
    return nbytes


def mla_bench_mfma(iters: int, sink=None, stream=None, device="cuda"):
    """Enqueue one dense bf16 MFMA loop (256 x 4 waves, `iters` rounds of four
    32x32x16 MFMAs each); returns its FLOP count."""
    sink = _bench_sink(device) if sink is None else sink
    _check(_lib.LIB.mla_bench_mfma(int(iters), _ptr(sink), _stream(stream)), "mla_bench_mfma")
    return 256 * 4 * 4 * int(iters) * 32768


def mla_debug_gather(kv_cache, block_table, seqlens, max_len: int, out=None, stream=None):
    """Logical rows [B, max_len, 576] gathered through the block table (zeros past L_b)."""
    B = block_table.shape[0]
    _need(kv_cache, "kv_cache", torch.bfloat16)
    _need(block_table, "block_table", torch.int32)
    _need(seqlens, "seqlens", torch.int32, (B,))
    if out is None:
        out = torch.empty((B, max_len, ROW), dtype=torch.bfloat16, device=kv_cache.device)
    _need(out, "out", torch.bfloat16, (B, max_len, ROW))
    _check(_lib.LIB.mla_debug_gather(_ptr(kv_cache), kv_cache.shape[0], _ptr(block_table), block_table.shape[1],
                                     _ptr(seqlens), B, int(max_len), _ptr(out), _stream(stream)),
           "mla_debug_gather")
    return out


ROPE_BASE = 10000.0


def mla_rope_table(max_pos: int, base: float = ROPE_BASE, device=None) -> torch.Tensor:
    """RoPE cos/sin table [max_pos, 32, 2] fp32, built by the library on the host
    (double, rounded to float) and copied to ``device`` (default: the current GPU)."""
    table = torch.empty((int(max_pos), D_R // 2, 2), dtype=torch.float32)
    _check(_lib.LIB.mla_rope_table(float(base), int(max_pos), table.data_ptr()), "mla_rope_table")
    if device is None:
        device = torch.device("cuda", torch.cuda.current_device())
    return table.to(device)


def mla_append_latent(kv_cache, block_table, seqlens, c_new, kr_new, rope, stream=None):
    """Write the chunk's tokens into the cache in place (row L_b - s_q + i of
    sequence b: c_new copied, kr_new rotated by that position); returns kv_cache."""
    B, s_q = c_new.shape[0], c_new.shape[1]
    _need(c_new, "c_new", torch.bfloat16, (B, s_q, D_C))
    _need(kr_new, "kr_new", torch.bfloat16, (B, s_q, D_R))
    if rope.dim() != 3 or rope.shape[1:] != (D_R // 2, 2):
        raise ValueError(f"rope must be [max_pos, 32, 2], got {tuple(rope.shape)}")
    _need(rope, "rope", torch.float32)
    if kv_cache.dim() != 3 or kv_cache.shape[1:] != (PAGE, ROW):
        raise ValueError(f"kv_cache must be [num_pages, 64, 576], got {tuple(kv_cache.shape)}")
    _need(kv_cache, "kv_cache", torch.bfloat16)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B, max_pages], got {tuple(block_table.shape)}")
    _need(block_table, "block_table", torch.int32)
    _need(seqlens, "seqlens", torch.int32, (B,))
    _check(_lib.LIB.mla_append_latent(_ptr(c_new), _ptr(kr_new), _ptr(rope), rope.shape[0], _ptr(kv_cache),
                                      kv_cache.shape[0], _ptr(block_table), block_table.shape[1], _ptr(seqlens),
                                      B, s_q, _stream(stream)), "mla_append_latent")
    return kv_cache


def mla_append_latent_fp8(kv_fp8, block_table, seqlens, c_new, kr_new, rope, stream=None):
    """mla_append_latent into the 8-bit cache (c_new quantized per token, kr_new
    rotated); returns kv_fp8."""
    _need_fp8_cache(kv_fp8)
    return _append_quantized("mla_append_latent_fp8", kv_fp8, block_table, seqlens, c_new, kr_new, rope, stream)


def mla_append_latent_mxfp4(kv_fp4, block_table, seqlens, c_new, kr_new, rope, stream=None):
    """mla_append_latent into the 4-bit cache (c_new quantized per 32-dim block,
    kr_new rotated); returns kv_fp4."""
    _need_mxfp4_cache(kv_fp4)
    return _append_quantized("mla_append_latent_mxfp4", kv_fp4, block_table, seqlens, c_new, kr_new, rope, stream)


def _append_quantized(fn, kv, block_table, seqlens, c_new, kr_new, rope, stream):
    B, s_q = c_new.shape[0], c_new.shape[1]
    _need(c_new, "c_new", torch.bfloat16, (B, s_q, D_C))
    _need(kr_new, "kr_new", torch.bfloat16, (B, s_q, D_R))
    if rope.dim() != 3 or rope.shape[1:] != (D_R // 2, 2):
        raise ValueError(f"rope must be [max_pos, 32, 2], got {tuple(rope.shape)}")
    _need(rope, "rope", torch.float32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B, max_pages], got {tuple(block_table.shape)}")
    _need(block_table, "block_table", torch.int32)
    _need(seqlens, "seqlens", torch.int32, (B,))
    _check(getattr(_lib.LIB, fn)(_ptr(c_new), _ptr(kr_new), _ptr(rope), rope.shape[0], _ptr(kv),
                                 kv.shape[0], _ptr(block_table), block_table.shape[1], _ptr(seqlens),
                                 B, s_q, _stream(stream)), fn)
    return kv


def mla_rope_q(q_r, seqlens, rope, stream=None):
    """Rotate q_r [B, s_q, H, 64] in place by each chunk token's position; returns q_r."""
    B, s_q = q_r.shape[0], q_r.shape[1]
    _need(q_r, "q_r", torch.bfloat16, (B, s_q, H, D_R))
    if rope.dim() != 3 or rope.shape[1:] != (D_R // 2, 2):
        raise ValueError(f"rope must be [max_pos, 32, 2], got {tuple(rope.shape)}")
    _need(rope, "rope", torch.float32)
    _need(seqlens, "seqlens", torch.int32, (B,))
    _check(_lib.LIB.mla_rope_q(_ptr(q_r), _ptr(rope), rope.shape[0], _ptr(seqlens), B, s_q, H, _stream(stream)),
           "mla_rope_q")
    return q_r


def mla_prefill_uses_absorption(s_q: int) -> bool:
    """Whether an s_q-token chunk takes the absorbed path (s_q <= 256)."""
    return bool(_lib.LIB.mla_prefill_uses_absorption(int(s_q)))


def _cache_args(kv_cache, block_table, seqlens, B):
    if kv_cache.dim() != 3 or kv_cache.shape[1:] != (PAGE, ROW):
        raise ValueError(f"kv_cache must be [num_pages, 64, 576], got {tuple(kv_cache.shape)}")
    _need(kv_cache, "kv_cache", torch.bfloat16)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B, max_pages], got {tuple(block_table.shape)}")
    _need(block_table, "block_table", torch.int32)
    _need(seqlens, "seqlens", torch.int32, (B,))


def mla_decompress_kv(kv_cache, block_table, seqlens, w_uk, w_uv, max_len: int, k_nope=None, v=None, stream=None):
    """Per-head keys (bf16) and values (fp16) [B, H, max_len, 128] of every
    cached token (rows past a sequence's length are left as they were)."""
    B = block_table.shape[0]
    _cache_args(kv_cache, block_table, seqlens, B)
    _need(w_uk, "w_uk", torch.bfloat16, (H, D_HC, D_C))
    _need(w_uv, "w_uv", torch.bfloat16, (H, D_HC, D_C))
    shape = (B, H, int(max_len), D_HC)
    if k_nope is None:
        k_nope = torch.empty(shape, dtype=torch.bfloat16, device=kv_cache.device)
    if v is None:
        v = torch.empty(shape, dtype=torch.float16, device=kv_cache.device)
    _need(k_nope, "k_nope", torch.bfloat16, shape)
    _need(v, "v", torch.float16, shape)
    _check(_lib.LIB.mla_decompress_kv(_ptr(kv_cache), kv_cache.shape[0], _ptr(block_table), block_table.shape[1],
                                      _ptr(seqlens), B, int(max_len), _ptr(w_uk), _ptr(w_uv), _ptr(k_nope), _ptr(v),
                                      _stream(stream)), "mla_decompress_kv")
    return k_nope, v


def mla_prefill_mha(q_c, q_r, k_nope, v, kv_cache, block_table, seqlens, softmax_scale: float = DEFAULT_SCALE,
                    out=None, lse=None, stream=None):
    """Causal attention over decompressed K/V; returns (out [B,s_q,H,128] bf16, lse [B,s_q,H] fp32)."""
    B, s_q = q_c.shape[0], q_c.shape[1]
    _need(q_c, "q_c", torch.bfloat16, (B, s_q, H, D_HC))
    _need(q_r, "q_r", torch.bfloat16, (B, s_q, H, D_R))
    max_len = k_nope.shape[2]
    _need(k_nope, "k_nope", torch.bfloat16, (B, H, max_len, D_HC))
    _need(v, "v", torch.float16, (B, H, max_len, D_HC))
    _cache_args(kv_cache, block_table, seqlens, B)
    if out is None:
        out = torch.empty((B, s_q, H, D_HC), dtype=torch.bfloat16, device=q_c.device)
    if lse is None:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=q_c.device)
    _need(out, "out", torch.bfloat16, (B, s_q, H, D_HC))
    _need(lse, "lse", torch.float32, (B, s_q, H))
    _check(_lib.LIB.mla_prefill_mha(_ptr(q_c), _ptr(q_r), _ptr(k_nope), _ptr(v), max_len, _ptr(kv_cache),
                                    kv_cache.shape[0], _ptr(block_table), block_table.shape[1], _ptr(seqlens), B, s_q,
                                    H, float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)), "mla_prefill_mha")
    return out, lse


def decode_layer(q_c, q_r, kv_cache, block_table, seqlens, w_uk, w_uv, num_splits: int | None = None,
                 softmax_scale: float = DEFAULT_SCALE, max_len: int | None = None, stream=None):
    """The whole hot path for one layer: absorb -> split scan -> combine -> up-projection.

    Returns a dict with every intermediate (q_abs, o_part, lse_part, o_lat, lse, out).
    ``max_len`` (longest sequence, host int) only feeds the split heuristic.
    ``kv_cache`` is the bf16 cache [P, 64, 576], the 8-bit one (uint8 [P, 41216]) or
    the 4-bit one (uint8 [P, 25600]).
    """
    B, s_q = q_c.shape[0], q_c.shape[1]
    if num_splits is None:
        ml = int(max_len) if max_len is not None else block_table.shape[1] * PAGE
        num_splits = mla_recommended_splits(B, s_q, ml)
    q_abs = mla_absorb_q(q_c, w_uk, stream=stream)
    scan = (mla_decode_paged_fp8 if is_fp8_cache(kv_cache) else
            mla_decode_paged_mxfp4 if is_mxfp4_cache(kv_cache) else mla_decode_paged)
    o_part, lse_part = scan(q_abs, q_r, kv_cache, block_table, seqlens, num_splits, softmax_scale, stream=stream)
    o_lat, lse = mla_combine_splits(o_part, lse_part, stream=stream)
    out = mla_up_proj(o_lat, w_uv, stream=stream)
    return dict(q_abs=q_abs, o_part=o_part, lse_part=lse_part, o_lat=o_lat, lse=lse, out=out)


def mla_decode_step(q_c, q_r, kv_cache, block_table, seqlens, w_uk, w_uv, num_splits: int,
                    softmax_scale: float = DEFAULT_SCALE, buffers: dict | None = None, stream=None):
    """The whole absorbed step in one launch (absorb -> scan -> merge -> up-projection),
    bit-identical to decode_layer; kv_cache is the bf16, the 8-bit or the 4-bit cache.
    Returns dict(q_abs, o_part, lse_part, o_lat, lse, out); ``buffers`` may
    supply any of them preallocated."""
    B, s_q = q_c.shape[0], q_c.shape[1]
    S = int(num_splits)
    dev = q_c.device
    shapes = dict(q_abs=((B, s_q, H, D_C), torch.bfloat16), o_part=((B, s_q, H, S, D_C), torch.float32),
                  lse_part=((B, s_q, H, S), torch.float32), o_lat=((B, s_q, H, D_C), torch.float32),
                  lse=((B, s_q, H), torch.float32), out=((B, s_q, H, D_HC), torch.bfloat16))
    buf = dict(buffers or {})
    for k, (shape, dt) in shapes.items():
        if k not in buf:
            buf[k] = torch.empty(shape, dtype=dt, device=dev)
        _need(buf[k], k, dt, shape)
    _need(q_c, "q_c", torch.bfloat16, (B, s_q, H, D_HC))
    _need(q_r, "q_r", torch.bfloat16, (B, s_q, H, D_R))
    _need(w_uk, "w_uk", torch.bfloat16, (H, D_HC, D_C))
    _need(w_uv, "w_uv", torch.bfloat16, (H, D_HC, D_C))
    if is_fp8_cache(kv_cache):
        fn = "mla_decode_step_fp8"
        _need_fp8_cache(kv_cache, "kv_cache")
    elif is_mxfp4_cache(kv_cache):
        fn = "mla_decode_step_mxfp4"
        _need_mxfp4_cache(kv_cache, "kv_cache")
    else:
        fn = "mla_decode_step"
        if kv_cache.dim() != 3 or kv_cache.shape[1:] != (PAGE, ROW):
            raise ValueError(f"kv_cache must be [num_pages, 64, 576], got {tuple(kv_cache.shape)}")
        _need(kv_cache, "kv_cache", torch.bfloat16)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table must be [B, max_pages], got {tuple(block_table.shape)}")
    _need(block_table, "block_table", torch.int32)
    _need(seqlens, "seqlens", torch.int32, (B,))
    _check(getattr(_lib.LIB, fn)(
        _ptr(q_c), _ptr(q_r), _ptr(kv_cache), kv_cache.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(seqlens), B, s_q, H, _ptr(w_uk), _ptr(w_uv), float(softmax_scale), S, _ptr(buf["q_abs"]),
        _ptr(buf["o_part"]), _ptr(buf["lse_part"]), _ptr(buf["o_lat"]), _ptr(buf["out"]), _ptr(buf["lse"]),
        _stream(stream)), fn)
    return buf


STATIC_SCRATCH_BYTES = 96 * 1024 * 1024


def mla_decode_step_static(q_c, q_r, kv_cache, block_table, seqlens, w_uk, w_uv, num_splits: int,
                           softmax_scale: float = DEFAULT_SCALE, out=None, lse=None, stream=None):
    """The decode step with no caller workspace (bf16 cache): q_abs and the
    split partials live in the library's static device array. Returns
    (out [B*s_q, H, 128] bf16, lse [B, s_q, H] fp32); allocates them through
    torch only when they are not given."""
    B, s_q = q_c.shape[0], q_c.shape[1]
    _need(q_c, "q_c", torch.bfloat16, (B, s_q, H, D_HC))
    _need(q_r, "q_r", torch.bfloat16, (B, s_q, H, D_R))
    _need(w_uk, "w_uk", torch.bfloat16, (H, D_HC, D_C))
    _need(w_uv, "w_uv", torch.bfloat16, (H, D_HC, D_C))
    _need(kv_cache, "kv_cache", torch.bfloat16)
    if kv_cache.dim() != 3 or kv_cache.shape[1:] != (PAGE, ROW):
        raise ValueError(f"kv_cache must be [P, {PAGE}, {ROW}], got {tuple(kv_cache.shape)}")
    _need(block_table, "block_table", torch.int32)
    _need(seqlens, "seqlens", torch.int32, (B,))
    if out is None:
        out = torch.empty((B * s_q, H, D_HC), dtype=torch.bfloat16, device=q_c.device)
    if lse is None:
        lse = torch.empty((B, s_q, H), dtype=torch.float32, device=q_c.device)
    _need(out, "out", torch.bfloat16, (B * s_q, H, D_HC))
    _need(lse, "lse", torch.float32, (B, s_q, H))
    _check(_lib.LIB.mla_decode_step_static(_ptr(q_c), _ptr(q_r), _ptr(kv_cache), kv_cache.shape[0],
                                           _ptr(block_table), block_table.shape[1], _ptr(seqlens), B, s_q, H,
                                           _ptr(w_uk), _ptr(w_uv), float(softmax_scale), int(num_splits), _ptr(out),
                                           _ptr(lse), _stream(stream)), "mla_decode_step_static")
    return out, lse


def attention_layer(q_c, q_r, kv_cache, block_table, seqlens, w_uk, w_uv, max_len: int,
                    softmax_scale: float = DEFAULT_SCALE, num_splits: int | None = None, absorbed: bool | None = None,
                    stream=None):
    """One MLA attention layer for a chunk of s_q new tokens per sequence,
    dispatched as the teardown page does (section 3): the absorbed path
    (decode_layer) for s_q <= 256, the decompressed branch (mla_decompress_kv,
    then mla_prefill_mha) above. ``absorbed`` forces a path; ``max_len`` is the
    longest sequence (host int). Returns a dict with ``path``, ``out``
    [B, s_q, H, 128] bf16 and ``lse`` [B, s_q, H] fp32 plus the intermediates."""
    B, s_q = q_c.shape[0], q_c.shape[1]
    use_absorbed = mla_prefill_uses_absorption(s_q) if absorbed is None else bool(absorbed)
    if use_absorbed:
        r = decode_layer(q_c, q_r, kv_cache, block_table, seqlens, w_uk, w_uv, num_splits, softmax_scale,
                         max_len, stream)
        r["path"] = "absorbed"
        return r
    if kv_cache.dtype == torch.uint8:
        raise ValueError("the decompressed branch reads the bf16 cache; the quantized caches serve the absorbed path")
    ml = -(-int(max_len) // PAGE) * PAGE
    k_nope, v = mla_decompress_kv(kv_cache, block_table, seqlens, w_uk, w_uv, ml, stream=stream)
    out, lse = mla_prefill_mha(q_c, q_r, k_nope, v, kv_cache, block_table, seqlens, softmax_scale, stream=stream)
    return dict(path="decompressed", k_nope=k_nope, v=v, out=out, lse=lse)
