"""The C ABI on the CPU: the library loads, exports what include/mla.h
declares, the header is valid C99, and host-side validation rejects bad
arguments before any launch (these calls never reach the GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from mla_latent_kv_06_amd import _lib
    return _lib.LIB


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) == 31, names
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "mla_latent_kv_06_amd", "libmla.so")],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mla_[a-z0-9_]+)\b", out))
    assert set(names) <= exported, set(names) - exported
    for n in names:
        assert getattr(lib, n) is not None


def test_header_is_c99():
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER], check=True)


def test_status_strings(lib):
    assert lib.mla_status_string(0) == b"MLA_OK"
    assert lib.mla_status_string(4) == b"MLA_ERR_WORKSPACE"
    assert lib.mla_status_string(99) == b"MLA_ERR_UNKNOWN"


A = 1 << 20  # an aligned, never-dereferenced fake address
MIS = A + 8


def _decode(lib, fn="mla_decode_paged", **kw):
    a = dict(q_abs=A, q_r=A, kv=A, num_pages=10, bt=A, max_pages=4, seqlens=A, B=2, s_q=1, H=128,
             scale=0.07, S=2, o_part=A, lse_part=A)
    a.update(kw)
    return getattr(lib, fn)(a["q_abs"], a["q_r"], a["kv"], a["num_pages"], a["bt"], a["max_pages"],
                                a["seqlens"], a["B"], a["s_q"], a["H"], a["scale"], a["S"], a["o_part"],
                                a["lse_part"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q_abs=None), 1), (dict(lse_part=None), 1), (dict(kv=MIS), 3), (dict(o_part=MIS), 3),
    (dict(H=64), 2), (dict(B=0), 2), (dict(s_q=0), 2), (dict(s_q=5000), 2), (dict(S=0), 2),
    (dict(S=5), 2), (dict(max_pages=0), 2), (dict(num_pages=0), 2), (dict(scale=float("nan")), 2),
    (dict(scale=float("inf")), 2), (dict(scale=0.0), 2), (dict(scale=-0.5), 2),
])
@pytest.mark.parametrize("fn", ["mla_decode_paged", "mla_decode_paged_fp8", "mla_decode_paged_mxfp4"])
def test_decode_validation(lib, kw, status, fn):
    assert _decode(lib, fn, **kw) == status
    assert lib.mla_last_error() != b""


def test_other_entry_validation(lib):
    assert lib.mla_absorb_q(None, A, A, 4, 128, None) == 1
    assert lib.mla_absorb_q(A, A, A, 0, 128, None) == 2
    assert lib.mla_absorb_q(A, MIS, A, 4, 128, None) == 3
    assert lib.mla_up_proj(A, A, A, 4, 127, None) == 2
    assert lib.mla_combine_splits(A, A, 1, 1, 128, 0, A, A, None) == 2
    assert lib.mla_combine_splits(A, A, 1, 1, 128, 2, MIS, A, None) == 3
    assert lib.mla_debug_gather(A, 3, A, 1, A, 1, 0, A, None) == 2
    # cache append: c_new, kr_new, rope, max_pos, kv, num_pages, bt, max_pages, seqlens, B, s_q
    assert lib.mla_append_latent(None, A, A, 64, A, 4, A, 2, A, 2, 1, None) == 1
    assert lib.mla_append_latent(A, A, None, 64, A, 4, A, 2, A, 2, 1, None) == 1
    assert lib.mla_append_latent(A, MIS, A, 64, A, 4, A, 2, A, 2, 1, None) == 3
    assert lib.mla_append_latent(A, A, A, 0, A, 4, A, 2, A, 2, 1, None) == 2
    assert lib.mla_append_latent(A, A, A, 64, A, 0, A, 2, A, 2, 1, None) == 2
    assert lib.mla_append_latent(A, A, A, 64, A, 4, A, 2, A, 2, 0, None) == 2
    assert lib.mla_append_latent(A, A, A, 64, A, 4, A, 2, A, 2, 5000, None) == 2
    # the same rules for the 8-bit append
    assert lib.mla_append_latent_fp8(None, A, A, 64, A, 4, A, 2, A, 2, 1, None) == 1
    assert lib.mla_append_latent_fp8(A, A, A, 64, MIS, 4, A, 2, A, 2, 1, None) == 3
    assert lib.mla_append_latent_fp8(A, A, A, 64, A, 4, A, 2, A, 2, 5000, None) == 2
    assert lib.mla_append_latent_mxfp4(None, A, A, 64, A, 4, A, 2, A, 2, 1, None) == 1
    assert lib.mla_append_latent_mxfp4(A, A, A, 64, MIS, 4, A, 2, A, 2, 1, None) == 3
    assert lib.mla_append_latent_mxfp4(A, A, A, 64, A, 4, A, 2, A, 2, 5000, None) == 2
    # one-launch step: q_c, q_r, kv, num_pages, bt, max_pages, seqlens, B, s_q, H, w_uk, w_uv, scale, S,
    # q_abs, o_part, lse_part, o_lat, out, lse
    for fn in (lib.mla_decode_step, lib.mla_decode_step_fp8, lib.mla_decode_step_mxfp4):
        assert fn(None, A, A, 10, A, 4, A, 2, 1, 128, A, A, 0.07, 2, A, A, A, A, A, A, None) == 1
        assert fn(A, A, A, 10, A, 4, A, 2, 1, 128, A, None, 0.07, 2, A, A, A, A, A, A, None) == 1
        assert fn(A, A, A, 10, A, 4, A, 2, 1, 128, A, A, 0.07, 2, A, A, A, MIS, A, A, None) == 3
        assert fn(A, A, A, 10, A, 4, A, 2, 1, 64, A, A, 0.07, 2, A, A, A, A, A, A, None) == 2
        assert fn(A, A, A, 10, A, 4, A, 2, 1, 128, A, A, 0.07, 5, A, A, A, A, A, A, None) == 2
        assert fn(A, A, A, 10, A, 4, A, 1 << 20, 2, 128, A, A, 0.07, 2, A, A, A, A, A, A, None) == 2
    # cache conversion: kv, num_pages, kv_fp8
    assert lib.mla_quantize_cache_fp8(None, 4, A, None) == 1
    assert lib.mla_quantize_cache_fp8(A, 4, MIS, None) == 3
    assert lib.mla_quantize_cache_fp8(A, 0, A, None) == 2
    assert lib.mla_quantize_cache_fp8(A, (1 << 26) + 1, A, None) == 2
    assert lib.mla_quantize_cache_mxfp4(None, 4, A, None) == 1
    assert lib.mla_quantize_cache_mxfp4(A, 4, MIS, None) == 3
    assert lib.mla_quantize_cache_mxfp4(A, 0, A, None) == 2
    assert lib.mla_quantize_cache_mxfp4(A, (1 << 26) + 1, A, None) == 2
    # query rotation: q_r, rope, max_pos, seqlens, B, s_q, H
    assert lib.mla_rope_q(None, A, 64, A, 2, 1, 128, None) == 1
    assert lib.mla_rope_q(A, A, 64, MIS, 2, 1, 128, None) == 3
    assert lib.mla_rope_q(A, A, 64, A, 2, 1, 64, None) == 2
    assert lib.mla_rope_q(A, A, 0, A, 2, 1, 128, None) == 2
    assert lib.mla_rope_q(A, A, 64, A, 1 << 20, 4, 128, None) == 2   # B * s_q > 2^21
    # decompressed branch: kv, num_pages, bt, max_pages, seqlens, B, max_len, w_uk, w_uv, k, v
    assert lib.mla_decompress_kv(A, 4, A, 2, A, 2, 128, None, A, A, A, None) == 1
    assert lib.mla_decompress_kv(A, 4, A, 2, A, 2, 100, A, A, A, A, None) == 2     # not a multiple of 64
    assert lib.mla_decompress_kv(A, 4, A, 2, A, 0, 128, A, A, A, A, None) == 2
    assert lib.mla_decompress_kv(A, 4, A, 2, A, 2, 128, A, A, MIS, A, None) == 3
    # q_c, q_r, k, v, max_len, kv, num_pages, bt, max_pages, seqlens, B, s_q, H, scale, out, lse
    assert lib.mla_prefill_mha(A, A, None, A, 128, A, 4, A, 2, A, 2, 300, 128, 0.07, A, A, None) == 1
    assert lib.mla_prefill_mha(A, A, A, A, 96, A, 4, A, 2, A, 2, 300, 128, 0.07, A, A, None) == 2
    assert lib.mla_prefill_mha(A, A, A, A, 128, A, 4, A, 2, A, 2, 300, 64, 0.07, A, A, None) == 2
    assert lib.mla_prefill_mha(A, A, A, A, 128, A, 4, A, 2, A, 2, 300, 128, 0.0, A, A, None) == 2
    assert lib.mla_prefill_mha(A, A, A, A, 128, A, 4, A, 2, A, 2, 0, 128, 0.07, A, A, None) == 2


def test_measurement_aid_validation(lib):
    # mla_bench_stream_read(buf, bytes, sink, stream), mla_bench_mfma(iters, sink, stream):
    # every rejection happens on the host, before any launch
    assert lib.mla_bench_stream_read(None, 1024, A, None) == 1
    assert lib.mla_bench_stream_read(A, 1024, None, None) == 1
    assert lib.mla_bench_stream_read(MIS, 1024, A, None) == 3
    assert lib.mla_bench_stream_read(A, 1024, MIS, None) == 3
    assert lib.mla_bench_stream_read(A, 0, A, None) == 2
    assert lib.mla_bench_stream_read(A, 1000, A, None) == 2
    assert b"multiple of 16" in lib.mla_last_error()
    assert lib.mla_bench_mfma(0, A, None) == 2
    assert lib.mla_bench_mfma(-5, A, None) == 2
    assert lib.mla_bench_mfma(10, None, None) == 1


def test_host_helpers(lib):
    assert lib.mla_decode_workspace_bytes(16, 1, 128, 16) == 16 * 128 * 16 * 513 * 4
    assert lib.mla_decode_workspace_bytes(0, 1, 128, 16) == 0
    # time model of the balanced scan: more splits for a single short sequence,
    # few for a batch that fills the GPU
    assert lib.mla_recommended_splits(1, 1, 2048, 256) == 32
    assert lib.mla_recommended_splits(4, 256, 16640, 256) in (1, 2)
    assert lib.mla_recommended_splits(16, 1, 4096, 256) in (8, 9, 11)


def test_prefill_dispatch_and_sizes(lib):
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "teardown_dispatch.json")))
    thr = g["kPrefillThresh"]
    assert lib.mla_prefill_uses_absorption(1) == 1
    assert lib.mla_prefill_uses_absorption(thr) == 1
    assert lib.mla_prefill_uses_absorption(thr + 1) == 0
    assert lib.mla_decompressed_kv_bytes(4, 16640) == 4 * 128 * 16640 * 128 * 2
    assert lib.mla_decompressed_kv_bytes(0, 64) == 0


def test_rope_table_host(lib):
    """The library's host table against the oracle's fp64 angles rounded to fp32."""
    import numpy as np
    import oracle as O
    n = 70000
    tab = np.zeros((n, 32, 2), np.float32)
    assert lib.mla_rope_table(10000.0, n, tab.ctypes.data) == 0
    a = O.rope_angles(np.arange(n), 64)
    ref = np.stack([np.cos(a), np.sin(a)], axis=-1)
    # rounding to float costs at most 2^-25 for values of magnitude <= 1; the
    # two sides form the angle with different pow routines (fp64 ulps of an
    # angle up to 7e4 rad), far below that
    assert np.abs(tab.astype(np.float64) - ref).max() <= 2.0 ** -24
    assert (tab[0, :, 0] == 1).all() and (tab[0, :, 1] == 0).all()
    assert lib.mla_rope_table(10000.0, 4, None) == 1
    assert lib.mla_rope_table(0.0, 4, tab.ctypes.data) == 2
    assert lib.mla_rope_table(float("inf"), 4, tab.ctypes.data) == 2
    assert lib.mla_rope_table(10000.0, 0, tab.ctypes.data) == 2
    assert lib.mla_rope_table(10000.0, (1 << 22) + 1, tab.ctypes.data) == 2


def test_plan_splits(lib):
    import ctypes
    from mla_inputs import CONFIGS, make_structure

    def plan(lens, width, s_q=1):
        arr = (ctypes.c_int32 * len(lens))(*lens)
        return lib.mla_plan_splits(ctypes.cast(arr, ctypes.c_void_p), len(lens), s_q, width, 256)
    # equal lengths: the same choice as the max-length model
    for B, L in [(16, 65536), (16, 4096), (1, 2048)]:
        assert plan([L] * B, -(-L // 64)) == lib.mla_recommended_splits(B, 1, L, 256)
    # 16 x 1024 pages: ranges of exactly 64 pages need S >= 17 (any row alignment)
    assert lib.mla_recommended_splits(16, 1, 65536, 256) == 17
    assert plan([16640] * 4, 260, s_q=256) in (1, 2)
    # a ragged batch: the chosen plan's ranges stay close to the balanced width
    st = make_structure(CONFIGS["ragged"], 42)
    lens = [int(x) for x in st.seqlens]
    S = plan(lens, st.block_table.shape[1])
    pages = [-(-L // 64) for L in lens]
    p_tot = sum(pages)
    W = max(-(-p_tot // 256), -(-(max(pages) - 1) // (S - 1)) if S > 1 else 0)
    assert S > 1 and W <= 1.25 * -(-p_tot // 256), (S, W)
    # degenerate inputs
    assert lib.mla_plan_splits(None, 4, 1, 8, 256) == 1
    assert plan([0, 0], 4) == 1


def test_validate_block_table(lib):
    """The host check of the block-table contract: first bad (sequence, page)
    in order, lengths past the table, -1 tails ignored (teardown page,
    section 5: the gather's address faults)."""
    import numpy as np

    def run(bt, lens, num_pages):
        bt = np.ascontiguousarray(bt, np.int32)
        lens = np.ascontiguousarray(lens, np.int32)
        bs, bp = ctypes.c_int(7), ctypes.c_int(7)
        st = lib.mla_validate_block_table(bt.ctypes.data, bt.shape[1], lens.ctypes.data, len(lens), num_pages,
                                          ctypes.addressof(bs), ctypes.addressof(bp))
        return st, bs.value, bp.value

    bt = [[3, 0, -1, -1], [1, 2, 4, -5]]
    assert run(bt, [65, 130], 5) == (0, -1, -1)          # tails past ceil(L/64) are not read
    assert run(bt, [0, 1], 5) == (0, -1, -1)
    assert run(bt, [129, 10], 5) == (2, 0, 2)            # sequence 0 needs page 2 (-1)
    assert b"block_table[0, 2] = -1" in lib.mla_last_error()
    assert run(bt, [65, 130], 4) == (2, 1, 2)            # entry 4 outside [0, 4)
    assert run(bt, [65, 257], 5) == (2, 1, -1)           # length past max_pages * 64
    assert run(bt, [-1, 3], 5) == (2, 0, -1)
    assert run(bt, [65, 130], 0)[0] == 2
    assert lib.mla_validate_block_table(None, 4, A, 1, 5, None, None) == 1
    assert lib.mla_validate_block_table(A, 4, None, 1, 5, None, None) == 1
    # NULL out-pointers are allowed
    arr = np.zeros((1, 1), np.int32)
    ln = np.array([64], np.int32)
    assert lib.mla_validate_block_table(arr.ctypes.data, 1, ln.ctypes.data, 1, 1, None, None) == 0


def test_static_step_validation(lib):
    """mla_decode_step_static rejects bad arguments, and requests whose scratch
    layout exceeds the static array, on the host before any HIP call."""
    def call(B=2, s_q=1, S=2, q_c=A, out=A, num_pages=10, max_pages=4):
        return lib.mla_decode_step_static(q_c, A, A, num_pages, A, max_pages, A, B, s_q, 128, A, A, 0.07, S, out,
                                          A, None)
    assert call(q_c=None) == 1
    assert call(out=MIS) == 3
    assert call(S=5) == 2
    # 16 x 128 rows with 64 splits: 2 MiB + 64 x 4 MiB of partials > 96 MiB
    assert call(B=16, S=64, max_pages=1024) == 4
    assert b"scratch" in lib.mla_last_error()
