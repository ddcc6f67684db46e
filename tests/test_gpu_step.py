"""GPU: the one-launch step (mla_decode_step over the bf16, 8-bit and 4-bit caches) against the
same four kernels launched one after another (bit for bit: every phase runs
the kernel's own workgroup body), and against the fp64 oracle."""
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


def _case(lens, s_q, seed, fmt="bf16"):
    g = torch.Generator().manual_seed(seed)
    need = [-(-int(L) // 64) for L in lens]
    pool = sum(need) + 3
    order = torch.randperm(pool, generator=g)
    bt = torch.full((len(lens), max(max(need), 1) + 1), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[off:off + n].to(torch.int32)
        off += n
    B = len(lens)
    q_c = torch.randn((B, s_q, 128, 128), generator=g).to(torch.bfloat16)
    q_r = torch.randn((B, s_q, 128, 64), generator=g).to(torch.bfloat16)
    kv = torch.randn((pool, 64, 576), generator=g).to(torch.bfloat16)
    w_uk = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    w_uv = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    cache = {"bf16": lambda: kv, "fp8": lambda: torch.from_numpy(O.pack_fp8_cache(O.bf16_bits(kv))),
             "mxfp4": lambda: torch.from_numpy(O.pack_mxfp4_cache(O.bf16_bits(kv)))}[fmt]()
    return dict(q_c=q_c, q_r=q_r, kv=cache, bt=bt, sl=torch.tensor(lens, dtype=torch.int32), w_uk=w_uk, w_uv=w_uv)


def _sequence(M, d, S):
    """absorb -> scan -> merge -> up-projection as four launches."""
    q_abs = M.mla_absorb_q(d["q_c"], d["w_uk"])
    scan = (M.mla_decode_paged_fp8 if M.is_fp8_cache(d["kv"]) else
            M.mla_decode_paged_mxfp4 if M.is_mxfp4_cache(d["kv"]) else M.mla_decode_paged)
    o_part, lse_part = scan(q_abs, d["q_r"], d["kv"], d["bt"], d["sl"], S, SCALE)
    o_lat, lse = M.mla_combine_splits(o_part, lse_part)
    out = M.mla_up_proj(o_lat, d["w_uv"])
    return dict(q_abs=q_abs, o_part=o_part, lse_part=lse_part, o_lat=o_lat, lse=lse, out=out)


@pytest.mark.parametrize("lens,s_q,S,fmt", [
    ([2048], 1, 32, "bf16"),               # one short sequence, many splits
    ([700] * 16, 1, 9, "bf16"),            # a batch of short sequences
    ([1, 130, 2047, 0, 64], 1, 5, "bf16"),  # ragged, with an empty row
    ([300, 77], 3, 3, "bf16"),             # causal chunk
    ([2048], 1, 32, "fp8"),                # the 8-bit cache
    ([700] * 16, 1, 9, "fp8"),
    ([2048], 1, 32, "mxfp4"),              # the 4-bit cache
    ([1, 130, 2047, 0, 64], 1, 5, "mxfp4"),
    ([300, 77], 3, 3, "mxfp4"),
])
def test_step_is_bit_identical_to_the_kernel_sequence(M, lens, s_q, S, fmt):
    c = _case(lens, s_q, seed=len(lens) * 7 + s_q + S, fmt=fmt)
    d = {k: v.to(DEV) for k, v in c.items()}
    _say(f"step lens={lens[:6]} s_q={s_q} S={S} cache={fmt}")
    ref = _sequence(M, d, S)
    got = M.mla_decode_step(d["q_c"], d["q_r"], d["kv"], d["bt"], d["sl"], d["w_uk"], d["w_uv"], S, SCALE)
    torch.cuda.synchronize()
    live = torch.isfinite(ref["lse_part"])
    for k in ("q_abs", "lse_part", "o_lat", "lse"):
        assert torch.equal(got[k], ref[k]), f"{k} differs"
    assert torch.equal(got["o_part"][live], ref["o_part"][live]), "o_part differs"
    assert torch.equal(got["out"].view(-1), ref["out"].reshape(-1)), "out differs"


def test_step_against_the_oracle(M):
    """Each phase on the exact inputs it received (the step writes q_abs and
    o_lat), with the per-entry-point bars; end to end against the fp64 naive
    path with the chain bar (the bf16 rounding of q_abs at the boundary adds
    error the fp64 chain does not have)."""
    c = _case([333, 2048, 64], 2, seed=41)
    d = {k: v.to(DEV) for k, v in c.items()}
    _say("step vs fp64 oracle")
    r = M.mla_decode_step(d["q_c"], d["q_r"], d["kv"], d["bt"], d["sl"], d["w_uk"], d["w_uv"], 7, SCALE)
    torch.cuda.synchronize()
    f = {k: O.as_f64(c[k]) for k in ("q_c", "q_r", "w_uk", "w_uv")}
    kvb, bt, sl = O.bf16_bits(c["kv"]), c["bt"].numpy(), c["sl"].numpy()
    q_abs = O.as_f64(r["q_abs"].cpu())
    assert_bar(q_abs, O.absorb(f["q_c"], f["w_uk"]), "step absorb")
    ref_o, ref_l = O.decode_absorbed(q_abs, f["q_r"], kvb, bt, sl, SCALE)
    assert_bar(r["o_lat"].cpu().numpy(), ref_o, "step o_lat")
    assert_lse(r["lse"].cpu().numpy(), ref_l, "step lse")
    assert_bar(O.as_f64(r["out"].cpu()), O.up_proj(r["o_lat"].cpu().double().numpy(), f["w_uv"]), "step up_proj")
    nv_o, nv_l = O.decode_naive(f["q_c"], f["q_r"], kvb, bt, sl, f["w_uk"], f["w_uv"], SCALE)
    assert_bar(O.as_f64(r["out"].cpu()), nv_o, "step end-to-end", l1_rel=5e-3)
    assert_lse(r["lse"].cpu().numpy(), nv_l, "step end-to-end lse", tol=5e-3)


def test_step_twice_in_a_row_with_a_smaller_batch(M):
    """Back-to-back launches with different sizes reuse nothing stale."""
    for lens, S in (([1500, 900, 64, 3], 6), ([200], 4)):
        c = _case(lens, 1, seed=len(lens))
        d = {k: v.to(DEV) for k, v in c.items()}
        _say(f"step lens={lens}")
        ref = _sequence(M, d, S)
        got = M.mla_decode_step(d["q_c"], d["q_r"], d["kv"], d["bt"], d["sl"], d["w_uk"], d["w_uv"], S, SCALE)
        torch.cuda.synchronize()
        assert torch.equal(got["out"].view(-1), ref["out"].reshape(-1))
        assert torch.equal(got["lse"], ref["lse"])
