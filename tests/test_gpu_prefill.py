"""GPU parity of the decompressed branch for long chunks (per-head K/V, then
causal multi-head attention) and of the absorbed/decompressed dispatch,
against the fp64 oracle.

Each stage is judged on exactly the inputs it received (the attention on the
GPU's own bf16 K and fp16 V); the dispatcher and the full-size run are judged end
to end against the fp64 definition with the chain bar (max error 1e-2 of
max |ref|, mean relative error 5e-3), since bf16 K, V and P roundings compound.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from mla_inputs import CONFIGS, make_inputs
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


def _case(lens, s_q, seed):
    """Random bf16 inputs with real dims, a permuted page pool and -1 tails."""
    g = torch.Generator().manual_seed(seed)
    need = [-(-L // 64) for L in lens]
    pool = sum(need) + 3
    order = torch.randperm(pool, generator=g)
    bt = torch.full((len(lens), max(need) + 1), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = order[off:off + n].to(torch.int32)
        off += n
    B = len(lens)
    kv = torch.randn((pool, 64, 576), generator=g).to(torch.bfloat16)
    q_c = torch.randn((B, s_q, 128, 128), generator=g).to(torch.bfloat16)
    q_r = torch.randn((B, s_q, 128, 64), generator=g).to(torch.bfloat16)
    w_uk = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    w_uv = (torch.randn((128, 128, 512), generator=g) / math.sqrt(512)).to(torch.bfloat16)
    return dict(kv=kv, bt=bt, sl=torch.tensor(lens, dtype=torch.int32), q_c=q_c, q_r=q_r, w_uk=w_uk, w_uv=w_uv)


def _nan_buffers(B, max_len):
    k = torch.full((B, 128, max_len, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    v = torch.full((B, 128, max_len, 128), float("nan"), dtype=torch.float16, device=DEV)
    return k, v


@pytest.mark.parametrize("lens", [[300, 77], [1, 513, 64]])
def test_decompress_kv_parity(M, lens):
    c = _case(lens, 1, seed=sum(lens))
    max_len = -(-max(lens) // 64) * 64 + 64
    _say(f"decompress lens={lens} max_len={max_len}")
    k, v = _nan_buffers(len(lens), max_len)
    M.mla_decompress_kv(c["kv"].to(DEV), c["bt"].to(DEV), c["sl"].to(DEV), c["w_uk"].to(DEV), c["w_uv"].to(DEV),
                        max_len, k_nope=k, v=v)
    torch.cuda.synchronize()
    refK, refV = O.decompress_kv(O.bf16_bits(c["kv"]), c["bt"].numpy(), c["sl"].numpy(), O.as_f64(c["w_uk"]),
                                 O.as_f64(c["w_uv"]), max_len)
    gk, gv = O.as_f64(k.cpu()), O.as_f64(v.cpu())
    for b, L in enumerate(lens):
        assert_bar(gk[b, :, :L], refK[b, :, :L], f"K b={b}")
        assert_bar(gv[b, :, :L], refV[b, :, :L], f"V b={b}")
        pad = -(-L // 64) * 64
        assert (gk[b, :, L:pad] == 0).all() and (gv[b, :, L:pad] == 0).all(), "the rest of L_b's page is not zero"
        assert np.isnan(gk[b, :, pad:]).all() and np.isnan(gv[b, :, pad:]).all(), "rows past L_b's page were written"


@pytest.mark.parametrize("lens,s_q", [([300, 77], 3), ([1000], 300), ([5, 130], 9)])
def test_prefill_mha_parity(M, lens, s_q):
    """The attention stage on the GPU's own K and V; NaN in every buffer row
    past a sequence's end must not reach the output."""
    c = _case(lens, s_q, seed=7 * s_q + len(lens))
    max_len = -(-max(lens) // 64) * 64 + 64
    _say(f"prefill_mha lens={lens} s_q={s_q}")
    kvd, btd, sld = c["kv"].to(DEV), c["bt"].to(DEV), c["sl"].to(DEV)
    k, v = _nan_buffers(len(lens), max_len)
    M.mla_decompress_kv(kvd, btd, sld, c["w_uk"].to(DEV), c["w_uv"].to(DEV), max_len, k_nope=k, v=v)
    out, lse = M.mla_prefill_mha(c["q_c"].to(DEV), c["q_r"].to(DEV), k, v, kvd, btd, sld, SCALE)
    torch.cuda.synchronize()
    K = np.nan_to_num(O.as_f64(k.cpu()))   # rows past L_b are never visible; zero them for the oracle
    V = np.nan_to_num(O.as_f64(v.cpu()))
    R = O.rope_keys(O.bf16_bits(c["kv"]), c["bt"].numpy(), c["sl"].numpy(), max_len)
    ref_o, ref_l = O.attend_mha(O.as_f64(c["q_c"]), O.as_f64(c["q_r"]), K, V, R, c["sl"].numpy(), SCALE)
    assert_bar(O.as_f64(out.cpu()), ref_o, "prefill_mha out")
    assert_lse(lse.cpu().numpy(), ref_l, "prefill_mha lse")


@pytest.mark.parametrize("s_q,path", [(256, "absorbed"), (257, "decompressed")])
def test_attention_layer_dispatch_vs_naive(M, s_q, path):
    lens = [600]
    c = _case(lens, s_q, seed=s_q)
    _say(f"attention_layer s_q={s_q}")
    r = M.attention_layer(c["q_c"].to(DEV), c["q_r"].to(DEV), c["kv"].to(DEV), c["bt"].to(DEV), c["sl"].to(DEV),
                          c["w_uk"].to(DEV), c["w_uv"].to(DEV), max_len=max(lens))
    torch.cuda.synchronize()
    assert r["path"] == path
    ref_o, ref_l = O.decode_naive(O.as_f64(c["q_c"]), O.as_f64(c["q_r"]), O.bf16_bits(c["kv"]), c["bt"].numpy(),
                                  c["sl"].numpy(), O.as_f64(c["w_uk"]), O.as_f64(c["w_uv"]), SCALE)
    assert_bar(O.as_f64(r["out"].cpu()), ref_o, f"{path} end-to-end", l1_rel=5e-3)
    assert_lse(r["lse"].cpu().numpy(), ref_l, f"{path} lse")


def test_decompressed_branch_prefill_config_sampled(M):
    """The decompressed branch at the full prefill workload (4 x 16640 tokens,
    256-token chunks), on sampled rows the oracle computes one by one."""
    inp = make_inputs("prefill")
    B, s_q = inp.q_c.shape[:2]
    _say(f"decompressed branch at the prefill workload B={B} s_q={s_q}")
    r = M.attention_layer(inp.q_c.to(DEV), inp.q_r.to(DEV), inp.kv_cache.to(DEV), inp.block_table.to(DEV),
                          inp.seqlens.to(DEV), inp.w_uk.to(DEV), inp.w_uv.to(DEV), max_len=int(inp.seqlens.max()),
                          absorbed=False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    picks = [(int(rng.integers(B)), int(i), int(rng.integers(128))) for i in list(rng.integers(s_q, size=22)) + [0, s_q - 1]]
    qa = O.absorb(O.as_f64(inp.q_c), O.as_f64(inp.w_uk))
    o_lat, ref_l = O.decode_rows(qa, O.as_f64(inp.q_r), O.bf16_bits(inp.kv_cache), inp.block_table.numpy(),
                                 inp.seqlens.numpy(), SCALE, picks)
    w_uv = O.as_f64(inp.w_uv)
    ref_o = np.stack([w_uv[h] @ o_lat[k] for k, (_, _, h) in enumerate(picks)])
    got = O.as_f64(r["out"].cpu())
    got_o = np.stack([got[b, i, h] for b, i, h in picks])
    got_l = np.array([float(r["lse"][b, i, h]) for b, i, h in picks])
    assert_bar(got_o, ref_o, "decompressed prefill sampled", l1_rel=5e-3)
    assert_lse(got_l, ref_l, "decompressed prefill sampled lse")


def test_prefill_mha_score_jump_triggers_exact_rescan(M):
    """A key far above every score of a query's first tile (more than 2^14 in
    weight) makes the workgroup rescan with the exact maxima; the result must
    still match the oracle."""
    lens, s_q = [700], 5
    c = _case(lens, s_q, seed=99)
    max_len = 704
    g = torch.Generator().manual_seed(100)
    k = (torch.randn((1, 128, max_len, 128), generator=g) * 0.1).to(torch.bfloat16)
    v = torch.randn((1, 128, max_len, 128), generator=g).to(torch.float16)
    k[:, :, 700:] = 0
    v[:, :, 700:] = 0
    k[0, :, 650, 0] = 400.0                          # score 400 * q_c[..., 0] / sqrt(192)
    q_c = c["q_c"].clone()
    q_c[..., 0] = 1.0
    _say("prefill_mha rescan")
    kvd, btd, sld = c["kv"].to(DEV), c["bt"].to(DEV), c["sl"].to(DEV)
    out, lse = M.mla_prefill_mha(q_c.to(DEV), c["q_r"].to(DEV), k.to(DEV), v.to(DEV), kvd, btd, sld, SCALE)
    torch.cuda.synchronize()
    R = O.rope_keys(O.bf16_bits(c["kv"]), c["bt"].numpy(), c["sl"].numpy(), max_len)
    ref_o, ref_l = O.attend_mha(O.as_f64(q_c), O.as_f64(c["q_r"]), O.as_f64(k), O.as_f64(v), R, c["sl"].numpy(), SCALE)
    assert_bar(O.as_f64(out.cpu()), ref_o, "prefill_mha rescan out")
    assert_lse(lse.cpu().numpy(), ref_l, "prefill_mha rescan lse")
