"""Host-side logic of bench.py, on the CPU: the roof an intensity selects, the
causal pair count, the algorithmic work per pair, the traffic lookup's digest
guard, and the one-GPU exit. (The timed paths need a GPU and run in smoke and
the bench itself.)"""
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_ridge_and_work_per_pair():
    # dense bf16 2.5 PFLOP/s over 8 TB/s, and per (query, key) pair all 128 heads do
    # QK over the 576 latent + RoPE dims and PV over the 512 latent dims
    assert bench.RIDGE == pytest.approx(312.5)
    assert bench.FLOP_PER_PAIR == 128 * 2 * 576 + 128 * 2 * 512
    assert bench.KV_BYTES_PER_TOKEN == 1152


@pytest.mark.parametrize("flop,nbytes", [(240.0e9, 1.0e9), (9483.0e9, 1.0e9), (312.5e9, 1.0e9)])
def test_roof_follows_intensity(flop, nbytes):
    r = bench.roof(flop, nbytes, 1e-3)
    if flop / nbytes > bench.RIDGE:
        assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
        assert r["frac"] == pytest.approx(flop / 1e-3 / 1e12 / bench.MFMA_BF16_PEAK_TFLOPS, abs=1e-4)
    else:  # at or below the ridge: bandwidth
        assert r["bound"] == "hbm" and r["unit"] == "GB/s"
        assert r["frac"] == pytest.approx(nbytes / 1e-3 / 1e9 / bench.HBM_PEAK_GBS, abs=1e-4)
    # both fractions are reported whatever the bound
    assert r["hbm_frac"] == pytest.approx(nbytes / 1e-3 / 1e9 / 8000.0, abs=1e-4)
    assert r["mfma_frac"] == pytest.approx(flop / 1e-3 / 1e12 / 2500.0, abs=1e-4)


def test_visible_pairs_brute_force():
    # query i of a chunk of s_q rows over L cached tokens (chunk included) sees keys 0 .. L - s_q + i
    for lens, s_q in (([5, 1, 0, 64], 1), ([7, 3], 4), ([300, 2, 17], 17), ([1], 1)):
        want = sum(1 for L in lens for i in range(s_q) for j in range(L) if j <= L - s_q + i)
        assert bench.visible_pairs(lens, s_q) == want


def test_traffic_lookup_requires_matching_source_and_splits(tmp_path, monkeypatch):
    entry = {"kernel_digest": bench.kernel_source_digest(), "splits": 17, "hbm_bytes_per_launch": 123}
    f = tmp_path / "t.json"
    f.write_text(json.dumps({"bf16/long": entry}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("long", 17) == 123
    assert bench.measured_traffic("long", 9) is None          # another launch configuration
    assert bench.measured_traffic("uniform", 17) is None      # no counters for it
    f.write_text(json.dumps({"bf16/long": dict(entry, kernel_digest="0" * 16)}))
    assert bench.measured_traffic("long", 17) is None         # counters of another source


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_projection_roofs_match_the_weight_bound():
    """Absorb and up-projection roofs: 16 MiB of weight plus the activations at
    8 TB/s (2.4 us at T = 16 and 23 us at T = 1024 for the absorb)."""
    class W:
        separate = False
    w = W()
    for T, absorb_us in ((16, 2.42), (1024, 23.07)):
        w.T = T
        w.kernel_ms = {"mla_absorb_q": 0.010, "mla_combine_up_proj": 0.020}
        r = bench.Workload.projection_roofs(w)
        assert r["absorb"]["roofline_time_us"] == absorb_us
        assert r["absorb"]["bound"] == r["up_proj"]["bound"] == "hbm"
        assert r["absorb"]["flop"] == 2 * T * 128 * 128 * 512
        assert r["up_proj"]["algorithmic_bytes"] == 128 * 128 * 512 * 2 + T * 128 * 512 * 4 + T * 128 * 128 * 2
        assert abs(r["absorb"]["frac"] - absorb_us / 10.0) < 1e-3
