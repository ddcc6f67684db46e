"""The measurement aids behind bench.py's "ceilings" (not on the decode path):
they run to completion through the C ABI, leave their sink untouched (they
write to it only under conditions that never hold for these inputs) and report
their work as the header states."""
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def M():
    import mla_latent_kv_06_amd as mod
    return mod


def test_stream_read_runs_and_counts_bytes(M):
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)   # 64 MiB
    sink = torch.zeros(M.BENCH_SINK_FLOATS, dtype=torch.float32, device=DEV)
    for nbytes in (16, 4096 + 48, 64 << 20):                      # one chunk, a ragged tail, the whole buffer
        assert M.mla_bench_stream_read(buf[:nbytes], sink) == nbytes
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0


def test_mfma_loop_runs_and_counts_flop(M):
    sink = torch.zeros(M.BENCH_SINK_FLOATS, dtype=torch.float32, device=DEV)
    assert M.mla_bench_mfma(1, sink) == 256 * 4 * 4 * 32768
    assert M.mla_bench_mfma(1000, sink) == 256 * 4 * 4 * 1000 * 32768
    torch.cuda.synchronize()
    assert torch.count_nonzero(sink).item() == 0
