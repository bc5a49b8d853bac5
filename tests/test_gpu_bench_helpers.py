"""The measurement helpers of include/ubs_bench.h run on the GPU and write nothing to
their sink for ordinary inputs (their results fold into a value they only store when it
equals a fixed constant)."""
import pytest
import torch

import unified_block_sparse_amd as ubs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def test_bench_read_reads_and_leaves_sink():
    buf = torch.arange(1 << 20, dtype=torch.int32, device=DEV)
    sink = torch.zeros(4, dtype=torch.int32, device=DEV)
    ubs.bench_read(buf, sink)
    torch.cuda.synchronize(DEV)
    assert int(sink[0].item()) == 0


def test_bench_mfma_runs_and_counts_its_flops():
    out = torch.zeros(4, dtype=torch.float32, device=DEV)
    flops = ubs.bench_mfma(10, out)
    torch.cuda.synchronize(DEV)
    assert flops == ubs.load().ubs_bench_mfma_waves() * 10 * 4 * 32768 and flops > 0
    assert float(out[0].item()) == 0.0
