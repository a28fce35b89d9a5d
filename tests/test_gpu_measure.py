"""The plain streaming read that bench.py reports beside the indexer's bandwidth: it runs on any
size that is a multiple of 16 bytes, is recorded under its timing name, and leaves its input alone."""
import pytest
import torch

from compressed_sparse_attention_03_amd import ops
from helpers import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 71_369_728])
def test_stream_read_runs_and_is_timed(nbytes):
    say(f"case: stream read {nbytes} B")
    src = torch.arange(nbytes, dtype=torch.int64, device="cuda").remainder(251).to(torch.uint8)
    before = src.clone()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    ops.timing_enable(True)
    for _ in range(3):
        ops.measure_stream_read(src, sink)
    torch.cuda.synchronize()
    ms, cnt = ops.timing_read("stream_read")
    ops.timing_enable(False)
    assert cnt == 3 and ms > 0.0
    assert torch.equal(src, before)
