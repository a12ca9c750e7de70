"""The streaming-read measurement helper (moe_stream_read) on the GPU: it runs
through the C ABI on ragged sizes and launch shapes, leaves memory it only
reads untouched, and writes nothing to its sink for data whose XOR is not the
kernel's keep-alive constant."""
import pytest
import torch

import quantized_expert_ffn_wave_amd as moe
from parity import say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("nbytes,grid", [(16, 0), (4096, 1), (1 << 20, 0), ((1 << 20) + 48, 7), (64 << 20, 2048)])
def test_stream_read_runs_and_only_reads(nbytes, grid):
    say(f"case stream_read bytes={nbytes} grid={grid}")
    src = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    moe.moe_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), grid, moe.current_stream())
    torch.cuda.synchronize()
    # 0x07070707 XORed an even number of times per 16 B vector is 0: never the constant
    assert int(sink.abs().sum()) == 0
    assert bool((src == 7).all())


def test_stream_read_rejects_bad_sizes_on_the_device():
    src = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.moe_stream_read(src.data_ptr(), 4095, sink.data_ptr(), 0, moe.current_stream())
    with pytest.raises(moe.MoeError):
        moe.moe_stream_read(src.data_ptr() + 8, 4080, sink.data_ptr(), 0, moe.current_stream())
