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


@pytest.mark.parametrize("kind", [0, 1, 2, 3])
def test_mfma_rate_helper_runs(kind):
    """The matrix-core rate helper launches each instruction kind and writes its sink."""
    sink = torch.full((256,), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_mfma_rate(kind, 16, 8, sink.data_ptr(), moe.current_stream())
    torch.cuda.synchronize()
    assert bool(torch.isfinite(sink).all())
    with pytest.raises(moe.MoeError):
        moe.moe_mfma_rate(4, 16, 8, sink.data_ptr(), moe.current_stream())


@pytest.mark.gpu
@pytest.mark.parametrize("pattern", [0, 1, 2, 3, 4])
def test_read_pattern_helper_runs(pattern):
    """The access-pattern helper reads ragged region counts and leaves its sink
    untouched (the kernel stores only when the XOR of what it read is its
    keep-alive constant, which equal bytes never give)."""
    rows = moe.READ_PATTERNS[pattern][1]
    for row_bytes, regions in ((256, 3), (1024, 37)):
        nbytes = rows * row_bytes * regions
        src = torch.full((nbytes,), 7, dtype=torch.uint8, device="cuda")
        sink = torch.full((256,), 7, dtype=torch.int32, device="cuda")
        moe.moe_read_pattern(pattern, src.data_ptr(), nbytes, row_bytes, 8, sink.data_ptr(), moe.current_stream())
        torch.cuda.synchronize()
        assert bool((sink == 7).all())


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4])
def test_release_cost_helper_counts_and_writes(mode):
    grid, pt = 300, 3
    data = torch.zeros(grid * 256 * pt, dtype=torch.float32, device="cuda")
    ctr = torch.zeros(4096, dtype=torch.int32, device="cuda")
    moe.moe_release_cost(mode, data.data_ptr(), ctr.data_ptr(), grid, pt, moe.current_stream())
    torch.cuda.synchronize()
    b = torch.arange(grid, device="cuda").repeat_interleave(256 * pt)
    i = torch.arange(pt, device="cuda").repeat_interleave(256).repeat(grid)
    assert torch.equal(data, (b + i).float())
    counted = int(ctr.view(256, 16)[:, 0].sum())
    assert counted == (grid if mode in (1, 2, 4) else 0)
    assert int(ctr.view(256, 16)[:, 1:].abs().sum()) == 0
