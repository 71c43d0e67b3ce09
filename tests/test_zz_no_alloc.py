"""The allocation-free scan entry point (ssd_chunk_scan_noalloc) on the GPU, through the C ABI.

It runs the same kernels as ssd_chunk_scan with a caller workspace, on the library's static
per-device array instead, so its results must equal that entry point's bit for bit -- on two calls
in a row, the second smaller (the array keeps the first call's contents, which the second must not
read).  Sizes whose workspace exceeds the 64 MiB array are refused before anything runs.
"""
import pytest
import torch

from selective_state_space_conv1d_amd import ssd
from selective_state_space_conv1d_amd.synth import LayerDims, scan_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def cuda(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def both(s, ydt, chunk=128):
    """(y, final) from ssd_chunk_scan with its own workspace, then from ssd_chunk_scan_noalloc."""
    x = s["x"]
    fin_ref = torch.full_like(s["init_state"], 7.0)
    y_ref = ssd.ssd_chunk_scan(x, s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], s["init_state"], fin_ref,
                               chunk=chunk, y_dtype=ydt)
    fin = torch.full_like(s["init_state"], 9.0)
    y = torch.full(x.shape, 5.0, dtype=ydt, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    ssd.ssd_chunk_scan_noalloc(x, s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], s["init_state"], fin, y, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return (y_ref, fin_ref), (y, fin)


@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float32])
def test_noalloc_equals_workspace_scan_two_calls(ydt):
    # first call: 2 x 1000 tokens, 8 heads in 2 groups (2 x 2 x 8 = 32 tiles); second: 1 x 300 tokens
    big = cuda(scan_inputs(LayerDims(2, 1000, 8, 64, 2, 128), 801))
    small = cuda(scan_inputs(LayerDims(1, 300, 8, 64, 2, 128), 802))
    for s in (big, small):
        (yr, fr), (y, f) = both(s, ydt)
        assert torch.equal(y, yr), "y differs from ssd_chunk_scan with a workspace"
        assert torch.equal(f, fr), "final state differs from ssd_chunk_scan with a workspace"


def test_noalloc_at_the_prefill_size_then_other_kernels():
    """The 8192-token, 8-group layer fits; sizes with no workspace run the other scans."""
    s = cuda(scan_inputs(LayerDims(1, 8192, 16, 64, 8, 128), 803))
    (yr, fr), (y, f) = both(s, torch.bfloat16)
    assert torch.equal(y, yr) and torch.equal(f, fr)
    s = cuda(scan_inputs(LayerDims(2, 200, 4, 32, 2, 64), 804))        # split-operand kernel, no workspace
    (yr, fr), (y, f) = both(s, torch.float32)
    assert torch.equal(y, yr) and torch.equal(f, fr)


def test_noalloc_refuses_sizes_past_the_static_array():
    s = cuda(scan_inputs(LayerDims(1, 128 * 100, 8, 64, 8, 128), 805))  # 800 tiles of 84 KiB: 69 MB
    fin = torch.empty_like(s["init_state"])
    y = torch.full(s["x"].shape, 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError, match="SSD_ERR_WORKSPACE"):
        ssd.ssd_chunk_scan_noalloc(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], s["init_state"], fin, y)
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()), "a refused call writes nothing"
