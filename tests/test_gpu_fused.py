"""The prefill conv fused into the chunked scan (ssd_conv_chunk_scan), on the GPU.

The fused call computes the width-4 conv + SiLU of x, B and C inside the scan's launches in the conv
kernel's order and rounding, so it must reproduce ssd_conv1d_fwd followed by ssd_chunk_scan (with a
workspace: the same fp16 scan) bit for bit -- y, the final SSM state and the new conv state -- on
ragged, exact-chunk and shorter-than-the-conv sequences, with and without states, bias and dt prologue,
with states updated in place; and the oracle's mixer (conv -> bf16 -> scan, fp64) within the bf16 bar.
"""
import numpy as np
import pytest
import torch

from gpu_util import BF16_BAR, assert_close, f64, oracle_mixer
from selective_state_space_conv1d_amd import ssd
from selective_state_space_conv1d_amd.synth import LayerDims, WORKLOADS, mixer_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def cuda(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def two_launch(d, inp, cs_in, init, ydt, **kw):
    """ssd_conv1d_fwd then ssd_chunk_scan (fp16 scan) on the views of the conv output."""
    cs_out = torch.full((d.batch, d.conv_dim, 4), 7.0, dtype=d.dtype, device=DEV)
    v = ssd.ssd_conv1d_fwd(inp["xbc"], inp["w"], inp.get("bias"), cs_in, cs_out)
    x, Bm, Cm = ssd.split_xbc(v, d.nheads, d.head_dim, d.ngroups, d.d_state)
    fin = torch.full((d.batch, d.nheads, d.head_dim, d.d_state), 3.0, device=DEV)
    y = ssd.ssd_chunk_scan(x, Bm, Cm, inp["dt"], inp["A"], inp["D"], init, fin, y_dtype=ydt, **kw)
    return y, fin, cs_out


def fused(d, inp, cs_in, init, ydt, cs_out=None, fin=None, **kw):
    if cs_out is None:
        cs_out = torch.full((d.batch, d.conv_dim, 4), 5.0, dtype=d.dtype, device=DEV)
    if fin is None:
        fin = torch.full((d.batch, d.nheads, d.head_dim, d.d_state), 9.0, device=DEV)
    y = ssd.ssd_conv_chunk_scan(inp["xbc"], inp["w"], inp.get("bias"), inp["dt"], inp["A"], inp["D"], d.nheads,
                                d.head_dim, d.ngroups, d.d_state, conv_state_in=cs_in, conv_state_out=cs_out,
                                init_state=init, final_state=fin, y_dtype=ydt, **kw)
    return y, fin, cs_out


CASES = [  # (batch, L, heads, groups)
    (2, 300, 4, 2),      # ragged last chunk
    (1, 256, 8, 2),      # exact chunks
    (2, 3, 4, 2),        # shorter than the conv window: the new conv state mixes old state and inputs
    (1, 1, 4, 1),
    (2, 515, 8, 8),
]


@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float32], ids=["ybf16", "yfp32"])
@pytest.mark.parametrize("states", [False, True], ids=["nostate", "states"])
@pytest.mark.parametrize("B,L,H,G", CASES)
def test_fused_equals_conv_then_scan_bitwise(B, L, H, G, states, ydt):
    d = LayerDims(B, L, H, 64, G, 128)
    inp = cuda(mixer_inputs(d, 900 + L + H, conv_state=states, init_state=states))
    cs_in, init = inp.get("conv_state"), inp.get("init_state")
    yr, fr, cr = two_launch(d, inp, cs_in, init, ydt)
    y, f, c = fused(d, inp, cs_in, init, ydt)
    torch.cuda.synchronize()
    assert torch.equal(c, cr), "conv state"
    assert torch.equal(y, yr), "y"
    assert torch.equal(f, fr), "final state"


def test_fused_in_place_states_no_bias_dt_prologue():
    """Conv state and SSM state updated in place, no conv bias, the dt prologue on."""
    d = LayerDims(2, 300, 8, 64, 2, 128)
    inp = cuda(mixer_inputs(d, 911, conv_state=True, init_state=True))
    inp["bias"] = None
    kw = dict(dt_bias=torch.randn(8, device=DEV), dt_softplus=True, dt_limit=(0.0, 2.0))
    raw = (torch.randn(2, 300, 8, device=DEV) - 1.0).to(torch.bfloat16)
    inp["dt"] = raw
    yr, fr, cr = two_launch(d, inp, inp["conv_state"], inp["init_state"], torch.float32, **kw)
    cs = inp["conv_state"].clone()
    st = inp["init_state"].clone()
    y, f, c = fused(d, inp, cs, st, torch.float32, cs_out=cs, fin=st, **kw)
    torch.cuda.synchronize()
    assert c.data_ptr() == cs.data_ptr() and f.data_ptr() == st.data_ptr()
    assert torch.equal(cs, cr) and torch.equal(y, yr) and torch.equal(st, fr)


def test_fused_no_tokens_carries_both_states():
    d = LayerDims(2, 0, 4, 64, 2, 128)
    inp = cuda(mixer_inputs(d, 912, conv_state=True, init_state=True))
    y, f, c = fused(d, inp, inp["conv_state"], inp["init_state"], torch.float32)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, 4, 64)
    assert torch.equal(c, inp["conv_state"]) and torch.equal(f, inp["init_state"])


def test_fused_prefill_8k_full_size():
    """The 1 x 8192-token, 256-head layer: fused == conv-then-scan bit for bit over every head and channel,
    and the new conv state equals the last four inputs exactly."""
    d = WORKLOADS["prefill_ultra_8k"]
    inp = mixer_inputs(d, 1002, device=DEV)
    yr, fr, cr = two_launch(d, inp, None, None, torch.bfloat16)
    y, f, c = fused(d, inp, None, None, torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y, yr) and torch.equal(f, fr)
    assert torch.equal(c, inp["xbc"][:, -4:].transpose(1, 2)) and torch.equal(c, cr)


def test_fused_against_the_oracle_mixer(orc):
    """End to end against the fp64 oracle (conv -> bf16 -> scan): a multi-chunk layer with both states."""
    d = LayerDims(2, 300, 8, 64, 2, 128)
    inp = cuda(mixer_inputs(d, 913, conv_state=True, init_state=True))
    y, f, c = fused(d, inp, inp["conv_state"], inp["init_state"], torch.float32)
    torch.cuda.synchronize()
    _, sr, yr, fr = oracle_mixer(orc, inp, d, conv_state=inp["conv_state"], init=inp["init_state"])
    assert np.array_equal(f64(c), sr), "conv state"
    assert_close(y, yr, BF16_BAR, "y")
    assert_close(f, fr, BF16_BAR, "final state")


def test_fused_refuses_unsupported_sizes():
    d = LayerDims(1, 100, 4, 32, 2, 128)      # head_dim 32: no fp16 scan
    inp = cuda(mixer_inputs(d, 914))
    with pytest.raises(RuntimeError, match="SSD_ERR_UNSUPPORTED"):
        fused(d, inp, None, None, torch.float32)
