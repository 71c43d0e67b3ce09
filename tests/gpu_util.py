"""Helpers for the GPU parity tests: run the oracle on the same inputs and
compare.  Expected values come only from the oracle (never from the HIP path).
"""
import numpy as np
import torch

BF16_BAR = 2e-3     # max|dy| <= 2e-3 max|y| for bf16 inputs
F32_BAR = 1e-5      # fp32 mode, normwise relative


def f64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def rel_max(gpu, ref):
    gpu = np.asarray(f64(gpu) if isinstance(gpu, torch.Tensor) else gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), "non-finite GPU output"
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / den) if den > 0 else float(np.max(np.abs(gpu)))


def assert_close(gpu, ref, tol, what=""):
    e = rel_max(gpu, ref)
    assert e <= tol, f"{what}: max|d|/max|ref| = {e:.3e} > {tol:.1e}"
    return e


def assert_bf16_elementwise(gpu, ref, what=""):
    """bf16 output of an fp32 computation vs the fp64 oracle: within one bf16 ulp of the
    value, plus 1e-6 absolute for the fp32 evaluation of O(1) sums near zero."""
    g = f64(gpu)
    r = np.asarray(ref, np.float64)
    bound = np.abs(r) * 2.0 ** -7 + 1e-6
    bad = np.abs(g - r) > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements off by more than 1 bf16 ulp"


def to_act(v64, dtype):
    """Round an oracle fp64 tensor to the activation dtype (what a bf16/fp32 buffer holds)."""
    return torch.from_numpy(np.ascontiguousarray(v64)).to(torch.float32).to(dtype).to(torch.float64).numpy()


def oracle_mixer(orc, inp, dims, conv_state=None, init=None):
    """Oracle pipeline of one prefill: conv (fp64) -> stored precision -> split -> scan."""
    v, s_out = orc.conv1d_fwd(f64(inp["xbc"]), f64(inp["w"]), f64(inp["bias"]), f64(conv_state))
    v = to_act(v, dims.dtype)
    I = dims.nheads * dims.head_dim
    GN = dims.ngroups * dims.d_state
    Bt, L = v.shape[:2]
    x = v[..., :I].reshape(Bt, L, dims.nheads, dims.head_dim)
    Bm = v[..., I:I + GN].reshape(Bt, L, dims.ngroups, dims.d_state)
    Cm = v[..., I + GN:].reshape(Bt, L, dims.ngroups, dims.d_state)
    y, fin = orc.scan(x, Bm, Cm, f64(inp["dt"]), f64(inp["A"]), f64(inp["D"]), f64(init))
    return v, s_out, y, fin


def oracle_scan_of_conv(orc, v, dims, dt, A, D, init=None):
    """Oracle scan fed a conv output v [B, L, CD] (e.g. the GPU's own bf16 conv output): split into
    x, B, C as the layer's channels are laid out, then scan.  This isolates the scan from the
    rounding of the stored conv output, which is checked elementwise on its own."""
    v = f64(v) if isinstance(v, torch.Tensor) else np.asarray(v, np.float64)
    I = dims.nheads * dims.head_dim
    GN = dims.ngroups * dims.d_state
    Bt, L = v.shape[:2]
    x = v[..., :I].reshape(Bt, L, dims.nheads, dims.head_dim)
    Bm = v[..., I:I + GN].reshape(Bt, L, dims.ngroups, dims.d_state)
    Cm = v[..., I + GN:].reshape(Bt, L, dims.ngroups, dims.d_state)
    return orc.scan(x, Bm, Cm, f64(dt), f64(A), f64(D), f64(init))
