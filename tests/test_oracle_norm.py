"""The oracle's gated group RMSNorm against torch's rms_norm and silu (CPU, fp64).

Source: "MAX 平台 Nemotron-H 混合架构解析", 5.4, item 4: the gate silu(z) multiplies y in fp32
before the norm, the RMS norm runs over each group of channels, then the fp32 weight multiplies.
"""
import numpy as np
import torch

from oracle_pins import rel_err


def test_gated_rmsnorm_matches_torch(orc):
    r = np.random.default_rng(21)
    T, G, gs, eps = 7, 4, 24, 1e-5
    y = r.standard_normal((T, G * gs)) * 3.0
    z = r.standard_normal((T, G * gs)) * 2.0
    w = r.uniform(0.5, 1.5, G * gs)
    out = orc.gated_rmsnorm(y, z, w, G, eps)
    yt, zt, wt = (torch.from_numpy(a) for a in (y, z, w))
    v = (yt * torch.nn.functional.silu(zt)).reshape(T, G, gs)
    ref = torch.nn.functional.rms_norm(v, (gs,), eps=eps).reshape(T, G * gs) * wt
    assert rel_err(out, ref.numpy()) < 1e-14


def test_gated_rmsnorm_groups_are_independent_and_scale_free(orc):
    r = np.random.default_rng(22)
    T, G, gs = 3, 2, 8
    y = r.standard_normal((T, G * gs))
    z = r.standard_normal((T, G * gs))
    w = np.ones(G * gs)
    out = orc.gated_rmsnorm(y, z, w, G, 0.0)
    # each group of the output has unit RMS when eps = 0
    g = out.reshape(T, G, gs)
    assert np.allclose(np.sqrt((g * g).mean(-1)), 1.0, atol=1e-12)
    # scaling one group of y leaves the output unchanged (eps = 0); other groups are untouched
    y2 = y.copy()
    y2[:, :gs] *= 7.5
    assert rel_err(orc.gated_rmsnorm(y2, z, w, G, 0.0), out) < 1e-13
