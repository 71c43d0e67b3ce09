"""Seeded synthetic inputs for the Mamba-2 mixer hot path.

This module draws random tensors and nothing else: it holds none of the
method's arithmetic and is shared, unchanged, by the tests, the benchmark and
the oracle checks, so both sides always see identical input values.

Distributions (one recipe for every workload):
  xBC (conv input)   N(0, 1)                 -> activation dtype (round to nearest even)
  conv w, bias       U(-0.5, 0.5)            -> activation dtype
  dt                 softplus(N(-2, 1)) fp32 -> activation dtype
  A[h]               -exp(U(0, 1))  fp32     (negative per-head decay rate)
  D[h]               N(0, 1)        fp32
  ssm state          N(0, 0.1^2)    fp32     (decode workload)
  slow decay variant A = -exp(U(-3, -1)), dt = softplus(N(-4, 1))

Packed serving batches (varlen): S request lengths >= 1 drawn as round(T * w_s / sum(w)) with
w_s ~ LogNormal(0, 1) (a mix of short and long prompts), adjusted to sum exactly to T tokens;
slots are a seeded random choice of distinct pool entries; every other sequence continues from
an initial state (pool states N(0, 0.1^2) fp32, conv-state pool N(0, 1)).

Layer shapes follow the Ultra-family Mamba layer (256 heads x head_dim 64,
d_state 128, 8 groups, conv width 4, conv_dim 18432).
"""
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class LayerDims:
    batch: int
    seqlen: int
    nheads: int
    head_dim: int
    ngroups: int
    d_state: int
    chunk: int = 128
    conv_width: int = 4
    dtype: torch.dtype = torch.bfloat16

    @property
    def d_inner(self):
        return self.nheads * self.head_dim

    @property
    def conv_dim(self):
        # x | B | C channels of the conv
        return self.d_inner + 2 * self.ngroups * self.d_state

    def with_(self, **kw):
        return replace(self, **kw)


# Named workloads (sizes from the Ultra-family Mamba layer).
WORKLOADS = {
    # tiny fp32 mixer: prefill 256 tokens then 8 decode steps
    "tiny_fp32": LayerDims(1, 256, 4, 16, 1, 16, chunk=64, dtype=torch.float32),
    # decode: batch 64, one token per step, fp32 state (64, 256, 64, 128)
    "decode_ultra_b64": LayerDims(64, 1, 256, 64, 8, 128),
    # prefill: batch 1 x 8192 tokens, Ultra layer, chunk 128
    "prefill_ultra_8k": LayerDims(1, 8192, 256, 64, 8, 128),
    # chunked-prefill continuation: batch 8 x 4096 tokens, 128 heads
    "continuation_h128_b8": LayerDims(8, 4096, 128, 64, 8, 128),
    # long context: batch 1 x 262144 tokens, Ultra layer
    "long_ultra_256k": LayerDims(1, 262144, 256, 64, 8, 128),
    # packed serving prefill: 8192 tokens in 24 requests (batch = requests), Ultra layer
    "varlen_ultra_8k": LayerDims(24, 8192, 256, 64, 8, 128),
}


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, std=1.0, mean=0.0):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std + mean


def _rand(shape, g, device, lo, hi):
    return torch.rand(shape, generator=g, device=device, dtype=torch.float32) * (hi - lo) + lo


def draw_dt(shape, g, device, slow=False):
    mu = -4.0 if slow else -2.0
    return torch.nn.functional.softplus(_randn(shape, g, device, 1.0, mu))


def draw_A(h, g, device, slow=False):
    lo, hi = (-3.0, -1.0) if slow else (0.0, 1.0)
    return -torch.exp(_rand((h,), g, device, lo, hi))


def mixer_inputs(dims, seed, device="cpu", slow=False, conv_state=False, init_state=False,
                 seqlen=None):
    """Inputs of one mixer layer prefill: conv input xbc [B,L,CD], taps w [CD,K],
    bias [CD], dt [B,L,H], A [H], D [H]; optional conv_state [B,CD,K] and
    ssm init state [B,H,P,N] (fp32)."""
    L = dims.seqlen if seqlen is None else seqlen
    g = _gen(seed, device)
    dt_ = dims.dtype
    B, H, P, N, CD, K = dims.batch, dims.nheads, dims.head_dim, dims.d_state, dims.conv_dim, dims.conv_width
    out = {}
    out["xbc"] = _randn((B, L, CD), g, device).to(dt_)
    out["w"] = _rand((CD, K), g, device, -0.5, 0.5).to(dt_)
    out["bias"] = _rand((CD,), g, device, -0.5, 0.5).to(dt_)
    out["dt"] = draw_dt((B, L, H), g, device, slow).to(dt_)
    out["A"] = draw_A(H, g, device, slow)
    out["D"] = _randn((H,), g, device)
    if conv_state:
        out["conv_state"] = _randn((B, CD, K), g, device).to(dt_)
    if init_state:
        out["init_state"] = _randn((B, H, P, N), g, device, 0.1)
    return out


def decode_tokens(dims, seed, steps, device="cpu", slow=False):
    """Per-step decode inputs: xbc [steps,B,CD] and dt [steps,B,H]."""
    g = _gen(seed, device)
    B, H, CD = dims.batch, dims.nheads, dims.conv_dim
    return {
        "xbc": _randn((steps, B, CD), g, device).to(dims.dtype),
        "dt": draw_dt((steps, B, H), g, device, slow).to(dims.dtype),
    }


def scan_inputs(dims, seed, device="cpu", slow=False, init_state=True, seqlen=None,
                x_std=1.0, bc_std=1.0):
    """Direct scan inputs (no conv in front): x [B,L,H,P], Bm/Cm [B,L,G,N],
    dt [B,L,H], A [H], D [H], init [B,H,P,N] fp32 (or None)."""
    L = dims.seqlen if seqlen is None else seqlen
    g = _gen(seed, device)
    B, H, P, G, N = dims.batch, dims.nheads, dims.head_dim, dims.ngroups, dims.d_state
    out = {
        "x": _randn((B, L, H, P), g, device, x_std).to(dims.dtype),
        "Bm": _randn((B, L, G, N), g, device, bc_std).to(dims.dtype),
        "Cm": _randn((B, L, G, N), g, device, bc_std).to(dims.dtype),
        "dt": draw_dt((B, L, H), g, device, slow).to(dims.dtype),
        "A": draw_A(H, g, device, slow),
        "D": _randn((H,), g, device),
    }
    out["init_state"] = _randn((B, H, P, N), g, device, 0.1) if init_state else None
    return out


def decode_state(dims, seed, device="cpu"):
    """Decode-workload fp32 state [B,H,P,N] ~ N(0, 0.1^2) and bf16 conv state ~ N(0,1)."""
    g = _gen(seed, device)
    B, H, P, N, CD, K = dims.batch, dims.nheads, dims.head_dim, dims.d_state, dims.conv_dim, dims.conv_width
    return {
        "state": _randn((B, H, P, N), g, device, 0.1),
        "conv_state": _randn((B, CD, K), g, device).to(dims.dtype),
    }


def varlen_lengths(total, nseq, seed):
    """nseq request lengths >= 1 summing to total (total >= nseq), log-normal mix."""
    r = np.random.default_rng(int(seed))
    w = r.lognormal(0.0, 1.0, nseq)
    lens = np.maximum(1, np.round(total * w / w.sum())).astype(np.int64)
    while lens.sum() != total:               # move the rounding error onto the longest / shortest
        if lens.sum() > total:
            i = int(np.argmax(lens))
            lens[i] -= min(lens[i] - 1, lens.sum() - total)
        else:
            lens[int(np.argmin(lens))] += total - lens.sum()
    return [int(v) for v in lens]


def varlen_tables(lens, nslots, seed, device="cpu"):
    """cu_seqlens [S+1], slot_idx [S] (distinct slots of an nslots pool) and has_initial_state [S]
    (every other request), all int32."""
    r = np.random.default_rng(int(seed))
    S = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slot = r.permutation(nslots)[:S].astype(np.int32)
    has_init = (np.arange(S) % 2).astype(np.int32)
    t = lambda a: torch.from_numpy(a).to(device)
    return t(cu), t(slot), t(has_init)


def varlen_inputs(dims, lens, nslots, seed, device="cpu"):
    """A packed prefill: mixer inputs for T = sum(lens) token rows (xbc [T,CD], dt [T,H], taps,
    A, D), the tables, and the pools: conv states [nslots,CD,K] and ssm states [nslots,H,P,N]."""
    T = int(sum(lens))
    inp = mixer_inputs(dims.with_(batch=1, seqlen=T), seed, device)
    inp["xbc"] = inp["xbc"][0]
    inp["dt"] = inp["dt"][0]
    g = _gen(int(seed) + 7919, device)
    H, P, N, CD, K = dims.nheads, dims.head_dim, dims.d_state, dims.conv_dim, dims.conv_width
    inp["conv_pool"] = _randn((nslots, CD, K), g, device).to(dims.dtype)
    inp["state_pool"] = _randn((nslots, H, P, N), g, device, 0.1)
    inp["cu_seqlens"], inp["slot_idx"], inp["has_initial_state"] = varlen_tables(lens, nslots, seed, device)
    return inp
