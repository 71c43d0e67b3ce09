"""Parity at the workloads' full sizes, in the launch configuration bench.py
times, with the oracle computing sampled heads / batch rows one by one.

Sampled heads are one per group, h = 33*g (0, 33, ..., 231).
"""
import numpy as np
import pytest
import torch

from gpu_util import BF16_BAR, assert_bf16_elementwise, assert_close, f64, to_act
from selective_state_space_conv1d_amd import ssd
from selective_state_space_conv1d_amd.synth import WORKLOADS, decode_state, decode_tokens, mixer_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def sample_heads(d):
    hpg = d.nheads // d.ngroups
    return [min(g * hpg + g % hpg, d.nheads - 1) for g in range(d.ngroups)]


def head_channels(d, h):
    """conv channels feeding head h: its x channels, then its group's B and C channels."""
    I, GN, N, P = d.d_inner, d.ngroups * d.d_state, d.d_state, d.head_dim
    g = h // (d.nheads // d.ngroups)
    return (list(range(h * P, (h + 1) * P)) + list(range(I + g * N, I + (g + 1) * N))
            + list(range(I + GN + g * N, I + GN + (g + 1) * N)))


def oracle_head_prefill(orc, d, inp, h, b=0, conv_state=None, init=None):
    """Oracle conv (only the head's channels) -> bf16 -> scan of head h of batch row b."""
    ch = torch.tensor(head_channels(d, h), device=inp["xbc"].device)
    u = f64(inp["xbc"][b:b + 1].index_select(2, ch))
    w = f64(inp["w"].index_select(0, ch))
    bias = f64(inp["bias"].index_select(0, ch))
    s_in = None if conv_state is None else f64(conv_state[b:b + 1].index_select(1, ch))
    v, s_out = orc.conv1d_fwd(u, w, bias, s_in)
    v = to_act(v, d.dtype)
    P, N = d.head_dim, d.d_state
    L = v.shape[1]
    x = v[..., :P].reshape(1, L, 1, P)
    Bm = v[..., P:P + N].reshape(1, L, 1, N)
    Cm = v[..., P + N:].reshape(1, L, 1, N)
    init_h = None if init is None else f64(init[b:b + 1, h:h + 1])
    y, fin = orc.scan(x, Bm, Cm, f64(inp["dt"][b:b + 1, :, h:h + 1]), f64(inp["A"][h:h + 1]),
                      f64(inp["D"][h:h + 1]), init_h)
    return v, s_out, y[0, :, 0], fin[0, 0]


def gpu_prefill(d, inp, conv_state=None, init=None, ydt=torch.bfloat16):
    so = torch.empty(d.batch, d.conv_dim, 4, dtype=d.dtype, device=DEV)
    v = ssd.ssd_conv1d_fwd(inp["xbc"], inp["w"], inp["bias"], conv_state, so)
    x, Bm, Cm = ssd.split_xbc(v, d.nheads, d.head_dim, d.ngroups, d.d_state)
    fin = torch.empty(d.batch, d.nheads, d.head_dim, d.d_state, device=DEV)
    y = ssd.ssd_chunk_scan(x, Bm, Cm, inp["dt"], inp["A"], inp["D"], init, fin, chunk=d.chunk, y_dtype=ydt)
    torch.cuda.synchronize()
    return v, so, y, fin


def test_prefill_ultra_8k(orc):
    d = WORKLOADS["prefill_ultra_8k"]
    inp = {k: v.to(DEV) for k, v in mixer_inputs(d, 1002, device=DEV).items()}
    v, so, y16, fin = gpu_prefill(d, inp)
    _, _, y32, fin32 = gpu_prefill(d, inp, ydt=torch.float32)
    assert torch.equal(y16, y32.to(torch.bfloat16)), "bf16 y must be RNE of the fp32 y"
    assert torch.equal(fin, fin32)
    heads = sample_heads(d)
    yg = torch.stack([y32[0, :, h] for h in heads])
    fg = torch.stack([fin[0, h] for h in heads])
    refs = [oracle_head_prefill(orc, d, inp, h) for h in heads]
    for h, (vr, sr, _, _) in zip(heads, refs):
        ch = head_channels(d, h)
        assert_bf16_elementwise(v[0][:, ch].cpu(), vr[0], f"conv head {h}")
    assert_close(yg, np.stack([r[2] for r in refs]), BF16_BAR, "y (fp32 output, sampled heads)")
    assert_close(fg, np.stack([r[3] for r in refs]), BF16_BAR, "final state (sampled heads)")
    # conv state: the last 4 inputs of every channel, bitwise
    assert torch.equal(so[0], inp["xbc"][0, -4:].transpose(0, 1))


def test_decode_ultra_b64(orc):
    d = WORKLOADS["decode_ultra_b64"]
    st0 = decode_state(d, 1001, device=DEV)
    inp = mixer_inputs(d.with_(seqlen=1), 1001, device=DEV)
    tok = decode_tokens(d, 1011, 4, device=DEV)
    state = st0["state"].clone()
    cs = st0["conv_state"].clone()
    rows = [0, 31, 63]
    s_ref = f64(st0["state"][rows])
    c_ref = f64(st0["conv_state"][rows])
    for k in range(4):
        u = ssd.ssd_conv1d_update(tok["xbc"][k], inp["w"], inp["bias"], cs)
        x, Bm, Cm = ssd.split_xbc(u, d.nheads, d.head_dim, d.ngroups, d.d_state)
        y = ssd.ssd_state_update(state, x, Bm, Cm, tok["dt"][k], inp["A"], inp["D"], y_dtype=torch.float32)
        torch.cuda.synchronize()
        ur, c_ref = orc.conv1d_update(f64(tok["xbc"][k][rows]), f64(inp["w"]), f64(inp["bias"]), c_ref)
        assert_bf16_elementwise(u[rows], ur, f"conv update step {k}")
        assert np.array_equal(f64(cs[rows]), c_ref)
        # the state update consumes the GPU's conv output (an input here); the oracle is fed the
        # same bf16 values so this checks the state update in isolation
        yr, s_ref = orc.state_update(s_ref, f64(x[rows]), f64(Bm[rows]), f64(Cm[rows]), f64(tok["dt"][k][rows]),
                                     f64(inp["A"]), f64(inp["D"]))
        assert_close(y[rows], yr, 1e-5, f"y step {k}")
    assert_close(state[rows], s_ref, 1e-5, "state after 4 steps")


def test_continuation_h128_b8(orc):
    """batch 8 x 4096 continuation from a prior 4096-token prefill == one 8192-token prefill."""
    d = WORKLOADS["continuation_h128_b8"]
    full = {k: v.to(DEV) for k, v in mixer_inputs(d, 1003, device=DEV, seqlen=2 * d.seqlen).items()}
    first = dict(full, xbc=full["xbc"][:, :d.seqlen].contiguous(), dt=full["dt"][:, :d.seqlen].contiguous())
    second = dict(full, xbc=full["xbc"][:, d.seqlen:].contiguous(), dt=full["dt"][:, d.seqlen:].contiguous())
    _, cs1, _, st1 = gpu_prefill(d, first)
    v2, cs2, y2, st2 = gpu_prefill(d, second, conv_state=cs1, init=st1, ydt=torch.float32)
    dl = d.with_(seqlen=2 * d.seqlen)
    _, csf, yf, stf = gpu_prefill(dl, full, ydt=torch.float32)
    assert torch.equal(cs2, csf)
    assert_close(y2, f64(yf[:, d.seqlen:]), BF16_BAR, "continuation y vs one long prefill")
    assert_close(st2, f64(stf), BF16_BAR, "continuation state vs one long prefill")
    for b in (0, 7):
        for h in sample_heads(d)[::3]:
            _, _, yr, fr = oracle_head_prefill(orc, dl, full, h, b=b)
            assert_close(y2[b, :, h], yr[d.seqlen:], BF16_BAR, f"y b{b} h{h}")
            assert_close(st2[b, h], fr, BF16_BAR, f"state b{b} h{h}")


def test_long_ultra_256k_then_decode(orc):
    """262144-token prefill, then 64 decode steps; oracle on the 8 sampled heads."""
    d = WORKLOADS["long_ultra_256k"]
    inp = {k: v.to(DEV) for k, v in mixer_inputs(d, 1004, device=DEV).items()}
    _, cs, y, st = gpu_prefill(d, inp, ydt=torch.float32)
    heads = sample_heads(d)
    ys_h = torch.stack([y[0, :, h] for h in heads]).cpu()
    del y
    steps = 64
    tok = decode_tokens(d.with_(batch=1), 1014, steps, device=DEV)
    ydec = []
    for k in range(steps):
        u = ssd.ssd_conv1d_update(tok["xbc"][k], inp["w"], inp["bias"], cs)
        x, Bm, Cm = ssd.split_xbc(u, d.nheads, d.head_dim, d.ngroups, d.d_state)
        ydec.append(ssd.ssd_state_update(st, x, Bm, Cm, tok["dt"][k], inp["A"], inp["D"], y_dtype=torch.float32))
    torch.cuda.synchronize()
    ydec = torch.stack(ydec, 1)[0]                              # [steps, H, P]
    # oracle: prefill + decode as one 262144+64 token sequence for each sampled head
    ext = dict(inp, xbc=torch.cat([inp["xbc"], tok["xbc"].transpose(0, 1)], 1),
               dt=torch.cat([inp["dt"], tok["dt"].transpose(0, 1)], 1))
    de = d.with_(seqlen=d.seqlen + steps)
    drift = []
    for i, h in enumerate(heads):
        _, _, yr, fr = oracle_head_prefill(orc, de, ext, h)
        assert_close(ys_h[i], yr[:d.seqlen], BF16_BAR, f"prefill y head {h}")
        assert_close(ydec[:, h], yr[d.seqlen:], BF16_BAR, f"decode y head {h}")
        drift.append(assert_close(st[0, h], fr, BF16_BAR, f"final state head {h}"))
    print(f"fp32 state drift vs oracle after {d.seqlen}+{steps} tokens: max {max(drift):.3e}")
