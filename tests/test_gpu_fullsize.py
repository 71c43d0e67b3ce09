"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

* prefill 1 x 8192 (Ultra layer): every conv channel, every head's y and final state;
* decode batch 64: all 256 steps of every row (conv outputs, y of each step, final state);
* continuation 8 x 4096 (128 heads): every (batch row, head) pair against the oracle's 8192-token
  prefill, and against the GPU's own 8192-token prefill;
* long context 1 x 262144 + 64 decode steps: the oracle on 8 sampled heads, one per group,
  h = 33*g (0, 33, ..., 231).
"""
import numpy as np
import pytest
import torch

from gpu_util import (BF16_BAR, assert_bf16_elementwise, assert_close, f64, oracle_mixer, oracle_scan_of_conv,
                      rel_max, to_act)
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


def oracle_row_prefill(orc, d, inp, b, conv_state=None, init=None):
    """Oracle conv over every channel of batch row b -> bf16 -> scan of every head of that row."""
    cs = None if conv_state is None else conv_state[b:b + 1]
    ini = None if init is None else init[b:b + 1]
    row = {k: (inp[k][b:b + 1] if k in ("xbc", "dt") else inp[k]) for k in ("xbc", "w", "bias", "dt", "A", "D")}
    v, s_out, y, fin = oracle_mixer(orc, row, d.with_(batch=1), cs, ini)
    return v[0], s_out[0], y[0], fin[0]


@pytest.mark.timeout(600)
def test_prefill_ultra_8k(orc):
    """Every head, every token and every conv channel of the 1 x 8192 prefill against the oracle."""
    d = WORKLOADS["prefill_ultra_8k"]
    inp = {k: v.to(DEV) for k, v in mixer_inputs(d, 1002, device=DEV).items()}
    v, so, y16, fin = gpu_prefill(d, inp)
    _, _, y32, fin32 = gpu_prefill(d, inp, ydt=torch.float32)
    assert torch.equal(y16, y32.to(torch.bfloat16)), "bf16 y must be RNE of the fp32 y"
    assert torch.equal(fin, fin32)
    # stage 1: the conv of every channel against the oracle's, within one bf16 ulp
    vr, sr, yr_e2e, _ = oracle_row_prefill(orc, d, inp, 0)
    assert_bf16_elementwise(v[0].cpu(), vr, "conv, all 18432 channels")
    assert np.array_equal(f64(so[0]), sr), "conv state"
    del vr
    # stage 2: the scan of every head, the oracle fed the GPU's bf16 conv output
    yr, fr = oracle_scan_of_conv(orc, v, d, inp["dt"], inp["A"], inp["D"])
    e_y = assert_close(y32, yr, BF16_BAR, "y (fp32 output), all 256 heads")
    e_s = assert_close(fin, fr, BF16_BAR, "final state, all 256 heads")
    # end to end (the oracle's own bf16 conv output in front of its scan): reported, and held to the same bar
    e_e2e = assert_close(y32[0], yr_e2e, BF16_BAR, "y end to end")
    print(f"prefill_ultra_8k vs oracle: y {e_y:.3e}, state {e_s:.3e}, y end to end {e_e2e:.3e}", flush=True)
    # conv state: the last 4 inputs of every channel, bitwise
    assert torch.equal(so[0], inp["xbc"][0, -4:].transpose(0, 1))


@pytest.mark.timeout(600)
def test_decode_ultra_b64(orc):
    """All 256 decode steps of all 64 rows.  The conv updates are checked against the oracle's conv
    of the 256 tokens continuing the initial conv state; the state updates, fed the GPU's own conv
    outputs, against the oracle's recurrence over those 256 tokens from the initial state (the
    decode update is that recurrence one token at a time): y of every step and the final state."""
    d = WORKLOADS["decode_ultra_b64"]
    steps = 256
    st0 = decode_state(d, 1001, device=DEV)
    inp = mixer_inputs(d.with_(seqlen=1), 1001, device=DEV)
    tok = decode_tokens(d, 1011, steps, device=DEV)
    state = st0["state"].clone()
    cs = st0["conv_state"].clone()
    us, ys = [], []
    for k in range(steps):
        u = ssd.ssd_conv1d_update(tok["xbc"][k], inp["w"], inp["bias"], cs)
        x, Bm, Cm = ssd.split_xbc(u, d.nheads, d.head_dim, d.ngroups, d.d_state)
        ys.append(ssd.ssd_state_update(state, x, Bm, Cm, tok["dt"][k], inp["A"], inp["D"], y_dtype=torch.float32))
        us.append(u)
    torch.cuda.synchronize()
    u_all = torch.stack(us, 1)                                    # [B, steps, CD] bf16
    y_all = torch.stack(ys, 1).cpu()                              # [B, steps, H, P]
    del us, ys
    xbc = tok["xbc"].transpose(0, 1)                              # [B, steps, CD]
    vr, sr = orc.conv1d_fwd(f64(xbc), f64(inp["w"]), f64(inp["bias"]), f64(st0["conv_state"]))
    assert_bf16_elementwise(u_all.cpu(), vr, "conv update outputs, all steps and rows")
    assert np.array_equal(f64(cs), sr), "conv state after 256 steps"
    del vr
    I, GN, P, N = d.d_inner, d.ngroups * d.d_state, d.head_dim, d.d_state
    ua = f64(u_all)
    B = d.batch
    x = ua[..., :I].reshape(B, steps, d.nheads, P)
    Bm = ua[..., I:I + GN].reshape(B, steps, d.ngroups, N)
    Cm = ua[..., I + GN:].reshape(B, steps, d.ngroups, N)
    del ua
    yr, fr = orc.scan(x, Bm, Cm, f64(tok["dt"].transpose(0, 1)), f64(inp["A"]), f64(inp["D"]), f64(st0["state"]))
    for k in (0, 1, steps // 2, steps - 1):
        assert_close(y_all[:, k], yr[:, k], 1e-5, f"y step {k}")
    e_y = assert_close(y_all, yr, 1e-5, "y, all steps")
    e_s = assert_close(state, fr, 1e-5, "state after 256 steps")
    print(f"decode_ultra_b64 vs oracle over {steps} steps: y {e_y:.3e}, state {e_s:.3e}", flush=True)


@pytest.mark.timeout(600)
def test_continuation_h128_b8(orc):
    """batch 8 x 4096 continuation from a prior 4096-token prefill == one 8192-token prefill, and every
    (batch row, head) of the continuation against the oracle's 8192-token prefill."""
    d = WORKLOADS["continuation_h128_b8"]
    full = {k: v.to(DEV) for k, v in mixer_inputs(d, 1003, device=DEV, seqlen=2 * d.seqlen).items()}
    first = dict(full, xbc=full["xbc"][:, :d.seqlen].contiguous(), dt=full["dt"][:, :d.seqlen].contiguous())
    second = dict(full, xbc=full["xbc"][:, d.seqlen:].contiguous(), dt=full["dt"][:, d.seqlen:].contiguous())
    v1, cs1, _, st1 = gpu_prefill(d, first)
    v2, cs2, y2, st2 = gpu_prefill(d, second, conv_state=cs1, init=st1, ydt=torch.float32)
    dl = d.with_(seqlen=2 * d.seqlen)
    _, csf, yf, stf = gpu_prefill(dl, full, ydt=torch.float32)
    assert torch.equal(cs2, csf)
    assert_close(y2, f64(yf[:, d.seqlen:]), BF16_BAR, "continuation y vs one long prefill")
    assert_close(st2, f64(stf), BF16_BAR, "continuation state vs one long prefill")
    del yf
    L = d.seqlen
    ey = es = 0.0
    e2e = 0.0
    for b in range(d.batch):
        # conv of both halves against the oracle's conv of the whole row; the scan of every head of
        # the row, the oracle fed the GPU's bf16 conv outputs of both halves from a zero state
        vr, sr, yr_e2e, _ = oracle_row_prefill(orc, dl, full, b)
        assert_bf16_elementwise(v1[b].cpu(), vr[:L], f"first-half conv, row {b}")
        assert_bf16_elementwise(v2[b].cpu(), vr[L:], f"continuation conv, row {b}")
        assert np.array_equal(f64(cs2[b]), sr), f"conv state, row {b}"
        e2e = max(e2e, rel_max(y2[b], yr_e2e[L:]))
        del vr, yr_e2e
        vb = torch.cat([v1[b:b + 1], v2[b:b + 1]], 1)
        yr, fr = oracle_scan_of_conv(orc, vb, dl.with_(batch=1), full["dt"][b:b + 1], full["A"], full["D"])
        ey = max(ey, assert_close(y2[b], yr[0, L:], BF16_BAR, f"continuation y, row {b}, all heads"))
        es = max(es, assert_close(st2[b], fr[0], BF16_BAR, f"continuation state, row {b}, all heads"))
    assert e2e <= BF16_BAR, f"continuation y end to end: {e2e:.3e}"
    print(f"continuation_h128_b8 vs oracle (all 8 x 128 pairs): y {ey:.3e}, state {es:.3e}, "
          f"y end to end {e2e:.3e}", flush=True)


@pytest.mark.timeout(600)
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
