"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Sizes the oracle finishes in seconds that still span several tiles and a
ragged tail, plus edge cases (L = 0, L = 1, L < 4, NULL states, aliasing,
strided views) and the method's invariants.  Full-size workloads are in
test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

from gpu_util import BF16_BAR, F32_BAR, assert_bf16_elementwise, assert_close, f64, oracle_mixer, to_act
from selective_state_space_conv1d_amd import ssd
from selective_state_space_conv1d_amd.synth import LayerDims, WORKLOADS, decode_tokens, mixer_inputs, scan_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def cuda(d):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


# --------------------------------------------------------------------------- conv
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("L", [0, 1, 2, 3, 5, 31, 32, 33, 100, 257])
@pytest.mark.parametrize("with_state", [False, True])
def test_conv1d_fwd(orc, dtype, L, with_state):
    d = LayerDims(3, L, 4, 16, 1, 16, dtype=dtype)  # CD = 96
    inp = cuda(mixer_inputs(d, 100 + L, conv_state=True))
    s_in = inp["conv_state"] if with_state else None
    s_out = torch.full_like(inp["conv_state"], 7.0)
    out = ssd.ssd_conv1d_fwd(inp["xbc"], inp["w"], inp["bias"], s_in, s_out)
    torch.cuda.synchronize()
    v, so = orc.conv1d_fwd(f64(inp["xbc"]), f64(inp["w"]), f64(inp["bias"]), f64(s_in))
    if dtype == torch.bfloat16:
        assert_bf16_elementwise(out, v, "conv out")
    elif L > 0:
        assert_close(out, v, F32_BAR, "conv out")
    assert np.array_equal(f64(s_out), so), "conv state must be a bitwise copy of inputs"


def test_conv1d_fwd_inplace_state_strided_input_no_bias(orc):
    d = LayerDims(2, 77, 8, 32, 2, 32)  # CD = 384
    inp = cuda(mixer_inputs(d, 7, conv_state=True))
    wide = torch.randn(2, 77, 384 + 64, device=DEV).to(torch.bfloat16)
    wide[..., 16:16 + 384] = inp["xbc"]
    xv = wide[..., 16:16 + 384]          # token stride 448, offset 32 bytes
    st = inp["conv_state"].clone()
    out = ssd.ssd_conv1d_fwd(xv, inp["w"], None, st, st)
    torch.cuda.synchronize()
    v, so = orc.conv1d_fwd(f64(inp["xbc"]), f64(inp["w"]), None, f64(inp["conv_state"]))
    assert_bf16_elementwise(out, v, "conv out")
    assert np.array_equal(f64(st), so)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_conv1d_update_steps(orc, dtype):
    d = LayerDims(3, 1, 4, 16, 1, 16, dtype=dtype)
    st0 = cuda(mixer_inputs(d, 11, conv_state=True))
    tok = cuda(decode_tokens(d, 12, 6))
    st = st0["conv_state"].clone()
    s_ref = f64(st)
    for k in range(6):
        out = ssd.ssd_conv1d_update(tok["xbc"][k], st0["w"], st0["bias"], st)
        torch.cuda.synchronize()
        v, s_ref = orc.conv1d_update(f64(tok["xbc"][k]), f64(st0["w"]), f64(st0["bias"]), s_ref)
        if dtype == torch.bfloat16:
            assert_bf16_elementwise(out, v, f"step {k}")
        else:
            assert_close(out, v, F32_BAR, f"step {k}")
        assert np.array_equal(f64(st), s_ref)


def test_conv_update_matches_prefill(orc):
    """Decode roll token by token == prefill conv (the state and the outputs)."""
    d = LayerDims(2, 9, 4, 16, 1, 16)
    inp = cuda(mixer_inputs(d, 13, conv_state=True))
    so = inp["conv_state"].clone()
    out = ssd.ssd_conv1d_fwd(inp["xbc"], inp["w"], inp["bias"], inp["conv_state"], so)
    st = inp["conv_state"].clone()
    outs = [ssd.ssd_conv1d_update(inp["xbc"][:, t], inp["w"], inp["bias"], st) for t in range(9)]
    torch.cuda.synchronize()
    assert torch.equal(torch.stack(outs, 1), out)
    assert torch.equal(st, so)


# --------------------------------------------------------------------------- state update
@pytest.mark.parametrize("shape", [(2, 4, 16, 1, 16), (3, 8, 64, 2, 128), (2, 6, 32, 3, 64), (1, 2, 128, 1, 32)])
@pytest.mark.parametrize("dtype,ydt", [(torch.float32, torch.float32), (torch.bfloat16, torch.float32),
                                       (torch.bfloat16, torch.bfloat16)])
def test_state_update(orc, shape, dtype, ydt):
    Bt, H, P, G, N = shape
    d = LayerDims(Bt, 1, H, P, G, N, dtype=dtype)
    s = cuda(scan_inputs(d, 21, seqlen=1))
    state = s["init_state"].clone()
    y = ssd.ssd_state_update(state, s["x"][:, 0], s["Bm"][:, 0], s["Cm"][:, 0], s["dt"][:, 0], s["A"], s["D"],
                             y_dtype=ydt)
    torch.cuda.synchronize()
    yr, sr = orc.state_update(f64(s["init_state"]), f64(s["x"][:, 0]), f64(s["Bm"][:, 0]), f64(s["Cm"][:, 0]),
                              f64(s["dt"][:, 0]), f64(s["A"]), f64(s["D"]))
    assert_close(state, sr, F32_BAR, "state")
    if ydt == torch.float32:
        assert_close(y, yr, F32_BAR, "y")
    else:
        assert_bf16_elementwise(y, yr, "y bf16")


def test_state_update_strided_views_no_D(orc):
    d = LayerDims(4, 1, 8, 64, 2, 128)
    CD = d.conv_dim
    v = torch.randn(4, CD + 32, device=DEV).to(torch.bfloat16)[:, :CD]   # batch stride CD+32
    x, Bm, Cm = ssd.split_xbc(v, 8, 64, 2, 128)
    s = cuda(scan_inputs(d, 22, seqlen=1))
    state = s["init_state"].clone()
    y = ssd.ssd_state_update(state, x, Bm, Cm, s["dt"][:, 0], s["A"], None, y_dtype=torch.float32)
    torch.cuda.synchronize()
    yr, sr = orc.state_update(f64(s["init_state"]), f64(x), f64(Bm), f64(Cm), f64(s["dt"][:, 0]), f64(s["A"]), None)
    assert_close(state, sr, F32_BAR, "state")
    assert_close(y, yr, F32_BAR, "y")


# --------------------------------------------------------------------------- chunk scan
def run_scan(s, chunk=128, ydt=torch.float32, init="given", final=True, ws=None):
    """ws None: the default scan (the fp16 one where it applies); False: the bf16 split-operand kernel."""
    init_t = s["init_state"] if init == "given" else None
    fin = torch.full_like(s["init_state"], 3.0) if final else None
    y = ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], init_t, fin, chunk=chunk, y_dtype=ydt,
                           workspace=ws)
    torch.cuda.synchronize()
    return y, fin


def oracle_scan(orc, s, init="given"):
    return orc.scan(f64(s["x"]), f64(s["Bm"]), f64(s["Cm"]), f64(s["dt"]), f64(s["A"]), f64(s["D"]),
                    f64(s["init_state"]) if init == "given" else None)


@pytest.mark.parametrize("L", [1, 31, 32, 33, 100, 256])
@pytest.mark.parametrize("init", ["given", None])
def test_scan_fp32(orc, L, init):
    d = WORKLOADS["tiny_fp32"].with_(seqlen=L)
    s = cuda(scan_inputs(d, 30 + L))
    y, fin = run_scan(s, chunk=64, init=init)
    yr, fr = oracle_scan(orc, s, init)
    assert_close(fin, fr, F32_BAR, "final state")
    assert_close(y, yr, F32_BAR, "y")


@pytest.mark.parametrize("ws", [pytest.param(None, id="f16"), pytest.param(False, id="split")])
@pytest.mark.parametrize("L", [1, 2, 127, 128, 129, 300, 515])
@pytest.mark.parametrize("slow", [False, True])
def test_scan_bf16_mfma(orc, L, slow, ws):
    d = LayerDims(2, L, 4, 64, 2, 128)
    s = cuda(scan_inputs(d, 40 + L, slow=slow))
    y, fin = run_scan(s, ws=ws)
    yr, fr = oracle_scan(orc, s)
    assert_close(y, yr, BF16_BAR, "y")
    assert_close(fin, fr, BF16_BAR, "final state")


@pytest.mark.parametrize("shape,chunk", [((2, 4, 32, 2, 64), 128), ((1, 3, 16, 1, 16), 64), ((1, 2, 128, 2, 32), 256),
                                         ((2, 4, 64, 2, 128), 64), ((2, 4, 64, 2, 128), 256)])
def test_scan_bf16_other_shapes(orc, shape, chunk):
    Bt, H, P, G, N = shape
    d = LayerDims(Bt, 200, H, P, G, N)
    s = cuda(scan_inputs(d, 50 + P + N))
    y, fin = run_scan(s, chunk=chunk)
    yr, fr = oracle_scan(orc, s)
    assert_close(y, yr, BF16_BAR, "y")
    assert_close(fin, fr, BF16_BAR, "final state")


@pytest.mark.parametrize("H,G", [(16, 2), (32, 2), (64, 2), (24, 1)])
@pytest.mark.parametrize("L", [130, 300])
@pytest.mark.parametrize("prologue", [False, True])
def test_scan_f16_dt_read_as_rows(orc, H, G, L, prologue):
    """The fp16 scan's pre-pass reads dt as whole token rows when a group's heads come in 16-byte pieces
    (8, 16 or 32 heads per group here; 24 per group and a dt view shifted by one element take the
    per-element path), with a ragged last chunk and, optionally, the dt_bias + softplus + clamp prologue."""
    d = LayerDims(2, L, H, 64, G, 128)
    s = cuda(scan_inputs(d, 60 + H + L))
    kw, dt_eff = {}, f64(s["dt"])
    if prologue:
        g = torch.Generator().manual_seed(H + L)
        bias = (torch.randn(H, generator=g) - 1.0).to("cuda")
        kw = dict(dt_bias=bias, dt_softplus=True, dt_limit=(0.0, 0.5))
        dt_eff = orc.dt_prologue(f64(s["dt"]), f64(bias), True, (0.0, 0.5))
    yr, fr = orc.scan(f64(s["x"]), f64(s["Bm"]), f64(s["Cm"]), dt_eff, f64(s["A"]), f64(s["D"]),
                      f64(s["init_state"]))
    for shift in (False, True):
        dt = s["dt"]
        if shift:   # same values, storage offset by one element (2 bytes): not 16-byte aligned
            buf = torch.empty(dt.numel() + 1, dtype=dt.dtype, device="cuda")
            dt = buf[1:].view(dt.shape)
            dt.copy_(s["dt"])
        fin = torch.empty_like(s["init_state"])
        y = ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], dt, s["A"], s["D"], s["init_state"], fin,
                               y_dtype=torch.float32, **kw)
        torch.cuda.synchronize()
        assert_close(y, yr, BF16_BAR, f"y (dt shifted: {shift})")
        assert_close(fin, fr, BF16_BAR, f"final state (dt shifted: {shift})")


@pytest.mark.parametrize("L", [32768 + 300, 2 * 32768])
def test_scan_f16_long_sequence_in_segments(orc, L):
    """A single sequence longer than 32768 tokens is scanned in 32768-token segments chained through an fp32
    state in the workspace (a ragged last segment; an initial state updated in place): against the oracle on
    two heads of different groups, and y and the final state equal to the same scan run as two calls."""
    d = LayerDims(1, L, 8, 64, 2, 128)
    s = cuda(scan_inputs(d, 70 + L % 7, slow=True))
    st = s["init_state"].clone()
    y = ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], st, st, y_dtype=torch.float32)
    torch.cuda.synchronize()
    for h in (1, 6):
        g = h // 4
        yr, fr = orc.scan(f64(s["x"][:, :, h:h + 1]), f64(s["Bm"][:, :, g:g + 1]), f64(s["Cm"][:, :, g:g + 1]),
                          f64(s["dt"][:, :, h:h + 1]), f64(s["A"][h:h + 1]), f64(s["D"][h:h + 1]),
                          f64(s["init_state"][:, h:h + 1]))
        assert_close(y[:, :, h:h + 1], yr, BF16_BAR, f"y head {h}")
        assert_close(st[:, h:h + 1], fr, BF16_BAR, f"final state head {h}")
    # the same in two calls at the segment boundary (each at most one segment): bitwise equal
    mid = torch.empty_like(st)
    k = 32768
    y1 = ssd.ssd_chunk_scan(s["x"][:, :k], s["Bm"][:, :k], s["Cm"][:, :k], s["dt"][:, :k], s["A"], s["D"],
                            s["init_state"], mid, y_dtype=torch.float32)
    st2 = torch.empty_like(st)
    y2 = ssd.ssd_chunk_scan(s["x"][:, k:], s["Bm"][:, k:], s["Cm"][:, k:], s["dt"][:, k:], s["A"], s["D"],
                            mid, st2, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([y1, y2], 1), y) and torch.equal(st2, st)


@pytest.mark.parametrize("ws", [pytest.param(None, id="f16"), pytest.param(False, id="split")])
def test_scan_bf16_output_is_rounded_fp32_output(ws):
    d = LayerDims(2, 300, 4, 64, 2, 128)
    s = cuda(scan_inputs(d, 60))
    y32, f32_ = run_scan(s, ydt=torch.float32, ws=ws)
    y16, f16_ = run_scan(s, ydt=torch.bfloat16, ws=ws)
    assert torch.equal(y16, y32.to(torch.bfloat16))
    assert torch.equal(f16_, f32_)


def test_scan_views_into_conv_output_and_aliased_state(orc):
    d = LayerDims(2, 260, 4, 64, 2, 128)
    inp = cuda(mixer_inputs(d, 61, init_state=True))
    v = ssd.ssd_conv1d_fwd(inp["xbc"], inp["w"], inp["bias"])
    x, Bm, Cm = ssd.split_xbc(v, 4, 64, 2, 128)
    st = inp["init_state"].clone()
    y = ssd.ssd_chunk_scan(x, Bm, Cm, inp["dt"], inp["A"], inp["D"], st, st, y_dtype=torch.float32)
    torch.cuda.synchronize()
    vr, _, yr, fr = oracle_mixer(orc, inp, d, init=inp["init_state"])
    assert_close(y, yr, BF16_BAR, "y")
    assert_close(st, fr, BF16_BAR, "state")


@pytest.mark.parametrize("scale", [(0.0, 0, 0), (-30, 0, 0), (24, 0, 0), (0, -40, 0), (0, 40, 0), (0, 0, -40),
                                   (0, 0, 40), (-20, 20, -20)])
def test_scan_f16_operand_scales(orc, scale):
    """The fp16 scan scales its operands by powers of two chosen from the data (x per chunk, B and C per
    (batch, group, chunk) tile, the weighted x, M and the state copy from scalar bounds): inputs far from
    O(1) -- x, B or C scaled by 2^ex, 2^eb, 2^ec, tiny and huge -- stay at the bf16 bar vs the oracle, and
    a tile that is entirely zero (scale (0, 0, 0) variant: B zero in the second chunk) is exact zeros."""
    ex, eb, ec = scale
    d = LayerDims(2, 300, 4, 64, 2, 128)
    s = cuda(scan_inputs(d, 63))
    s["x"] = (s["x"].float() * 2.0 ** ex).to(torch.bfloat16)
    s["Bm"] = (s["Bm"].float() * 2.0 ** eb).to(torch.bfloat16)
    s["Cm"] = (s["Cm"].float() * 2.0 ** ec).to(torch.bfloat16)
    s["init_state"] = s["init_state"] * 2.0 ** (ex + eb)
    if scale == (0.0, 0, 0):
        s["Bm"][:, 128:256] = 0
    y, fin = run_scan(s)
    yr, fr = oracle_scan(orc, s)
    assert_close(y, yr, BF16_BAR, "y")
    assert_close(fin, fr, BF16_BAR, "final state")


def test_scan_f16_workspace_given_or_allocated():
    """A caller-provided workspace (reused across calls of different sizes) gives the same bits as the
    one the binding allocates; a smaller one is rejected."""
    d = LayerDims(2, 300, 4, 64, 2, 128)
    s = cuda(scan_inputs(d, 64))
    y0, f0 = run_scan(s)
    n = ssd.ssd_chunk_scan_workspace_size(2, 300, 4, 64, 2, 128)
    assert n > 0
    ws = torch.empty(n + 4096, dtype=torch.uint8, device=DEV)
    y1, f1 = run_scan(s, ws=ws)
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    small = {k: (v[:1, :130] if k in ("x", "Bm", "Cm", "dt") else (v[:1] if k == "init_state" else v))
             for k, v in s.items()}
    small = {k: (v.contiguous() if isinstance(v, torch.Tensor) else v) for k, v in small.items()}
    y2, f2 = run_scan(small, ws=ws)
    y3, f3 = run_scan(small)
    assert torch.equal(y2, y3) and torch.equal(f2, f3)
    with pytest.raises(RuntimeError, match="WORKSPACE"):
        run_scan(s, ws=ws[:n - 16])


def test_scan_L0_copies_state():
    d = LayerDims(2, 0, 4, 64, 2, 128)
    s = cuda(scan_inputs(d, 62))
    fin = torch.empty_like(s["init_state"])
    ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], s["init_state"], fin)
    fin0 = torch.full_like(fin, 5.0)
    ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], None, fin0)
    torch.cuda.synchronize()
    assert torch.equal(fin, s["init_state"]) and torch.count_nonzero(fin0) == 0


# --------------------------------------------------------------------------- invariants on the GPU
# The bf16 scans at (P, N) = (64, 128) run on two kernels: the fp16 single-pass one (the default, with a
# workspace) and the bf16 split-operand one (workspace=False).  Each invariant runs on both.
KERNELS = [pytest.param(None, id="f16"), pytest.param(False, id="split")]


@pytest.mark.parametrize("ws", KERNELS)
@pytest.mark.parametrize("P,N", [(64, 128), (16, 16)])
def test_invariant_null_init_equals_zero_init_and_determinism(P, N, ws):
    d = LayerDims(2, 333, 4, P, 2, N)
    s = cuda(scan_inputs(d, 70))
    y0, f0 = run_scan(s, init=None, ws=ws)
    s0 = dict(s)
    s0["init_state"] = torch.zeros_like(s["init_state"])
    yz, fz = run_scan(s0, ws=ws)
    assert torch.equal(y0, yz) and torch.equal(f0, fz)
    y1, f1 = run_scan(s, ws=ws)
    y2, f2 = run_scan(s, ws=ws)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


@pytest.mark.parametrize("ws", KERNELS)
def test_invariant_dt_zero_keeps_state(ws):
    d = LayerDims(2, 300, 4, 64, 2, 128)
    s = cuda(scan_inputs(d, 71))
    s["dt"] = torch.zeros_like(s["dt"])
    _, fin = run_scan(s, ws=ws)
    assert torch.equal(fin, s["init_state"])


@pytest.mark.parametrize("ws", KERNELS)
def test_invariant_reset_under_huge_decay(orc, ws):
    d = LayerDims(2, 200, 4, 64, 2, 128)
    s = cuda(scan_inputs(d, 72))
    s["A"] = torch.full_like(s["A"], -1e6)
    y, fin = run_scan(s, ws=ws)
    assert torch.isfinite(y).all() and torch.isfinite(fin).all()
    yr, fr = oracle_scan(orc, s)
    assert_close(y, yr, BF16_BAR, "y")
    assert_close(fin, fr, BF16_BAR, "state")


@pytest.mark.parametrize("ws", KERNELS)
def test_invariant_linearity_and_batch_permutation(ws):
    """Batch entries are independent: permuting them permutes the results bit for bit.  Doubling x and the
    initial state doubles y and the state: exactly on the split kernel (every product scales by an exact
    factor 2); within fp16 rounding on the fp16 one, whose operand scales follow the data and whose
    smallest weighted-x values round as fp16 subnormals."""
    d = LayerDims(3, 260, 4, 64, 2, 128)
    s = cuda(scan_inputs(d, 73))
    y, f = run_scan(s, ws=ws)
    s2 = dict(s)
    s2["x"] = s["x"] * 2
    s2["init_state"] = s["init_state"] * 2
    y2, f2 = run_scan(s2, ws=ws)
    if ws is False:
        assert torch.equal(y2, 2 * y) and torch.equal(f2, 2 * f)
    else:
        assert_close(y2, f64(2 * y), 2e-4, "2x y")
        assert_close(f2, f64(2 * f), 2e-4, "2x state")
    perm = torch.tensor([2, 0, 1], device=DEV)
    sp = {k: (v[perm] if k in ("x", "Bm", "Cm", "dt", "init_state") else v) for k, v in s.items()}
    yp, fp_ = run_scan(sp, ws=ws)
    assert torch.equal(yp, y[perm]) and torch.equal(fp_, f[perm])


@pytest.mark.parametrize("ws", KERNELS)
def test_invariant_split_prefill_and_decode_continuation(orc, ws):
    """prefill(L1) -> prefill(L2 from its state) == prefill(L1+L2); then decode steps continue it.  The two
    ways agree to 1e-5 on the split kernel (fp32 products of bf16 halves) and to fp16 rounding (2e-4 of
    the largest value, well inside the bf16 bar) on the fp16 one, where chunk boundaries move."""
    d = LayerDims(2, 384, 4, 64, 2, 128)
    s = cuda(scan_inputs(d, 74))
    y_all, f_all = run_scan(s, ws=ws)
    L1 = 200
    a = {k: (v[:, :L1].contiguous() if k in ("x", "Bm", "Cm", "dt") else v) for k, v in s.items()}
    bpart = {k: (v[:, L1:].contiguous() if k in ("x", "Bm", "Cm", "dt") else v) for k, v in s.items()}
    y1, f1 = run_scan(a, ws=ws)
    bpart["init_state"] = f1
    y2, f2 = run_scan(bpart, ws=ws)
    tol = 1e-5 if ws is False else 1e-3
    assert_close(torch.cat([y1, y2], 1), f64(y_all), tol, "split y")
    assert_close(f2, f64(f_all), tol, "split state")
    # decode: continue from f_all with the state update, compare with the oracle over the longer sequence
    st = f_all.clone()
    dec = cuda(scan_inputs(d.with_(seqlen=4), 75))
    ys = [ssd.ssd_state_update(st, dec["x"][:, t], dec["Bm"][:, t], dec["Cm"][:, t], dec["dt"][:, t].contiguous(),
                               s["A"], s["D"], y_dtype=torch.float32) for t in range(4)]
    torch.cuda.synchronize()
    cat = {k: torch.cat([s[k], dec[k]], 1) for k in ("x", "Bm", "Cm", "dt")}
    yr, fr = orc.scan(f64(cat["x"]), f64(cat["Bm"]), f64(cat["Cm"]), f64(cat["dt"]), f64(s["A"]), f64(s["D"]),
                      f64(s["init_state"]))
    assert_close(torch.stack(ys, 1), yr[:, -4:], BF16_BAR, "decode y")
    assert_close(st, fr, BF16_BAR, "decode state")


@pytest.mark.parametrize("ws", KERNELS)
def test_invariant_scan_L1_equals_state_update(ws):
    """A one-token scan is one state update: to 1e-5 on the split kernel, to fp16 rounding of the state
    copy and operands (1e-3) on the fp16 one."""
    d = LayerDims(2, 1, 4, 64, 2, 128)
    s = cuda(scan_inputs(d, 76))
    y, fin = run_scan(s, ws=ws)
    st = s["init_state"].clone()
    yu = ssd.ssd_state_update(st, s["x"][:, 0], s["Bm"][:, 0], s["Cm"][:, 0], s["dt"][:, 0], s["A"], s["D"],
                              y_dtype=torch.float32)
    torch.cuda.synchronize()
    tol = 1e-5 if ws is False else 1e-3
    assert_close(fin, f64(st), tol, "state")
    assert_close(y[:, 0], f64(yu), tol, "y")


@pytest.mark.parametrize("ws", KERNELS)
def test_invariant_identical_groups_equal_one_group(ws):
    d = LayerDims(2, 200, 4, 64, 1, 128)
    s = cuda(scan_inputs(d, 77))
    y1, f1 = run_scan(s, ws=ws)
    s2 = dict(s)
    s2["Bm"] = s["Bm"].repeat(1, 1, 2, 1)
    s2["Cm"] = s["Cm"].repeat(1, 1, 2, 1)
    y2, f2 = run_scan(s2, ws=ws)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


# --------------------------------------------------------------------------- whole mixer
def test_tiny_fp32_mixer_prefill_then_decode(orc):
    """Tiny fp32 mixer: 256-token prefill (chunk 64) then 8 decode steps, vs the oracle."""
    d = WORKLOADS["tiny_fp32"]
    inp = cuda(mixer_inputs(d, 1000))
    cs = torch.zeros(1, d.conv_dim, 4, device=DEV)
    v = ssd.ssd_conv1d_fwd(inp["xbc"], inp["w"], inp["bias"], None, cs)
    x, Bm, Cm = ssd.split_xbc(v, d.nheads, d.head_dim, d.ngroups, d.d_state)
    st = torch.empty(1, d.nheads, d.head_dim, d.d_state, device=DEV)
    y = ssd.ssd_chunk_scan(x, Bm, Cm, inp["dt"], inp["A"], inp["D"], None, st, chunk=d.chunk)
    dec = cuda(decode_tokens(d, 1001, 8))
    ys = []
    for k in range(8):
        u = ssd.ssd_conv1d_update(dec["xbc"][k], inp["w"], inp["bias"], cs)
        xk, Bk, Ck = ssd.split_xbc(u, d.nheads, d.head_dim, d.ngroups, d.d_state)
        ys.append(ssd.ssd_state_update(st, xk, Bk, Ck, dec["dt"][k], inp["A"], inp["D"]))
    torch.cuda.synchronize()
    # oracle: the whole 264-token sequence as one prefill
    full = dict(inp)
    full["xbc"] = torch.cat([inp["xbc"], dec["xbc"].transpose(0, 1)], 1)
    full["dt"] = torch.cat([inp["dt"], dec["dt"].transpose(0, 1)], 1)
    _, sr, yr, fr = oracle_mixer(orc, full, d)
    assert_close(y, yr[:, :256], F32_BAR, "prefill y")
    assert_close(torch.stack(ys, 1), yr[:, 256:], F32_BAR, "decode y")
    assert_close(st, fr, F32_BAR, "final state")
    assert np.array_equal(f64(cs), sr)


def test_ultra_geometry_mini_smoke(orc):
    """Real Ultra-layer geometry (CD 18432, 256 heads) at a short prefill, all heads checked."""
    d = WORKLOADS["prefill_ultra_8k"].with_(batch=2, seqlen=192)
    inp = cuda(mixer_inputs(d, 1002, conv_state=True, init_state=True))
    so = torch.empty_like(inp["conv_state"])
    v = ssd.ssd_conv1d_fwd(inp["xbc"], inp["w"], inp["bias"], inp["conv_state"], so)
    x, Bm, Cm = ssd.split_xbc(v, d.nheads, d.head_dim, d.ngroups, d.d_state)
    st = torch.empty_like(inp["init_state"])
    y = ssd.ssd_chunk_scan(x, Bm, Cm, inp["dt"], inp["A"], inp["D"], inp["init_state"], st, y_dtype=torch.float32)
    torch.cuda.synchronize()
    vr, sr, yr, fr = oracle_mixer(orc, inp, d, conv_state=inp["conv_state"], init=inp["init_state"])
    assert_bf16_elementwise(v, vr, "conv")
    assert np.array_equal(f64(so), sr)
    # the scan consumed the GPU's bf16 conv output; the oracle its own bf16-rounded conv output
    assert_close(y, yr, BF16_BAR, "y")
    assert_close(st, fr, BF16_BAR, "state")


def test_split_scan_bounded_wait_running_out_is_visible():
    """The split kernel's state waves wait (boundedly) for the y waves to have read the carried state
    before overwriting it.  Forced to run out at once (SSD_SCAN_SPIN_MAX=0, read when the library
    launches its first split scan, so in a child process), they poison the state: every y after the
    first chunk and the final state are NaN, where a silent race could otherwise pass unnoticed.  The
    kernel still ends normally."""
    import os
    import subprocess
    import sys
    code = r'''
import torch
from selective_state_space_conv1d_amd import ssd
from selective_state_space_conv1d_amd.synth import LayerDims, scan_inputs
s = {k: (v.to("cuda") if isinstance(v, torch.Tensor) else v) for k, v in scan_inputs(LayerDims(1, 300, 4, 64, 2, 128), 78).items()}
fin = torch.empty_like(s["init_state"])
y = ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], s["init_state"], fin, y_dtype=torch.float32,
                       workspace=False)
torch.cuda.synchronize()
print(int(torch.isfinite(y[:, :128]).all()), int(torch.isnan(y[:, 128:]).all()), int(torch.isnan(fin).all()))
'''
    env = dict(os.environ, SSD_SCAN_SPIN_MAX="0")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=240,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split()[-3:] == ["1", "1", "1"], r.stdout
