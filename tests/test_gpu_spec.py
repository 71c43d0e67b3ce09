"""Parity of the multi-token (speculative) decode calls and the accept step, on the GPU.

Checked against the oracle's multi-token forms (pinned in tests/test_oracle_spec.py), and bitwise
against k calls of the single-token kernels, which run the same fp32 arithmetic per token.
Cases: per-request states and slot pools with padding; accept lengths 0, 1, k and above k.
"""
import numpy as np
import pytest
import torch

from gpu_util import BF16_BAR, F32_BAR, assert_bf16_elementwise, assert_close, f64
from selective_state_space_conv1d_amd import ssd
from selective_state_space_conv1d_amd.synth import WORKLOADS, LayerDims, scan_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def ssm_inputs(d, k, seed):
    return {n: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for n, v in scan_inputs(d, seed, seqlen=k).items()}


def conv_inputs(d, k, nstate, seed):
    CD = d.conv_dim
    g = torch.Generator(device="cpu").manual_seed(seed)
    xbc = torch.randn(d.batch, k, CD, generator=g).to(d.dtype).to(DEV)
    w = (torch.rand(CD, 4, generator=g) - 0.5).to(d.dtype).to(DEV)
    bias = (torch.rand(CD, generator=g) - 0.5).to(d.dtype).to(DEV)
    pool = torch.randn(nstate, CD, 4, generator=g).to(d.dtype).to(DEV)
    return xbc, w, bias, pool


@pytest.mark.parametrize("H,P,N,dtype", [(8, 64, 128, torch.bfloat16), (8, 16, 32, torch.float32),
                                         (6, 16, 16, torch.bfloat16)])   # the last: blocks straddle requests
@pytest.mark.parametrize("use_slots", [False, True])
def test_state_update_multi_matches_oracle(orc, H, P, N, dtype, use_slots):
    d = LayerDims(4, 1, H, P, 2, N, dtype=dtype)
    k = 5
    s = ssm_inputs(d, k, 400)
    if use_slots:
        pool0 = torch.randn(6, H, P, N, device=DEV) * 0.1
        slots = [5, -1, 0, 3]
        slot = torch.tensor(slots, dtype=torch.int32, device=DEV)
    else:
        pool0, slots, slot = s["init_state"], None, None
    pool = pool0.clone()
    y, inter = ssd.ssd_state_update_multi(pool, s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], slot_idx=slot,
                                          y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool0), "the multi-token update must not write the main state"
    yr, ir = orc.state_update_multi(f64(pool0), None if slots is None else np.array(slots), f64(s["x"]),
                                    f64(s["Bm"]), f64(s["Cm"]), f64(s["dt"]), f64(s["A"]), f64(s["D"]))
    assert_close(y, yr, F32_BAR, "y")
    assert_close(inter, ir, F32_BAR, "intermediate states")


# (batch, H, P, G, N): the Ultra layer; blocks of 256 float4 that straddle requests (H*P*N/4 = 192
# and 384) and so find each thread's request on their own; other row widths (N/8 lanes per row)
STRADDLE = [(5, 3, 16, 1, 16), (4, 3, 16, 3, 32), (3, 5, 32, 5, 64)]


@pytest.mark.parametrize("shape", [None] + STRADDLE)
def test_state_update_multi_is_k_single_updates_bitwise(shape):
    d = WORKLOADS["decode_ultra_b64"].with_(batch=6) if shape is None else LayerDims(shape[0], 1, *shape[1:])
    k = 4
    s = ssm_inputs(d, k, 410)
    y, inter = ssd.ssd_state_update_multi(s["init_state"], s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"])
    st = s["init_state"].clone()
    for j in range(k):
        yj = ssd.ssd_state_update(st, s["x"][:, j], s["Bm"][:, j], s["Cm"][:, j], s["dt"][:, j].contiguous(),
                                  s["A"], s["D"])
        torch.cuda.synchronize()
        assert torch.equal(y[:, j], yj), j
        assert torch.equal(inter[:, j], st), j


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("shape", [None] + STRADDLE + ["fp32", "fp32_straddle"])
def test_multi_y_only_form(orc, k, shape):
    """y without intermediate states: for 2 <= k <= 4 the chunk (dual) form, which sums the same value
    in another order -- within the fp32 bar of the oracle and of the sequential form; k = 1 and k > 4
    run the sequential form, bitwise the y of the call with intermediate states (k = 1: the
    single-token update)."""
    if shape is None:
        d = WORKLOADS["decode_ultra_b64"].with_(batch=5)
    elif shape == "fp32":                      # fp32 activations: the quads are f32x4, C.B by FMAs
        d = LayerDims(3, 1, 8, 64, 2, 128, dtype=torch.float32)
    elif shape == "fp32_straddle":
        d = LayerDims(5, 1, 3, 16, 1, 16, dtype=torch.float32)
    else:
        d = LayerDims(shape[0], 1, *shape[1:])
    s = ssm_inputs(d, k, 415)
    args = (s["init_state"], s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"])
    y_seq, _ = ssd.ssd_state_update_multi(*args, y_dtype=torch.float32)
    y_only, none = ssd.ssd_state_update_multi(*args, inter_states=None, y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert none is None
    if k == 1 or k > 4:
        assert torch.equal(y_only, y_seq)
    if k == 1:
        st = s["init_state"].clone()
        y1 = ssd.ssd_state_update(st, s["x"][:, 0], s["Bm"][:, 0], s["Cm"][:, 0], s["dt"][:, 0].contiguous(),
                                  s["A"], s["D"], y_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y_only[:, 0], y1)
    assert_close(y_only, f64(y_seq), F32_BAR, "y against the sequential form")
    yr, _ = orc.state_update_multi(f64(s["init_state"]), None, f64(s["x"]), f64(s["Bm"]), f64(s["Cm"]),
                                   f64(s["dt"]), f64(s["A"]), f64(s["D"]))
    assert_close(y_only, yr, F32_BAR, "y against the oracle")


def test_state_update_multi_dt_prologue(orc):
    d = LayerDims(3, 1, 4, 64, 2, 128)
    k = 3
    s = ssm_inputs(d, k, 420)
    raw = (torch.randn(3, k, 4, device=DEV) - 1.0).to(torch.bfloat16)
    bias = torch.randn(4, device=DEV)
    y, inter = ssd.ssd_state_update_multi(s["init_state"], s["x"], s["Bm"], s["Cm"], raw, s["A"], s["D"],
                                          y_dtype=torch.float32, dt_bias=bias, dt_softplus=True, dt_limit=(0.0, 2.0))
    torch.cuda.synchronize()
    dt_eff = orc.dt_prologue(f64(raw), f64(bias), True, (0.0, 2.0))
    yr, ir = orc.state_update_multi(f64(s["init_state"]), None, f64(s["x"]), f64(s["Bm"]), f64(s["Cm"]), dt_eff,
                                    f64(s["A"]), f64(s["D"]))
    assert_close(y, yr, F32_BAR, "y")
    assert_close(inter, ir, F32_BAR, "intermediate states")
    y2, _ = ssd.ssd_state_update_multi(s["init_state"], s["x"], s["Bm"], s["Cm"], raw, s["A"], s["D"],
                                       inter_states=None, y_dtype=torch.float32, dt_bias=bias, dt_softplus=True,
                                       dt_limit=(0.0, 2.0))
    torch.cuda.synchronize()
    assert_close(y2, yr, F32_BAR, "y without intermediate states")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_conv_update_multi_matches_oracle_and_single_steps(orc, dtype):
    d = LayerDims(5, 1, 4, 16, 1, 16, dtype=dtype)       # CD = 96
    k = 4
    xbc, w, bias, pool0 = conv_inputs(d, k, 7, 430)
    slots = [6, -1, 2, 0, 7]                              # -1 and 7 (>= nslots) are padding
    slot = torch.tensor(slots, dtype=torch.int32, device=DEV)
    out, inter = ssd.ssd_conv1d_update_multi(xbc, w, bias, pool0, slot_idx=slot)
    torch.cuda.synchronize()
    vr, ir = orc.conv1d_update_multi(f64(xbc), f64(w), f64(bias), f64(pool0), np.array(slots))
    if dtype == torch.bfloat16:
        assert_bf16_elementwise(out.cpu(), vr, "conv out")
    else:
        assert_close(out, vr, F32_BAR, "conv out")
    assert np.array_equal(f64(inter), ir), "intermediate windows are copies of inputs"
    # bitwise against k single-token updates of the same slots (padding requests excluded: the
    # multi-token call rolls their zero-started window, a single-token call restarts it each time)
    pool = pool0.clone()
    real = [b for b, sl in enumerate(slots) if 0 <= sl < pool0.shape[0]]
    for j in range(k):
        vj = ssd.ssd_conv1d_update_slots(xbc[:, j], w, bias, pool, slot)
        torch.cuda.synchronize()
        assert torch.equal(out[real, j], vj[real]), j


@pytest.mark.parametrize("use_slots", [False, True])
def test_accept_writes_back_the_state_after_n_tokens(use_slots):
    d = LayerDims(5, 1, 8, 64, 2, 128)
    k = 4
    s = ssm_inputs(d, k, 440)
    xbc, w, bias, cpool0 = conv_inputs(d, k, 8 if use_slots else 5, 441)
    if use_slots:
        spool0 = torch.randn(8, 8, 64, 128, device=DEV) * 0.1
        slots = [7, 2, -1, 0, 5]
        slot = torch.tensor(slots, dtype=torch.int32, device=DEV)
    else:
        spool0, slots, slot = s["init_state"], list(range(5)), None
    acc = torch.tensor([2, 0, 3, 4, 9], dtype=torch.int32, device=DEV)   # 9 > k clamps to k
    _, inter = ssd.ssd_state_update_multi(spool0, s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], slot_idx=slot)
    _, cinter = ssd.ssd_conv1d_update_multi(xbc, w, bias, cpool0, slot_idx=slot)
    spool, cpool = spool0.clone(), cpool0.clone()
    ssd.ssd_accept_states(acc, spool, inter, cpool, cinter, slot_idx=slot)
    torch.cuda.synchronize()
    named = set()
    for b, n in enumerate(acc.tolist()):
        sl = slots[b]
        if sl < 0:
            continue
        named.add(sl)
        n = min(n, k)
        # reference: n single-token updates from the slot's state
        st = spool0[sl:sl + 1].clone()
        cs = cpool0[sl:sl + 1].clone()
        for j in range(n):
            ssd.ssd_state_update(st, s["x"][b:b + 1, j], s["Bm"][b:b + 1, j], s["Cm"][b:b + 1, j],
                                 s["dt"][b:b + 1, j].contiguous(), s["A"], s["D"])
            ssd.ssd_conv1d_update(xbc[b:b + 1, j], w, bias, cs)
        torch.cuda.synchronize()
        assert torch.equal(spool[sl], st[0]), (b, n)
        assert torch.equal(cpool[sl], cs[0]), (b, n)
    for sl in range(spool.shape[0]):
        if sl not in named:
            assert torch.equal(spool[sl], spool0[sl]) and torch.equal(cpool[sl], cpool0[sl]), sl


def test_accept_one_pair_only():
    d = LayerDims(3, 1, 4, 16, 1, 32, dtype=torch.float32)
    k = 2
    s = ssm_inputs(d, k, 450)
    _, inter = ssd.ssd_state_update_multi(s["init_state"], s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"])
    st = s["init_state"].clone()
    ssd.ssd_accept_states(torch.tensor([1, 2, 0], dtype=torch.int32, device=DEV), st, inter)
    torch.cuda.synchronize()
    assert torch.equal(st[0], inter[0, 0]) and torch.equal(st[1], inter[1, 1])
    assert torch.equal(st[2], s["init_state"][2])


def test_full_size_speculative_step_sampled(orc):
    """Batch 64 of the Ultra decode layer with k = 4 candidates and a 96-slot pool: bitwise against
    single-token updates on sampled requests, and the oracle on one head per group of one request."""
    d = WORKLOADS["decode_ultra_b64"]
    k = 4
    s = ssm_inputs(d, k, 460)
    g = torch.Generator(device="cpu").manual_seed(461)
    pool0 = torch.randn(96, d.nheads, d.head_dim, d.d_state, generator=g).to(DEV) * 0.1
    slot = torch.randperm(96, generator=g)[:64].to(torch.int32).to(DEV)
    acc = torch.randint(0, k + 1, (64,), generator=g).to(torch.int32).to(DEV)
    y, inter = ssd.ssd_state_update_multi(pool0, s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], slot_idx=slot,
                                          y_dtype=torch.float32)
    pool = pool0.clone()
    ssd.ssd_accept_states(acc, pool, inter, slot_idx=slot)
    torch.cuda.synchronize()
    for b in (0, 17, 63):
        sl = int(slot[b])
        st = pool0[sl:sl + 1].clone()
        n = int(acc[b])
        for j in range(k):
            yj = ssd.ssd_state_update(st, s["x"][b:b + 1, j], s["Bm"][b:b + 1, j], s["Cm"][b:b + 1, j],
                                      s["dt"][b:b + 1, j].contiguous(), s["A"], s["D"], y_dtype=torch.float32)
            torch.cuda.synchronize()
            assert torch.equal(y[b:b + 1, j], yj) and torch.equal(inter[b, j], st[0]), (b, j)
            if j + 1 == n:
                assert torch.equal(pool[sl], st[0]), b
        if n == 0:
            assert torch.equal(pool[sl], pool0[sl]), b
    # oracle on request 17, one head per group: sampled head i belongs to group i, so the 8 heads
    # with all 8 groups' B and C form a consistent smaller layer
    b = 17
    sl = int(slot[b])
    heads = [gi * (d.nheads // d.ngroups) for gi in range(d.ngroups)]
    sub = lambda t: f64(t[b:b + 1])
    yr, ir = orc.state_update_multi(f64(pool0[sl:sl + 1, heads]), None, sub(s["x"])[:, :, heads], sub(s["Bm"]),
                                    sub(s["Cm"]), sub(s["dt"])[:, :, heads], f64(s["A"])[heads], f64(s["D"])[heads])
    assert_close(y[b:b + 1, :, heads], yr, F32_BAR, "y sampled heads")
    assert_close(inter[b:b + 1, :, heads], ir, F32_BAR, "intermediate states sampled heads")


# --------------------------------------------------------------------------- state snapshots
@pytest.mark.parametrize("P,N,dtype,L,iv", [(64, 128, torch.bfloat16, 700, 128), (64, 128, torch.bfloat16, 1024, 256),
                                            (16, 32, torch.float32, 300, 128), (16, 32, torch.float32, 256, 128)])
def test_scan_snapshots(orc, P, N, dtype, L, iv):
    d = LayerDims(2, L, 4, P, 2, N, dtype=dtype)
    s = {n: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for n, v in scan_inputs(d, 470).items()}
    fin = torch.empty_like(s["init_state"])
    snaps = torch.full((2, L // iv, 4, P, N), float("nan"), device=DEV)
    y = ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], s["init_state"], fin,
                           y_dtype=torch.float32, snapshots=snaps, snapshot_interval=iv)
    # snapshot calls run on the split-operand kernel: the same call without snapshots on that kernel
    fin2 = torch.empty_like(fin)
    y2 = ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], s["init_state"], fin2,
                            y_dtype=torch.float32, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(y, y2) and torch.equal(fin, fin2), "snapshots must not change y or the final state"
    if L % iv == 0:
        assert torch.equal(snaps[:, -1], fin), "the last snapshot is the final state"
    yr, fr, sr = orc.scan_snapshots(f64(s["x"]), f64(s["Bm"]), f64(s["Cm"]), f64(s["dt"]), f64(s["A"]), f64(s["D"]),
                                    f64(s["init_state"]), iv)
    bar = BF16_BAR if dtype == torch.bfloat16 else F32_BAR
    assert_close(y, yr, bar, "y")
    assert_close(snaps, sr, bar, "snapshots")


# --------------------------------------------------------------------------- accept by recomputation
@pytest.mark.parametrize("use_slots", [False, True])
@pytest.mark.parametrize("k,H,P,N", [(4, 8, 64, 128), (7, 8, 64, 128), (4, 3, 16, 16)])   # the last: straddling blocks
def test_accept_by_recomputation_is_the_stored_intermediate(use_slots, k, H, P, N):
    d = LayerDims(6, 1, H, P, 1, N)
    s = ssm_inputs(d, k, 480)
    xbc, w, bias, cpool0 = conv_inputs(d, k, 9 if use_slots else 6, 481)
    if use_slots:
        spool0 = torch.randn(9, H, P, N, device=DEV) * 0.1
        slots = [7, 2, -1, 0, 5, 8]
        slot = torch.tensor(slots, dtype=torch.int32, device=DEV)
    else:
        spool0, slots, slot = s["init_state"], list(range(6)), None
    acc = torch.tensor([2, 0, 3, k, 9, 1], dtype=torch.int32, device=DEV)    # 9 > k clamps to k
    # y with and without intermediate states: the same values (summed in another order for k <= 4)
    y1, inter = ssd.ssd_state_update_multi(spool0, s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], slot_idx=slot)
    y2, none = ssd.ssd_state_update_multi(spool0, s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], slot_idx=slot,
                                          inter_states=None)
    _, cinter = ssd.ssd_conv1d_update_multi(xbc, w, bias, cpool0, slot_idx=slot)
    sp_copy, cp_copy = spool0.clone(), cpool0.clone()
    ssd.ssd_accept_states(acc, sp_copy, inter, cp_copy, cinter, slot_idx=slot)
    sp_re, cp_re = spool0.clone(), cpool0.clone()
    ssd.ssd_state_update_accept(sp_re, s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], acc, slot_idx=slot)
    ssd.ssd_conv1d_update_accept(xbc, cp_re, acc, slot_idx=slot)
    torch.cuda.synchronize()
    assert none is None
    assert_close(y2, f64(y1), BF16_BAR, "y without intermediate states")
    assert torch.equal(sp_re, sp_copy), "recomputed states must equal the stored intermediate ones"
    assert torch.equal(cp_re, cp_copy), "recomputed conv windows must equal the stored ones"


@pytest.mark.parametrize("H,P,N", [(8, 64, 128), (3, 16, 16)])
def test_multi_y_with_x_rows_not_a_multiple_of_four_apart(H, P, N):
    """x token rows H*P + 2 elements apart (the four x values of a row group are then loaded one by
    one): y, and the recomputed accept, bitwise as with packed x."""
    d = LayerDims(5, 1, H, P, 1, N)
    k = 3
    s = ssm_inputs(d, k, 490)
    wide = torch.zeros(d.batch, k, H * P + 2, dtype=s["x"].dtype, device=DEV)
    wide[..., :H * P] = s["x"].reshape(d.batch, k, H * P)
    xo = wide[..., :H * P].view(d.batch, k, H, P)
    assert xo.stride(1) == H * P + 2
    args = (s["Bm"], s["Cm"], s["dt"], s["A"], s["D"])
    y1, _ = ssd.ssd_state_update_multi(s["init_state"], s["x"], *args, inter_states=None)
    y2, _ = ssd.ssd_state_update_multi(s["init_state"], xo, *args, inter_states=None)
    acc = torch.tensor([1, 3, 0, 2, 3], dtype=torch.int32, device=DEV)
    st1, st2 = s["init_state"].clone(), s["init_state"].clone()
    ssd.ssd_state_update_accept(st1, s["x"], *args[:2], s["dt"], s["A"], s["D"], acc)
    ssd.ssd_state_update_accept(st2, xo, *args[:2], s["dt"], s["A"], s["D"], acc)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(st1, st2)
