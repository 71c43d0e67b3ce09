"""Parity of the packed-batch (varlen) and state-pool entry points with the oracle, on the GPU.

The oracle's varlen forms run its pinned per-sequence routines (tests/test_oracle_varlen.py).
Cases: empty, one-token and ragged sequences; conv token tiles straddling sequence boundaries;
permuted slots; padding slots; mixed has_initial_state.  Also the packed call with equal lengths
must reproduce the batched call bitwise, and a full-size serving mix is checked on sampled heads.
"""
import numpy as np
import pytest
import torch

from gpu_util import BF16_BAR, F32_BAR, assert_bf16_elementwise, assert_close, f64, to_act
from selective_state_space_conv1d_amd import ssd
from selective_state_space_conv1d_amd.synth import (LayerDims, WORKLOADS, scan_inputs, varlen_inputs,
                                                    varlen_lengths)

pytestmark = pytest.mark.gpu
DEV = "cuda"

LENS = [1, 0, 127, 128, 129, 300, 5, 256, 33]


def tables(lens, slots, has_init):
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    mk = lambda a: None if a is None else torch.tensor(a, dtype=torch.int32, device=DEV)
    return cu, mk(slots), mk(has_init)


def packed_scan(d, lens, seed, slow=False):
    T = int(sum(lens))
    s = scan_inputs(d.with_(batch=1, seqlen=T), seed, slow=slow, init_state=False)
    return {k: v[0].to(DEV) if k in ("x", "Bm", "Cm", "dt") else v.to(DEV) for k, v in s.items() if v is not None}


def run_scan_varlen(s, cu, slot, has_init, pool, chunk=128, ydt=torch.float32, ws=None):
    """ws None: the default (the fp16 scan where it applies); False: the bf16 split-operand kernel."""
    y = ssd.ssd_chunk_scan_varlen(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], cu, pool, slot, has_init,
                                  chunk=chunk, y_dtype=ydt, workspace=ws)
    torch.cuda.synchronize()
    return y


# --------------------------------------------------------------------------- scan
WS = [pytest.param(None, id="f16"), pytest.param(False, id="split")]


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("slow", [False, True])
def test_scan_varlen_mfma(orc, slow, ws):
    d = LayerDims(1, 1, 4, 64, 2, 128)
    s = packed_scan(d, LENS, 200 + slow, slow=slow)
    nslots = 12
    slots = [7, 3, -1, 0, 12, 5, 9, 1, 11]          # -1 and 12 (>= nslots) are padding
    has_init = [1, 0, 1, 1, 1, 0, 1, 1, 0]
    cu, slot, hi = tables(LENS, slots, has_init)
    pool0 = torch.randn(nslots, 4, 64, 128, device=DEV) * 0.1
    pool = pool0.clone()
    y = run_scan_varlen(s, cu, slot, hi, pool, ws=ws)
    yr, pr = orc.scan_varlen(f64(s["x"]), f64(s["Bm"]), f64(s["Cm"]), f64(s["dt"]), f64(s["A"]), f64(s["D"]),
                             cu.cpu().numpy(), f64(pool0), np.array(slots), np.array(has_init))
    assert_close(y, yr, BF16_BAR, "y")
    named = [k for k in slots if 0 <= k < nslots]
    assert_close(pool[named], pr[named], BF16_BAR, "final states")
    others = [k for k in range(nslots) if k not in named]
    assert torch.equal(pool[others], pool0[others]), "slots no sequence names must be untouched"
    # bf16 output mode is the RNE of the fp32 output
    pool2 = pool0.clone()
    y16 = run_scan_varlen(s, cu, slot, hi, pool2, ydt=torch.bfloat16, ws=ws)
    assert torch.equal(y16, y.to(torch.bfloat16)) and torch.equal(pool2, pool)


def test_scan_varlen_fp32_path(orc):
    d = LayerDims(1, 1, 4, 16, 1, 16, chunk=64, dtype=torch.float32)
    lens = [3, 64, 0, 65, 1, 100]
    s = packed_scan(d, lens, 210)
    nslots = 8
    slots, has_init = [2, 7, 4, -1, 0, 5], [1, 1, 0, 1, 0, 1]
    cu, slot, hi = tables(lens, slots, has_init)
    pool0 = torch.randn(nslots, 4, 16, 16, device=DEV) * 0.1
    pool = pool0.clone()
    y = run_scan_varlen(s, cu, slot, hi, pool, chunk=64)
    yr, pr = orc.scan_varlen(f64(s["x"]), f64(s["Bm"]), f64(s["Cm"]), f64(s["dt"]), f64(s["A"]), f64(s["D"]),
                             cu.cpu().numpy(), f64(pool0), np.array(slots), np.array(has_init))
    assert_close(y, yr, F32_BAR, "y")
    assert_close(pool, pr, F32_BAR, "pool")


@pytest.mark.parametrize("ws", WS)
@pytest.mark.parametrize("P,N", [(64, 128), (16, 32)])
def test_scan_varlen_equal_lengths_is_the_batched_scan(P, N, ws):
    d = LayerDims(3, 300, 8, P, 2, N)
    s = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in scan_inputs(d, 220).items()}
    fin = torch.empty_like(s["init_state"])
    # the packed scan runs the batched scan's kernel (fp16 with a workspace, else split-operand): bitwise equal
    yb = ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], s["init_state"], fin,
                            y_dtype=torch.float32, workspace=ws)
    pool = s["init_state"][[2, 0, 1]].clone()          # sequence b lives in slot perm[b]
    perm = torch.tensor([1, 2, 0], dtype=torch.int32, device=DEV)
    cu = torch.arange(4, dtype=torch.int32, device=DEV) * 300
    flat = lambda t: t.reshape((t.shape[0] * t.shape[1],) + tuple(t.shape[2:]))
    y = ssd.ssd_chunk_scan_varlen(flat(s["x"]), flat(s["Bm"]), flat(s["Cm"]), flat(s["dt"]), s["A"], s["D"],
                                  cu, pool, perm, torch.ones(3, dtype=torch.int32, device=DEV),
                                  y_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(3, 300, 8, P), yb)
    assert torch.equal(pool[perm.long()], fin)


def test_scan_varlen_f16_workspace_too_small_is_refused():
    d = LayerDims(1, 1, 4, 64, 2, 128)
    s = packed_scan(d, [130, 7], 231)
    cu, slot, hi = tables([130, 7], [0, 1], [0, 0])
    pool = torch.zeros(2, 4, 64, 128, device=DEV)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(Exception, match="WORKSPACE|workspace"):
        run_scan_varlen(s, cu, slot, hi, pool, ws=small)


def test_scan_varlen_no_tokens_copies_or_zeroes_states():
    d = LayerDims(1, 1, 4, 64, 2, 128)
    s = packed_scan(d, [0, 0], 230)
    pool0 = torch.randn(3, 4, 64, 128, device=DEV)
    pool = pool0.clone()
    cu, slot, hi = tables([0, 0], [2, 0], [1, 0])
    run_scan_varlen(s, cu, slot, hi, pool)
    assert torch.equal(pool[2], pool0[2]) and torch.equal(pool[1], pool0[1])
    assert not pool[0].any(), "an empty sequence without an initial state ends at zero"


# (H, P, G, N, dtype, chunk, lens): the MFMA scan walking sequence ranges (64 heads, 14 requests),
# and the FMA scan (fp32, chunk 64, one request per workgroup)
SNAP_CASES = [(64, 64, 8, 128, torch.bfloat16, 128, [0, 300, 128, 1, 700, 256, 5, 129, 384, 2, 40, 511, 127, 260]),
              (4, 16, 1, 16, torch.float32, 64, [130, 0, 256, 5, 400])]


@pytest.mark.parametrize("case", range(len(SNAP_CASES)))
def test_scan_varlen_snapshots(orc, case):
    H, P, G, N, dtype, chunk, lens = SNAP_CASES[case]
    d = LayerDims(1, 1, H, P, G, N, chunk=chunk, dtype=dtype)
    s = packed_scan(d, lens, 240 + case)
    S, iv = len(lens), 128
    r = np.random.default_rng(241 + case)
    nslots = S + 2
    slots = r.permutation(nslots)[:S].astype(np.int32)
    slots[3] = -1
    has_init = (r.random(S) < 0.5).astype(np.int32)
    cu, slot, hi = tables(lens, slots, has_init)
    maxs = 5
    nsnap = S * maxs // 2
    table = np.full((S, maxs), -1, dtype=np.int32)
    free = list(r.permutation(nsnap + 3))          # distinct slots, a few past the pool's end
    for q in range(S):
        for k in range(maxs):
            if free and r.random() < 0.8:
                table[q, k] = free.pop()
    pool0 = torch.randn(nslots, H, P, N, device=DEV) * 0.1
    snap0 = torch.randn(nsnap, H, P, N, device=DEV)
    pool, snaps = pool0.clone(), snap0.clone()
    tab = torch.tensor(table, device=DEV)
    y = ssd.ssd_chunk_scan_varlen(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], cu, pool, slot, hi, chunk=chunk,
                                  y_dtype=torch.float32, snapshot_pool=snaps, snapshot_table=tab,
                                  snapshot_interval=iv)
    pool2 = pool0.clone()     # the snapshot scan runs the split-operand kernel: compare with it without snapshots
    y2 = run_scan_varlen(s, cu, slot, hi, pool2, chunk=chunk, ws=False)
    assert torch.equal(y, y2) and torch.equal(pool, pool2), "snapshots must not change y or the states"
    hpg = H // G
    heads = list(range(H)) if H <= 4 else [g * hpg + (5 * g) % hpg for g in range(0, G, 3)]
    bar = F32_BAR if dtype == torch.float32 else BF16_BAR
    for h in heads:
        g = h // hpg
        yr, pr, sr = orc.scan_varlen_snapshots(
            f64(s["x"][:, h:h + 1]), f64(s["Bm"][:, g:g + 1]), f64(s["Cm"][:, g:g + 1]), f64(s["dt"][:, h:h + 1]),
            f64(s["A"][h:h + 1]), f64(s["D"][h:h + 1]), cu.cpu().numpy(), f64(pool0[:, h:h + 1]), slots, has_init,
            f64(snap0[:, h:h + 1]), table, iv)
        assert_close(y[:, h], yr[:, 0], bar, f"y head {h}")
        assert_close(snaps[:, h], sr[:, 0], bar, f"snapshot pool head {h}")
    written = {int(table[q, k]) for q in range(S) for k in range(min(lens[q] // iv, maxs))
               if 0 <= table[q, k] < nsnap}
    kept = [k for k in range(nsnap) if k not in written]
    assert torch.equal(snaps[kept], snap0[kept]), "slots the table does not name for a reached interval are untouched"


# --------------------------------------------------------------------------- conv
# token tiles are 24 rows: in the first layout a tile starts 2 rows into a sequence (row 48), in the
# second 1 row (row 24) and 0 rows (row 48); the window then takes state columns and input rows
CONV_LAYOUTS = {"mixed": [3, 0, 1, 2, 40, 31, 33, 65, 4], "tile_offsets": [23, 2, 20, 3, 1, 40, 0, 9, 5]}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("layout", list(CONV_LAYOUTS))
def test_conv_varlen(orc, dtype, layout):
    d = LayerDims(1, 1, 4, 16, 1, 16, dtype=dtype)      # CD = 96
    lens = CONV_LAYOUTS[layout]
    T, CD = sum(lens), d.conv_dim
    g = torch.Generator(device="cpu").manual_seed(240)
    xbc = torch.randn(T, CD, generator=g).to(dtype).to(DEV)
    w = (torch.rand(CD, 4, generator=g) - 0.5).to(dtype).to(DEV)
    bias = (torch.rand(CD, generator=g) - 0.5).to(dtype).to(DEV)
    nslots = 11
    slots, has_init = [4, 10, 0, -1, 7, 2, 9, 5, 1], [1, 1, 0, 1, 1, 0, 1, 0, 1]
    cu, slot, hi = tables(lens, slots, has_init)
    pool0 = torch.randn(nslots, CD, 4, generator=g).to(dtype).to(DEV)
    pool = pool0.clone()
    v = ssd.ssd_conv1d_fwd_varlen(xbc, w, bias, cu, pool, slot, hi)
    torch.cuda.synchronize()
    vr, pr = orc.conv1d_fwd_varlen(f64(xbc), f64(w), f64(bias), cu.cpu().numpy(), f64(pool0), np.array(slots),
                                   np.array(has_init))
    if dtype == torch.bfloat16:
        assert_bf16_elementwise(v.cpu(), vr, "conv out")
    else:
        assert_close(v, vr, F32_BAR, "conv out")
    assert np.array_equal(f64(pool), pr), "conv-state pool (copies of inputs) must be exact"


def test_conv_varlen_strided_rows_and_no_pool(orc):
    d = LayerDims(1, 1, 4, 16, 1, 16)
    lens = [5, 37, 1]
    T, CD = sum(lens), d.conv_dim
    base = torch.randn(T, CD + 32, device=DEV).to(torch.bfloat16)
    xbc = base[:, :CD]                                   # row stride CD + 32
    w = (torch.rand(CD, 4, device=DEV) - 0.5).to(torch.bfloat16)
    cu, _, _ = tables(lens, None, None)
    v = ssd.ssd_conv1d_fwd_varlen(xbc, w, None, cu)
    torch.cuda.synchronize()
    vr, _ = orc.conv1d_fwd_varlen(f64(xbc), f64(w), None, cu.cpu().numpy())
    assert_bf16_elementwise(v.cpu(), vr, "conv out")


# --------------------------------------------------------------------------- decode on pools
def test_conv_update_slots(orc):
    d = LayerDims(5, 1, 4, 16, 1, 16)
    CD = d.conv_dim
    g = torch.Generator(device="cpu").manual_seed(250)
    xbc = torch.randn(5, CD, generator=g).to(torch.bfloat16).to(DEV)
    w = (torch.rand(CD, 4, generator=g) - 0.5).to(torch.bfloat16).to(DEV)
    bias = (torch.rand(CD, generator=g) - 0.5).to(torch.bfloat16).to(DEV)
    pool0 = torch.randn(7, CD, 4, generator=g).to(torch.bfloat16).to(DEV)
    pool = pool0.clone()
    slots = [6, -1, 2, 0, 7]                              # -1 and 7 (>= nslots) are padding
    slot = torch.tensor(slots, dtype=torch.int32, device=DEV)
    v = ssd.ssd_conv1d_update_slots(xbc, w, bias, pool, slot)
    torch.cuda.synchronize()
    vr, pr = orc.conv1d_update_slots(f64(xbc), f64(w), f64(bias), f64(pool0), np.array(slots))
    assert_bf16_elementwise(v.cpu(), vr, "conv update out")
    assert np.array_equal(f64(pool), pr)


@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16])
def test_state_update_slots(orc, ydt):
    d = LayerDims(6, 1, 8, 64, 2, 128)
    s = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in scan_inputs(d, 260, seqlen=1).items()}
    pool0 = torch.randn(9, 8, 64, 128, device=DEV) * 0.1
    pool = pool0.clone()
    slots = [8, 0, -1, 4, 9, 2]
    slot = torch.tensor(slots, dtype=torch.int32, device=DEV)
    y = ssd.ssd_state_update_slots(pool, slot, s["x"][:, 0], s["Bm"][:, 0], s["Cm"][:, 0], s["dt"][:, 0],
                                   s["A"], s["D"], y_dtype=ydt)
    torch.cuda.synchronize()
    yr, pr = orc.state_update_slots(f64(pool0), np.array(slots), f64(s["x"][:, 0]), f64(s["Bm"][:, 0]),
                                    f64(s["Cm"][:, 0]), f64(s["dt"][:, 0]), f64(s["A"]), f64(s["D"]))
    assert_close(pool, pr, F32_BAR, "pool")
    if ydt == torch.float32:
        assert_close(y, yr, F32_BAR, "y")
    else:
        assert_bf16_elementwise(y, yr, "y bf16")


def test_state_update_slots_identity_is_the_plain_update():
    d = WORKLOADS["decode_ultra_b64"].with_(batch=8)
    s = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in scan_inputs(d, 270, seqlen=1).items()}
    st1 = s["init_state"].clone()
    st2 = s["init_state"].clone()
    args = (s["x"][:, 0], s["Bm"][:, 0], s["Cm"][:, 0], s["dt"][:, 0], s["A"], s["D"])
    y1 = ssd.ssd_state_update(st1, *args, y_dtype=torch.float32)
    y2 = ssd.ssd_state_update_slots(st2, torch.arange(8, dtype=torch.int32, device=DEV), *args,
                                    y_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(st1, st2)


# --------------------------------------------------------------------------- full size
def test_varlen_ultra_serving_mix(orc):
    """8192 packed tokens in 24 requests at the Ultra layer: varlen conv -> split -> varlen scan,
    in the launch configuration bench.py times; the oracle checks one sampled head per group."""
    d = WORKLOADS["varlen_ultra_8k"]
    lens = varlen_lengths(d.seqlen, d.batch, 1006)
    nslots = 32
    inp = {k: v.to(DEV) for k, v in varlen_inputs(d, lens, nslots, 1006, device=DEV).items()}
    cpool0, spool0 = inp["conv_pool"].clone(), inp["state_pool"].clone()
    cpool, spool = inp["conv_pool"], inp["state_pool"]
    tab = (inp["cu_seqlens"], cpool, inp["slot_idx"], inp["has_initial_state"])
    v = ssd.ssd_conv1d_fwd_varlen(inp["xbc"], inp["w"], inp["bias"], inp["cu_seqlens"], cpool,
                                  inp["slot_idx"], inp["has_initial_state"])
    x, Bm, Cm = ssd.split_xbc(v, d.nheads, d.head_dim, d.ngroups, d.d_state)
    y = ssd.ssd_chunk_scan_varlen(x, Bm, Cm, inp["dt"], inp["A"], inp["D"], inp["cu_seqlens"], spool,
                                  inp["slot_idx"], inp["has_initial_state"], y_dtype=torch.float32)
    torch.cuda.synchronize()
    del tab
    cu = inp["cu_seqlens"].cpu().numpy()
    slots = inp["slot_idx"].cpu().numpy()
    hinit = inp["has_initial_state"].cpu().numpy()
    hpg = d.nheads // d.ngroups
    I, GN, N, P = d.d_inner, d.ngroups * d.d_state, d.d_state, d.head_dim
    for g in range(d.ngroups):
        h = g * hpg + g % hpg
        ch = list(range(h * P, (h + 1) * P)) + list(range(I + g * N, I + (g + 1) * N)) + \
            list(range(I + GN + g * N, I + GN + (g + 1) * N))
        cht = torch.tensor(ch, device=DEV)
        vr, cpr = orc.conv1d_fwd_varlen(f64(inp["xbc"].index_select(1, cht)), f64(inp["w"].index_select(0, cht)),
                                        f64(inp["bias"].index_select(0, cht)), cu,
                                        f64(cpool0.index_select(1, cht)), slots, hinit)
        assert_bf16_elementwise(v.index_select(1, cht).cpu(), vr, f"conv head {h}")
        assert np.array_equal(f64(cpool.index_select(1, cht)), cpr), f"conv pool head {h}"
        va = to_act(vr, d.dtype)
        T = va.shape[0]
        yr, spr = orc.scan_varlen(va[:, :P].reshape(T, 1, P), va[:, P:P + N].reshape(T, 1, N),
                                  va[:, P + N:].reshape(T, 1, N), f64(inp["dt"][:, h:h + 1]),
                                  f64(inp["A"][h:h + 1]), f64(inp["D"][h:h + 1]), cu,
                                  f64(spool0[:, h:h + 1]), slots, hinit)
        assert_close(y[:, h], yr[:, 0], BF16_BAR, f"y head {h}")
        assert_close(spool[:, h], spr[:, 0], BF16_BAR, f"state pool head {h}")


# --------------------------------------------------------------------------- dt prologue
DT_OPTS = [dict(dt_bias=True, dt_softplus=True, dt_limit=(0.0, 0.5)), dict(dt_bias=True, dt_softplus=True),
           dict(dt_bias=False, dt_softplus=False, dt_limit=(0.05, 0.2))]


def dt_args(H, opts, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    bias = (torch.randn(H, generator=g) - 1.0).to(DEV) if opts.get("dt_bias") else None
    kw = dict(dt_bias=bias, dt_softplus=opts.get("dt_softplus", False), dt_limit=opts.get("dt_limit"))
    okw = dict(bias=None if bias is None else f64(bias), softplus=kw["dt_softplus"], limit=kw["dt_limit"])
    return kw, okw


@pytest.mark.parametrize("opts", DT_OPTS)
@pytest.mark.parametrize("P,N,dtype,chunk", [(64, 128, torch.bfloat16, 128), (16, 32, torch.float32, 64)])
def test_scan_dt_prologue(orc, opts, P, N, dtype, chunk):
    d = LayerDims(2, 300, 4, P, 2, N, dtype=dtype)
    s = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in scan_inputs(d, 280).items()}
    raw = (torch.randn(2, 300, 4, device=DEV) * 2.0 - 1.0).to(dtype)   # pre-softplus values
    kw, okw = dt_args(4, opts, 281)
    fin = torch.empty_like(s["init_state"])
    y = ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], raw, s["A"], s["D"], s["init_state"], fin, chunk=chunk,
                           y_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    dt_eff = orc.dt_prologue(f64(raw), **okw)
    yr, fr = orc.scan(f64(s["x"]), f64(s["Bm"]), f64(s["Cm"]), dt_eff, f64(s["A"]), f64(s["D"]), f64(s["init_state"]))
    bar = BF16_BAR if dtype == torch.bfloat16 else F32_BAR
    assert_close(y, yr, bar, "y")
    assert_close(fin, fr, bar, "final state")


@pytest.mark.parametrize("opts", DT_OPTS)
def test_state_update_and_slots_dt_prologue(orc, opts):
    d = LayerDims(5, 1, 8, 64, 2, 128)
    s = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in scan_inputs(d, 290, seqlen=1).items()}
    raw = (torch.randn(5, 8, device=DEV) * 2.0 - 1.0).to(torch.bfloat16)
    kw, okw = dt_args(8, opts, 291)
    dt_eff = orc.dt_prologue(f64(raw), **okw)
    args = (s["x"][:, 0], s["Bm"][:, 0], s["Cm"][:, 0], raw, s["A"], s["D"])
    st = s["init_state"].clone()
    y = ssd.ssd_state_update(st, *args, y_dtype=torch.float32, **kw)
    pool = s["init_state"][[4, 2, 0, 3, 1]].clone()
    slot = torch.tensor([2, 4, 1, 3, 0], dtype=torch.int32, device=DEV)
    y2 = ssd.ssd_state_update_slots(pool, slot, *args, y_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    yr, sr = orc.state_update(f64(s["init_state"]), f64(s["x"][:, 0]), f64(s["Bm"][:, 0]), f64(s["Cm"][:, 0]),
                              dt_eff, f64(s["A"]), f64(s["D"]))
    assert_close(y, yr, F32_BAR, "y")
    assert_close(st, sr, F32_BAR, "state")
    assert torch.equal(y2, y) and torch.equal(pool[slot.long()], st)


@pytest.mark.parametrize("ws", WS)
def test_scan_varlen_dt_prologue_matches_batched(ws):
    d = LayerDims(2, 200, 4, 64, 2, 128)
    s = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in scan_inputs(d, 300).items()}
    raw = (torch.randn(2, 200, 4, device=DEV) - 1.0).to(torch.bfloat16)
    bias = torch.randn(4, device=DEV)
    kw = dict(dt_bias=bias, dt_softplus=True, dt_limit=(0.0, 1.0))
    fin = torch.empty_like(s["init_state"])
    yb = ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], raw, s["A"], s["D"], s["init_state"], fin,
                            y_dtype=torch.float32, workspace=ws, **kw)
    pool = s["init_state"].clone()
    flat = lambda t: t.reshape((t.shape[0] * t.shape[1],) + tuple(t.shape[2:]))
    cu = torch.tensor([0, 200, 400], dtype=torch.int32, device=DEV)
    y = ssd.ssd_chunk_scan_varlen(flat(s["x"]), flat(s["Bm"]), flat(s["Cm"]), flat(raw), s["A"], s["D"], cu, pool,
                                  None, torch.ones(2, dtype=torch.int32, device=DEV), y_dtype=torch.float32,
                                  workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y.reshape(2, 200, 4, 64), yb) and torch.equal(pool, fin)
