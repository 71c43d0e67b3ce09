"""Parity of the chunked scans on 16-bit state arrays (ssd_chunk_scan_lp, ssd_chunk_scan_varlen_lp)
with the oracle, on the GPU, for the fp16 scan (bf16 inputs with a workspace), the bf16
split-operand scan (no workspace) and the generic scan (fp32 inputs).

* A = 0 with inputs on a coarse dyadic grid: the scan's fp32 final state is exact, so the stored
  codes -- random numbers and rounding decisions included -- must equal the oracle's bit for bit
  (oracle.scan_lp / scan_varlen_lp, pinned in tests/test_oracle_lowprec.py).
* General inputs: y is the fp32-state scan's y from the decoded codes, bit for bit; rounded to
  nearest, the final codes are torch's conversion of that scan's fp32 final state; rounded
  stochastically, each is one of the two codes around it, and within one spacing (plus the scan's
  error bar) of the oracle's fp64 final state.
Sources: the modeling_nemotron_h.py walk-through page, 部署时如何调这些缓存 (fp16 state cache with
Philox stochastic rounding); "MAX 平台 Nemotron-H 混合架构解析" 5.4 (narrow stored state, fp32
accumulation).
"""
import numpy as np
import pytest
import torch

from gpu_util import BF16_BAR, F32_BAR, assert_close, f64
from selective_state_space_conv1d_amd import ssd
from selective_state_space_conv1d_amd.synth import LayerDims, scan_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"
FMT = {torch.float16: "f16", torch.bfloat16: "bf16"}
# kernel -> (activation dtype, head_dim, d_state, workspace argument)
KERNELS = {"f16": (torch.bfloat16, 64, 128, None), "mfma": (torch.bfloat16, 64, 128, False),
           "fma": (torch.float32, 32, 64, None)}


def codes_of(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def spacing_of(v, fmt):
    av = np.abs(v)
    if fmt == "f16":
        return 2.0 ** (np.floor(np.log2(np.maximum(av, 2.0 ** -14))) - 10)
    return 2.0 ** (np.floor(np.log2(np.maximum(av, 2.0 ** -126))) - 7)


def dyadic(lead, H, P, G, N, act, sdt, seed, nstate):
    """A = 0 inputs on the grid of tests/test_oracle_lowprec.py (every partial sum exact in fp32);
    lead is (B, L) or (T,).  The initial codes are torch's conversion of multiples of 2^-10."""
    r = np.random.default_rng(seed)
    mk = lambda a: torch.from_numpy(a).to(act).to(DEV)
    x = mk(r.integers(-16, 17, lead + (H, P)) / 64.0)
    Bm = mk(r.integers(-16, 17, lead + (G, N)) / 64.0)
    Cm = mk(r.integers(-16, 17, lead + (G, N)) / 64.0)
    dt = mk(2.0 ** -r.integers(3, 6, lead + (H,)).astype(np.float64))
    A = torch.zeros(H, device=DEV)
    D = torch.from_numpy(r.standard_normal(H)).float().to(DEV)
    init = torch.from_numpy(r.integers(-1024, 1025, (nstate, H, P, N)) / 1024.0).float().to(sdt).to(DEV)
    return x, Bm, Cm, dt, A, D, init


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("sdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("sr", [None, (0x5EED, 41, 5), (2 ** 40 + 3, 7, 9)])
def test_scan_lp_codes_bitwise_dyadic(orc, kernel, sdt, sr):
    act, P, N, ws = KERNELS[kernel]
    Bt, L, H, G = 2, 300, 4, 2                   # three chunks of 128, the last one ragged
    x, Bm, Cm, dt, A, D, init = dyadic((Bt, L), H, P, G, N, act, sdt, 600, Bt)
    fin = torch.empty_like(init)
    y = ssd.ssd_chunk_scan_lp(x, Bm, Cm, dt, A, D, init, fin, sr=sr, y_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    fmt = FMT[sdt]
    yr, fr, want = orc.scan_lp(f64(x), f64(Bm), f64(Cm), f64(dt), f64(A), f64(D), codes_of(init), fmt, sr)
    got = codes_of(fin)
    assert np.array_equal(got, want), f"{(got != want).sum()} codes differ"
    assert_close(y, yr, BF16_BAR if act == torch.bfloat16 else F32_BAR, "y")
    # in place (final aliasing init): the same codes
    st = init.clone()
    ssd.ssd_chunk_scan_lp(x, Bm, Cm, dt, A, D, st, st, sr=sr, y_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(st, fin)


@pytest.mark.parametrize("kernel", list(KERNELS))
@pytest.mark.parametrize("sdt", [torch.float16, torch.bfloat16])
def test_scan_lp_is_the_fp32_scan_rounded(orc, kernel, sdt):
    act, P, N, ws = KERNELS[kernel]
    d = LayerDims(2, 257, 4, P, 2, N, dtype=act)
    s = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in scan_inputs(d, 610).items()}
    init = (s["init_state"] * 4.0).to(sdt)
    args = (s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"])
    fin32 = torch.empty(init.shape, device=DEV)
    y32 = ssd.ssd_chunk_scan(*args, init_state=init.float(), final_state=fin32, y_dtype=torch.float32, workspace=ws)
    rne = torch.empty_like(init)
    y16 = ssd.ssd_chunk_scan_lp(*args, init, rne, y_dtype=torch.float32, workspace=ws)
    srf = torch.empty_like(init)
    ssd.ssd_chunk_scan_lp(*args, init, srf, sr=(77, 5, 5), y_dtype=torch.float32, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(y16, y32), "the scan must not depend on how its states are stored"
    assert torch.equal(rne, fin32.to(sdt)), "nearest-even codes of the fp32 final state"
    fmt = FMT[sdt]
    v = f64(fin32)
    gap = np.abs(f64(srf) - v)
    assert (gap < spacing_of(v, fmt)).all(), "stochastic rounding gives one of the two neighbouring codes"
    assert (f64(srf) != f64(rne)).any() and (f64(srf) == f64(rne)).any()
    # and against the oracle's fp64 final state: one spacing plus the scan's error bar
    _, fr = orc.scan(*(f64(t) for t in args), f64(init))
    bar = BF16_BAR if act == torch.bfloat16 else F32_BAR
    bound = spacing_of(fr, fmt) + bar * np.abs(fr).max()
    assert (np.abs(f64(srf) - fr) <= bound).all()


@pytest.mark.parametrize("kernel", ["mfma", "fma"])
@pytest.mark.parametrize("sdt", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("sr", [None, (0xFACE, 3, 5)])
def test_scan_varlen_lp_codes_bitwise_dyadic(orc, kernel, sdt, sr):
    act, P, N, _ = KERNELS[kernel]
    lens = [1, 0, 127, 129, 300, 5, 33]
    slots = [7, 3, -1, 0, 9, 5, 1]                  # -1 and 9 (>= nslots) are padding
    has_init = [1, 0, 1, 1, 1, 0, 1]
    nslots, H, G = 9, 4, 2
    T = sum(lens)
    x, Bm, Cm, dt, A, D, pool0 = dyadic((T,), H, P, G, N, act, sdt, 620, nslots)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    slot = torch.tensor(slots, dtype=torch.int32, device=DEV)
    hi = torch.tensor(has_init, dtype=torch.int32, device=DEV)
    pool = pool0.clone()
    y = ssd.ssd_chunk_scan_varlen_lp(x, Bm, Cm, dt, A, D, cu, pool, slot, hi, sr=sr, y_dtype=torch.float32)
    torch.cuda.synchronize()
    yr, want = orc.scan_varlen_lp(f64(x), f64(Bm), f64(Cm), f64(dt), f64(A), f64(D), cu.cpu().numpy(),
                                  codes_of(pool0), FMT[sdt], np.array(slots), np.array(has_init), sr)
    got = codes_of(pool)
    assert np.array_equal(got, want), f"{(got != want).sum()} codes differ"
    assert_close(y, yr, BF16_BAR if act == torch.bfloat16 else F32_BAR, "y")


def test_scan_lp_rejects_mixed_or_wide_states():
    act, P, N, _ = KERNELS["fma"]
    x, Bm, Cm, dt, A, D, init = dyadic((1, 4), 2, P, 1, N, act, torch.float16, 630, 1)
    with pytest.raises(ValueError):
        ssd.ssd_chunk_scan_lp(x, Bm, Cm, dt, A, D, init, init.to(torch.bfloat16))
    with pytest.raises(ValueError):
        ssd.ssd_chunk_scan_lp(x, Bm, Cm, dt, A, D, init.float(), None)
