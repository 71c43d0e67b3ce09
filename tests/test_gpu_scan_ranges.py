"""The MFMA scan when one workgroup walks a range of sequences (more sequences x heads than the
chip holds workgroups), on the GPU.

Each sequence's arithmetic is the same whichever workgroup runs it, so a call over many
sequences must reproduce, bit for bit, the same sequences scanned one call each (one sequence
per workgroup); the oracle checks sampled heads.  Cases: packed batches whose ranges start and
end on empty, one-token and padding sequences, a range that is one long sequence, a batch of
equal sequences split into ranges, and state snapshots taken inside ranges.
"""
import numpy as np
import pytest
import torch

from gpu_util import BF16_BAR, assert_close, f64
from selective_state_space_conv1d_amd import ssd
from selective_state_space_conv1d_amd.synth import LayerDims, scan_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def mixed_lengths(S, seed):
    """S lengths: zeros, ones, chunk multiples, ragged and a few long ones."""
    r = np.random.default_rng(seed)
    pick = r.integers(0, 6, S)
    lens = np.where(pick == 0, 0, np.where(pick == 1, 1, np.where(pick == 2, 128 * r.integers(1, 3, S),
                    np.where(pick == 3, r.integers(2, 400, S), r.integers(2, 60, S)))))
    lens[r.integers(0, S)] = 700                       # one long sequence
    return [int(v) for v in lens]


def packed(H, lens, seed):
    d = LayerDims(1, int(sum(lens)), H, 64, 8 if H >= 8 else 1, 128)
    s = scan_inputs(d, seed, init_state=False)
    return d, {k: v[0].to(DEV) if k in ("x", "Bm", "Cm", "dt") else v.to(DEV) for k, v in s.items() if v is not None}


def i32(a):
    return torch.tensor(np.asarray(a), dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("H,S", [(256, 40), (64, 37)])     # one range per head; about 4 ranges per head
def test_varlen_ranges_match_one_call_per_sequence(orc, H, S):
    lens = mixed_lengths(S, 700 + H)
    lens[0], lens[-1] = 0, 1                           # ranges begin and end on degenerate sequences
    d, s = packed(H, lens, 701)
    r = np.random.default_rng(702)
    nslots = S + 4
    slots = r.permutation(nslots)[:S].astype(np.int32)
    slots[r.integers(0, S, 3)] = -1                    # padding: nothing read or stored
    has_init = (r.random(S) < 0.6).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pool0 = torch.randn(nslots, H, 64, 128, device=DEV) * 0.1
    pool = pool0.clone()
    y = ssd.ssd_chunk_scan_varlen(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], i32(cu), pool, i32(slots),
                                  i32(has_init), y_dtype=torch.float32, workspace=False)
    # the same sequences, one call each
    pool1 = pool0.clone()
    y1 = torch.empty_like(y)
    for q in range(S):
        a, b = int(cu[q]), int(cu[q + 1])
        y1[a:b] = ssd.ssd_chunk_scan_varlen(s["x"][a:b], s["Bm"][a:b], s["Cm"][a:b], s["dt"][a:b], s["A"], s["D"],
                                            i32([0, b - a]), pool1, i32(slots[q:q + 1]), i32(has_init[q:q + 1]),
                                            y_dtype=torch.float32, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(y, y1), "y differs from the per-sequence calls"
    assert torch.equal(pool, pool1), "state pool differs from the per-sequence calls"
    named = set(int(v) for v in slots if v >= 0)
    others = [k for k in range(nslots) if k not in named]
    assert torch.equal(pool[others], pool0[others]), "slots no sequence names must be untouched"
    # the oracle on one head per group
    hpg = H // d.ngroups
    for h in [g * hpg + (g * 5) % hpg for g in range(0, d.ngroups, 3)]:
        yr, pr = orc.scan_varlen(f64(s["x"][:, h:h + 1]), f64(s["Bm"][:, h // hpg:h // hpg + 1]),
                                 f64(s["Cm"][:, h // hpg:h // hpg + 1]), f64(s["dt"][:, h:h + 1]),
                                 f64(s["A"][h:h + 1]), f64(s["D"][h:h + 1]), cu, f64(pool0[:, h:h + 1]), slots,
                                 has_init)
        assert_close(y[:, h], yr[:, 0], BF16_BAR, f"y head {h}")
        assert_close(pool[:, h], pr[:, 0], BF16_BAR, f"state pool head {h}")


def test_varlen_range_of_empty_sequences_only():
    """Ranges made only of empty sequences still store each named slot's final state."""
    H, S = 128, 12
    lens = [0] * 10 + [300, 0]
    d, s = packed(H, lens, 710)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    slots = np.arange(S, dtype=np.int32)[::-1].copy()
    has_init = np.array([1, 0] * 6, dtype=np.int32)
    pool0 = torch.randn(S, H, 64, 128, device=DEV)
    pool = pool0.clone()
    ssd.ssd_chunk_scan_varlen(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], i32(cu), pool, i32(slots),
                              i32(has_init), workspace=False)
    torch.cuda.synchronize()
    for q in range(S):
        if lens[q] == 0:
            want = pool0[slots[q]] if has_init[q] else torch.zeros_like(pool0[0])
            assert torch.equal(pool[slots[q]], want), q


@pytest.mark.parametrize("snap", [False, True])
@pytest.mark.parametrize("L", [256, 300])     # exact chunks; a ragged last chunk in every entry
def test_batched_ranges_match_one_call_per_entry(orc, snap, L):
    H, B = 16, 40
    d = LayerDims(B, L, H, 64, 2, 128)
    s = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in scan_inputs(d, 720).items()}
    kw = dict(y_dtype=torch.float32)
    fin = torch.empty_like(s["init_state"])
    snaps = torch.empty(B, L // 128, H, 64, 128, device=DEV) if snap else None
    if snap:
        kw.update(snapshots=snaps, snapshot_interval=128)
    y = ssd.ssd_chunk_scan(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], s["init_state"], fin, **kw)
    for b in range(B):
        f1 = torch.empty_like(fin[b:b + 1])
        kw1 = dict(y_dtype=torch.float32)
        if snap:
            sn1 = torch.empty_like(snaps[b:b + 1])
            kw1.update(snapshots=sn1, snapshot_interval=128)
        y1 = ssd.ssd_chunk_scan(s["x"][b:b + 1], s["Bm"][b:b + 1], s["Cm"][b:b + 1], s["dt"][b:b + 1], s["A"],
                                s["D"], s["init_state"][b:b + 1], f1, **kw1)
        torch.cuda.synchronize()
        assert torch.equal(y[b:b + 1], y1) and torch.equal(fin[b:b + 1], f1), b
        if snap:
            assert torch.equal(snaps[b:b + 1], sn1), b
    b, h = 23, 9
    yr, fr = orc.scan(f64(s["x"][b:b + 1, :, h:h + 1]), f64(s["Bm"][b:b + 1, :, h // 8:h // 8 + 1]),
                            f64(s["Cm"][b:b + 1, :, h // 8:h // 8 + 1]), f64(s["dt"][b:b + 1, :, h:h + 1]),
                            f64(s["A"][h:h + 1]), f64(s["D"][h:h + 1]), f64(s["init_state"][b:b + 1, h:h + 1]))
    assert_close(y[b:b + 1, :, h:h + 1], yr, BF16_BAR, "y")
    assert_close(fin[b:b + 1, h:h + 1], fr, BF16_BAR, "final state")


def test_varlen_ranges_without_tables():
    """No slot table (sequence s uses slot s) and no initial-state flags (every sequence starts from
    zeros): the walk equals one call per sequence, and every slot receives its final state."""
    H, S = 256, 30
    lens = mixed_lengths(S, 730)
    d, s = packed(H, lens, 731)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    pool0 = torch.randn(S, H, 64, 128, device=DEV)
    pool = pool0.clone()
    y = ssd.ssd_chunk_scan_varlen(s["x"], s["Bm"], s["Cm"], s["dt"], s["A"], s["D"], i32(cu), pool,
                                  y_dtype=torch.float32, workspace=False)
    pool1 = pool0.clone()
    y1 = torch.empty_like(y)
    for q in range(S):
        a, b = int(cu[q]), int(cu[q + 1])
        y1[a:b] = ssd.ssd_chunk_scan_varlen(s["x"][a:b], s["Bm"][a:b], s["Cm"][a:b], s["dt"][a:b], s["A"], s["D"],
                                            i32([0, b - a]), pool1[q:q + 1], y_dtype=torch.float32, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(y, y1) and torch.equal(pool, pool1)
    empty = [q for q in range(S) if lens[q] == 0]
    assert all(not pool[q].any() for q in empty), "an empty sequence without an initial state ends at zero"
