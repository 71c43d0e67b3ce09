"""The binding checks every tensor argument before anything reaches the C ABI (CPU only).

The C entry points see only pointers, so a buffer of the wrong dtype, shape or device would be read or
written out of bounds on the GPU.  Here the binding's device check is widened to CPU tensors and the
library is replaced by a recorder: a well-formed call reaches the recorder once, and each malformed
variant raises ValueError with nothing recorded.
"""
import pytest
import torch

from selective_state_space_conv1d_amd import ssd

bf, f32 = torch.bfloat16, torch.float32


class Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def f(*args):
            if not name.endswith("_size"):       # size queries launch nothing
                self.calls.append(name)
            return 0
        return f


@pytest.fixture
def rec(monkeypatch):
    r = Recorder()
    monkeypatch.setattr(ssd, "_DEVICE_TYPES", ("cpu",))
    monkeypatch.setattr(ssd, "_lib", lambda: r)
    monkeypatch.setattr(ssd, "_stream", lambda s: None)
    return r


B_, L_, H_, P_, G_, N_ = 2, 8, 4, 16, 2, 32
CD = H_ * P_ + 2 * G_ * N_


def t(*shape, dtype=bf):
    return torch.zeros(*shape, dtype=dtype)


def scan_args():
    v = t(B_, L_, CD)
    x, Bm, Cm = ssd.split_xbc(v, H_, P_, G_, N_)
    return dict(x=x, B=Bm, C=Cm, dt=t(B_, L_, H_), A=t(H_, dtype=f32), D=t(H_, dtype=f32),
                init_state=t(B_, H_, P_, N_, dtype=f32), final_state=t(B_, H_, P_, N_, dtype=f32),
                y=t(B_, L_, H_, P_, dtype=f32))


def update_args():
    u = t(B_, CD)
    x, Bm, Cm = ssd.split_xbc(u, H_, P_, G_, N_)
    return dict(state=t(B_, H_, P_, N_, dtype=f32), x=x, B=Bm, C=Cm, dt=t(B_, H_), A=t(H_, dtype=f32),
                D=t(H_, dtype=f32), y=t(B_, H_, P_))


def conv_args():
    return dict(xbc=t(B_, L_, CD), w=t(CD, 4), bias=t(CD), conv_state_in=t(B_, CD, 4), conv_state_out=t(B_, CD, 4),
                out=t(B_, L_, CD))


def conv_update_args():
    return dict(xbc=t(B_, CD), w=t(CD, 4), bias=t(CD), conv_state=t(B_, CD, 4), out=t(B_, CD))


def meta(x):
    return torch.empty(x.shape, dtype=x.dtype, device="meta")


CASES = {
    "ssd_chunk_scan": (scan_args, [
        ("B", lambda a: a["B"].float()), ("dt", lambda a: a["dt"].float()), ("dt", lambda a: t(B_, L_, H_ + 1)),
        ("A", lambda a: a["A"].to(bf)), ("A", lambda a: t(H_ + 1, dtype=f32)), ("D", lambda a: t(H_, dtype=bf)),
        ("init_state", lambda a: a["init_state"].to(bf)), ("init_state", lambda a: t(B_, H_, N_, P_, dtype=f32)),
        ("final_state", lambda a: t(B_, H_, P_, N_, dtype=f32).transpose(2, 3)),
        ("final_state", lambda a: meta(a["final_state"])), ("y", lambda a: t(B_, L_, H_, P_ + 1, dtype=f32)),
        ("y", lambda a: t(B_, L_, H_, P_, dtype=torch.float16)), ("A", lambda a: meta(a["A"])),
    ]),
    "ssd_state_update": (update_args, [
        ("state", lambda a: a["state"].to(bf)), ("state", lambda a: t(B_, H_, P_, N_ + 8, dtype=f32)),
        ("B", lambda a: a["B"].float()), ("C", lambda a: meta(a["C"])), ("dt", lambda a: t(B_, H_, dtype=f32)),
        ("A", lambda a: t(H_, dtype=bf)), ("D", lambda a: t(H_ - 1, dtype=f32)), ("y", lambda a: t(B_, H_, P_ - 1)),
        ("state", lambda a: t(B_, H_, N_, P_, dtype=f32).transpose(2, 3)),
    ]),
    "ssd_conv1d_fwd": (conv_args, [
        ("w", lambda a: t(CD, 4, dtype=f32)), ("w", lambda a: t(CD, 3)), ("bias", lambda a: t(CD + 1)),
        ("conv_state_in", lambda a: t(B_, CD, 4, dtype=f32)), ("conv_state_out", lambda a: t(B_, CD, 3)),
        ("conv_state_in", lambda a: t(B_, 4, CD).transpose(1, 2)), ("out", lambda a: t(B_, L_ + 1, CD)),
        ("out", lambda a: meta(a["out"])),
    ]),
    "ssd_conv1d_update": (conv_update_args, [
        ("w", lambda a: t(CD, 4, dtype=f32)), ("conv_state", lambda a: t(B_, CD, 4, dtype=f32)),
        ("conv_state", lambda a: t(B_ + 1, CD, 4)), ("out", lambda a: t(B_, CD - 1)), ("bias", lambda a: meta(a["bias"])),
    ]),
}


@pytest.mark.parametrize("fn", sorted(CASES))
def test_well_formed_call_reaches_the_library(rec, fn):
    make, _ = CASES[fn]
    getattr(ssd, fn)(**make())
    assert rec.calls == [fn]


@pytest.mark.parametrize("fn,i", [(fn, i) for fn in sorted(CASES) for i in range(len(CASES[fn][1]))])
def test_malformed_argument_is_rejected_before_the_library(rec, fn, i):
    make, bad = CASES[fn]
    args = make()
    name, mutate = bad[i]
    args[name] = mutate(args)
    with pytest.raises(ValueError):
        getattr(ssd, fn)(**args)
    assert rec.calls == []


def test_serving_forms_reject_a_wrong_pool(rec):
    a = update_args()
    pool = t(5, H_, P_, N_, dtype=f32)
    slot = torch.zeros(B_, dtype=torch.int32)
    ssd.ssd_state_update_slots(pool, slot, a["x"], a["B"], a["C"], a["dt"], a["A"], a["D"], y=a["y"])
    assert rec.calls == ["ssd_state_update_slots"]
    for bad_pool, bad_slot in ((pool.to(bf), slot), (pool, slot.long()), (pool, meta(slot))):
        with pytest.raises(ValueError):
            ssd.ssd_state_update_slots(bad_pool, bad_slot, a["x"], a["B"], a["C"], a["dt"], a["A"], a["D"], y=a["y"])
    s = scan_args()
    T = L_
    flat = {k: s[k][0] for k in ("x", "B", "C", "dt")}
    cu = torch.tensor([0, 3, T], dtype=torch.int32)
    ssd.ssd_chunk_scan_varlen(flat["x"], flat["B"], flat["C"], flat["dt"], s["A"], s["D"], cu,
                              state_pool=pool, slot_idx=slot, y=t(T, H_, P_))
    assert rec.calls[-1] == "ssd_chunk_scan_varlen"
    n = len(rec.calls)
    for kw in (dict(state_pool=pool.to(bf)), dict(y=t(T, H_, P_ + 1)), dict(slot_idx=meta(slot))):
        args = dict(state_pool=pool, slot_idx=slot, y=t(T, H_, P_))
        args.update(kw)
        with pytest.raises(ValueError):
            ssd.ssd_chunk_scan_varlen(flat["x"], flat["B"], flat["C"], flat["dt"], s["A"], s["D"], cu, **args)
    assert len(rec.calls) == n
