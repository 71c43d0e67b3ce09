"""The oracle's packed-batch (varlen) and state-pool forms against independent references (CPU).

Per sequence, the scan is compared with the brute-force semiseparable form and the conv with
torch.nn.functional.conv1d (the pins of oracle_pins.py).  The table semantics are checked
directly: slots, padding, has_initial_state, and independence of the sequences.
Sources: modeling_nemotron_h.py walk-through, "Mamba SSM 缓存详解" / "Prefill 阶段" (per-request
cache slots written in place); "MAX 平台 Nemotron-H 混合架构解析", 5.4 (slots read and written
by the kernels).
"""
import numpy as np
import torch

from oracle_pins import rel_err, semiseparable_scan, softplus, torch_conv

LENS = [5, 0, 1, 9, 3, 12]   # includes an empty and a one-token sequence


def packed_scan_inputs(seed, lens=LENS, H=4, P=3, G=2, N=5, nslots=9):
    r = np.random.default_rng(seed)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    x = r.standard_normal((T, H, P))
    Bm = r.standard_normal((T, G, N))
    Cm = r.standard_normal((T, G, N))
    dt = softplus(r.normal(-2.0, 1.0, (T, H)))
    A = -np.exp(r.uniform(0, 1, H))
    D = r.standard_normal(H)
    pool = r.standard_normal((nslots, H, P, N))
    return cu, x, Bm, Cm, dt, A, D, pool


def test_scan_varlen_matches_bruteforce_per_sequence(orc):
    cu, x, Bm, Cm, dt, A, D, pool = packed_scan_inputs(1)
    S = len(cu) - 1
    slot = np.array([7, 2, -1, 0, 11, 4])      # -1 and 11 (>= nslots) are padding
    has_init = np.array([1, 1, 1, 0, 1, 1])
    y, new = orc.scan_varlen(x, Bm, Cm, dt, A, D, cu, pool, slot, has_init)
    touched = set()
    for s in range(S):
        a, b = cu[s], cu[s + 1]
        k = slot[s] if 0 <= slot[s] < pool.shape[0] else -1
        S0 = pool[k][None] if (k >= 0 and has_init[s]) else np.zeros((1,) + pool.shape[1:])
        if b > a:
            yr, fr = semiseparable_scan(x[None, a:b], Bm[None, a:b], Cm[None, a:b], dt[None, a:b], A, D, S0)
            assert rel_err(y[a:b], yr[0]) < 1e-12, s
        else:                            # an empty sequence carries its starting state through
            fr = S0
        if k >= 0:
            touched.add(k)
            assert rel_err(new[k], fr[0]) < 1e-12, s
    for k in range(pool.shape[0]):       # slots no sequence names keep their contents
        if k not in touched:
            assert np.array_equal(new[k], pool[k]), k


def test_scan_varlen_equal_lengths_is_the_batched_scan(orc):
    r = np.random.default_rng(2)
    Bt, L, H, P, G, N = 3, 11, 4, 3, 2, 5
    x = r.standard_normal((Bt, L, H, P))
    Bm = r.standard_normal((Bt, L, G, N))
    Cm = r.standard_normal((Bt, L, G, N))
    dt = softplus(r.normal(-2.0, 1.0, (Bt, L, H)))
    A = -np.exp(r.uniform(0, 1, H))
    D = r.standard_normal(H)
    S0 = r.standard_normal((Bt, H, P, N))
    yb, fb = orc.scan(x, Bm, Cm, dt, A, D, S0)
    cu = np.arange(Bt + 1) * L
    perm = np.array([2, 0, 1])
    pool = np.zeros((Bt, H, P, N))
    pool[perm] = S0
    y, new = orc.scan_varlen(x.reshape(Bt * L, H, P), Bm.reshape(Bt * L, G, N), Cm.reshape(Bt * L, G, N),
                             dt.reshape(Bt * L, H), A, D, cu, pool, perm, np.ones(Bt))
    assert np.array_equal(y.reshape(Bt, L, H, P), yb)
    assert np.array_equal(new[perm], fb)


def test_scan_varlen_sequences_are_independent(orc):
    cu, x, Bm, Cm, dt, A, D, pool = packed_scan_inputs(3)
    y1, p1 = orc.scan_varlen(x, Bm, Cm, dt, A, D, cu, pool, None, np.ones(len(cu) - 1))
    x2, B2 = x.copy(), Bm.copy()
    x2[cu[3]:cu[4]] += 1.0        # change sequence 3 only
    B2[cu[3]:cu[4]] *= -2.0
    y2, p2 = orc.scan_varlen(x2, B2, Cm, dt, A, D, cu, pool, None, np.ones(len(cu) - 1))
    for s in range(len(cu) - 1):
        same = np.array_equal(y1[cu[s]:cu[s + 1]], y2[cu[s]:cu[s + 1]]) and np.array_equal(p1[s], p2[s])
        assert same == (s != 3 or cu[s] == cu[s + 1]), s


def test_scan_varlen_without_initial_state_ignores_the_pool(orc):
    cu, x, Bm, Cm, dt, A, D, pool = packed_scan_inputs(4)
    y1, p1 = orc.scan_varlen(x, Bm, Cm, dt, A, D, cu, pool, None, None)
    y2, p2 = orc.scan_varlen(x, Bm, Cm, dt, A, D, cu, pool * 0 + 123.0, None, np.zeros(len(cu) - 1))
    assert np.array_equal(y1, y2)
    assert np.array_equal(p1[:len(cu) - 1], p2[:len(cu) - 1])


def test_conv_varlen_matches_torch_conv_per_sequence(orc):
    r = np.random.default_rng(5)
    lens, CD, K, nslots = [6, 2, 0, 9, 1], 12, 4, 7
    cu = np.concatenate([[0], np.cumsum(lens)])
    u = r.standard_normal((cu[-1], CD))
    w = r.uniform(-0.5, 0.5, (CD, K))
    bias = r.uniform(-0.5, 0.5, CD)
    pool = r.standard_normal((nslots, CD, K))
    slot = np.array([3, 6, 0, -1, 5])
    has_init = np.array([1, 1, 0, 1, 0])
    v, new = orc.conv1d_fwd_varlen(u, w, bias, cu, pool, slot, has_init)
    for s in range(len(lens)):
        a, b = cu[s], cu[s + 1]
        k = slot[s] if 0 <= slot[s] < nslots else -1
        s_in = pool[k][None] if (k >= 0 and has_init[s]) else None
        if b > a:
            vr, sr = torch_conv(u[None, a:b], w, bias, s_in)
            assert rel_err(v[a:b], vr[0]) < 1e-12, s
        else:                            # an empty sequence keeps its window (zeros without one)
            sr = s_in if s_in is not None else np.zeros((1, CD, K))
        if k >= 0:
            assert np.array_equal(new[k], sr[0]), s
    for k in (1, 2, 4):                 # slots no sequence names keep their contents
        assert np.array_equal(new[k], pool[k])


def test_conv_update_slots_matches_torch_conv(orc):
    r = np.random.default_rng(6)
    Bt, CD, K, nslots = 4, 12, 4, 6
    u = r.standard_normal((Bt, CD))
    w = r.uniform(-0.5, 0.5, (CD, K))
    bias = r.uniform(-0.5, 0.5, CD)
    pool = r.standard_normal((nslots, CD, K))
    slot = np.array([5, -1, 1, 2])
    v, new = orc.conv1d_update_slots(u, w, bias, pool, slot)
    for b in range(Bt):
        k = slot[b]
        s_in = pool[k][None] if k >= 0 else np.zeros((1, CD, K))
        vr, sr = torch_conv(u[None, b:b + 1], w, bias, s_in)
        assert rel_err(v[b], vr[0, 0]) < 1e-12, b
        if k >= 0:
            assert np.array_equal(new[k], sr[0]), b
    for k in (0, 3, 4):
        assert np.array_equal(new[k], pool[k])


def test_state_update_slots_matches_bruteforce(orc):
    r = np.random.default_rng(7)
    Bt, H, P, G, N, nslots = 5, 4, 3, 2, 5, 8
    x = r.standard_normal((Bt, H, P))
    Bm = r.standard_normal((Bt, G, N))
    Cm = r.standard_normal((Bt, G, N))
    dt = softplus(r.normal(-2.0, 1.0, (Bt, H)))
    A = -np.exp(r.uniform(0, 1, H))
    D = r.standard_normal(H)
    pool = r.standard_normal((nslots, H, P, N))
    slot = np.array([6, 0, -1, 3, 9])   # -1 and 9 (>= nslots) are padding
    y, new = orc.state_update_slots(pool, slot, x, Bm, Cm, dt, A, D)
    for b in range(Bt):
        k = slot[b] if 0 <= slot[b] < nslots else -1
        S0 = pool[k][None] if k >= 0 else np.zeros((1, H, P, N))
        yr, fr = semiseparable_scan(x[None, None, b], Bm[None, None, b], Cm[None, None, b], dt[None, None, b],
                                    A, D, S0)
        assert rel_err(y[b], yr[0, 0]) < 1e-12, b
        if k >= 0:
            assert rel_err(new[k], fr[0]) < 1e-12, b
    for k in (1, 2, 4, 5, 7):
        assert np.array_equal(new[k], pool[k])


def test_dt_prologue_matches_torch_softplus(orc):
    """The dt prologue against torch's softplus and clamp in fp64 (the page's plugin takes dt_bias
    with softplus)."""
    r = np.random.default_rng(8)
    dt = r.normal(-1.0, 6.0, (3, 50, 4))                 # spans both tails of the softplus
    bias = r.normal(0.0, 2.0, 4)
    v = orc.dt_prologue(dt, bias, True, (0.001, 3.0))
    t = torch.nn.functional.softplus(torch.from_numpy(dt + bias), beta=1.0, threshold=1e9)
    ref = torch.clamp(t, 0.001, 3.0).numpy()
    assert rel_err(v, ref) < 1e-14
    assert np.array_equal(orc.dt_prologue(dt), dt)
    assert np.array_equal(orc.dt_prologue(dt, bias), dt + bias)
    assert np.array_equal(orc.dt_prologue(dt, None, False, (1.0, 1.0)), dt)   # lo >= hi: no clamp


def test_torch_is_cpu_only_here():
    assert torch.tensor([1.0]).device.type == "cpu"
