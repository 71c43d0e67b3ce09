"""The oracle's multi-token (speculative) decode forms against independent references (CPU).

The intermediate state after token j must be the final state of the brute-force semiseparable
scan over the first j+1 tokens, and the intermediate conv state the final window of torch's
conv1d over those rows; accepting n tokens must leave the slot at the state after n tokens.
Source: "Mamba 与 Nemotron 系列模型深度调研", 状态契约 / "MTP / speculative decoding" (candidate tokens leave
intermediate recurrent and conv states; the accepted length picks the one scattered back).
"""
import numpy as np

from oracle_pins import rel_err, semiseparable_scan, softplus, torch_conv


def spec_inputs(seed, Bt=4, k=5, H=4, P=3, G=2, N=5, nslots=7):
    r = np.random.default_rng(seed)
    x = r.standard_normal((Bt, k, H, P))
    Bm = r.standard_normal((Bt, k, G, N))
    Cm = r.standard_normal((Bt, k, G, N))
    dt = softplus(r.normal(-2.0, 1.0, (Bt, k, H)))
    A = -np.exp(r.uniform(0, 1, H))
    D = r.standard_normal(H)
    pool = r.standard_normal((nslots, H, P, N))
    return x, Bm, Cm, dt, A, D, pool


def test_state_update_multi_matches_bruteforce_prefixes(orc):
    x, Bm, Cm, dt, A, D, pool = spec_inputs(11)
    slot = np.array([5, -1, 0, 3])                   # -1 is padding: starts from zeros
    y, inter = orc.state_update_multi(pool, slot, x, Bm, Cm, dt, A, D)
    Bt, k = x.shape[:2]
    for b in range(Bt):
        S0 = pool[slot[b]][None] if slot[b] >= 0 else np.zeros((1,) + pool.shape[1:])
        yr, _ = semiseparable_scan(x[b:b + 1], Bm[b:b + 1], Cm[b:b + 1], dt[b:b + 1], A, D, S0)
        assert rel_err(y[b], yr[0]) < 1e-12, b
        for j in range(k):
            _, fr = semiseparable_scan(x[b:b + 1, :j + 1], Bm[b:b + 1, :j + 1], Cm[b:b + 1, :j + 1],
                                       dt[b:b + 1, :j + 1], A, D, S0)
            assert rel_err(inter[b, j], fr[0]) < 1e-12, (b, j)


def test_conv_update_multi_matches_torch_conv_prefixes(orc):
    r = np.random.default_rng(12)
    Bt, k, CD, K, nslots = 3, 6, 10, 4, 5
    u = r.standard_normal((Bt, k, CD))
    w = r.uniform(-0.5, 0.5, (CD, K))
    bias = r.uniform(-0.5, 0.5, CD)
    pool = r.standard_normal((nslots, CD, K))
    slot = np.array([4, 1, -1])
    v, inter = orc.conv1d_update_multi(u, w, bias, pool, slot)
    for b in range(Bt):
        s_in = pool[slot[b]][None] if slot[b] >= 0 else np.zeros((1, CD, K))
        vr, _ = torch_conv(u[b:b + 1], w, bias, s_in)
        assert rel_err(v[b], vr[0]) < 1e-12, b
        for j in range(k):
            _, sr = torch_conv(u[b:b + 1, :j + 1], w, bias, s_in)
            assert np.array_equal(inter[b, j], sr[0]), (b, j)


def test_accept_is_the_state_after_n_tokens(orc):
    x, Bm, Cm, dt, A, D, pool = spec_inputs(13)
    slot = np.array([6, 2, 0, -1])
    _, inter = orc.state_update_multi(pool, slot, x, Bm, Cm, dt, A, D)
    acc = np.array([3, 0, 9, 2])                      # 0 keeps the slot; 9 > k clamps to k
    new = orc.accept_states(pool, inter, acc, slot)
    k = x.shape[1]
    for b, n in enumerate(acc):
        if slot[b] < 0:
            continue
        n = min(n, k)
        if n == 0:
            assert np.array_equal(new[slot[b]], pool[slot[b]])
            continue
        _, fr = semiseparable_scan(x[b:b + 1, :n], Bm[b:b + 1, :n], Cm[b:b + 1, :n], dt[b:b + 1, :n], A, D,
                                   pool[slot[b]][None])
        assert rel_err(new[slot[b]], fr[0]) < 1e-12, b
    for s in (1, 3, 4, 5):                            # slots no request names are untouched
        assert np.array_equal(new[s], pool[s])


def test_single_candidate_is_the_plain_update(orc):
    x, Bm, Cm, dt, A, D, pool = spec_inputs(14, k=1, nslots=4)
    y, inter = orc.state_update_multi(pool, None, x, Bm, Cm, dt, A, D)
    yr, sr = orc.state_update(pool, x[:, 0], Bm[:, 0], Cm[:, 0], dt[:, 0], A, D)
    assert np.array_equal(y[:, 0], yr) and np.array_equal(inter[:, 0], sr)


def test_scan_varlen_snapshots_are_the_prefix_states(orc):
    """Packed sequences with snapshots into a pool: the slot that the table names for (sequence s,
    interval k) holds the brute-force final state of that sequence's first (k + 1) * interval
    tokens, from its initial state when it has one; table entries past a sequence's snapshot
    count, negative ones and ones outside the pool store nothing; y and the state pool are the
    plain packed scan's."""
    r = np.random.default_rng(16)
    lens, H, P, G, N, iv = [11, 0, 4, 16, 5], 4, 3, 2, 5, 5
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    x = r.standard_normal((T, H, P))
    Bm = r.standard_normal((T, G, N))
    Cm = r.standard_normal((T, G, N))
    dt = softplus(r.normal(-2.0, 1.0, (T, H)))
    A = -np.exp(r.uniform(0, 1, H))
    D = r.standard_normal(H)
    pool = r.standard_normal((6, H, P, N))
    slot, has_init = np.array([3, 0, -1, 5, 1]), np.array([1, 0, 0, 1, 0])
    snap0 = r.standard_normal((9, H, P, N))
    table = np.array([[2, 7, 8], [4, -1, 0], [0, 1, 2], [6, 3, 9], [5, -2, 1]])
    y, newp, snaps = orc.scan_varlen_snapshots(x, Bm, Cm, dt, A, D, cu, pool, slot, has_init, snap0, table, iv)
    yr, pr = orc.scan_varlen(x, Bm, Cm, dt, A, D, cu, pool, slot, has_init)
    assert rel_err(y, yr) == 0 and rel_err(newp, pr) == 0
    want = snap0.copy()
    for s, L in enumerate(lens):
        S0 = pool[slot[s]][None] if slot[s] >= 0 and has_init[s] else np.zeros((1, H, P, N))
        for k in range(min(L // iv, table.shape[1])):
            if 0 <= table[s, k] < 9:
                a, e = cu[s], cu[s] + (k + 1) * iv
                _, fr = semiseparable_scan(x[None, a:e], Bm[None, a:e], Cm[None, a:e], dt[None, a:e], A, D, S0)
                want[table[s, k]] = fr[0]
    assert rel_err(snaps, want) < 1e-12
    # slot 8 is named only by sequence 0's third interval, which its 11 tokens do not reach
    assert np.array_equal(snaps[8], snap0[8]), "an entry past a sequence's snapshot count stores nothing"


def test_scan_snapshots_are_the_prefix_states(orc):
    """State snapshots every `interval` tokens ("modeling_nemotron_h.py" walk-through page,
    部署时如何调这些缓存: a state snapshot every N tokens): snapshot k equals the brute-force final
    state of tokens [0, (k + 1) * interval), and the segmented scan's y and final state equal the
    one-pass scan's."""
    r = np.random.default_rng(15)
    Bt, L, H, P, G, N, iv = 2, 23, 4, 3, 2, 5, 5
    x = r.standard_normal((Bt, L, H, P))
    Bm = r.standard_normal((Bt, L, G, N))
    Cm = r.standard_normal((Bt, L, G, N))
    dt = softplus(r.normal(-2.0, 1.0, (Bt, L, H)))
    A = -np.exp(r.uniform(0, 1, H))
    D = r.standard_normal(H)
    S0 = r.standard_normal((Bt, H, P, N))
    y, fin, snaps = orc.scan_snapshots(x, Bm, Cm, dt, A, D, S0, iv)
    assert snaps.shape == (Bt, L // iv, H, P, N)
    for k in range(L // iv):
        e = (k + 1) * iv
        _, fr = semiseparable_scan(x[:, :e], Bm[:, :e], Cm[:, :e], dt[:, :e], A, D, S0)
        assert rel_err(snaps[:, k], fr) < 1e-12, k
    yr, fr = orc.scan(x, Bm, Cm, dt, A, D, S0)
    assert rel_err(y, yr) < 1e-12 and rel_err(fin, fr) < 1e-12
