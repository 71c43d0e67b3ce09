"""Pins for the oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes a loaded oracle and raises AssertionError on a mismatch.
They are run on the real oracle (test_oracle_pins.py) and on deliberately
broken copies of it (test_oracle_mutants.py), so that every plausible slip in
the oracle -- a dropped term, a wrong sign, a wrong index, a transposed
operand -- is caught by at least one of them.

What pins what (sources cited by page title and section):
  * scan           brute-force semiseparable (quadratic) form built from the
                   unrolled recurrence -- "Mamba 与 Nemotron 系列模型深度调研",
                   "Mamba 架构" (Mamba-2 ties the SSM to a structured
                   semiseparable matrix; recurrence in section 1).
  * scan, N=1      exact solution of the scalar recurrence by cumprod/cumsum
                   (variation of parameters) -- the "Mamba" tag page
                   (baguaai.com), item on SM1 (Scalar Mamba1).
  * conv           torch.nn.functional.conv1d(groups=channels) in fp64 + SiLU
                   -- "MAX 平台 Nemotron-H 混合架构解析", 5.4 (depthwise SiLU
                   conv); modeling_nemotron_h.py walk-through, "Prefill 阶段".
  * conv update    token-by-token roll equals the prefill conv --
                   modeling_nemotron_h.py walk-through, "Decode 阶段".
  * invariants     dt=0 keeps the state; A*dt -> -inf resets it;
                   prefill-then-decode equals a longer prefill; split prefill;
                   NULL init == zero init; identical groups == one group;
                   linearity in (x, init); B=0 / C=0 leave y = D*x; state layout
                   [P, N] via one-hot C.
"""
import numpy as np
import torch


def softplus(z):
    return np.log1p(np.exp(z))


def rand_scan(seed, Bt=2, L=37, H=4, P=3, G=2, N=5, init=True, slow=False):
    r = np.random.default_rng(seed)
    x = r.standard_normal((Bt, L, H, P))
    Bm = r.standard_normal((Bt, L, G, N))
    Cm = r.standard_normal((Bt, L, G, N))
    dt = softplus(r.normal(-4.0 if slow else -2.0, 1.0, (Bt, L, H)))
    A = -np.exp(r.uniform(-3 if slow else 0, -1 if slow else 1, H))
    D = r.standard_normal(H)
    S0 = r.standard_normal((Bt, H, P, N)) if init else None
    return x, Bm, Cm, dt, A, D, S0


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------
# brute force: the unrolled recurrence as one quadratic (semiseparable) form
# --------------------------------------------------------------------------
def semiseparable_scan(x, Bm, Cm, dt, A, D, S0):
    """y[t] = sum_{s<=t} (C_t.B_s) exp(A(cum_t - cum_s)) dt_s x_s
              + exp(A cum_t) (C_t . S0) + D x_t,  cum_t = sum_{k<=t} dt_k.
    Final state = sum_s exp(A(cum_{L-1}-cum_s)) dt_s x_s (x) B_s + exp(A cum_{L-1}) S0."""
    Bt, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    hpg = H // G
    y = np.zeros((Bt, L, H, P))
    fin = np.zeros((Bt, H, P, N))
    tri = np.tril(np.ones((L, L), dtype=bool))
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            cum = np.cumsum(dt[b, :, h])
            seg = A[h] * (cum[:, None] - cum[None, :])                 # [t, s]
            decay = np.where(tri, np.exp(np.where(tri, seg, 0.0)), 0.0)
            CB = Cm[b, :, g, :] @ Bm[b, :, g, :].T                       # [t, s]
            M = CB * decay * dt[b, None, :, h]
            y[b, :, h, :] = M @ x[b, :, h, :]
            w_last = np.exp(A[h] * (cum[-1] - cum)) * dt[b, :, h]        # [s]
            fin[b, h] = (x[b, :, h, :] * w_last[:, None]).T @ Bm[b, :, g, :]
            if S0 is not None:
                y[b, :, h, :] += np.exp(A[h] * cum)[:, None] * (Cm[b, :, g, :] @ S0[b, h].T)
                fin[b, h] += np.exp(A[h] * cum[-1]) * S0[b, h]
            if D is not None:
                y[b, :, h, :] += D[h] * x[b, :, h, :]
    return y, fin


def pin_scan_bruteforce(orc):
    for seed, kw in [(1, {}), (2, dict(init=False)), (3, dict(slow=True, L=64, G=1)),
                     (4, dict(Bt=1, L=1)), (5, dict(H=6, G=3, P=2, N=7, L=20))]:
        x, Bm, Cm, dt, A, D, S0 = rand_scan(seed, **kw)
        y, fin = orc.scan(x, Bm, Cm, dt, A, D, S0)
        yr, finr = semiseparable_scan(x, Bm, Cm, dt, A, D, S0)
        assert rel_err(y, yr) < 1e-11, ("y", seed, rel_err(y, yr))
        assert rel_err(fin, finr) < 1e-11, ("state", seed, rel_err(fin, finr))


# --------------------------------------------------------------------------
# closed form for d_state = 1 via cumprod / cumsum (variation of parameters)
# --------------------------------------------------------------------------
def closed_form_n1(x, Bm, Cm, dt, A, D, S0):
    """s_t = Pi_t (s_0 + sum_{k<=t} dt_k B_k x_k / Pi_k),  Pi_t = prod_{k<=t} exp(dt_k A)."""
    xt = torch.from_numpy(x)
    Bt, L, H, P = x.shape
    G = Bm.shape[2]
    g_of_h = torch.arange(H) // (H // G)
    Bh = torch.from_numpy(Bm[..., 0])[:, :, g_of_h]                  # [Bt, L, H]
    Ch = torch.from_numpy(Cm[..., 0])[:, :, g_of_h]
    dtt = torch.from_numpy(dt)
    At = torch.from_numpy(A)
    Pi = torch.cumprod(torch.exp(dtt * At), dim=1)                   # [Bt, L, H]
    drive = (dtt * Bh)[..., None] * xt                               # [Bt, L, H, P]
    s0 = torch.zeros(Bt, H, P) if S0 is None else torch.from_numpy(S0[..., 0])
    s = Pi[..., None] * (s0[:, None] + torch.cumsum(drive / Pi[..., None], dim=1))
    y = Ch[..., None] * s + torch.from_numpy(D)[None, None, :, None] * xt
    return y.numpy(), s[:, -1].numpy()[..., None]


def pin_scan_closed_form_n1(orc):
    for seed, kw in [(11, dict(N=1, L=48)), (12, dict(N=1, L=30, G=1, H=3, init=False)),
                     (13, dict(N=1, L=64, slow=True))]:
        x, Bm, Cm, dt, A, D, S0 = rand_scan(seed, **kw)
        y, fin = orc.scan(x, Bm, Cm, dt, A, D, S0)
        yr, finr = closed_form_n1(x, Bm, Cm, dt, A, D, S0)
        assert rel_err(y, yr) < 1e-10, ("y", seed, rel_err(y, yr))
        assert rel_err(fin, finr) < 1e-10, ("state", seed, rel_err(fin, finr))


# --------------------------------------------------------------------------
# conv against the library routine
# --------------------------------------------------------------------------
def torch_conv(u, w, bias, s_in):
    """Depthwise causal conv + SiLU with torch.nn.functional.conv1d (fp64, CPU).
    The K-1 columns of the previous window (s_in[:, :, 1:]) are prepended."""
    Bt, L, CD = u.shape
    K = w.shape[1]
    ut = torch.from_numpy(u).transpose(1, 2)                         # [Bt, CD, L]
    halo = torch.zeros(Bt, CD, K - 1, dtype=torch.float64) if s_in is None \
        else torch.from_numpy(s_in[:, :, 1:])
    ext = torch.cat([halo, ut], dim=2)                               # [Bt, CD, L+K-1]
    z = torch.nn.functional.conv1d(ext, torch.from_numpy(w)[:, None, :],
                                   None if bias is None else torch.from_numpy(bias), groups=CD)
    v = torch.nn.functional.silu(z).transpose(1, 2).contiguous()
    s_out = ext[:, :, -K:].contiguous()
    return v.numpy(), s_out.numpy()


def rand_conv(seed, Bt=2, L=19, CD=12, K=4, state=True, bias=True):
    r = np.random.default_rng(seed)
    u = r.standard_normal((Bt, L, CD))
    w = r.uniform(-0.5, 0.5, (CD, K))
    b = r.uniform(-0.5, 0.5, CD) if bias else None
    s = r.standard_normal((Bt, CD, K)) if state else None
    return u, w, b, s


def pin_conv_torch(orc):
    for seed, kw in [(21, {}), (22, dict(state=False)), (23, dict(L=2)), (24, dict(L=1, bias=False)),
                     (25, dict(L=3, CD=5)), (26, dict(K=3, L=7))]:
        u, w, b, s = rand_conv(seed, **kw)
        v, so = orc.conv1d_fwd(u, w, b, s)
        vr, sor = torch_conv(u, w, b, s)
        assert rel_err(v, vr) < 1e-13, ("conv v", seed, rel_err(v, vr))
        assert np.array_equal(so, sor), ("conv state", seed)


def pin_conv_update_equals_prefill(orc):
    for seed, kw in [(31, {}), (32, dict(state=False, L=6)), (33, dict(L=2, CD=7))]:
        u, w, b, s = rand_conv(seed, **kw)
        vp, sp = orc.conv1d_fwd(u, w, b, s)
        st = np.zeros_like(sp) if s is None else s.copy()
        vs = []
        for t in range(u.shape[1]):
            vt, st = orc.conv1d_update(u[:, t], w, b, st)
            vs.append(vt)
        assert np.array_equal(np.stack(vs, 1), vp), ("update vs prefill v", seed)
        assert np.array_equal(st, sp), ("update vs prefill state", seed)


# --------------------------------------------------------------------------
# invariants
# --------------------------------------------------------------------------
def pin_dt_zero_keeps_state(orc):
    x, Bm, Cm, dt, A, D, S0 = rand_scan(41)
    dt = np.zeros_like(dt)
    y, fin = orc.scan(x, Bm, Cm, dt, A, D, S0)
    assert np.array_equal(fin, S0)
    hpg = x.shape[2] // Bm.shape[2]
    # y_t = C_t . S0 + D x_t, per head
    for h in range(x.shape[2]):
        g = h // hpg
        yh = np.einsum("bln,bpn->blp", Cm[:, :, g], S0[:, h]) + D[h] * x[:, :, h]
        assert rel_err(y[:, :, h], yh) < 1e-13


def pin_reset_with_huge_decay(orc):
    x, Bm, Cm, dt, A, D, S0 = rand_scan(42)
    A = np.full_like(A, -1e6)
    y, fin = orc.scan(x, Bm, Cm, dt, A, D, S0)
    assert np.all(np.isfinite(y)) and np.all(np.isfinite(fin))
    hpg = x.shape[2] // Bm.shape[2]
    for h in range(x.shape[2]):
        g = h // hpg
        CB = np.einsum("bln,bln->bl", Cm[:, :, g], Bm[:, :, g])
        yh = (dt[:, :, h] * CB)[..., None] * x[:, :, h] + D[h] * x[:, :, h]
        assert rel_err(y[:, :, h], yh) < 1e-13
        fh = dt[:, -1, h][:, None, None] * x[:, -1, h][:, :, None] * Bm[:, -1, g][:, None, :]
        assert rel_err(fin[:, h], fh) < 1e-13


def pin_prefill_then_decode(orc):
    x, Bm, Cm, dt, A, D, S0 = rand_scan(43, L=30)
    L1 = 22
    y_all, fin_all = orc.scan(x, Bm, Cm, dt, A, D, S0)
    y1, st = orc.scan(x[:, :L1], Bm[:, :L1], Cm[:, :L1], dt[:, :L1], A, D, S0)
    assert rel_err(y1, y_all[:, :L1]) < 1e-14
    for t in range(L1, x.shape[1]):
        yt, st = orc.state_update(st, x[:, t], Bm[:, t], Cm[:, t], dt[:, t], A, D)
        assert rel_err(yt, y_all[:, t]) < 1e-12, ("decode y", t)
    assert rel_err(st, fin_all) < 1e-12


def pin_split_prefill(orc):
    x, Bm, Cm, dt, A, D, S0 = rand_scan(44, L=40)
    L1 = 17
    y_all, fin_all = orc.scan(x, Bm, Cm, dt, A, D, S0)
    y1, f1 = orc.scan(x[:, :L1], Bm[:, :L1], Cm[:, :L1], dt[:, :L1], A, D, S0)
    y2, f2 = orc.scan(x[:, L1:], Bm[:, L1:], Cm[:, L1:], dt[:, L1:], A, D, f1)
    assert rel_err(np.concatenate([y1, y2], 1), y_all) < 1e-12
    assert rel_err(f2, fin_all) < 1e-12


def pin_null_init_is_zero(orc):
    x, Bm, Cm, dt, A, D, _ = rand_scan(45, init=False)
    y0, f0 = orc.scan(x, Bm, Cm, dt, A, D, None)
    yz, fz = orc.scan(x, Bm, Cm, dt, A, D, np.zeros((x.shape[0], x.shape[2], x.shape[3], Bm.shape[3])))
    assert np.array_equal(y0, yz) and np.array_equal(f0, fz)


def pin_groups_identical_equals_one_group(orc):
    x, Bm, Cm, dt, A, D, S0 = rand_scan(46, G=1, H=6)
    y1, f1 = orc.scan(x, Bm, Cm, dt, A, D, S0)
    y3, f3 = orc.scan(x, np.repeat(Bm, 3, axis=2), np.repeat(Cm, 3, axis=2), dt, A, D, S0)
    assert np.array_equal(y1, y3) and np.array_equal(f1, f3)
    # distinct groups: head h must read group h // (H/G) -- compare with per-head G=1 runs
    x, Bm, Cm, dt, A, D, S0 = rand_scan(47, G=3, H=6)
    y, f = orc.scan(x, Bm, Cm, dt, A, D, S0)
    for h in range(6):
        g = h // 2
        yh, fh = orc.scan(x[:, :, h:h + 1], Bm[:, :, g:g + 1], Cm[:, :, g:g + 1], dt[:, :, h:h + 1],
                          A[h:h + 1], D[h:h + 1], S0[:, h:h + 1])
        assert np.array_equal(y[:, :, h:h + 1], yh) and np.array_equal(f[:, h:h + 1], fh)


def pin_linearity(orc):
    x, Bm, Cm, dt, A, D, S0 = rand_scan(48)
    y, f = orc.scan(x, Bm, Cm, dt, A, D, S0)
    y2, f2 = orc.scan(2 * x, Bm, Cm, dt, A, D, 2 * S0)
    assert np.array_equal(y2, 2 * y) and np.array_equal(f2, 2 * f)
    xb = np.random.default_rng(49).standard_normal(x.shape)
    ya, fa = orc.scan(x, Bm, Cm, dt, A, D, None)
    yb, fb = orc.scan(xb, Bm, Cm, dt, A, D, None)
    yab, fab = orc.scan(x + xb, Bm, Cm, dt, A, D, None)
    assert rel_err(ya + yb, yab) < 1e-12 and rel_err(fa + fb, fab) < 1e-12


def pin_zero_B_or_C(orc):
    x, Bm, Cm, dt, A, D, S0 = rand_scan(50)
    y, _ = orc.scan(x, np.zeros_like(Bm), Cm, dt, A, D, None)
    assert np.array_equal(y, D[None, None, :, None] * x)
    y, _ = orc.scan(x, Bm, np.zeros_like(Cm), dt, A, D, S0)
    assert np.array_equal(y, D[None, None, :, None] * x)


def pin_state_layout_one_hot_C(orc):
    x, Bm, Cm, dt, A, D, S0 = rand_scan(51, P=3, N=5)
    for n in range(Cm.shape[3]):
        C1 = np.zeros_like(Cm)
        C1[..., n] = 1.0
        y, fin = orc.scan(x, Bm, C1, dt, A, None, S0)
        assert np.array_equal(y[:, -1], fin[..., n]), n


def pin_state_update_matches_bruteforce(orc):
    r = np.random.default_rng(52)
    Bt, H, P, G, N = 3, 4, 3, 2, 5
    st = r.standard_normal((Bt, H, P, N))
    x = r.standard_normal((Bt, H, P))
    Bm = r.standard_normal((Bt, G, N))
    Cm = r.standard_normal((Bt, G, N))
    dt = softplus(r.normal(-2, 1, (Bt, H)))
    A = -np.exp(r.uniform(0, 1, H))
    D = r.standard_normal(H)
    y, new = orc.state_update(st, x, Bm, Cm, dt, A, D)
    yr, fr = semiseparable_scan(x[:, None], Bm[:, None], Cm[:, None], dt[:, None], A, D, st)
    assert rel_err(y, yr[:, 0]) < 1e-13 and rel_err(new, fr) < 1e-13


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
