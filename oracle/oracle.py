"""ctypes marshalling for the oracle's C library (no arithmetic here).

TEST INFRASTRUCTURE ONLY.  All inputs are converted to C-contiguous float64
numpy arrays; outputs are returned as new float64 arrays.
"""
import ctypes
import os

import numpy as np

from . import build_oracle, lowprec

_D = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64
_I32 = ctypes.c_int


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_D)


class Oracle:
    """Thin wrapper around one loaded copy of the oracle library."""

    def __init__(self, libpath):
        self.libpath = libpath
        lib = ctypes.CDLL(libpath)
        lib.oracle_conv1d_fwd.argtypes = [_I64, _I64, _I64, _I32, _D, _D, _D, _D, _D, _D]
        lib.oracle_conv1d_fwd.restype = None
        lib.oracle_conv1d_update.argtypes = [_I64, _I64, _I32, _D, _D, _D, _D, _D]
        lib.oracle_conv1d_update.restype = None
        lib.oracle_ssm_scan.argtypes = [_I64, _I64, _I32, _I32, _I32, _I32,
                                        _D, _D, _D, _D, _D, _D, _D, _D, _D]
        lib.oracle_ssm_scan.restype = None
        lib.oracle_state_update.argtypes = [_I64, _I32, _I32, _I32, _I32, _D,
                                            _D, _D, _D, _D, _D, _D, _D]
        lib.oracle_state_update.restype = None
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = _I32
        self.lib = lib

    def num_threads(self):
        return int(self.lib.oracle_num_threads())

    # u [B,L,CD], w [CD,K], bias [CD]|None, s_in [B,CD,K]|None -> v [B,L,CD], s_out [B,CD,K]
    def conv1d_fwd(self, u, w, bias=None, s_in=None):
        u, w, bias, s_in = _f64(u), _f64(w), _f64(bias), _f64(s_in)
        Bt, L, CD = u.shape
        K = w.shape[1]
        assert w.shape == (CD, K)
        assert bias is None or bias.shape == (CD,)
        assert s_in is None or s_in.shape == (Bt, CD, K)
        v = np.empty((Bt, L, CD), np.float64)
        s_out = np.empty((Bt, CD, K), np.float64)
        self.lib.oracle_conv1d_fwd(Bt, L, CD, K, _ptr(u), _ptr(w), _ptr(bias), _ptr(s_in),
                                   _ptr(v), _ptr(s_out))
        return v, s_out

    # u [B,CD], s [B,CD,K] -> v [B,CD], s_new [B,CD,K] (input s is not modified)
    def conv1d_update(self, u, w, bias, s):
        u, w, bias = _f64(u), _f64(w), _f64(bias)
        s = np.array(s, dtype=np.float64, order="C", copy=True)
        Bt, CD = u.shape
        K = w.shape[1]
        assert s.shape == (Bt, CD, K)
        v = np.empty((Bt, CD), np.float64)
        self.lib.oracle_conv1d_update(Bt, CD, K, _ptr(u), _ptr(w), _ptr(bias), _ptr(s), _ptr(v))
        return v, s

    # x [B,L,H,P], Bm/Cm [B,L,G,N], dt [B,L,H], A [H], D [H]|None, init [B,H,P,N]|None
    def scan(self, x, Bm, Cm, dt, A, D=None, init=None):
        x, Bm, Cm, dt, A, D, init = map(_f64, (x, Bm, Cm, dt, A, D, init))
        Bt, L, H, P = x.shape
        G, N = Bm.shape[2], Bm.shape[3]
        assert Bm.shape == (Bt, L, G, N) and Cm.shape == (Bt, L, G, N)
        assert dt.shape == (Bt, L, H) and A.shape == (H,) and H % G == 0
        assert D is None or D.shape == (H,)
        assert init is None or init.shape == (Bt, H, P, N)
        y = np.empty((Bt, L, H, P), np.float64)
        fin = np.empty((Bt, H, P, N), np.float64)
        self.lib.oracle_ssm_scan(Bt, L, H, P, G, N, _ptr(x), _ptr(Bm), _ptr(Cm), _ptr(dt),
                                 _ptr(A), _ptr(D), _ptr(init), _ptr(y), _ptr(fin))
        return y, fin

    # state [B,H,P,N], x [B,H,P], Bm/Cm [B,G,N], dt [B,H] -> y [B,H,P], new state (copy)
    def state_update(self, state, x, Bm, Cm, dt, A, D=None):
        x, Bm, Cm, dt, A, D = map(_f64, (x, Bm, Cm, dt, A, D))
        st = np.array(state, dtype=np.float64, order="C", copy=True)
        Bt, H, P, N = st.shape
        G = Bm.shape[1]
        assert x.shape == (Bt, H, P) and Bm.shape == (Bt, G, N) and Cm.shape == (Bt, G, N)
        assert dt.shape == (Bt, H) and H % G == 0
        y = np.empty((Bt, H, P), np.float64)
        self.lib.oracle_state_update(Bt, H, P, G, N, _ptr(st), _ptr(x), _ptr(Bm), _ptr(Cm),
                                     _ptr(dt), _ptr(A), _ptr(D), _ptr(y))
        return y, st

    # The state after every `interval` tokens: the scan run segment by segment, each segment
    # starting from the previous one's final state.  -> y, final state, snapshots [B, L // interval, H, P, N]
    def scan_snapshots(self, x, Bm, Cm, dt, A, D=None, init=None, interval=128):
        x, Bm, Cm, dt = map(_f64, (x, Bm, Cm, dt))
        Bt, L, H, P = x.shape
        N = Bm.shape[3]
        st = np.zeros((Bt, H, P, N)) if init is None else _f64(init)
        ys, snaps = [], []
        for a in range(0, L, interval):
            b = min(a + interval, L)
            yk, st = self.scan(x[:, a:b], Bm[:, a:b], Cm[:, a:b], dt[:, a:b], A, D, st)
            ys.append(yk)
            if b - a == interval:
                snaps.append(st)
        snaps = np.stack(snaps, 1) if snaps else np.zeros((Bt, 0, H, P, N))
        return (np.concatenate(ys, 1) if ys else np.zeros((Bt, 0, H, P))), st, snaps

    # Gated group RMSNorm after the scan, gate applied before the norm ("MAX 平台 Nemotron-H 混合架构解析",
    # 5.4, item 4: silu gate in fp32, RMS norm over each group of channels, fp32 weight):
    # v = y * silu(z); out = v / sqrt(mean over the group of v^2 + eps) * w.
    # y, z [..., I] with I = ngroups * group size, w [I] -> out [..., I] (fp64)
    @staticmethod
    def gated_rmsnorm(y, z, w, ngroups, eps):
        y, z, w = (np.asarray(t, dtype=np.float64) for t in (y, z, w))
        v = y * (z / (1.0 + np.exp(-z)))
        g = v.reshape(v.shape[:-1] + (ngroups, -1))
        r = 1.0 / np.sqrt((g * g).mean(-1, keepdims=True) + eps)
        return (g * r).reshape(v.shape) * w

    # dt prologue (fp64), applied to dt [..., H] before the routines above: v = dt + bias[h];
    # softplus v = log(1 + e^v); clamp to [lo, hi] when lo < hi.
    @staticmethod
    def dt_prologue(dt, bias=None, softplus=False, limit=None):
        v = np.array(dt, dtype=np.float64)
        if bias is not None:
            v = v + np.asarray(bias, dtype=np.float64)
        if softplus:
            v = np.logaddexp(0.0, v)
        if limit is not None and limit[0] < limit[1]:
            v = np.clip(v, limit[0], limit[1])
        return v

    # ------------------------------------------------------------------ packed batches
    # The plain per-sequence definition of the packed calls: sequence s is rows
    # [cu[s], cu[s+1]) of the packed [T, ...] tensors and is run on its own by the routines
    # above.  Its states are slot slot[s] (s when slot is None) of the pools; has_init[s] != 0
    # starts it from that slot, else from zeros.  A slot outside [0, nslots) is padding: zero
    # start, nothing stored.  Pools are returned as updated copies.
    @staticmethod
    def _slot(slot, s, nslots):
        v = s if slot is None else int(slot[s])
        return v if 0 <= v < nslots else -1

    # u [T,CD], pool [nslots,CD,K]|None -> v [T,CD], new pool
    def conv1d_fwd_varlen(self, u, w, bias, cu, pool=None, slot=None, has_init=None):
        u = _f64(u)
        cu = [int(c) for c in cu]
        v = np.zeros_like(u)
        new = None if pool is None else np.array(pool, dtype=np.float64, order="C", copy=True)
        nslots = 0 if pool is None else new.shape[0]
        for s in range(len(cu) - 1):
            a, b = cu[s], cu[s + 1]
            k = self._slot(slot, s, nslots)
            start = k >= 0 and has_init is not None and int(has_init[s]) != 0
            vs, s_out = self.conv1d_fwd(u[None, a:b], w, bias, new[k][None] if start else None)
            v[a:b] = vs[0]
            if k >= 0:
                new[k] = s_out[0]
        return v, new

    # x [T,H,P], Bm/Cm [T,G,N], dt [T,H], pool [nslots,H,P,N]|None -> y [T,H,P], new pool
    def scan_varlen(self, x, Bm, Cm, dt, A, D, cu, pool=None, slot=None, has_init=None):
        x, Bm, Cm, dt = map(_f64, (x, Bm, Cm, dt))
        cu = [int(c) for c in cu]
        y = np.zeros_like(x)
        new = None if pool is None else np.array(pool, dtype=np.float64, order="C", copy=True)
        nslots = 0 if pool is None else new.shape[0]
        for s in range(len(cu) - 1):
            a, b = cu[s], cu[s + 1]
            k = self._slot(slot, s, nslots)
            start = k >= 0 and has_init is not None and int(has_init[s]) != 0
            ys, fin = self.scan(x[None, a:b], Bm[None, a:b], Cm[None, a:b], dt[None, a:b], A, D,
                                new[k][None] if start else None)
            y[a:b] = ys[0]
            if k >= 0:
                new[k] = fin[0]
        return y, new

    # The packed scan with snapshots into a pool (the modeling_nemotron_h.py walk-through page,
    # 部署时如何调这些缓存: a state snapshot every N tokens for prefix caching): each sequence is
    # scanned with scan_snapshots, and its k-th snapshot goes to pool slot snap_table[s, k] when
    # that names a slot.  -> y, new state pool, new snapshot pool
    def scan_varlen_snapshots(self, x, Bm, Cm, dt, A, D, cu, pool, slot, has_init, snap_pool, snap_table,
                              interval):
        x, Bm, Cm, dt = map(_f64, (x, Bm, Cm, dt))
        cu = [int(c) for c in cu]
        y = np.zeros_like(x)
        new = None if pool is None else np.array(pool, dtype=np.float64, order="C", copy=True)
        snaps = np.array(snap_pool, dtype=np.float64, order="C", copy=True)
        nslots = 0 if pool is None else new.shape[0]
        table = np.asarray(snap_table)
        for s in range(len(cu) - 1):
            a, b = cu[s], cu[s + 1]
            k = self._slot(slot, s, nslots)
            start = k >= 0 and has_init is not None and int(has_init[s]) != 0
            ys, fin, sn = self.scan_snapshots(x[None, a:b], Bm[None, a:b], Cm[None, a:b], dt[None, a:b], A, D,
                                              new[k][None] if start else None, interval)
            y[a:b] = ys[0]
            if k >= 0:
                new[k] = fin[0]
            for j in range(min(sn.shape[1], table.shape[1])):
                sl = int(table[s, j])
                if 0 <= sl < snaps.shape[0]:
                    snaps[sl] = sn[0, j]
        return y, new, snaps

    # u [B,CD], pool [nslots,CD,K], slot [B] -> v [B,CD], new pool
    def conv1d_update_slots(self, u, w, bias, pool, slot):
        u = _f64(u)
        new = np.array(pool, dtype=np.float64, order="C", copy=True)
        v = np.zeros_like(u)
        for b in range(u.shape[0]):
            k = self._slot(slot, b, new.shape[0])
            win = new[k][None] if k >= 0 else np.zeros((1,) + new.shape[1:])
            vb, wb = self.conv1d_update(u[b:b + 1], w, bias, win)
            v[b] = vb[0]
            if k >= 0:
                new[k] = wb[0]
        return v, new

    # pool [nslots,H,P,N], slot [B], x [B,H,P], Bm/Cm [B,G,N], dt [B,H] -> y [B,H,P], new pool
    def state_update_slots(self, pool, slot, x, Bm, Cm, dt, A, D=None):
        x, Bm, Cm, dt = map(_f64, (x, Bm, Cm, dt))
        new = np.array(pool, dtype=np.float64, order="C", copy=True)
        y = np.zeros_like(x)
        for b in range(x.shape[0]):
            k = self._slot(slot, b, new.shape[0])
            st = new[k][None] if k >= 0 else np.zeros((1,) + new.shape[1:])
            yb, sb = self.state_update(st, x[b:b + 1], Bm[b:b + 1], Cm[b:b + 1], dt[b:b + 1], A, D)
            y[b] = yb[0]
            if k >= 0:
                new[k] = sb[0]
        return y, new

    # ------------------------------------------------------------------ speculative decode
    # ("Mamba 与 Nemotron 系列模型深度调研", 状态契约, MTP / speculative decoding: each candidate
    # token leaves an intermediate recurrent and conv state; the accepted length selects the one
    # written back to the request's state.)
    # The plain definition of multi-token decode: the k candidate tokens of request b run one
    # after another through the single-token routines above, starting from slot slot[b] of the
    # pool (b when slot is None; zeros for padding), and the state after every token is kept.
    # The pool itself is not changed.  accept_states then copies the state after token n
    # (n = accept_len[b], clamped to [0, k]; n = 0 keeps the slot) back into the slot.

    # pool [nslots,H,P,N], x [B,k,H,P], Bm/Cm [B,k,G,N], dt [B,k,H] -> y [B,k,H,P], inter [B,k,H,P,N]
    def state_update_multi(self, pool, slot, x, Bm, Cm, dt, A, D=None):
        x, Bm, Cm, dt, pool = map(_f64, (x, Bm, Cm, dt, pool))
        Bt, k = x.shape[:2]
        y = np.zeros_like(x)
        inter = np.zeros((Bt, k) + pool.shape[1:])
        for b in range(Bt):
            s = self._slot(slot, b, pool.shape[0])
            st = pool[s][None] if s >= 0 else np.zeros((1,) + pool.shape[1:])
            for j in range(k):
                yj, st = self.state_update(st, x[b:b + 1, j], Bm[b:b + 1, j], Cm[b:b + 1, j], dt[b:b + 1, j], A, D)
                y[b, j] = yj[0]
                inter[b, j] = st[0]
        return y, inter

    # u [B,k,CD], pool [nslots,CD,K] -> v [B,k,CD], inter [B,k,CD,K]
    def conv1d_update_multi(self, u, w, bias, pool, slot):
        u, pool = _f64(u), _f64(pool)
        Bt, k = u.shape[:2]
        v = np.zeros_like(u)
        inter = np.zeros((Bt, k) + pool.shape[1:])
        for b in range(Bt):
            s = self._slot(slot, b, pool.shape[0])
            st = pool[s][None] if s >= 0 else np.zeros((1,) + pool.shape[1:])
            for j in range(k):
                vj, st = self.conv1d_update(u[b:b + 1, j], w, bias, st)
                v[b, j] = vj[0]
                inter[b, j] = st[0]
        return v, inter

    # pool [nslots, ...], inter [B, k, ...], accept_len [B] -> updated copy of the pool
    @classmethod
    def accept_states(cls, pool, inter, accept_len, slot=None):
        new = np.array(pool, dtype=np.float64, order="C", copy=True)
        k = inter.shape[1]
        for b in range(inter.shape[0]):
            s = cls._slot(slot, b, new.shape[0])
            n = min(max(int(accept_len[b]), 0), k)
            if s >= 0 and n >= 1:
                new[s] = inter[b, n - 1]
        return new

    # ------------------------------------------------------------------ reduced-precision state
    # The state is stored as uint16 codes of fmt ('f16' or 'bf16', see lowprec) and decoded for
    # the fp64 update above; the new state before rounding is returned, since which of the two
    # neighbouring codes stores it depends on the fp32 value the kernel rounds.
    # codes [nslots, H, P, N] uint16, slot [B]|None -> y [B,H,P], new state [B,H,P,N] (fp64, unrounded)
    def state_update_lp(self, codes, fmt, slot, x, Bm, Cm, dt, A, D=None):
        vals = lowprec.decode(codes, fmt)
        Bt = np.asarray(x).shape[0]
        st = np.zeros((Bt,) + vals.shape[1:])
        for b in range(Bt):
            s = self._slot(slot, b, vals.shape[0])
            if s >= 0:
                st[b] = vals[s]
        return self.state_update(st, x, Bm, Cm, dt, A, D)

    # With A = 0 for every head the update of an element is s + (dt*x)*B with the product dt*x,
    # its product with B and the sum each rounded to fp32: the exact value the fp32 kernels
    # compute.  Rounding it to fmt (round-to-nearest-even, or stochastically with
    # sr = (seed, offset, rounds), the element index being its flat index in the pool) gives the
    # codes that must be stored.  Returns the new pool of codes.
    @classmethod
    def state_update_lp_codes_a0(cls, codes, fmt, slot, x, Bm, Cm, dt, sr=None):
        codes = np.array(codes, dtype=np.uint16, copy=True)
        nslots, H, P, N = codes.shape
        x, Bm, Cm, dt = (np.asarray(t, dtype=np.float32) for t in (x, Bm, Cm, dt))
        G = Bm.shape[1]
        vals = lowprec.decode(codes, fmt).astype(np.float32)
        for b in range(x.shape[0]):
            s = cls._slot(slot, b, nslots)
            if s < 0:
                continue
            Bh = np.repeat(Bm[b], H // G, axis=0)                               # [H, N], group of each head
            dx = (dt[b][:, None] * x[b]).astype(np.float32)                      # [H, P]
            v = (vals[s] + (dx[:, :, None] * Bh[:, None, :]).astype(np.float32)).astype(np.float32)
            r16 = None
            if sr is not None:
                e = s * H * P * N + np.arange(H * P * N, dtype=np.int64).reshape(H, P, N)
                r16 = lowprec.random16(e, sr[0], sr[1], sr[2])
            codes[s] = lowprec.round_state(v, fmt, r16)
        return codes


    # ------------------------------------------------------------------ 16-bit state arrays
    # The scans on a state held as fp16 / bf16 codes (the modeling_nemotron_h.py walk-through,
    # 部署时如何调这些缓存: the Mamba state cache in fp16 with Philox stochastic rounding; "MAX
    # 平台 Nemotron-H 混合架构解析" 5.4: the state stored narrower than the fp32 the scan
    # accumulates in): the initial codes decode exactly, the scan runs on their values, and each
    # final state is rounded to fp32 and then to a code, element e (its flat index in the array or
    # pool) drawing its random number as in state_update_lp_codes_a0.  The kernels round their own
    # fp32 final state, so the codes returned here are theirs exactly when the fp64 final state is
    # representable in fp32 (A = 0 with inputs on a coarse dyadic grid); otherwise they are one of
    # the two codes around it.

    @staticmethod
    def round_states(vals, fmt, sr=None, first=0):
        """fp64 states [n, H, P, N], entries first .. first + n - 1 of their array -> uint16 codes."""
        v32 = np.asarray(vals, dtype=np.float64).astype(np.float32)
        r16 = None
        if sr is not None:
            e = first * int(np.prod(v32.shape[1:])) + np.arange(v32.size, dtype=np.int64).reshape(v32.shape)
            r16 = lowprec.random16(e, sr[0], sr[1], sr[2])
        return lowprec.round_state(v32, fmt, r16)

    # codes [B,H,P,N] uint16|None (zeros) -> y, final state (fp64), final codes
    def scan_lp(self, x, Bm, Cm, dt, A, D, codes, fmt, sr=None):
        init = None if codes is None else lowprec.decode(codes, fmt)
        y, fin = self.scan(x, Bm, Cm, dt, A, D, init)
        return y, fin, self.round_states(fin, fmt, sr)

    # pool codes [nslots,H,P,N] -> y [T,H,P], new pool codes (slots no sequence names keep theirs)
    def scan_varlen_lp(self, x, Bm, Cm, dt, A, D, cu, codes, fmt, slot=None, has_init=None, sr=None):
        codes = np.array(codes, dtype=np.uint16, copy=True)
        y, new = self.scan_varlen(x, Bm, Cm, dt, A, D, cu, lowprec.decode(codes, fmt), slot, has_init)
        for s in range(len(cu) - 1):
            k = self._slot(slot, s, codes.shape[0])
            if k >= 0:
                codes[k] = self.round_states(new[k][None], fmt, sr, first=k)[0]
        return y, codes


_DEFAULT = None


def load(rebuild_if_missing=True):
    """Return the oracle built in-tree (building it with gcc if absent)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(build_oracle.LIB) and rebuild_if_missing:
            build_oracle.build()
        _DEFAULT = Oracle(build_oracle.LIB)
    return _DEFAULT
