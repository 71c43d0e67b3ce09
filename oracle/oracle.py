"""ctypes marshalling for the oracle's C library (no arithmetic here).

TEST INFRASTRUCTURE ONLY.  All inputs are converted to C-contiguous float64
numpy arrays; outputs are returned as new float64 arrays.
"""
import ctypes
import os

import numpy as np

from . import build_oracle

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


_DEFAULT = None


def load(rebuild_if_missing=True):
    """Return the oracle built in-tree (building it with gcc if absent)."""
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(build_oracle.LIB) and rebuild_if_missing:
            build_oracle.build()
        _DEFAULT = Oracle(build_oracle.LIB)
    return _DEFAULT
