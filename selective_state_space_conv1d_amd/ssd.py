"""Python binding of libssd (ctypes): argument marshalling only.

Every function here checks tensor shapes/strides, derives the ABI's sizes and
row strides, and calls the C entry point of the same name on the current HIP
stream.  All arithmetic runs in the library's HIP kernels; there is no other
code path.  If libssd.so is missing this module raises on first use.

torch is used for device memory and streams only.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssd.so")

SSD_F32, SSD_BF16 = 0, 1
_DT = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}
STATUS = ["SSD_OK", "SSD_ERR_NULL", "SSD_ERR_SHAPE", "SSD_ERR_DTYPE", "SSD_ERR_ALIGN",
          "SSD_ERR_UNSUPPORTED", "SSD_ERR_WORKSPACE", "SSD_ERR_HIP"]
EXPORTS = ["ssd_conv_dim", "ssd_conv1d_fwd", "ssd_conv1d_update", "ssd_chunk_scan_workspace_size",
           "ssd_chunk_scan", "ssd_state_update", "ssd_status_string", "ssd_conv1d_fwd_varlen",
           "ssd_chunk_scan_varlen", "ssd_conv1d_update_slots", "ssd_state_update_slots",
           "ssd_state_update_multi", "ssd_conv1d_update_multi", "ssd_accept_states", "ssd_state_update_lp",
           "ssd_chunk_scan_snapshots", "ssd_gated_rmsnorm", "ssd_decode_step", "ssd_state_update_accept",
           "ssd_conv1d_update_accept", "ssd_chunk_scan_varlen_snapshots", "ssd_chunk_scan_noalloc",
           "ssd_conv_chunk_scan", "ssd_chunk_scan_lp", "ssd_chunk_scan_varlen_lp",
           "ssd_chunk_scan_varlen_workspace_size"]


class SsdDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ngroups", ctypes.c_int32), ("d_state", ctypes.c_int32),
                ("conv_width", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("y_dtype", ctypes.c_int32)]


class SsdError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        name = STATUS[code] if 0 <= code < len(STATUS) else str(code)
        super().__init__(f"{where}: {name} ({_lib().ssd_status_string(code).decode()})")


_LIB = None
class SsdDtParams(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("softplus", ctypes.c_int32), ("lo", ctypes.c_float),
                ("hi", ctypes.c_float)]


_VP = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_PD = ctypes.POINTER(SsdDims)


class SsdSrParams(ctypes.Structure):
    """Stochastic rounding of a 16-bit state: Philox key, counter offset and rounds."""
    _fields_ = [("seed", ctypes.c_uint64), ("offset", ctypes.c_uint64), ("rounds", ctypes.c_int32)]


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libssd.so is not built ({LIB_PATH}); run "
                               "python -m selective_state_space_conv1d_amd.build_lib")
        lib = ctypes.CDLL(LIB_PATH)
        lib.ssd_conv_dim.argtypes = [_PD]
        lib.ssd_conv_dim.restype = _I64
        lib.ssd_conv1d_fwd.argtypes = [_PD, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP]
        lib.ssd_conv1d_update.argtypes = [_PD, _VP, _I64, _VP, _VP, _VP, _VP, _VP]
        lib.ssd_chunk_scan_workspace_size.argtypes = [_PD, _I32]
        lib.ssd_chunk_scan_workspace_size.restype = ctypes.c_size_t
        lib.ssd_chunk_scan_varlen_workspace_size.argtypes = [_PD, _I32]
        lib.ssd_chunk_scan_varlen_workspace_size.restype = ctypes.c_size_t
        _PDT = ctypes.POINTER(SsdDtParams)
        lib.ssd_chunk_scan.argtypes = [_PD, _I32, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP, _PDT, _VP, _VP, _VP,
                                       _VP, ctypes.c_size_t, _VP]
        lib.ssd_conv_chunk_scan.argtypes = [_PD, _I32, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _PDT, _VP,
                                            _VP, _VP, _VP, ctypes.c_size_t, _VP]
        lib.ssd_chunk_scan_noalloc.argtypes = [_PD, _I32, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP, _PDT, _VP,
                                               _VP, _VP, _VP]
        lib.ssd_state_update.argtypes = [_PD, _VP, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP, _PDT, _VP, _VP]
        lib.ssd_conv1d_fwd_varlen.argtypes = [_PD, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _I64, _VP, _VP]
        lib.ssd_conv1d_update_slots.argtypes = [_PD, _VP, _I64, _VP, _VP, _VP, _VP, _I64, _VP, _VP]
        lib.ssd_chunk_scan_varlen.argtypes = [_PD, _I32, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP, _PDT, _VP,
                                              _VP, _VP, _VP, _I64, _VP, _VP, ctypes.c_size_t, _VP]
        lib.ssd_chunk_scan_varlen_snapshots.argtypes = [_PD, _I32, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP, _PDT,
                                                        _VP, _VP, _VP, _VP, _I64, _VP, _I64, _VP, _I32, _I64, _VP,
                                                        _VP, ctypes.c_size_t, _VP]
        lib.ssd_state_update_slots.argtypes = [_PD, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP,
                                               _PDT, _VP, _VP]
        lib.ssd_state_update_multi.argtypes = [_PD, _VP, _VP, _I64, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP,
                                               _PDT, _VP, _VP, _VP]
        lib.ssd_conv1d_update_multi.argtypes = [_PD, _VP, _I64, _VP, _VP, _VP, _VP, _I64, _VP, _VP, _VP]
        lib.ssd_accept_states.argtypes = [_PD, _VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP]
        lib.ssd_state_update_accept.argtypes = [_PD, _VP, _VP, _I64, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP,
                                                _PDT, _VP, _VP]
        lib.ssd_conv1d_update_accept.argtypes = [_PD, _VP, _I64, _VP, _VP, _I64, _VP, _VP]
        lib.ssd_decode_step.argtypes = [_PD, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _PDT, _VP, _VP]
        lib.ssd_gated_rmsnorm.argtypes = [_PD, _VP, _I64, _VP, _I64, _VP, ctypes.c_float, _VP, _VP]
        lib.ssd_chunk_scan_snapshots.argtypes = [_PD, _I32, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP, _PDT, _VP,
                                                 _VP, _VP, _I64, _VP, _VP, ctypes.c_size_t, _VP]
        lib.ssd_state_update_lp.argtypes = [_PD, _VP, _I32, _VP, _I64, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP,
                                            _PDT, ctypes.POINTER(SsdSrParams), _VP, _VP]
        _PSR = ctypes.POINTER(SsdSrParams)
        lib.ssd_chunk_scan_lp.argtypes = [_PD, _I32, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP, _PDT, _VP, _VP,
                                          _I32, _PSR, _VP, _VP, ctypes.c_size_t, _VP]
        lib.ssd_chunk_scan_varlen_lp.argtypes = [_PD, _I32, _VP, _I64, _VP, _VP, _I64, _VP, _VP, _VP, _PDT, _VP,
                                                 _VP, _VP, _VP, _I32, _I64, _PSR, _VP, _VP, ctypes.c_size_t, _VP]
        for f in ("ssd_conv1d_fwd", "ssd_conv1d_update", "ssd_chunk_scan", "ssd_state_update",
                  "ssd_conv1d_fwd_varlen", "ssd_conv1d_update_slots", "ssd_chunk_scan_varlen",
                  "ssd_state_update_slots", "ssd_state_update_multi", "ssd_conv1d_update_multi",
                  "ssd_accept_states", "ssd_state_update_lp", "ssd_chunk_scan_snapshots", "ssd_gated_rmsnorm",
                  "ssd_decode_step", "ssd_state_update_accept", "ssd_conv1d_update_accept",
                  "ssd_chunk_scan_varlen_snapshots", "ssd_chunk_scan_noalloc", "ssd_conv_chunk_scan",
                  "ssd_chunk_scan_lp", "ssd_chunk_scan_varlen_lp"):
            getattr(lib, f).restype = ctypes.c_int
        lib.ssd_status_string.argtypes = [ctypes.c_int]
        lib.ssd_status_string.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def lib_handle():
    """The loaded ctypes library (loads it on first call)."""
    return _lib()


def _ptr(t):
    return None if t is None else _VP(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return _VP(stream.cuda_stream)


def _uniform_rows(t, L):
    """[B, L, ...] view whose batch stride is L token strides (trivially true when empty)."""
    return t.shape[0] <= 1 or L == 0 or t.stride(0) == L * t.stride(1)


def _check(code, where):
    if code != 0:
        raise SsdError(code, where)


def _dt_params(dt_bias, dt_softplus, dt_limit):
    """ssd_dt_params_t for the optional dt prologue, or None (dt used as given).  dt_bias [H] fp32
    on the device; dt_limit (lo, hi) clamps after the softplus."""
    if dt_bias is None and not dt_softplus and dt_limit is None:
        return None
    if dt_bias is not None and (dt_bias.dtype != torch.float32 or not dt_bias.is_contiguous()):
        raise ValueError("dt_bias must be a contiguous fp32 [H] tensor")
    lo, hi = (0.0, 0.0) if dt_limit is None else (float(dt_limit[0]), float(dt_limit[1]))
    if dt_limit is not None and not lo < hi:
        raise ValueError("dt_limit needs lo < hi")
    return ctypes.byref(SsdDtParams(None if dt_bias is None else dt_bias.data_ptr(), int(bool(dt_softplus)),
                                    lo, hi))


def _dims(batch, seqlen, H, P, G, N, act, ydt):
    if act not in _DT or ydt not in _DT:
        raise ValueError(f"activation and y dtypes must be float32 or bfloat16 (got {act}, {ydt})")
    return SsdDims(batch, seqlen, H, P, G, N, 4, _DT[act], _DT[ydt])


# device types a call accepts (tensors must be GPU memory; the CPU tests of the argument checks widen it)
_DEVICE_TYPES = ("cuda",)


def _need(t, name, dev, shape=None, dtype=None, contiguous=True, optional=False):
    """Check one tensor argument before anything is launched: it lives on the call's GPU device,
    has the given dtype and shape, and is contiguous where the kernel assumes a dense layout.  The
    C ABI sees only pointers, so a wrong buffer would otherwise be read or written out of bounds."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.device != dev or t.device.type not in _DEVICE_TYPES:
        raise ValueError(f"{name} must be on {dev} (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _device(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type not in _DEVICE_TYPES:
        raise ValueError(f"{name} must be a tensor on a GPU device")
    return t.device


def _head_params(dev, H, A, D, name_a="A", name_d="D"):
    """A [H] fp32 (required) and D [H] fp32 (optional)."""
    _need(A, name_a, dev, (H,), torch.float32)
    _need(D, name_d, dev, (H,), torch.float32, optional=True)


def _conv_params(dev, CD, act, w, bias):
    """Conv taps w [CD, 4] and bias [CD] (optional) in the activation dtype."""
    _need(w, "w", dev, (CD, 4), act)
    _need(bias, "bias", dev, (CD,), act, optional=True)


def ssd_status_string(code):
    return _lib().ssd_status_string(code).decode()


def ssd_conv1d_fwd(xbc, w, bias=None, conv_state_in=None, conv_state_out=None, out=None,
                   nheads=None, head_dim=None, ngroups=None, d_state=None, stream=None):
    """Prefill conv.  xbc [B, L, CD] (token rows may be strided, channels packed),
    w [CD, 4], bias [CD]|None, conv states [B, CD, 4]|None (out may alias in).
    Returns out [B, L, CD].  The conv only needs CD; (H, P, G, N) may be given
    to describe the layer (CD = H*P + 2*G*N), otherwise any consistent split is used."""
    dev = _device(xbc, "xbc")
    Bt, L, CD = xbc.shape
    if (xbc.stride(2) != 1 and CD > 1) or not _uniform_rows(xbc, L):
        raise ValueError("xbc must be [B, L, CD] with packed channels and uniform token stride")
    H, P, G, N = _split_cd(CD, nheads, head_dim, ngroups, d_state)
    _conv_params(dev, CD, xbc.dtype, w, bias)
    _need(conv_state_in, "conv_state_in", dev, (Bt, CD, 4), xbc.dtype, optional=True)
    _need(conv_state_out, "conv_state_out", dev, (Bt, CD, 4), xbc.dtype, optional=True)
    if out is None:
        out = torch.empty((Bt, L, CD), dtype=xbc.dtype, device=xbc.device)
    _need(out, "out", dev, (Bt, L, CD), xbc.dtype)
    d = _dims(Bt, L, H, P, G, N, xbc.dtype, xbc.dtype)
    xs = CD if L == 0 else xbc.stride(1)
    if L == 0:
        xbc = None
    _check(_lib().ssd_conv1d_fwd(ctypes.byref(d), _ptr(xbc), xs, _ptr(w), _ptr(bias),
                                 _ptr(conv_state_in), _ptr(conv_state_out), _ptr(out), _stream(stream)),
           "ssd_conv1d_fwd")
    return out


def _split_cd(CD, H, P, G, N):
    if H is None:
        # any split with the right total channel count; the conv only uses CD
        G, N, P = 1, 8, 8
        H = (CD - 2 * G * N) // P
    if H * P + 2 * G * N != CD:
        raise ValueError(f"conv channels {CD} != H*P + 2*G*N")
    return H, P, G, N


def ssd_conv1d_update(xbc, w, bias, conv_state, out=None, nheads=None, head_dim=None, ngroups=None,
                      d_state=None, stream=None):
    """One-token conv.  xbc [B, CD] (rows may be strided), conv_state [B, CD, 4] updated in place.
    Returns out [B, CD]."""
    dev = _device(xbc, "xbc")
    Bt, CD = xbc.shape
    if xbc.stride(1) != 1:
        raise ValueError("xbc channels must be packed")
    H, P, G, N = _split_cd(CD, nheads, head_dim, ngroups, d_state)
    _conv_params(dev, CD, xbc.dtype, w, bias)
    _need(conv_state, "conv_state", dev, (Bt, CD, 4), xbc.dtype)
    if out is None:
        out = torch.empty((Bt, CD), dtype=xbc.dtype, device=xbc.device)
    _need(out, "out", dev, (Bt, CD), xbc.dtype)
    d = _dims(Bt, 1, H, P, G, N, xbc.dtype, xbc.dtype)
    _check(_lib().ssd_conv1d_update(ctypes.byref(d), _ptr(xbc), xbc.stride(0), _ptr(w), _ptr(bias),
                                    _ptr(conv_state), _ptr(out), _stream(stream)), "ssd_conv1d_update")
    return out


def ssd_chunk_scan_workspace_size(batch, seqlen, nheads, head_dim, ngroups, d_state, chunk=128,
                                  act_dtype=torch.bfloat16, y_dtype=torch.bfloat16):
    d = _dims(batch, seqlen, nheads, head_dim, ngroups, d_state, act_dtype, y_dtype)
    return int(_lib().ssd_chunk_scan_workspace_size(ctypes.byref(d), chunk))


def ssd_chunk_scan_varlen_workspace_size(nseq, rows, nheads, head_dim, ngroups, d_state, chunk=128,
                                         act_dtype=torch.bfloat16, y_dtype=torch.bfloat16):
    """Bytes of the fp16 packed scan's workspace for nseq sequences over rows packed token rows (0: none)."""
    d = _dims(nseq, rows, nheads, head_dim, ngroups, d_state, act_dtype, y_dtype)
    return int(_lib().ssd_chunk_scan_varlen_workspace_size(ctypes.byref(d), chunk))


def ssd_chunk_scan(x, B, C, dt, A, D=None, init_state=None, final_state=None, y=None, chunk=128,
                   y_dtype=None, workspace=None, stream=None, dt_bias=None, dt_softplus=False, dt_limit=None,
                   snapshots=None, snapshot_interval=None):
    """SSD chunked scan.  x [B, L, H, P], B/C [B, L, G, N] (token rows may be strided, e.g.
    views into the conv output), dt [B, L, H], A [H] fp32, D [H] fp32|None,
    init_state/final_state [B, H, P, N] fp32|None (may be the same tensor).  Optional dt prologue:
    dt <- clamp(softplus(dt + dt_bias), *dt_limit).  workspace: None allocates the one the fp16 scan needs
    (ssd_chunk_scan_workspace_size bytes; bf16 inputs with head_dim 64, d_state 128, chunk 128), a uint8
    tensor of at least that size is used as given, False runs without one (the bf16 split-operand
    kernel).  Returns y [B, L, H, P] in y_dtype (default x's)."""
    ydt = y_dtype or x.dtype
    if y is None:
        y = torch.empty(x.shape, dtype=ydt, device=x.device)
    dev, d, xs, bcs = _scan_args(x, B, C, dt, A, D, init_state, final_state, y, dt_bias)
    Bt, L, H, P = x.shape
    N = B.shape[3]
    if workspace is None and snapshot_interval is None:
        # the fp16 scan's workspace (pre-pass tiles of B and C), from torch's caching allocator
        n = int(_lib().ssd_chunk_scan_workspace_size(ctypes.byref(d), chunk))
        workspace = torch.empty(n, dtype=torch.uint8, device=dev) if n > 0 else None
    elif workspace is False:
        workspace = None         # no workspace: the bf16 split-operand kernel
    _need(workspace, "workspace", dev, optional=True)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if L == 0:
        x = B = C = dt = None
    if snapshot_interval is None:
        _check(_lib().ssd_chunk_scan(ctypes.byref(d), chunk, _ptr(x), xs, _ptr(B), _ptr(C), bcs,
                                     _ptr(dt), _ptr(A), _ptr(D), _dt_params(dt_bias, dt_softplus, dt_limit),
                                     _ptr(init_state), _ptr(final_state), _ptr(y),
                                     _ptr(workspace), ws, _stream(stream)), "ssd_chunk_scan")
        return y
    # state every snapshot_interval tokens into snapshots [B, L // interval, H, P, N] fp32
    if snapshot_interval <= 0:
        raise ValueError("snapshot_interval must be positive")
    if snapshots is None or snapshots.shape != (Bt, L // snapshot_interval, H, P, N) or \
            snapshots.dtype != torch.float32 or not snapshots.is_contiguous():
        raise ValueError("snapshots must be contiguous fp32 [B, L // snapshot_interval, H, P, N]")
    _need(snapshots, "snapshots", dev)
    _check(_lib().ssd_chunk_scan_snapshots(ctypes.byref(d), chunk, _ptr(x), xs, _ptr(B), _ptr(C), bcs,
                                           _ptr(dt), _ptr(A), _ptr(D), _dt_params(dt_bias, dt_softplus, dt_limit),
                                           _ptr(init_state), _ptr(final_state), _ptr(snapshots),
                                           int(snapshot_interval), _ptr(y), _ptr(workspace), ws, _stream(stream)),
           "ssd_chunk_scan_snapshots")
    return y


def ssd_conv_chunk_scan(xbc, w, bias, dt, A, D, nheads, head_dim, ngroups, d_state, conv_state_in=None,
                        conv_state_out=None, init_state=None, final_state=None, y=None, chunk=128, y_dtype=None,
                        workspace=None, stream=None, dt_bias=None, dt_softplus=False, dt_limit=None):
    """The prefill conv fused into the chunked scan: xbc [B, L, CD] (token rows may be strided, channels
    packed; CD = H*P + 2*G*N), taps w [CD, 4], bias [CD]|None, conv states [B, CD, 4]|None (out may alias
    in), dt [B, L, H], A/D [H], SSM states [B, H, P, N] fp32|None.  Equals ssd_conv1d_fwd followed by
    ssd_chunk_scan on the x, B, C views of its output, without materialising that output.  bf16, P 64,
    N 128, chunk 128.  workspace: None allocates one (ssd_chunk_scan_workspace_size bytes).  Returns y."""
    dev = _device(xbc, "xbc")
    Bt, L, CD = xbc.shape
    if (xbc.stride(2) != 1 and CD > 1) or not _uniform_rows(xbc, L):
        raise ValueError("xbc must be [B, L, CD] with packed channels and uniform token stride")
    H, P, G, N = _split_cd(CD, nheads, head_dim, ngroups, d_state)
    _conv_params(dev, CD, xbc.dtype, w, bias)
    _need(conv_state_in, "conv_state_in", dev, (Bt, CD, 4), xbc.dtype, optional=True)
    _need(conv_state_out, "conv_state_out", dev, (Bt, CD, 4), xbc.dtype, optional=True)
    _need(dt, "dt", dev, (Bt, L, H), xbc.dtype)
    _head_params(dev, H, A, D)
    _need(init_state, "init_state", dev, (Bt, H, P, N), torch.float32, optional=True)
    _need(final_state, "final_state", dev, (Bt, H, P, N), torch.float32, optional=True)
    _need(dt_bias, "dt_bias", dev, (H,), torch.float32, optional=True)
    if y is None:
        y = torch.empty((Bt, L, H, P), dtype=y_dtype or xbc.dtype, device=xbc.device)
    _need(y, "y", dev, (Bt, L, H, P))
    d = _dims(Bt, L, H, P, G, N, xbc.dtype, y.dtype)
    if workspace is None:
        n = int(_lib().ssd_chunk_scan_workspace_size(ctypes.byref(d), chunk))
        workspace = torch.empty(n, dtype=torch.uint8, device=dev) if n > 0 else None
    _need(workspace, "workspace", dev, optional=True)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    xs = CD if L == 0 else xbc.stride(1)
    if L == 0:
        xbc = dt = None
    _check(_lib().ssd_conv_chunk_scan(ctypes.byref(d), chunk, _ptr(xbc), xs, _ptr(w), _ptr(bias),
                                      _ptr(conv_state_in), _ptr(conv_state_out), _ptr(dt), _ptr(A), _ptr(D),
                                      _dt_params(dt_bias, dt_softplus, dt_limit), _ptr(init_state),
                                      _ptr(final_state), _ptr(y), _ptr(workspace), ws, _stream(stream)),
           "ssd_conv_chunk_scan")
    return y


def ssd_chunk_scan_noalloc(x, B, C, dt, A, D, init_state, final_state, y, chunk=128, stream=None, dt_bias=None,
                           dt_softplus=False, dt_limit=None):
    """ssd_chunk_scan that allocates nothing (for graph capture and serving loops): the caller passes y
    [B, L, H, P] (bf16 or fp32) and the states; the fp16 scan's workspace is the library's static
    per-device array (workspaces up to 64 MiB, else SSD_ERR_WORKSPACE).
    Calls that overlap on one device race on that array.  Returns y."""
    if y is None:
        raise ValueError("ssd_chunk_scan_noalloc needs y from the caller")
    dev, d, xs, bcs = _scan_args(x, B, C, dt, A, D, init_state, final_state, y, dt_bias)
    if x.shape[1] == 0:
        x = B = C = dt = None
    _check(_lib().ssd_chunk_scan_noalloc(ctypes.byref(d), chunk, _ptr(x), xs, _ptr(B), _ptr(C), bcs,
                                         _ptr(dt), _ptr(A), _ptr(D), _dt_params(dt_bias, dt_softplus, dt_limit),
                                         _ptr(init_state), _ptr(final_state), _ptr(y), _stream(stream)),
           "ssd_chunk_scan_noalloc")
    return y


def _scan_args(x, B, C, dt, A, D, init_state, final_state, y, dt_bias, state_dtype=torch.float32):
    """Checks the batched scan's tensors; returns (device, dims, x row stride, B/C row stride)."""
    dev = _device(x, "x")
    Bt, L, H, P = x.shape
    _need(B, "B", dev, dtype=x.dtype, contiguous=False)
    _need(C, "C", dev, dtype=x.dtype, contiguous=False)
    G, N = B.shape[2], B.shape[3]
    if L > 0 and (x.stride(3) != 1 or x.stride(2) != P or not _uniform_rows(x, L)):
        raise ValueError("x must be [B, L, H, P] with packed (H, P) and uniform token stride")
    for t, nm in ((B, "B"), (C, "C")):
        if t.shape != (Bt, L, G, N) or (L > 0 and (t.stride(3) != 1 or t.stride(2) != N
                                                    or not _uniform_rows(t, L))):
            raise ValueError(f"{nm} must be [B, L, G, N] with packed (G, N) and uniform token stride")
    if B.stride(1) != C.stride(1):
        raise ValueError("B and C must share a token stride")
    _need(dt, "dt", dev, (Bt, L, H), x.dtype)
    _head_params(dev, H, A, D)
    _need(init_state, "init_state", dev, (Bt, H, P, N), state_dtype, optional=True)
    _need(final_state, "final_state", dev, (Bt, H, P, N), state_dtype, optional=True)
    _need(dt_bias, "dt_bias", dev, (H,), torch.float32, optional=True)
    _need(y, "y", dev, (Bt, L, H, P))
    d = _dims(Bt, L, H, P, G, N, x.dtype, y.dtype)
    xs, bcs = (P * H, G * N) if L == 0 else (x.stride(1), B.stride(1))
    return dev, d, xs, bcs


def ssd_state_update(state, x, B, C, dt, A, D=None, y=None, y_dtype=None, stream=None, dt_bias=None,
                     dt_softplus=False, dt_limit=None):
    """One decode token, in place on state [B, H, P, N] fp32.  x [B, H, P], B/C [B, G, N]
    (batch rows may be strided, e.g. views into the conv-update output), dt [B, H].
    Returns y [B, H, P]."""
    dev = _device(x, "x")
    _need(state, "state", dev, dtype=torch.float32)
    if state.dim() != 4:
        raise ValueError("state must be [B, H, P, N]")
    Bt, H, P, N = state.shape
    _need(B, "B", dev, dtype=x.dtype, contiguous=False)
    _need(C, "C", dev, dtype=x.dtype, contiguous=False)
    G = B.shape[1]
    if x.shape != (Bt, H, P) or x.stride(2) != 1 or x.stride(1) != P:
        raise ValueError("x must be [B, H, P] with packed (H, P)")
    for t, nm in ((B, "B"), (C, "C")):
        if t.shape != (Bt, G, N) or t.stride(2) != 1 or t.stride(1) != N:
            raise ValueError(f"{nm} must be [B, G, N] with packed (G, N)")
    if B.stride(0) != C.stride(0):
        raise ValueError("B and C must share a batch stride")
    _need(dt, "dt", dev, (Bt, H), x.dtype)
    _head_params(dev, H, A, D)
    _need(dt_bias, "dt_bias", dev, (H,), torch.float32, optional=True)
    ydt = y_dtype or x.dtype
    if y is None:
        y = torch.empty((Bt, H, P), dtype=ydt, device=x.device)
    _need(y, "y", dev, (Bt, H, P))
    d = _dims(Bt, 1, H, P, G, N, x.dtype, y.dtype)
    _check(_lib().ssd_state_update(ctypes.byref(d), _ptr(state), _ptr(x), x.stride(0), _ptr(B), _ptr(C),
                                   B.stride(0), _ptr(dt), _ptr(A), _ptr(D),
                                   _dt_params(dt_bias, dt_softplus, dt_limit), _ptr(y), _stream(stream)),
           "ssd_state_update")
    return y


# --------------------------------------------------------------------------- packed batches
def _table(t, n, name):
    """An int32 sequence table on the device ([n], contiguous), or None."""
    if t is None:
        return None
    if t.dtype != torch.int32 or tuple(t.shape) != (n,) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor of shape [{n}]")
    return t


def ssd_conv1d_fwd_varlen(xbc, w, bias, cu_seqlens, conv_state_pool=None, slot_idx=None,
                          has_initial_state=None, out=None, nheads=None, head_dim=None, ngroups=None,
                          d_state=None, stream=None):
    """Prefill conv of a packed batch.  xbc [T, CD] (token rows may be strided, channels packed),
    cu_seqlens [S + 1] int32, slot_idx / has_initial_state [S] int32|None, conv_state_pool
    [nslots, CD, 4]|None, updated in place.  Returns out [T, CD]."""
    dev = _device(xbc, "xbc")
    T, CD = xbc.shape
    _need(cu_seqlens, "cu_seqlens", dev, dtype=torch.int32)
    S = cu_seqlens.numel() - 1
    if S < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if xbc.stride(1) != 1 and CD > 1:
        raise ValueError("xbc channels must be packed")
    H, P, G, N = _split_cd(CD, nheads, head_dim, ngroups, d_state)
    _conv_params(dev, CD, xbc.dtype, w, bias)
    _need(conv_state_pool, "conv_state_pool", dev, dtype=xbc.dtype, optional=True)
    _need(slot_idx, "slot_idx", dev, optional=True)
    _need(has_initial_state, "has_initial_state", dev, optional=True)
    nslots = 0
    if conv_state_pool is not None:
        if conv_state_pool.dim() != 3 or conv_state_pool.shape[1:] != (CD, 4) or not conv_state_pool.is_contiguous():
            raise ValueError("conv_state_pool must be contiguous [nslots, CD, 4]")
        nslots = conv_state_pool.shape[0]
    if out is None:
        out = torch.empty((T, CD), dtype=xbc.dtype, device=xbc.device)
    _need(out, "out", dev, (T, CD), xbc.dtype)
    d = _dims(S, T, H, P, G, N, xbc.dtype, xbc.dtype)
    xs = CD if T == 0 else xbc.stride(0)
    _check(_lib().ssd_conv1d_fwd_varlen(ctypes.byref(d), _ptr(xbc if T else None), xs, _ptr(w), _ptr(bias),
                                        _ptr(_table(cu_seqlens, S + 1, "cu_seqlens")),
                                        _ptr(_table(slot_idx, S, "slot_idx")),
                                        _ptr(_table(has_initial_state, S, "has_initial_state")),
                                        _ptr(conv_state_pool), nslots, _ptr(out), _stream(stream)),
           "ssd_conv1d_fwd_varlen")
    return out


def ssd_conv1d_update_slots(xbc, w, bias, conv_state_pool, slot_idx, out=None, nheads=None, head_dim=None,
                            ngroups=None, d_state=None, stream=None):
    """One-token conv for B requests whose windows live in conv_state_pool [nslots, CD, 4]
    (updated in place) at slot_idx [B] int32.  xbc [B, CD] (rows may be strided).  Returns out [B, CD]."""
    dev = _device(xbc, "xbc")
    Bt, CD = xbc.shape
    if xbc.stride(1) != 1:
        raise ValueError("xbc channels must be packed")
    _need(conv_state_pool, "conv_state_pool", dev, dtype=xbc.dtype)
    if conv_state_pool.dim() != 3 or conv_state_pool.shape[1:] != (CD, 4) or not conv_state_pool.is_contiguous():
        raise ValueError("conv_state_pool must be contiguous [nslots, CD, 4]")
    H, P, G, N = _split_cd(CD, nheads, head_dim, ngroups, d_state)
    _conv_params(dev, CD, xbc.dtype, w, bias)
    _need(slot_idx, "slot_idx", dev)
    if out is None:
        out = torch.empty((Bt, CD), dtype=xbc.dtype, device=xbc.device)
    _need(out, "out", dev, (Bt, CD), xbc.dtype)
    d = _dims(Bt, 1, H, P, G, N, xbc.dtype, xbc.dtype)
    _check(_lib().ssd_conv1d_update_slots(ctypes.byref(d), _ptr(xbc), xbc.stride(0), _ptr(w), _ptr(bias),
                                          _ptr(_table(slot_idx, Bt, "slot_idx")), _ptr(conv_state_pool),
                                          conv_state_pool.shape[0], _ptr(out), _stream(stream)),
           "ssd_conv1d_update_slots")
    return out


def _varlen_args(x, B, C, dt, A, D, cu_seqlens, state_pool, slot_idx, has_initial_state, y, y_dtype, workspace,
                 dt_bias, state_dtype):
    """Checks the packed scan's tensors; returns (device, dims, x row stride, B/C row stride, the
    three sequence tables, y, workspace bytes, nslots, S)."""
    dev = _device(x, "x")
    T, H, P = x.shape
    _need(B, "B", dev, dtype=x.dtype, contiguous=False)
    _need(C, "C", dev, dtype=x.dtype, contiguous=False)
    _need(cu_seqlens, "cu_seqlens", dev, dtype=torch.int32)
    G, N = B.shape[1], B.shape[2]
    S = cu_seqlens.numel() - 1
    if S < 0:
        raise ValueError("cu_seqlens needs at least one entry")
    if T > 0 and (x.stride(2) != 1 or x.stride(1) != P):
        raise ValueError("x must be [T, H, P] with packed (H, P)")
    for t, nm in ((B, "B"), (C, "C")):
        if t.shape != (T, G, N) or (T > 0 and (t.stride(2) != 1 or t.stride(1) != N)):
            raise ValueError(f"{nm} must be [T, G, N] with packed (G, N)")
    if B.stride(0) != C.stride(0):
        raise ValueError("B and C must share a token stride")
    _need(dt, "dt", dev, (T, H), x.dtype)
    _head_params(dev, H, A, D)
    _need(dt_bias, "dt_bias", dev, (H,), torch.float32, optional=True)
    _need(state_pool, "state_pool", dev, dtype=state_dtype, optional=True)
    _need(slot_idx, "slot_idx", dev, optional=True)
    _need(has_initial_state, "has_initial_state", dev, optional=True)
    nslots = 0
    if state_pool is not None:
        if state_pool.dim() != 4 or state_pool.shape[1:] != (H, P, N) or not state_pool.is_contiguous():
            raise ValueError("state_pool must be contiguous [nslots, H, P, N]")
        nslots = state_pool.shape[0]
    ydt = y_dtype or x.dtype
    if y is None:
        y = torch.empty((T, H, P), dtype=ydt, device=x.device)
    _need(y, "y", dev, (T, H, P))
    _need(workspace, "workspace", dev, optional=True)
    d = _dims(S, T, H, P, G, N, x.dtype, y.dtype)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    xs, bcs = (P * H, G * N) if T == 0 else (x.stride(0), B.stride(0))
    tabs = (_ptr(_table(cu_seqlens, S + 1, "cu_seqlens")), _ptr(_table(slot_idx, S, "slot_idx")),
            _ptr(_table(has_initial_state, S, "has_initial_state")))
    return dev, d, xs, bcs, tabs, y, ws, nslots, S


def ssd_chunk_scan_varlen(x, B, C, dt, A, D, cu_seqlens, state_pool=None, slot_idx=None,
                          has_initial_state=None, y=None, chunk=128, y_dtype=None, workspace=None, stream=None,
                          dt_bias=None, dt_softplus=False, dt_limit=None, snapshot_pool=None, snapshot_table=None,
                          snapshot_interval=None):
    """SSD chunked scan of a packed batch.  x [T, H, P], B/C [T, G, N] (token rows may be strided,
    e.g. views into the varlen conv output), dt [T, H], A [H] fp32, D [H] fp32|None,
    cu_seqlens [S + 1] int32, slot_idx / has_initial_state [S] int32|None, state_pool
    [nslots, H, P, N] fp32|None, updated in place.  With snapshot_table [S, max_snaps] int32 the
    state after every snapshot_interval tokens of sequence s goes to snapshot_pool
    [nsnap_slots, H, P, N] fp32 slot snapshot_table[s, k] (ssd_chunk_scan_varlen_snapshots).
    workspace: None allocates the one the fp16 scan needs where it applies (ssd_chunk_scan_varlen_workspace_size
    bytes; no snapshots), a uint8 tensor is used as given, False runs without one (the bf16 split-operand
    kernel).  Returns y [T, H, P] in y_dtype (default x's)."""
    allocate = workspace is None and snapshot_table is None
    if workspace is False:
        workspace = None
    dev, d, xs, bcs, tabs, y, ws, nslots, S = _varlen_args(x, B, C, dt, A, D, cu_seqlens, state_pool, slot_idx,
                                                           has_initial_state, y, y_dtype, workspace, dt_bias,
                                                           torch.float32)
    if allocate:
        n = int(_lib().ssd_chunk_scan_varlen_workspace_size(ctypes.byref(d), chunk))
        if n > 0:
            workspace = torch.empty(n, dtype=torch.uint8, device=dev)
            ws = n
    T, H, P = x.shape
    N = B.shape[2]
    if T == 0:
        x = B = C = dt = None
    if snapshot_table is None:
        _check(_lib().ssd_chunk_scan_varlen(ctypes.byref(d), chunk, _ptr(x), xs, _ptr(B), _ptr(C), bcs, _ptr(dt),
                                            _ptr(A), _ptr(D), _dt_params(dt_bias, dt_softplus, dt_limit), *tabs,
                                            _ptr(state_pool), nslots, _ptr(y), _ptr(workspace), ws, _stream(stream)),
               "ssd_chunk_scan_varlen")
        return y
    if snapshot_interval is None:
        raise ValueError("snapshot_table needs snapshot_interval")
    if (snapshot_table.dim() != 2 or snapshot_table.shape[0] != S or snapshot_table.dtype != torch.int32
            or not snapshot_table.is_contiguous() or snapshot_table.device != y.device):
        raise ValueError("snapshot_table must be contiguous int32 [S, max_snaps] on the scan's device")
    if snapshot_interval <= 0:
        raise ValueError("snapshot_interval must be positive")
    nsnap = 0
    _need(snapshot_pool, "snapshot_pool", dev, optional=True)
    if snapshot_pool is not None:
        if (snapshot_pool.dim() != 4 or snapshot_pool.shape[1:] != (H, P, N) or snapshot_pool.dtype != torch.float32
                or not snapshot_pool.is_contiguous()):
            raise ValueError("snapshot_pool must be contiguous fp32 [nsnap_slots, H, P, N]")
        nsnap = snapshot_pool.shape[0]
    _check(_lib().ssd_chunk_scan_varlen_snapshots(ctypes.byref(d), chunk, _ptr(x), xs, _ptr(B), _ptr(C), bcs,
                                                  _ptr(dt), _ptr(A), _ptr(D),
                                                  _dt_params(dt_bias, dt_softplus, dt_limit), *tabs,
                                                  _ptr(state_pool), nslots, _ptr(snapshot_pool), nsnap,
                                                  _ptr(snapshot_table), snapshot_table.shape[1], snapshot_interval,
                                                  _ptr(y), _ptr(workspace), ws, _stream(stream)),
           "ssd_chunk_scan_varlen_snapshots")
    return y


def ssd_state_update_slots(state_pool, slot_idx, x, B, C, dt, A, D=None, y=None, y_dtype=None, stream=None,
                           dt_bias=None, dt_softplus=False, dt_limit=None):
    """One decode token for B requests whose states live in state_pool [nslots, H, P, N] fp32
    (updated in place) at slot_idx [B] int32.  x [B, H, P], B/C [B, G, N], dt [B, H].
    Returns y [B, H, P]."""
    dev = _device(x, "x")
    _need(state_pool, "state_pool", dev, dtype=torch.float32)
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [nslots, H, P, N]")
    nslots, H, P, N = state_pool.shape
    Bt = x.shape[0]
    _need(B, "B", dev, dtype=x.dtype, contiguous=False)
    _need(C, "C", dev, dtype=x.dtype, contiguous=False)
    _need(slot_idx, "slot_idx", dev)
    G = B.shape[1]
    if x.shape != (Bt, H, P) or x.stride(2) != 1 or x.stride(1) != P:
        raise ValueError("x must be [B, H, P] with packed (H, P)")
    for t, nm in ((B, "B"), (C, "C")):
        if t.shape != (Bt, G, N) or t.stride(2) != 1 or t.stride(1) != N:
            raise ValueError(f"{nm} must be [B, G, N] with packed (G, N)")
    if B.stride(0) != C.stride(0):
        raise ValueError("B and C must share a batch stride")
    _need(dt, "dt", dev, (Bt, H), x.dtype)
    _head_params(dev, H, A, D)
    _need(dt_bias, "dt_bias", dev, (H,), torch.float32, optional=True)
    ydt = y_dtype or x.dtype
    if y is None:
        y = torch.empty((Bt, H, P), dtype=ydt, device=x.device)
    _need(y, "y", dev, (Bt, H, P))
    d = _dims(Bt, 1, H, P, G, N, x.dtype, y.dtype)
    _check(_lib().ssd_state_update_slots(ctypes.byref(d), _ptr(state_pool), nslots,
                                         _ptr(_table(slot_idx, Bt, "slot_idx")), _ptr(x), x.stride(0),
                                         _ptr(B), _ptr(C), B.stride(0), _ptr(dt), _ptr(A), _ptr(D),
                                         _dt_params(dt_bias, dt_softplus, dt_limit), _ptr(y), _stream(stream)),
           "ssd_state_update_slots")
    return y


# --------------------------------------------------------------------------- speculative decode
def _state_pool_args(state, slot_idx, Bt):
    """(pointer tensor, nslots, slot table) of a main state given per request or as a slot pool."""
    if slot_idx is None:
        if state.shape[0] != Bt:
            raise ValueError("without slot_idx the state needs one entry per request")
        return state, 0, None
    return state, state.shape[0], _table(slot_idx, Bt, "slot_idx")


def ssd_state_update_multi(state, x, B, C, dt, A, D=None, slot_idx=None, inter_states=True, y=None,
                           y_dtype=None, stream=None, dt_bias=None, dt_softplus=False, dt_limit=None):
    """k candidate tokens per request from state [B or nslots, H, P, N] fp32 (read only; with
    slot_idx [B] int32 it is a pool).  x [B, k, H, P], B/C [B, k, G, N] (token rows may be
    strided, e.g. views into the multi-token conv output), dt [B, k, H].  inter_states: True
    allocates [B, k, H, P, N] fp32, a tensor is written, None/False skips it.
    Returns (y [B, k, H, P], inter_states or None)."""
    dev = _device(x, "x")
    Bt, k, H, P = x.shape
    _need(state, "state", dev, dtype=torch.float32)
    _need(B, "B", dev, dtype=x.dtype, contiguous=False)
    _need(C, "C", dev, dtype=x.dtype, contiguous=False)
    N = state.shape[3]
    G = B.shape[2]
    if state.dim() != 4 or state.shape[1:] != (H, P, N) or not state.is_contiguous():
        raise ValueError("state must be contiguous [B or nslots, H, P, N]")
    if k > 0 and (x.stride(3) != 1 or x.stride(2) != P or not _uniform_rows(x, k)):
        raise ValueError("x must be [B, k, H, P] with packed (H, P) and uniform token stride")
    for t, nm in ((B, "B"), (C, "C")):
        if t.shape != (Bt, k, G, N) or (k > 0 and (t.stride(3) != 1 or t.stride(2) != N
                                                    or not _uniform_rows(t, k))):
            raise ValueError(f"{nm} must be [B, k, G, N] with packed (G, N) and uniform token stride")
    if B.stride(1) != C.stride(1):
        raise ValueError("B and C must share a token stride")
    _need(dt, "dt", dev, (Bt, k, H), x.dtype)
    _head_params(dev, H, A, D)
    _need(dt_bias, "dt_bias", dev, (H,), torch.float32, optional=True)
    _need(slot_idx, "slot_idx", dev, optional=True)
    st, nslots, tab = _state_pool_args(state, slot_idx, Bt)
    if inter_states is True:
        inter_states = torch.empty((Bt, k, H, P, N), dtype=torch.float32, device=x.device)
    elif inter_states is False:
        inter_states = None
    if inter_states is not None and (inter_states.shape != (Bt, k, H, P, N) or not inter_states.is_contiguous()
                                     or inter_states.dtype != torch.float32):
        raise ValueError("inter_states must be contiguous fp32 [B, k, H, P, N]")
    _need(inter_states, "inter_states", dev, optional=True)
    ydt = y_dtype or x.dtype
    if y is None:
        y = torch.empty((Bt, k, H, P), dtype=ydt, device=x.device)
    _need(y, "y", dev, (Bt, k, H, P))
    d = _dims(Bt, k, H, P, G, N, x.dtype, y.dtype)
    xs, bcs = (P * H, G * N) if k == 0 else (x.stride(1), B.stride(1))
    _check(_lib().ssd_state_update_multi(ctypes.byref(d), _ptr(st), _ptr(tab), nslots, _ptr(x), xs, _ptr(B),
                                         _ptr(C), bcs, _ptr(dt), _ptr(A), _ptr(D),
                                         _dt_params(dt_bias, dt_softplus, dt_limit), _ptr(inter_states), _ptr(y),
                                         _stream(stream)), "ssd_state_update_multi")
    return y, inter_states


def ssd_conv1d_update_multi(xbc, w, bias, conv_state, slot_idx=None, inter_conv_states=True, out=None,
                            nheads=None, head_dim=None, ngroups=None, d_state=None, stream=None):
    """k candidate tokens per request through the conv from conv_state [B or nslots, CD, 4]
    (read only).  xbc [B, k, CD] (token rows may be strided, uniform).  inter_conv_states: True
    allocates [B, k, CD, 4], a tensor is written, None/False skips it.
    Returns (out [B, k, CD], inter_conv_states or None)."""
    dev = _device(xbc, "xbc")
    Bt, k, CD = xbc.shape
    if k > 0 and (xbc.stride(2) != 1 or not _uniform_rows(xbc, k)):
        raise ValueError("xbc must be [B, k, CD] with packed channels and uniform token stride")
    _need(conv_state, "conv_state", dev, dtype=xbc.dtype)
    if conv_state.dim() != 3 or conv_state.shape[1:] != (CD, 4) or not conv_state.is_contiguous():
        raise ValueError("conv_state must be contiguous [B or nslots, CD, 4]")
    H, P, G, N = _split_cd(CD, nheads, head_dim, ngroups, d_state)
    _conv_params(dev, CD, xbc.dtype, w, bias)
    _need(slot_idx, "slot_idx", dev, optional=True)
    st, nslots, tab = _state_pool_args(conv_state, slot_idx, Bt)
    if inter_conv_states is True:
        inter_conv_states = torch.empty((Bt, k, CD, 4), dtype=xbc.dtype, device=xbc.device)
    elif inter_conv_states is False:
        inter_conv_states = None
    if inter_conv_states is not None and (inter_conv_states.shape != (Bt, k, CD, 4)
                                          or not inter_conv_states.is_contiguous()
                                          or inter_conv_states.dtype != xbc.dtype):
        raise ValueError("inter_conv_states must be contiguous [B, k, CD, 4] in xbc's dtype")
    _need(inter_conv_states, "inter_conv_states", dev, optional=True)
    if out is None:
        out = torch.empty((Bt, k, CD), dtype=xbc.dtype, device=xbc.device)
    _need(out, "out", dev, (Bt, k, CD), xbc.dtype)
    d = _dims(Bt, k, H, P, G, N, xbc.dtype, xbc.dtype)
    xs = CD if k == 0 else xbc.stride(1)
    _check(_lib().ssd_conv1d_update_multi(ctypes.byref(d), _ptr(xbc), xs, _ptr(w), _ptr(bias), _ptr(st),
                                          _ptr(tab), nslots, _ptr(inter_conv_states), _ptr(out),
                                          _stream(stream)), "ssd_conv1d_update_multi")
    return out, inter_conv_states


def ssd_accept_states(accept_len, state=None, inter_states=None, conv_state=None, inter_conv_states=None,
                      slot_idx=None, stream=None):
    """Write back the state after each request's last accepted token: accept_len [B] int32
    (clamped to [0, k]; 0 keeps the state).  state [B or nslots, H, P, N] fp32 with inter_states
    [B, k, H, P, N]; conv_state [B or nslots, CD, 4] with inter_conv_states [B, k, CD, 4]; either
    pair may be None.  Slots as for the multi-token calls."""
    if inter_states is None and inter_conv_states is None:
        raise ValueError("nothing to accept")
    ref = inter_states if inter_states is not None else inter_conv_states
    dev = _device(ref, "intermediate states")
    for t, nm in ((state, "state"), (inter_states, "inter_states"), (conv_state, "conv_state"),
                  (inter_conv_states, "inter_conv_states"), (slot_idx, "slot_idx")):
        _need(t, nm, dev, optional=True)
    _need(accept_len, "accept_len", dev)
    if inter_states is not None and inter_states.dtype != torch.float32:
        raise ValueError("SSM states are fp32")
    Bt, k = ref.shape[:2]
    # the call's dims: (H, P, N) from the SSM states, CD = H*P + 2*G*N from the conv states
    G, N, dtype = 1, 16, torch.float32
    if inter_states is not None:
        H, P, N = inter_states.shape[2:]
    if inter_conv_states is not None:
        CD, dtype = inter_conv_states.shape[2], inter_conv_states.dtype
        if inter_states is None:
            H, P, G, N = _split_cd(CD, None, None, None, None)
        else:
            G = (CD - H * P) // (2 * N)
            if G <= 0 or H * P + 2 * G * N != CD or H % G:
                raise ValueError("conv channels do not match the state's (H, P, N)")
    for main, inter, nm in ((state, inter_states, "state"), (conv_state, inter_conv_states, "conv_state")):
        if (main is None) != (inter is None):
            raise ValueError(f"{nm} and its intermediate states go together")
        if main is not None:
            if not main.is_contiguous() or not inter.is_contiguous() or main.shape[1:] != inter.shape[2:]:
                raise ValueError(f"{nm} [.., {tuple(inter.shape[2:])}] and its intermediates must be contiguous")
            if inter.shape[:2] != (Bt, k) or main.dtype != inter.dtype:
                raise ValueError(f"intermediate {nm}s must be [B, k, ...] in the state's dtype")
            if slot_idx is None and main.shape[0] != Bt:
                raise ValueError(f"without slot_idx {nm} needs one entry per request")
    nslots = 0
    if slot_idx is not None:
        nslots = (state if state is not None else conv_state).shape[0]
        if state is not None and conv_state is not None and conv_state.shape[0] != nslots:
            raise ValueError("state and conv_state pools must have the same number of slots")
    d = _dims(Bt, k, H, P, G, N, dtype, dtype)
    _check(_lib().ssd_accept_states(ctypes.byref(d), _ptr(_table(accept_len, Bt, "accept_len")),
                                    _ptr(_table(slot_idx, Bt, "slot_idx")), nslots, _ptr(state),
                                    _ptr(inter_states), _ptr(conv_state), _ptr(inter_conv_states),
                                    _stream(stream)), "ssd_accept_states")


# --------------------------------------------------------------------------- 16-bit state
SSD_F16 = 2
_STATE_DT = {torch.float16: SSD_F16, torch.bfloat16: SSD_BF16}


def ssd_state_update_lp(state, x, B, C, dt, A, D=None, slot_idx=None, sr=None, y=None, y_dtype=None, stream=None,
                        dt_bias=None, dt_softplus=False, dt_limit=None):
    """One decode token on a 16-bit state [B or nslots, H, P, N] (float16 or bfloat16, updated in
    place; with slot_idx [B] int32 it is a pool).  The update runs in fp32 and is rounded back to
    nearest even, or stochastically with sr = (seed, offset, rounds) (Philox4x32; use a new offset
    per call).  x [B, H, P], B/C [B, G, N] (16-byte aligned rows), dt [B, H].  Returns y [B, H, P]."""
    dev = _device(x, "x")
    _need(state, "state", dev)
    if state.dtype not in _STATE_DT or state.dim() != 4 or not state.is_contiguous():
        raise ValueError("state must be a contiguous float16 or bfloat16 [B or nslots, H, P, N] tensor")
    _, H, P, N = state.shape
    Bt = x.shape[0]
    _need(B, "B", dev, dtype=x.dtype, contiguous=False)
    _need(C, "C", dev, dtype=x.dtype, contiguous=False)
    G = B.shape[1]
    if x.shape != (Bt, H, P) or x.stride(2) != 1 or x.stride(1) != P:
        raise ValueError("x must be [B, H, P] with packed (H, P)")
    for t, nm in ((B, "B"), (C, "C")):
        if t.shape != (Bt, G, N) or t.stride(2) != 1 or t.stride(1) != N:
            raise ValueError(f"{nm} must be [B, G, N] with packed (G, N)")
    if B.stride(0) != C.stride(0):
        raise ValueError("B and C must share a batch stride")
    _need(dt, "dt", dev, (Bt, H), x.dtype)
    _head_params(dev, H, A, D)
    _need(dt_bias, "dt_bias", dev, (H,), torch.float32, optional=True)
    _need(slot_idx, "slot_idx", dev, optional=True)
    st, nslots, tab = _state_pool_args(state, slot_idx, Bt)
    ydt = y_dtype or x.dtype
    if y is None:
        y = torch.empty((Bt, H, P), dtype=ydt, device=x.device)
    _need(y, "y", dev, (Bt, H, P))
    d = _dims(Bt, 1, H, P, G, N, x.dtype, y.dtype)
    srp = None if sr is None else ctypes.byref(SsdSrParams(int(sr[0]), int(sr[1]), int(sr[2])))
    _check(_lib().ssd_state_update_lp(ctypes.byref(d), _ptr(st), _STATE_DT[state.dtype], _ptr(tab), nslots,
                                      _ptr(x), x.stride(0), _ptr(B), _ptr(C), B.stride(0), _ptr(dt), _ptr(A),
                                      _ptr(D), _dt_params(dt_bias, dt_softplus, dt_limit), srp, _ptr(y),
                                      _stream(stream)), "ssd_state_update_lp")
    return y


# --------------------------------------------------------------------------- one-launch decode step
def _sr_params(sr):
    return None if sr is None else ctypes.byref(SsdSrParams(int(sr[0]), int(sr[1]), int(sr[2])))


def _states16_dtype(*states):
    dts = {t.dtype for t in states if t is not None}
    if len(dts) > 1 or not dts <= set(_STATE_DT):
        raise ValueError("16-bit states must all be float16 or all bfloat16")
    return dts.pop() if dts else torch.float16


def ssd_chunk_scan_lp(x, B, C, dt, A, D=None, init_state=None, final_state=None, sr=None, y=None, chunk=128,
                      y_dtype=None, workspace=None, stream=None, dt_bias=None, dt_softplus=False, dt_limit=None):
    """ssd_chunk_scan with 16-bit states: init_state / final_state [B, H, P, N] float16 or bfloat16
    codes (one dtype; may be the same tensor), read exactly; the final state is rounded to nearest
    even, or stochastically with sr = (seed, offset, rounds) (Philox4x32, as ssd_state_update_lp).
    The other arguments as ssd_chunk_scan.  Returns y."""
    sdt = _states16_dtype(init_state, final_state)
    ydt = y_dtype or x.dtype
    if y is None:
        y = torch.empty(x.shape, dtype=ydt, device=x.device)
    dev, d, xs, bcs = _scan_args(x, B, C, dt, A, D, init_state, final_state, y, dt_bias, sdt)
    if workspace is None:
        n = int(_lib().ssd_chunk_scan_workspace_size(ctypes.byref(d), chunk))
        workspace = torch.empty(n, dtype=torch.uint8, device=dev) if n > 0 else None
    elif workspace is False:
        workspace = None
    _need(workspace, "workspace", dev, optional=True)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if x.shape[1] == 0:
        x = B = C = dt = None
    _check(_lib().ssd_chunk_scan_lp(ctypes.byref(d), chunk, _ptr(x), xs, _ptr(B), _ptr(C), bcs, _ptr(dt), _ptr(A),
                                    _ptr(D), _dt_params(dt_bias, dt_softplus, dt_limit), _ptr(init_state),
                                    _ptr(final_state), _STATE_DT[sdt], _sr_params(sr), _ptr(y), _ptr(workspace), ws,
                                    _stream(stream)), "ssd_chunk_scan_lp")
    return y


def ssd_chunk_scan_varlen_lp(x, B, C, dt, A, D, cu_seqlens, state_pool=None, slot_idx=None, has_initial_state=None,
                             sr=None, y=None, chunk=128, y_dtype=None, stream=None, dt_bias=None, dt_softplus=False,
                             dt_limit=None):
    """ssd_chunk_scan_varlen on a 16-bit state pool [nslots, H, P, N] (float16 or bfloat16 codes,
    updated in place): initial states read exactly, final states rounded as ssd_chunk_scan_lp.
    Returns y [T, H, P]."""
    sdt = _states16_dtype(state_pool)
    dev, d, xs, bcs, tabs, y, ws, nslots, S = _varlen_args(x, B, C, dt, A, D, cu_seqlens, state_pool, slot_idx,
                                                           has_initial_state, y, y_dtype, None, dt_bias, sdt)
    if x.shape[0] == 0:
        x = B = C = dt = None
    _check(_lib().ssd_chunk_scan_varlen_lp(ctypes.byref(d), chunk, _ptr(x), xs, _ptr(B), _ptr(C), bcs, _ptr(dt),
                                           _ptr(A), _ptr(D), _dt_params(dt_bias, dt_softplus, dt_limit), *tabs,
                                           _ptr(state_pool), _STATE_DT[sdt], nslots, _sr_params(sr), _ptr(y), None, 0,
                                           _stream(stream)), "ssd_chunk_scan_varlen_lp")
    return y


def ssd_decode_step(xbc, w, bias, conv_state_in, conv_state_out, state, dt, A, D=None, nheads=None, head_dim=None,
                    ngroups=None, y=None, y_dtype=None, stream=None, dt_bias=None, dt_softplus=False, dt_limit=None):
    """Conv update + state update in one launch.  xbc [B, CD] (rows may be strided); conv_state_in
    [B, CD, 4] is read, conv_state_out [B, CD, 4] (a different buffer) receives the rolled windows;
    state [B, H, P, N] fp32 is updated in place; dt [B, H].  Returns y [B, H, P]."""
    dev = _device(xbc, "xbc")
    _need(state, "state", dev, dtype=torch.float32)
    if state.dim() != 4:
        raise ValueError("state must be [B, H, P, N]")
    Bt, CD = xbc.shape
    _, H, P, N = state.shape
    G = ngroups if ngroups is not None else (CD - H * P) // (2 * N)
    if H * P + 2 * G * N != CD or (nheads is not None and nheads != H) or (head_dim is not None and head_dim != P):
        raise ValueError("xbc channels must be H*P + 2*G*N for the state's (H, P, N)")
    if xbc.stride(1) != 1:
        raise ValueError("xbc channels must be packed")
    for t, nm in ((conv_state_in, "conv_state_in"), (conv_state_out, "conv_state_out")):
        if t.shape != (Bt, CD, 4) or not t.is_contiguous() or t.dtype != xbc.dtype:
            raise ValueError(f"{nm} must be contiguous [B, CD, 4] in xbc's dtype")
    if state.shape[0] != Bt or not state.is_contiguous() or dt.shape != (Bt, H) or not dt.is_contiguous():
        raise ValueError("state [B, H, P, N] and dt [B, H] must be contiguous")
    _conv_params(dev, CD, xbc.dtype, w, bias)
    _need(conv_state_in, "conv_state_in", dev)
    _need(conv_state_out, "conv_state_out", dev)
    _need(dt, "dt", dev, (Bt, H), xbc.dtype)
    _head_params(dev, H, A, D)
    _need(dt_bias, "dt_bias", dev, (H,), torch.float32, optional=True)
    ydt = y_dtype or xbc.dtype
    if y is None:
        y = torch.empty((Bt, H, P), dtype=ydt, device=xbc.device)
    _need(y, "y", dev, (Bt, H, P))
    d = _dims(Bt, 1, H, P, G, N, xbc.dtype, y.dtype)
    _check(_lib().ssd_decode_step(ctypes.byref(d), _ptr(xbc), xbc.stride(0), _ptr(w), _ptr(bias), _ptr(conv_state_in),
                                  _ptr(conv_state_out), _ptr(state), _ptr(dt), _ptr(A), _ptr(D),
                                  _dt_params(dt_bias, dt_softplus, dt_limit), _ptr(y), _stream(stream)),
           "ssd_decode_step")
    return y


# --------------------------------------------------------------------------- gated norm
def ssd_gated_rmsnorm(y, z, weight, ngroups, eps=1e-5, out=None, stream=None):
    """out = rmsnorm over each of ngroups channel groups of y * silu(z), times weight (fp32
    arithmetic).  y [..., I] (e.g. the scan output viewed as [B, L, H*P]; rows may be strided),
    z [..., I] in the activation dtype (rows may be strided), weight [I] fp32.  Returns out
    [..., I] in z's dtype."""
    dev = _device(y, "y")
    _need(z, "z", dev, contiguous=False)
    _need(weight, "weight", dev)
    I = y.shape[-1]
    if z.shape != y.shape or y.stride(-1) != 1 or z.stride(-1) != 1 or y.dim() < 2:
        raise ValueError("y and z must have the same shape [..., I] with packed channels")
    y2 = y.reshape(-1, I) if y.dim() > 2 else y
    z2 = z.reshape(-1, I) if z.dim() > 2 else z
    if weight.shape != (I,) or weight.dtype != torch.float32 or not weight.is_contiguous():
        raise ValueError("weight must be contiguous fp32 [I]")
    if I % ngroups:
        raise ValueError("ngroups must divide the channel count")
    if out is None:
        out = torch.empty(y.shape, dtype=z.dtype, device=y.device)
    _need(out, "out", dev, y.shape, z.dtype)
    rows = y2.shape[0]
    d = _dims(rows, 1, ngroups, I // ngroups, ngroups, 16, z.dtype, y.dtype)   # one "head" per group
    _check(_lib().ssd_gated_rmsnorm(ctypes.byref(d), _ptr(y2), y2.stride(0) if rows else I, _ptr(z2),
                                    z2.stride(0) if rows else I, _ptr(weight), float(eps), _ptr(out),
                                    _stream(stream)), "ssd_gated_rmsnorm")
    return out


def ssd_state_update_accept(state, x, B, C, dt, A, D, accept_len, slot_idx=None, stream=None, dt_bias=None,
                            dt_softplus=False, dt_limit=None):
    """Accept step by recomputation: apply each request's first accept_len[b] (clamped to [0, k])
    candidate tokens to state [B or nslots, H, P, N] fp32 in place.  x, B, C, dt as given to
    ssd_state_update_multi ([B, k, ...])."""
    dev = _device(x, "x")
    Bt, k, H, P = x.shape
    _need(state, "state", dev, dtype=torch.float32)
    _need(B, "B", dev, dtype=x.dtype, contiguous=False)
    _need(C, "C", dev, dtype=x.dtype, contiguous=False)
    N = state.shape[3]
    G = B.shape[2]
    if state.dim() != 4 or state.shape[1:] != (H, P, N) or not state.is_contiguous():
        raise ValueError("state must be contiguous [B or nslots, H, P, N]")
    if k > 0 and (x.stride(3) != 1 or x.stride(2) != P or not _uniform_rows(x, k)):
        raise ValueError("x must be [B, k, H, P] with packed (H, P) and uniform token stride")
    for t, nm in ((B, "B"), (C, "C")):
        if t.shape != (Bt, k, G, N) or (k > 0 and (t.stride(3) != 1 or t.stride(2) != N
                                                    or not _uniform_rows(t, k))):
            raise ValueError(f"{nm} must be [B, k, G, N] with packed (G, N) and uniform token stride")
    if B.stride(1) != C.stride(1):
        raise ValueError("B and C must share a token stride")
    _need(dt, "dt", dev, (Bt, k, H), x.dtype)
    _head_params(dev, H, A, D)
    _need(dt_bias, "dt_bias", dev, (H,), torch.float32, optional=True)
    _need(accept_len, "accept_len", dev)
    _need(slot_idx, "slot_idx", dev, optional=True)
    st, nslots, tab = _state_pool_args(state, slot_idx, Bt)
    d = _dims(Bt, k, H, P, G, N, x.dtype, x.dtype)
    xs, bcs = (P * H, G * N) if k == 0 else (x.stride(1), B.stride(1))
    _check(_lib().ssd_state_update_accept(ctypes.byref(d), _ptr(st), _ptr(tab), nslots, _ptr(x), xs, _ptr(B), _ptr(C),
                                          bcs, _ptr(dt), _ptr(A), _ptr(D), _dt_params(dt_bias, dt_softplus, dt_limit),
                                          _ptr(_table(accept_len, Bt, "accept_len")), _stream(stream)),
           "ssd_state_update_accept")


def ssd_conv1d_update_accept(xbc, conv_state, accept_len, slot_idx=None, nheads=None, head_dim=None, ngroups=None,
                             d_state=None, stream=None):
    """Accept step by recomputation for the conv windows: request b's window in conv_state
    [B or nslots, CD, 4] becomes the last 4 of (its old window, rows 0 .. n-1 of xbc [B, k, CD]),
    n = accept_len[b] clamped to [0, k]."""
    dev = _device(xbc, "xbc")
    Bt, k, CD = xbc.shape
    if k > 0 and (xbc.stride(2) != 1 or not _uniform_rows(xbc, k)):
        raise ValueError("xbc must be [B, k, CD] with packed channels and uniform token stride")
    _need(conv_state, "conv_state", dev, dtype=xbc.dtype)
    if conv_state.dim() != 3 or conv_state.shape[1:] != (CD, 4) or not conv_state.is_contiguous():
        raise ValueError("conv_state must be contiguous [B or nslots, CD, 4]")
    H, P, G, N = _split_cd(CD, nheads, head_dim, ngroups, d_state)
    _need(accept_len, "accept_len", dev)
    _need(slot_idx, "slot_idx", dev, optional=True)
    st, nslots, tab = _state_pool_args(conv_state, slot_idx, Bt)
    d = _dims(Bt, k, H, P, G, N, xbc.dtype, xbc.dtype)
    _check(_lib().ssd_conv1d_update_accept(ctypes.byref(d), _ptr(xbc), CD if k == 0 else xbc.stride(1), _ptr(st),
                                           _ptr(tab), nslots, _ptr(_table(accept_len, Bt, "accept_len")),
                                           _stream(stream)), "ssd_conv1d_update_accept")


def split_xbc(v, nheads, head_dim, ngroups, d_state):
    """Views x [.., H, P], B [.., G, N], C [.., G, N] into a conv output v [.., CD] (no copy)."""
    I = nheads * head_dim
    GN = ngroups * d_state
    lead = v.shape[:-1]
    x = v[..., :I].unflatten(-1, (nheads, head_dim))
    Bm = v[..., I:I + GN].unflatten(-1, (ngroups, d_state))
    Cm = v[..., I + GN:I + 2 * GN].unflatten(-1, (ngroups, d_state))
    assert x.shape[:-2] == lead
    return x, Bm, Cm
