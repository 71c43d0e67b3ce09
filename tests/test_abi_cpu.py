"""The C ABI on the host: exports and argument validation (no GPU needed).

Every call below fails validation before anything is launched, so it never
reaches the device; pointers are fake 16-byte-aligned addresses that are
never dereferenced.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


@pytest.fixture(scope="module")
def ssd():
    from selective_state_space_conv1d_amd import ssd as mod
    if not os.path.exists(mod.LIB_PATH):
        from selective_state_space_conv1d_amd import build_lib
        build_lib.build()
    return mod


@pytest.fixture(scope="module")
def lib(ssd):
    return ssd.lib_handle()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree(ssd):
    assert declared_functions() == sorted(ssd.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def dims(ssd, **kw):
    d = dict(batch=2, seqlen=300, nheads=4, head_dim=64, ngroups=2, d_state=128, conv_width=4,
             act_dtype=1, y_dtype=0)
    d.update(kw)
    return ssd.SsdDims(**d)


P0 = 0x10000  # fake aligned device addresses (never dereferenced: every case fails validation)


def fp(i=0):
    return ctypes.c_void_p(P0 + 0x1000 * i)


def scan(lib, d, chunk=128, x=fp(1), xs=256, B=fp(2), C=fp(3), bcs=256, dt=fp(4), A=fp(5), D=None,
         init=None, fin=None, y=fp(6), ws=None, wsb=0):
    return lib.ssd_chunk_scan(ctypes.byref(d), chunk, x, xs, B, C, bcs, dt, A, D, None, init, fin, y, ws, wsb, None)


def test_status_strings(ssd, lib):
    for code in range(8):
        assert ssd.ssd_status_string(code)
    assert ssd.ssd_status_string(99) == "unknown status"


def test_conv_dim(ssd, lib):
    d = dims(ssd, nheads=256, head_dim=64, ngroups=8, d_state=128)
    assert lib.ssd_conv_dim(ctypes.byref(d)) == 18432
    assert lib.ssd_conv_dim(None) == -1


def test_scan_validation(ssd, lib):
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    assert lib.ssd_chunk_scan(None, 128, fp(1), 256, fp(2), fp(3), 256, fp(4), fp(5), None, None, None, None,
                              fp(6), None, 0, None) == E["SSD_ERR_NULL"]
    assert scan(lib, dims(ssd, act_dtype=7)) == E["SSD_ERR_DTYPE"]
    assert scan(lib, dims(ssd, y_dtype=-1)) == E["SSD_ERR_DTYPE"]
    assert scan(lib, dims(ssd, batch=-1)) == E["SSD_ERR_SHAPE"]
    assert scan(lib, dims(ssd, seqlen=-5)) == E["SSD_ERR_SHAPE"]
    assert scan(lib, dims(ssd, nheads=6, ngroups=4)) == E["SSD_ERR_SHAPE"]
    assert scan(lib, dims(ssd, nheads=0)) == E["SSD_ERR_SHAPE"]
    assert scan(lib, dims(ssd, conv_width=3)) == E["SSD_ERR_UNSUPPORTED"]
    assert scan(lib, dims(ssd), x=None) == E["SSD_ERR_NULL"]
    assert scan(lib, dims(ssd), dt=None) == E["SSD_ERR_NULL"]
    assert scan(lib, dims(ssd), A=None) == E["SSD_ERR_NULL"]
    assert scan(lib, dims(ssd), y=None) == E["SSD_ERR_NULL"]
    assert scan(lib, dims(ssd), chunk=96) == E["SSD_ERR_UNSUPPORTED"]
    assert scan(lib, dims(ssd, head_dim=48)) == E["SSD_ERR_UNSUPPORTED"]
    assert scan(lib, dims(ssd, d_state=256)) == E["SSD_ERR_UNSUPPORTED"]
    assert scan(lib, dims(ssd), xs=255) == E["SSD_ERR_SHAPE"]          # shorter than H*P
    assert scan(lib, dims(ssd), bcs=200) == E["SSD_ERR_SHAPE"]         # shorter than G*N
    assert scan(lib, dims(ssd), xs=260) == E["SSD_ERR_ALIGN"]          # 520 B rows
    assert scan(lib, dims(ssd), x=ctypes.c_void_p(P0 + 2)) == E["SSD_ERR_ALIGN"]
    assert scan(lib, dims(ssd), y=ctypes.c_void_p(P0 + 8)) == E["SSD_ERR_ALIGN"]
    assert scan(lib, dims(ssd), init=ctypes.c_void_p(P0 + 4)) == E["SSD_ERR_ALIGN"]


def test_workspace_size(ssd, lib):
    """The fp16 scan's workspace: per (batch, group, 128-token chunk) the fp16 B and C tiles (2 x 32 KiB),
    the ten causal 32 x 32 fp16 tiles of C.B^T (20 KiB) and two int32 scale exponents, and per (batch, head,
    chunk) the 128 fp32 dt values; no workspace for other sizes, dtypes or chunks."""
    ws = lib.ssd_chunk_scan_workspace_size
    assert ws(ctypes.byref(dims(ssd)), 128) == 2 * 2 * 3 * (65536 + 20480 + 8) + 2 * 4 * 3 * 512          # B 2, G 2, ceil(300/128) = 3
    assert ws(ctypes.byref(dims(ssd, seqlen=8192, batch=1, ngroups=8, nheads=256)), 128) == 8 * 64 * 86024 + 256 * 64 * 512
    assert ws(ctypes.byref(dims(ssd)), 64) == 0
    assert ws(ctypes.byref(dims(ssd, act_dtype=0)), 128) == 0
    assert ws(ctypes.byref(dims(ssd, head_dim=32)), 128) == 0
    assert ws(ctypes.byref(dims(ssd, seqlen=0)), 128) == 0
    assert ws(None, 128) == 0
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    # a workspace that is given must be large enough and aligned; NULL selects the split-operand kernel
    need = ws(ctypes.byref(dims(ssd)), 128)
    assert scan(lib, dims(ssd), ws=fp(7), wsb=need - 1, x=None) == E["SSD_ERR_NULL"]     # validation order
    assert scan(lib, dims(ssd), ws=fp(7), wsb=need - 1) == E["SSD_ERR_WORKSPACE"]
    assert scan(lib, dims(ssd), ws=ctypes.c_void_p(P0 + 8), wsb=need) == E["SSD_ERR_ALIGN"]


def test_varlen_workspace_size(ssd, lib):
    """The fp16 packed scan's workspace: S + ceil(T / 128) chunk slots per group (tiles and scales) and per head
    (dt rows), S = d->batch sequences over T = d->seqlen packed rows; none where the fp16 scan does not apply."""
    ws = lib.ssd_chunk_scan_varlen_workspace_size
    ws.argtypes = [ctypes.c_void_p, ctypes.c_int32]
    ws.restype = ctypes.c_size_t
    # 24 requests over 8192 rows, 256 heads, 8 groups: 24 + 64 = 88 slots
    assert ws(ctypes.byref(dims(ssd, batch=24, seqlen=8192, ngroups=8, nheads=256)), 128) == \
        8 * 88 * (65536 + 20480 + 8) + 256 * 88 * 512
    assert ws(ctypes.byref(dims(ssd, batch=3, seqlen=300)), 128) == 2 * 6 * 86024 + 4 * 6 * 512   # 3 + 3 slots
    assert ws(ctypes.byref(dims(ssd, batch=3, seqlen=300)), 256) == 0
    assert ws(ctypes.byref(dims(ssd, batch=3, seqlen=0)), 128) == 0
    assert ws(ctypes.byref(dims(ssd, batch=3, seqlen=300, d_state=64)), 128) == 0
    assert ws(None, 128) == 0


def test_conv_validation(ssd, lib):
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd)  # CD = 4*64 + 2*2*128 = 768
    ok = dict(xbc=fp(1), xs=768, w=fp(2), bias=None, sin=None, sout=None, out=fp(3))

    def call(dd=d, **kw):
        a = dict(ok)
        a.update(kw)
        return lib.ssd_conv1d_fwd(ctypes.byref(dd), a["xbc"], a["xs"], a["w"], a["bias"], a["sin"],
                                  a["sout"], a["out"], None)
    assert call(xbc=None) == E["SSD_ERR_NULL"]
    assert call(w=None) == E["SSD_ERR_NULL"]
    assert call(out=None) == E["SSD_ERR_NULL"]
    assert call(xs=700) == E["SSD_ERR_SHAPE"]
    assert call(xs=772) == E["SSD_ERR_ALIGN"]
    assert call(bias=ctypes.c_void_p(P0 + 6)) == E["SSD_ERR_ALIGN"]
    assert call(dims(ssd, conv_width=2)) == E["SSD_ERR_UNSUPPORTED"]
    assert call(dims(ssd, nheads=3, head_dim=1, ngroups=1, d_state=2)) == E["SSD_ERR_UNSUPPORTED"]  # CD=7
    assert lib.ssd_conv1d_update(ctypes.byref(d), fp(1), 768, fp(2), None, None, fp(3), None) == E["SSD_ERR_NULL"]
    assert lib.ssd_conv1d_update(ctypes.byref(d), fp(1), 767, fp(2), None, fp(4), fp(3), None) == E["SSD_ERR_SHAPE"]


def test_state_update_validation(ssd, lib):
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd)

    def call(dd=d, state=fp(1), x=fp(2), xs=256, B=fp(3), C=fp(4), bcs=256, dt=fp(5), A=fp(6), y=fp(7)):
        return lib.ssd_state_update(ctypes.byref(dd), state, x, xs, B, C, bcs, dt, A, None, None, y, None)
    assert call(state=None) == E["SSD_ERR_NULL"]
    assert call(y=None) == E["SSD_ERR_NULL"]
    assert call(dims(ssd, head_dim=24)) == E["SSD_ERR_UNSUPPORTED"]
    assert call(xs=100) == E["SSD_ERR_SHAPE"]
    assert call(state=ctypes.c_void_p(P0 + 4)) == E["SSD_ERR_ALIGN"]
    assert call(dims(ssd, nheads=5, ngroups=2)) == E["SSD_ERR_SHAPE"]


def test_varlen_and_slot_validation(ssd, lib):
    """The packed-batch and state-pool entry points reject bad host arguments before any launch."""
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd, batch=3, seqlen=300)   # 3 sequences, 300 packed rows; CD = 768

    def scan_v(dd=d, cu=fp(8), slot=None, hi=None, pool=fp(9), nslots=4, x=fp(1), y=fp(6), chunk=128):
        return lib.ssd_chunk_scan_varlen(ctypes.byref(dd), chunk, x, 256, fp(2), fp(3), 256, fp(4), fp(5), None,
                                         None, cu, slot, hi, pool, nslots, y, None, 0, None)
    assert scan_v(cu=None) == E["SSD_ERR_NULL"]
    assert scan_v(pool=None) == E["SSD_ERR_NULL"]                     # nslots > 0 needs a pool
    assert scan_v(nslots=-1) == E["SSD_ERR_SHAPE"]
    assert scan_v(pool=ctypes.c_void_p(P0 + 4)) == E["SSD_ERR_ALIGN"]
    assert scan_v(x=None) == E["SSD_ERR_NULL"]
    assert scan_v(chunk=32) == E["SSD_ERR_UNSUPPORTED"]
    assert scan_v(dims(ssd, batch=3, seqlen=300, d_state=24)) == E["SSD_ERR_UNSUPPORTED"]

    def conv_v(dd=d, cu=fp(8), pool=fp(9), nslots=4, xbc=fp(1), xs=768, w=fp(2), out=fp(3)):
        return lib.ssd_conv1d_fwd_varlen(ctypes.byref(dd), xbc, xs, w, None, cu, None, None, pool, nslots, out,
                                         None)
    assert conv_v(cu=None) == E["SSD_ERR_NULL"]
    assert conv_v(pool=None) == E["SSD_ERR_NULL"]
    assert conv_v(nslots=-2) == E["SSD_ERR_SHAPE"]
    assert conv_v(w=None) == E["SSD_ERR_NULL"]
    assert conv_v(xs=700) == E["SSD_ERR_SHAPE"]
    assert conv_v(xs=772) == E["SSD_ERR_ALIGN"]

    dd = dims(ssd, batch=2)
    assert lib.ssd_conv1d_update_slots(ctypes.byref(dd), fp(1), 768, fp(2), None, None, fp(3), 4, fp(4),
                                       None) == E["SSD_ERR_NULL"]        # slot_idx is required
    assert lib.ssd_conv1d_update_slots(ctypes.byref(dd), fp(1), 768, fp(2), None, fp(5), None, 4, fp(4),
                                       None) == E["SSD_ERR_NULL"]
    assert lib.ssd_conv1d_update_slots(ctypes.byref(dd), fp(1), 768, fp(2), None, fp(5), fp(3), -1, fp(4),
                                       None) == E["SSD_ERR_SHAPE"]

    def upd(pool=fp(1), nslots=4, slot=fp(8), y=fp(7)):
        return lib.ssd_state_update_slots(ctypes.byref(dd), pool, nslots, slot, fp(2), 256, fp(3), fp(4), 256,
                                          fp(5), fp(6), None, None, y, None)
    assert upd(slot=None) == E["SSD_ERR_NULL"]
    assert upd(pool=None) == E["SSD_ERR_NULL"]
    assert upd(nslots=-3) == E["SSD_ERR_SHAPE"]
    assert upd(pool=ctypes.c_void_p(P0 + 8)) == E["SSD_ERR_ALIGN"]
    assert upd(y=None) == E["SSD_ERR_NULL"]


def test_multi_token_and_accept_validation(ssd, lib):
    """The speculative-decode entry points reject bad host arguments before any launch."""
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd, batch=2, seqlen=3)   # 2 requests x 3 candidate tokens; CD = 768

    def upd(dd=d, state=fp(1), slot=None, nslots=0, x=fp(2), xs=256, inter=fp(9), y=fp(7)):
        return lib.ssd_state_update_multi(ctypes.byref(dd), state, slot, nslots, x, xs, fp(3), fp(4), 256, fp(5),
                                          fp(6), None, None, inter, y, None)
    assert upd(state=None) == E["SSD_ERR_NULL"]                   # no state without a slot table
    assert upd(state=None, slot=fp(8), nslots=2) == E["SSD_ERR_NULL"]
    assert upd(x=None) == E["SSD_ERR_NULL"]
    assert upd(y=None) == E["SSD_ERR_NULL"]
    assert upd(nslots=-1) == E["SSD_ERR_SHAPE"]
    assert upd(xs=100) == E["SSD_ERR_SHAPE"]
    assert upd(inter=ctypes.c_void_p(P0 + 4)) == E["SSD_ERR_ALIGN"]
    assert lib.ssd_state_update_multi(ctypes.byref(d), fp(1), None, 0, fp(2), 256, fp(3), fp(4), 260, fp(5), fp(6),
                                      None, None, None, fp(7), None) == E["SSD_ERR_ALIGN"]   # B/C row stride
    assert lib.ssd_state_update_multi(ctypes.byref(d), fp(1), None, 0, fp(2), 256, ctypes.c_void_p(P0 + 8), fp(4),
                                      256, fp(5), fp(6), None, None, None, fp(7), None) == E["SSD_ERR_ALIGN"]
    assert upd(dims(ssd, batch=2, seqlen=3, head_dim=24)) == E["SSD_ERR_UNSUPPORTED"]
    assert upd(dims(ssd, batch=2, seqlen=-1)) == E["SSD_ERR_SHAPE"]

    def conv(dd=d, xbc=fp(1), xs=768, state=fp(2), slot=None, nslots=0, inter=fp(3), out=fp(4)):
        return lib.ssd_conv1d_update_multi(ctypes.byref(dd), xbc, xs, fp(5), None, state, slot, nslots, inter, out,
                                           None)
    assert conv(state=None) == E["SSD_ERR_NULL"]
    assert conv(out=None) == E["SSD_ERR_NULL"]
    assert conv(xs=700) == E["SSD_ERR_SHAPE"]
    assert conv(xs=772) == E["SSD_ERR_ALIGN"]
    assert conv(inter=ctypes.c_void_p(P0 + 8)) == E["SSD_ERR_ALIGN"]
    assert conv(nslots=-5) == E["SSD_ERR_SHAPE"]

    def acc(dd=d, alen=fp(1), slot=None, nslots=0, st=fp(2), ist=fp(3), cs=fp(4), ics=fp(5)):
        return lib.ssd_accept_states(ctypes.byref(dd), alen, slot, nslots, st, ist, cs, ics, None)
    assert acc(alen=None) == E["SSD_ERR_NULL"]
    assert acc(ist=None) == E["SSD_ERR_NULL"]                     # a pair is both or neither
    assert acc(cs=None) == E["SSD_ERR_NULL"]
    assert acc(st=ctypes.c_void_p(P0 + 4)) == E["SSD_ERR_ALIGN"]
    assert acc(nslots=-1) == E["SSD_ERR_SHAPE"]
    assert acc(dims(ssd, batch=70000, seqlen=3)) == E["SSD_ERR_UNSUPPORTED"]
    # nothing to do: no states, no tokens, or an empty pool -- no launch, no table read
    assert acc(st=None, ist=None, cs=None, ics=None, alen=None) == E["SSD_OK"]
    assert acc(dims(ssd, batch=2, seqlen=0), alen=None) == E["SSD_OK"]
    assert acc(slot=fp(8), nslots=0, alen=None) == E["SSD_OK"]


def test_lowprec_state_validation(ssd, lib):
    """The 16-bit state update rejects bad host arguments before any launch."""
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd, batch=2, seqlen=1)

    def upd(dd=d, state=fp(1), sdt=2, slot=None, nslots=0, B=fp(3), bcs=256, sr=None, y=fp(7)):
        return lib.ssd_state_update_lp(ctypes.byref(dd), state, sdt, slot, nslots, fp(2), 256, B, fp(4), bcs, fp(5),
                                       fp(6), None, None, sr, y, None)
    assert upd(sdt=0) == E["SSD_ERR_DTYPE"]                 # fp32 is not a 16-bit state
    assert upd(sdt=7) == E["SSD_ERR_DTYPE"]
    assert upd(state=None) == E["SSD_ERR_NULL"]
    assert upd(y=None) == E["SSD_ERR_NULL"]
    assert upd(nslots=-1) == E["SSD_ERR_SHAPE"]
    assert upd(state=ctypes.c_void_p(P0 + 2)) == E["SSD_ERR_ALIGN"]
    assert upd(B=ctypes.c_void_p(P0 + 8)) == E["SSD_ERR_ALIGN"]
    assert upd(bcs=260) == E["SSD_ERR_ALIGN"]
    assert upd(sr=ctypes.byref(ssd.SsdSrParams(1, 2, 0))) == E["SSD_ERR_UNSUPPORTED"]
    assert upd(sr=ctypes.byref(ssd.SsdSrParams(1, 2, 17))) == E["SSD_ERR_UNSUPPORTED"]
    assert upd(dims(ssd, batch=2, seqlen=1, d_state=24)) == E["SSD_ERR_UNSUPPORTED"]


def test_scan_lp_validation(ssd, lib):
    """The scans on 16-bit states reject a bad state dtype, bad rounding parameters and misaligned
    code arrays before any launch; the scans' own checks still apply."""
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd, batch=2, seqlen=300)

    def sc(dd=d, init=fp(8), fin=fp(9), sdt=1, sr=None, x=fp(1)):
        return lib.ssd_chunk_scan_lp(ctypes.byref(dd), 128, x, 256, fp(2), fp(3), 256, fp(4), fp(5), None, None,
                                     init, fin, sdt, sr, fp(6), None, 0, None)
    assert sc(sdt=0) == E["SSD_ERR_DTYPE"]                  # fp32 is not a 16-bit state
    assert sc(sdt=5) == E["SSD_ERR_DTYPE"]
    assert sc(sr=ctypes.byref(ssd.SsdSrParams(1, 2, 0))) == E["SSD_ERR_UNSUPPORTED"]
    assert sc(sr=ctypes.byref(ssd.SsdSrParams(1, 2, 17))) == E["SSD_ERR_UNSUPPORTED"]
    assert sc(init=ctypes.c_void_p(P0 + 8)) == E["SSD_ERR_ALIGN"]
    assert sc(fin=ctypes.c_void_p(P0 + 2)) == E["SSD_ERR_ALIGN"]
    assert sc(x=None) == E["SSD_ERR_NULL"]
    assert sc(dims(ssd, batch=2, seqlen=300, head_dim=48)) == E["SSD_ERR_UNSUPPORTED"]
    d3 = dims(ssd, batch=3, seqlen=300)

    def vl(dd=d3, pool=fp(9), nslots=4, sdt=2, sr=None, cu=fp(11)):
        return lib.ssd_chunk_scan_varlen_lp(ctypes.byref(dd), 128, fp(1), 256, fp(2), fp(3), 256, fp(4), fp(5), None,
                                            None, cu, None, None, pool, sdt, nslots, sr, fp(6), None, 0, None)
    assert vl(sdt=3) == E["SSD_ERR_DTYPE"]
    assert vl(sr=ctypes.byref(ssd.SsdSrParams(1, 2, 0))) == E["SSD_ERR_UNSUPPORTED"]
    assert vl(pool=ctypes.c_void_p(P0 + 4)) == E["SSD_ERR_ALIGN"]
    assert vl(pool=None) == E["SSD_ERR_NULL"]
    assert vl(cu=None) == E["SSD_ERR_NULL"]
    assert vl(nslots=-1) == E["SSD_ERR_SHAPE"]


def test_snapshot_scan_validation(ssd, lib):
    """The snapshot form of the scan rejects a bad interval or a missing buffer before any launch."""
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd, batch=2, seqlen=300)

    def snap(dd=d, buf=fp(9), iv=128, x=fp(1)):
        return lib.ssd_chunk_scan_snapshots(ctypes.byref(dd), 128, x, 256, fp(2), fp(3), 256, fp(4), fp(5), None,
                                            None, None, None, buf, iv, fp(6), None, 0, None)
    assert snap(iv=0) == E["SSD_ERR_UNSUPPORTED"]
    assert snap(iv=100) == E["SSD_ERR_UNSUPPORTED"]
    assert snap(buf=None) == E["SSD_ERR_NULL"]
    assert snap(buf=ctypes.c_void_p(P0 + 4)) == E["SSD_ERR_ALIGN"]
    assert snap(x=None) == E["SSD_ERR_NULL"]                    # the scan's own checks still apply
    assert lib.ssd_chunk_scan_snapshots(None, 128, fp(1), 256, fp(2), fp(3), 256, fp(4), fp(5), None, None, None,
                                        None, fp(9), 128, fp(6), None, 0, None) == E["SSD_ERR_NULL"]


def test_scan_varlen_snapshots_validation(ssd, lib):
    """The packed scan with snapshots rejects a bad interval, a missing pool or table, negative
    sizes and a misaligned pool before any launch; the packed scan's own checks still apply."""
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd, batch=3, seqlen=300)

    def snap(dd=d, pool=fp(9), nsnap=4, table=fp(10), maxs=2, iv=128, x=fp(1), cu=fp(11)):
        return lib.ssd_chunk_scan_varlen_snapshots(ctypes.byref(dd), 128, x, 256, fp(2), fp(3), 256, fp(4), fp(5),
                                                   None, None, cu, None, None, None, 0, pool, nsnap, table, maxs, iv,
                                                   fp(6), None, 0, None)
    assert snap(iv=0) == E["SSD_ERR_UNSUPPORTED"]
    assert snap(iv=192) == E["SSD_ERR_UNSUPPORTED"]
    assert snap(pool=None) == E["SSD_ERR_NULL"]
    assert snap(table=None) == E["SSD_ERR_NULL"]
    assert snap(nsnap=-1) == E["SSD_ERR_SHAPE"]
    assert snap(maxs=-1) == E["SSD_ERR_SHAPE"]
    assert snap(pool=ctypes.c_void_p(P0 + 8)) == E["SSD_ERR_ALIGN"]
    assert snap(cu=None) == E["SSD_ERR_NULL"]                   # the packed scan's own checks still apply
    assert snap(x=None) == E["SSD_ERR_NULL"]
    assert lib.ssd_chunk_scan_varlen_snapshots(None, 128, fp(1), 256, fp(2), fp(3), 256, fp(4), fp(5), None, None,
                                               fp(11), None, None, None, 0, fp(9), 4, fp(10), 2, 128, fp(6), None, 0,
                                               None) == E["SSD_ERR_NULL"]


def test_gated_rmsnorm_validation(ssd, lib):
    """The gated norm rejects bad host arguments before any launch."""
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd, batch=4, seqlen=2)     # 8 rows, I = 256 channels in 2 groups of 128

    def nrm(dd=d, y=fp(1), ys=256, z=fp(2), zs=256, w=fp(3), eps=1e-5, out=fp(4)):
        return lib.ssd_gated_rmsnorm(ctypes.byref(dd), y, ys, z, zs, w, eps, out, None)
    assert nrm(y=None) == E["SSD_ERR_NULL"]
    assert nrm(w=None) == E["SSD_ERR_NULL"]
    assert nrm(ys=200) == E["SSD_ERR_SHAPE"]
    assert nrm(zs=260) == E["SSD_ERR_ALIGN"]
    assert nrm(eps=-1.0) == E["SSD_ERR_SHAPE"]
    assert nrm(out=ctypes.c_void_p(P0 + 2)) == E["SSD_ERR_ALIGN"]
    assert nrm(dims(ssd, batch=4, seqlen=2, nheads=4, head_dim=20, ngroups=4)) == E["SSD_ERR_UNSUPPORTED"]   # group of 20
    assert nrm(dims(ssd, batch=0, seqlen=2), y=None, z=None, w=None, out=None) == E["SSD_OK"]


def test_decode_step_validation(ssd, lib):
    """The one-launch decode step rejects bad host arguments, and overlapping conv windows, before any launch."""
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd, batch=2, seqlen=1)     # CD = 768: conv windows of 2 * 768 * 4 bf16 = 12 KiB

    def step(dd=d, xs=768, cin=fp(3), cout=fp(8), state=fp(5), y=fp(7)):
        return lib.ssd_decode_step(ctypes.byref(dd), fp(1), xs, fp(2), None, cin, cout, state, fp(4), fp(6), None,
                                   None, y, None)
    assert step(cin=None) == E["SSD_ERR_NULL"]
    assert step(state=None) == E["SSD_ERR_NULL"]
    assert step(y=None) == E["SSD_ERR_NULL"]
    assert step(xs=700) == E["SSD_ERR_SHAPE"]
    assert step(cout=fp(3)) == E["SSD_ERR_SHAPE"]                           # same buffer
    assert step(cout=ctypes.c_void_p(P0 + 0x3000 + 4096)) == E["SSD_ERR_SHAPE"]  # overlapping
    assert step(state=ctypes.c_void_p(P0 + 8)) == E["SSD_ERR_ALIGN"]
    assert step(dims(ssd, batch=2, seqlen=1, d_state=24)) == E["SSD_ERR_UNSUPPORTED"]


def test_accept_by_recomputation_validation(ssd, lib):
    """The recomputing accept calls reject bad host arguments before any launch, and launch nothing
    when there is nothing to apply."""
    E = {n: i for i, n in enumerate(ssd.STATUS)}
    d = dims(ssd, batch=2, seqlen=3)

    def sacc(dd=d, state=fp(1), slot=None, nslots=0, alen=fp(9), B=fp(3), bcs=256):
        return lib.ssd_state_update_accept(ctypes.byref(dd), state, slot, nslots, fp(2), 256, B, fp(4), bcs, fp(5),
                                           fp(6), None, None, alen, None)
    assert sacc(alen=None) == E["SSD_ERR_NULL"]
    assert sacc(state=None) == E["SSD_ERR_NULL"]
    assert sacc(nslots=-1) == E["SSD_ERR_SHAPE"]
    assert sacc(B=ctypes.c_void_p(P0 + 8)) == E["SSD_ERR_ALIGN"]
    assert sacc(bcs=260) == E["SSD_ERR_ALIGN"]
    assert sacc(dims(ssd, batch=2, seqlen=0), alen=None, state=None) == E["SSD_OK"]
    assert sacc(slot=fp(8), nslots=0, alen=None, state=None) == E["SSD_OK"]

    def cacc(dd=d, xbc=fp(1), xs=768, cs=fp(2), alen=fp(9)):
        return lib.ssd_conv1d_update_accept(ctypes.byref(dd), xbc, xs, cs, None, 0, alen, None)
    assert cacc(alen=None) == E["SSD_ERR_NULL"]
    assert cacc(cs=None) == E["SSD_ERR_NULL"]
    assert cacc(xs=700) == E["SSD_ERR_SHAPE"]
    assert cacc(xs=772) == E["SSD_ERR_ALIGN"]
    assert cacc(dims(ssd, batch=0, seqlen=3), xbc=None, cs=None, alen=None) == E["SSD_OK"]


def test_binding_raises_without_library(ssd, monkeypatch):
    monkeypatch.setattr(ssd, "_LIB", None)
    monkeypatch.setattr(ssd, "LIB_PATH", "/nonexistent/libssd.so")
    with pytest.raises(RuntimeError, match="not built"):
        ssd.lib_handle()
