"""Reduced-precision SSM state storage: the Philox generator and the rounding of fp32 state
values to fp16 or bf16 codes.

TEST INFRASTRUCTURE ONLY (imported by ``oracle.oracle`` for the tests).

Source of the method: the modeling_nemotron_h.py walk-through page, 部署时如何调这些缓存
(inference-engine settings: an fp16 Mamba state cache with stochastic rounding driven by a
Philox generator of 5 rounds), and "MAX 平台 Nemotron-H 混合架构解析", 5.4 (the state pool
stored in a narrower type while the scan accumulates in fp32).  The pages name the generator and its round
count only; the generator is Philox4x32-R as published by Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3" (SC 2011), and the rest is this reading:

* element e of the state array (its flat index in the pool when a slot table is used) draws the
  16-bit number r16(e): half (e mod 2) -- low half first -- of word (e mod 8) div 2 of
  Philox4x32-R(counter = (o mod 2^32, o div 2^32, offset mod 2^32, offset div 2^32),
  key = (seed mod 2^32, seed div 2^32)) with o = e div 8;
* an fp32 value v is stored as lo, the format's value next to v toward zero (v itself when
  representable), or as the next code away from zero, which it takes iff
  r16 < 65536 * (|v| - |lo|) / spacing, spacing being the distance from lo to that next code
  (for the largest finite value, the distance continued from its binade);
* fp16 values of magnitude 65536 or more become infinities, and NaN or infinite v are converted
  with round-to-nearest-even, which is also the rounding used without a generator.
"""
import numpy as np

# Philox constants as published (multipliers; Weyl key increments, golden ratio and sqrt(3) - 1)
PHILOX4x32_M = (0xD2511F53, 0xCD9E8D57)
PHILOX4x32_W = (0x9E3779B9, 0xBB67AE85)
PHILOX4x64_M = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
PHILOX4x64_W = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def philox4(ctr, key, rounds, w=32, M=PHILOX4x32_M, W=PHILOX4x32_W):
    """Philox4xW-R of one counter (4 words) under one key (2 words), as Python ints.  Each round
    multiplies counter words 0 and 2 by the two multipliers and mixes the high halves of the
    products with words 1 and 3 and the key; the key is advanced by the Weyl increments before
    every round after the first."""
    mask = (1 << w) - 1
    c0, c1, c2, c3 = (int(v) & mask for v in ctr)
    k0, k1 = (int(v) & mask for v in key)
    for r in range(rounds):
        if r:
            k0, k1 = (k0 + W[0]) & mask, (k1 + W[1]) & mask
        p0, p1 = M[0] * c0, M[1] * c2
        hi0, lo0, hi1, lo1 = p0 >> w, p0 & mask, p1 >> w, p1 & mask
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def philox4x32(c0, c1, c2, c3, key, rounds):
    """philox4 with w = 32 over uint32 numpy arrays of counter words (the same steps, vectorised)."""
    m32 = np.uint64(0xFFFFFFFF)
    c = [np.asarray(v, dtype=np.uint64) & m32 for v in (c0, c1, c2, c3)]
    k0, k1 = np.uint64(int(key[0]) & 0xFFFFFFFF), np.uint64(int(key[1]) & 0xFFFFFFFF)
    for r in range(rounds):
        if r:
            k0 = (k0 + np.uint64(PHILOX4x32_W[0])) & m32
            k1 = (k1 + np.uint64(PHILOX4x32_W[1])) & m32
        p0 = np.uint64(PHILOX4x32_M[0]) * c[0]
        p1 = np.uint64(PHILOX4x32_M[1]) * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ k0, p1 & m32, (p0 >> np.uint64(32)) ^ c[3] ^ k1, p0 & m32]
    return [v.astype(np.uint32) for v in c]


def random16(e, seed, offset, rounds):
    """r16 of state elements e (int64 array of flat indices)."""
    e = np.asarray(e, dtype=np.int64)
    o = (e // 8).astype(np.uint64)
    words = philox4x32(o & np.uint64(0xFFFFFFFF), o >> np.uint64(32),
                       np.full(o.shape, offset & 0xFFFFFFFF, np.uint64), np.full(o.shape, offset >> 32, np.uint64),
                       (seed & 0xFFFFFFFF, seed >> 32), rounds)
    sel = (e % 8) // 2
    w = np.choose(sel, words)
    return ((w >> (16 * (e % 2)).astype(np.uint32)) & np.uint32(0xFFFF)).astype(np.uint32)


# ----------------------------------------------------------------------------- formats
def _bf16_value(code):
    """float64 values of bf16 codes (uint16 arrays)."""
    return (np.asarray(code, np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode(codes, fmt):
    codes = np.asarray(codes, dtype=np.uint16)
    if fmt == "f16":
        return codes.view(np.float16).astype(np.float64)
    return _bf16_value(codes)


def _rne(v32, fmt):
    if fmt == "f16":
        with np.errstate(over="ignore"):
            return v32.astype(np.float16).view(np.uint16)
    import torch
    return torch.from_numpy(np.ascontiguousarray(v32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def round_state(v32, fmt, r16=None):
    """fp32 values -> uint16 codes of fmt ('f16' or 'bf16'): round to nearest even without r16,
    else the stochastic rounding of the module docstring."""
    v32 = np.ascontiguousarray(v32, dtype=np.float32)
    if r16 is None:
        return _rne(v32, fmt)
    r16 = np.asarray(r16, dtype=np.float64)
    av = np.abs(v32.astype(np.float64))
    neg = np.signbit(v32)
    finite = np.isfinite(v32)
    out = _rne(v32, fmt).copy()
    if fmt == "f16":
        with np.errstate(over="ignore"):
            return _round_f16(v32, av, neg, finite, r16, out)
    lo_code = (np.abs(v32).view(np.uint32) >> np.uint32(16))     # truncation = toward zero
    lov = _bf16_value(lo_code)
    with np.errstate(over="ignore"):
        nxt = _bf16_value(lo_code + 1)
    spacing = np.where(np.isinf(nxt), 2.0 ** 120, nxt - lov)       # past the largest finite: its binade's
    frac = (av - lov) / spacing                                      # exact: power-of-two spacing
    code = lo_code + (r16 < frac * 65536.0).astype(np.uint32)
    code = (code | np.where(neg, 0x8000, 0)).astype(np.uint16)
    return np.where(finite, code, out).astype(np.uint16)


def _round_f16(v32, av, neg, finite, r16, out):
    big = finite & (av >= 65536.0)
    c = np.minimum(av, 65504.0).astype(np.float16)                   # RNE of |v| (<= max finite)
    lo = np.where(c.astype(np.float64) > av, np.nextafter(c, np.float16(0)), c)   # next value toward zero
    lov = lo.astype(np.float64)
    nxt = np.nextafter(lo, np.float16(np.inf)).astype(np.float64)
    spacing = np.where(np.isinf(nxt), 32.0, nxt - lov)               # past 65504: the binade's spacing
    lo_code = lo.view(np.uint16).astype(np.uint32)
    frac = (av - lov) / spacing                                      # exact: power-of-two spacing
    code = lo_code + (r16 < frac * 65536.0).astype(np.uint32)
    code = np.where(big, 0x7C00, code)                               # |v| >= 65536: infinity
    code = (code | np.where(neg, 0x8000, 0)).astype(np.uint16)
    return np.where(finite, code, out).astype(np.uint16)

