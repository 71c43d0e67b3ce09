"""The oracle's reduced-precision state storage (Philox + rounding to fp16/bf16) against
independent references (CPU).

* The Philox round structure, written once for any word size, reproduces numpy's Philox4x64-10
  bit generator (a library routine); the 32-bit Weyl increments follow from the same closed
  forms as the 64-bit ones.
* Stochastic rounding: for values across the ranges of both formats (fp16 subnormals, the top
  of fp16, negative values, zero), enumerating all 65536 random numbers gives exactly
  ceil(65536 * frac) round-ups, where lo and frac come from an exact derivation with Fractions
  from each format's bit layout; every result is lo or the next code; the mean over all random
  numbers is the value within 2^-16 of a spacing (unbiased).
* Round-to-nearest-even matches the exact nearest value, ties to the even code.
* The A = 0 update path rounds values within one spacing of the fp64 update.
Sources: the modeling_nemotron_h.py walk-through page, 部署时如何调这些缓存 (fp16 state cache,
stochastic rounding, Philox with 5 rounds); Salmon et al., SC 2011 (Philox).
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

from oracle import lowprec as lp
from oracle_pins import rel_err, softplus


def fmt_lo_spacing(v, fmt):
    """Exact (lo, spacing) of the finite fp32 value v in fmt, from the format's parameters
    (exponent bits, mantissa bits): lo = |v| rounded down to the spacing of its binade."""
    av = abs(Fraction(float(np.float32(v))))
    ebits, mbits = (5, 10) if fmt == "f16" else (8, 7)
    emin = 2 - (1 << (ebits - 1))
    e = emin
    while av >= Fraction(2) ** (e + 1):
        e += 1
    spacing = Fraction(2) ** (e - mbits)
    return (av // spacing) * spacing, spacing


def probe_values(fmt):
    r = np.random.default_rng(3)
    v = [r.normal(0, 0.1, 40), r.normal(0, 3.0, 10), -np.abs(r.normal(0, 0.05, 10)),
         np.array([0.0, 1.0, -1.0, 0.1, 2.0 ** -20, 1e-30])]
    if fmt == "f16":
        v += [r.normal(0, 2e-6, 12), r.uniform(-6.1e-5, 6.1e-5, 8), np.array([65504.0, 65519.0, 65535.5, -65520.0])]
    else:
        v += [r.normal(0, 1e-38, 6), np.array([3.0e38, -2.9e38])]
    return np.concatenate(v).astype(np.float32)


def test_philox_structure_matches_numpy_philox4x64():
    for key in [(0x1234567890ABCDEF, 0x0FEDCBA987654321), (0, 0), (2 ** 64 - 1, 7)]:
        raw = np.random.Philox(key=np.array(key, dtype=np.uint64)).random_raw(12)
        ours = []
        for c in (1, 2, 3):                      # numpy advances its counter before each block
            ours += lp.philox4((c, 0, 0, 0), key, 10, 64, lp.PHILOX4x64_M, lp.PHILOX4x64_W)
        assert [int(v) for v in raw] == ours, hex(key[0])
    # a counter that carries into word 1
    bg = np.random.Philox(key=np.array((5, 6), dtype=np.uint64), counter=np.array([2 ** 64 - 1, 0, 0, 0], dtype=np.uint64))
    assert [int(v) for v in bg.random_raw(4)] == list(lp.philox4((0, 1, 0, 0), (5, 6), 10, 64, lp.PHILOX4x64_M,
                                                                 lp.PHILOX4x64_W))


def test_weyl_increments_from_closed_forms():
    getcontext().prec = 60
    phi_m1 = (Decimal(5).sqrt() - 1) / 2
    s3_m1 = Decimal(3).sqrt() - 1
    for w, W in ((32, lp.PHILOX4x32_W), (64, lp.PHILOX4x64_W)):
        assert W[0] == int(phi_m1 * (1 << w)) and W[1] == int(s3_m1 * (1 << w)), w


def test_philox4x32_vectorised_and_random16_uniform():
    c = np.array([0, 1, 2 ** 32 - 1, 12345, 987654321], dtype=np.uint64)
    key = (0xDEADBEEF, 0x12345678)
    v = lp.philox4x32(c, c * 3 & 0xFFFFFFFF, c * 5 & 0xFFFFFFFF, c * 7 & 0xFFFFFFFF, key, 5)
    for i in range(len(c)):
        ctr = [int(c[i]) * m & 0xFFFFFFFF for m in (1, 3, 5, 7)]
        assert tuple(int(w[i]) for w in v) == lp.philox4(ctr, key, 5)
    r = lp.random16(np.arange(1 << 18), 99, 3, 5).astype(np.int64)
    assert abs(r.mean() / 65535 - 0.5) < 0.005
    for bit in range(16):
        assert abs(((r >> bit) & 1).mean() - 0.5) < 0.01, bit
    hist = np.bincount(r >> 8, minlength=256)
    chi2 = ((hist - hist.mean()) ** 2 / hist.mean()).sum()
    assert chi2 < 256 + 6 * math.sqrt(2 * 256)
    # element e takes the 16-bit half (e mod 2) of word (e mod 8) // 2 of block e // 8
    e = np.array([8 * 7 + 5])
    w = lp.philox4((7, 0, 3, 0), (99, 0), 5)[2]
    assert int(lp.random16(e, 99, 3, 5)[0]) == (w >> 16) & 0xFFFF


def test_stochastic_rounding_up_count_is_exact():
    allr = np.arange(65536)
    for fmt in ("f16", "bf16"):
        for v in probe_values(fmt):
            codes = lp.round_state(np.full(65536, v, np.float32), fmt, allr)
            vals = lp.decode(codes, fmt)
            if fmt == "f16" and abs(float(v)) >= 65536:
                assert np.all(np.isinf(vals))
                continue
            lo, sp = fmt_lo_spacing(v, fmt)
            frac = (abs(Fraction(float(v))) - lo) / sp
            sign = -1.0 if np.signbit(v) else 1.0
            is_lo = vals == sign * float(lo)
            hi = sign * float(lo + sp)
            assert np.all(is_lo | (vals == hi) | (np.isinf(vals) & (float(lo + sp) > 65504))), (fmt, v)
            assert int((~is_lo).sum()) == math.ceil(frac * 65536), (fmt, v)
            # unbiased to 2^-16 of a spacing
            mean = Fraction(int(is_lo.sum())) * lo + Fraction(int((~is_lo).sum())) * (lo + sp)
            assert abs(mean / 65536 - abs(Fraction(float(v)))) <= sp / 65536, (fmt, v)


def test_round_to_nearest_even():
    for fmt in ("f16", "bf16"):
        vals = probe_values(fmt)
        codes = lp.round_state(vals, fmt)
        got = lp.decode(codes, fmt)
        for v, g, c in zip(vals, got, codes):
            if fmt == "f16" and abs(float(v)) >= 65520:
                assert np.isinf(g)
                continue
            lo, sp = fmt_lo_spacing(v, fmt)
            av = abs(Fraction(float(v)))
            d_lo, d_hi = av - lo, lo + sp - av
            assert abs(Fraction(float(abs(g)))) in ((lo,) if d_lo < d_hi else (lo + sp,) if d_hi < d_lo
                                                    else (lo, lo + sp)), (fmt, v)
            if d_lo == d_hi:          # a tie: the stored code must be even
                assert int(c) % 2 == 0, (fmt, v)


def test_lp_update_a0_codes_round_the_fp64_update(orc):
    r = np.random.default_rng(9)
    Bt, H, P, G, N = 3, 4, 8, 2, 16
    x = r.standard_normal((Bt, H, P)).astype(np.float32)
    Bm = r.standard_normal((Bt, G, N)).astype(np.float32)
    Cm = r.standard_normal((Bt, G, N)).astype(np.float32)
    dt = softplus(r.normal(-2, 1, (Bt, H))).astype(np.float32)
    for fmt in ("f16", "bf16"):
        codes = lp.round_state((r.standard_normal((5, H, P, N)) * 0.1).astype(np.float32), fmt)
        slot = np.array([4, 0, 2])
        for sr in (None, (1234, 7, 5)):
            new = orc.state_update_lp_codes_a0(codes, fmt, slot, x, Bm, Cm, dt, sr)
            _, exact = orc.state_update_lp(codes, fmt, slot, x, Bm, Cm, dt, np.zeros(H))
            for b, s in enumerate(slot):
                got = lp.decode(new[s], fmt)
                sp = np.array([float(fmt_lo_spacing(v, fmt)[1]) for v in exact[b].ravel()]).reshape(got.shape)
                assert np.all(np.abs(got - exact[b]) <= sp * (0.5 if sr is None else 1.0) + 1e-6 * np.abs(exact[b]))
            for s in (1, 3):
                assert np.array_equal(new[s], codes[s])
    y, st = orc.state_update_lp(codes, "bf16", None, x, Bm, Cm, dt, np.zeros(H))
    assert rel_err(st[0], orc.state_update(lp.decode(codes[:3], "bf16"), x, Bm, Cm, dt, np.zeros(H))[1][0]) == 0


# ----------------------------------------------------------------------------- element -> counter
# The Philox number that rounds a state element is selected by the element's flat index in the
# pool, so it follows the element's pool slot, not the request's position in the batch.  The three
# pins below fix that mapping without re-deriving it from the oracle's own formula: a batch
# permutation, a reshaping of the pool that keeps every element's flat index, and an absolute
# count on a tiny pool whose halfway values expose the top bit of each 16-bit number.

def _a0_inputs(r, Bt, H, P, G, N):
    x = r.standard_normal((Bt, H, P)).astype(np.float32)
    Bm = r.standard_normal((Bt, G, N)).astype(np.float32)
    Cm = r.standard_normal((Bt, G, N)).astype(np.float32)
    dt = softplus(r.normal(-2, 1, (Bt, H))).astype(np.float32)
    return x, Bm, Cm, dt


def test_lp_codes_follow_the_slot_not_the_batch_position(orc):
    r = np.random.default_rng(21)
    Bt, H, P, G, N, nslots = 4, 2, 8, 1, 16, 6
    x, Bm, Cm, dt = _a0_inputs(r, Bt, H, P, G, N)
    slot = np.array([5, 0, 3, 2])
    for fmt in ("f16", "bf16"):
        codes = lp.round_state((r.standard_normal((nslots, H, P, N)) * 0.1).astype(np.float32), fmt)
        want = orc.state_update_lp_codes_a0(codes, fmt, slot, x, Bm, Cm, dt, (77, 3, 5))
        for perm in ([3, 2, 1, 0], [1, 3, 0, 2]):
            got = orc.state_update_lp_codes_a0(codes, fmt, slot[perm], x[perm], Bm[perm], Cm[perm], dt[perm],
                                               (77, 3, 5))
            assert np.array_equal(got, want), (fmt, perm)
        # the same request and starting values in another slot draw other numbers: with slots 1 and 5
        # holding equal codes, moving request 0 from slot 5 to slot 1 changes some of its codes
        twin = codes.copy()
        twin[1] = twin[5]
        at5 = orc.state_update_lp_codes_a0(twin, fmt, slot, x, Bm, Cm, dt, (77, 3, 5))
        at1 = orc.state_update_lp_codes_a0(twin, fmt, np.array([1, 0, 3, 2]), x, Bm, Cm, dt, (77, 3, 5))
        assert not np.array_equal(at1[1], at5[5]), fmt
        assert np.array_equal(orc.state_update_lp_codes_a0(twin, fmt, slot, x, Bm, Cm, dt, None)[5],
                              orc.state_update_lp_codes_a0(twin, fmt, np.array([1, 0, 3, 2]), x, Bm, Cm, dt,
                                                           None)[1]), fmt


def test_lp_codes_depend_on_the_flat_pool_index(orc):
    """Slot s of a pool [S, H, P, N] holds the flat elements [s*H*P*N, (s+1)*H*P*N): a request in slot 1
    of a 2-slot pool of H heads is rounded exactly like heads H..2H-1 of a 1-slot pool of 2H heads
    holding the same values (A = 0, each head's B from a group of its own)."""
    r = np.random.default_rng(22)
    H, P, N = 2, 4, 16
    x, Bm, Cm, dt = _a0_inputs(r, 1, H, P, H, N)
    for fmt in ("f16", "bf16"):
        st = lp.round_state((r.standard_normal((2, H, P, N)) * 0.1).astype(np.float32), fmt)
        two = orc.state_update_lp_codes_a0(st, fmt, np.array([1]), x, Bm, Cm, dt, (5, 9, 5))
        wide = st.reshape(1, 2 * H, P, N)
        z = np.zeros_like(x)
        one = orc.state_update_lp_codes_a0(wide, fmt, None, np.concatenate([z, x], 1),
                                           np.concatenate([Bm, Bm], 1), np.concatenate([Cm, Cm], 1),
                                           np.concatenate([dt, dt], 1), (5, 9, 5))
        assert np.array_equal(one[0, H:], two[1]), fmt
        assert np.array_equal(two[0], st[0]), fmt                        # slot 0 is not in the batch


def test_lp_codes_absolute_index_on_a_tiny_pool(orc):
    """Every element of the request sits exactly halfway between two codes, so it rounds up iff its
    16-bit number is below 2^15.  Slot 2 of a pool of 16-element slots covers flat elements 32..47,
    i.e. Philox blocks 4 and 5 (8 elements per block, two 16-bit halves per word, low half first);
    using the batch position, or starting one block off, changes the pattern."""
    H, P, N = 1, 2, 8
    seed, offset, rounds = 0x1234ABCD, 11, 5
    for fmt, half in (("f16", 2.0 ** -11), ("bf16", 2.0 ** -8)):
        ones = lp.round_state(np.ones((3, H, P, N), np.float32), fmt)
        x = np.ones((1, H, P), np.float32)
        Bm = np.full((1, 1, N), half, np.float32)
        dt = np.ones((1, H), np.float32)
        got = orc.state_update_lp_codes_a0(ones, fmt, np.array([2]), x, Bm, Bm, dt, (seed, offset, rounds))
        up = lp.decode(got[2], fmt).ravel() > 1.0
        want = []
        for block in (4, 5):
            words = lp.philox4((block, 0, offset, 0), (seed, 0), rounds)
            for k in range(8):
                want.append(((words[k // 2] >> (16 * (k % 2))) & 0xFFFF) < 0x8000)
        assert up.tolist() == want, fmt
        assert np.array_equal(got[:2], ones[:2])


# ----------------------------------------------------------------------------- scans on 16-bit states
def dyadic_scan_inputs(r, Bt, L, H, P, G, N, fmt, nstate=None):
    """Inputs on a coarse dyadic grid with A = 0: every product dt*x*B is a multiple of 2^-17 below
    2^-8 in magnitude and every initial value a code of fmt that is a multiple of 2^-17 below 2, so
    every partial sum of a scan over a few hundred tokens is exact in fp32 (and in fp64)."""
    x = r.integers(-16, 17, (Bt, L, H, P)) / 64.0
    Bm = r.integers(-16, 17, (Bt, L, G, N)) / 64.0
    Cm = r.integers(-16, 17, (Bt, L, G, N)) / 64.0
    dt = 2.0 ** -r.integers(3, 6, (Bt, L, H)).astype(np.float64)
    k = r.integers(-1024, 1025, (nstate or Bt, H, P, N)) / 1024.0
    codes = lp.round_state(k.astype(np.float32), fmt)
    return x, Bm, Cm, dt, codes


def test_scan_lp_of_one_token_is_the_a0_update(orc):
    """The 16-bit scan of one token with A = 0 stores the codes of the pinned A = 0 decode update:
    same values, same flat element indices, same random numbers."""
    r = np.random.default_rng(31)
    Bt, H, P, G, N = 3, 4, 8, 2, 16
    for fmt in ("f16", "bf16"):
        x, Bm, Cm, dt, codes = dyadic_scan_inputs(r, Bt, 1, H, P, G, N, fmt)
        A = np.zeros(H)
        for sr in (None, (0xC0FFEE, 17, 5), (3, 2 ** 33 + 1, 7)):
            _, fin, got = orc.scan_lp(x, Bm, Cm, dt, A, None, codes, fmt, sr)
            want = orc.state_update_lp_codes_a0(codes, fmt, None, x[:, 0], Bm[:, 0], Cm[:, 0], dt[:, 0], sr)
            assert np.array_equal(got, want), (fmt, sr)
            assert np.array_equal(fin.astype(np.float32).astype(np.float64), fin)   # exact in fp32
        # no tokens: the final state is the initial one, stored unchanged
        _, _, same = orc.scan_lp(x[:, :0], Bm[:, :0], Cm[:, :0], dt[:, :0], A, None, codes, fmt, (9, 9, 5))
        assert np.array_equal(same, codes), fmt


def test_scan_varlen_lp_rounds_at_the_slot_index(orc):
    """Packed one-token sequences into pool slots: the codes of the A = 0 update at the same slots;
    a sequence without an initial state starts from zeros; padding and unnamed slots keep their
    codes."""
    r = np.random.default_rng(32)
    H, P, G, N, nslots = 2, 8, 1, 16, 7
    slot = np.array([5, 0, -1, 3, 6])
    has_init = np.array([1, 1, 1, 0, 1])
    S = len(slot)
    for fmt in ("f16", "bf16"):
        x, Bm, Cm, dt, codes = dyadic_scan_inputs(r, S, 1, H, P, G, N, fmt, nstate=nslots)
        cu = np.arange(S + 1)
        sr = (0xABCDEF, 5, 5)
        _, got = orc.scan_varlen_lp(x[:, 0], Bm[:, 0], Cm[:, 0], dt[:, 0], np.zeros(H), None, cu, codes, fmt, slot,
                                    has_init, sr)
        start = codes.copy()
        start[3] = lp.round_state(np.zeros((H, P, N), np.float32), fmt)      # sequence 3 starts from zeros
        want = orc.state_update_lp_codes_a0(start, fmt, slot, x[:, 0], Bm[:, 0], Cm[:, 0], dt[:, 0], sr)
        assert np.array_equal(got, want), fmt
        for k in (1, 2, 4):                                                  # no sequence names these
            assert np.array_equal(got[k], codes[k]), (fmt, k)
