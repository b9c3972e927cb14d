"""Pins for the oracle's number formats and quantizer (CPU only).

Each test checks the oracle against something other than itself: hand-derived fixtures,
a brute-force search over every candidate value, closed-form invariants of the rule, or a
library conversion.  The rule is the one of the gllm page, section "Quantization Design"
(symmetric, amax/127, round to nearest, clamp to +-127) with one scale per 32 values
(half-the-memory page, section "Is 8 bits enough?").
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from workloads import f32_to_bf16_bits, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q8_0_groups.txt")

# every finite non-negative binary16 value, decoded by numpy (a library routine), followed
# by 2^16: the value the encoding 0x7C00 (infinity) takes the place of when rounding
_F16_POS = np.append(np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64), 65536.0)


def _nearest_f16_bruteforce(x: float) -> int:
    """binary16 bits of the value nearest to x, ties to the even encoding; inf past 65520."""
    sign = 0x8000 if (x < 0 or (x == 0 and np.signbit(x))) else 0
    a = abs(float(x))
    if a >= 65520.0:  # half-way between 65504 and 2^16 and beyond rounds to infinity
        return sign | 0x7C00
    i = int(np.searchsorted(_F16_POS, a))
    if i < len(_F16_POS) and _F16_POS[i] == a:
        return sign | i
    lo, hi = i - 1, i
    dlo, dhi = a - _F16_POS[lo], _F16_POS[hi] - a
    if dlo < dhi:
        return sign | lo
    if dhi < dlo:
        return sign | hi
    return sign | (lo if lo % 2 == 0 else hi)


def test_f16_to_f32_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.f16_to_f32(bits)
    ref = bits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_against_bruteforce_nearest():
    rng = np.random.default_rng(7)
    # random magnitudes from far below the subnormal range to past overflow, both signs
    xs = (rng.standard_normal(4000) * np.exp2(rng.uniform(-30, 18, 4000))).astype(np.float32)
    # exact midpoints between neighbouring binary16 values, and their fp32 neighbours
    lo = _F16_POS[:-1][::97]
    hi = _F16_POS[1:][::97]
    mids = ((lo + hi) / 2).astype(np.float32)
    special = np.array([0.0, -0.0, 65504, 65519.996, 65520, 65536, 1e-8, 2.0 ** -25, 2.0 ** -24,
                        3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25], dtype=np.float32)
    xs = np.concatenate([xs, mids, np.nextafter(mids, np.float32(np.inf)),
                         np.nextafter(mids, np.float32(0)), special, -special])
    ours = O.f32_to_f16(xs)
    for x, h in zip(xs, ours):
        assert int(h) == _nearest_f16_bruteforce(float(x)), (float(x), hex(int(h)))
    # the library conversion agrees too
    assert np.array_equal(ours, xs.astype(np.float16).view(np.uint16))


def test_bf16_to_f32_known_values():
    L = O.lib()
    assert L.oracle_bf16_to_f32(0x3F80) == 1.0
    assert L.oracle_bf16_to_f32(0xC000) == -2.0
    assert L.oracle_bf16_to_f32(0x4049) == 3.140625
    assert L.oracle_bf16_to_f32(0x0001) == 2.0 ** -133
    assert L.oracle_bf16_to_f32(0x7F7F) == float(np.float32(3.3895313892515355e38))


def _load_golden():
    cases = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, vals, sc, codes = [p.strip() for p in line.split(";")]
        x = np.zeros(32, dtype=np.float32)
        v = [float(t) for t in vals.split()]
        x[: len(v)] = v
        c = np.zeros(32, dtype=np.int8)
        cv = [int(t) for t in codes.split()]
        c[: len(cv)] = cv
        cases.append((name, x, int(sc, 16), c))
    return cases


@pytest.mark.parametrize("name,x,scale_bits,codes", _load_golden(), ids=[c[0] for c in _load_golden()])
def test_quantizer_golden(name, x, scale_bits, codes):
    xb = f32_to_bf16_bits(x)
    assert np.array_equal(bf16_bits_to_f32(xb), x), "fixture values must be bf16-exact"
    q, s = O.quantize_groups(xb[None])
    assert int(s[0]) == scale_bits, (name, hex(int(s[0])))
    assert np.array_equal(q[0], codes), (name, q[0][:8], codes[:8])


def _random_groups(n, seed):
    rng = np.random.default_rng(seed)
    mags = np.exp2(rng.uniform(-18, 14, size=(n, 1))).astype(np.float32)
    x = rng.standard_normal((n, 32)).astype(np.float32) * mags
    # a few outlier channels, as in the workloads
    idx = rng.integers(0, 32, size=(n, 2))
    np.put_along_axis(x, idx, np.take_along_axis(x, idx, axis=1) * 20, axis=1)
    return f32_to_bf16_bits(x)


def test_scale_is_nearest_fp16_of_correctly_rounded_quotient():
    xb = _random_groups(600, 1)
    x = bf16_bits_to_f32(xb).astype(np.float64)
    q, s = O.quantize_groups(xb)
    amax = np.abs(x).max(axis=1)
    for a, sb in zip(amax, s):
        d = np.float32(a) / np.float32(127)  # IEEE single division (a library operation)
        # d is the single nearest to the exact quotient
        exact = Fraction(float(a)) / 127
        ulp = Fraction(float(np.spacing(d)))
        assert abs(Fraction(float(d)) - exact) <= ulp / 2
        ds = min(float(d), 65504.0)
        assert int(sb) == _nearest_f16_bruteforce(ds)


def test_codes_are_nearest_multiple_of_stored_scale():
    """Brute force: each code is the c in [-127, 127] minimising |x - c*s|, ties to even c."""
    xb = _random_groups(300, 2)
    x = bf16_bits_to_f32(xb).astype(np.float64)
    q, s = O.quantize_groups(xb)
    sv = s.view(np.float16).astype(np.float64)
    cands = np.arange(-127, 128, dtype=np.int64)
    for gi in range(x.shape[0]):
        if sv[gi] == 0:
            assert not q[gi].any()
            continue
        for i in range(32):
            xf = Fraction(float(x[gi, i]))
            sf = Fraction(float(sv[gi]))
            errs = [abs(xf - int(c) * sf) for c in cands]
            best = min(errs)
            tied = [int(c) for c, e in zip(cands, errs) if e == best]
            want = tied[0] if len(tied) == 1 else [c for c in tied if c % 2 == 0][0]
            assert int(q[gi, i]) == want, (gi, i, float(x[gi, i]), float(sv[gi]), int(q[gi, i]), want)


def test_quantizer_invariants():
    xb = _random_groups(5000, 3)
    x = bf16_bits_to_f32(xb).astype(np.float64)
    q, s = O.quantize_groups(xb)
    sv = s.view(np.float16).astype(np.float64)
    normal = (sv >= 2.0 ** -14) & (sv < 65504)
    assert normal.sum() > 3000 and (~normal).sum() > 200  # both kinds are exercised
    qi = q.astype(np.int64)
    # the largest value always lands on +-127 when the scale is a normal fp16
    assert np.all(np.abs(qi[normal]).max(axis=1) == 127)
    # reconstruction error at most half a scale step
    err = np.abs(x - qi * sv[:, None])
    assert np.all(err[normal] <= sv[normal, None] / 2)
    # odd symmetry: quantize(-x) = -quantize(x) with the same scale
    qn, sn = O.quantize_groups(xb ^ np.uint16(0x8000))
    assert np.array_equal(sn, s)
    assert np.array_equal(qn.astype(np.int64), -qi)


def test_on_grid_values_are_lossless_and_idempotent():
    """Groups that already are integers times 2^e with amax = 127*2^e quantize exactly."""
    rng = np.random.default_rng(4)
    for e in range(-20, 9):
        ints = rng.integers(-127, 128, size=32)
        ints[rng.integers(0, 32)] = 127 * (1 if rng.random() < 0.5 else -1)
        x = (ints * 2.0 ** e).astype(np.float32)
        xb = f32_to_bf16_bits(x)
        assert np.array_equal(bf16_bits_to_f32(xb), x)
        q, s = O.quantize_groups(xb[None])
        assert float(s.view(np.float16)[0]) == 2.0 ** e
        assert np.array_equal(q[0].astype(np.int64), ints)
        # dequantize (q * s is exact and bf16-exact here) and quantize again: same bytes
        q2, s2 = O.quantize_groups(f32_to_bf16_bits((q[0] * 2.0 ** e).astype(np.float32))[None])
        assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_kv_write_slot_rules():
    """slot < 0 writes nothing, no byte outside written slots changes, a rewrite replaces the slot."""
    rng = np.random.default_rng(5)
    Hkv, D, NB = 2, 64, 3
    c = O.OracleCache.empty("int8", NB, Hkv, D)
    before_k, before_ks = c.k.copy(), c.k_scales.copy()
    k = f32_to_bf16_bits(rng.standard_normal((4, Hkv, D)).astype(np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((4, Hkv, D)).astype(np.float32))
    slots = np.array([17, -1, 5, 47], dtype=np.int32)
    O.kv_write(c, k, v, slots)
    written = {17, 5, 47}
    for blk in range(NB):
        for off in range(16):
            slot = blk * 16 + off
            same = np.array_equal(c.k[blk, :, off], before_k[blk, :, off]) and \
                np.array_equal(c.k_scales[blk, :, off], before_ks[blk, :, off])
            assert same == (slot not in written), slot
    # the stored bytes are the quantized token rows
    for t, slot in [(0, 17), (2, 5), (3, 47)]:
        qk, sk = O.quantize_groups(k[t].reshape(Hkv, D // 32, 32))
        assert np.array_equal(c.k[slot // 16, :, slot % 16], qk.reshape(Hkv, D))
        assert np.array_equal(c.k_scales[slot // 16, :, slot % 16], sk)
    # rewrite slot 5 with new values: every code and scale of that slot is replaced
    k2 = f32_to_bf16_bits((rng.standard_normal((1, Hkv, D)) * 3).astype(np.float32))
    O.kv_write(c, k2, k2, np.array([5], dtype=np.int32))
    qk, sk = O.quantize_groups(k2[0].reshape(Hkv, D // 32, 32))
    assert np.array_equal(c.k[0, :, 5], qk.reshape(Hkv, D))
    assert np.array_equal(c.v_scales[0, :, 5], sk)
