"""Pins for the oracle's per-head INT8 format: one fp32 scale per (token, KV head) row (the
half-the-memory page's description of vLLM's int8_per_token_head cache, section "Is 8 bits
enough?": one shared 32-bit scale per 256 values), symmetric amax/127 codes.

Pinned against: hand-derived rows (ties to even at unit scale, half scale, zero row), the fp32
steps checked in exact arithmetic (correctly rounded amax/127 and x/s, then ties to even), a
reconstruction bound of half a step plus the quotient's rounding, invariants on
random rows, lossless on-grid rows, an independent numpy float32 quantizer, a brute-force
decode over the decoded cache, and on-grid data decoding the same in all three cache formats.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from workloads import bf16_bits_to_f32, f32_to_bf16_bits

PAGE = 16


def _row(vals, D=64, amax=None):
    x = np.zeros(D, np.float32)
    x[:len(vals)] = vals
    if amax is not None:
        x[-1] = amax
    return f32_to_bf16_bits(x)


def test_hand_derived_rows():
    # amax 127: s = 1 exactly; 2.5 -> 2, 3.5 -> 4, -2.5 -> -2, -0.5 -> 0, 0.5 -> 0, 1.5 -> 2 (ties to even)
    q, s = O.quantize_rows_head(_row([2.5, 3.5, -2.5, -0.5, 0.5, 1.5], amax=127.0)[None])
    assert float(s[0]) == 1.0
    assert list(q[0, :6]) == [2, 4, -2, 0, 0, 2] and q[0, -1] == 127
    # amax 63.5: s = 0.5; 1.25 -> 2.5 -> 2, 0.75 -> 1.5 -> 2
    q, s = O.quantize_rows_head(_row([1.25, 0.75], amax=63.5)[None])
    assert float(s[0]) == 0.5 and list(q[0, :2]) == [2, 2]
    # a zero row: scale 0, codes 0
    q, s = O.quantize_rows_head(np.zeros((1, 256), np.uint16))
    assert float(s[0]) == 0.0 and not q.any()
    # amax 1: s = fl(1/127); 0.5 / s = 63.5000... just above the tie -> 64
    q, s = O.quantize_rows_head(_row([0.5], amax=1.0)[None])
    assert s[0] == np.float32(1.0) / np.float32(127.0) and q[0, 0] == 64


def _random_rows(n, D, seed):
    rng = np.random.default_rng(seed)
    mags = np.exp2(rng.uniform(-30, 30, size=(n, 1))).astype(np.float32)
    x = rng.standard_normal((n, D)).astype(np.float32) * mags
    idx = rng.integers(0, D, size=(n, 4))
    np.put_along_axis(x, idx, np.take_along_axis(x, idx, axis=1) * 20, axis=1)
    return f32_to_bf16_bits(x)


def _round_half_even(f: Fraction) -> int:
    lo = f.numerator // f.denominator
    rem = f - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        return lo + 1
    return lo


def test_scale_and_codes_follow_the_fp32_steps():
    """s is the correctly rounded quotient amax/127; each code is the quotient x/s correctly
    rounded to fp32, then rounded half to even and clamped (checked in exact arithmetic)."""
    xb = _random_rows(40, 64, 1)
    x = bf16_bits_to_f32(xb).astype(np.float64)
    q, s = O.quantize_rows_head(xb)
    for r in range(xb.shape[0]):
        a = np.abs(x[r]).max()
        exact = Fraction(float(a)) / 127
        assert abs(Fraction(float(s[r])) - exact) <= Fraction(float(np.spacing(np.float32(s[r])))) / 2
        sf = Fraction(float(s[r]))
        for i in range(64):
            qe = Fraction(float(x[r, i])) / sf                       # exact quotient
            d = np.float32(x[r, i]) / np.float32(s[r])               # IEEE single division
            assert abs(Fraction(float(d)) - qe) <= Fraction(float(np.spacing(np.abs(d)))) / 2
            want = max(-127, min(127, _round_half_even(Fraction(float(d)))))
            assert int(q[r, i]) == want
            # the code is the nearest multiple of s up to the quotient's rounding
            assert abs(Fraction(float(x[r, i])) - want * sf) <= sf * (Fraction(1, 2) + Fraction(1, 2 ** 16))


def test_invariants_on_random_rows():
    xb = _random_rows(3000, 256, 2)
    x = bf16_bits_to_f32(xb).astype(np.float64)
    q, s = O.quantize_rows_head(xb)
    sv = s.astype(np.float64)
    normal = sv >= np.finfo(np.float32).tiny
    assert normal.sum() > 2000
    qi = q.astype(np.int64)
    assert np.all(np.abs(qi[normal]).max(axis=1) == 127)
    # at most half a step, plus the rounding of the fp32 quotient x/s (|x/s| < 128: 2^-18)
    assert np.all(np.abs(x - qi * sv[:, None])[normal] <= sv[normal, None] * (0.5 + 2.0 ** -16))
    qn, sn = O.quantize_rows_head(xb ^ np.uint16(0x8000))
    assert np.array_equal(sn, s) and np.array_equal(qn.astype(np.int64), -qi)


def test_on_grid_rows_are_lossless():
    rng = np.random.default_rng(3)
    for e in range(-40, 40, 3):
        ints = rng.integers(-127, 128, size=128)
        ints[rng.integers(0, 128)] = -127
        x = (ints * 2.0 ** e).astype(np.float32)
        xb = f32_to_bf16_bits(x)
        assert np.array_equal(bf16_bits_to_f32(xb), x)
        q, s = O.quantize_rows_head(xb[None])
        assert float(s[0]) == 2.0 ** e and np.array_equal(q[0].astype(np.int64), ints)


def _numpy_quantizer(xb):
    """An independent implementation with numpy float32 operations."""
    x = bf16_bits_to_f32(xb)
    amax = np.abs(x).max(axis=-1)
    s = (amax / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(x / s[..., None]).astype(np.float32)
    r = np.where(np.isnan(r), np.float32(0), r)
    r = np.clip(r, -127, 127)
    r = np.where(s[..., None] == 0, np.float32(0), r)
    return r.astype(np.int8), s


@pytest.mark.parametrize("D", [128, 256])
def test_matches_independent_numpy_quantizer(D):
    xb = _random_rows(4000, D, 4 + D)
    xb[:50] &= np.uint16(0x807F)        # tiny rows (subnormal-range bf16 exponents)
    xb[50:60] = 0
    q, s = O.quantize_rows_head(xb)
    qn, sn = _numpy_quantizer(xb)
    assert np.array_equal(s.view(np.uint32), sn.view(np.uint32))
    assert np.array_equal(q, qn)


def _cache_and_queries(seed, dtype, lens, Hq, Hkv, D, values):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, np.int32)
    pages = (lens + PAGE - 1) // PAGE
    nb = int(pages.sum()) + 2
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((len(lens), int(pages.max())), -1, np.int32)
    pos = 0
    for s_, p in enumerate(pages):
        bt[s_, :p] = perm[pos:pos + p]
        pos += p
    cache = O.OracleCache.empty(dtype, nb, Hkv, D)
    for s_, L in enumerate(lens):
        k, v = values(np.random.default_rng(seed * 100 + s_), L, Hkv, D)
        t = np.arange(L)
        O.kv_write(cache, k, v, (bt[s_, t // PAGE] * PAGE + t % PAGE).astype(np.int32))
    q = f32_to_bf16_bits(rng.standard_normal((len(lens), Hq, D)).astype(np.float32))
    return cache, q, bt, lens


def _normal_values(rng, L, Hkv, D):
    return (f32_to_bf16_bits(rng.standard_normal((L, Hkv, D)).astype(np.float32) * 2),
            f32_to_bf16_bits(rng.standard_normal((L, Hkv, D)).astype(np.float32)))


def test_decode_bruteforce():
    cache, q, bt, lens = _cache_and_queries(5, "int8_head", [37, 70, 1], 6, 2, 64, _normal_values)
    out, lse = O.decode(cache, q, bt, lens)
    # brute force over the decoded cache, decoded here: code * fp32 scale
    K = cache.k.astype(np.float64) * cache.k_scales.astype(np.float64)[..., None]
    V = cache.v.astype(np.float64) * cache.v_scales.astype(np.float64)[..., None]
    qf = bf16_bits_to_f32(q).astype(np.float64)
    for s_ in range(len(lens)):
        t = np.arange(lens[s_])
        blk, off = bt[s_, t // PAGE], t % PAGE
        for hq in range(6):
            z = K[blk, hq // 3, off] @ qf[s_, hq] / 8.0
            w = np.exp(z - z.max())
            assert np.allclose(out[s_, hq], w @ V[blk, hq // 3, off] / w.sum(), rtol=1e-12, atol=1e-12)
            assert abs(lse[s_, hq] - (z.max() + np.log(w.sum()))) < 1e-12
    # and every split count gives the same result
    for ns in (1, 2, 5):
        o2, l2 = O.decode(cache, q, bt, lens, num_splits=ns)
        assert np.allclose(o2, out, rtol=1e-12, atol=1e-12) and np.allclose(l2, lse, rtol=1e-12, atol=1e-12)


def test_on_grid_data_decodes_the_same_in_every_format():
    """Rows whose 32-groups and whole rows are both on the grid (integers times 2^e, amax 127*2^e
    in every group): all three caches hold the exact values."""
    def on_grid(rng, L, Hkv, D):
        out = []
        for _ in range(2):
            ints = rng.integers(-127, 128, size=(L, Hkv, D))
            ints[..., ::32] = 127
            e = rng.integers(-6, 3, size=(L, Hkv, 1))
            out.append(f32_to_bf16_bits((ints * np.exp2(e)).astype(np.float32)))
        return out[0], out[1]
    res = []
    for dtype in ("int8", "int8_head", "bf16"):
        cache, q, bt, lens = _cache_and_queries(6, dtype, [50, 17], 4, 2, 128, on_grid)
        res.append(O.decode(cache, q, bt, lens))
    for o, l in res[1:]:
        assert np.array_equal(o, res[0][0]) and np.array_equal(l, res[0][1])


def test_per_32_scales_follow_outlier_channels_better():
    """The pages' reason for per-32 scales: with outlier channels (x20, as in the workloads) one
    scale per row spends its range on the outliers.  On such data the decode error against the
    unquantized BF16 cache is smaller with per-32 scales."""
    def outliers(rng, L, Hkv, D):
        mult = np.ones((Hkv, D), np.float32)
        for h in range(Hkv):
            mult[h, rng.choice(D, 4, replace=False)] = 20
        return (f32_to_bf16_bits((rng.standard_normal((L, Hkv, D)) * mult).astype(np.float32)),
                f32_to_bf16_bits((rng.standard_normal((L, Hkv, D)) * mult).astype(np.float32)))
    res = {}
    for dtype in ("int8", "int8_head", "bf16"):
        cache, q, bt, lens = _cache_and_queries(7, dtype, [500, 300], 8, 2, 256, outliers)
        res[dtype] = O.decode(cache, q, bt, lens)[0]
    e32 = np.abs(res["int8"] - res["bf16"]).mean()
    ehead = np.abs(res["int8_head"] - res["bf16"]).mean()
    assert e32 < ehead / 2, (e32, ehead)
