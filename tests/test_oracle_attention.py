"""Pins for the oracle's decode attention (CPU only).

Pinned against: a numpy brute force softmax(q K^T / sqrt(D)) V over the decoded cache on tiny
inputs, closed forms (uniform scores, one token, two tokens, a dominant key), invariants
(every split count gives the same result -- the long-context page, section "Give more GPU
workers a piece of the attention calculation"; physical page placement does not matter;
GQA head mapping), the empty context, and lossless on-grid INT8 versus the BF16 cache.
"""
import numpy as np
import pytest

import oracle as O
from workloads import f32_to_bf16_bits, bf16_bits_to_f32

PAGE = 16


def _problem(seed, lens, Hq, Hkv, D, dtype, spare=3, values=None):
    """Random tokens written through the oracle's kv_write into a shuffled pool."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    S = len(lens)
    pages = (lens + PAGE - 1) // PAGE
    nb = int(pages.sum()) + spare
    perm = rng.permutation(nb).astype(np.int32)
    mb = max(1, int(pages.max()))
    bt = np.full((S, mb), -1, dtype=np.int32)
    pos = 0
    for s in range(S):
        bt[s, : pages[s]] = perm[pos: pos + pages[s]]
        pos += pages[s]
    cache = O.OracleCache.empty(dtype, nb, Hkv, D)
    toks_k, toks_v = [], []
    for s in range(S):
        if values is None:
            k = rng.standard_normal((lens[s], Hkv, D)).astype(np.float32) * 2
            v = rng.standard_normal((lens[s], Hkv, D)).astype(np.float32)
        else:
            k, v = values(rng, s, lens[s])
        kb, vb = f32_to_bf16_bits(k), f32_to_bf16_bits(v)
        t = np.arange(lens[s])
        slots = (bt[s, t // PAGE] * PAGE + t % PAGE).astype(np.int32)
        O.kv_write(cache, kb, vb, slots)
        toks_k.append(kb)
        toks_v.append(vb)
    q = f32_to_bf16_bits(rng.standard_normal((S, Hq, D)).astype(np.float32))
    return cache, q, bt, lens


def _decoded(cache, which):
    """Decoded cache, computed here independently: code * fp16 scale (numpy decode), or bf16."""
    if cache.dtype == "int8":
        codes = cache.k if which == "k" else cache.v
        sc = (cache.k_scales if which == "k" else cache.v_scales).view(np.float16).astype(np.float64)
        return codes.astype(np.float64) * np.repeat(sc, 32, axis=-1)
    arr = cache.k if which == "k" else cache.v
    return bf16_bits_to_f32(arr).astype(np.float64)


def _bruteforce(cache, q, bt, lens):
    K, V = _decoded(cache, "k"), _decoded(cache, "v")
    S, Hq, D = q.shape
    G = Hq // cache.num_kv_heads
    qf = bf16_bits_to_f32(q).astype(np.float64)
    out = np.zeros((S, Hq, D))
    lse = np.full((S, Hq), -np.inf)
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        t = np.arange(L)
        blk, off = bt[s, t // PAGE], t % PAGE
        for hq in range(Hq):
            h = hq // G
            Kt, Vt = K[blk, h, off], V[blk, h, off]          # [L][D]
            z = Kt @ qf[s, hq] / np.sqrt(D)
            m = z.max()
            w = np.exp(z - m)
            out[s, hq] = (w @ Vt) / w.sum()
            lse[s, hq] = m + np.log(w.sum())
    return out, lse


@pytest.mark.parametrize("dtype", ["int8", "bf16"])
@pytest.mark.parametrize("D", [32, 128, 256])
def test_bruteforce_tiny(dtype, D):
    for seed, lens, Hq, Hkv in [(1, [37], 6, 1), (2, [64, 5], 4, 2), (3, [1, 16, 17], 8, 4)]:
        cache, q, bt, lens = _problem(seed, lens, Hq, Hkv, D, dtype)
        out, lse = O.decode(cache, q, bt, lens)
        ref, rlse = _bruteforce(cache, q, bt, lens)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
        assert np.allclose(lse, rlse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype", ["int8", "bf16"])
def test_every_split_count_gives_the_same_result(dtype):
    cache, q, bt, lens = _problem(11, [200, 45, 16, 1], 6, 2, 64, dtype)
    out, lse = O.decode(cache, q, bt, lens)
    max_pages = int((lens.max() + PAGE - 1) // PAGE)
    for ns in list(range(1, max_pages + 1)) + [max_pages + 3, 64]:
        o2, l2 = O.decode(cache, q, bt, lens, num_splits=ns)
        assert np.allclose(o2, out, rtol=1e-12, atol=1e-12), ns
        assert np.allclose(l2, lse, rtol=1e-12, atol=1e-12), ns


def test_uniform_scores_give_mean_of_values():
    cache, q, bt, lens = _problem(12, [77, 300], 4, 2, 128, "int8")
    q[:] = 0  # bf16 +0.0: every score is 0
    out, lse = O.decode(cache, q, bt, lens)
    V = _decoded(cache, "v")
    for s in range(2):
        t = np.arange(lens[s])
        for hq in range(4):
            mean = V[bt[s, t // PAGE], hq // 2, t % PAGE].mean(axis=0)
            assert np.allclose(out[s, hq], mean, rtol=1e-12, atol=1e-13)
            assert abs(lse[s, hq] - np.log(lens[s])) < 1e-12


def test_single_token_returns_its_value():
    cache, q, bt, lens = _problem(13, [1, 1], 6, 3, 256, "int8")
    out, lse = O.decode(cache, q, bt, lens)
    V = _decoded(cache, "v")
    K = _decoded(cache, "k")
    qf = bf16_bits_to_f32(q).astype(np.float64)
    for s in range(2):
        for hq in range(6):
            assert np.array_equal(out[s, hq], V[bt[s, 0], hq // 2, 0])
            z0 = K[bt[s, 0], hq // 2, 0] @ qf[s, hq] / 16.0
            assert abs(lse[s, hq] - z0) < 1e-12 * max(1, abs(z0))


def test_two_tokens_closed_form():
    """q = b e0, K0 = a e0, K1 = 0: z0 = a b / sqrt(D), z1 = 0, out = sigmoid(z0) V0 + (1 - sigmoid(z0)) V1."""
    D = 128
    a, b = 3.0, 5.0

    def values(rng, s, L):
        k = np.zeros((L, 1, D), np.float32)
        k[0, 0, 0] = a
        v = np.zeros((L, 1, D), np.float32)
        v[0, 0, :] = 1.5
        v[1, 0, :] = -0.25
        return k, v

    cache, q, bt, lens = _problem(14, [2], 1, 1, D, "bf16", values=values)
    q[:] = 0
    q[0, 0, 0] = f32_to_bf16_bits(np.array([b], dtype=np.float32))[0]
    out, lse = O.decode(cache, q, bt, lens)
    z0 = a * b / np.sqrt(D)
    sig = 1.0 / (1.0 + np.exp(-z0))
    assert np.allclose(out[0, 0], sig * 1.5 + (1 - sig) * (-0.25), rtol=1e-13, atol=0)
    assert abs(lse[0, 0] - np.log1p(np.exp(z0))) < 1e-13


def test_gqa_head_mapping():
    """V of KV head h is the constant h + 1 (lossless on the INT8 grid): query head hq gets hq // G + 1."""
    Hq, Hkv, D = 12, 4, 64

    def values(rng, s, L):
        k = rng.standard_normal((L, Hkv, D)).astype(np.float32)
        v = np.broadcast_to((np.arange(Hkv, dtype=np.float32) + 1)[None, :, None], (L, Hkv, D)).copy()
        return k, v

    cache, q, bt, lens = _problem(15, [40, 9], Hq, Hkv, D, "int8", values=values)
    out, _ = O.decode(cache, q, bt, lens)
    # constant groups quantize to code 127 and scale fp16((h+1)/127); dequantized value is that product
    for hq in range(Hq):
        h = hq // (Hq // Hkv)
        s16 = np.float32(np.float16(np.float32(h + 1) / np.float32(127)))
        assert np.allclose(out[:, hq], 127 * float(s16), rtol=1e-13, atol=0), hq


def test_page_placement_does_not_matter():
    cache, q, bt, lens = _problem(16, [150, 33], 6, 2, 128, "int8", spare=7)
    out, lse = O.decode(cache, q, bt, lens)
    rng = np.random.default_rng(0)
    perm = rng.permutation(cache.num_blocks)          # block b moves to perm[b]
    moved = O.OracleCache.empty("int8", cache.num_blocks, 2, 128)
    for arr_src, arr_dst in [(cache.k, moved.k), (cache.v, moved.v), (cache.k_scales, moved.k_scales),
                             (cache.v_scales, moved.v_scales)]:
        arr_dst[perm] = arr_src
    bt2 = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    out2, lse2 = O.decode(moved, q, bt2, lens)
    assert np.array_equal(out2, out) and np.array_equal(lse2, lse)


def test_dominant_key_selects_its_value():
    D = 256

    def values(rng, s, L):
        k = rng.standard_normal((L, 1, D)).astype(np.float32) * 0.1
        v = rng.standard_normal((L, 1, D)).astype(np.float32)
        return k, v

    cache, q, bt, lens = _problem(17, [96], 1, 1, D, "bf16", values=values)
    qf = bf16_bits_to_f32(q)[0, 0]
    # overwrite token 40's key with 8 * q (z ~ 8 |q|^2 / 16, far above the others)
    blk, off = bt[0, 40 // PAGE], 40 % PAGE
    cache.k[blk, 0, off] = f32_to_bf16_bits(8 * qf)
    out, _ = O.decode(cache, q, bt, lens)
    v40 = bf16_bits_to_f32(cache.v[blk, 0, off]).astype(np.float64)
    assert np.allclose(out[0, 0], v40, rtol=0, atol=1e-9)


def test_empty_context():
    cache, q, bt, lens = _problem(18, [20, 3], 4, 1, 64, "int8")
    lens = lens.copy()
    lens[1] = 0
    out, lse = O.decode(cache, q, bt, lens)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    for ns in (1, 2, 5):
        o2, l2 = O.decode(cache, q, bt, lens, num_splits=ns)
        assert np.all(o2[1] == 0) and np.all(np.isneginf(l2[1]))
        assert np.allclose(o2[0], out[0], rtol=1e-12, atol=1e-12)


def test_lossless_int8_matches_bf16_cache():
    """K and V already on the q8_0 grid (integers times 2^e, amax 127*2^e per group) lose nothing."""
    D, Hkv = 128, 2

    def values(rng, s, L):
        e = rng.integers(-6, 3, size=(L, Hkv, D // 32, 1))
        ints = rng.integers(-127, 128, size=(L, Hkv, D // 32, 32))
        ints[..., 0] = 127
        k = (ints * np.exp2(e)).astype(np.float32).reshape(L, Hkv, D)
        ints = rng.integers(-127, 128, size=(L, Hkv, D // 32, 32))
        ints[..., 5] = -127
        v = (ints * np.exp2(e)).astype(np.float32).reshape(L, Hkv, D)
        return k, v

    c8, q, bt, lens = _problem(19, [70, 18], 6, Hkv, D, "int8", values=values)
    c16, q2, bt2, _ = _problem(19, [70, 18], 6, Hkv, D, "bf16", values=values)
    assert np.array_equal(q, q2) and np.array_equal(bt, bt2)
    o8, l8 = O.decode(c8, q, bt, lens)
    o16, l16 = O.decode(c16, q, bt, lens)
    assert np.allclose(o8, o16, rtol=1e-13, atol=1e-13) and np.allclose(l8, l16, rtol=1e-13, atol=1e-13)


def test_row_subset_matches_full():
    cache, q, bt, lens = _problem(20, [100, 60, 7], 8, 2, 128, "int8")
    out, lse = O.decode(cache, q, bt, lens)
    rows = np.array([0, 5, 9, 23, 17], dtype=np.int64)
    o2, l2 = O.decode(cache, q, bt, lens, rows=rows)
    assert np.array_equal(o2, out.reshape(-1, 128)[rows]) and np.array_equal(l2, lse.reshape(-1)[rows])


# ------------------------------------------------------------------ several query tokens

def _bruteforce_mq(cache, q, bt, lens):
    """Causal attention written out directly: the score matrix of the n_q queries against every
    key of the context, with the keys after each query's position masked."""
    K, V = _decoded(cache, "k"), _decoded(cache, "v")
    S, nq, Hq, D = q.shape
    G = Hq // cache.num_kv_heads
    qf = bf16_bits_to_f32(q).astype(np.float64)
    out = np.zeros((S, nq, Hq, D))
    lse = np.full((S, nq, Hq), -np.inf)
    for s in range(S):
        L = int(lens[s])
        if L == 0:
            continue
        t = np.arange(L)
        blk, off = bt[s, t // PAGE], t % PAGE
        pos = L - nq + np.arange(nq)                          # position of each query token
        visible = t[None, :] <= pos[:, None]                  # [nq][L]
        for hq in range(Hq):
            Kt, Vt = K[blk, hq // G, off], V[blk, hq // G, off]
            z = qf[s, :, hq] @ Kt.T / np.sqrt(D)              # [nq][L]
            z = np.where(visible, z, -np.inf)
            for i in range(nq):
                if not visible[i].any():
                    continue
                m = z[i].max()
                w = np.exp(z[i] - m)
                out[s, i, hq] = (w @ Vt) / w.sum()
                lse[s, i, hq] = m + np.log(w.sum())
    return out, lse


def _q_mq(seed, S, nq, Hq, D):
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((S, nq, Hq, D)).astype(np.float32))


@pytest.mark.parametrize("dtype", ["int8", "bf16"])
def test_multi_token_bruteforce(dtype):
    for seed, lens, Hq, Hkv, D, nq in [(21, [37, 70], 6, 1, 64, 3), (22, [16, 17, 5], 8, 4, 128, 5),
                                       (23, [40], 4, 2, 256, 16)]:
        cache, _, bt, lens = _problem(seed, lens, Hq, Hkv, D, dtype)
        q = _q_mq(seed, len(lens), nq, Hq, D)
        out, lse = O.decode_mq(cache, q, bt, lens)
        ref, rlse = _bruteforce_mq(cache, q, bt, lens)
        assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)
        assert np.array_equal(np.isinf(lse), np.isinf(rlse))
        fin = np.isfinite(rlse)
        assert np.allclose(lse[fin], rlse[fin], rtol=1e-12, atol=1e-12)


def test_multi_token_one_query_is_decode():
    cache, q1, bt, lens = _problem(24, [300, 33], 6, 2, 64, "int8")
    out, lse = O.decode_mq(cache, q1[:, None], bt, lens)
    ref, rlse = O.decode(cache, q1, bt, lens)
    assert np.array_equal(out[:, 0], ref) and np.array_equal(lse[:, 0], rlse)


def test_multi_token_is_causal():
    """Changing the last token's key and value changes only the last query's output."""
    cache, _, bt, lens = _problem(25, [90], 6, 2, 64, "int8")
    q = _q_mq(25, 1, 4, 6, 64)
    out, _ = O.decode_mq(cache, q, bt, lens)
    rng = np.random.default_rng(26)
    L = int(lens[0])
    slot = np.array([bt[0, (L - 1) // PAGE] * PAGE + (L - 1) % PAGE], np.int32)
    O.kv_write(cache, f32_to_bf16_bits(rng.standard_normal((1, 2, 64)).astype(np.float32) * 5),
               f32_to_bf16_bits(rng.standard_normal((1, 2, 64)).astype(np.float32) * 5), slot)
    out2, _ = O.decode_mq(cache, q, bt, lens)
    assert np.array_equal(out[:, :3], out2[:, :3])
    assert not np.allclose(out[:, 3], out2[:, 3])


def test_multi_token_more_queries_than_context():
    """Query tokens before the first position see no key: out 0, lse -inf."""
    cache, _, bt, lens = _problem(27, [3, 0], 4, 2, 32, "int8")
    q = _q_mq(27, 2, 5, 4, 32)
    out, lse = O.decode_mq(cache, q, bt, lens)
    assert np.all(out[0, :2] == 0) and np.all(np.isneginf(lse[0, :2]))
    assert np.all(np.isfinite(lse[0, 2:]))
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))
    ref, rlse = _bruteforce_mq(cache, q, bt, lens)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ integer Q.K (opt-in)

def test_quantized_q_error_bound_and_on_grid():
    rng = np.random.default_rng(31)
    q = f32_to_bf16_bits((rng.standard_normal((3, 6, 64)) * np.exp2(rng.uniform(-6, 6, (3, 6, 1)))).astype(np.float32))
    qd = O.quantized_q(q)
    x = bf16_bits_to_f32(q).astype(np.float64).reshape(-1, 32)
    amax = np.abs(x).max(axis=1, keepdims=True)
    # half a scale step, the scale being within half an fp16 ulp of amax/127
    assert np.all(np.abs(x - qd.reshape(-1, 32)) <= amax / 127 * (0.5 + 2.0 ** -10) + 1e-300)
    # values on the q8_0 grid are reproduced exactly
    ints = rng.integers(-127, 128, size=(2, 4, 64))
    ints[..., ::32] = 127
    qg = f32_to_bf16_bits((ints * 2.0 ** -3).astype(np.float32))
    assert np.array_equal(O.quantized_q(qg), ints * 2.0 ** -3)


@pytest.mark.parametrize("dtype", ["int8", "bf16"])
def test_integer_qk_equals_decode_on_grid_queries(dtype):
    """With queries already on the q8_0 grid, quantizing Q changes nothing: the integer-Q.K
    definition must equal the (independently pinned) decode."""
    cache, _, bt, lens = _problem(32, [70, 16, 1], 8, 2, 128, dtype)
    rng = np.random.default_rng(33)
    ints = rng.integers(-127, 128, size=(3, 8, 128))
    ints[..., ::32] = 127
    q = f32_to_bf16_bits((ints * 2.0 ** -5).astype(np.float32))
    out, lse = O.decode_int8_qk(cache, q, bt, lens)
    ref, rlse = O.decode(cache, q, bt, lens)
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12) and np.allclose(lse, rlse, rtol=1e-12, atol=1e-12)


def test_integer_qk_error_is_the_query_rounding():
    """On random queries the integer-Q.K result differs from decode with the exact query, by a
    small amount set by the query's rounding (the pages report about 1-2%)."""
    cache, q, bt, lens = _problem(34, [200, 33], 6, 2, 64, "int8")
    out, lse = O.decode_int8_qk(cache, q, bt, lens)
    ref, _ = O.decode(cache, q, bt, lens)
    d = np.abs(out - ref)
    assert 0 < d.max() < 0.1
