"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded inputs.

Cache writes must match byte for byte (codes, scales, and every untouched poisoned byte);
decode outputs must satisfy |gpu - oracle| <= 2e-3 + 1e-3 |oracle| element by element, for
every swept split count.
"""
import numpy as np
import pytest
import torch

import decode_attention_quantized_amd as K
import oracle as O
import workloads as W
from tests.gpu_util import Pair, assert_close, bf16_dev, dev, fill_from_layer, log

pytestmark = pytest.mark.gpu

PAGE = 16


def _rand_bits(rng, shape, scale=1.0):
    return W.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def _tables(rng, lens, spare=5, rule="permutation"):
    lens = np.asarray(lens, dtype=np.int32)
    pages = (lens + PAGE - 1) // PAGE
    nb = int(pages.sum()) + spare
    order = rng.permutation(nb).astype(np.int32)
    bt = np.full((len(lens), max(1, int(pages.max()))), -1, dtype=np.int32)
    pos = 0
    for s, p in enumerate(pages):
        bt[s, :p] = order[pos:pos + p]
        pos += p
    return bt, nb


def _small_problem(seed, lens, Hq, Hkv, D, dtype, aligned=False):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    bt, nb = _tables(rng, lens)
    pair = Pair(dtype, nb, Hkv, D)
    mult = np.ones((Hkv, D), np.float32)
    outl = [rng.choice(D, 4, replace=False) for _ in range(Hkv)]
    for h in range(Hkv):
        mult[h, outl[h]] = 20
    for s, L in enumerate(lens):
        if L == 0:
            continue
        t = np.arange(L)
        slots = (bt[s, t // PAGE] * PAGE + t % PAGE).astype(np.int32)
        k = W.f32_to_bf16_bits((rng.standard_normal((L, Hkv, D)) * mult).astype(np.float32))
        v = W.f32_to_bf16_bits((rng.standard_normal((L, Hkv, D)) * mult).astype(np.float32))
        pair.write(k, v, slots)
    qm = np.ones((Hq, D), np.float32)
    for hq in range(Hq):
        qm[hq, outl[hq // (Hq // Hkv)] if aligned else rng.choice(D, 4, replace=False)] = 20
    q = W.f32_to_bf16_bits((rng.standard_normal((len(lens), Hq, D)) * qm).astype(np.float32))
    return pair, q, bt, lens


def _check_decode(pair, q, bt, lens, splits, what, mcl=None):
    mcl = int(lens.max()) if mcl is None else mcl
    ref = O.decode(pair.o, q, bt, lens)
    for ns in splits:
        log(f"decode {what} splits={ns}")
        out, lse = K.decode(pair.g, bf16_dev(q), dev(bt), dev(lens), max(mcl, 1), ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref[0], ref[1], f"{what} ns={ns}")


# ------------------------------------------------------------------ kv_write

@pytest.mark.parametrize("dtype", ["int8", "bf16"])
@pytest.mark.parametrize("D", [128, 256])
def test_write_edge_slots_bitexact(dtype, D):
    """slot -1 and out-of-pool slots skipped, first/last block, offset 15, rewrite of a slot."""
    rng = np.random.default_rng(100 + D)
    Hkv, NB = 3, 9
    pair = Pair(dtype, NB, Hkv, D)
    slots = np.array([0, -1, 15, NB * 16 - 1, NB * 16, 77, -5, 16 * 4 + 15], dtype=np.int32)
    log(f"write edge slots {dtype} D={D}")
    pair.write(_rand_bits(rng, (len(slots), Hkv, D), 3), _rand_bits(rng, (len(slots), Hkv, D)), slots)
    pair.assert_cache_equal()
    # rewrite two slots with new data, including tiny, zero and saturating groups
    k2 = _rand_bits(rng, (2, Hkv, D), 1e-6)
    k2[0, 0, :32] = 0
    k2[1, 1, 32:64] = W.f32_to_bf16_bits(np.full(32, 3e38, np.float32))
    v2 = _rand_bits(rng, (2, Hkv, D), 1e4)
    pair.write(k2, v2, np.array([77, 0], dtype=np.int32))
    pair.assert_cache_equal()


@pytest.mark.parametrize("dtype", ["int8", "bf16"])
def test_write_random_bitexact(dtype):
    rng = np.random.default_rng(7)
    for D, Hkv, T in [(256, 4, 300), (128, 8, 513)]:
        NB = (T + 15) // 16 + 4
        pair = Pair(dtype, NB, Hkv, D)
        slots = rng.permutation(NB * 16)[:T].astype(np.int32)
        scale = np.exp2(rng.uniform(-20, 20, size=(T, Hkv, 1))).astype(np.float32)
        k = W.f32_to_bf16_bits((rng.standard_normal((T, Hkv, D)) * scale).astype(np.float32))
        v = W.f32_to_bf16_bits((rng.standard_normal((T, Hkv, D)) * scale).astype(np.float32))
        log(f"write random {dtype} D={D} T={T}")
        pair.write(k, v, slots)
        pair.assert_cache_equal()


def _prefill_slots(rng, nb):
    """A prefill-shaped slot map over a pool of nb blocks, in pieces with distinct blocks:
    sequences of ragged lengths filling their pages in order (so whole pages begin at every
    position of a 16-token window), a page whose run is broken by a skipped token, a page written
    in reverse order, a run of 16 consecutive slots that straddles two pages, a page with an
    out-of-pool slot in its middle, and the last block of the pool."""
    blocks = list(rng.permutation(nb - 1))
    take = lambda: int(blocks.pop())
    slots = []
    for L in (37, 16, 1, 50, 33, 18, 31, 47):
        pages = [take() for _ in range((L + PAGE - 1) // PAGE)]
        slots += [pages[t // PAGE] * PAGE + t % PAGE for t in range(L)]
    b = take()
    slots += [b * PAGE + k for k in range(PAGE) if k != 5] + [-1]
    b = take()
    slots += [b * PAGE + PAGE - 1 - k for k in range(PAGE)]
    b1, b2 = take(), take()
    slots += [b1 * PAGE + 3 + k for k in range(PAGE - 3)] + [b2 * PAGE + k for k in range(3)]
    b = take()
    slots += [b * PAGE + k if k != 9 else nb * PAGE + 9 for k in range(PAGE)]
    slots += [(nb - 1) * PAGE + k for k in range(PAGE)]
    return np.array(slots, dtype=np.int32)


@pytest.mark.parametrize("dtype", ["int8", "bf16", "int8_head"])
@pytest.mark.parametrize("D", [128, 256])
def test_write_prefill_pages_bitexact(dtype, D):
    rng = np.random.default_rng(300 + D)
    Hkv, nb = 3, 40
    slots = _prefill_slots(rng, nb)
    T = len(slots)
    pair = Pair(dtype, nb, Hkv, D)
    scale = np.exp2(rng.uniform(-12, 12, size=(T, Hkv, 1))).astype(np.float32)
    k = W.f32_to_bf16_bits((rng.standard_normal((T, Hkv, D)) * scale).astype(np.float32))
    v = W.f32_to_bf16_bits((rng.standard_normal((T, Hkv, D)) * scale).astype(np.float32))
    log(f"write prefill pages {dtype} D={D} T={T}")
    pair.write(k, v, slots)
    pair.assert_cache_equal()
    # the same rows shifted by 1 .. 15 batch positions (pages now start elsewhere in the windows)
    for shift in (1, 7, 15):
        pair2 = Pair(dtype, nb, Hkv, D)
        s2 = np.concatenate([np.full(shift, -1, np.int32), slots])
        k2 = np.concatenate([k[:shift], k])
        v2 = np.concatenate([v[:shift], v])
        log(f"write prefill pages {dtype} D={D} shift={shift}")
        pair2.write(k2, v2, s2)
        pair2.assert_cache_equal()


def _near_tie_rows(rng, T, Hkv, D, per_head):
    """bf16 rows whose quotients x / s by their own stored scale are exact half-integers (ties, to
    even) or lie within 2^-10 of one, so that the rounding decision is as close as it gets.  The
    scale follows the quantizer's rule from the row's (or 32-group's) maximum: fp32 amax / 127,
    then (q8_0) binary16 round to nearest even."""
    glen = D if per_head else 32
    out = np.zeros((T, Hkv, D), np.float32)
    for t in range(T):
        for h in range(Hkv):
            for g0 in range(0, D, glen):
                e = int(rng.integers(-12, 12))
                if rng.random() < 0.3:   # power-of-two scale: amax 127 * 2^e, exact ties (n + 1/2) 2^e
                    n = rng.integers(-127, 127, size=glen)
                    vals = (n + 0.5) * 2.0 ** e
                    vals[0] = 127 * 2.0 ** e
                else:
                    amax = float(W.bf16_bits_to_f32(W.f32_to_bf16_bits(np.array([rng.uniform(20, 127) * 2.0 ** e], np.float32)))[0])
                    d = np.float32(amax) / np.float32(127)
                    sc = np.float32(d) if per_head else np.float32(np.float16(min(d, 65504)))
                    cand = W.bf16_bits_to_f32(W.f32_to_bf16_bits(
                        rng.uniform(-amax, amax, size=16384).astype(np.float32)))
                    qt = cand / sc                                    # IEEE float32 division
                    fr = np.abs((qt - np.floor(qt)) - 0.5)
                    pick = cand[np.argsort(fr)[:glen]]
                    vals = np.concatenate([[amax], pick[:glen - 1]])
                out[t, h, g0:g0 + glen] = rng.permutation(vals)
    return W.f32_to_bf16_bits(out)


@pytest.mark.parametrize("dtype", ["int8", "int8_head"])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("T", [8, 64])
def test_write_rounding_ties_bitexact(dtype, D, T):
    """Codes at and next to rounding ties, through both writers (fewer than 16 tokens, and the
    16-token windows), against the oracle byte for byte."""
    rng = np.random.default_rng(500 + D + T)
    Hkv = 2
    nb = (T + PAGE - 1) // PAGE + 2
    k = _near_tie_rows(rng, T, Hkv, D, dtype == "int8_head")
    v = _near_tie_rows(rng, T, Hkv, D, dtype == "int8_head")
    slots = np.arange(T, dtype=np.int32) + PAGE  # whole pages from block 1 on (the windows' page path)
    pair = Pair(dtype, nb, Hkv, D)
    log(f"write rounding ties {dtype} D={D} T={T}")
    pair.write(k, v, slots)
    pair.assert_cache_equal()
    pair2 = Pair(dtype, nb, Hkv, D)
    pair2.write(k, v, rng.permutation(nb * PAGE)[:T].astype(np.int32))  # scattered: per-token stores
    pair2.assert_cache_equal()


@pytest.mark.parametrize("cid", [1, 2])
@pytest.mark.parametrize("dtype", ["int8", "bf16"])
def test_write_config_bitexact(cid, dtype):
    layer = W.make_layer(cid, 0)
    cfg = layer.cfg
    pair = Pair(dtype, layer.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    log(f"write config {cid} {dtype}")
    fill_from_layer(pair, layer)
    pair.assert_cache_equal()


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("dtype", ["int8", "bf16"])
@pytest.mark.parametrize("D,Hq,Hkv", [(256, 24, 4), (128, 32, 8), (256, 4, 4), (128, 16, 1), (256, 8, 1)])
def test_decode_small_shapes(dtype, D, Hq, Hkv):
    lens = [1, 15, 16, 17, 33, 100, 1000]
    pair, q, bt, lens = _small_problem(200 + D + Hq, lens, Hq, Hkv, D, dtype)
    _check_decode(pair, q, bt, lens, [1, 2, 3, 7, 0, 70], f"{dtype} D={D} Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("dtype", ["int8", "bf16"])
def test_decode_independent_of_kv_write(dtype):
    """Decode over a cache image made by the oracle and laid out by the test."""
    pair, q, bt, lens = _small_problem(300, [700, 45, 2], 24, 4, 256, dtype)
    pair.g.fill()
    pair.upload_oracle_cache()
    _check_decode(pair, q, bt, lens, [1, 5, 0], f"{dtype} uploaded cache")


@pytest.mark.parametrize("dtype", ["int8", "bf16"])
def test_decode_peaked_softmax(dtype):
    """Queries share their KV head's outlier channels: sharply peaked score distributions."""
    pair, q, bt, lens = _small_problem(400, [2048, 333], 24, 4, 256, dtype, aligned=True)
    _check_decode(pair, q, bt, lens, [1, 16, 0], f"{dtype} aligned outliers")


def test_decode_empty_and_single_token():
    pair, q, bt, lens = _small_problem(500, [0, 1, 37], 24, 4, 256, "int8")
    _check_decode(pair, q, bt, lens, [1, 4], "empty/single")


def test_decode_ragged_batch_interleaved_pages():
    layer = W.make_layer(4, 0, context_lens=(40, 300, 1201, 17, 64), table_rule="interleaved")
    cfg = layer.cfg
    pair = Pair("int8", layer.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    fill_from_layer(pair, layer)
    pair.assert_cache_equal()
    # (split counts that fill the merge's blocks of 8, 16, 32 and 64 splits in part, and the
    # largest count the library takes: 4096, nearly all of them empty)
    _check_decode(pair, layer.q, layer.block_tables, layer.context_lens, [1, 4, 8, 12, 20, 33, 4096, 0],
                  "ragged interleaved")


def test_write_then_decode_stream_order():
    """The step's kv_write and the decode run back to back on one stream; the new key is made
    dominant (aligned with q), so the output must be close to the new token's value."""
    rng = np.random.default_rng(600)
    D, Hq, Hkv, L = 256, 24, 4, 700
    bt, nb = _tables(rng, [L])
    pair = Pair("int8", nb, Hkv, D)
    t = np.arange(L - 1)
    pair.write(_rand_bits(rng, (L - 1, Hkv, D), 0.1), _rand_bits(rng, (L - 1, Hkv, D)),
               (bt[0, t // PAGE] * PAGE + t % PAGE).astype(np.int32))
    qf = (rng.standard_normal((1, Hq, D))).astype(np.float32)
    q = W.f32_to_bf16_bits(qf)
    knew = W.f32_to_bf16_bits(np.stack([qf[0, h * 6] * 4 for h in range(Hkv)])[None])
    vnew = _rand_bits(rng, (1, Hkv, D))
    slot = np.array([bt[0, (L - 1) // PAGE] * PAGE + (L - 1) % PAGE], dtype=np.int32)
    # write and decode with no synchronisation in between
    K.write(pair.g, bf16_dev(knew), bf16_dev(vnew), dev(slot))
    out, lse = K.decode(pair.g, bf16_dev(q), dev(bt), dev(np.array([L], np.int32)), L, 0)
    torch.cuda.synchronize()
    O.kv_write(pair.o, knew, vnew, slot)
    ref = O.decode(pair.o, q, bt, np.array([L], np.int32))
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref[0], ref[1], "write->decode")
    vhat = ref[0][0, 0]
    assert np.abs(out.cpu().numpy()[0, 0] - vhat).max() < 0.05


@pytest.mark.parametrize("cid", [1, 2])
@pytest.mark.parametrize("dtype", ["int8", "bf16"])
def test_decode_config(cid, dtype):
    layer = W.make_layer(cid, 0)
    cfg = layer.cfg
    pair = Pair(dtype, layer.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    fill_from_layer(pair, layer)
    _check_decode(pair, layer.q, layer.block_tables, layer.context_lens, list(cfg.splits) + [0],
                  f"config {cid} {dtype}")


# ------------------------------------------------------------------ checked mode

def test_checked_write_rejects_contract_violations():
    rng = np.random.default_rng(700)
    g = K.Cache("int8", 4, 2, 128).fill()
    k = bf16_dev(_rand_bits(rng, (3, 2, 128)))
    for slots, what in [([1, 5, 1], "duplicate"), ([0, 64, 2], "out of pool")]:
        with pytest.raises(K.KvqError) as ei:
            K.write(g, k, k, dev(np.array(slots, np.int32)), checked=True)
        assert ei.value.status == -5, what
    bad = _rand_bits(rng, (3, 2, 128))
    bad[1, 1, 7] = 0x7FC0
    with pytest.raises(K.KvqError):
        K.write(g, bf16_dev(bad), k, dev(np.array([0, 1, 2], np.int32)), checked=True)
    # valid call: same bytes as the fast path
    g2 = K.Cache("int8", 4, 2, 128).fill()
    sl = dev(np.array([3, -1, 9], np.int32))
    K.write(g, k, k, sl, checked=True)
    K.write(g2, k, k, sl)
    torch.cuda.synchronize()
    assert torch.equal(g.k, g2.k) and torch.equal(g.k_scales.view(torch.int16), g2.k_scales.view(torch.int16))


def test_checked_decode_rejects_contract_violations():
    pair, q, bt, lens = _small_problem(800, [40, 17], 8, 2, 128, "int8")
    qd, btd = bf16_dev(q), dev(bt)
    for L, mcl in [([41, 17], 40), ([40, -1], 40)]:
        with pytest.raises(K.KvqError) as ei:
            K.decode(pair.g, qd, btd, dev(np.array(L, np.int32)), mcl, 2, checked=True)
        assert ei.value.status == -5
    bt2 = bt.copy()
    bt2[1, 0] = pair.g.num_blocks
    with pytest.raises(K.KvqError):
        K.decode(pair.g, qd, dev(bt2), dev(lens), 40, 2, checked=True)
    out_c, lse_c = K.decode(pair.g, qd, btd, dev(lens), 40, 2, checked=True)
    out_f, lse_f = K.decode(pair.g, qd, btd, dev(lens), 40, 2)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_f) and torch.equal(lse_c, lse_f)
