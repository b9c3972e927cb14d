"""GPU parity of the per-head INT8 format (one fp32 scale per token and KV head): cache writes
bit-exact against the oracle (codes and scale bits, every untouched poisoned byte), decode,
the fused step and several query tokens within |gpu - oracle| <= 2e-3 + 1e-3 |oracle|."""
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


@pytest.mark.parametrize("D", [128, 256])
def test_write_bitexact(D):
    rng = np.random.default_rng(3000 + D)
    Hkv, NB = 3, 9
    pair = Pair("int8_head", NB, Hkv, D)
    slots = np.array([0, -1, 15, NB * 16 - 1, NB * 16, 77, -5, 16 * 4 + 15], dtype=np.int32)
    log(f"per-head write edge slots D={D}")
    k = _rand_bits(rng, (len(slots), Hkv, D), 3)
    k[0, 0] = 0                                                       # zero row
    k[2, 1] = W.f32_to_bf16_bits(np.full(D, 3e38, np.float32))        # saturating row
    k[3, 2] = _rand_bits(rng, (D,), 1e-30)                            # tiny row (fp32 scale far below f16)
    pair.write(k, _rand_bits(rng, (len(slots), Hkv, D), 1e4), slots)
    pair.assert_cache_equal()
    for T in (1, 300):
        sl = rng.permutation(NB * 16)[:min(T, NB * 16)].astype(np.int32)
        scale = np.exp2(rng.uniform(-40, 40, size=(len(sl), Hkv, 1))).astype(np.float32)
        pair.write(W.f32_to_bf16_bits((rng.standard_normal((len(sl), Hkv, D)) * scale).astype(np.float32)),
                   W.f32_to_bf16_bits((rng.standard_normal((len(sl), Hkv, D)) * scale).astype(np.float32)), sl)
        pair.assert_cache_equal()


def _problem(seed, lens, Hq, Hkv, D, vscale=1.0):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    pages = (lens + PAGE - 1) // PAGE
    nb = int(pages.sum()) + 5
    order = rng.permutation(nb).astype(np.int32)
    bt = np.full((len(lens), max(1, int(pages.max()))), -1, dtype=np.int32)
    pos = 0
    for s, p in enumerate(pages):
        bt[s, :p] = order[pos:pos + p]
        pos += p
    pair = Pair("int8_head", nb, Hkv, D)
    mult = np.ones((Hkv, D), np.float32)
    for h in range(Hkv):
        mult[h, rng.choice(D, 4, replace=False)] = 20
    for s, L in enumerate(lens):
        if L == 0:
            continue
        t = np.arange(L)
        # per-token magnitudes spread over many binades: exercises the running V-scale exponent
        mag = np.exp2(rng.uniform(-8, 8, size=(L, 1, 1))).astype(np.float32) * vscale
        pair.write(W.f32_to_bf16_bits((rng.standard_normal((L, Hkv, D)) * mult).astype(np.float32)),
                   W.f32_to_bf16_bits((rng.standard_normal((L, Hkv, D)) * mult * mag).astype(np.float32)),
                   (bt[s, t // PAGE] * PAGE + t % PAGE).astype(np.int32))
    q = W.f32_to_bf16_bits((rng.standard_normal((len(lens), Hq, D)) * 3).astype(np.float32))
    return pair, q, bt, lens


@pytest.mark.parametrize("D,Hq,Hkv", [(256, 24, 4), (128, 32, 8), (128, 16, 1)])
def test_decode_small_shapes(D, Hq, Hkv):
    pair, q, bt, lens = _problem(3100 + D + Hq, [1, 15, 16, 17, 33, 100, 1000], Hq, Hkv, D)
    ref = O.decode(pair.o, q, bt, lens)
    for ns in (1, 2, 7, 0, 70):
        log(f"per-head decode D={D} Hq={Hq} Hkv={Hkv} splits={ns}")
        out, lse = K.decode(pair.g, bf16_dev(q), dev(bt), dev(lens), int(lens.max()), ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref[0], ref[1], f"per-head D={D} ns={ns}")


@pytest.mark.parametrize("vscale", [1e-30, 1e30])
def test_decode_extreme_value_scales(vscale):
    """V rows whose fp32 scales lie far outside the f16 range."""
    pair, q, bt, lens = _problem(3200, [300, 40], 24, 4, 256, vscale=vscale)
    ref = O.decode(pair.o, q, bt, lens)
    out, lse = K.decode(pair.g, bf16_dev(q), dev(bt), dev(lens), 300, 0)
    torch.cuda.synchronize()
    # compare relative to the value scale (the tolerance is stated for O(1) values)
    assert_close(out.cpu().numpy() / vscale, lse.cpu().numpy(), ref[0] / vscale, ref[1], f"vscale={vscale}")


def test_fused_step_and_several_query_tokens():
    pair, q, bt, lens = _problem(3300, [700, 45, 2], 24, 4, 256)
    # step: the last token of every sequence is rewritten by the split kernel with new values
    rng = np.random.default_rng(3301)
    kn, vn = _rand_bits(rng, (3, 4, 256), 2), _rand_bits(rng, (3, 4, 256), 2)
    slots = np.array([bt[s, (L - 1) // PAGE] * PAGE + (L - 1) % PAGE for s, L in enumerate(lens)], np.int32)
    O.kv_write(pair.o, kn, vn, slots)
    ref = O.decode(pair.o, q, bt, lens)
    for ns in (1, 5, 0, 44):
        log(f"per-head step splits={ns}")
        out, lse = K.decode_step(pair.g, bf16_dev(kn), bf16_dev(vn), bf16_dev(q), dev(bt), dev(lens), 700, ns)
        torch.cuda.synchronize()
        pair.assert_cache_equal()
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref[0], ref[1], f"per-head step ns={ns}")
    qm = W.f32_to_bf16_bits(rng.standard_normal((3, 4, 24, 256)).astype(np.float32))
    refm = O.decode_mq(pair.o, qm, bt, lens)
    for ns in (1, 0):
        out, lse = K.decode_mq(pair.g, bf16_dev(qm), dev(bt), dev(lens), 700, ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().reshape(12, 24, 256), lse.cpu().numpy().reshape(12, 24),
                     refm[0].reshape(12, 24, 256), refm[1].reshape(12, 24), f"per-head mq ns={ns}")


@pytest.mark.parametrize("D,Hq,Hkv,nq", [(256, 24, 4, 8), (256, 24, 4, 23), (128, 32, 8, 40)])
def test_four_tile_workgroups_and_prompt_sections(D, Hq, Hkv, nq):
    """Runs of query tokens that fill 4-tile workgroups (one wave per tile, partials stored from
    registers) and, beyond 64 / G tokens, several query chunks, on the per-head format."""
    pair, _, bt, lens = _problem(3400 + nq, [nq, nq + 3, 300, 900], Hq, Hkv, D)
    rng = np.random.default_rng(3401 + nq)
    qm = _rand_bits(rng, (len(lens), nq, Hq, D), 2)
    ref = O.decode_mq(pair.o, qm, bt, lens)
    S = len(lens)
    for ns in (1, 3, 0):
        log(f"per-head mq D={D} nq={nq} splits={ns}")
        out, lse = K.decode_mq(pair.g, bf16_dev(qm), dev(bt), dev(lens), int(lens.max()), ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().reshape(S * nq, Hq, D), lse.cpu().numpy().reshape(S * nq, Hq),
                     ref[0].reshape(S * nq, Hq, D), ref[1].reshape(S * nq, Hq), f"per-head mq D={D} nq={nq} ns={ns}")


@pytest.mark.parametrize("cid", [2, 3])
def test_config(cid):
    layer = W.make_layer(cid, 0)
    cfg = layer.cfg
    pair = Pair("int8_head", layer.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    log(f"per-head config {cid}: writing")
    fill_from_layer(pair, layer)
    pair.assert_cache_equal()
    ref = O.decode(pair.o, layer.q, layer.block_tables, layer.context_lens)
    for ns in (list(cfg.splits)[-2:] + [0]):
        log(f"per-head config {cid} splits={ns}")
        out, lse = K.decode(pair.g, bf16_dev(layer.q), dev(layer.block_tables), dev(layer.context_lens),
                            int(layer.context_lens.max()), ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref[0], ref[1], f"per-head config {cid} ns={ns}")
