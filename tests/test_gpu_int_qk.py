"""GPU parity of integer Q.K (kvq_decode_attention_int8qk): against the oracle's definition of it
(attention with the query quantized by the cache's q8_0 rule) within
|gpu - oracle| <= 2e-3 + 1e-3 |oracle|, for every swept split count.  The difference from exact
attention (the query's rounding) is reported, not bounded."""
import numpy as np
import pytest
import torch

import decode_attention_quantized_amd as K
import oracle as O
import workloads as W
from tests.gpu_util import Pair, assert_close, bf16_dev, dev, fill_from_layer, log

pytestmark = pytest.mark.gpu

PAGE = 16


def _problem(seed, lens, Hq, Hkv, D):
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
    pair = Pair("int8", nb, Hkv, D)
    mult = np.ones((Hkv, D), np.float32)
    for h in range(Hkv):
        mult[h, rng.choice(D, 4, replace=False)] = 20
    for s, L in enumerate(lens):
        if L == 0:
            continue
        t = np.arange(L)
        pair.write(W.f32_to_bf16_bits((rng.standard_normal((L, Hkv, D)) * mult).astype(np.float32)),
                   W.f32_to_bf16_bits((rng.standard_normal((L, Hkv, D)) * mult).astype(np.float32)),
                   (bt[s, t // PAGE] * PAGE + t % PAGE).astype(np.int32))
    q = W.f32_to_bf16_bits((rng.standard_normal((len(lens), Hq, D)) * 3).astype(np.float32))
    return pair, q, bt, lens


def _check(pair, q, bt, lens, splits, what):
    ref = O.decode_int8_qk(pair.o, q, bt, lens)
    exact = O.decode(pair.o, q, bt, lens)
    for ns in splits:
        log(f"int8 Q.K {what} splits={ns}")
        out, lse = K.decode(pair.g, bf16_dev(q), dev(bt), dev(lens), max(int(lens.max()), 1), ns, int_qk=True)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref[0], ref[1], f"{what} ns={ns}")
    d = np.abs(ref[0] - exact[0])
    log(f"int8 Q.K {what}: difference from exact attention: mean {d.mean():.2e}, max {d.max():.2e}")


@pytest.mark.parametrize("D,Hq,Hkv", [(256, 24, 4), (128, 32, 8), (128, 16, 1)])
def test_int_qk_small_shapes(D, Hq, Hkv):
    pair, q, bt, lens = _problem(4000 + D + Hq, [0, 1, 15, 16, 17, 33, 100, 1000], Hq, Hkv, D)
    _check(pair, q, bt, lens, [1, 3, 0, 70], f"D={D} Hq={Hq} Hkv={Hkv}")


def test_int_qk_config():
    layer = W.make_layer(2, 0)
    cfg = layer.cfg
    pair = Pair("int8", layer.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    fill_from_layer(pair, layer)
    _check(pair, layer.q, layer.block_tables, layer.context_lens, [8, 0], "hybrid-4k")


def test_int_qk_needs_q8_0_cache():
    for dtype in ("bf16", "int8_head"):
        g = K.Cache(dtype, 4, 2, 128)
        q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
        with pytest.raises(K.KvqError) as ei:
            K.decode(g, q, torch.zeros((1, 2), dtype=torch.int32, device="cuda"),
                     torch.full((1,), 20, dtype=torch.int32, device="cuda"), 20, 2, int_qk=True)
        assert ei.value.status == -2
