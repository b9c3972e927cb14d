"""GPU parity of decode with several query tokens per sequence (kvq_decode_attention_mq): the
queries are the last n_q positions of each sequence and attend causally (query token i sees
positions 0 .. L - n_q + i).  Outputs must satisfy |gpu - oracle| <= 2e-3 + 1e-3 |oracle|
against the oracle's plain definition, for every swept split count."""
import numpy as np
import pytest
import torch

import decode_attention_quantized_amd as K
import oracle as O
import workloads as W
from tests.gpu_util import Pair, assert_close, bf16_dev, dev, log

pytestmark = pytest.mark.gpu

PAGE = 16


def _problem(seed, lens, Hq, Hkv, D, nq):
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
        k = W.f32_to_bf16_bits((rng.standard_normal((L, Hkv, D)) * mult).astype(np.float32))
        v = W.f32_to_bf16_bits((rng.standard_normal((L, Hkv, D)) * mult).astype(np.float32))
        pair.write(k, v, (bt[s, t // PAGE] * PAGE + t % PAGE).astype(np.int32))
    q = W.f32_to_bf16_bits((rng.standard_normal((len(lens), nq, Hq, D)) * 3).astype(np.float32))
    return pair, q, bt, lens


def _check(pair, q, bt, lens, splits, what):
    S, nq, Hq, D = q.shape
    ref_out, ref_lse = O.decode_mq(pair.o, q, bt, lens)
    qd, btd, ld = bf16_dev(q), dev(bt), dev(lens)
    mcl = max(int(lens.max()), 1)
    for ns in splits:
        log(f"decode_mq {what} splits={ns}")
        out, lse = K.decode_mq(pair.g, qd, btd, ld, mcl, ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy().reshape(S * nq, Hq, D), lse.cpu().numpy().reshape(S * nq, Hq),
                     ref_out.reshape(S * nq, Hq, D), ref_lse.reshape(S * nq, Hq), f"{what} ns={ns}")


@pytest.mark.parametrize("D,Hq,Hkv", [(256, 24, 4), (128, 32, 8), (128, 16, 1)])
@pytest.mark.parametrize("nq", [2, 3, 5, 16])
def test_mq_small_shapes(D, Hq, Hkv, nq):
    """Query tokens that straddle page boundaries, contexts shorter than n_q, row tiles from one
    (n_q * G <= 16) to several."""
    lens = [nq, 15, 16, 17, 40, 333, max(nq - 1, 1)]
    pair, q, bt, lens = _problem(2000 + D + Hq + nq, lens, Hq, Hkv, D, nq)
    _check(pair, q, bt, lens, [1, 3, 0, 40], f"D={D} Hq={Hq} Hkv={Hkv} nq={nq}")


def test_mq_one_token_is_decode():
    pair, q, bt, lens = _problem(2100, [700, 45, 2], 24, 4, 256, 1)
    out1, lse1 = K.decode_mq(pair.g, bf16_dev(q), dev(bt), dev(lens), 700, 5)
    out2, lse2 = K.decode(pair.g, bf16_dev(q[:, 0]), dev(bt), dev(lens), 700, 5)
    torch.cuda.synchronize()
    assert torch.equal(out1[:, 0], out2) and torch.equal(lse1[:, 0], lse2)


def test_mq_long_context_interleaved():
    """A 4-sequence batch with interleaved pages, 4 and 8 query tokens, at several split counts."""
    layer = W.make_layer(4, 0, context_lens=(40, 300, 3001, 17), table_rule="interleaved")
    cfg = layer.cfg
    pair = Pair("int8", layer.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    rows = np.arange(layer.k.shape[0])
    pair.write(layer.k[rows], layer.v[rows], layer.slots[rows])
    rng = np.random.default_rng(2200)
    for nq in (4, 8):
        q = W.f32_to_bf16_bits(rng.standard_normal((layer.S, nq, cfg.num_q_heads, cfg.head_dim)).astype(np.float32))
        _check(pair, q, layer.block_tables, layer.context_lens, [1, 8, 0], f"interleaved nq={nq}")


def test_mq_rejects_bad_arguments():
    g = K.Cache("bf16", 8, 2, 128)
    q = torch.zeros((1, 2, 4, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((1, 4), dtype=torch.int32, device="cuda")
    cl = torch.full((1,), 20, dtype=torch.int32, device="cuda")
    with pytest.raises(K.KvqError) as ei:
        K.decode_mq(g, q, bt, cl, 20, 2)
    assert ei.value.status == -2  # several query tokens need the INT8 cache
    g8 = K.Cache("int8", 8, 2, 128)
    with pytest.raises(K.KvqError) as ei:
        K.decode_mq(g8, torch.zeros((1, 65537, 4, 128), dtype=torch.bfloat16, device="cuda"), bt, cl, 20, 2)
    assert ei.value.status == -1


@pytest.mark.parametrize("nq", [11, 40, 100, 257])
def test_prompt_sections(nq):
    """Runs of query tokens longer than one workgroup's 64 rows (a prompt section over the cache):
    cut into chunks, each attending over the keys up to its own last token."""
    pair, q, bt, lens = _problem(2300 + nq, [nq, nq + 5, 700, 1500], 24, 4, 256, nq)
    _check(pair, q, bt, lens, [1, 4, 0], f"prompt section nq={nq}")


def test_prompt_section_dense_geometry():
    pair, q, bt, lens = _problem(2400, [300, 1000], 32, 8, 128, 64)
    _check(pair, q, bt, lens, [2, 0], "prompt section G=4 D=128 nq=64")


@pytest.mark.parametrize("D,Hq,Hkv,nq", [(256, 24, 4, 4), (256, 24, 4, 8), (256, 24, 4, 10), (128, 32, 8, 5),
                                         (128, 32, 8, 9), (128, 16, 1, 3)])
def test_mq_short_splits(D, Hq, Hkv, nq):
    """Splits of one to three pages.  In the two-tile workgroup (4 waves per tile) and the
    single-chunk one (two page groups) some waves or a whole group then hold only pages past the
    split, and the first query tokens' rows have no keys in the later splits: the folds inside
    the workgroup must give those parts weight 0."""
    lens = [nq, nq + 15, 40, 48, 100, 129]
    pair, q, bt, lens = _problem(2500 + D + Hq + nq, lens, Hq, Hkv, D, nq)
    mp = (int(lens.max()) + PAGE - 1) // PAGE  # pages of the longest sequence
    _check(pair, q, bt, lens, [mp, (mp + 1) // 2, (mp + 2) // 3, 0], f"short splits D={D} Hq={Hq} Hkv={Hkv} nq={nq}")
