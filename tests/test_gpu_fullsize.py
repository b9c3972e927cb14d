"""GPU parity at the full sizes of the long-context, mixed-batch and dense-8B workloads (one
layer each), in the launch configuration the benchmark times (the fused step at the split count chosen from the
batch's lengths): whole-cache byte comparison, and every output row against the oracle, then for
each swept split count and both automatic choices."""
import numpy as np
import pytest
import torch

import decode_attention_quantized_amd as K
import oracle as O
import workloads as W
from tests.gpu_util import Pair, assert_close, bf16_dev, dev, fill_from_layer, log

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cid", [3, 4, 5])
def test_fullsize_int8(cid):
    log(f"config {cid}: generating")
    layer = W.make_layer(cid, 0)
    cfg = layer.cfg
    pair = Pair("int8", layer.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    log(f"config {cid}: writing {int(layer.context_lens.sum())} tokens")
    pre, stp = layer.prefill_rows(), layer.step_rows()
    pair.write(layer.k[pre], layer.v[pre], layer.slots[pre])
    O.kv_write(pair.o, layer.k[stp], layer.v[stp], layer.slots[stp])
    mcl = int(layer.context_lens.max())
    log(f"config {cid}: oracle decode")
    ref = O.decode(pair.o, layer.q, layer.block_tables, layer.context_lens)
    qd, btd, ld = bf16_dev(layer.q), dev(layer.block_tables), dev(layer.context_lens)
    # the benchmarked step: the new tokens written by the split kernel, the split count from the lengths
    log(f"config {cid}: fused decode step")
    ns_bench = K.choose_num_splits_lengths(pair.g, layer.context_lens, cfg.num_q_heads)
    out, lse = K.decode_step(pair.g, bf16_dev(layer.k[stp]), bf16_dev(layer.v[stp]), qd, btd, ld, mcl, ns_bench)
    torch.cuda.synchronize()
    pair.assert_cache_equal()
    assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref[0], ref[1], f"config {cid} fused step")
    # every swept count, the maximum-length choice (0) and the lengths-aware one the benchmark uses
    for ns in list(cfg.splits) + [0, K.choose_num_splits_lengths(pair.g, layer.context_lens, cfg.num_q_heads)]:
        log(f"config {cid}: decode splits={ns}")
        out, lse = K.decode(pair.g, qd, btd, ld, mcl, ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref[0], ref[1], f"config {cid} ns={ns}")


def test_fullsize_bf16_long_context():
    layer = W.make_layer(3, 0)
    cfg = layer.cfg
    pair = Pair("bf16", layer.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    log("config 3 bf16: writing")
    fill_from_layer(pair, layer)
    pair.assert_cache_equal()
    ref = O.decode(pair.o, layer.q, layer.block_tables, layer.context_lens)
    for ns in (32, 0):
        log(f"config 3 bf16: decode splits={ns}")
        out, lse = K.decode(pair.g, bf16_dev(layer.q), dev(layer.block_tables), dev(layer.context_lens),
                            int(layer.context_lens.max()), ns)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref[0], ref[1], f"config 3 bf16 ns={ns}")


def _mq_queries(n, Hq, D, seed):
    """Seeded bf16 queries [1][n][Hq][D] with the workloads' x20 outlier channels."""
    rng = np.random.default_rng(seed)
    mult = np.ones((Hq, D), np.float32)
    for h in range(Hq):
        mult[h, rng.choice(D, 4, replace=False)] = 20
    return W.f32_to_bf16_bits((rng.standard_normal((1, n, Hq, D)) * mult).astype(np.float32))


@pytest.mark.parametrize("nq,sample,context", [(2, None, None), (4, None, None), (8, None, None), (2048, 24, None),
                                                (65536, 24, 66560)])
def test_fullsize_several_query_tokens(nq, sample, context):
    """The long-context layer with n_q query tokens at the end of the sequence, in the launch
    configuration the benchmark times (automatic split count): 2, 4 and 8 tokens (verification
    steps; one 16-row tile, two tiles, and the two-page-group form of four tiles) and a 2048-token
    prompt section; and the largest n_q the library takes, 65536, over a 66560-token sequence.
    Every row of the 2-, 4- and 8-token decodes, and every head of a seeded sample of the longer
    runs' query tokens (first and last included), against the oracle: query token i of n attends to
    the first L - n + i + 1 keys."""
    layer = W.make_layer(3, 0) if context is None else W.make_layer(3, 0, context_lens=(context,))
    cfg = layer.cfg
    Hq, D = cfg.num_q_heads, cfg.head_dim
    pair = Pair("int8", layer.num_blocks, cfg.num_kv_heads, D)
    log(f"n_q {nq}: writing")
    fill_from_layer(pair, layer)
    L = int(layer.context_lens[0])
    q = _mq_queries(nq, Hq, D, 100 + nq)
    ns = K.choose_num_splits_mq(pair.g, 1, nq, Hq, L)
    log(f"n_q {nq}: decode_mq at {ns} splits")
    out, lse = K.decode_mq(pair.g, bf16_dev(q), dev(layer.block_tables), dev(layer.context_lens), L, 0)
    torch.cuda.synchronize()
    if sample is None:
        toks = np.arange(nq)
    else:
        rng = np.random.default_rng(nq)
        toks = np.unique(np.concatenate([[0, nq - 1], rng.choice(nq, sample - 2, replace=False)]))
    lens = (L - nq + 1 + toks).astype(np.int32)
    log(f"n_q {nq}: oracle over {len(toks)} query tokens")
    ref, ref_lse = O.decode(pair.o, np.ascontiguousarray(q[0, toks]), np.repeat(layer.block_tables, len(toks), axis=0),
                            lens)
    assert_close(out.cpu().numpy()[0, toks], lse.cpu().numpy()[0, toks], ref, ref_lse,
                 f"long-context layer, {nq} query tokens, {ns} splits")
