"""GPU parity of the fused decode step (kvq_decode_step): the split kernel writes each sequence's
new token into its last page, then attends over the context that includes it.

The cache must afterwards equal, byte for byte, the oracle's cache after kv_write of the same
tokens at their slots (position context_len - 1), and the outputs must meet the decode
tolerance against the oracle's plain definition over that cache.
"""
import numpy as np
import pytest
import torch

import decode_attention_quantized_amd as K
import oracle as O
import workloads as W
from tests.gpu_util import Pair, assert_close, bf16_dev, dev, log

pytestmark = pytest.mark.gpu

PAGE = 16


def _problem(seed, lens, Hq, Hkv, D, dtype, spare=5, extra_cols=0):
    """Caches holding every token but each sequence's last; returns the new tokens separately."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    pages = (lens + PAGE - 1) // PAGE
    nb = int(pages.sum()) + spare
    order = rng.permutation(nb).astype(np.int32)
    bt = np.full((len(lens), max(1, int(pages.max())) + extra_cols), -1, dtype=np.int32)
    pos = 0
    for s, p in enumerate(pages):
        bt[s, :p] = order[pos:pos + p]
        pos += p
    pair = Pair(dtype, nb, Hkv, D)
    mult = np.ones((Hkv, D), np.float32)
    for h in range(Hkv):
        mult[h, rng.choice(D, 4, replace=False)] = 20
    k_new = np.zeros((len(lens), Hkv, D), np.uint16)
    v_new = np.zeros((len(lens), Hkv, D), np.uint16)
    for s, L in enumerate(lens):
        k = W.f32_to_bf16_bits((rng.standard_normal((max(L, 1), Hkv, D)) * mult).astype(np.float32))
        v = W.f32_to_bf16_bits((rng.standard_normal((max(L, 1), Hkv, D)) * mult).astype(np.float32))
        k_new[s], v_new[s] = k[-1], v[-1]
        if L > 1:
            t = np.arange(L - 1)
            pair.write(k[:-1], v[:-1], (bt[s, t // PAGE] * PAGE + t % PAGE).astype(np.int32))
    q = W.f32_to_bf16_bits((rng.standard_normal((len(lens), Hq, D)) * 3).astype(np.float32))
    return pair, q, bt, lens, k_new, v_new


def _new_slots(bt, lens):
    """Slot of token L - 1 of each sequence, -1 for an empty one."""
    out = np.full(len(lens), -1, np.int32)
    for s, L in enumerate(lens):
        if L > 0:
            out[s] = bt[s, (L - 1) // PAGE] * PAGE + (L - 1) % PAGE
    return out


def _step_and_check(pair, q, bt, lens, k_new, v_new, splits, what, mcl=None, checked=False):
    mcl = max(int(lens.max()), 1) if mcl is None else mcl
    O.kv_write(pair.o, k_new, v_new, _new_slots(bt, lens))
    ref = O.decode(pair.o, q, bt, lens)
    kd, vd, qd, btd, ld = bf16_dev(k_new), bf16_dev(v_new), bf16_dev(q), dev(bt), dev(lens)
    for ns in splits:
        log(f"step {what} splits={ns}")
        # every call writes the same token again: the cache and outputs must not change
        out, lse = K.decode_step(pair.g, kd, vd, qd, btd, ld, mcl, ns, checked=checked)
        torch.cuda.synchronize()
        pair.assert_cache_equal()
        assert_close(out.cpu().numpy(), lse.cpu().numpy(), ref[0], ref[1], f"step {what} ns={ns}")


@pytest.mark.parametrize("dtype", ["int8", "bf16"])
@pytest.mark.parametrize("D,Hq,Hkv", [(256, 24, 4), (128, 32, 8), (128, 16, 1)])
def test_step_small_shapes(dtype, D, Hq, Hkv):
    """New token at in-page offsets 0, 14, 15 and others; splits from one to one page each (the
    writing wave's first page is then the new token's page)."""
    lens = [1, 15, 16, 17, 33, 100, 1000]
    pair, q, bt, lens, kn, vn = _problem(1000 + D + Hq, lens, Hq, Hkv, D, dtype)
    _step_and_check(pair, q, bt, lens, kn, vn, [1, 2, 3, 7, 0, 70], f"{dtype} D={D} Hq={Hq} Hkv={Hkv}")


def test_step_empty_sequence_writes_nothing():
    pair, q, bt, lens, kn, vn = _problem(1100, [0, 1, 37, 0], 24, 4, 256, "int8")
    _step_and_check(pair, q, bt, lens, kn, vn, [1, 4], "empty/single")


def test_step_max_context_shorter_than_table():
    """max_context_len above every context, below the table's capacity (unused table entries -1)."""
    pair, q, bt, lens, kn, vn = _problem(1200, [513, 40], 8, 2, 128, "int8", spare=40, extra_cols=10)
    _step_and_check(pair, q, bt, lens, kn, vn, [3, 0], "mcl", mcl=600)


@pytest.mark.parametrize("cid", [1, 2])
@pytest.mark.parametrize("dtype", ["int8", "bf16"])
def test_step_config(cid, dtype):
    layer = W.make_layer(cid, 0)
    cfg = layer.cfg
    pair = Pair(dtype, layer.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    pre, stp = layer.prefill_rows(), layer.step_rows()
    pair.write(layer.k[pre], layer.v[pre], layer.slots[pre])
    _step_and_check(pair, layer.q, layer.block_tables, layer.context_lens, layer.k[stp], layer.v[stp],
                    list(cfg.splits) + [0], f"config {cid} {dtype}")


def test_step_ragged_interleaved_checked():
    layer = W.make_layer(4, 0, context_lens=(40, 300, 1201, 17, 64), table_rule="interleaved")
    cfg = layer.cfg
    pair = Pair("int8", layer.num_blocks, cfg.num_kv_heads, cfg.head_dim)
    pre, stp = layer.prefill_rows(), layer.step_rows()
    pair.write(layer.k[pre], layer.v[pre], layer.slots[pre])
    _step_and_check(pair, layer.q, layer.block_tables, layer.context_lens, layer.k[stp], layer.v[stp],
                    [1, 8, 33, 0], "ragged interleaved", checked=True)


def test_step_same_as_write_then_decode():
    """The fused step and kvq_write + kvq_decode_attention give the same cache bytes and the same
    outputs bit for bit (the new token's page is read after it is written)."""
    pair, q, bt, lens, kn, vn = _problem(1300, [700, 45, 2], 24, 4, 256, "int8")
    other = K.Cache("int8", pair.g.num_blocks, 4, 256)
    for a, b in [(other.k, pair.g.k), (other.v, pair.g.v), (other.k_scales, pair.g.k_scales),
                 (other.v_scales, pair.g.v_scales)]:
        a.copy_(b)
    kd, vd, qd, btd, ld = bf16_dev(kn), bf16_dev(vn), bf16_dev(q), dev(bt), dev(lens)
    out1, lse1 = K.decode_step(pair.g, kd, vd, qd, btd, ld, 700, 5)
    K.write(other, kd, vd, dev(_new_slots(bt, lens)))
    out2, lse2 = K.decode(other, qd, btd, ld, 700, 5)
    torch.cuda.synchronize()
    for a, b in [(other.k, pair.g.k), (other.v, pair.g.v), (other.k_scales, pair.g.k_scales),
                 (other.v_scales, pair.g.v_scales)]:
        assert torch.equal(a.view(torch.int8) if a.dtype == torch.int8 else a.view(torch.int16),
                           b.view(torch.int8) if b.dtype == torch.int8 else b.view(torch.int16))
    # same kernels over the same bytes: identical results
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_step_dominant_new_key():
    """The new key is aligned with q and large: every head of its group must attend to it."""
    rng = np.random.default_rng(1400)
    pair, q, bt, lens, kn, vn = _problem(1400, [700], 24, 4, 256, "int8")
    qf = W.bf16_bits_to_f32(q)
    kn = W.f32_to_bf16_bits(np.stack([qf[0, h * 6] * 4 for h in range(4)])[None])
    vn = W.f32_to_bf16_bits(rng.standard_normal((1, 4, 256)).astype(np.float32))
    _step_and_check(pair, q, bt, lens, kn, vn, [0], "dominant")
    out, _ = K.decode_step(pair.g, bf16_dev(kn), bf16_dev(vn), bf16_dev(q), dev(bt), dev(lens), 700, 0)
    torch.cuda.synchronize()
    vhat = O.decode(pair.o, q, bt, lens)[0][0, 0]
    assert np.abs(out.cpu().numpy()[0, 0] - vhat).max() < 0.05


def test_checked_step_rejects_contract_violations():
    pair, q, bt, lens, kn, vn = _problem(1500, [40, 17], 8, 2, 128, "int8")
    kd, vd, qd, ld = bf16_dev(kn), bf16_dev(vn), bf16_dev(q), dev(lens)
    # the block receiving sequence 1's new token is also a page of sequence 0
    bt2 = bt.copy()
    bt2[0, 0] = bt[1, 1]
    # both sequences write into one block
    bt3 = bt.copy()
    bt3[0, 2] = bt[1, 1]
    for table, what in [(bt2, "read by another sequence"), (bt3, "two writers")]:
        with pytest.raises(K.KvqError) as ei:
            K.decode_step(pair.g, kd, vd, qd, dev(table), ld, 40, 2, checked=True)
        assert ei.value.status == -5, what
    bad = kn.copy()
    bad[1, 1, 3] = 0x7F80
    with pytest.raises(K.KvqError) as ei:
        K.decode_step(pair.g, bf16_dev(bad), vd, qd, dev(bt), ld, 40, 2, checked=True)
    assert ei.value.status == -5
    with pytest.raises(ValueError):
        K.decode_step(pair.g, kd[:1], vd, qd, dev(bt), ld, 40, 2)


@pytest.mark.parametrize("dtype", ["int8", "int8_head", "bf16"])
def test_step_length_above_max_context_writes_nothing(dtype):
    """A context length above max_context_len breaks the contract; the step must still not write
    that sequence's token anywhere (its output is unspecified).  The other sequences' tokens are
    written as usual: the cache equals a copy given only those tokens through kvq_write."""
    pair, q, bt, lens, kn, vn = _problem(1500, [100, 200, 37], 24, 4, 256, dtype, spare=4)
    g = pair.g
    ref = K.Cache(dtype, g.num_blocks, 4, 256)
    planes = lambda c: [t for t in (c.k, c.v, c.k_scales, c.v_scales) if t is not None]
    for a, b in zip(planes(ref), planes(g)):
        a.copy_(b)
    slots = _new_slots(bt, lens)
    slots[1] = -1  # sequence 1 (200 tokens) is above max_context_len 150: not written
    K.write(ref, bf16_dev(kn), bf16_dev(vn), dev(slots))
    K.decode_step(g, bf16_dev(kn), bf16_dev(vn), bf16_dev(q), dev(bt), dev(lens), 150, 4)
    torch.cuda.synchronize()
    for a, b in zip(planes(ref), planes(g)):
        assert torch.equal(a.view(torch.int8) if a.element_size() == 1 else a.view(torch.int16 if a.element_size() == 2 else torch.int32),
                           b.view(torch.int8) if b.element_size() == 1 else b.view(torch.int16 if b.element_size() == 2 else torch.int32))
