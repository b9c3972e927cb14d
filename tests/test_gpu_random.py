"""Seeded random GPU parity.

Shapes, GQA ratios, head dims, batch lengths (empty, one token, page boundaries, ragged), split
counts and query-token counts are drawn from one seeded generator. Each case runs one entry
point through the C ABI, on a cache filled through kvq_write:
- decode: kvq_decode_attention, for the q8_0, BF16 and per-head caches;
- step: kvq_decode_step, whose split kernel writes each sequence's last token;
- mq: kvq_decode_attention_mq, several query tokens, for the q8_0 and per-head caches;
- int8qk: kvq_decode_attention_int8qk (q8_0), against the oracle's quantized-query definition;
- noalloc: kvq_decode_step_noalloc, the fused step with the library's own partials buffer (shapes
  drawn so that the partials fit it).
A last group draws wide batches (32 to 128 sequences of up to 300 tokens).

Each case is compared with the oracle's plain definition over the oracle's own cache, which was
written from the same rows: |gpu - oracle| <= 2e-3 + 1e-3 |oracle| for every output and lse
element. Cache bytes must equal the oracle's after every write, including the step's.
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
NUM_CASES = 120


def _draw_cases():
    rng = np.random.default_rng(20261202)
    cases = []
    for i in range(NUM_CASES):
        op = ("decode", "step", "mq")[i % 3]
        D = int(rng.choice([128, 256]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.integers(1, 17 if op != "mq" else 9))
        S = int(rng.integers(1, 6))
        lens = []
        for _ in range(S):
            kind = rng.integers(0, 5)
            if kind == 0:
                lens.append(int(rng.choice([0, 1, 2])))
            elif kind == 1:
                lens.append(int(PAGE * rng.integers(1, 40) + rng.choice([-1, 0, 1])))
            else:
                lens.append(int(rng.integers(3, 2000)))
        if op == "step":
            dtype = str(rng.choice(["int8", "bf16", "int8_head"]))
        elif op == "mq":
            dtype = str(rng.choice(["int8", "int8_head"]))
        else:
            dtype = str(rng.choice(["int8", "bf16", "int8_head"]))
        splits = int(rng.choice([0, 0, 1, 2, 3, 5, 9, 16, 33, 70]))
        nq = int(rng.choice([2, 3, 4, 6, 8, 11, 16, 33])) if op == "mq" else 1
        cases.append(dict(i=i, seed=int(rng.integers(1 << 30)), op=op, D=D, Hkv=Hkv, Hq=G * Hkv, lens=lens,
                          dtype=dtype, splits=splits, nq=nq))
    return cases


def _draw_extra_cases():
    rng = np.random.default_rng(20261203)
    cases = []
    for i in range(NUM_EXTRA):
        op = ("int8qk", "noalloc")[i % 2]
        D = int(rng.choice([128, 256]))
        Hkv = int(rng.choice([1, 2, 4]))
        G = int(rng.integers(1, 9))
        S = int(rng.integers(1, 4))
        lens = [int(rng.choice([0, 1, 15, 16, 17])) if rng.integers(0, 4) == 0 else int(rng.integers(3, 1800))
                for _ in range(S)]
        dtype = "int8" if op == "int8qk" else str(rng.choice(["int8", "bf16", "int8_head"]))
        splits = int(rng.choice([0, 1, 3, 7, 16]))
        cases.append(dict(i=NUM_CASES + i, seed=int(rng.integers(1 << 30)), op=op, D=D, Hkv=Hkv, Hq=G * Hkv,
                          lens=lens, dtype=dtype, splits=splits, nq=1))
    return cases


def _draw_batch_cases():
    """Wide batches: 32 to 128 sequences of 0 to 300 tokens."""
    rng = np.random.default_rng(20261204)
    cases = []
    for i in range(NUM_BATCH):
        op = ("decode", "step", "mq")[i % 3]
        D = int(rng.choice([128, 256]))
        Hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.integers(1, 9))
        S = int(rng.integers(32, 129))
        lens = [int(x) for x in rng.integers(0, 301, S)]
        dtype = str(rng.choice(["int8", "int8_head"] if op == "mq" else ["int8", "bf16", "int8_head"]))
        splits = int(rng.choice([0, 1, 2, 5]))
        nq = int(rng.choice([2, 4, 9])) if op == "mq" else 1
        cases.append(dict(i=NUM_CASES + NUM_EXTRA + i, seed=int(rng.integers(1 << 30)), op=op, D=D, Hkv=Hkv,
                          Hq=G * Hkv, lens=lens, dtype=dtype, splits=splits, nq=nq))
    return cases


NUM_EXTRA = 30
NUM_BATCH = 9
CASES = _draw_cases() + _draw_extra_cases() + _draw_batch_cases()


def _build(seed, lens, Hq, Hkv, D, dtype, nq):
    """Caches (GPU and oracle) with tokens 0 .. L - 2 of each sequence written; the last token's
    rows and the queries are returned."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    pages = (lens + PAGE - 1) // PAGE
    nb = int(pages.sum()) + 3
    order = rng.permutation(nb).astype(np.int32)
    bt = np.full((len(lens), max(1, int(pages.max()))), -1, dtype=np.int32)
    pos = 0
    for s, p in enumerate(pages):
        bt[s, :p] = order[pos:pos + p]
        pos += p
    pair = Pair(dtype, nb, Hkv, D)
    mult = np.ones((Hkv, D), np.float32)
    for h in range(Hkv):
        mult[h, rng.choice(D, 4, replace=False)] = 20
    last = np.zeros((2, len(lens), Hkv, D), np.uint16)
    for s, L in enumerate(lens):
        k = W.f32_to_bf16_bits((rng.standard_normal((max(L, 1), Hkv, D)) * mult).astype(np.float32))
        v = W.f32_to_bf16_bits((rng.standard_normal((max(L, 1), Hkv, D)) * mult).astype(np.float32))
        last[0, s], last[1, s] = k[-1], v[-1]
        if L > 1:
            t = np.arange(L - 1)
            pair.write(k[:-1], v[:-1], (bt[s, t // PAGE] * PAGE + t % PAGE).astype(np.int32))
    shape = (len(lens), Hq, D) if nq == 1 else (len(lens), nq, Hq, D)
    q = W.f32_to_bf16_bits((rng.standard_normal(shape) * 3).astype(np.float32))
    return pair, q, bt, lens, last


def _last_slots(bt, lens):
    out = np.full(len(lens), -1, np.int32)
    for s, L in enumerate(lens):
        if L > 0:
            out[s] = bt[s, (L - 1) // PAGE] * PAGE + (L - 1) % PAGE
    return out


@pytest.mark.parametrize("case", CASES, ids=[f"{c['i']}-{c['op']}-{c['dtype']}" for c in CASES])
def test_random_case(case):
    c = case
    what = (f"case {c['i']}: {c['op']} {c['dtype']} D={c['D']} Hq={c['Hq']} Hkv={c['Hkv']} lens={c['lens']} "
            f"splits={c['splits']} nq={c['nq']}")
    log(what)
    pair, q, bt, lens, last = _build(c["seed"], c["lens"], c["Hq"], c["Hkv"], c["D"], c["dtype"], c["nq"])
    mcl = max(int(lens.max()), 1)
    slots = _last_slots(bt, lens)
    if c["op"] == "step":
        O.kv_write(pair.o, last[0], last[1], slots)
        out, lse = K.decode_step(pair.g, bf16_dev(last[0]), bf16_dev(last[1]), bf16_dev(q), dev(bt), dev(lens), mcl,
                                 c["splits"])
        ref = O.decode(pair.o, q, bt, lens)
    elif c["op"] == "noalloc":
        O.kv_write(pair.o, last[0], last[1], slots)
        out = torch.empty((len(lens), c["Hq"], c["D"]), dtype=torch.float32, device="cuda")
        lse = torch.empty((len(lens), c["Hq"]), dtype=torch.float32, device="cuda")
        K.decode_step_noalloc(pair.g, bf16_dev(last[0]), bf16_dev(last[1]), bf16_dev(q), dev(bt), dev(lens), mcl,
                              c["splits"], out=out, lse=lse)
        ref = O.decode(pair.o, q, bt, lens)
    else:
        pair.write(last[0], last[1], slots)
        if c["op"] == "mq":
            out, lse = K.decode_mq(pair.g, bf16_dev(q), dev(bt), dev(lens), mcl, c["splits"])
            ref = O.decode_mq(pair.o, q, bt, lens)
        elif c["op"] == "int8qk":
            out, lse = K.decode(pair.g, bf16_dev(q), dev(bt), dev(lens), mcl, c["splits"], int_qk=True)
            ref = O.decode_int8_qk(pair.o, q, bt, lens)
        else:
            out, lse = K.decode(pair.g, bf16_dev(q), dev(bt), dev(lens), mcl, c["splits"])
            ref = O.decode(pair.o, q, bt, lens)
    torch.cuda.synchronize()
    pair.assert_cache_equal()
    S, Hq, D = len(lens), c["Hq"], c["D"]
    rows = S * c["nq"]
    assert_close(out.cpu().numpy().reshape(rows, Hq, D), lse.cpu().numpy().reshape(rows, Hq),
                 ref[0].reshape(rows, Hq, D), ref[1].reshape(rows, Hq), what)
