"""GPU parity over GQA ratios the other tests do not reach (G = 2, 3, 5, 7, 12 query heads per KV
head): the G heads of a KV head fill a 16-row MFMA tile only partly, and with several query
tokens the (token, head) rows n_q * G straddle tile boundaries at every offset.  Plain decode
(both caches), the fused step, the per-head format and several query tokens, each against the
oracle's plain definition at |gpu - oracle| <= 2e-3 + 1e-3 |oracle|, cache bytes exact."""
import numpy as np
import pytest
import torch

import decode_attention_quantized_amd as K
import oracle as O
from tests.gpu_util import assert_close, bf16_dev, dev, log
from tests.test_gpu_mq import _check as _check_mq
from tests.test_gpu_mq import _problem as _mq_problem
from tests.test_gpu_parity import _check_decode, _small_problem
from tests.test_gpu_step import _problem as _step_problem
from tests.test_gpu_step import _step_and_check

pytestmark = pytest.mark.gpu

RATIOS = [(2, 4, 256), (3, 3, 128), (5, 2, 256), (7, 1, 128), (12, 2, 256)]  # (G, Hkv, D)


@pytest.mark.parametrize("dtype", ["int8", "bf16", "int8_head"])
@pytest.mark.parametrize("G,Hkv,D", RATIOS)
def test_decode_gqa_ratios(dtype, G, Hkv, D):
    pair, q, bt, lens = _small_problem(6000 + 10 * G + D, [1, 17, 100, 700], G * Hkv, Hkv, D, dtype)
    _check_decode(pair, q, bt, lens, [1, 5, 0], f"G={G} {dtype} D={D}")


@pytest.mark.parametrize("dtype", ["int8", "bf16", "int8_head"])
@pytest.mark.parametrize("G,Hkv,D", RATIOS)
def test_step_gqa_ratios(dtype, G, Hkv, D):
    pair, q, bt, lens, kn, vn = _step_problem(6100 + 10 * G + D, [1, 16, 33, 500], G * Hkv, Hkv, D, dtype)
    _step_and_check(pair, q, bt, lens, kn, vn, [1, 4, 0], f"G={G} {dtype} D={D}")


@pytest.mark.parametrize("G,Hkv,D", RATIOS)
@pytest.mark.parametrize("nq", [2, 3, 5, 9])
def test_several_query_tokens_gqa_ratios(G, Hkv, D, nq):
    pair, q, bt, lens = _mq_problem(6200 + 10 * G + D + nq, [nq, 40, 333, 900], G * Hkv, Hkv, D, nq)
    _check_mq(pair, q, bt, lens, [1, 3, 0], f"G={G} D={D} nq={nq}")
