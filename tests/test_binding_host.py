"""The Python binding's argument checks (no GPU): tensors in host memory, on which a kernel would
fault, and output buffers of the wrong shape or type are refused before the library is called."""
import pytest
import torch

import decode_attention_quantized_amd as K


def _host_problem():
    cache = K.Cache("int8", 4, 1, 128, device="cpu")
    q = torch.zeros((1, 2, 128), dtype=torch.bfloat16)
    bt = torch.zeros((1, 4), dtype=torch.int32)
    cl = torch.full((1,), 10, dtype=torch.int32)
    return cache, q, bt, cl


def test_host_tensors_are_refused():
    cache, q, bt, cl = _host_problem()
    kv = torch.zeros((1, 1, 128), dtype=torch.bfloat16)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    calls = {
        "write": lambda: K.write(cache, kv, kv, torch.zeros(1, dtype=torch.int32)),
        "decode": lambda: K.decode(cache, q, bt, cl, 10, 1),
        "decode_mq": lambda: K.decode_mq(cache, q[:, None], bt, cl, 10, 1),
        "decode_step": lambda: K.decode_step(cache, kv, kv, q, bt, cl, 10, 1),
        "decode_partials": lambda: K.decode_partials(cache, q, bt, cl, 10, 1, ws),
        "decode_merge": lambda: K.decode_merge(cache, cl, 10, 1, 2, 1, ws, torch.zeros((1, 2, 128))),
    }
    for name, call in calls.items():
        with pytest.raises(ValueError, match="GPU"):
            call()


def test_output_buffers_are_checked():
    cache, q, bt, cl = _host_problem()
    with pytest.raises(ValueError, match="out must be"):
        K.decode(cache, q, bt, cl, 10, 1, out=torch.zeros((1, 2, 64)))
    with pytest.raises(ValueError, match="out must be"):
        K.decode(cache, q, bt, cl, 10, 1, out=torch.zeros((1, 2, 128), dtype=torch.float16))
    with pytest.raises(ValueError, match="lse must be"):
        K.decode(cache, q, bt, cl, 10, 1, lse=torch.zeros((2, 1)))
    with pytest.raises(ValueError, match="out must be"):
        K.decode_mq(cache, q[:, None], bt, cl, 10, 1, out=torch.zeros((1, 2, 128)))
    with pytest.raises(ValueError, match="workspace"):
        K.decode(cache, q, bt, cl, 10, 1, workspace=torch.zeros((64, 64), dtype=torch.uint8).t())


def test_partials_and_merge_check_their_inputs():
    # the library sizes its Q reads from the cache's head_dim and reads int32 tables: a smaller D,
    # 64-bit tables or lengths, or a strided tensor must be refused before the library is called
    cache, q, bt, cl = _host_problem()
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="head_dim"):
        K.decode_partials(cache, torch.zeros((1, 2, 64), dtype=torch.bfloat16), bt, cl, 10, 1, ws)
    with pytest.raises(ValueError, match="head_dim"):
        K.decode_partials(cache, torch.zeros((1, 128, 2), dtype=torch.bfloat16).transpose(1, 2), bt, cl, 10, 1, ws)
    with pytest.raises(ValueError, match="int32"):
        K.decode_partials(cache, q, bt.to(torch.int64), cl, 10, 1, ws)
    with pytest.raises(ValueError, match="int32"):
        K.decode_partials(cache, q, bt, cl.to(torch.int64), 10, 1, ws)
    with pytest.raises(ValueError, match="required"):
        K.decode_partials(cache, q, torch.zeros((1, 8), dtype=torch.int32)[:, ::2], cl, 10, 1, ws)
    with pytest.raises(ValueError, match="context_lens"):
        K.decode_merge(cache, cl.to(torch.int64), 10, 1, 2, 1, ws, torch.zeros((1, 2, 128)))
    with pytest.raises(ValueError, match="context_lens"):
        K.decode_merge(cache, torch.zeros(2, dtype=torch.int32), 10, 1, 2, 1, ws, torch.zeros((1, 2, 128)))
    with pytest.raises(ValueError, match="out must be"):
        K.decode_merge(cache, cl, 10, 1, 2, 1, ws, torch.zeros((1, 2, 64)))


def test_noalloc_step_checks_its_inputs():
    cache, q, bt, cl = _host_problem()
    kv = torch.zeros((1, 1, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must be given"):
        K.decode_step_noalloc(cache, kv, kv, q, bt, cl, 10, 1, out=None)
    with pytest.raises(ValueError, match="int32"):
        K.decode_step_noalloc(cache, kv, kv, q, bt.to(torch.int64), cl, 10, 1, out=torch.zeros((1, 2, 128)))
    with pytest.raises(ValueError, match="GPU"):
        K.decode_step_noalloc(cache, kv, kv, q, bt, cl, 10, 1, out=torch.zeros((1, 2, 128)))


def test_split_count_from_lengths_checks_its_input():
    # (refused before the library is called; the values are pinned through the C-ABI)
    cache, q, bt, cl = _host_problem()
    with pytest.raises(ValueError, match="lengths"):
        K.choose_num_splits_lengths(cache, [512, -1], 2)
    with pytest.raises(ValueError, match="lengths"):
        K.choose_num_splits_lengths(cache, [], 2)
