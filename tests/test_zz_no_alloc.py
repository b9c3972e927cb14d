"""kvq_decode_step_noalloc (the step without a workspace, for callers that cannot allocate) against
kvq_decode_step on the same inputs: two calls in a row through the C ABI, the second smaller than
the first, each compared element by element with the workspace form at the same split count."""
import numpy as np
import pytest
import torch

import decode_attention_quantized_amd as K
import oracle as O
from tests.gpu_util import assert_close, log
from tests.test_gpu_step import _problem

pytestmark = pytest.mark.gpu


def _run_both(seed, lens, Hq, Hkv, D, ns):
    pair, q, bt, lens, k_new, v_new = _problem(seed, lens, Hq, Hkv, D, "int8")
    g = pair.g
    S = len(lens)
    mcl = int(max(lens))
    dev = lambda x, dt=None: torch.from_numpy(np.ascontiguousarray(x)).cuda() if dt is None else \
        torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(dt).cuda()
    qd, kd, vd = dev(q, torch.bfloat16), dev(k_new, torch.bfloat16), dev(v_new, torch.bfloat16)
    btd, lensd = dev(bt), dev(lens)
    out_ws, lse_ws = K.decode_step(g, kd, vd, qd, btd, lensd, mcl, ns)
    out_na = torch.full((S, Hq, D), float("nan"), dtype=torch.float32, device="cuda")
    lse_na = torch.full((S, Hq), float("nan"), dtype=torch.float32, device="cuda")
    K.decode_step_noalloc(g, kd, vd, qd, btd, lensd, mcl, ns, out=out_na, lse=lse_na)
    torch.cuda.synchronize()
    a, b = out_ws.cpu().numpy(), out_na.cpu().numpy()
    la, lb = lse_ws.cpu().numpy(), lse_na.cpu().numpy()
    log(f"no-alloc step S={S} lens {list(lens)[:4]} ns {ns}: max |diff| {np.abs(a - b).max():.3e}")
    assert_close(b, lb, a.astype(np.float64), la.astype(np.float64), "no-alloc vs workspace step")
    assert np.array_equal(a, b) and np.array_equal(la, lb)  # same kernels, same split count
    # and both against the oracle over the cache that now holds the new tokens
    slots = np.array([bt[s, (L - 1) // 16] * 16 + (L - 1) % 16 for s, L in enumerate(lens)], np.int32)
    O.kv_write(pair.o, k_new, v_new, slots)
    ref, ref_lse = O.decode(pair.o, q, bt, lens)
    assert_close(b, lb, ref, ref_lse, "no-alloc vs oracle")


def test_noalloc_matches_workspace_step_twice():
    # first call: 3 sequences up to 3000 tokens, 24/4 heads, D 256; second: smaller (1 sequence, D 128)
    _run_both(11, [3000, 700, 1], 24, 4, 256, 0)
    _run_both(12, [257], 8, 2, 128, 3)


def test_noalloc_rejects_partials_above_its_buffer():
    # 64 sequences x 32 heads x 64 splits x (256 + 2) floats is far above the fixed buffer: refused
    S, Hq, Hkv, D = 64, 32, 8, 256
    cache = K.Cache("int8", 64, Hkv, D)
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((S, Hkv, D), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((S, 4), dtype=torch.int32, device="cuda")
    lens = torch.full((S,), 64, dtype=torch.int32, device="cuda")
    out = torch.empty((S, Hq, D), dtype=torch.float32, device="cuda")
    assert K.workspace_bytes(cache, S, Hq, 64) > K.noalloc_max_bytes()
    with pytest.raises(K.KvqError) as e:
        K.decode_step_noalloc(cache, kn, kn, q, bt, lens, 64, 64, out=out)
    assert e.value.status == -3
