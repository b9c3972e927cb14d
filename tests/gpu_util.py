"""Helpers for the GPU parity tests: build the same cache on the GPU (through the C ABI) and in
the oracle from one seeded workload, compare caches byte for byte and outputs to tolerance."""
import sys

import numpy as np
import torch

import decode_attention_quantized_amd as K
import oracle as O
from tests.layout import scales_to_logical, scales_to_physical, to_logical, to_physical

# Output tolerance: every element must satisfy |gpu - oracle| <= ATOL + RTOL * |oracle|.
ATOL, RTOL = 2e-3, 1e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def bf16_dev(bits):
    return dev(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16), torch.bfloat16)


class Pair:
    """A GPU cache and an oracle cache holding the same tokens."""

    def __init__(self, dtype, num_blocks, Hkv, D):
        self.dtype, self.D = dtype, D
        self.g = K.Cache(dtype, num_blocks, Hkv, D).fill()
        self.o = O.OracleCache.empty(dtype, num_blocks, Hkv, D)

    def write(self, k_bits, v_bits, slots, checked=False):
        O.kv_write(self.o, k_bits, v_bits, slots)
        K.write(self.g, bf16_dev(k_bits), bf16_dev(v_bits), dev(np.asarray(slots, dtype=np.int32)), checked=checked)

    def gpu_logical(self):
        torch.cuda.synchronize()
        g = self.g
        if self.dtype == "int8_head":  # codes as INT8; scales fp32 [NB][Hkv][16] (compared as bits)
            kc = to_logical(g.k.cpu().numpy(), "int8", self.D, "k")
            vc = to_logical(g.v.cpu().numpy(), "int8", self.D, "v")
            return kc, vc, g.k_scales.cpu().numpy().view(np.uint32), g.v_scales.cpu().numpy().view(np.uint32)
        if self.dtype == "int8":
            kc = to_logical(g.k.cpu().numpy(), "int8", self.D, "k")
            vc = to_logical(g.v.cpu().numpy(), "int8", self.D, "v")
            ks = scales_to_logical(g.k_scales.cpu().view(torch.int16).numpy().view(np.uint16))
            vs = scales_to_logical(g.v_scales.cpu().view(torch.int16).numpy().view(np.uint16))
            return kc, vc, ks, vs
        kc = to_logical(g.k.cpu().numpy().view(np.uint16), "bf16", self.D, "k")
        vc = to_logical(g.v.cpu().numpy().view(np.uint16), "bf16", self.D, "v")
        return kc, vc

    def assert_cache_equal(self):
        got = self.gpu_logical()
        if self.dtype == "int8":
            want = (self.o.k, self.o.v, self.o.k_scales, self.o.v_scales)
            names = ("k codes", "v codes", "k scales", "v scales")
        elif self.dtype == "int8_head":
            want = (self.o.k, self.o.v, self.o.k_scales.view(np.uint32), self.o.v_scales.view(np.uint32))
            names = ("k codes", "v codes", "k scales", "v scales")
        else:
            want = (self.o.k, self.o.v)
            names = ("k", "v")
        for n, g, w in zip(names, got, want):
            bad = np.count_nonzero(g != w)
            assert bad == 0, f"{n}: {bad} of {w.size} entries differ"

    def upload_oracle_cache(self):
        """Overwrite the GPU cache with the oracle's bytes (decode tests independent of kv_write)."""
        o, g = self.o, self.g
        if self.dtype == "int8_head":
            g.k.copy_(torch.from_numpy(to_physical(o.k, "int8", self.D, "k")))
            g.v.copy_(torch.from_numpy(to_physical(o.v, "int8", self.D, "v")))
            g.k_scales.copy_(torch.from_numpy(o.k_scales))
            g.v_scales.copy_(torch.from_numpy(o.v_scales))
        elif self.dtype == "int8":
            g.k.copy_(torch.from_numpy(to_physical(o.k, "int8", self.D, "k")))
            g.v.copy_(torch.from_numpy(to_physical(o.v, "int8", self.D, "v")))
            g.k_scales.view(torch.int16).copy_(torch.from_numpy(scales_to_physical(o.k_scales).view(np.int16)))
            g.v_scales.view(torch.int16).copy_(torch.from_numpy(scales_to_physical(o.v_scales).view(np.int16)))
        else:
            g.k.copy_(torch.from_numpy(to_physical(o.k, "bf16", self.D, "k").view(np.int16)))
            g.v.copy_(torch.from_numpy(to_physical(o.v, "bf16", self.D, "v").view(np.int16)))
        torch.cuda.synchronize()


def fill_from_layer(pair, layer, rows=None):
    """Write the layer's prefill tokens, then its step tokens (two kv_write calls, as a model does)."""
    pre = layer.prefill_rows() if rows is None else rows
    if len(pre):
        pair.write(layer.k[pre], layer.v[pre], layer.slots[pre])
    step = layer.step_rows()
    pair.write(layer.k[step], layer.v[step], layer.slots[step])


def assert_close(out_g, lse_g, out_r, lse_r, what=""):
    out_g = np.asarray(out_g, dtype=np.float64)
    lse_g = np.asarray(lse_g, dtype=np.float64)
    err = np.abs(out_g - out_r)
    tol = ATOL + RTOL * np.abs(out_r)
    nbad = int(np.count_nonzero(~(err <= tol)))
    fin = np.isfinite(lse_r)
    lerr = np.abs(lse_g[fin] - lse_r[fin])
    ltol = ATOL + RTOL * np.abs(lse_r[fin])
    lbad = int(np.count_nonzero(~(lerr <= ltol))) + int(np.count_nonzero(np.isfinite(lse_g[~fin])))
    rel = err / np.maximum(np.abs(out_r), 1e-30)
    msg = (f"{what}: max abs err {err.max():.3e}, max rel err {rel[np.abs(out_r) > 1e-3].max() if (np.abs(out_r) > 1e-3).any() else 0:.3e},"
           f" lse max err {lerr.max() if lerr.size else 0:.3e}, out bad {nbad}, lse bad {lbad}")
    log(msg)
    assert nbad == 0 and lbad == 0, msg
    return err.max()


def decode_both(pair, layer_q, bt, lens, max_context_len, num_splits, oracle_out=None, rows=None):
    """GPU decode at num_splits; oracle plain definition (computed once if given)."""
    out, lse = K.decode(pair.g, bf16_dev(layer_q), dev(bt), dev(lens), max_context_len, num_splits)
    torch.cuda.synchronize()
    if oracle_out is None:
        oracle_out = O.decode(pair.o, layer_q, bt, lens, rows=rows)
    return out.cpu().numpy(), lse.cpu().numpy(), oracle_out
