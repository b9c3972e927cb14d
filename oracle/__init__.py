"""CPU oracle for the INT8 paged decode-attention path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product library (``decode_attention_quantized_amd``) never imports
it and shares no code with it.

The arithmetic lives in ``kvq_oracle.c`` (plain C, built with gcc, no fast-math, no FP
contraction, OpenMP over independent output rows).  This module only marshals numpy arrays.

Cache images use the LOGICAL layout::

    INT8:  k_codes, v_codes  int8   [num_blocks][Hkv][16][D]
           k_scales, v_scales uint16 [num_blocks][Hkv][16][D/32]   (binary16 bits)
    BF16:  k, v               uint16 [num_blocks][Hkv][16][D]      (bfloat16 bits)
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
PAGE = 16
GROUP = 32

_lib = None


def build() -> str:
    """Compile kvq_oracle.c into liboracle.so with gcc (IEEE arithmetic, OpenMP)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           "-Wall", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int, ctypes.c_int64
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_f16_array.argtypes = [P, P, i64]
        L.oracle_f16_to_f32_array.argtypes = [P, P, i64]
        L.oracle_quantize_groups.argtypes = [P, i64, P, P]
        L.oracle_kv_write_int8.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_kv_write_bf16.argtypes = [i32, i32, i32, i32, P, P, P, P, P]
        L.oracle_decode_int8.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, i64, i32, i32, P, P]
        L.oracle_decode_bf16.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, i64, i32, i32, P, P]
        L.oracle_kv_write_int8_head.argtypes = [i32, i32, i32, i32, P, P, P, P, P, P, P]
        L.oracle_decode_int8_head.argtypes = [i32, i32, i32, i32, i32, i32, P, P, P, P, P, P, P, P, i64, i32, i32,
                                              P, P]
        L.oracle_quantize_rows_f32.argtypes = [P, i64, i32, P, P]
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ------------------------------------------------------------------ number formats

def f32_to_f16(x) -> np.ndarray:
    """fp32 -> binary16 bits, round to nearest even (the oracle's own routine)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    h = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_f16_array(_p(x), _p(h), x.size)
    return h


def f16_to_f32(h) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    x = np.empty(h.shape, dtype=np.float32)
    lib().oracle_f16_to_f32_array(_p(h), _p(x), h.size)
    return x


def quantize_groups(x_bf16) -> tuple[np.ndarray, np.ndarray]:
    """Groups of 32 bf16 values (last axis 32) -> (int8 codes [..., 32], fp16-bit scales [...])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    assert x.shape[-1] == GROUP
    ng = x.size // GROUP
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(x.shape[:-1], dtype=np.uint16)
    lib().oracle_quantize_groups(_p(x), ng, _p(codes), _p(scales))
    return codes, scales


def quantize_rows_head(x_bf16) -> tuple[np.ndarray, np.ndarray]:
    """Per-head format: rows of D bf16 values (last axis) -> (int8 codes [..., D], fp32 scales [...])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    n = x.shape[-1]
    assert 0 < n <= 256
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    lib().oracle_quantize_rows_f32(_p(x), x.size // n, n, _p(codes), _p(scales))
    return codes, scales


# ------------------------------------------------------------------ cache images

@dataclass
class OracleCache:
    dtype: str               # "int8" (q8_0: fp16 scale per 32 values), "int8_head" (fp32 scale per row) or "bf16"
    num_blocks: int
    num_kv_heads: int
    head_dim: int
    k: np.ndarray            # int8 codes or bf16 bits
    v: np.ndarray
    k_scales: np.ndarray | None = None
    v_scales: np.ndarray | None = None

    @staticmethod
    def empty(dtype: str, num_blocks: int, num_kv_heads: int, head_dim: int,
              code_fill: int = 0x7F, scale_fill: int = 0x7BFF, bf16_fill: int = 0x7FC0) -> "OracleCache":
        """A pool filled with poison: codes 0x7F and scales 65504 (INT8), or NaN (BF16)."""
        shape = (num_blocks, num_kv_heads, PAGE, head_dim)
        if dtype == "int8":
            k = np.full(shape, np.int8(np.uint8(code_fill).view(np.int8)), dtype=np.int8)
            v = k.copy()
            sshape = (num_blocks, num_kv_heads, PAGE, head_dim // GROUP)
            ks = np.full(sshape, scale_fill, dtype=np.uint16)
            return OracleCache(dtype, num_blocks, num_kv_heads, head_dim, k, v, ks, ks.copy())
        if dtype == "int8_head":  # poison scale: the largest finite fp32
            k = np.full(shape, np.int8(np.uint8(code_fill).view(np.int8)), dtype=np.int8)
            ks = np.full((num_blocks, num_kv_heads, PAGE), np.finfo(np.float32).max, dtype=np.float32)
            return OracleCache(dtype, num_blocks, num_kv_heads, head_dim, k, k.copy(), ks, ks.copy())
        if dtype == "bf16":
            k = np.full(shape, bf16_fill, dtype=np.uint16)
            return OracleCache(dtype, num_blocks, num_kv_heads, head_dim, k, k.copy())
        raise ValueError(dtype)


def kv_write(cache: OracleCache, k_bf16: np.ndarray, v_bf16: np.ndarray, slot_mapping: np.ndarray) -> None:
    """Quantize-on-write (INT8) or scatter copy (BF16) of k, v [T][Hkv][D] into the cache."""
    k = np.ascontiguousarray(k_bf16, dtype=np.uint16)
    v = np.ascontiguousarray(v_bf16, dtype=np.uint16)
    sm = np.ascontiguousarray(slot_mapping, dtype=np.int32)
    T = sm.shape[0]
    assert k.shape == (T, cache.num_kv_heads, cache.head_dim) and v.shape == k.shape
    L = lib()
    if cache.dtype == "int8":
        L.oracle_kv_write_int8(T, cache.num_kv_heads, cache.head_dim, cache.num_blocks, _p(k), _p(v), _p(sm),
                               _p(cache.k), _p(cache.v), _p(cache.k_scales), _p(cache.v_scales))
    elif cache.dtype == "int8_head":
        L.oracle_kv_write_int8_head(T, cache.num_kv_heads, cache.head_dim, cache.num_blocks, _p(k), _p(v), _p(sm),
                                    _p(cache.k), _p(cache.v), _p(cache.k_scales), _p(cache.v_scales))
    else:
        L.oracle_kv_write_bf16(T, cache.num_kv_heads, cache.head_dim, cache.num_blocks, _p(k), _p(v), _p(sm),
                               _p(cache.k), _p(cache.v))


def decode(cache: OracleCache, q_bf16: np.ndarray, block_tables: np.ndarray, context_lens: np.ndarray,
           rows=None, num_splits: int = 0, max_context_len: int | None = None):
    """Decode attention in fp64.

    q_bf16 [S][Hq][D] bf16 bits; block_tables [S][max_blocks]; context_lens [S].
    rows: optional flat indices s*Hq + hq to compute.  num_splits 0 gives the plain
    definition; > 0 runs the split/merge algorithm (partition sized by max_context_len).
    Returns (out fp64 [n_rows][D] or [S][Hq][D], lse fp64 [n_rows] or [S][Hq]).
    """
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    S, Hq, D = q.shape
    assert D == cache.head_dim and D <= 256 and Hq % cache.num_kv_heads == 0
    assert bt.ndim == 2 and bt.shape[0] == S and cl.shape == (S,)
    if max_context_len is None:
        max_context_len = int(cl.max()) if S else 0
    assert 0 <= num_splits <= 4096
    if rows is None:
        rows_arr = None
        n = S * Hq
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows_arr.shape[0]
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty((n,), dtype=np.float64)
    rp = _p(rows_arr) if rows_arr is not None else None
    L = lib()
    if cache.dtype == "int8":
        L.oracle_decode_int8(S, Hq, cache.num_kv_heads, D, cache.num_blocks, bt.shape[1], _p(q), _p(bt), _p(cl),
                             _p(cache.k), _p(cache.v), _p(cache.k_scales), _p(cache.v_scales), rp, n,
                             num_splits, max_context_len, _p(out), _p(lse))
    elif cache.dtype == "int8_head":
        L.oracle_decode_int8_head(S, Hq, cache.num_kv_heads, D, cache.num_blocks, bt.shape[1], _p(q), _p(bt),
                                  _p(cl), _p(cache.k), _p(cache.v), _p(cache.k_scales), _p(cache.v_scales), rp, n,
                                  num_splits, max_context_len, _p(out), _p(lse))
    else:
        L.oracle_decode_bf16(S, Hq, cache.num_kv_heads, D, cache.num_blocks, bt.shape[1], _p(q), _p(bt), _p(cl),
                             _p(cache.k), _p(cache.v), rp, n, num_splits, max_context_len, _p(out), _p(lse))
    if rows is None:
        return out.reshape(S, Hq, D), lse.reshape(S, Hq)
    return out, lse


def quantized_q(q_bf16: np.ndarray) -> np.ndarray:
    """Integer Q.K (opt-in): Q [..., D] quantized with the cache's own q8_0 rule (one fp16 scale per
    32 values, codes against the stored scale) and decoded, code * scale, as fp64."""
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    D = q.shape[-1]
    codes, scales = quantize_groups(q.reshape(-1, GROUP))
    qd = codes.astype(np.float64) * f16_to_f32(scales).astype(np.float64)[:, None]
    return qd.reshape(q.shape[:-1] + (D,))


def decode_int8_qk(cache: OracleCache, q_bf16: np.ndarray, block_tables: np.ndarray, context_lens: np.ndarray):
    """Decode attention with integer Q.K (the long-context page's integer dot-product option:
    Q quantized per 32 values like the cache): the plain definition softmax(q^ K^T / sqrt(D)) V in
    fp64 over the decoded cache, with q^ = quantized_q(q).  Returns (out [S][Hq][D], lse [S][Hq])."""
    qd = quantized_q(q_bf16)
    S, Hq, D = qd.shape
    K = dequantized_rows(cache, "k")
    V = dequantized_rows(cache, "v")
    G = Hq // cache.num_kv_heads
    out = np.zeros((S, Hq, D))
    lse = np.full((S, Hq), -np.inf)
    bt = np.asarray(block_tables)
    for s_ in range(S):
        L = int(context_lens[s_])
        if L <= 0:
            continue
        t = np.arange(L)
        blk, off = bt[s_, t // PAGE], t % PAGE
        for hq in range(Hq):
            z = K[blk, hq // G, off] @ qd[s_, hq] / np.sqrt(D)
            m = z.max()
            w = np.exp(z - m)
            out[s_, hq] = (w @ V[blk, hq // G, off]) / w.sum()
            lse[s_, hq] = m + np.log(w.sum())
    return out, lse


def decode_mq(cache: OracleCache, q_bf16: np.ndarray, block_tables: np.ndarray, context_lens: np.ndarray):
    """Decode attention for n_q query tokens per sequence, causal among them, in fp64.

    q_bf16 [S][n_q][Hq][D]: the queries of the last n_q positions L-n_q .. L-1 of sequence s
    (L = context_lens[s]).  Query token i attends to the keys at positions 0 .. L-n_q+i, which is
    ordinary decode attention over the first L-n_q+i+1 tokens; that is how it is computed here
    (each query token is a sequence of its own with that context length and the same block
    table).  Returns (out [S][n_q][Hq][D], lse [S][n_q][Hq]); a query with no visible key gives
    out 0 and lse -inf.
    """
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    S, nq, Hq, D = q.shape
    bt = np.ascontiguousarray(block_tables, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    lens = (cl[:, None] - nq + 1 + np.arange(nq, dtype=np.int32)[None, :]).clip(min=0).astype(np.int32)
    out, lse = decode(cache, q.reshape(S * nq, Hq, D), np.repeat(bt, nq, axis=0), lens.reshape(-1))
    return out.reshape(S, nq, Hq, D), lse.reshape(S, nq, Hq)


def dequantized_rows(cache: OracleCache, which: str) -> np.ndarray:
    """Decoded K or V of every (block, head, offset) in fp64: code * scale, or the bf16 value."""
    if cache.dtype == "int8":
        codes = cache.k if which == "k" else cache.v
        sc = f16_to_f32(cache.k_scales if which == "k" else cache.v_scales).astype(np.float64)
        return codes.astype(np.float64) * np.repeat(sc, GROUP, axis=-1)
    if cache.dtype == "int8_head":
        codes = cache.k if which == "k" else cache.v
        sc = (cache.k_scales if which == "k" else cache.v_scales).astype(np.float64)
        return codes.astype(np.float64) * sc[..., None]
    arr = cache.k if which == "k" else cache.v
    return (arr.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads the oracle's OpenMP loops use from now on (timing only; results do not depend on it)."""
    lib().oracle_set_num_threads(int(n))
