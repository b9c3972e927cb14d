"""Python binding of libkvq: INT8 paged KV cache writes and split-KV decode attention on MI355X.

Argument marshalling only: every step runs in the HIP kernels of ``libkvq.so`` (built from
``csrc/`` by ``build.py``).  PyTorch provides device memory and the current HIP stream; the
library itself never allocates.  Importing this package fails if the library is missing.

    cache = Cache("int8", num_blocks, num_kv_heads, head_dim)          # device planes
    write(cache, k, v, slot_mapping)                                   # quantize-on-write
    out, lse = decode(cache, q, block_tables, context_lens, max_context_len)
    out, lse = decode_step(cache, k_new, v_new, q, block_tables, context_lens, max_context_len)
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["Cache", "KvqError", "write", "decode", "decode_mq", "choose_num_splits_mq", "decode_step", "decode_step_noalloc", "noalloc_max_bytes", "decode_partials", "decode_merge", "workspace_bytes", "choose_num_splits", "choose_num_splits_lengths", "page_offset",
           "status_string", "lib", "LIB_PATH", "INT8", "BF16", "INT8_HEAD"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")
INT8, BF16, INT8_HEAD = 0, 1, 2
_DTYPES = {"int8": INT8, "bf16": BF16, "int8_head": INT8_HEAD}
PAGE = 16

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python decode_attention_quantized_amd/build.py` "
                      "(or __graft_entry__.build()) first")

_P = ctypes.c_void_p
_i32 = ctypes.c_int32


class _CacheDesc(ctypes.Structure):
    _fields_ = [("dtype", _i32), ("num_blocks", _i32), ("block_size", _i32), ("num_kv_heads", _i32),
                ("head_dim", _i32), ("k", _P), ("v", _P), ("k_scales", _P), ("v_scales", _P)]


lib = ctypes.CDLL(LIB_PATH)
_CP = ctypes.POINTER(_CacheDesc)
lib.kvq_write.argtypes = [_CP, _P, _P, _P, _i32, _P]
lib.kvq_write.restype = ctypes.c_int
lib.kvq_check_write.argtypes = [_CP, _P, _P, _P, _i32, _P]
lib.kvq_check_write.restype = ctypes.c_int
lib.kvq_decode_workspace_bytes.argtypes = [_CP, _i32, _i32, _i32]
lib.kvq_decode_workspace_bytes.restype = ctypes.c_size_t
lib.kvq_choose_num_splits.argtypes = [_CP, _i32, _i32, _i32]
lib.kvq_choose_num_splits.restype = _i32
lib.kvq_choose_num_splits_lengths.argtypes = [_CP, _i32, _i32, _P]
lib.kvq_choose_num_splits_lengths.restype = _i32
_DEC = [_CP, _P, _P, _i32, _P, _i32, _i32, _i32, _i32, _P, _P, _P, ctypes.c_size_t, _P]
lib.kvq_decode_attention.argtypes = _DEC
lib.kvq_decode_attention.restype = ctypes.c_int
lib.kvq_decode_attention_int8qk.argtypes = _DEC
lib.kvq_decode_attention_int8qk.restype = ctypes.c_int
lib.kvq_check_decode.argtypes = _DEC
lib.kvq_check_decode.restype = ctypes.c_int
_STEP = [_CP, _P, _P] + _DEC[1:]
lib.kvq_decode_attention_mq.argtypes = [_CP, _P, _i32] + _DEC[2:]
lib.kvq_decode_attention_mq.restype = ctypes.c_int
lib.kvq_choose_num_splits_mq.argtypes = [_CP, _i32, _i32, _i32, _i32]
lib.kvq_choose_num_splits_mq.restype = _i32
lib.kvq_decode_step.argtypes = _STEP
lib.kvq_decode_step.restype = ctypes.c_int
lib.kvq_check_decode_step.argtypes = _STEP
lib.kvq_check_decode_step.restype = ctypes.c_int
lib.kvq_decode_step_noalloc.argtypes = [_CP, _P, _P, _P, _P, _i32, _P, _i32, _i32, _i32, _i32, _P, _P, _P]
lib.kvq_decode_step_noalloc.restype = ctypes.c_int
lib.kvq_decode_step_noalloc_max_bytes.argtypes = []
lib.kvq_decode_step_noalloc_max_bytes.restype = ctypes.c_size_t
lib.kvq_decode_partials.argtypes = [_CP, _P, _P, _i32, _P, _i32, _i32, _i32, _i32, _P, ctypes.c_size_t, _P]
lib.kvq_decode_partials.restype = ctypes.c_int
lib.kvq_decode_merge.argtypes = [_CP, _P, _i32, _i32, _i32, _i32, _P, ctypes.c_size_t, _P, _P, _P]
lib.kvq_decode_merge.restype = ctypes.c_int
lib.kvq_page_offset.argtypes = [_i32, _i32, _i32, _i32, _i32]
lib.kvq_page_offset.restype = _i32
lib.kvq_status_string.argtypes = [ctypes.c_int]
lib.kvq_status_string.restype = ctypes.c_char_p


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


def status_string(status: int) -> str:
    return lib.kvq_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise KvqError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _on_device(what, *tensors):
    """Every tensor handed to the library must live in GPU memory, all on one device: a kernel
    given a host pointer would fault.  (The library takes plain pointers and cannot tell.)"""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{what}: every tensor must be on the GPU (got one on {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{what}: tensors on different devices ({dev} and {t.device})")


def _check_outputs(what, out, out_shape, lse, lse_shape, workspace):
    if out is not None and (out.dtype != torch.float32 or tuple(out.shape) != tuple(out_shape)
                            or not out.is_contiguous()):
        raise ValueError(f"{what}: out must be contiguous fp32 {list(out_shape)}")
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != tuple(lse_shape)
                            or not lse.is_contiguous()):
        raise ValueError(f"{what}: lse must be contiguous fp32 {list(lse_shape)}")
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError(f"{what}: the workspace must be contiguous")


def _cache_planes(cache):
    return (cache.k, cache.v, cache.k_scales, cache.v_scales)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


class Cache:
    """One layer's paged KV cache pool in device memory (layout of include/kvq.h).

    k, v: int8 [num_blocks][Hkv][16*D] (INT8 formats) or bf16 bits as int16 [num_blocks][Hkv][16*D];
    k_scales, v_scales: fp16 [num_blocks][Hkv][D/32][16] ("int8": q8_0, group-major pages) or
    fp32 [num_blocks][Hkv][16] ("int8_head": one scale per token and head).
    """

    def __init__(self, dtype: str, num_blocks: int, num_kv_heads: int, head_dim: int, device="cuda"):
        if dtype not in _DTYPES:
            raise ValueError(dtype)
        self.dtype = dtype
        self.num_blocks, self.num_kv_heads, self.head_dim = num_blocks, num_kv_heads, head_dim
        shape = (num_blocks, num_kv_heads, PAGE * head_dim)
        if dtype in ("int8", "int8_head"):
            self.k = torch.empty(shape, dtype=torch.int8, device=device)
            self.v = torch.empty(shape, dtype=torch.int8, device=device)
            if dtype == "int8":
                sshape, sdt = (num_blocks, num_kv_heads, head_dim // 32, PAGE), torch.float16
            else:
                sshape, sdt = (num_blocks, num_kv_heads, PAGE), torch.float32
            self.k_scales = torch.empty(sshape, dtype=sdt, device=device)
            self.v_scales = torch.empty(sshape, dtype=sdt, device=device)
        else:
            self.k = torch.empty(shape, dtype=torch.int16, device=device)
            self.v = torch.empty(shape, dtype=torch.int16, device=device)
            self.k_scales = self.v_scales = None
        self.desc = _CacheDesc(_DTYPES[dtype], num_blocks, PAGE, num_kv_heads, head_dim,
                               _ptr(self.k), _ptr(self.v), _ptr(self.k_scales), _ptr(self.v_scales))

    def fill(self, code: int = 0x7F, scale_bits: int = 0x7BFF, bf16_bits: int = 0x7FC0):
        """Fill every byte of the pool with a poison pattern (codes, scale bits or bf16 bits)."""
        def s16(x):
            return x - 65536 if x >= 32768 else x
        if self.dtype == "int8":
            c = code - 256 if code >= 128 else code
            self.k.fill_(c)
            self.v.fill_(c)
            self.k_scales.view(torch.int16).fill_(s16(scale_bits))
            self.v_scales.view(torch.int16).fill_(s16(scale_bits))
        elif self.dtype == "int8_head":  # scales: the largest finite fp32
            c = code - 256 if code >= 128 else code
            self.k.fill_(c)
            self.v.fill_(c)
            self.k_scales.fill_(torch.finfo(torch.float32).max)
            self.v_scales.fill_(torch.finfo(torch.float32).max)
        else:
            self.k.fill_(s16(bf16_bits))
            self.v.fill_(s16(bf16_bits))
        return self


def _as_bits16(t):
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16, torch.uint16):
        return t
    raise TypeError(f"expected bfloat16 (or raw 16-bit) tensor, got {t.dtype}")


def write(cache: Cache, k, v, slot_mapping, *, checked: bool = False, stream=None) -> None:
    """Quantize-on-write (INT8) or scatter copy (BF16) of k, v [T][Hkv][D] bf16 into their slots."""
    k, v = _as_bits16(k), _as_bits16(v)
    T = int(slot_mapping.shape[0])
    if tuple(k.shape) != (T, cache.num_kv_heads, cache.head_dim) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"k/v must be [{T}][{cache.num_kv_heads}][{cache.head_dim}]")
    if slot_mapping.dtype != torch.int32 or not (k.is_contiguous() and v.is_contiguous()
                                                 and slot_mapping.is_contiguous()):
        raise ValueError("contiguous bf16 k/v and int32 slot_mapping required")
    _on_device("kvq_write", k, v, slot_mapping, *_cache_planes(cache))
    fn = lib.kvq_check_write if checked else lib.kvq_write
    _check(fn(ctypes.byref(cache.desc), _ptr(k), _ptr(v), _ptr(slot_mapping), T, _stream(stream)), "kvq_write")


def workspace_bytes(cache: Cache, num_seqs: int, num_q_heads: int, num_splits: int) -> int:
    return int(lib.kvq_decode_workspace_bytes(ctypes.byref(cache.desc), num_seqs, num_q_heads, num_splits))


def choose_num_splits(cache: Cache, num_seqs: int, num_q_heads: int, max_context_len: int) -> int:
    r = int(lib.kvq_choose_num_splits(ctypes.byref(cache.desc), num_seqs, num_q_heads, max_context_len))
    if r < 0:
        raise KvqError(r, "kvq_choose_num_splits")
    return r


def choose_num_splits_lengths(cache: Cache, context_lens, num_q_heads: int) -> int:
    """Split count from the batch's actual lengths (a host sequence of ints, one per sequence)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int64))
    if lens.ndim != 1 or lens.size == 0 or lens.min() < 0 or lens.max() > 2**31 - 1:
        raise ValueError("context_lens must be a non-empty 1-D sequence of lengths in [0, 2^31)")
    lens32 = lens.astype(np.int32)
    r = int(lib.kvq_choose_num_splits_lengths(ctypes.byref(cache.desc), lens32.size, num_q_heads,
                                              lens32.ctypes.data_as(ctypes.c_void_p)))
    if r < 0:
        raise KvqError(r, "kvq_choose_num_splits_lengths")
    return r


def page_offset(dtype: int, head_dim: int, which: int, token: int, channel: int) -> int:
    return int(lib.kvq_page_offset(dtype, head_dim, which, token, channel))


def _check_tables(what, block_tables, context_lens, S):
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError(f"{what}: block_tables and context_lens must be int32")
    if not (block_tables.is_contiguous() and context_lens.is_contiguous()) or block_tables.dim() != 2 \
            or block_tables.shape[0] != S or tuple(context_lens.shape) != (S,):
        raise ValueError(f"{what}: block_tables [S][max_blocks] and context_lens [S] required")


def _decode_args(cache, q, block_tables, context_lens, max_context_len, num_splits, out, lse, workspace, want_lse):
    q = _as_bits16(q)
    S, Hq, D = (int(x) for x in q.shape)
    if D != cache.head_dim or not q.is_contiguous():
        raise ValueError("q must be contiguous [S][Hq][D] bf16")
    _check_tables("decode", block_tables, context_lens, S)
    _check_outputs("decode", out, (S, Hq, D), lse, (S, Hq), workspace)
    _on_device("decode", q, block_tables, context_lens, out, lse, workspace, *_cache_planes(cache))
    ns = num_splits if num_splits else choose_num_splits(cache, S, Hq, max_context_len)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((S, Hq), dtype=torch.float32, device=q.device)
    need = workspace_bytes(cache, S, Hq, ns)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    args = [_ptr(q), _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), int(max_context_len), S, Hq,
            int(ns), _ptr(out), _ptr(lse), _ptr(workspace), int(workspace.numel() * workspace.element_size())]
    return args, out, lse


def decode(cache: Cache, q, block_tables, context_lens, max_context_len: int, num_splits: int = 0, *,
           out=None, lse=None, workspace=None, want_lse: bool = True, checked: bool = False, int_qk: bool = False,
           stream=None):
    """Split-KV decode attention; returns (out fp32 [S][Hq][D], lse fp32 [S][Hq] or None).
    int_qk: integer Q.K (Q quantized like the cache; q8_0 cache only; not with checked)."""
    if int_qk and checked:
        raise ValueError("integer Q.K has no checked mode")
    args, out, lse = _decode_args(cache, q, block_tables, context_lens, max_context_len, num_splits, out, lse,
                                  workspace, want_lse)
    fn = lib.kvq_check_decode if checked else (lib.kvq_decode_attention_int8qk if int_qk else lib.kvq_decode_attention)
    _check(fn(ctypes.byref(cache.desc), *args, _stream(stream)), "kvq_decode_attention")
    return out, lse


def choose_num_splits_mq(cache: Cache, num_seqs: int, num_query_tokens: int, num_q_heads: int,
                         max_context_len: int) -> int:
    r = int(lib.kvq_choose_num_splits_mq(ctypes.byref(cache.desc), num_seqs, num_query_tokens, num_q_heads,
                                         max_context_len))
    if r < 0:
        raise KvqError(r, "kvq_choose_num_splits_mq")
    return r


def decode_mq(cache: Cache, q, block_tables, context_lens, max_context_len: int, num_splits: int = 0, *,
              out=None, lse=None, workspace=None, want_lse: bool = True, stream=None):
    """Decode attention for q [S][n_q][Hq][D] bf16 (the last n_q positions of each sequence, causal
    among them); returns (out fp32 [S][n_q][Hq][D], lse fp32 [S][n_q][Hq] or None)."""
    q = _as_bits16(q)
    S, nq, Hq, D = (int(x) for x in q.shape)
    if D != cache.head_dim or not q.is_contiguous():
        raise ValueError("q must be contiguous [S][n_q][Hq][D] bf16")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32 or block_tables.dim() != 2 \
            or block_tables.shape[0] != S or context_lens.shape != (S,) \
            or not (block_tables.is_contiguous() and context_lens.is_contiguous()):
        raise ValueError("int32 block_tables [S][max_blocks] and context_lens [S] required")
    _check_outputs("decode_mq", out, (S, nq, Hq, D), lse, (S, nq, Hq), workspace)
    _on_device("decode_mq", q, block_tables, context_lens, out, lse, workspace, *_cache_planes(cache))
    ns = num_splits if num_splits else choose_num_splits_mq(cache, S, nq, Hq, max_context_len)
    if out is None:
        out = torch.empty((S, nq, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((S, nq, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(cache, S * nq, Hq, ns), 256), dtype=torch.uint8, device=q.device)
    st = lib.kvq_decode_attention_mq(ctypes.byref(cache.desc), _ptr(q), nq, _ptr(block_tables),
                                     int(block_tables.shape[1]), _ptr(context_lens), int(max_context_len), S, Hq,
                                     int(ns), _ptr(out), _ptr(lse), _ptr(workspace),
                                     int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check(st, "kvq_decode_attention_mq")
    return out, lse


def decode_step(cache: Cache, k_new, v_new, q, block_tables, context_lens, max_context_len: int,
                num_splits: int = 0, *, out=None, lse=None, workspace=None, want_lse: bool = True,
                checked: bool = False, stream=None):
    """One decode step: k_new, v_new [S][Hkv][D] bf16 (token context_lens[s]-1 of each sequence)
    are written into the cache by the split kernel, then attention and merge as ``decode``."""
    k_new, v_new = _as_bits16(k_new), _as_bits16(v_new)
    S = int(q.shape[0])
    if tuple(k_new.shape) != (S, cache.num_kv_heads, cache.head_dim) or tuple(v_new.shape) != tuple(k_new.shape) \
            or not (k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError(f"k_new/v_new must be contiguous [{S}][{cache.num_kv_heads}][{cache.head_dim}] bf16")
    _on_device("decode_step", k_new, v_new, q)
    args, out, lse = _decode_args(cache, q, block_tables, context_lens, max_context_len, num_splits, out, lse,
                                  workspace, want_lse)
    fn = lib.kvq_check_decode_step if checked else lib.kvq_decode_step
    _check(fn(ctypes.byref(cache.desc), _ptr(k_new), _ptr(v_new), *args, _stream(stream)), "kvq_decode_step")
    return out, lse


def decode_step_noalloc(cache: Cache, k_new, v_new, q, block_tables, context_lens, max_context_len: int,
                        num_splits: int = 0, *, out, lse=None, stream=None) -> None:
    """decode_step without a workspace: the library's fixed per-device buffer holds the partials
    (kvq_decode_step_noalloc).  ``out`` (and ``lse`` if wanted) must be given: nothing is allocated."""
    k_new, v_new, q = _as_bits16(k_new), _as_bits16(v_new), _as_bits16(q)
    S, Hq, D = (int(x) for x in q.shape)
    if D != cache.head_dim or not q.is_contiguous():
        raise ValueError("q must be contiguous [S][Hq][D] bf16")
    if tuple(k_new.shape) != (S, cache.num_kv_heads, D) or tuple(v_new.shape) != tuple(k_new.shape) \
            or not (k_new.is_contiguous() and v_new.is_contiguous()):
        raise ValueError(f"k_new/v_new must be contiguous [{S}][{cache.num_kv_heads}][{D}] bf16")
    _check_tables("decode_step_noalloc", block_tables, context_lens, S)
    if out is None:
        raise ValueError("decode_step_noalloc: out must be given (nothing is allocated)")
    _check_outputs("decode_step_noalloc", out, (S, Hq, D), lse, (S, Hq), None)
    _on_device("decode_step_noalloc", k_new, v_new, q, block_tables, context_lens, out, lse, *_cache_planes(cache))
    st = lib.kvq_decode_step_noalloc(ctypes.byref(cache.desc), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(block_tables),
                                     int(block_tables.shape[1]), _ptr(context_lens), int(max_context_len), S, Hq,
                                     int(num_splits), _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "kvq_decode_step_noalloc")


def noalloc_max_bytes() -> int:
    return int(lib.kvq_decode_step_noalloc_max_bytes())


def decode_partials(cache: Cache, q, block_tables, context_lens, max_context_len: int, num_splits: int, workspace,
                    *, stream=None) -> None:
    """First half of decode: split partials into ``workspace`` (num_splits must be explicit)."""
    q = _as_bits16(q)
    if q.dim() != 3 or int(q.shape[2]) != cache.head_dim or not q.is_contiguous():
        raise ValueError("decode_partials: q must be contiguous [S][Hq][D] bf16 with D the cache's head_dim")
    S, Hq, _ = (int(x) for x in q.shape)
    _check_tables("decode_partials", block_tables, context_lens, S)
    _check_outputs("decode_partials", None, (), None, (), workspace)
    _on_device("decode_partials", q, block_tables, context_lens, workspace, *_cache_planes(cache))
    st = lib.kvq_decode_partials(ctypes.byref(cache.desc), _ptr(q), _ptr(block_tables), int(block_tables.shape[1]),
                                 _ptr(context_lens), int(max_context_len), S, Hq, int(num_splits), _ptr(workspace),
                                 int(workspace.numel() * workspace.element_size()), _stream(stream))
    _check(st, "kvq_decode_partials")


def decode_merge(cache: Cache, context_lens, max_context_len: int, num_seqs: int, num_q_heads: int, num_splits: int,
                 workspace, out, lse=None, *, stream=None) -> None:
    """Second half of decode: combine the partials in ``workspace`` into out (and lse)."""
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous() \
            or tuple(context_lens.shape) != (int(num_seqs),):
        raise ValueError("decode_merge: context_lens must be contiguous int32 [num_seqs]")
    if out is None:
        raise ValueError("decode_merge: out must be given")
    _check_outputs("decode_merge", out, (num_seqs, num_q_heads, cache.head_dim), lse, (num_seqs, num_q_heads),
                   workspace)
    _on_device("decode_merge", context_lens, workspace, out, lse)
    st = lib.kvq_decode_merge(ctypes.byref(cache.desc), _ptr(context_lens), int(max_context_len), int(num_seqs),
                              int(num_q_heads), int(num_splits), _ptr(workspace),
                              int(workspace.numel() * workspace.element_size()), _ptr(out), _ptr(lse),
                              _stream(stream))
    _check(st, "kvq_decode_merge")
