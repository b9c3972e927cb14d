"""The C ABI library on the host (no GPU needed): it loads, exports every declared symbol,
rejects invalid arguments before launching anything, and its layout / sizing helpers agree
with the documented formulas."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import decode_attention_quantized_amd as K
from tests.layout import page_index

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

# Fake, 256-aligned, never dereferenced addresses: every call below fails host validation first.
FAKE = 0x10000


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_header_symbols_are_exported():
    names = _declared()
    assert "kvq_write" in names and "kvq_decode_attention" in names
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (kvq_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(K.lib, n) is not None


def test_status_strings():
    for code, name in [(0, "KVQ_OK"), (-1, "KVQ_ERR_INVALID_ARG"), (-2, "KVQ_ERR_UNSUPPORTED"),
                       (-3, "KVQ_ERR_WORKSPACE_TOO_SMALL"), (-4, "KVQ_ERR_LAUNCH_FAILED"),
                       (-5, "KVQ_ERR_VALIDATION_FAILED"), (-6, "KVQ_ERR_CAPTURING")]:
        assert K.status_string(code) == name
    assert K.status_string(7) == "KVQ_ERR_UNKNOWN"


@pytest.mark.parametrize("dtype,dt", [("int8", K.INT8), ("bf16", K.BF16)])
@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("which", ["k", "v"])
def test_page_offset_matches_documented_layout(dtype, dt, D, which):
    idx = page_index(dtype, D, which)
    got = np.array([[K.page_offset(dt, D, 0 if which == "k" else 1, t, c) for c in range(D)] for t in range(16)])
    assert np.array_equal(got, idx)
    # a bijection onto the page
    assert np.array_equal(np.sort(idx.ravel()), np.arange(16 * D))


def test_page_offset_rejects_bad_arguments():
    assert K.page_offset(K.INT8, 64, 0, 0, 0) == -1
    assert K.page_offset(K.INT8, 128, 2, 0, 0) == -1
    assert K.page_offset(K.INT8, 128, 0, 16, 0) == -1
    assert K.page_offset(K.INT8, 128, 0, 0, 128) == -1
    assert K.page_offset(5, 128, 0, 0, 0) == -1


def _desc(dtype=K.INT8, nb=64, bs=16, hkv=4, d=256, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE):
    return K._CacheDesc(dtype, nb, bs, hkv, d, k, v, ks, vs)


def _write(desc, k=FAKE, v=FAKE, sm=FAKE, T=1):
    return K.lib.kvq_write(ctypes.byref(desc), k, v, sm, T, None)


def _decode(desc, q=FAKE, bt=FAKE, mb=32, cl=FAKE, mcl=512, S=1, Hq=24, ns=4, out=FAKE, lse=None, ws=FAKE,
            wsb=1 << 30):
    return K.lib.kvq_decode_attention(ctypes.byref(desc), q, bt, mb, cl, mcl, S, Hq, ns, out, lse, ws, wsb, None)


def test_write_rejects_invalid_arguments():
    assert _write(_desc(d=64)) == -2
    assert _write(_desc(bs=32)) == -2
    assert _write(_desc(dtype=3)) == -2
    assert _write(_desc(nb=0)) == -1
    assert _write(_desc(hkv=0)) == -1
    assert _write(_desc(hkv=65536)) == -2              # more KV heads than the writers' grid has rows
    assert _write(_desc(k=None)) == -1
    assert _write(_desc(k=FAKE + 16)) == -1            # plane base not 256-aligned
    assert _write(_desc(ks=None)) == -1                # INT8 needs scale planes
    assert _write(_desc(), k=None) == -1
    assert _write(_desc(), v=FAKE + 2) == -1           # bf16 input not 16-aligned
    assert _write(_desc(), sm=None) == -1
    assert _write(_desc(), T=-1) == -1
    assert _write(_desc(), T=0) == 0                   # no-op, nothing launched
    assert K.lib.kvq_write(None, FAKE, FAKE, FAKE, 1, None) == -1


def test_decode_rejects_invalid_arguments():
    d = _desc()
    assert _decode(d, Hq=25) == -1                     # Hq % Hkv != 0
    assert _decode(_desc(hkv=1), Hq=17) == -2          # GQA ratio above 16
    assert _decode(d, S=0) == -1
    assert _decode(d, mb=0) == -1
    assert _decode(d, mcl=0) == -1
    assert _decode(d, mcl=32 * 16 + 1) == -1           # above max_blocks * 16
    assert _decode(d, ns=-1) == -1
    assert _decode(d, ns=4097) == -1
    assert _decode(d, q=None) == -1
    assert _decode(d, q=FAKE + 8) == -1
    assert _decode(d, bt=None) == -1
    assert _decode(d, cl=None) == -1
    assert _decode(d, out=None) == -1
    assert _decode(d, ws=None) == -1
    assert _decode(d, ws=FAKE + 64) == -1              # workspace not 256-aligned
    assert _decode(_desc(d=96)) == -2
    need = K.lib.kvq_decode_workspace_bytes(ctypes.byref(d), 1, 24, 4)
    assert need > 0
    assert _decode(d, wsb=need - 1) == -3


def _step(desc, kn=FAKE, vn=FAKE, q=FAKE, bt=FAKE, mb=32, cl=FAKE, mcl=512, S=1, Hq=24, ns=4, out=FAKE, lse=None,
          ws=FAKE, wsb=1 << 30):
    return K.lib.kvq_decode_step(ctypes.byref(desc), kn, vn, q, bt, mb, cl, mcl, S, Hq, ns, out, lse, ws, wsb, None)


def test_decode_step_rejects_invalid_arguments():
    d = _desc()
    assert _step(d, kn=None) == -1                     # the new token is required
    assert _step(d, vn=None) == -1
    assert _step(d, kn=FAKE + 8) == -1                 # not 16-aligned
    assert _step(d, vn=FAKE + 2) == -1
    assert _step(d, Hq=25) == -1                       # the decode checks apply too
    assert _step(d, mcl=0) == -1
    assert _step(d, out=None) == -1
    assert _step(_desc(d=96)) == -2
    need = K.lib.kvq_decode_workspace_bytes(ctypes.byref(d), 1, 24, 4)
    assert _step(d, wsb=need - 1) == -3
    assert K.lib.kvq_check_decode_step(ctypes.byref(d), None, FAKE, FAKE, FAKE, 32, FAKE, 512, 1, 24, 4, FAKE,
                                       None, FAKE, 1 << 30, None) == -1


def test_decode_mq_rejects_invalid_arguments():
    d = _desc()

    def mq(desc, nq=2, q=FAKE, Hq=24, ns=4, wsb=1 << 30):
        return K.lib.kvq_decode_attention_mq(ctypes.byref(desc), q, nq, FAKE, 32, FAKE, 512, 1, Hq, ns, FAKE, None,
                                             FAKE, wsb, None)
    assert mq(d, nq=0) == -1
    assert mq(d, nq=65537) == -1
    assert mq(d, q=None) == -1
    assert mq(d, Hq=25) == -1
    assert mq(_desc(dtype=K.BF16, ks=None, vs=None)) == -2      # INT8 cache only for n_q > 1
    need = K.lib.kvq_decode_workspace_bytes(ctypes.byref(d), 1 * 2, 24, 4)
    assert mq(d, wsb=need - 1) == -3                            # rows = num_seqs * n_q * Hq
    assert K.lib.kvq_choose_num_splits_mq(ctypes.byref(d), 1, 0, 24, 512) == -1
    assert 1 <= K.lib.kvq_choose_num_splits_mq(ctypes.byref(d), 1, 4, 24, 32768) <= 4096


def test_workspace_bytes_formula():
    d = _desc()
    for S, Hq, ns, D in [(1, 24, 64, 256), (32, 32, 7, 128), (4, 24, 256, 256)]:
        dd = _desc(d=D, hkv=8 if Hq == 32 else 4)
        rows = S * Hq * ns
        o = (rows * D * 4 + 255) // 256 * 256
        assert K.lib.kvq_decode_workspace_bytes(ctypes.byref(dd), S, Hq, ns) == o + rows * 8
    assert K.lib.kvq_decode_workspace_bytes(ctypes.byref(d), 1, 24, 0) == 0
    assert K.lib.kvq_decode_workspace_bytes(ctypes.byref(d), 0, 24, 4) == 0
    assert K.lib.kvq_decode_workspace_bytes(ctypes.byref(d), 1, 23, 4) == 0


def test_split_heuristic_is_sane():
    for S, Hkv, Hq, D, L in [(1, 4, 24, 256, 512), (1, 4, 24, 256, 4096), (1, 4, 24, 256, 32768),
                             (4, 4, 24, 256, 32768), (32, 8, 32, 128, 8192), (1, 4, 24, 256, 1)]:
        d = _desc(hkv=Hkv, d=D)
        ns = K.lib.kvq_choose_num_splits(ctypes.byref(d), S, Hq, L)
        pages = (L + 15) // 16
        assert 1 <= ns <= 4096
        assert ns <= max(1, pages)
    assert K.lib.kvq_choose_num_splits(ctypes.byref(_desc()), 1, 24, 0) == -1
    assert K.lib.kvq_choose_num_splits(ctypes.byref(_desc()), 1, 23, 64) == -1


def _by_lengths(desc, lens, Hq):
    a = np.ascontiguousarray(np.asarray(lens, np.int32))
    return K.lib.kvq_choose_num_splits_lengths(ctypes.byref(desc), len(a), Hq, a.ctypes.data_as(ctypes.c_void_p))


def test_split_count_from_lengths():
    """With no GPU the library counts 256 compute units (an MI355X's).  A ragged batch of few
    (sequence, head) pairs gets splits of cpp pages (a multiple of 4) such that the non-empty ones
    make about four rounds of the CUs: 4 sequences of 2K/8K/16K/32K tokens hold 128 + 512 + 1024 +
    2048 pages per KV head, x 4 heads / 1024 workgroups -> 14.5 -> cpp 16 -> 2048 / 16 = 128
    splits; 4 x 32K -> cpp 32 -> 64.  One sequence or many pairs: the same as the maximum-length
    rule."""
    d = _desc()
    assert _by_lengths(d, [2048, 8192, 16384, 32768], 24) == 128
    assert _by_lengths(d, [32768] * 4, 24) == 64
    for lens in ([32768], [4096], [512]):
        assert _by_lengths(d, lens, 24) == K.lib.kvq_choose_num_splits(ctypes.byref(d), 1, 24, max(lens))
    d8 = _desc(hkv=8, d=128)
    lens = np.random.default_rng(0).integers(512, 8192, 32)
    assert _by_lengths(d8, lens, 32) == K.lib.kvq_choose_num_splits(ctypes.byref(d8), 32, 32, int(lens.max()))
    assert _by_lengths(d, [0, 0], 24) == 1
    assert _by_lengths(d, [-1, 5], 24) == -1
    assert _by_lengths(d, [5, 5], 23) == -1
    assert K.lib.kvq_choose_num_splits_lengths(ctypes.byref(d), 2, 24, None) == -1
    # every length up to the int32 range stays within 1 .. 4096 splits
    for lens in ([1, 2**31 - 1], [16] * 3, [2**20, 1, 7]):
        assert 1 <= _by_lengths(d, lens, 24) <= 4096


def test_split_count_several_tokens():
    """With no GPU the library counts 256 compute units.  One 32K sequence, 24/4 heads: 2 and 4
    query tokens (one and two row tiles) and a q8_0 chunk of 3 or 4 tiles (8 tokens) fill the
    CUs once, one workgroup each, at 64 splits; the per-head format's 4-tile workgroups fit two
    per CU (128); a 2048-token section (205 chunks of 10 tokens, three workgroups per CU) gets at
    least four rounds: 3072 workgroups over 820 (chunk, KV head) groups -> 4 splits."""
    d = _desc()
    for nq, ns in [(2, 64), (4, 64), (8, 64), (10, 64), (2048, 4)]:
        assert K.lib.kvq_choose_num_splits_mq(ctypes.byref(d), 1, nq, 24, 32768) == ns, nq
    dh = _desc(dtype=K.INT8_HEAD)
    assert K.lib.kvq_choose_num_splits_mq(ctypes.byref(dh), 1, 8, 24, 32768) == 128


def test_noalloc_step_rejects_before_launch():
    d = _desc()
    f = K.lib.kvq_decode_step_noalloc
    # missing new-token rows, bad head counts, bad split count: invalid before anything else
    assert f(ctypes.byref(d), None, FAKE, FAKE, FAKE, 32, FAKE, 512, 1, 24, 4, FAKE, None, None) == -1
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 32, FAKE, 512, 1, 25, 4, FAKE, None, None) == -1
    assert f(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 32, FAKE, 512, 1, 24, 5000, FAKE, None, None) == -1
    # partials above the fixed buffer (64 x 32 heads x 64 splits x 258 floats): refused, nothing launched
    d8 = _desc(hkv=8)
    assert K.lib.kvq_decode_step_noalloc_max_bytes() == 8 << 20
    assert f(ctypes.byref(d8), FAKE, FAKE, FAKE, FAKE, 32, FAKE, 512, 64, 32, 64, FAKE, None, None) == -3
