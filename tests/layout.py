"""The in-page byte order of the GPU cache, written out from the formulas in include/kvq.h,
independently of the library, so that tests can turn device pages into the oracle's logical
[num_blocks][Hkv][16][D] layout (and back)."""
import numpy as np

PAGE = 16


def page_index(dtype: str, head_dim: int, which: str) -> np.ndarray:
    """idx[t, c] = position (byte for INT8, element for BF16) of token t, channel c in a page."""
    t = np.arange(PAGE)[:, None]
    c = np.arange(head_dim)[None, :]
    if dtype == "int8" and which == "k":
        return ((((c >> 6) << 6) | (((c >> 3) & 3) << 4) | t) << 4) | (((c >> 5) & 1) << 3) | (c & 7)
    if dtype == "int8" and which == "v":
        return ((((c >> 6) << 6) | ((t >> 2) << 4) | (c & 15)) << 4) | (((c >> 4) & 3) << 2) | (t & 3)
    if dtype == "bf16" and which == "k":
        return ((((c >> 5) << 6) | (((c >> 3) & 3) << 4) | t) << 3) | (c & 7)
    if dtype == "bf16" and which == "v":
        return ((((c >> 5) << 6) | ((t >> 2) << 4) | (c & 15)) << 3) | (((c >> 4) & 1) << 2) | (t & 3)
    raise ValueError((dtype, which))


def to_logical(pages: np.ndarray, dtype: str, head_dim: int, which: str) -> np.ndarray:
    """[NB][Hkv][16*D] physical pages -> [NB][Hkv][16][D] logical rows."""
    idx = page_index(dtype, head_dim, which)
    return pages[..., idx]


def to_physical(rows: np.ndarray, dtype: str, head_dim: int, which: str) -> np.ndarray:
    """[NB][Hkv][16][D] logical rows -> [NB][Hkv][16*D] physical pages."""
    idx = page_index(dtype, head_dim, which)
    out = np.empty(rows.shape[:-2] + (PAGE * head_dim,), dtype=rows.dtype)
    out[..., idx] = rows
    return out


def scales_to_logical(s: np.ndarray) -> np.ndarray:
    """[NB][Hkv][D/32][16] device scale pages (group-major) -> [NB][Hkv][16][D/32]."""
    return np.ascontiguousarray(np.swapaxes(s, -1, -2))


def scales_to_physical(s: np.ndarray) -> np.ndarray:
    """[NB][Hkv][16][D/32] logical scales -> [NB][Hkv][D/32][16] device scale pages."""
    return np.ascontiguousarray(np.swapaxes(s, -1, -2))
