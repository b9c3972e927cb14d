"""Seeded synthetic inputs for the INT8 paged decode-attention path.

This module only makes inputs: bf16 K/V/Q tensors, block tables, context lengths, slot
mappings and pool sizes.  It holds none of the method's arithmetic (no quantization, no
attention) and is shared by the tests, the oracle calls and bench.py.

Recipe (the same for every configuration):
  * numpy PCG64, seeded by SeedSequence([config_id, layer, stream]) so that each layer and
    each tensor has its own reproducible stream; context lengths of a batch depend on the
    configuration only.
  * K, V and Q values are fp32 N(0, 1).  Per (layer, KV head) four channel indices are
    drawn without replacement and scaled by 20 in both K and V ("outlier channels");
    each query head draws its own four (or, with ``aligned=True``, uses its KV head's four,
    which gives sharply peaked score distributions).  Values are rounded to bf16 with
    round-to-nearest-even.
  * Pool: the pages the batch needs plus 10% spare blocks.  Block tables follow the
    configuration's rule: "subset" (a random subset of a larger pool, random order),
    "permutation" (a random permutation of the pool), "interleaved" (blocks handed out
    round-robin across the sequences that still need pages).
  * The cache is filled by writing tokens 0..L-2 of every sequence ("prefill"); the decode
    step then writes token L-1 and attends over all L tokens.

The five configurations are the workloads of the long-context decode study: the hybrid
model's full-attention geometry (24 query heads, 4 KV heads of dimension 256, GQA 6:1) at
512, 4K and 32K context and a four-sequence mixed batch, plus a dense 8B-class geometry
(32 query heads, 8 KV heads of dimension 128, batch 32).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE = 16


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    layers: int
    context_lens: tuple  # per sequence, or None for a seeded draw
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    table_rule: str       # "subset" | "permutation" | "interleaved"
    splits: tuple         # split counts swept in tests and sweeps
    pool_blocks: int | None = None  # explicit pool size (subset rule)
    seeded_lens: tuple | None = None  # (batch, lo, hi) for a seeded uniform draw


CONFIGS = {
    1: Config(1, "tiny-512", 1, (512,), 24, 4, 256, "subset", (1, 4), pool_blocks=64),
    2: Config(2, "hybrid-4k", 16, (4096,), 24, 4, 256, "permutation", (1, 2, 4, 8, 16, 32, 64)),
    3: Config(3, "long-32k", 16, (32768,), 24, 4, 256, "permutation", (8, 16, 32, 64, 128, 256)),
    4: Config(4, "mixed-4seq", 16, (2048, 8192, 16384, 32768), 24, 4, 256, "interleaved",
              (8, 16, 32, 64, 128, 256)),
    5: Config(5, "dense8b-b32", 32, None, 32, 8, 128, "permutation", (1, 2, 4, 8, 16),
              seeded_lens=(32, 512, 8192)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns, round to nearest even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def context_lens_for(cfg: Config) -> np.ndarray:
    if cfg.context_lens is not None:
        return np.array(cfg.context_lens, dtype=np.int32)
    b, lo, hi = cfg.seeded_lens
    return _rng(cfg.cid, 999).integers(lo, hi + 1, size=b).astype(np.int32)


@dataclass
class Layer:
    """One layer's inputs.  All bf16 tensors are uint16 bit patterns."""
    cfg: Config
    layer: int
    context_lens: np.ndarray       # int32 [S]   (includes the token written by the step)
    block_tables: np.ndarray       # int32 [S][max_blocks]
    num_blocks: int
    used_blocks: np.ndarray        # int32, the blocks any table refers to
    k: np.ndarray                  # bf16 [total_tokens][Hkv][D], tokens of seq 0 then seq 1 ...
    v: np.ndarray
    q: np.ndarray                  # bf16 [S][Hq][D]
    token_seq: np.ndarray          # int32 [total_tokens] sequence of each token row
    token_pos: np.ndarray          # int32 [total_tokens] position of each token row
    slots: np.ndarray              # int32 [total_tokens] physical slot of each token row
    extra: dict = field(default_factory=dict)

    @property
    def S(self):
        return int(self.context_lens.shape[0])

    def prefill_rows(self) -> np.ndarray:
        """Token rows written before the step: every position but the last of each sequence."""
        last = self.context_lens[self.token_seq] - 1
        return np.nonzero(self.token_pos < last)[0]

    def step_rows(self) -> np.ndarray:
        """Token rows written by the decode step: the last position of each sequence."""
        last = self.context_lens[self.token_seq] - 1
        return np.nonzero(self.token_pos == last)[0]


def block_tables_for(cfg: Config, lens: np.ndarray, rng: np.random.Generator, spare: float = 0.10):
    pages = (lens.astype(np.int64) + PAGE - 1) // PAGE
    need = int(pages.sum())
    S = lens.shape[0]
    max_blocks = int(pages.max()) if S else 1
    if cfg.pool_blocks is not None:
        nb = max(cfg.pool_blocks, need)
    else:
        nb = need + max(1, int(np.ceil(need * spare)))
    bt = np.full((S, max_blocks), -1, dtype=np.int32)
    if cfg.table_rule in ("subset", "permutation"):
        order = rng.permutation(nb)[:need].astype(np.int32)
        pos = 0
        for s in range(S):
            bt[s, : pages[s]] = order[pos: pos + pages[s]]
            pos += pages[s]
    elif cfg.table_rule == "interleaved":
        nxt = 0
        filled = np.zeros(S, dtype=np.int64)
        while (filled < pages).any():
            for s in range(S):
                if filled[s] < pages[s]:
                    bt[s, filled[s]] = nxt
                    filled[s] += 1
                    nxt += 1
    else:
        raise ValueError(cfg.table_rule)
    used = bt[bt >= 0]
    return bt, nb, used


def make_layer(cid: int, layer: int = 0, *, aligned: bool = False, context_lens=None,
               num_q_heads=None, num_kv_heads=None, head_dim=None, table_rule=None,
               outlier_scale: float = 20.0, num_outliers: int = 4, spare: float = 0.10) -> Layer:
    """Inputs of one layer of configuration ``cid`` (overrides make smaller variants)."""
    base = CONFIGS[cid]
    cfg = Config(base.cid, base.name, base.layers,
                 tuple(context_lens) if context_lens is not None else base.context_lens,
                 num_q_heads or base.num_q_heads, num_kv_heads or base.num_kv_heads,
                 head_dim or base.head_dim, table_rule or base.table_rule, base.splits,
                 base.pool_blocks if context_lens is None else None,
                 base.seeded_lens if context_lens is None else None)
    lens = context_lens_for(cfg)
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    S = lens.shape[0]
    g_tab = _rng(cid, layer, 1)
    bt, nb, used = block_tables_for(cfg, lens, g_tab, spare)
    total = int(lens.sum())
    token_seq = np.repeat(np.arange(S, dtype=np.int32), lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    token_pos = (np.arange(total, dtype=np.int64) - np.repeat(starts, lens)).astype(np.int32)
    slots = bt[token_seq, token_pos // PAGE].astype(np.int64) * PAGE + token_pos % PAGE
    # outlier channels per KV head (shared by K and V), and per query head
    g_out = _rng(cid, layer, 2)
    kv_out = np.stack([g_out.choice(D, num_outliers, replace=False) for _ in range(Hkv)]) if num_outliers else \
        np.zeros((Hkv, 0), dtype=np.int64)
    G = Hq // Hkv
    if aligned:
        q_out = np.stack([kv_out[h // G] for h in range(Hq)])
    else:
        q_out = np.stack([g_out.choice(D, num_outliers, replace=False) for _ in range(Hq)]) if num_outliers else \
            np.zeros((Hq, 0), dtype=np.int64)
    mult_kv = np.ones((Hkv, D), dtype=np.float32)
    for h in range(Hkv):
        mult_kv[h, kv_out[h]] = outlier_scale
    mult_q = np.ones((Hq, D), dtype=np.float32)
    for h in range(Hq):
        mult_q[h, q_out[h]] = outlier_scale
    k = _rng(cid, layer, 3).standard_normal((total, Hkv, D), dtype=np.float32)
    k *= mult_kv[None]
    kb = f32_to_bf16_bits(k)
    del k
    v = _rng(cid, layer, 4).standard_normal((total, Hkv, D), dtype=np.float32)
    v *= mult_kv[None]
    vb = f32_to_bf16_bits(v)
    del v
    q = _rng(cid, layer, 5).standard_normal((S, Hq, D), dtype=np.float32) * mult_q[None]
    qb = f32_to_bf16_bits(q)
    return Layer(cfg, layer, lens, bt, nb, used.astype(np.int32), kb, vb, qb, token_seq, token_pos,
                 slots.astype(np.int32), {"kv_outliers": kv_out, "q_outliers": q_out})


def algorithmic_bytes_int8(lens, num_kv_heads: int, head_dim: int) -> int:
    """K and V codes plus their fp16 scales over every context token, for one layer."""
    per_token_head = 2 * head_dim + 2 * (head_dim // 32) * 2
    return int(np.sum(lens, dtype=np.int64)) * num_kv_heads * per_token_head


def algorithmic_bytes_bf16(lens, num_kv_heads: int, head_dim: int) -> int:
    return int(np.sum(lens, dtype=np.int64)) * num_kv_heads * 4 * head_dim


def make_layer_device(cid: int, layer: int = 0, device="cuda", *, aligned: bool = False,
                      outlier_scale: float = 20.0, num_outliers: int = 4, spare: float = 0.10):
    """The same recipe as make_layer, with the K/V/Q draws made by torch on the device (seeded
    torch.Generator) so that multi-gigabyte benchmark inputs need no host round trip.  Block
    tables, context lengths, slots and outlier channels come from the numpy streams of
    make_layer.  Returns (Layer with k/v/q set to None, dict of device tensors k, v, q as bf16)."""
    import torch

    cfg = CONFIGS[cid]
    lens = context_lens_for(cfg)
    Hq, Hkv, D = cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    S = lens.shape[0]
    bt, nb, used = block_tables_for(cfg, lens, _rng(cid, layer, 1), spare)
    total = int(lens.sum())
    token_seq = np.repeat(np.arange(S, dtype=np.int32), lens)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    token_pos = (np.arange(total, dtype=np.int64) - np.repeat(starts, lens)).astype(np.int32)
    slots = bt[token_seq, token_pos // PAGE].astype(np.int64) * PAGE + token_pos % PAGE
    g_out = _rng(cid, layer, 2)
    kv_out = np.stack([g_out.choice(D, num_outliers, replace=False) for _ in range(Hkv)])
    G = Hq // Hkv
    q_out = np.stack([kv_out[h // G] for h in range(Hq)]) if aligned else \
        np.stack([g_out.choice(D, num_outliers, replace=False) for _ in range(Hq)])
    mult_kv = torch.ones((Hkv, D), dtype=torch.float32)
    for h in range(Hkv):
        mult_kv[h, torch.from_numpy(kv_out[h])] = outlier_scale
    mult_q = torch.ones((Hq, D), dtype=torch.float32)
    for h in range(Hq):
        mult_q[h, torch.from_numpy(q_out[h])] = outlier_scale
    mult_kv, mult_q = mult_kv.to(device), mult_q.to(device)
    gen = torch.Generator(device=device)
    out = {}
    for name, shape, mult, stream in (("k", (total, Hkv, D), mult_kv, 3), ("v", (total, Hkv, D), mult_kv, 4),
                                      ("q", (S, Hq, D), mult_q, 5)):
        gen.manual_seed(int(np.random.SeedSequence([cid, layer, stream]).generate_state(1)[0]))
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        x.mul_(mult)
        out[name] = x.to(torch.bfloat16)  # round to nearest even
        del x
    lay = Layer(cfg, layer, lens, bt, nb, used.astype(np.int32), None, None, None, token_seq, token_pos,
                slots.astype(np.int32), {"kv_outliers": kv_out, "q_outliers": q_out})
    return lay, out
