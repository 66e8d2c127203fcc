"""Seeded synthetic inputs for the MLA forward pass (prefill and absorbed decode).

This module is shared by the tests, the CPU oracle and the benchmark.  It holds
no arithmetic of the attention method itself: it only draws random numbers in a
fixed order, rounds them to bfloat16 where the workload asks for it, and builds
the integer bookkeeping (document cut points, paged block tables) that the
workloads describe.

Draw order for one workload, all from ``numpy.random.Generator(PCG64(seed))``:

  1. x                      N(0, 1)
  2. W_q_a (or W_q)         N(0, 0.02)
  3. gamma_q                ones (no draw)
  4. W_q_b                  N(0, 0.02)
  5. W_kv_a                 N(0, 0.02)
  6. gamma_kv               ones (no draw)
  7. W_kv_b                 N(0, 0.02)
  8. W_o                    N(0, 0.02)
  9. W_g                    N(0, 0.02)   (gated variant only)
 10. document lengths       integers / choice
 11. block permutation      permutation  (decode only)
 12. cache                  N(0, 1)      (decode only)
 13. q_nope, q_pe           N(0, 1)      (decode only)

Values are drawn in float32; bfloat16 workloads then round every value to
bfloat16 with round-to-nearest-even, so the GPU and the oracle consume the very
same numbers.  Weights follow the ``nn.Linear`` layout ``[out_features,
in_features]``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "MLAShape", "RopeSpec", "WORKLOADS", "bf16_round", "bf16_bits",
    "bf16_from_bits", "make_prefill_case", "make_decode_case", "PrefillCase",
    "DecodeCase", "doc_lengths_for", "ChunkCase", "make_chunk_case",
]


# --------------------------------------------------------------------------
# bfloat16 rounding (input quantisation only)
# --------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16.  NaN stays a quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(nan, (u >> 16) | 0x0040, r)
    return r.astype(np.uint16)


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value, returned as float32."""
    return bf16_from_bits(bf16_bits(x))


# --------------------------------------------------------------------------
# Workload descriptions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class RopeSpec:
    kind: str = "plain"            # "none" | "plain" | "yarn"
    theta: float = 10000.0
    factor: float = 1.0            # YaRN scale s
    original_max_pos: int = 4096
    beta_fast: float = 32.0
    beta_slow: float = 1.0
    mscale: float = 1.0
    mscale_all_dim: float = 0.0


@dataclasses.dataclass(frozen=True)
class MLAShape:
    name: str
    dtype: str                      # "bf16" | "f32"
    hidden: int
    num_heads: int
    q_lora_rank: int                # 0 => direct q projection
    kv_lora_rank: int
    qk_nope_dim: int
    qk_rope_dim: int
    v_head_dim: int
    rope: RopeSpec
    output_gate: bool = False
    norm_eps: float = 1e-6
    rope_interleave: bool = False   # RoPE on interleaved pairs (2i, 2i+1)
    o_groups: int = 0               # > 0: grouped low-rank output projection W_o_b . blockdiag(W_o_a)
    o_lora_rank: int = 0
    # token layout
    num_docs: int = 1
    total_tokens: int = 0
    doc_split: str = "equal"        # "equal" | "random"
    seed: int = 1

    @property
    def qk_head_dim(self) -> int:
        return self.qk_nope_dim + self.qk_rope_dim

    def replace(self, **kw) -> "MLAShape":
        return dataclasses.replace(self, **kw)


YARN_V3 = RopeSpec(kind="yarn", theta=10000.0, factor=40.0, original_max_pos=4096,
                   beta_fast=32.0, beta_slow=1.0, mscale=1.0, mscale_all_dim=1.0)

WORKLOADS: Dict[str, MLAShape] = {
    # Tiny fp32 layer: B=1, T=64.
    "tiny_fp32_t64": MLAShape(
        name="tiny_fp32_t64", dtype="f32", hidden=256, num_heads=4, q_lora_rank=64,
        kv_lora_rank=32, qk_nope_dim=32, qk_rope_dim=16, v_head_dim=32,
        rope=RopeSpec(kind="plain", theta=10000.0), num_docs=1, total_tokens=64, seed=1),
    # Megatron-default-style prefill: 2 sequences of 2048, direct q projection.
    "megatron_2x2048": MLAShape(
        name="megatron_2x2048", dtype="bf16", hidden=2048, num_heads=16, q_lora_rank=0,
        kv_lora_rank=512, qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128,
        rope=RopeSpec(kind="plain", theta=10000.0), num_docs=2, total_tokens=4096, seed=2),
    # DeepSeek-V3-shaped prefill: 1 x 4096, 128 heads, YaRN.
    "dsv3_prefill_4096": MLAShape(
        name="dsv3_prefill_4096", dtype="bf16", hidden=7168, num_heads=128, q_lora_rank=1536,
        kv_lora_rank=512, qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128,
        rope=YARN_V3, num_docs=1, total_tokens=4096, seed=3),
    # DeepSeek-V3-shaped absorbed decode: 64 sequences, lengths U[1024, 8192].
    "dsv3_decode_64": MLAShape(
        name="dsv3_decode_64", dtype="bf16", hidden=7168, num_heads=128, q_lora_rank=1536,
        kv_lora_rank=512, qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128,
        rope=YARN_V3, num_docs=64, total_tokens=0, seed=4),
    # Kimi-style gated NoPE prefill: 4 packed documents summing to 8192.
    "kimi_gated_varlen_8192": MLAShape(
        name="kimi_gated_varlen_8192", dtype="bf16", hidden=7168, num_heads=96,
        q_lora_rank=1536, kv_lora_rank=512, qk_nope_dim=128, qk_rope_dim=64, v_head_dim=128,
        rope=RopeSpec(kind="none"), output_gate=True, num_docs=4, total_tokens=8192,
        doc_split="random", seed=5),
}


# --------------------------------------------------------------------------
# Cases
# --------------------------------------------------------------------------
@dataclasses.dataclass
class PrefillCase:
    shape: MLAShape
    x: np.ndarray                   # [N, hidden] float32 (bf16 values for bf16 workloads)
    w: Dict[str, Optional[np.ndarray]]
    cu_seqlens: np.ndarray          # [S+1] int32


@dataclasses.dataclass
class DecodeCase:
    shape: MLAShape
    w_kv_b: np.ndarray              # [H*(nope+v), kv_lora] float32 (bf16 values)
    q_nope: np.ndarray              # [B, H, nope]
    q_pe: np.ndarray                # [B, H, rope]   (already rotated)
    cache: np.ndarray               # [n_blocks, block_size, kv_lora+rope]
    block_table: np.ndarray         # [B, max_blocks] int32, -1 for unused entries
    seq_lens: np.ndarray            # [B] int32
    block_size: int


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def doc_lengths_for(shape: MLAShape, rng: np.random.Generator) -> np.ndarray:
    """Document lengths for a packed prefill batch (draw 10)."""
    t, s = shape.total_tokens, shape.num_docs
    if shape.doc_split == "equal":
        assert t % s == 0
        return np.full(s, t // s, dtype=np.int64)
    cuts = np.sort(rng.choice(np.arange(1, t), size=s - 1, replace=False))
    edges = np.concatenate([[0], cuts, [t]])
    return np.diff(edges).astype(np.int64)


def make_prefill_case(shape: MLAShape, doc_lengths: Optional[Sequence[int]] = None,
                      seed: Optional[int] = None) -> PrefillCase:
    """Seeded prefill inputs.  ``doc_lengths`` overrides the packed layout (the
    draws for x use the overridden total)."""
    rng = np.random.Generator(np.random.PCG64(shape.seed if seed is None else seed))
    n = int(sum(doc_lengths)) if doc_lengths is not None else shape.total_tokens
    h = shape.num_heads
    x = _normal(rng, (n, shape.hidden), 1.0)                                   # 1
    w: Dict[str, Optional[np.ndarray]] = {}
    if shape.q_lora_rank > 0:
        w["w_q_a"] = _normal(rng, (shape.q_lora_rank, shape.hidden), 0.02)     # 2
        w["q_a_gamma"] = np.ones(shape.q_lora_rank, np.float32)                 # 3
        w["w_q_b"] = _normal(rng, (h * shape.qk_head_dim, shape.q_lora_rank), 0.02)  # 4
        w["w_q"] = None
    else:
        w["w_q"] = _normal(rng, (h * shape.qk_head_dim, shape.hidden), 0.02)   # 2
        w["w_q_a"] = w["q_a_gamma"] = w["w_q_b"] = None
    w["w_kv_a"] = _normal(rng, (shape.kv_lora_rank + shape.qk_rope_dim, shape.hidden), 0.02)  # 5
    w["kv_a_gamma"] = np.ones(shape.kv_lora_rank, np.float32)                    # 6
    w["w_kv_b"] = _normal(rng, (h * (shape.qk_nope_dim + shape.v_head_dim), shape.kv_lora_rank), 0.02)  # 7
    w["w_o"] = _normal(rng, (shape.hidden, h * shape.v_head_dim), 0.02)        # 8
    w["w_g"] = _normal(rng, (h * shape.v_head_dim, shape.hidden), 0.02) if shape.output_gate else None  # 9
    if doc_lengths is None:
        lens = doc_lengths_for(shape, rng)                                      # 10
    else:
        lens = np.asarray(doc_lengths, dtype=np.int64)
    if shape.o_groups:
        fg = h * shape.v_head_dim // shape.o_groups
        w["w_o_a"] = _normal(rng, (shape.o_groups * shape.o_lora_rank, fg), 0.02)          # 11
        w["w_o_b"] = _normal(rng, (shape.hidden, shape.o_groups * shape.o_lora_rank), 0.02)  # 12
    else:
        w["w_o_a"] = w["w_o_b"] = None
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    if shape.dtype == "bf16":
        x = bf16_round(x)
        for k, v in list(w.items()):
            if v is not None:
                w[k] = bf16_round(v)
    return PrefillCase(shape=shape, x=x, w=w, cu_seqlens=cu)


def make_decode_case(shape: MLAShape, batch: int = 64, len_lo: int = 1024, len_hi: int = 8192,
                     block_size: int = 64, max_blocks: Optional[int] = None,
                     seq_lens: Optional[Sequence[int]] = None, poison_tail: bool = True,
                     seed: Optional[int] = None) -> DecodeCase:
    """Seeded absorbed-decode inputs: a paged latent cache of ``block_size``-token
    blocks with a permuted block table, lengths U[len_lo, len_hi] inclusive.
    Cache slots past each sequence's length are filled with NaN when
    ``poison_tail`` is set (they must never be read)."""
    rng = np.random.Generator(np.random.PCG64(shape.seed if seed is None else seed))
    h, r, dr = shape.num_heads, shape.kv_lora_rank, shape.qk_rope_dim
    nope, dv = shape.qk_nope_dim, shape.v_head_dim
    # draws 1-9 of the layer are not needed for decode except W_kv_b; keep the
    # documented order by drawing W_kv_b first.
    w_kv_b = _normal(rng, (h * (nope + dv), r), 0.02)                          # 7
    if seq_lens is None:
        lens = rng.integers(len_lo, len_hi, size=batch, endpoint=True)           # 10
    else:
        lens = np.asarray(seq_lens, dtype=np.int64)
        batch = len(lens)
    nblk = (lens + block_size - 1) // block_size
    pool = int(nblk.sum())
    mb = int(nblk.max()) if max_blocks is None else max_blocks
    assert mb >= int(nblk.max())
    perm = rng.permutation(pool).astype(np.int32)                                # 11
    table = np.full((batch, mb), -1, dtype=np.int32)
    o = 0
    for b in range(batch):
        table[b, : nblk[b]] = perm[o: o + nblk[b]]
        o += nblk[b]
    cache = _normal(rng, (pool, block_size, r + dr), 1.0)                        # 12
    q_nope = _normal(rng, (batch, h, nope), 1.0)                                 # 13
    q_pe = _normal(rng, (batch, h, dr), 1.0)
    w_kv_b, cache, q_nope, q_pe = (bf16_round(a) for a in (w_kv_b, cache, q_nope, q_pe))
    if poison_tail:
        for b in range(batch):
            last = nblk[b] - 1
            used = int(lens[b] - last * block_size)
            if used < block_size:
                cache[table[b, last], used:, :] = np.nan
    return DecodeCase(shape=shape, w_kv_b=w_kv_b, q_nope=q_nope, q_pe=q_pe, cache=cache,
                      block_table=table, seq_lens=lens.astype(np.int32), block_size=block_size)


@dataclasses.dataclass
class ChunkCase:
    """New tokens of sequences whose first tokens are already cached."""
    shape: MLAShape
    x: np.ndarray                   # [N, hidden] new tokens, packed by cu_seqlens
    w: Dict[str, Optional[np.ndarray]]
    cu_seqlens: np.ndarray          # [S+1] int32 (new tokens)
    prefix_lens: np.ndarray         # [S] int32 cached tokens per sequence
    cache: np.ndarray               # [n_blocks, block_size, kv_lora+rope] the cached latent rows
    block_table: np.ndarray         # [S, max_blocks] int32, -1 for unused entries
    block_size: int


def make_chunk_case(shape: MLAShape, chunk_lens: Sequence[int], prefix_lens: Sequence[int],
                    block_size: int = 64, max_blocks: Optional[int] = None, poison_tail: bool = True,
                    seed: Optional[int] = None) -> ChunkCase:
    """Seeded inputs of a prefill chunk over a cached prefix: the layer inputs
    of ``make_prefill_case`` for the new tokens (documents = ``chunk_lens``),
    then, from a second stream seeded with seed + 1000, the block permutation
    and the cached latent rows (N(0, 1), the scale of a normalised latent and
    of the shared rope key), bf16 for bf16 workloads.  Each sequence's blocks
    hold only its prefix; slots past it are NaN when ``poison_tail`` is set
    (they must never be read).  A sequence with prefix 0 owns no block."""
    base = make_prefill_case(shape, doc_lengths=chunk_lens, seed=seed)
    pre = np.asarray(prefix_lens, dtype=np.int64)
    assert len(pre) == len(chunk_lens)
    rng = np.random.Generator(np.random.PCG64((shape.seed if seed is None else seed) + 1000))
    width = shape.kv_lora_rank + shape.qk_rope_dim
    nblk = (pre + block_size - 1) // block_size
    pool = max(1, int(nblk.sum()))
    mb = max(1, int(nblk.max())) if max_blocks is None else max_blocks
    assert mb >= int(nblk.max())
    perm = rng.permutation(pool).astype(np.int32)                               # 1
    table = np.full((len(pre), mb), -1, dtype=np.int32)
    o = 0
    for b in range(len(pre)):
        table[b, : nblk[b]] = perm[o: o + nblk[b]]
        o += nblk[b]
    cache = _normal(rng, (pool, block_size, width), 1.0)                        # 2
    if shape.dtype == "bf16":
        cache = bf16_round(cache)
    if poison_tail:
        used = np.zeros(pool, dtype=np.int64)
        for b in range(len(pre)):
            for i in range(nblk[b]):
                used[table[b, i]] = min(block_size, int(pre[b]) - i * block_size)
        for blk in range(pool):
            cache[blk, used[blk]:, :] = np.nan
    return ChunkCase(shape=shape, x=base.x, w=base.w, cu_seqlens=base.cu_seqlens,
                     prefix_lens=pre.astype(np.int32), cache=cache, block_table=table, block_size=block_size)
