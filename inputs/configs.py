"""Seeded synthetic inputs for single-token paged decode.

Recipe (stated once, used by the tests, the bench and the oracle's pins):

* Every tensor value is drawn as float32 from ``numpy.random.default_rng(seed)``
  with ``standard_normal`` and rounded to bfloat16 with round-to-nearest-even.
  bfloat16 tensors are carried as ``uint16`` bit patterns.
* Draw order is fixed: sequence lengths, then the physical-page permutation,
  then q, then the K pool, then the V pool, then (index-gather workloads only)
  the index lists.
* CSR workloads have page size 1, so a page is one token and
  ``kv_indptr[b+1] - kv_indptr[b]`` is the length of sequence ``b``. Pools are
  ``[num_pages, 1, H_kv, D]``; the pages of all sequences are a random
  permutation of the pool, cut in sequence order, so neighbouring tokens of a
  sequence sit at unrelated addresses.
* Block-table workloads have page size ``ps`` > 1 (pools
  ``[num_pages, ps, H_kv, D]``): sequence ``b`` of length ``n`` owns
  ``ceil(n / ps)`` pages, taken in sequence order from a random permutation
  of the pool and listed in row ``b`` of ``block_table``; its last page is
  partly filled when ``ps`` does not divide ``n``. Entries past a row's pages
  hold ``pad_value``.

The five named workloads follow the paged GQA decode definition (32 query heads,
4 KV heads, head_dim 128, page size 1) and the index-gather latent-attention
decode (128 heads over one 576-wide latent KV row whose first 512 dims are V).
The pages name no public benchmark suite; these synthetic inputs stand in for
the kernels' own workloads.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

CONFIG_NAMES = ("tiny", "gqa", "edge", "throughput", "mla", "gqa_ps16", "gqa_ps64", "edge_ps16",
                "mla_fp8")

# Sequence lengths of the edge-case batch: empty, single token, tile edges,
# a long tail and one 32768-token sequence that holds about half the bytes.
EDGE_LENGTHS = (0, 1, 2, 127, 128, 129, 1000, 4095, 4096, 8191, 16384, 32768,
                3, 64, 513, 2049)
EDGE_PEAKY_SEQ = 10      # K of this sequence is multiplied by 30 before rounding
EDGE_CONST_V_SEQ = 7     # V of this sequence is the constant 0.75
EDGE_CONST_V = 0.75


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    rounded = (bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


@dataclasses.dataclass
class GqaWorkload:
    """Inputs of one paged GQA decode call (page size 1)."""

    name: str
    seed: int
    q: np.ndarray            # uint16 bf16 bits [B, Hq, D]
    k_pool: np.ndarray       # uint16 bf16 bits [P, 1, Hkv, D]
    v_pool: np.ndarray       # uint16 bf16 bits [P, 1, Hkv, D]
    kv_indptr: np.ndarray    # int32 [B + 1]
    kv_indices: np.ndarray   # int32 [kv_indptr[B]]
    sm_scale: float
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int = 1

    @property
    def batch(self) -> int:
        return int(self.kv_indptr.shape[0] - 1)

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.kv_indptr[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.kv_indptr.astype(np.int64))


@dataclasses.dataclass
class BlockTableWorkload:
    """Inputs of one paged GQA decode call through a block table."""

    name: str
    seed: int
    q: np.ndarray            # uint16 bf16 bits [B, Hq, D]
    k_pool: np.ndarray       # uint16 bf16 bits [P, ps, Hkv, D]
    v_pool: np.ndarray       # uint16 bf16 bits [P, ps, Hkv, D]
    block_table: np.ndarray  # int32 [B, max_pages]
    seq_lens: np.ndarray     # int32 [B]
    sm_scale: float
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def page_size(self) -> int:
        return int(self.k_pool.shape[1])

    @property
    def num_pages(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())

    @property
    def lengths(self) -> np.ndarray:
        return self.seq_lens.astype(np.int64)

    @property
    def pages_per_seq(self) -> np.ndarray:
        return -(-self.lengths // self.page_size)


@dataclasses.dataclass
class MlaWorkload:
    """Inputs of one index-gather latent-attention decode call."""

    name: str
    seed: int
    q: np.ndarray            # uint16 bf16 bits [B, Hq, Dqk]
    kv_pool: np.ndarray      # uint16 bf16 bits [T, Dqk]
    indices: np.ndarray      # int32 [B, topk]; -1 marks a masked entry
    sm_scale: float
    d_v: int

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_qo_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def d_qk(self) -> int:
        return int(self.q.shape[2])

    @property
    def pool_tokens(self) -> int:
        return int(self.kv_pool.shape[0])

    @property
    def topk(self) -> int:
        return int(self.indices.shape[1])


def lognormal_lengths(rng: np.random.Generator, batch: int, median: float = 1024.0,
                      sigma: float = 1.0, lo: int = 1, hi: int = 16384) -> np.ndarray:
    """Lengths ``clip(rint(exp(N(ln median, sigma))), lo, hi)``."""
    z = rng.normal(math.log(median), sigma, size=batch)
    return np.clip(np.rint(np.exp(z)), lo, hi).astype(np.int64)


def _draw_bf16(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_gqa(seed: int, lengths: Sequence[int], *, num_qo_heads: int = 32,
             num_kv_heads: int = 4, head_dim: int = 128, pool_pages: Optional[int] = None,
             peaky_seq: Optional[int] = None, peaky_factor: float = 30.0,
             const_v_seq: Optional[int] = None, const_v: float = EDGE_CONST_V,
             sm_scale: Optional[float] = None, name: str = "custom",
             rng: Optional[np.random.Generator] = None) -> GqaWorkload:
    """Build one paged GQA decode input.

    ``pool_pages`` defaults to the total token count. With a larger pool the
    indices are the first ``sum(lengths)`` entries of a permutation of the
    pool, so some pages are never referenced.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    batch = int(lengths.shape[0])
    total = int(lengths.sum())
    pages = total if pool_pages is None else int(pool_pages)
    if pages < total:
        raise ValueError("pool smaller than the number of tokens")
    perm = rng.permutation(max(pages, 0)).astype(np.int32)
    indices = perm[:total].copy()
    indptr = np.zeros(batch + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(lengths)

    q32 = _draw_bf16(rng, (batch, num_qo_heads, head_dim))
    k32 = _draw_bf16(rng, (pages, 1, num_kv_heads, head_dim))
    if peaky_seq is not None:
        sel = indices[indptr[peaky_seq]:indptr[peaky_seq + 1]]
        k32[sel] *= np.float32(peaky_factor)
    k_bits = bf16_bits_from_f32(k32)
    del k32
    v32 = _draw_bf16(rng, (pages, 1, num_kv_heads, head_dim))
    if const_v_seq is not None:
        sel = indices[indptr[const_v_seq]:indptr[const_v_seq + 1]]
        v32[sel] = np.float32(const_v)
    v_bits = bf16_bits_from_f32(v32)
    del v32
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    return GqaWorkload(name=name, seed=seed, q=bf16_bits_from_f32(q32), k_pool=k_bits,
                       v_pool=v_bits, kv_indptr=indptr, kv_indices=indices,
                       sm_scale=float(sm_scale), num_qo_heads=num_qo_heads,
                       num_kv_heads=num_kv_heads, head_dim=head_dim)


def make_block_table(seed: int, lengths: Sequence[int], page_size: int, *,
                     num_qo_heads: int = 32, num_kv_heads: int = 4, head_dim: int = 128,
                     pool_pages: Optional[int] = None, extra_cols: int = 0,
                     pad_value: int = 0, peaky_seq: Optional[int] = None,
                     peaky_factor: float = 30.0, const_v_seq: Optional[int] = None,
                     const_v: float = EDGE_CONST_V, sm_scale: Optional[float] = None,
                     name: str = "custom",
                     rng: Optional[np.random.Generator] = None) -> BlockTableWorkload:
    """Build one paged GQA decode input addressed through a block table.

    ``pool_pages`` defaults to the pages the batch needs; with a larger pool
    some pages are never referenced. The table has ``max(pages) + extra_cols``
    columns; unused entries hold ``pad_value``. The peaky / constant-V edits
    cover every slot of the chosen sequence's pages.
    """
    if rng is None:
        rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    batch = int(lengths.shape[0])
    need = -(-lengths // page_size)
    total_pages = int(need.sum())
    pages = total_pages if pool_pages is None else int(pool_pages)
    if pages < total_pages:
        raise ValueError("pool smaller than the number of pages the batch needs")
    perm = rng.permutation(max(pages, 0)).astype(np.int32)
    cols = int(need.max(initial=0)) + int(extra_cols)
    table = np.full((batch, cols), pad_value, dtype=np.int32)
    first = np.concatenate([[0], np.cumsum(need)])
    for b in range(batch):
        table[b, :need[b]] = perm[first[b]:first[b + 1]]

    q32 = _draw_bf16(rng, (batch, num_qo_heads, head_dim))
    k32 = _draw_bf16(rng, (pages, page_size, num_kv_heads, head_dim))
    if peaky_seq is not None:
        k32[table[peaky_seq, :need[peaky_seq]]] *= np.float32(peaky_factor)
    k_bits = bf16_bits_from_f32(k32)
    del k32
    v32 = _draw_bf16(rng, (pages, page_size, num_kv_heads, head_dim))
    if const_v_seq is not None:
        v32[table[const_v_seq, :need[const_v_seq]]] = np.float32(const_v)
    v_bits = bf16_bits_from_f32(v32)
    del v32
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(head_dim)
    return BlockTableWorkload(name=name, seed=seed, q=bf16_bits_from_f32(q32), k_pool=k_bits,
                              v_pool=v_bits, block_table=table,
                              seq_lens=lengths.astype(np.int32), sm_scale=float(sm_scale),
                              num_qo_heads=num_qo_heads, num_kv_heads=num_kv_heads,
                              head_dim=head_dim)


def make_mla(seed: int, *, batch: int = 32, num_qo_heads: int = 128, d_qk: int = 576,
             d_v: int = 512, pool_tokens: int = 65536, topk: int = 2048,
             masked_per_row: Optional[int] = None, sm_scale: Optional[float] = None,
             name: str = "custom") -> MlaWorkload:
    """Build one index-gather decode input.

    Each row's list holds ``topk`` distinct ids drawn uniformly without
    replacement from the pool; then ``masked_per_row`` positions of the row,
    chosen uniformly without replacement, are set to -1.
    """
    rng = np.random.default_rng(seed)
    if masked_per_row is None:
        masked_per_row = int(round(0.05 * topk))
    q32 = _draw_bf16(rng, (batch, num_qo_heads, d_qk))
    kv32 = _draw_bf16(rng, (pool_tokens, d_qk))
    idx = np.empty((batch, topk), dtype=np.int32)
    for b in range(batch):
        idx[b] = rng.choice(pool_tokens, size=topk, replace=False).astype(np.int32)
        if masked_per_row:
            pos = rng.choice(topk, size=masked_per_row, replace=False)
            idx[b, pos] = -1
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d_qk)
    return MlaWorkload(name=name, seed=seed, q=bf16_bits_from_f32(q32),
                       kv_pool=bf16_bits_from_f32(kv32), indices=idx,
                       sm_scale=float(sm_scale), d_v=d_v)


FP8_TOKEN_BYTES = 656   # 512 e4m3 values, 4 fp32 scales, 64 bf16 values


@dataclasses.dataclass
class MlaFp8Workload:
    """Inputs of one index-gather decode call over an FP8 latent pool."""

    name: str
    seed: int
    q: np.ndarray            # uint16 bf16 bits [B, Hq, 576]
    kv_pool: np.ndarray      # uint8 [T, 656]: e4m3 [0:512), fp32 scales [512:528), bf16 [528:656)
    indices: np.ndarray      # int32 [B, topk]; -1 marks a masked entry
    sm_scale: float
    d_v: int = 512

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_qo_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def d_qk(self) -> int:
        return int(self.q.shape[2])

    @property
    def pool_tokens(self) -> int:
        return int(self.kv_pool.shape[0])

    @property
    def topk(self) -> int:
        return int(self.indices.shape[1])


def encode_fp8_rows(x: np.ndarray) -> np.ndarray:
    """Pack float32 latent rows ``[T, 576]`` into 656-byte FP8 tokens.

    Dims 0..511 are stored as e4m3 (OCP ``float8_e4m3fn``, via torch's
    round-to-nearest conversion) of ``x / scale`` with one fp32 scale per 128
    dims, ``scale = max|x| / 448`` over those dims (1 for an all-zero block);
    dims 512..575 are stored as bf16. This builds cache contents only; the
    decode reads them back.
    """
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    t = x.shape[0]
    nope = x[:, :512].reshape(t, 4, 128)
    amax = np.abs(nope).max(axis=2)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    scaled = (nope / scale[:, :, None]).reshape(t, 512)
    codes = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    out = np.empty((t, FP8_TOKEN_BYTES), dtype=np.uint8)
    out[:, :512] = codes
    out[:, 512:528] = scale.view(np.uint8).reshape(t, 16)
    out[:, 528:656] = bf16_bits_from_f32(x[:, 512:576]).view(np.uint8).reshape(t, 128)
    return out


def make_mla_fp8(seed: int, *, batch: int = 32, num_qo_heads: int = 128,
                 pool_tokens: int = 65536, topk: int = 2048,
                 masked_per_row: Optional[int] = None, sm_scale: Optional[float] = None,
                 name: str = "custom") -> MlaFp8Workload:
    """Build one index-gather decode input over an FP8 pool (same recipe as
    ``make_mla``, the latent rows then packed by ``encode_fp8_rows``)."""
    rng = np.random.default_rng(seed)
    if masked_per_row is None:
        masked_per_row = int(round(0.05 * topk))
    q32 = _draw_bf16(rng, (batch, num_qo_heads, 576))
    kv32 = _draw_bf16(rng, (pool_tokens, 576))
    idx = np.empty((batch, topk), dtype=np.int32)
    for b in range(batch):
        idx[b] = rng.choice(pool_tokens, size=topk, replace=False).astype(np.int32)
        if masked_per_row:
            pos = rng.choice(topk, size=masked_per_row, replace=False)
            idx[b, pos] = -1
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(576)
    return MlaFp8Workload(name=name, seed=seed, q=bf16_bits_from_f32(q32),
                          kv_pool=encode_fp8_rows(kv32), indices=idx, sm_scale=float(sm_scale))


def make_config(name: str):
    """The named workloads: five with page size 1 (seeds 1..5), three
    block-table workloads with page size 16 or 64 (seeds 6..8) and the
    index-gather workload over an FP8 pool (seed 10)."""
    if name == "tiny":
        return make_gqa(1, [17, 64], pool_pages=128, name="tiny")
    if name == "gqa":
        rng = np.random.default_rng(2)
        lengths = rng.integers(512, 4096, size=64, endpoint=True)
        return make_gqa(2, lengths, name="gqa", rng=rng)
    if name == "edge":
        return make_gqa(3, EDGE_LENGTHS, peaky_seq=EDGE_PEAKY_SEQ,
                        const_v_seq=EDGE_CONST_V_SEQ, name="edge")
    if name == "throughput":
        rng = np.random.default_rng(4)
        lengths = lognormal_lengths(rng, 256)
        return make_gqa(4, lengths, name="throughput", rng=rng)
    if name == "mla":
        return make_mla(5, name="mla")
    if name in ("gqa_ps16", "gqa_ps64"):
        seed, ps = (6, 16) if name == "gqa_ps16" else (7, 64)
        rng = np.random.default_rng(seed)
        lengths = rng.integers(512, 4096, size=64, endpoint=True)
        return make_block_table(seed, lengths, ps, name=name, rng=rng)
    if name == "mla_fp8":
        return make_mla_fp8(10, name="mla_fp8")
    if name == "edge_ps16":
        return make_block_table(8, EDGE_LENGTHS, 16, peaky_seq=EDGE_PEAKY_SEQ,
                                const_v_seq=EDGE_CONST_V_SEQ, name="edge_ps16")
    raise KeyError(name)
