"""fp64 CPU oracle for single-token paged attention decode.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the library. It shares no code with the HIP
path and reads the inputs only as raw bfloat16 bit patterns.

Sources (page title, then the function or step on it):

* [GQA page] kernelindex.com, "flashinfer gemini-2.5-pro / triton h7ykt0":
  the kernel ``gqa_paged_decode_h32_kv4_d128_ps1_kernel`` (its numbered steps
  2, 4, 7, 8 and 9) and its wrapper ``run``.
* [MLA page] FlagGems docs, coverage page of ``flash_mla_with_kvcache.py``:
  ``_sparse_decode_kernel`` (index masking, the 576/512 latent split, the
  656-byte FP8 token and its dequantisation) and
  ``_dense_decode_kernel`` (pages of several tokens found through a block
  table, sequence lengths that end inside a page).
* [QSA page] vLLM fork, ``vllm/models/qwen4_exp/amd/ops/qsa.py``:
  ``_qsa_sparse_paged_gqa_splitk_kernel`` (normalised partials with a base-2
  LSE), ``_qsa_merge_splitk_kernel`` (the LSE merge) and
  ``qsa_store_cache_rows`` / ``_store_qsa_rows_kernel`` (storing new rows at
  slot positions of a paged cache).

What is computed, for one query row q_h and the rows k_j, v_j it attends to:

    s_j   = sm_scale * (q_h . k_j)
    out_h = sum_j exp(s_j) v_j / sum_j exp(s_j)
    lse_h = log2( sum_j exp(s_j) )

The online softmax and split-KV of the kernels only reorder this sum. Here the
largest score is subtracted before ``exp`` purely to keep fp64 in range. With
no rows, out = 0 and lse = -inf ([GQA page] step 4). Every pin of this module
lives in ``tests/test_oracle.py``.
"""

from __future__ import annotations

import math

import numpy as np

LN2 = math.log(2.0)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns: the 16 bits are the top half of a float32."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """Softmax attention of the query rows ``q [H, Dqk]`` over ``k [n, Dqk]``, ``v [n, Dv]``.

    Returns ``out [H, Dv]`` (fp64) and the base-2 log-sum-exp ``lse [H]``.
    Follows [GQA page] steps 8b-9: scores scaled by ``sm_scale`` in floating
    point, normalised exponentials, base-2 LSE of the natural-exp sum; and
    step 4 for ``n == 0``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    h = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((h, v.shape[1])), np.full(h, -np.inf)
    s = sm_scale * (q @ k.T)                      # [H, n]
    m = s.max(axis=1, keepdims=True)              # only keeps exp() in range
    w = np.exp(s - m)                             # [H, n]
    z = w.sum(axis=1)                             # [H]
    out = (w @ v) / z[:, None]
    lse = (m[:, 0] + np.log(z)) / LN2
    return out, lse


def gqa_group_of(head: int, num_qo_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``head``: consecutive groups of Hq/Hkv heads share one.

    [GQA page] step 7 (``offs_h // gqa_ratio``); [QSA page] partial kernel
    (``first_head = kv_head * GROUP_SIZE``).
    """
    return head // (num_qo_heads // num_kv_heads)


def gqa_decode_range(q_bits, k_bits, v_bits, kv_indptr, kv_indices, sm_scale: float,
                     b: int, tok_begin: int, tok_end: int):
    """Attention of sequence ``b`` over its tokens ``[tok_begin, tok_end)``.

    Pages are looked up through the CSR list: token ``j`` of sequence ``b`` is
    page ``kv_indices[kv_indptr[b] + j]`` ([GQA page] steps 2 and 8a). With page
    size 1 the page holds exactly that token. Returns ``out [Hq, D]``, ``lse [Hq]``.
    """
    num_qo_heads, head_dim = q_bits.shape[1], q_bits.shape[2]
    num_kv_heads = k_bits.shape[2]
    base = int(kv_indptr[b])
    pages = np.asarray(kv_indices[base + tok_begin: base + tok_end], dtype=np.int64)
    q = bf16_to_f64(q_bits[b])                                   # [Hq, D]
    out = np.zeros((num_qo_heads, v_bits.shape[3]))
    lse = np.full(num_qo_heads, -np.inf)
    for g in range(num_kv_heads):
        heads = [h for h in range(num_qo_heads)
                 if gqa_group_of(h, num_qo_heads, num_kv_heads) == g]
        k = bf16_to_f64(k_bits[pages, 0, g, :])                  # [n, D]
        v = bf16_to_f64(v_bits[pages, 0, g, :])
        o_g, l_g = attend(q[heads], k, v, sm_scale)
        out[heads] = o_g
        lse[heads] = l_g
    return out, lse


def gqa_paged_decode(q_bits, k_bits, v_bits, kv_indptr, kv_indices, sm_scale: float,
                     batches=None):
    """Paged GQA decode of every sequence (or of the listed ``batches``).

    ``q_bits [B, Hq, D]``; pools ``[P, 1, Hkv, D]``; all bfloat16 bits.
    Returns ``out [B, Hq, D]`` and ``lse [B, Hq]`` in fp64 (rows not listed in
    ``batches`` are left as NaN).
    """
    batch = q_bits.shape[0]
    num_qo_heads = q_bits.shape[1]
    out = np.full((batch, num_qo_heads, v_bits.shape[3]), np.nan)
    lse = np.full((batch, num_qo_heads), np.nan)
    for b in (range(batch) if batches is None else batches):
        n = int(kv_indptr[b + 1]) - int(kv_indptr[b])
        out[b], lse[b] = gqa_decode_range(q_bits, k_bits, v_bits, kv_indptr, kv_indices,
                                          sm_scale, b, 0, n)
    return out, lse


def gqa_block_table_decode(q_bits, k_bits, v_bits, block_table, seq_lens, sm_scale: float,
                           batches=None):
    """Paged GQA decode with pages of several tokens, found through a block table.

    Pools are ``[P, page_size, Hkv, D]``. Sequence ``b`` has ``seq_lens[b]``
    tokens; its token ``j`` sits in page ``block_table[b, j // page_size]`` at
    slot ``j % page_size`` ([MLA page] ``_dense_decode_kernel``: the page
    number from the table, the row inside the page from the remainder, and the
    tokens past the sequence length masked). Only the first
    ``ceil(seq_lens[b] / page_size)`` entries of a table row are read, and in
    the last page only the slots below the length. Per KV head the attention is
    the same as with single-token pages. Returns ``out [B, Hq, D]`` and
    ``lse [B, Hq]`` in fp64 (rows not listed in ``batches`` are NaN).
    """
    batch, num_qo_heads, _ = q_bits.shape
    page_size, num_kv_heads = k_bits.shape[1], k_bits.shape[2]
    out = np.full((batch, num_qo_heads, v_bits.shape[3]), np.nan)
    lse = np.full((batch, num_qo_heads), np.nan)
    for b in (range(batch) if batches is None else batches):
        j = np.arange(int(seq_lens[b]), dtype=np.int64)
        pages = np.asarray(block_table[b], dtype=np.int64)[j // page_size]
        slots = j % page_size
        q = bf16_to_f64(q_bits[b])
        for g in range(num_kv_heads):
            heads = [h for h in range(num_qo_heads)
                     if gqa_group_of(h, num_qo_heads, num_kv_heads) == g]
            k = bf16_to_f64(k_bits[pages, slots, g, :])          # [n, D]
            v = bf16_to_f64(v_bits[pages, slots, g, :])
            out[b, heads], lse[b, heads] = attend(q[heads], k, v, sm_scale)
    return out, lse


def kv_append(k_pool, v_pool, k_rows, v_rows, slot_mapping):
    """Store new K/V rows into paged pools at flat slot positions.

    Pools are ``[P, page_size, Hkv, D]`` and rows ``[n, Hkv, D]`` (any dtype;
    the rows are copied bit for bit). Row ``i`` goes to page
    ``slot // page_size``, position ``slot % page_size`` with
    ``slot = slot_mapping[i]``; a slot outside ``[0, P * page_size)`` (e.g.
    -1 for padding) stores nothing ([QSA page] ``_store_qsa_rows_kernel``:
    the validity test, page and position from the quotient and remainder).
    Rows are applied in order. Returns new pools; the inputs are not modified.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    num_pages, page_size = k_out.shape[0], k_out.shape[1]
    for i, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64).tolist()):
        if 0 <= slot < num_pages * page_size:
            k_out[slot // page_size, slot % page_size] = k_rows[i]
            v_out[slot // page_size, slot % page_size] = v_rows[i]
    return k_out, v_out


def merge_lse2(parts_out: np.ndarray, parts_lse: np.ndarray):
    """Combine normalised partial results over disjoint key sets.

    ``parts_out [S, H, D]`` holds each part's normalised output and
    ``parts_lse [S, H]`` its base-2 LSE (-inf for a part with no keys). Weights
    are ``2^(lse_i - max lse)``; the output is the weighted mean and the merged
    LSE is ``max + log2(sum of weights)``. All parts empty gives 0 and -inf.
    [QSA page] ``_qsa_merge_splitk_kernel``; the merged LSE is not written
    there, it is the same log-sum-exp identity taken one step further.
    """
    parts_out = np.asarray(parts_out, dtype=np.float64)
    parts_lse = np.asarray(parts_lse, dtype=np.float64)
    top = parts_lse.max(axis=0)                                  # [H]
    empty = np.isneginf(top)
    safe_top = np.where(empty, 0.0, top)
    w = np.where(np.isneginf(parts_lse), 0.0, np.exp2(parts_lse - safe_top[None, :]))
    den = w.sum(axis=0)
    out = np.einsum("sh,shd->hd", w, parts_out) / np.where(empty, 1.0, den)[:, None]
    out[empty] = 0.0
    lse = np.where(empty, -np.inf, safe_top + np.log2(np.where(empty, 1.0, den)))
    return out, lse


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Decode OCP float8 e4m3 ("fn") codes: 1 sign bit, 4 exponent bits with
    bias 7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111
    is NaN and there is no infinity."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e > 0, (1.0 + m / 8.0) * np.exp2(e - 7.0), (m / 8.0) * 2.0 ** -6)
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def _f32_to_bf16_bits(x) -> np.ndarray:
    """float32 -> bfloat16 bit pattern, round to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def dequant_fp8_rows(tokens: np.ndarray) -> np.ndarray:
    """656-byte FP8 tokens ``[n, 656]`` -> bf16 bit patterns ``[n, 576]``.

    [MLA page] FP8 sparse mode: bytes 0..511 are e4m3 values, bytes 512..527
    four float32 scales (scale j for values 128j..128j+127), bytes 528..655
    64 bfloat16 values. Value i is ``e4m3[i] * scale[i // 128]``, multiplied
    in float32 and then rounded to bfloat16 (the page converts the product to
    bf16 before both matrix products); the last 64 dims are the bf16 values
    as stored.
    """
    tokens = np.ascontiguousarray(tokens, dtype=np.uint8)
    n = tokens.shape[0]
    vals = e4m3_to_f64(tokens[:, :512]).astype(np.float32)        # exact in float32
    scales = tokens[:, 512:528].copy().view(np.float32).reshape(n, 4)
    prod = (vals.reshape(n, 4, 128) * scales[:, :, None]).reshape(n, 512)   # float32 product
    out = np.empty((n, 576), dtype=np.uint16)
    out[:, :512] = _f32_to_bf16_bits(prod)
    out[:, 512:] = tokens[:, 528:656].copy().view(np.uint16).reshape(n, 64)
    return out


def mla_gather_decode_fp8(q_bits, kv_tokens, indices, sm_scale: float, d_v: int = 512,
                          batches=None, attn_sink=None, topk_length=None):
    """Index-gather decode over an FP8 latent pool ``[T, 656]`` (uint8).

    Each selected token is dequantised to 576 bf16 values (``dequant_fp8_rows``);
    from there the decode is ``mla_gather_decode``: scores over all 576 dims,
    values the first 512 ([MLA page]: the dequantised part serves as both K
    and V). Only listed rows need dequantising; the result is the same as
    dequantising the whole pool.
    """
    ids = np.asarray(indices, dtype=np.int64)
    pool_tokens = kv_tokens.shape[0]
    used = np.unique(ids[(ids >= 0) & (ids < pool_tokens)])
    pool = np.zeros((pool_tokens, 576), dtype=np.uint16)
    pool[used] = dequant_fp8_rows(kv_tokens[used])
    return mla_gather_decode(q_bits, pool, indices, sm_scale, d_v, batches=batches,
                             attn_sink=attn_sink, topk_length=topk_length)


def mla_gather_decode(q_bits, kv_bits, indices, sm_scale: float, d_v: int,
                      batches=None, attn_sink=None, topk_length=None):
    """Index-gather latent-attention decode.

    For row ``b`` the keys are the pool rows ``kv[t]`` for every list entry
    ``t = indices[b, i]`` with ``0 <= t < T``; entries outside that range are
    masked and contribute nothing ([MLA page] ``_sparse_decode_kernel``, index
    masking). Scores use all ``Dqk`` dims; the values are the first ``d_v``
    dims of the same row. Every entry counts, repeated ids included.

    ``topk_length`` (int per row, optional): only the first
    ``min(max(topk_length[b], 0), topk)`` entries of row ``b`` are read
    ([MLA page] ``HAVE_TOPK_LENGTH``: entries at or past the length masked).

    ``attn_sink`` (float per query head, optional): a logit, in the same
    natural-log units as ``sm_scale * q.k``, that joins the softmax
    denominator with no value: ``out = sum_j e^(s_j) v_j / (sum_j e^(s_j) +
    e^(sink_h))`` ([MLA page] ``HAVE_ATTN_SINK``: the output factor
    ``exp(max) / (exp(lse) + exp(sink))``). The returned LSE is that of the
    entries alone, as the page stores it before the sink is applied.
    Returns ``out [B, Hq, d_v]`` and base-2 ``lse [B, Hq]``.
    """
    batch, num_qo_heads, _ = q_bits.shape
    pool_tokens = kv_bits.shape[0]
    topk = indices.shape[1]
    out = np.full((batch, num_qo_heads, d_v), np.nan)
    lse = np.full((batch, num_qo_heads), np.nan)
    for b in (range(batch) if batches is None else batches):
        length = topk if topk_length is None else min(max(int(topk_length[b]), 0), topk)
        ids = np.asarray(indices[b][:length], dtype=np.int64)
        ids = ids[(ids >= 0) & (ids < pool_tokens)]
        rows = bf16_to_f64(kv_bits[ids])                         # [n, Dqk]
        q = bf16_to_f64(q_bits[b])
        if attn_sink is None or len(ids) == 0:
            out[b], lse[b] = attend(q, rows, rows[:, :d_v], sm_scale)
            continue
        sink = np.asarray(attn_sink, dtype=np.float64)            # [Hq]
        s = sm_scale * (q @ rows.T)                               # [Hq, n]
        m = s.max(axis=1)                                         # only keeps exp() in range
        w = np.exp(s - m[:, None])
        z_keys = w.sum(axis=1)
        out[b] = (w @ rows[:, :d_v]) / (z_keys + np.exp(sink - m))[:, None]
        lse[b] = (m + np.log(z_keys)) / LN2
    return out, lse
