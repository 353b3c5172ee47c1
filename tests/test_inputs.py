"""The seeded input generators: rounding, determinism and workload structure."""

import hashlib

import numpy as np
import torch

from inputs import bf16_bits_from_f32, lognormal_lengths, make_config
from inputs.configs import EDGE_LENGTHS


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -2.5, 0.0, -0.0, 1e-40, 3e38],
                                 dtype=np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_f32(x), want)
    # ties go to even: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7
    assert bf16_bits_from_f32(np.array([1.00390625], np.float32))[0] == 0x3F80
    assert bf16_bits_from_f32(np.array([1.01171875], np.float32))[0] == 0x3F82


def _digest(w):
    h = hashlib.sha256()
    for a in (w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_determinism():
    assert _digest(make_config("tiny")) == _digest(make_config("tiny"))


def test_tiny_structure():
    w = make_config("tiny")
    assert list(w.lengths) == [17, 64] and w.num_pages == 128
    assert len(set(w.kv_indices.tolist())) == 81
    assert w.q.shape == (2, 32, 128) and w.k_pool.shape == (128, 1, 4, 128)
    assert abs(w.sm_scale - 128 ** -0.5) < 1e-15


def test_gqa_structure():
    w = make_config("gqa")
    assert w.batch == 64 and w.lengths.min() >= 512 and w.lengths.max() <= 4096
    assert np.array_equal(np.sort(w.kv_indices), np.arange(w.total_tokens))


def test_edge_structure():
    w = make_config("edge")
    assert tuple(w.lengths) == EDGE_LENGTHS and w.total_tokens == 69550
    assert np.array_equal(np.sort(w.kv_indices), np.arange(69550))
    pages = w.kv_indices[w.kv_indptr[7]:w.kv_indptr[8]]
    assert np.all(w.v_pool[pages] == 0x3F40)      # 0.75


def test_throughput_lengths():
    n = lognormal_lengths(np.random.default_rng(4), 256)
    assert n.min() >= 1 and n.max() <= 16384
    assert 200_000 < n.sum() < 700_000


def test_mla_structure():
    w = make_config("mla")
    assert w.q.shape == (32, 128, 576) and w.kv_pool.shape == (65536, 576)
    assert w.indices.shape == (32, 2048)
    for b in range(32):
        row = w.indices[b]
        assert int((row == -1).sum()) == 102
        kept = row[row >= 0]
        assert len(np.unique(kept)) == len(kept) and kept.max() < 65536


def test_block_table_structure():
    for name, ps in (("gqa_ps16", 16), ("gqa_ps64", 64), ("edge_ps16", 16)):
        w = make_config(name)
        assert w.page_size == ps and w.k_pool.shape[1:] == (ps, 4, 128)
        need = w.pages_per_seq
        assert w.block_table.shape == (w.batch, need.max())
        used = np.concatenate([w.block_table[b, :need[b]] for b in range(w.batch)])
        assert np.array_equal(np.sort(used), np.arange(w.num_pages))   # each page once
    w = make_config("edge_ps16")
    assert tuple(w.lengths) == EDGE_LENGTHS
    pages = w.block_table[7, :w.pages_per_seq[7]]
    assert np.all(w.v_pool[pages] == 0x3F40)


def test_block_table_padding_and_extra_columns():
    from inputs import make_block_table
    w = make_block_table(9, [0, 1, 16, 17], 16, extra_cols=2, pad_value=-1, pool_pages=10)
    assert list(w.pages_per_seq) == [0, 1, 1, 2]
    assert w.block_table.shape == (4, 4) and w.num_pages == 10
    assert np.all(w.block_table[0] == -1) and np.all(w.block_table[3, 2:] == -1)


def test_fp8_pool_encoding():
    """The packed FP8 tokens decode close to the drawn values (e4m3 keeps 3
    mantissa bits: error <= 2^-4 of the block's max per value, plus bf16)."""
    from inputs import encode_fp8_rows
    from oracle import ref
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 576)).astype(np.float32)
    x[3, :128] = 0.0                                  # an all-zero block keeps scale 1
    tok = encode_fp8_rows(x)
    assert tok.shape == (50, 656) and tok.dtype == np.uint8
    scales = tok[:, 512:528].copy().view(np.float32).reshape(50, 4)
    assert scales[3, 0] == 1.0
    dq = ref.bf16_to_f64(ref.dequant_fp8_rows(tok))
    amax = np.abs(x[:, :512]).reshape(50, 4, 128).max(axis=2)
    err = np.abs(dq[:, :512] - x[:, :512]).reshape(50, 4, 128)
    assert np.all(err <= amax[:, :, None] * 2.0 ** -4 + 1e-30)
    assert np.array_equal(ref.dequant_fp8_rows(tok)[:, 512:], bf16_bits_from_f32(x[:, 512:]))
