"""Randomised parity sweep on the GPU against the fp64 oracle: seeded random
batch shapes, lengths (with empty sequences), split settings, page sizes,
pool slack, gather list lengths, masking, sinks and row lengths. Each case is
small enough for the oracle to finish quickly. Tolerances as in the other
GPU tests: |out - ref| <= 1e-2 + 1e-2 |ref|, |lse - ref| <= 1e-3, -inf where
the oracle has -inf.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_gqa_amd as pkv
from gpu_util import assert_lse_close, assert_out_close, bf16_to_np, to_dev, upload_gqa
from inputs import make_block_table, make_gqa, make_mla, make_mla_fp8
from oracle import ref

pytestmark = pytest.mark.gpu


def check(want, got, what):
    assert_out_close(got[0], want[0], what + " out")
    assert_lse_close(got[1], want[1], what + " lse")


def random_lengths(rng, batch, max_len):
    lengths = rng.integers(0, max_len + 1, size=batch)
    lengths[rng.random(batch) < 0.15] = 0
    return [int(x) for x in lengths]


@pytest.mark.parametrize("engine", ["mfma", "dot2"])
@pytest.mark.parametrize("seed", range(12))
def test_random_csr_decode(seed, engine):
    rng = np.random.default_rng(1000 + seed)
    batch = int(rng.integers(1, 40))
    lengths = random_lengths(rng, batch, int(rng.choice([40, 300, 3000])))
    if sum(lengths) == 0:
        lengths[0] = 1
    w = make_gqa(2000 + seed, lengths, pool_pages=sum(lengths) + int(rng.integers(0, 50)))
    split = bool(rng.random() < 0.8)
    chunk = int(rng.choice([0, 0, 32, 64, 100, 512]))
    dev = upload_gqa(w)
    out, lse = pkv.decode(dev["q"], dev["k"], dev["v"], dev["indptr"], dev["indices"], w.sm_scale,
                          kv_indptr_host=w.kv_indptr, allow_split=split, chunk_tokens=chunk,
                          engine=engine)
    torch.cuda.synchronize()
    want = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices, w.sm_scale)
    check(want, (bf16_to_np(out), lse.cpu().numpy().astype(np.float64)),
          f"csr {engine} seed={seed} B={batch} split={split} chunk={chunk}")


@pytest.mark.parametrize("engine", ["mfma", "dot2"])
@pytest.mark.parametrize("seed", range(10))
def test_random_block_table_decode(seed, engine):
    rng = np.random.default_rng(3000 + seed)
    batch = int(rng.integers(1, 30))
    ps = int(rng.choice([2, 8, 16, 64, 256]))
    lengths = random_lengths(rng, batch, int(rng.choice([50, 700, 2500])))
    pages = sum(-(-n // ps) for n in lengths)
    w = make_block_table(4000 + seed, lengths, ps, pool_pages=max(1, pages + int(rng.integers(0, 9))),
                         extra_cols=int(rng.integers(0, 3)))
    chunk = int(rng.choice([0, 0, 64, 160]))
    out, lse = pkv.decode_block_table(to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool),
                                      to_dev(w.block_table), w.seq_lens, w.sm_scale,
                                      chunk_tokens=chunk, engine=engine)
    torch.cuda.synchronize()
    want = ref.gqa_block_table_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens,
                                      w.sm_scale)
    check(want, (bf16_to_np(out), lse.cpu().numpy().astype(np.float64)),
          f"table {engine} seed={seed} B={batch} ps={ps} chunk={chunk}")


@pytest.mark.parametrize("seed", range(10))
@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_random_gather(seed, fp8):
    rng = np.random.default_rng(5000 + seed + (100 if fp8 else 0))
    batch = int(rng.integers(1, 6))
    heads = int(rng.choice([16, 48, 64, 128]))
    topk = int(rng.choice([1, 17, 64, 200, 777]))
    pool = int(rng.integers(topk, topk + 2000))
    masked = int(rng.integers(0, topk // 3 + 1))
    make = make_mla_fp8 if fp8 else make_mla
    w = make(6000 + seed, batch=batch, num_qo_heads=heads, pool_tokens=pool, topk=topk,
             masked_per_row=masked)
    sink = (rng.normal(size=heads) * 2).astype(np.float32) if rng.random() < 0.5 else None
    length = rng.integers(-3, topk + 5, size=batch).astype(np.int32) if rng.random() < 0.5 else None
    fn = pkv.gather_mla_fp8 if fp8 else pkv.gather_mla
    out, lse = fn(to_dev(w.q), to_dev(w.kv_pool), to_dev(w.indices), w.sm_scale,
                  attn_sink=None if sink is None else to_dev(sink),
                  topk_length=None if length is None else to_dev(length))
    torch.cuda.synchronize()
    oracle = ref.mla_gather_decode_fp8 if fp8 else ref.mla_gather_decode
    want = oracle(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v, attn_sink=sink, topk_length=length)
    check(want, (bf16_to_np(out), lse.cpu().numpy().astype(np.float64)),
          f"gather fp8={fp8} seed={seed} B={batch} H={heads} topk={topk} sink={sink is not None} "
          f"len={length is not None}")


@pytest.mark.parametrize("seed", range(6))
def test_random_append(seed):
    rng = np.random.default_rng(7000 + seed)
    ps = int(rng.choice([1, 4, 16, 64]))
    pages = int(rng.integers(1, 60))
    total = pages * ps
    n = int(rng.integers(0, total + 5))
    k_pool = rng.integers(0, 1 << 16, size=(pages, ps, 4, 128), dtype=np.uint16)
    v_pool = rng.integers(0, 1 << 16, size=(pages, ps, 4, 128), dtype=np.uint16)
    k_rows = rng.integers(0, 1 << 16, size=(n, 4, 128), dtype=np.uint16)
    v_rows = rng.integers(0, 1 << 16, size=(n, 4, 128), dtype=np.uint16)
    slots = np.full(n, -1, np.int64)
    distinct = rng.permutation(total)[:n]
    slots[:len(distinct)] = distinct
    slots[rng.random(n) < 0.1] = -1
    slots[rng.random(n) < 0.05] = total + int(rng.integers(0, 100))
    want_k, want_v = ref.kv_append(k_pool, v_pool, k_rows, v_rows, slots)
    k, v = to_dev(k_pool), to_dev(v_pool)
    pkv.pkv_append_kv(k, v, to_dev(k_rows), to_dev(v_rows), to_dev(slots))
    torch.cuda.synchronize()
    got_k = k.view(torch.int16).cpu().numpy().view(np.uint16)
    got_v = v.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v), f"append seed={seed}"
