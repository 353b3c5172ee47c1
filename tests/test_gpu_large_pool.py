"""Pools past 2^31 elements: listed pages on both sides of element offset 2^31.

One page-size-1 K (or V) row is Hkv * D = 512 elements, so page 4,194,304 is
the first whose elements start at or beyond 2^31; with 16-token pages it is
page 262,144. The decode kernel forms pool offsets in 64-bit arithmetic, as the
vLLM fork qsa.py page's split-K kernel (_qsa_sparse_paged_gqa_splitk_kernel)
widens its page offsets because they can overflow int32.

Relabelling the physical pages of a workload is exact in the oracle, and on the
GPU it changes no accumulation order, so the expected values come from the
oracle run on the compact pool of the listed rows, and the big-pool GPU result
must equal the compact-pool GPU result bit for bit. The big pools are
allocated uninitialised: rows no page list names are never read.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_gqa_amd as pkv
from gpu_util import assert_lse_close, assert_out_close, bf16_to_np, to_dev
from inputs import make_block_table, make_gqa
from oracle import ref

pytestmark = pytest.mark.gpu

HKV, D = 4, 128
BOUNDARY_ROW = 2**31 // (HKV * D)          # 4,194,304
ROWS = BOUNDARY_ROW + 64 * 16              # also 262,208 pages of 16 rows
LENGTHS = [100, 257, 37, 1, 640]


@pytest.fixture(scope="module")
def big_pools():
    k = torch.empty((ROWS, HKV, D), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    yield k, v
    del k, v
    torch.cuda.empty_cache()


def _physical(n, boundary, last, seed):
    """n distinct physical pages: about half below `boundary`, the rest at or
    above it, always including boundary - 1, boundary and `last`."""
    rng = np.random.default_rng(seed)
    lo = rng.choice(np.arange(boundary - 40000, boundary - 1), size=n // 2 - 1, replace=False)
    hi = rng.choice(np.arange(boundary + 1, last), size=n - n // 2 - 2, replace=False)
    phys = np.concatenate([lo, [boundary - 1], hi, [boundary, last]]).astype(np.int64)
    rng.shuffle(phys)
    return phys


def _place(pool_view, phys, rows_bits):
    """pool_view[phys[c]] = compact page c (bf16 bits [n, ...])."""
    pool_view[torch.from_numpy(phys).cuda()] = to_dev(rows_bits).view(pool_view.dtype).reshape(
        (len(phys),) + tuple(pool_view.shape[1:]))


@pytest.mark.parametrize("engine", ["mfma", "dot2"])
@pytest.mark.parametrize("chunk", [0, 64])
def test_csr_pages_across_2_31_elements(big_pools, chunk, engine):
    k, v = big_pools
    w = make_gqa(710 + chunk, LENGTHS)
    n = w.k_pool.shape[0]
    phys = _physical(n, BOUNDARY_ROW, ROWS - 1, 711 + chunk)
    _place(k, phys, w.k_pool.reshape(n, HKV, D))
    _place(v, phys, w.v_pool.reshape(n, HKV, D))
    assert phys.max() * HKV * D >= 2**31 and phys.min() * HKV * D < 2**31
    indices = phys[w.kv_indices].astype(np.int32)
    q = to_dev(w.q)
    indptr = to_dev(w.kv_indptr)
    out, lse = pkv.decode(q, k.view(ROWS, 1, HKV, D), v.view(ROWS, 1, HKV, D), indptr,
                          to_dev(indices), w.sm_scale, kv_indptr_host=w.kv_indptr,
                          chunk_tokens=chunk, engine=engine)
    ref_out, ref_lse = pkv.decode(q, to_dev(w.k_pool), to_dev(w.v_pool), indptr,
                                  to_dev(w.kv_indices), w.sm_scale, kv_indptr_host=w.kv_indptr,
                                  chunk_tokens=chunk, engine=engine)
    torch.cuda.synchronize()
    want = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices, w.sm_scale)
    assert_out_close(bf16_to_np(out), want[0], "big pool out")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), want[1], "big pool lse")
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse, ref_lse)


@pytest.mark.parametrize("engine", ["mfma", "dot2"])
@pytest.mark.parametrize("chunk", [0, 64])
def test_block_table_pages_across_2_31_elements(big_pools, chunk, engine):
    ps = 16
    k, v = big_pools
    pages = ROWS // ps
    boundary = BOUNDARY_ROW // ps                  # 262,144
    w = make_block_table(720 + chunk, LENGTHS, ps)
    n = w.k_pool.shape[0]
    phys = _physical(n, boundary, pages - 1, 721 + chunk)
    kp = k.view(pages, ps, HKV, D)
    vp = v.view(pages, ps, HKV, D)
    _place(kp, phys, w.k_pool)
    _place(vp, phys, w.v_pool)
    need = -(-w.seq_lens.astype(np.int64) // ps)
    table = w.block_table.copy()
    for b in range(table.shape[0]):
        table[b, :need[b]] = phys[w.block_table[b, :need[b]]]
    assert table.max() >= boundary
    q = to_dev(w.q)
    out, lse = pkv.decode_block_table(q, kp, vp, to_dev(table), w.seq_lens, w.sm_scale,
                                      chunk_tokens=chunk, engine=engine)
    ref_out, ref_lse = pkv.decode_block_table(q, to_dev(w.k_pool), to_dev(w.v_pool),
                                              to_dev(w.block_table), w.seq_lens, w.sm_scale,
                                              chunk_tokens=chunk, engine=engine)
    torch.cuda.synchronize()
    want = ref.gqa_block_table_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens,
                                      w.sm_scale)
    assert_out_close(bf16_to_np(out), want[0], "big pool (block table) out")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), want[1], "big pool (block table) lse")
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(lse, ref_lse)
