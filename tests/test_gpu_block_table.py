"""Paged GQA decode through a block table (pages of several tokens) on the GPU,
against the fp64 oracle, through the C ABI.

Same tolerances as the page-size-1 path: |out - ref| <= 1e-2 + 1e-2 |ref| per
element, |lse - ref| <= 1e-3, and -inf exactly where the oracle has -inf.
Every block-table entry a kernel could reach is a valid page; "never read"
is checked with NaN-filled pages, never with out-of-range ids.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_gqa_amd as pkv
from gpu_util import assert_lse_close, assert_out_close, bf16_to_np, to_dev
from inputs import make_block_table, make_config
from oracle import ref

pytestmark = pytest.mark.gpu

NAN_BF16 = 0x7FC0
_W = {}
_REF = {}


def workload(name):
    if name not in _W:
        _W[name] = make_config(name)
    return _W[name]


def oracle_of(w):
    return ref.gqa_block_table_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens,
                                      w.sm_scale)


def oracle(name):
    if name not in _REF:
        _REF[name] = oracle_of(workload(name))
    return _REF[name]


def upload(w):
    return dict(q=to_dev(w.q), k=to_dev(w.k_pool), v=to_dev(w.v_pool), table=to_dev(w.block_table))


def run_gpu(w, dev=None, **kw):
    dev = dev or upload(w)
    out, lse = pkv.decode_block_table(dev["q"], dev["k"], dev["v"], dev["table"], w.seq_lens,
                                      w.sm_scale, **kw)
    torch.cuda.synchronize()
    return bf16_to_np(out), lse.cpu().numpy().astype(np.float64)


def check(want, got, what):
    assert_out_close(got[0], want[0], what + " out")
    assert_lse_close(got[1], want[1], what + " lse")


@pytest.mark.parametrize("name", ["gqa_ps16", "gqa_ps64", "edge_ps16"])
@pytest.mark.parametrize("split", [True, False], ids=["split", "nosplit"])
def test_config_vs_oracle(name, split):
    check(oracle(name), run_gpu(workload(name), allow_split=split), f"{name} split={split}")


RAGGED = [0, 1, 15, 16, 17, 31, 32, 33, 100, 257, 1023, 1025, 2]


@pytest.mark.parametrize("ps", [1, 2, 4, 8, 16, 32, 64, 128, 256, 1024])
@pytest.mark.parametrize("chunk", [0, 32, 48])
def test_page_sizes_ragged(ps, chunk):
    w = make_block_table(400 + ps, RAGGED, ps, extra_cols=2)
    check(oracle_of(w), run_gpu(w, chunk_tokens=chunk), f"ps={ps} chunk={chunk}")


def test_same_rows_as_csr_bit_identical():
    """Token rows listed one by one through the CSR call give the same bits:
    the plan, the tiles and the accumulation order are the same."""
    w = workload("edge_ps16")
    a = run_gpu(w)
    ps = w.page_size
    k1 = w.k_pool.reshape(-1, 1, w.num_kv_heads, w.head_dim)
    v1 = w.v_pool.reshape(-1, 1, w.num_kv_heads, w.head_dim)
    rows = np.concatenate([w.block_table[b, np.arange(n) // ps].astype(np.int64) * ps
                           + np.arange(n) % ps for b, n in enumerate(w.lengths)]).astype(np.int32)
    indptr = np.concatenate([[0], np.cumsum(w.lengths)]).astype(np.int32)
    out, lse = pkv.decode(to_dev(w.q), to_dev(k1), to_dev(v1), to_dev(indptr), to_dev(rows),
                          w.sm_scale, kv_indptr_host=indptr)
    torch.cuda.synchronize()
    b = bf16_to_np(out), lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_unread_slots_entries_and_pages():
    """NaN in the slots past each length, in unlisted pages and in the pages the
    padding entries point to must not reach the output."""
    lengths = [5, 16, 17, 40, 0, 1, 33]
    ps = 16
    # one spare page, listed by no sequence, is what every padding entry names
    w = make_block_table(500, lengths, ps, extra_cols=3, pool_pages=20)
    used = set()
    for b, n in enumerate(w.lengths):
        used.update(w.block_table[b, :w.pages_per_seq[b]].tolist())
    spare = min(set(range(w.num_pages)) - used)
    table = w.block_table.copy()
    for b in range(w.batch):
        table[b, w.pages_per_seq[b]:] = spare
    want = ref.gqa_block_table_decode(w.q, w.k_pool, w.v_pool, table, w.seq_lens, w.sm_scale)
    k = w.k_pool.copy()
    v = w.v_pool.copy()
    for b, n in enumerate(w.lengths):
        if n % ps:
            last = table[b, w.pages_per_seq[b] - 1]
            k[last, n % ps:] = NAN_BF16
            v[last, n % ps:] = NAN_BF16
    unused = [p for p in range(w.num_pages) if p not in used]
    k[unused] = NAN_BF16
    v[unused] = NAN_BF16
    w.k_pool, w.v_pool, w.block_table = k, v, table
    for chunk in (0, 32):
        check(want, run_gpu(w, chunk_tokens=chunk), f"NaN unread chunk={chunk}")


def test_rerun_and_relabel_bit_identical():
    w = workload("gqa_ps16")
    dev = upload(w)
    a = run_gpu(w, dev)
    b = run_gpu(w, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    rng = np.random.default_rng(23)
    perm = rng.permutation(w.num_pages)
    k = np.empty_like(w.k_pool)
    v = np.empty_like(w.v_pool)
    k[perm] = w.k_pool
    v[perm] = w.v_pool
    w2 = make_block_table(3, [1], 16)   # container; fields replaced below
    w2.q, w2.k_pool, w2.v_pool, w2.seq_lens, w2.sm_scale = w.q, k, v, w.seq_lens, w.sm_scale
    w2.block_table = perm[w.block_table].astype(np.int32)
    c = run_gpu(w2)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_prepared_call_matches():
    w = workload("edge_ps16")
    dev = upload(w)
    ws = torch.empty(pkv.pkv_block_table_workspace_size(w.seq_lens, page_size=w.page_size),
                     dtype=torch.uint8, device="cuda")
    plan = pkv.pkv_block_table_plan_create(w.seq_lens, page_size=w.page_size, workspace=ws)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    run = pkv.prepare_block_table_run(plan, dev["q"], dev["k"], dev["v"], dev["table"],
                                      w.sm_scale, ws, out, lse)
    merge = pkv.prepare_merge(plan, ws, out, lse)
    for _ in range(2):
        run()
        merge()
    torch.cuda.synchronize()
    check(oracle("edge_ps16"), (bf16_to_np(out), lse.cpu().numpy().astype(np.float64)),
          "prepared")


def test_plan_kind_and_shape_mismatch_raise():
    w = make_block_table(600, [20, 3], 16)
    dev = upload(w)
    ws = torch.empty(pkv.pkv_block_table_workspace_size(w.seq_lens, page_size=16),
                     dtype=torch.uint8, device="cuda")
    plan = pkv.pkv_block_table_plan_create(w.seq_lens, page_size=16, workspace=ws)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):     # table one column short
        pkv.pkv_block_table_run(plan, dev["q"], dev["k"], dev["v"], dev["table"][:, :1].contiguous(),
                                w.sm_scale, ws, out, lse)
    with pytest.raises(ValueError):     # pool with another page size
        k8 = dev["k"].reshape(-1, 8, 4, 128)
        pkv.pkv_block_table_run(plan, dev["q"], k8, k8, dev["table"], w.sm_scale, ws, out, lse)
    with pytest.raises(ValueError):     # CSR call on a block-table plan
        pkv.pkv_run(plan, dev["q"], dev["k"], dev["v"], to_dev(np.array([0, 20, 23], np.int32)),
                    to_dev(np.arange(23, dtype=np.int32)), w.sm_scale, ws, out, lse)
