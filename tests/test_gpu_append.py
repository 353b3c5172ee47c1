"""KV append on the GPU against the oracle, through the C ABI.

The append moves bytes only, so the comparison is bit-exact over the whole
pools. Slots outside the pool (-1 padding, one past the end, large negative)
must store nothing.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_gqa_amd as pkv
from gpu_util import assert_lse_close, assert_out_close, bf16_to_np, to_dev
from inputs import make_block_table
from oracle import ref

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def random_bits(rng, shape):
    return rng.integers(0, 1 << 16, size=shape, dtype=np.uint16)


def run_append(k_pool, v_pool, k_rows, v_rows, slots):
    k = to_dev(k_pool)
    v = to_dev(v_pool)
    pkv.pkv_append_kv(k, v, to_dev(k_rows), to_dev(v_rows), to_dev(np.asarray(slots, np.int64)))
    torch.cuda.synchronize()
    return bits(k), bits(v)


@pytest.mark.parametrize("pages,ps,hkv,d,n", [
    (50, 1, 4, 128, 37),
    (20, 16, 4, 128, 200),
    (7, 64, 4, 128, 300),
    (9, 16, 1, 8, 40),        # 16-byte rows
    (5, 4, 2, 576, 11),       # rows wider than one wave's 1 KB
])
def test_append_bit_exact(pages, ps, hkv, d, n):
    rng = np.random.default_rng(pages * 1000 + ps)
    k_pool = random_bits(rng, (pages, ps, hkv, d))
    v_pool = random_bits(rng, (pages, ps, hkv, d))
    k_rows = random_bits(rng, (n, hkv, d))
    v_rows = random_bits(rng, (n, hkv, d))
    total = pages * ps
    slots = rng.permutation(total)[:n].astype(np.int64) if n <= total else None
    if slots is None:
        slots = np.concatenate([rng.permutation(total), np.full(n - total, -1)]).astype(np.int64)
    # padding and out-of-range entries
    slots[::7] = -1
    slots[3::11] = total
    slots[5::13] = -(1 << 40)
    want_k, want_v = ref.kv_append(k_pool, v_pool, k_rows, v_rows, slots)
    got_k, got_v = run_append(k_pool, v_pool, k_rows, v_rows, slots)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)


def test_append_nothing():
    rng = np.random.default_rng(3)
    k_pool = random_bits(rng, (4, 16, 4, 128))
    v_pool = random_bits(rng, (4, 16, 4, 128))
    got = run_append(k_pool, v_pool, k_pool[:0, 0], v_pool[:0, 0], np.zeros(0, np.int64))
    assert np.array_equal(got[0], k_pool) and np.array_equal(got[1], v_pool)
    slots = np.full(9, -1, np.int64)
    rows = random_bits(rng, (9, 4, 128))
    got = run_append(k_pool, v_pool, rows, rows, slots)
    assert np.array_equal(got[0], k_pool) and np.array_equal(got[1], v_pool)


def test_append_duplicate_slots_hold_pieces_of_the_rows():
    """Rows that name the same slot race, and nothing orders their stores, so
    only each 16-byte unit of the slot is promised: it holds the same unit of
    one of the rows that name the slot (the units of a slot, and K and V, may
    come from different rows). Every other slot is as the oracle has it."""
    rng = np.random.default_rng(4)
    k_pool = random_bits(rng, (8, 16, 4, 128))
    v_pool = random_bits(rng, (8, 16, 4, 128))
    rows_k = random_bits(rng, (6, 4, 128))
    rows_v = random_bits(rng, (6, 4, 128))
    slots = np.array([17, 40, 17, 99, 40, 3], np.int64)
    got_k, got_v = run_append(k_pool, v_pool, rows_k, rows_v, slots)
    flat_k = got_k.reshape(-1, 4, 128)
    flat_v = got_v.reshape(-1, 4, 128)
    for slot in (17, 40):
        cand = np.nonzero(slots == slot)[0]
        for got, rows in ((flat_k[slot], rows_k), (flat_v[slot], rows_v)):
            units = got.reshape(-1, 8)                     # 16-byte units of the 1 KB row
            options = [rows[i].reshape(-1, 8) for i in cand]
            ok = np.zeros(units.shape[0], bool)
            for o in options:
                ok |= np.all(units == o, axis=1)
            assert ok.all(), f"slot {slot}: a 16-byte unit matches none of its rows"
    unique = [i for i in range(6) if (slots == slots[i]).sum() == 1]
    want_k, want_v = ref.kv_append(k_pool, v_pool, rows_k[unique], rows_v[unique], slots[unique])
    other = np.ones(8 * 16, bool)
    other[[17, 40]] = False
    assert np.array_equal(flat_k[other], want_k.reshape(-1, 4, 128)[other])
    assert np.array_equal(flat_v[other], want_v.reshape(-1, 4, 128)[other])


def test_append_then_decode():
    """One decode step: append each sequence's next token on the GPU, then
    decode the longer sequences through the block table."""
    w = make_block_table(70, [5, 16, 31, 32, 100, 0], 16, extra_cols=1, pool_pages=30)
    rng = np.random.default_rng(71)
    new_k = random_bits(rng, (w.batch, 4, 128)) & np.uint16(0xBFFF)   # finite values
    new_v = random_bits(rng, (w.batch, 4, 128)) & np.uint16(0xBFFF)
    table = w.block_table.copy()
    used = set(table[b, j] for b in range(w.batch) for j in range(w.pages_per_seq[b]))
    spare = [p for p in range(w.num_pages) if p not in used]
    slots = []
    for b, n in enumerate(w.lengths):
        if n % 16 == 0:
            table[b, n // 16] = spare.pop()
        slots.append(int(table[b, n // 16]) * 16 + int(n % 16))
    slots = np.array(slots, np.int64)
    k2, v2 = ref.kv_append(w.k_pool, w.v_pool, new_k, new_v, slots)
    want = ref.gqa_block_table_decode(w.q, k2, v2, table, w.seq_lens + 1, w.sm_scale)

    k = to_dev(w.k_pool)
    v = to_dev(w.v_pool)
    pkv.pkv_append_kv(k, v, to_dev(new_k), to_dev(new_v), to_dev(slots))
    out, lse = pkv.decode_block_table(to_dev(w.q), k, v, to_dev(table), w.seq_lens + 1, w.sm_scale)
    torch.cuda.synchronize()
    assert np.array_equal(bits(k), k2) and np.array_equal(bits(v), v2)
    assert_out_close(bf16_to_np(out), want[0], "append+decode out")
    assert_lse_close(lse.cpu().numpy().astype(np.float64), want[1], "append+decode lse")
