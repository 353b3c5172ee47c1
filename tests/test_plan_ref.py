"""Invariants of the split-KV partition rule (the Python statement of it)."""

import numpy as np
import pytest

from oracle import plan_ref


def _check(indptr, num_cus, allow_split, chunk_tokens):
    c_len, items, merges, slots = plan_ref.make_plan(indptr, num_cus, allow_split, chunk_tokens)
    batch = len(indptr) - 1
    covered = {b: [] for b in range(batch)}
    for b, lo, hi, slot in items:
        covered[b].append((lo, hi, slot))
        assert hi - lo <= c_len
    seen_slots = []
    merged = {m[0]: m for m in merges}
    for b in range(batch):
        n = int(indptr[b + 1] - indptr[b])
        parts = sorted(covered[b])
        if n == 0:
            assert parts == [(0, 0, -1)]
            continue
        assert parts[0][0] == 0 and parts[-1][1] == n
        for (lo0, hi0, _), (lo1, _, _) in zip(parts, parts[1:]):
            assert hi0 == lo1
        assert all(hi > lo for lo, hi, _ in parts)
        if len(parts) == 1:
            assert parts[0][2] == -1 and b not in merged
        else:
            _, first, k, _ = merged[b]
            assert k == len(parts)
            assert [p[2] for p in parts] == list(range(first, first + k))
            assert all(lo % plan_ref.TILE == 0 for lo, _, _ in parts)
            seen_slots.extend(range(first, first + k))
    assert sorted(seen_slots) == list(range(slots))
    sizes = [hi - lo for _, lo, hi, _ in items]
    assert sizes == sorted(sizes, reverse=True)


@pytest.mark.parametrize("seed", range(20))
def test_plan_invariants_random(seed):
    rng = np.random.default_rng(seed)
    batch = int(rng.integers(1, 300))
    lengths = rng.integers(0, 20000, size=batch) * (rng.random(batch) < 0.9)
    indptr = np.concatenate([[0], np.cumsum(lengths)])
    num_cus = int(rng.choice([1, 8, 80, 256, 304]))
    chunk = int(rng.choice([0, 0, 1, 31, 32, 100, 4096]))
    _check(indptr, num_cus, bool(rng.random() < 0.85), chunk)


def test_plan_no_split_is_one_item_per_sequence():
    indptr = [0, 5, 5, 70000]
    c_len, items, merges, slots = plan_ref.make_plan(indptr, 256, allow_split=False)
    assert sorted(items) == [(0, 0, 5, -1), (1, 0, 0, -1), (2, 0, 69995, -1)]
    assert merges == [] and slots == 0


def test_plan_hand_example():
    # 600 tokens with chunk 256: k = 3, c = roundup(200, 32) = 224 -> 224, 224, 152
    c_len, items, merges, slots = plan_ref.make_plan([0, 600, 610], 1, chunk_tokens=256)
    assert c_len == 256
    assert items == [(0, 0, 224, 0), (0, 224, 448, 1), (0, 448, 600, 2), (1, 0, 10, -1)]
    assert merges == [(0, 0, 3, 0)] and slots == 3
