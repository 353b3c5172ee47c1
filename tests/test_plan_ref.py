"""Invariants of the split-KV partition rule (the Python statement of it)."""

import numpy as np
import pytest

from oracle import plan_ref


def _check(indptr, num_cus, allow_split, chunk_tokens):
    per_worker, merges, slots = plan_ref.make_plan(indptr, num_cus, allow_split, chunk_tokens)
    batch = len(indptr) - 1
    total = int(indptr[-1])
    covered = {b: [] for b in range(batch)}
    for w, segs in enumerate(per_worker):
        assert segs, "a worker without segments"
        for b, lo, hi, slot in segs:
            assert hi > lo
            covered[b].append((lo, hi, slot, w))
    merged = {m[0]: m for m in merges}
    seen_slots = []
    for b in range(batch):
        n = int(indptr[b + 1] - indptr[b])
        parts = sorted(covered[b])
        if n == 0:
            assert parts == [] and merged[b] == (b, 0, 0, 0)
            continue
        assert parts[0][0] == 0 and parts[-1][1] == n
        for p0, p1 in zip(parts, parts[1:]):
            assert p0[1] == p1[0] and p1[3] == p0[3] + 1     # contiguous, next worker
        if len(parts) == 1:
            assert parts[0][2] == -1 and b not in merged
        else:
            _, first, k, _ = merged[b]
            assert k == len(parts)
            assert [p[2] for p in parts] == list(range(first, first + k))
            seen_slots.extend(range(first, first + k))
    assert sorted(seen_slots) == list(range(slots))
    assert [m[0] for m in merges] == sorted(m[0] for m in merges)
    if allow_split and total:
        sizes = [sum(hi - lo for _, lo, hi, _ in segs) for segs in per_worker]
        snapped = len(per_worker) > 1 and total // len(per_worker) >= plan_ref.SNAP_MIN_SHARE
        assert max(sizes) - min(sizes) <= (1 + 4 * (plan_ref.TILE // 2) if snapped else 1)
        if snapped:   # interior pieces of a sequence are whole tiles
            for segs in per_worker:
                for b, lo, hi, slot in segs:
                    if slot >= 0 and hi < int(indptr[b + 1] - indptr[b]):
                        assert (hi - lo) % plan_ref.TILE == 0 or lo % plan_ref.TILE != 0
        if chunk_tokens == 0:
            assert len(per_worker) <= num_cus * plan_ref.WORKERS_PER_CU
    if not allow_split:
        assert slots == 0 and all(len(s) == 1 for s in per_worker)


@pytest.mark.parametrize("seed", range(20))
def test_plan_invariants_random(seed):
    rng = np.random.default_rng(seed)
    batch = int(rng.integers(1, 300))
    lengths = rng.integers(0, 20000, size=batch) * (rng.random(batch) < 0.9)
    indptr = np.concatenate([[0], np.cumsum(lengths)])
    num_cus = int(rng.choice([1, 8, 80, 256, 304]))
    chunk = int(rng.choice([0, 0, 31, 32, 100, 4096]))
    _check(indptr, num_cus, bool(rng.random() < 0.85), chunk)


def test_plan_no_split_is_one_worker_per_sequence():
    per_worker, merges, slots = plan_ref.make_plan([0, 5, 5, 70000], 256, allow_split=False)
    assert per_worker == [[(2, 0, 69995, -1)], [(0, 0, 5, -1)]]
    assert merges == [(1, 0, 0, 0)] and slots == 0


def test_plan_hand_example():
    # 610 tokens over ceil(610/256) = 3 workers: cuts at 203 and 406, moved to
    # the nearest multiple of 32 into sequence 0: 192 (203 = 6*32 + 11) and 416
    per_worker, merges, slots = plan_ref.make_plan([0, 600, 600, 610], 1, chunk_tokens=256)
    assert per_worker == [[(0, 0, 192, 0)], [(0, 192, 416, 1)], [(0, 416, 600, 2), (2, 0, 10, -1)]]
    assert merges == [(0, 0, 3, 0), (1, 0, 0, 0)] and slots == 3
    assert plan_ref.export([0, 600, 600, 610], 1, chunk_tokens=256) == (
        [3, 4, 2, 3, 0, 1, 2, 4, 0, 0, 192, 0, 0, 192, 416, 1, 0, 416, 600, 2, 2, 0, 10, -1,
         0, 0, 3, 0, 1, 0, 0, 0])


def test_plan_snap_ties_and_sequence_end():
    # a cut at 80 = 2.5 tiles into the sequence (a tie) goes down to 64
    pw, _, _ = plan_ref.make_plan([0, 160], 1, chunk_tokens=80)
    assert [s[:3] for ws in pw for s in ws] == [(0, 0, 64), (0, 64, 160)]
    # a cut at 115 (3.6 tiles into a 120-token sequence) stops at its end
    pw, _, _ = plan_ref.make_plan([0, 120, 230], 1, chunk_tokens=115)
    assert pw == [[(0, 0, 120, -1)], [(1, 0, 110, -1)]]
    # shares under SNAP_MIN_SHARE are not moved
    pw, _, _ = plan_ref.make_plan([0, 96], 1, chunk_tokens=48)
    assert [s[:3] for ws in pw for s in ws] == [(0, 0, 48), (0, 48, 96)]
