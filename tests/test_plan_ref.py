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
        tile, seg = plan_ref.TILE, plan_ref.SEGMENT_COST
        for segs in per_worker:
            for b, lo, hi, slot in segs:
                assert lo % tile == 0                    # cuts fall on whole tiles
        costs = [sum(plan_ref.piece_cost(hi - lo) for _, lo, hi, _ in segs) for segs in per_worker]
        budget = max(costs)
        # every worker but the last was closed with less room left than one
        # tile plus a segment
        assert all(c > budget - tile - seg for c in costs[:-1])
        limit = (-(-total // chunk_tokens) if chunk_tokens > 0
                 else min(num_cus * plan_ref.WORKERS_PER_CU,
                          max(-(-total // plan_ref.MIN_WORKER_TOKENS),
                              sum(1 for b in range(batch) if indptr[b + 1] > indptr[b]))))
        assert len(per_worker) <= limit
        # the budget is the smallest that fits: one less needs more workers
        if budget > tile + seg:
            used, _ = plan_ref.fill([int(indptr[b + 1] - indptr[b]) for b in range(batch)],
                                    budget - 1, record=False)
            assert used is None or used > limit
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
    # 610 tokens, at most ceil(610/256) = 3 workers. Costs: sequence 0 (600
    # tokens) 608 + 32, sequence 2 (10 tokens) 32 + 32. Budget 256: workers 0
    # and 1 take (256 - 32) // 32 * 32 = 224 tokens each, worker 2 the last 152
    # (160 + 32) and sequence 2 (64): 256. Budget 255 takes 192 a worker and
    # would need a fourth worker for the rest.
    per_worker, merges, slots = plan_ref.make_plan([0, 600, 600, 610], 1, chunk_tokens=256)
    assert per_worker == [[(0, 0, 224, 0)], [(0, 224, 448, 1)], [(0, 448, 600, 2), (2, 0, 10, -1)]]
    assert merges == [(0, 0, 3, 0), (1, 0, 0, 0)] and slots == 3
    assert plan_ref.export([0, 600, 600, 610], 1, chunk_tokens=256) == (
        [3, 4, 2, 3, 0, 1, 2, 4, 0, 0, 224, 0, 0, 224, 448, 1, 0, 448, 600, 2, 2, 0, 10, -1,
         0, 0, 3, 0, 1, 0, 0, 0])


def test_plan_small_hand_examples():
    # 160 tokens, 2 workers: budget 128 gives 96 + (64 + 32); 127 gives 64 a worker
    pw, _, _ = plan_ref.make_plan([0, 160], 1, chunk_tokens=80)
    assert [s[:3] for ws in pw for s in ws] == [(0, 0, 96), (0, 96, 160)]
    # two sequences of 120 and 110 tokens, 2 workers: each whole (costs 160 and 144)
    pw, _, _ = plan_ref.make_plan([0, 120, 230], 1, chunk_tokens=115)
    assert pw == [[(0, 0, 120, -1)], [(1, 0, 110, -1)]]
    # 96 tokens, 2 workers: budget 96 gives 64 + (32 + 32)
    pw, _, _ = plan_ref.make_plan([0, 96], 1, chunk_tokens=48)
    assert [s[:3] for ws in pw for s in ws] == [(0, 0, 64), (0, 64, 96)]
    # a short sequence shares a worker with the start of a long one: budget
    # 128 holds sequence 0 (32 + 32) and one tile of sequence 1 (32 + 32)
    pw, _, _ = plan_ref.make_plan([0, 20, 100], 1, chunk_tokens=50)
    assert pw == [[(0, 0, 20, -1), (1, 0, 32, 0)], [(1, 32, 80, 1)]]
