"""Independent Python statement of the split-KV work partition.

TEST INFRASTRUCTURE ONLY: the tests compare the library's exported plan with
this, integer for integer. It shares no code with the library.

The pages fix only the ideas: a plan object captured once and reused
([MLA page] ``FlashMLASchedMeta`` / ``get_mla_metadata``), splitting one row's
keys into contiguous pieces with no empty piece and merging the partials by
LSE ([QSA page] ``qsa_sparse_paged_attention`` and its split-K kernel). The
exact rule is this library's own and is stated here once:

* The batch's ``N = kv_indptr[B]`` tokens, in ``kv_indices`` order, go to
  ``W`` workers; worker ``w`` owns positions ``[s_w, s_(w+1))`` with
  ``s_w = w*N//W``. When ``N//W >= SNAP_MIN_SHARE``, every interior ``s_w`` is
  moved to the nearest (ties: lower) position ``indptr[b] + TILE*k`` inside
  the sequence ``b`` that holds it (``indptr[b] <= s_w < indptr[b+1]``),
  capped at ``indptr[b+1]``, so that a sequence's pieces are whole tiles.
  ``W = ceil(N / chunk_tokens)`` when ``chunk_tokens > 0``, else
  ``min(num_cus * WORKERS_PER_CU, ceil(N / MIN_WORKER_TOKENS))``; ``W = 0``
  when ``N = 0``.
* Each non-empty sequence becomes one segment per worker it overlaps:
  ``(b, lo, hi, slot)`` with ``lo, hi`` relative to the sequence. A sequence
  inside one worker has ``slot = -1`` (written directly); a sequence cut into
  ``k`` segments gets slots ``s0 .. s0+k-1`` in token order and a merge record
  ``(b, s0, k, 0)``; slots are numbered in sequence order.
* An empty sequence has no segment and a merge record ``(b, 0, 0, 0)``.
  Merge records are in sequence order.
* Without splitting, every non-empty sequence is its own worker with one
  segment ``(b, 0, n, -1)``, workers ordered longest first (ties by ``b``).

Export layout: ``[W, n_segments, n_merges, n_slots]``, then ``W + 1`` worker
offsets into the segment list, then the segments (4 int32 each), then the
merge records (4 int32 each).
"""

from __future__ import annotations

import bisect

WORKERS_PER_CU = 1
MIN_WORKER_TOKENS = 128
TILE = 32
SNAP_MIN_SHARE = 64


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def round_half_down(x: float) -> int:
    """Nearest integer, halves rounded down (x >= 0)."""
    import math
    f = math.floor(x)
    return f + 1 if x - f > 0.5 else f


def make_plan(kv_indptr, num_cus: int, allow_split: bool = True, chunk_tokens: int = 0):
    """Return ``(worker_segments, merges, n_slots)``; worker_segments is a list of lists."""
    indptr = [int(x) for x in kv_indptr]
    batch = len(indptr) - 1
    total = indptr[-1]
    merges = []
    if not allow_split:
        seqs = [b for b in range(batch) if indptr[b + 1] > indptr[b]]
        merges = [(b, 0, 0, 0) for b in range(batch) if indptr[b + 1] == indptr[b]]
        seqs.sort(key=lambda b: (-(indptr[b + 1] - indptr[b]), b))
        return [[(b, 0, indptr[b + 1] - indptr[b], -1)] for b in seqs], merges, 0

    if total == 0:
        workers = 0
    elif chunk_tokens > 0:
        workers = _cdiv(total, chunk_tokens)
    else:
        workers = min(num_cus * WORKERS_PER_CU, _cdiv(total, MIN_WORKER_TOKENS))
    bounds = [w * total // workers for w in range(workers)] + [total] if workers else [0]
    if workers > 1 and total // workers >= SNAP_MIN_SHARE:
        for w in range(1, workers):
            pos = bounds[w]
            b = bisect.bisect_right(indptr, pos) - 1          # indptr[b] <= pos < indptr[b+1]
            k = round_half_down((pos - indptr[b]) / TILE)
            bounds[w] = min(indptr[b] + TILE * k, indptr[b + 1])
    per_worker = [[] for _ in range(workers)]
    slot = 0
    for b in range(batch):
        lo, hi = indptr[b], indptr[b + 1]
        if lo == hi:
            merges.append((b, 0, 0, 0))
            continue
        pieces = []
        w = bisect.bisect_right(bounds, lo) - 1          # worker holding position lo
        while w < workers and bounds[w] < hi:
            a, e = max(lo, bounds[w]), min(hi, bounds[w + 1])
            if e > a:
                pieces.append((w, a - lo, e - lo))
            w += 1
        if len(pieces) == 1:
            w, a, e = pieces[0]
            per_worker[w].append((b, a, e, -1))
        else:
            for j, (w, a, e) in enumerate(pieces):
                per_worker[w].append((b, a, e, slot + j))
            merges.append((b, slot, len(pieces), 0))
            slot += len(pieces)
    return per_worker, merges, slot


def export(kv_indptr, num_cus: int, allow_split: bool = True, chunk_tokens: int = 0):
    per_worker, merges, slots = make_plan(kv_indptr, num_cus, allow_split, chunk_tokens)
    segments = [s for ws in per_worker for s in ws]
    flat = [len(per_worker), len(segments), len(merges), slots]
    off = 0
    flat.append(0)
    for ws in per_worker:
        off += len(ws)
        flat.append(off)
    for s in segments:
        flat.extend(s)
    for m in merges:
        flat.extend(m)
    return flat
