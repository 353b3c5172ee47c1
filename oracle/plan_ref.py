"""Independent Python statement of the split-KV work partition.

TEST INFRASTRUCTURE ONLY: the tests compare the library's exported plan with
this, integer for integer. It shares no code with the library.

The pages fix only the ideas: a plan object captured once and reused
([MLA page] ``FlashMLASchedMeta`` / ``get_mla_metadata``), splitting one row's
keys into contiguous pieces with no empty piece and merging the partials by
LSE ([QSA page] ``qsa_sparse_paged_attention`` and its split-K kernel). The
exact rule is this library's own and is stated here once:

* The batch's ``N = kv_indptr[B]`` tokens go, sequence by sequence in order,
  to at most ``W`` workers, ``W = ceil(N / chunk_tokens)`` when
  ``chunk_tokens > 0``, else ``min(num_cus * WORKERS_PER_CU,
  max(ceil(N / MIN_WORKER_TOKENS), non-empty sequences))``; no workers when
  ``N = 0``. A piece of ``n``
  tokens of one sequence costs ``ceil(n / TILE) * TILE + SEGMENT_COST`` (its
  tiles, plus one tile's worth for starting a segment). Workers are filled
  greedily with a cost budget ``C``: the rest of the current sequence goes to
  the current worker whole if its cost fits in what the worker has left;
  otherwise the worker takes the largest whole number of tiles whose cost
  fits (possibly none) and the next worker continues. ``C`` is the smallest
  budget from ``TILE + SEGMENT_COST`` up that needs at most ``W`` workers,
  found by bisection (``lo, hi = TILE + SEGMENT_COST, max(lo, sum of the
  whole sequences' costs)``; while ``lo < hi``: ``mid = (lo + hi) // 2``,
  ``hi = mid`` if ``mid`` needs at most ``W`` workers, else ``lo = mid + 1``).
  The plan has as many workers as that fill uses, possibly fewer than ``W``.
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

WORKERS_PER_CU = 1
MIN_WORKER_TOKENS = 128
TILE = 32
SEGMENT_COST = 32


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def piece_cost(n: int) -> int:
    return _cdiv(n, TILE) * TILE + SEGMENT_COST


def fill(lengths, budget: int, record: bool = True):
    """Greedy fill of the sequences' tokens into workers of cost ``budget``.

    Returns ``(workers used, pieces (w, b, lo, hi) in order)``, or
    ``(None, [])`` when the budget is below one tile plus a segment. The
    pieces are only listed when ``record`` is set."""
    if (budget - SEGMENT_COST) // TILE <= 0:
        return None, []
    pieces = []
    w, room, used = 0, budget, 0
    for b, n in enumerate(lengths):
        pos = 0
        while pos < n:
            rest = n - pos
            if piece_cost(rest) <= room:
                # the rest of the sequence fits the current worker whole
                if record:
                    pieces.append((w, b, pos, n))
                room -= piece_cost(rest)
                used = w + 1
                pos = n
            else:
                # the worker takes the whole tiles that fit, then is closed
                take = max(0, (room - SEGMENT_COST) // TILE * TILE)
                if take:
                    if record:
                        pieces.append((w, b, pos, pos + take))
                    used = w + 1
                    pos += take
                w, room = w + 1, budget
    return used, pieces


def make_plan(kv_indptr, num_cus: int, allow_split: bool = True, chunk_tokens: int = 0):
    """Return ``(worker_segments, merges, n_slots)``; worker_segments is a list of lists."""
    indptr = [int(x) for x in kv_indptr]
    batch = len(indptr) - 1
    total = indptr[-1]
    lengths = [indptr[b + 1] - indptr[b] for b in range(batch)]
    merges = []
    if not allow_split:
        seqs = [b for b in range(batch) if lengths[b] > 0]
        merges = [(b, 0, 0, 0) for b in range(batch) if lengths[b] == 0]
        seqs.sort(key=lambda b: (-lengths[b], b))
        return [[(b, 0, lengths[b], -1)] for b in seqs], merges, 0

    if total == 0:
        limit = 0
    elif chunk_tokens > 0:
        limit = _cdiv(total, chunk_tokens)
    else:
        nonempty = sum(1 for n in lengths if n > 0)
        limit = min(num_cus * WORKERS_PER_CU, max(_cdiv(total, MIN_WORKER_TOKENS), nonempty))
    pieces = []
    if limit:
        lo = TILE + SEGMENT_COST
        hi = max(lo, sum(piece_cost(n) for n in lengths if n))
        while lo < hi:
            mid = (lo + hi) // 2
            used, _ = fill(lengths, mid, record=False)
            if used is not None and used <= limit:
                hi = mid
            else:
                lo = mid + 1
        _, pieces = fill(lengths, lo)
    per_worker = [[] for _ in range(pieces[-1][0] + 1 if pieces else 0)]
    by_seq = {}
    for w, b, lo_, hi_ in pieces:
        by_seq.setdefault(b, []).append((w, lo_, hi_))
    slot = 0
    for b in range(batch):
        if lengths[b] == 0:
            merges.append((b, 0, 0, 0))
            continue
        parts = by_seq[b]
        if len(parts) == 1:
            w, a, e = parts[0]
            per_worker[w].append((b, a, e, -1))
        else:
            for j, (w, a, e) in enumerate(parts):
                per_worker[w].append((b, a, e, slot + j))
            merges.append((b, slot, len(parts), 0))
            slot += len(parts)
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
