"""Independent Python statement of the split-KV work partition.

TEST INFRASTRUCTURE ONLY: the tests compare the library's exported plan with
this, integer for integer. It shares no code with the library.

The pages fix only the ideas: a plan object captured once and reused
([MLA page] ``FlashMLASchedMeta`` / ``get_mla_metadata``), splitting one row's
keys into contiguous tiles with no empty split and merging the partials by LSE
([QSA page] ``qsa_sparse_paged_attention`` and its split-K kernel). The exact
rule is this library's own and is stated here once:

* ``N = kv_indptr[B]``. The chunk length ``C`` is ``chunk_tokens`` rounded up to
  a multiple of ``TILE`` when given; otherwise
  ``max(MIN_CHUNK, roundup(ceil(N / (num_cus * ITEMS_PER_CU)), TILE))``.
  Without splitting, ``C`` is unbounded.
* A sequence with ``n = 0`` tokens gets one item ``(b, 0, 0, -1)`` that writes
  zeros and -inf. A sequence with ``0 < n <= C`` gets one item
  ``(b, 0, n, -1)`` that writes the final output directly.
* A longer sequence gets ``k = ceil(n / C)`` chunks of equal tile-rounded
  length ``c = roundup(ceil(n / k), TILE)`` (then ``k = ceil(n / c)``, so no
  chunk is empty): items ``(b, j*c, min((j+1)*c, n), slot0 + j)``, and one
  merge record ``(b, slot0, k, 0)``. Partial slots are numbered in sequence
  order.
* Items are ordered by token count, longest first; equal counts keep the order
  in which they were made (sequence order, then chunk order).

The export layout is ``[C, n_items, n_merges, n_slots]`` then the items
(4 int32 each) then the merge records (4 int32 each).
"""

from __future__ import annotations

TILE = 32
MIN_CHUNK = 256
ITEMS_PER_CU = 2
NO_SPLIT_CHUNK = 2**31 - 1


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def _roundup(a: int, m: int) -> int:
    return _cdiv(a, m) * m


def chunk_length(total_tokens: int, num_cus: int, allow_split: bool, chunk_tokens: int) -> int:
    if not allow_split:
        return NO_SPLIT_CHUNK
    if chunk_tokens > 0:
        return _roundup(chunk_tokens, TILE)
    per_item = _cdiv(total_tokens, num_cus * ITEMS_PER_CU) if total_tokens > 0 else 0
    return max(MIN_CHUNK, _roundup(per_item, TILE))


def make_plan(kv_indptr, num_cus: int, allow_split: bool = True, chunk_tokens: int = 0):
    """Return ``(C, items, merges, n_slots)`` with items/merges as lists of 4-tuples."""
    indptr = [int(x) for x in kv_indptr]
    batch = len(indptr) - 1
    c_len = chunk_length(indptr[-1], num_cus, allow_split, chunk_tokens)
    items, merges = [], []
    slot = 0
    for b in range(batch):
        n = indptr[b + 1] - indptr[b]
        if n <= c_len:
            items.append((b, 0, n, -1))
            continue
        k = _cdiv(n, c_len)
        c = _roundup(_cdiv(n, k), TILE)
        k = _cdiv(n, c)
        for j in range(k):
            items.append((b, j * c, min((j + 1) * c, n), slot + j))
        merges.append((b, slot, k, 0))
        slot += k
    order = sorted(range(len(items)), key=lambda i: (-(items[i][2] - items[i][1]), i))
    items = [items[i] for i in order]
    return c_len, items, merges, slot


def export(kv_indptr, num_cus: int, allow_split: bool = True, chunk_tokens: int = 0):
    c_len, items, merges, slots = make_plan(kv_indptr, num_cus, allow_split, chunk_tokens)
    flat = [c_len, len(items), len(merges), slots]
    for it in items:
        flat.extend(it)
    for m in merges:
        flat.extend(m)
    return flat
