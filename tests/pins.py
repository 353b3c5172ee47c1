"""Pins of the CPU oracle: facts fixed by the pages or by mathematics.

Each ``pin_*`` function takes the oracle module (normally ``oracle.ref``) and
raises ``AssertionError`` when the oracle disagrees with a closed form, an
invariant, a library routine or a brute-force sum. They are run once against
the real oracle (``test_oracle.py``) and once against planted mistakes
(``test_oracle_mutants.py``) to show that each plausible slip is caught.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from inputs import bf16_bits_from_f32, make_block_table, make_config, make_gqa, make_mla
from inputs.configs import EDGE_CONST_V, EDGE_CONST_V_SEQ, EDGE_LENGTHS

_CACHE = {}


def _cfg(name):
    if name not in _CACHE:
        _CACHE[name] = make_config(name)
    return _CACHE[name]


def _small_edge():
    """The edge batch without its three longest sequences (fast on the CPU)."""
    if "small_edge" not in _CACHE:
        lengths = [n if n <= 4096 else 5 for n in EDGE_LENGTHS]
        _CACHE["small_edge"] = make_gqa(3, lengths, peaky_seq=10, const_v_seq=EDGE_CONST_V_SEQ)
    return _CACHE["small_edge"]


def _decode(ref, w, batches=None):
    return ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices,
                                w.sm_scale, batches=batches)


def _f64(bits):
    # Independent decode for the pins: build the float32 from the bit pattern.
    return np.frombuffer((np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).tobytes(),
                         dtype=np.float32).astype(np.float64).reshape(np.shape(bits))


# ---------------------------------------------------------------- encodings

def pin_bf16_decode(ref):
    bits = np.array([0x3F80, 0xBF40, 0x4049, 0x0000, 0x8000, 0x7F80, 0x3C00], dtype=np.uint16)
    want = [1.0, -0.75, 3.140625, 0.0, -0.0, math.inf, 2.0 ** -7]
    got = ref.bf16_to_f64(bits)
    assert got.dtype == np.float64
    assert list(got) == want


# --------------------------------------------------------- GQA special cases

def pin_empty_sequence(ref):
    w = _small_edge()
    assert w.lengths[0] == 0
    out, lse = _decode(ref, w, batches=[0])
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))


def pin_single_token(ref):
    """n = 1: the output is that V row exactly; the LSE is the one score over ln 2."""
    w = _small_edge()
    b = 1
    assert w.lengths[b] == 1
    out, lse = _decode(ref, w, batches=[b])
    page = int(w.kv_indices[w.kv_indptr[b]])
    q = _f64(w.q[b])
    for h in range(w.num_qo_heads):
        g = h // (w.num_qo_heads // w.num_kv_heads)
        v = _f64(w.v_pool[page, 0, g])
        k = _f64(w.k_pool[page, 0, g])
        assert np.array_equal(out[b, h], v)
        s = w.sm_scale * math.fsum(float(a) * float(c) for a, c in zip(q[h], k))
        assert abs(lse[b, h] - s / math.log(2.0)) <= 1e-12 * max(1.0, abs(s))


def pin_uniform_v(ref):
    """Every token carries V = 0.75, so every head outputs 0.75."""
    w = _small_edge()
    b = EDGE_CONST_V_SEQ
    out, _ = _decode(ref, w, batches=[b])
    assert np.max(np.abs(out[b] - EDGE_CONST_V)) <= 1e-15


def pin_equal_keys(ref):
    """All keys equal: weights 1/n, out = mean of the V rows, lse = s/ln2 + log2 n."""
    w = make_gqa(11, [37, 5], pool_pages=50)
    k = w.k_pool.copy()
    for b in range(2):
        pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        k[pages] = k[pages[0]]
    w.k_pool = k
    out, lse = _decode(ref, w)
    for b in range(2):
        pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        n = len(pages)
        for h in range(w.num_qo_heads):
            g = h // 8
            mean_v = _f64(w.v_pool[pages, 0, g]).mean(axis=0)
            assert np.max(np.abs(out[b, h] - mean_v)) <= 1e-13
            s = w.sm_scale * float(np.dot(_f64(w.q[b, h]), _f64(k[pages[0], 0, g])))
            assert abs(lse[b, h] - (s / math.log(2.0) + math.log2(n))) <= 1e-12


def pin_zero_scale(ref):
    """sm_scale = 0 makes every weight equal: out = mean(V), lse = log2 n."""
    w = make_gqa(12, [9, 1, 40], pool_pages=60, sm_scale=0.0)
    out, lse = _decode(ref, w)
    for b in range(3):
        pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        for g in range(4):
            mean_v = _f64(w.v_pool[pages, 0, g]).mean(axis=0)
            for h in range(8 * g, 8 * g + 8):
                assert np.max(np.abs(out[b, h] - mean_v)) <= 1e-13
        assert np.max(np.abs(lse[b] - math.log2(len(pages)))) <= 1e-12


def pin_brute_force_tiny(ref):
    """The tiny batch, summed term by term in Python with exact-rounded sums.

    No max is subtracted here; ``math.fsum`` rounds each sum once.
    """
    w = _cfg("tiny")
    out, lse = _decode(ref, w)
    q = _f64(w.q)
    for b in range(w.batch):
        pages = [int(p) for p in w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]]
        for h in range(w.num_qo_heads):
            g = h // 8
            s = []
            for p in pages:
                k = _f64(w.k_pool[p, 0, g])
                s.append(w.sm_scale * math.fsum(float(a) * float(c) for a, c in zip(q[b, h], k)))
            e = [math.exp(x) for x in s]
            z = math.fsum(e)
            assert abs(lse[b, h] - math.log2(z)) <= 1e-12 * max(1.0, abs(math.log2(z)))
            vrows = [_f64(w.v_pool[p, 0, g]) for p in pages]
            for d in range(0, w.head_dim, 7):
                o = math.fsum(ei * float(vr[d]) for ei, vr in zip(e, vrows)) / z
                assert abs(out[b, h, d] - o) <= 1e-12


def pin_sdpa_cross_check(ref):
    """Against torch's scaled_dot_product_attention (CPU, float64, grouped heads)."""
    for w in (_cfg("tiny"), _small_edge()):
        out, lse = _decode(ref, w)
        for b in range(w.batch):
            pages = torch.as_tensor(w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]].astype(np.int64))
            if pages.numel() == 0:
                continue
            q = torch.as_tensor(_f64(w.q[b]))[:, None, :]                   # [Hq, 1, D]
            k = torch.as_tensor(_f64(w.k_pool))[pages, 0].transpose(0, 1)  # [Hkv, n, D]
            v = torch.as_tensor(_f64(w.v_pool))[pages, 0].transpose(0, 1)
            o = torch.nn.functional.scaled_dot_product_attention(
                q[None], k[None].contiguous(), v[None].contiguous(), scale=w.sm_scale,
                enable_gqa=True)[0, :, 0, :]
            assert np.max(np.abs(out[b] - o.numpy())) <= 1e-12
            kk = k.repeat_interleave(w.num_qo_heads // w.num_kv_heads, dim=0)
            scores = w.sm_scale * torch.bmm(q, kk.transpose(1, 2).contiguous())[:, 0, :]
            l2 = (torch.logsumexp(scores, dim=-1) / math.log(2.0)).numpy()
            assert np.max(np.abs(lse[b] - l2)) <= 1e-12


def pin_head_map(ref):
    """KV head g holds the constant V c_g; query head h must output c_(h // 8)."""
    w = make_gqa(13, [20, 33], pool_pages=64)
    v = w.v_pool.copy()
    consts = [0.5, -1.25, 2.0, 3.5]
    for g, c in enumerate(consts):
        v[:, 0, g, :] = bf16_bits_from_f32(np.float32(c) * np.ones(w.head_dim, np.float32))
    w.v_pool = v
    out, _ = _decode(ref, w)
    for h in range(w.num_qo_heads):
        assert np.max(np.abs(out[:, h, :] - consts[h // 8])) <= 1e-14


def pin_head_map_keys(ref):
    """Only KV head g's keys may move query head h = 8g..8g+7: replace the keys
    of every other KV head and the outputs of those 8 heads stay bit-equal."""
    w = make_gqa(14, [25, 7], pool_pages=40)
    out0, lse0 = _decode(ref, w)
    for g in range(4):
        k = w.k_pool.copy()
        others = [x for x in range(4) if x != g]
        k[:, 0, others, :] = k[::-1, 0, others, :]
        w2 = make_gqa(14, [25, 7], pool_pages=40)
        w2.k_pool = k
        out1, lse1 = _decode(ref, w2)
        heads = list(range(8 * g, 8 * g + 8))
        assert np.array_equal(out0[:, heads], out1[:, heads])
        assert np.array_equal(lse0[:, heads], lse1[:, heads])
        rest = [h for h in range(32) if h not in heads]
        assert not np.allclose(lse0[:, rest], lse1[:, rest])


def pin_page_relabel(ref):
    """Permuting the physical pages (and remapping the indices) changes nothing."""
    w = _cfg("tiny")
    out0, lse0 = _decode(ref, w)
    rng = np.random.default_rng(99)
    perm = rng.permutation(w.num_pages)
    k = np.empty_like(w.k_pool)
    v = np.empty_like(w.v_pool)
    k[perm] = w.k_pool
    v[perm] = w.v_pool
    idx = perm[w.kv_indices].astype(np.int32)
    out1, lse1 = ref.gqa_paged_decode(w.q, k, v, w.kv_indptr, idx, w.sm_scale)
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def pin_unused_pages_never_read(ref):
    """NaN in the pages no sequence lists must not reach the result."""
    w = _cfg("tiny")
    used = np.zeros(w.num_pages, dtype=bool)
    used[w.kv_indices] = True
    k = w.k_pool.copy()
    v = w.v_pool.copy()
    k[~used] = 0x7FC0
    v[~used] = 0x7FC0
    out, lse = ref.gqa_paged_decode(w.q, k, v, w.kv_indptr, w.kv_indices, w.sm_scale)
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def pin_token_order(ref):
    """Decode has no positions: reordering a sequence's page list changes only rounding."""
    w = _small_edge()
    out0, lse0 = _decode(ref, w)
    rng = np.random.default_rng(7)
    idx = w.kv_indices.copy()
    for b in range(w.batch):
        seg = idx[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        idx[w.kv_indptr[b]:w.kv_indptr[b + 1]] = seg[rng.permutation(len(seg))]
    out1, lse1 = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, idx, w.sm_scale)
    assert np.max(np.abs(out0 - out1)) <= 1e-12
    fin = np.isfinite(lse0)
    assert np.array_equal(fin, np.isfinite(lse1))
    assert np.max(np.abs(lse0[fin] - lse1[fin])) <= 1e-12


def pin_lse_bounds_and_convexity(ref):
    """max_j s_j/ln2 <= lse <= max_j s_j/ln2 + log2 n; out lies in the V rows' hull."""
    w = _small_edge()
    out, lse = _decode(ref, w)
    q = _f64(w.q)
    for b in range(w.batch):
        pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        if len(pages) == 0:
            continue
        for g in range(4):
            k = _f64(w.k_pool[pages, 0, g])
            v = _f64(w.v_pool[pages, 0, g])
            for h in range(8 * g, 8 * g + 8):
                smax = w.sm_scale * np.max(k @ q[b, h]) / math.log(2.0)
                assert smax - 1e-12 <= lse[b, h] <= smax + math.log2(len(pages)) + 1e-12
                assert np.all(out[b, h] >= v.min(axis=0) - 1e-12)
                assert np.all(out[b, h] <= v.max(axis=0) + 1e-12)


def pin_peaky(ref):
    """Keys scaled by 30: the output sits on V of the best-scoring token."""
    w = _small_edge()
    b = 10
    out, lse = _decode(ref, w, batches=[b])
    pages = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
    q = _f64(w.q[b])
    hits = 0
    for g in range(4):
        k = _f64(w.k_pool[pages, 0, g])
        v = _f64(w.v_pool[pages, 0, g])
        for h in range(8 * g, 8 * g + 8):
            s = w.sm_scale * (k @ q[h])
            order = np.argsort(s)
            gap = s[order[-1]] - s[order[-2]]
            if gap > 40.0:   # every other weight is below e^-40
                hits += 1
                assert np.max(np.abs(out[b, h] - v[order[-1]])) <= 1e-12 * len(pages) + 1e-15
                assert abs(lse[b, h] - s[order[-1]] / math.log(2.0)) <= 1e-12 * len(pages)
    assert hits > 0


# --------------------------------------------------------------- split/merge

def pin_split_merge_identity(ref):
    """Merging the partials of any partition equals the unsplit result."""
    w = make_gqa(15, [300, 1, 77, 0, 129], pool_pages=600)
    rng = np.random.default_rng(5)
    full_out, full_lse = _decode(ref, w)
    for b in range(w.batch):
        n = int(w.lengths[b])
        cuts = sorted(set([0, n] + [int(x) for x in rng.integers(0, n + 1, size=3)]))
        cuts = [0] + cuts if cuts[0] != 0 else cuts
        parts = [(cuts[i], cuts[i + 1]) for i in range(len(cuts) - 1)] + [(n, n)]
        po, pl = [], []
        for lo, hi in parts:
            o, l_ = ref.gqa_decode_range(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices,
                                         w.sm_scale, b, lo, hi)
            po.append(o)
            pl.append(l_)
        mo, ml = ref.merge_lse2(np.stack(po), np.stack(pl))
        assert np.max(np.abs(mo - full_out[b])) <= 1e-12
        fin = np.isfinite(full_lse[b])
        assert np.array_equal(fin, np.isfinite(ml))
        if fin.any():
            assert np.max(np.abs(ml[fin] - full_lse[b][fin])) <= 1e-12


def pin_merge_closed_forms(ref):
    """Two parts with equal LSE average; a -inf part is ignored; all -inf gives 0 / -inf."""
    o = np.array([[[1.0, 2.0]], [[3.0, 6.0]]])
    mo, ml = ref.merge_lse2(o, np.array([[5.0], [5.0]]))
    assert np.allclose(mo, [[2.0, 4.0]], rtol=0, atol=1e-15) and abs(ml[0] - 6.0) <= 1e-15
    mo, ml = ref.merge_lse2(o, np.array([[-np.inf], [1.5]]))
    assert np.array_equal(mo, [[3.0, 6.0]]) and ml[0] == 1.5
    mo, ml = ref.merge_lse2(o, np.array([[-np.inf], [-np.inf]]))
    assert np.array_equal(mo, [[0.0, 0.0]]) and np.isneginf(ml[0])
    # weights 2^0 and 2^-1 (base 2): (1*1 + 0.5*3) / 1.5
    mo, ml = ref.merge_lse2(o, np.array([[2.0], [1.0]]))
    assert abs(mo[0, 0] - 2.5 / 1.5) <= 1e-15 and abs(ml[0] - (2.0 + math.log2(1.5))) <= 1e-15


# --------------------------------------------------------------- MLA gather

def _small_mla():
    if "small_mla" not in _CACHE:
        _CACHE["small_mla"] = make_mla(21, batch=3, num_qo_heads=16, pool_tokens=300, topk=64,
                                       masked_per_row=6)
    return _CACHE["small_mla"]


def pin_mla_masked_is_deleted(ref):
    w = _small_mla()
    out, lse = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v)
    for b in range(w.batch):
        kept = w.indices[b][w.indices[b] >= 0][None, :]
        o1, l1 = ref.mla_gather_decode(w.q[b:b + 1], w.kv_pool, kept, w.sm_scale, w.d_v)
        assert np.array_equal(out[b], o1[0]) and np.array_equal(lse[b], l1[0])
    # an id past the pool end behaves like -1
    idx = w.indices.copy()
    idx[idx < 0] = w.pool_tokens + 17
    o2, l2 = ref.mla_gather_decode(w.q, w.kv_pool, idx, w.sm_scale, w.d_v)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    # everything masked: zeros and -inf
    o3, l3 = ref.mla_gather_decode(w.q, w.kv_pool, -np.ones_like(w.indices), w.sm_scale, w.d_v)
    assert np.all(o3 == 0.0) and np.all(np.isneginf(l3))


def pin_mla_sdpa(ref):
    """Against torch SDPA: keys are the whole 576-wide row, values its first 512 dims."""
    w = _small_mla()
    out, lse = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v)
    pool = torch.as_tensor(_f64(w.kv_pool))
    for b in range(w.batch):
        ids = torch.as_tensor(w.indices[b][w.indices[b] >= 0].astype(np.int64))
        rows = pool[ids]                                   # [n, 576]
        q = torch.as_tensor(_f64(w.q[b]))                  # [H, 576]
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None, :, None, :], rows[None, None].expand(1, q.shape[0], -1, -1),
            rows[None, None, :, :w.d_v].expand(1, q.shape[0], -1, -1), scale=w.sm_scale)
        assert np.max(np.abs(out[b] - o[0, :, 0].numpy())) <= 1e-12
        scores = w.sm_scale * (q @ rows.T)
        l2 = (torch.logsumexp(scores, dim=-1) / math.log(2.0)).numpy()
        assert np.max(np.abs(lse[b] - l2)) <= 1e-12


def pin_mla_duplicates_count(ref):
    """A repeated id counts twice: same as adding log2(2) weight to that row."""
    w = _small_mla()
    ids = np.array([[5, 9, 9, 200]], dtype=np.int32)
    out, lse = ref.mla_gather_decode(w.q[:1], w.kv_pool, ids, w.sm_scale, w.d_v)
    q = _f64(w.q[0])
    rows = _f64(w.kv_pool[[5, 9, 200]])
    s = w.sm_scale * (q @ rows.T)
    e = np.exp(s) * np.array([1.0, 2.0, 1.0])
    want = (e @ rows[:, :w.d_v]) / e.sum(axis=1, keepdims=True)
    assert np.max(np.abs(out[0] - want)) <= 1e-12
    assert np.max(np.abs(lse[0] - np.log2(e.sum(axis=1)))) <= 1e-12


# ------------------------------------------------------ block-table decode

def _small_bt(page_size=16):
    key = f"small_bt{page_size}"
    if key not in _CACHE:
        _CACHE[key] = make_block_table(31 + page_size, [0, 1, 15, 16, 17, 40, 64, 5],
                                       page_size, extra_cols=3, pool_pages=None)
    return _CACHE[key]


def _bt(ref, w, **kw):
    return ref.gqa_block_table_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens,
                                      w.sm_scale, **kw)


def pin_bt_sdpa(ref):
    """Against torch SDPA over rows gathered one token at a time from the flat pool."""
    for ps in (4, 16):
        w = _small_bt(ps)
        out, lse = _bt(ref, w)
        flat_k = torch.as_tensor(_f64(w.k_pool)).reshape(-1, w.num_kv_heads, w.head_dim)
        flat_v = torch.as_tensor(_f64(w.v_pool)).reshape(-1, w.num_kv_heads, w.head_dim)
        for b in range(w.batch):
            n = int(w.seq_lens[b])
            if n == 0:
                assert np.all(out[b] == 0.0) and np.all(np.isneginf(lse[b]))
                continue
            rows = []
            for j in range(n):
                page, slot = divmod(j, ps)
                rows.append(int(w.block_table[b, page]) * ps + slot)
            rows = torch.tensor(rows)
            q = torch.as_tensor(_f64(w.q[b]))[:, None, :]                 # [Hq, 1, D]
            k = flat_k[rows].transpose(0, 1).contiguous()                  # [Hkv, n, D]
            v = flat_v[rows].transpose(0, 1).contiguous()
            o = torch.nn.functional.scaled_dot_product_attention(
                q[None], k[None], v[None], scale=w.sm_scale, enable_gqa=True)[0, :, 0, :]
            assert np.max(np.abs(out[b] - o.numpy())) <= 1e-12
            kk = k.repeat_interleave(w.num_qo_heads // w.num_kv_heads, dim=0)
            scores = w.sm_scale * torch.bmm(q, kk.transpose(1, 2).contiguous())[:, 0, :]
            l2 = (torch.logsumexp(scores, dim=-1) / math.log(2.0)).numpy()
            assert np.max(np.abs(lse[b] - l2)) <= 1e-12


def pin_bt_brute_force(ref):
    """Page size 4, lengths 3 and 9 (a partial page each), summed term by term."""
    w = make_block_table(41, [3, 9], 4, extra_cols=1)
    out, lse = _bt(ref, w)
    for b in range(2):
        q = _f64(w.q[b])
        for h in range(0, 32, 3):
            g = h // 8
            ks, vs = [], []
            for j in range(int(w.seq_lens[b])):
                page = int(w.block_table[b][j // 4])
                ks.append(_f64(w.k_pool[page, j % 4, g]))
                vs.append(_f64(w.v_pool[page, j % 4, g]))
            s = [w.sm_scale * math.fsum(float(a) * float(c) for a, c in zip(q[h], k)) for k in ks]
            e = [math.exp(x) for x in s]
            z = math.fsum(e)
            assert abs(lse[b, h] - math.log2(z)) <= 1e-12 * max(1.0, abs(math.log2(z)))
            for d in range(0, 128, 5):
                o = math.fsum(ei * float(vr[d]) for ei, vr in zip(e, vs)) / z
                assert abs(out[b, h, d] - o) <= 1e-12


def pin_bt_reduces_to_single_token_pages(ref):
    """Split every page into single-token pages and list them through the CSR
    function: the same rows in the same order give the same result, bit for bit."""
    for ps in (4, 16):
        w = _small_bt(ps)
        out, lse = _bt(ref, w)
        k1 = w.k_pool.reshape(-1, 1, w.num_kv_heads, w.head_dim)
        v1 = w.v_pool.reshape(-1, 1, w.num_kv_heads, w.head_dim)
        idx = []
        for b in range(w.batch):
            for j in range(int(w.seq_lens[b])):
                idx.append(int(w.block_table[b, j // ps]) * ps + j % ps)
        indptr = np.concatenate([[0], np.cumsum(w.seq_lens)]).astype(np.int32)
        o1, l1 = ref.gqa_paged_decode(w.q, k1, v1, indptr, np.array(idx, np.int32), w.sm_scale)
        assert np.array_equal(out, o1) and np.array_equal(lse, l1)


def pin_bt_unread_entries_and_slots(ref):
    """Table entries past a sequence's pages, slots past its length in the last
    page and pages nobody lists never reach the result."""
    w = _small_bt(16)
    out, lse = _bt(ref, w)
    table = w.block_table.copy()
    k = w.k_pool.copy()
    v = w.v_pool.copy()
    for b in range(w.batch):
        n = int(w.seq_lens[b])
        used = -(-n // 16)
        table[b, used:] = -1
        if n % 16:
            k[table[b, used - 1], n % 16:] = 0x7FC0
            v[table[b, used - 1], n % 16:] = 0x7FC0
    listed = np.zeros(w.num_pages, dtype=bool)
    for b in range(w.batch):
        listed[table[b][table[b] >= 0]] = True
    k[~listed] = 0x7FC0
    v[~listed] = 0x7FC0
    o1, l1 = ref.gqa_block_table_decode(w.q, k, v, table, w.seq_lens, w.sm_scale)
    assert np.array_equal(out, o1) and np.array_equal(lse, l1)


def pin_bt_single_token_and_empty(ref):
    w = _small_bt(16)
    out, lse = _bt(ref, w)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    page = int(w.block_table[1, 0])
    for h in range(32):
        assert np.array_equal(out[1, h], _f64(w.v_pool[page, 0, h // 8]))


def pin_mla_topk_length_is_a_prefix(ref):
    """A per-row length reads exactly that prefix of the row's list; lengths
    below 0 read nothing and above topk read the whole list."""
    w = _small_mla()
    lens = np.array([0, 37, 64], dtype=np.int32)
    out, lse = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v,
                                     topk_length=lens)
    for b, n in enumerate(lens):
        o1, l1 = ref.mla_gather_decode(w.q[b:b + 1], w.kv_pool, w.indices[b:b + 1, :n],
                                       w.sm_scale, w.d_v)
        assert np.array_equal(out[b], o1[0]) and np.array_equal(lse[b], l1[0])
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    o2, l2 = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v,
                                   topk_length=np.array([-5, 10 ** 6, 64], np.int32))
    full = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v)
    assert np.all(o2[0] == 0.0) and np.array_equal(o2[1:], full[0][1:])
    assert np.array_equal(l2[1:], full[1][1:])


def pin_mla_sink_as_zero_value_token(ref):
    """The sink is one more logit whose value row is zero: torch softmax over
    the scores with the sink appended, times the V rows with a zero row
    appended. The LSE stays that of the entries alone."""
    w = _small_mla()
    rng = np.random.default_rng(61)
    sink = rng.normal(0.0, 2.0, size=w.num_qo_heads)
    out, lse = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v,
                                     attn_sink=sink)
    _, lse0 = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v)
    assert np.array_equal(lse, lse0)
    pool = torch.as_tensor(_f64(w.kv_pool))
    for b in range(w.batch):
        ids = torch.as_tensor(w.indices[b][w.indices[b] >= 0].astype(np.int64))
        rows = pool[ids]
        q = torch.as_tensor(_f64(w.q[b]))
        logits = torch.cat([w.sm_scale * (q @ rows.T), torch.as_tensor(sink)[:, None]], dim=1)
        vals = torch.cat([rows[:, :w.d_v], torch.zeros(1, w.d_v, dtype=torch.float64)], dim=0)
        want = torch.softmax(logits, dim=1) @ vals
        assert np.max(np.abs(out[b] - want.numpy())) <= 1e-12


def pin_mla_sink_closed_forms(ref):
    """One valid entry with score s: out = v * e^s / (e^s + e^sink). A sink of
    -inf changes nothing; with no valid entry the sink leaves 0 and -inf."""
    w = _small_mla()
    ids = np.array([[42, -1, -1]], dtype=np.int32)
    sink = np.linspace(-3.0, 3.0, w.num_qo_heads)
    out, lse = ref.mla_gather_decode(w.q[:1], w.kv_pool, ids, w.sm_scale, w.d_v, attn_sink=sink)
    q = _f64(w.q[0])
    row = _f64(w.kv_pool[42])
    for h in range(w.num_qo_heads):
        s = w.sm_scale * math.fsum(float(a) * float(c) for a, c in zip(q[h], row))
        frac = 1.0 / (1.0 + math.exp(sink[h] - s))
        assert np.max(np.abs(out[0, h] - frac * row[:w.d_v])) <= 1e-12
        assert abs(lse[0, h] - s / math.log(2.0)) <= 1e-12
    o1, l1 = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v,
                                   attn_sink=np.full(w.num_qo_heads, -np.inf))
    o0, l0 = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v)
    assert np.max(np.abs(o1 - o0)) <= 1e-15 and np.array_equal(l1, l0)
    o2, l2 = ref.mla_gather_decode(w.q[:1], w.kv_pool, -np.ones((1, 4), np.int32), w.sm_scale,
                                   w.d_v, attn_sink=sink)
    assert np.all(o2 == 0.0) and np.all(np.isneginf(l2))


# --------------------------------------------------------------- FP8 gather

def pin_e4m3_decode(ref):
    """All 256 codes against torch's float8_e4m3fn, plus hand-checked values."""
    codes = np.arange(256, dtype=np.uint8)
    got = ref.e4m3_to_f64(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok]) and np.array_equal(np.signbit(got[ok]), np.signbit(want[ok]))
    hand = {0x38: 1.0, 0xB8: -1.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x08: 2.0 ** -6, 0x3C: 1.5,
            0x00: 0.0, 0x41: 2.25}
    for c, v in hand.items():
        assert ref.e4m3_to_f64(np.array([c], np.uint8))[0] == v, hex(c)
    assert np.isnan(ref.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()


def _fp8_token(codes, scales, rope_bits):
    t = np.zeros(656, dtype=np.uint8)
    t[:512] = codes
    t[512:528] = np.asarray(scales, dtype=np.float32).view(np.uint8)
    t[528:656] = np.asarray(rope_bits, dtype=np.uint16).view(np.uint8)
    return t


def pin_fp8_dequant_layout(ref):
    """Value i uses scale i // 128; the last 64 dims are the stored bf16 bits."""
    rope = np.arange(64, dtype=np.uint16) + 0x3F00
    tok = _fp8_token(np.full(512, 0x38, np.uint8), [1.0, 2.0, 0.25, 8.0], rope)   # all codes 1.0
    got = ref.dequant_fp8_rows(tok[None])[0]
    want = np.concatenate([np.full(128, 0x3F80), np.full(128, 0x4000), np.full(128, 0x3E80),
                           np.full(128, 0x4100)]).astype(np.uint16)
    assert np.array_equal(got[:512], want)
    assert np.array_equal(got[512:], rope)


def pin_fp8_dequant_rounding(ref):
    """Random codes and scales against torch: float8 -> float32, times the
    float32 scale, rounded to bfloat16."""
    rng = np.random.default_rng(71)
    n = 64
    codes = rng.integers(0, 256, size=(n, 512), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A                 # no NaN codes
    scales = (rng.random((n, 4)) * 0.02 + 1e-3).astype(np.float32)
    rope = rng.integers(0, 0x7F00, size=(n, 64), dtype=np.uint16)
    toks = np.stack([_fp8_token(codes[i], scales[i], rope[i]) for i in range(n)])
    got = ref.dequant_fp8_rows(toks)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).reshape(n, 4, 128)
    prod = (vals * torch.from_numpy(scales)[:, :, None]).reshape(n, 512)
    want = prod.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[:, :512], want)
    assert np.array_equal(got[:, 512:], rope)


def pin_fp8_gather_matches_known_values(ref):
    """Tokens built from values known exactly (e4m3 codes times powers of two)
    decode to the bf16 pool of those values: the FP8 gather then equals the
    bf16 gather over that pool."""
    rng = np.random.default_rng(72)
    t = 120
    codes = rng.integers(0, 0x7E, size=(t, 512), dtype=np.uint8) | (rng.integers(0, 2, size=(t, 512), dtype=np.uint8) << 7)
    exps = rng.integers(-8, 2, size=(t, 4))
    scales = np.exp2(exps).astype(np.float32)
    rope_vals = rng.standard_normal((t, 64)).astype(np.float32)
    rope = bf16_bits_from_f32(rope_vals)
    toks = np.stack([_fp8_token(codes[i], scales[i], rope[i]) for i in range(t)])
    vals = np.empty((t, 576), dtype=np.float32)
    for i in range(t):
        for j in range(512):
            c = int(codes[i, j])
            e, m = (c >> 3) & 15, c & 7
            mag = (1 + m / 8) * 2.0 ** (e - 7) if e else (m / 8) * 2.0 ** -6
            vals[i, j] = (-mag if c >> 7 else mag) * scales[i, j // 128]
    vals[:, 512:] = rope_vals
    pool_bits = bf16_bits_from_f32(vals)
    assert np.array_equal(ref.dequant_fp8_rows(toks), pool_bits)
    w = make_mla(73, batch=2, num_qo_heads=16, pool_tokens=t, topk=40, masked_per_row=3)
    o1, l1 = ref.mla_gather_decode_fp8(w.q, toks, w.indices, w.sm_scale)
    o2, l2 = ref.mla_gather_decode(w.q, pool_bits, w.indices, w.sm_scale, 512)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- KV append

def pin_append_round_trip(ref):
    """Each valid row reads back at its slot; every other slot keeps its bits;
    slots -1 and P * page_size store nothing."""
    rng = np.random.default_rng(51)
    pages, ps = 6, 4
    k = rng.integers(0, 1 << 16, size=(pages, ps, 2, 8), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(pages, ps, 2, 8), dtype=np.uint16)
    slots = np.array([5, -1, 0, 23, 24, 13, -7], dtype=np.int64)
    kr = rng.integers(0, 1 << 16, size=(7, 2, 8), dtype=np.uint16)
    vr = rng.integers(0, 1 << 16, size=(7, 2, 8), dtype=np.uint16)
    k2, v2 = ref.kv_append(k, v, kr, vr, slots)
    flat_k = k2.reshape(pages * ps, 2, 8)
    flat_v = v2.reshape(pages * ps, 2, 8)
    written = {5: 0, 0: 2, 23: 3, 13: 5}
    for slot in range(pages * ps):
        if slot in written:
            assert np.array_equal(flat_k[slot], kr[written[slot]])
            assert np.array_equal(flat_v[slot], vr[written[slot]])
        else:
            assert np.array_equal(flat_k[slot], k.reshape(-1, 2, 8)[slot])
            assert np.array_equal(flat_v[slot], v.reshape(-1, 2, 8)[slot])
    assert np.array_equal(k, k.copy())      # inputs untouched
    k3, _ = ref.kv_append(k, v, kr[:0], vr[:0], slots[:0])
    assert np.array_equal(k3, k)


def pin_append_then_decode(ref):
    """Appending a sequence's next token at the slot after its last one gives
    the decode of the longer sequence (the row enters the softmax)."""
    w = make_block_table(52, [5, 16, 30], 16, extra_cols=1, pool_pages=8)
    new_k = bf16_bits_from_f32(np.random.default_rng(53).standard_normal(
        (3, w.num_kv_heads, w.head_dim)).astype(np.float32))
    new_v = bf16_bits_from_f32(np.random.default_rng(54).standard_normal(
        (3, w.num_kv_heads, w.head_dim)).astype(np.float32))
    table = w.block_table.copy()
    spare = [p for p in range(w.num_pages)
             if p not in set(table[b, j] for b in range(3) for j in range(w.pages_per_seq[b]))]
    slots = []
    for b, n in enumerate(w.lengths):
        if n % 16 == 0:                       # a full last page: the next token opens a new one
            table[b, n // 16] = spare.pop()
        slots.append(int(table[b, n // 16]) * 16 + int(n % 16))
    k2, v2 = ref.kv_append(w.k_pool, w.v_pool, new_k, new_v, np.array(slots))
    out, lse = ref.gqa_block_table_decode(w.q, k2, v2, table, w.seq_lens + 1, w.sm_scale)
    for b, n in enumerate(w.lengths):
        rows = [(int(table[b, j // 16]), j % 16) for j in range(int(n))]
        kk = np.stack([_f64(w.k_pool[p, s]) for p, s in rows] + [_f64(new_k[b])])
        vv = np.stack([_f64(w.v_pool[p, s]) for p, s in rows] + [_f64(new_v[b])])
        q = _f64(w.q[b])
        for h in range(0, 32, 5):
            g = h // 8
            s = w.sm_scale * (kk[:, g] @ q[h])
            e = np.exp(s - s.max())
            assert np.max(np.abs(out[b, h] - (e @ vv[:, g]) / e.sum())) <= 1e-12
            assert abs(lse[b, h] - (s.max() + np.log(e.sum())) / math.log(2.0)) <= 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
