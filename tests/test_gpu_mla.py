"""Index-gather latent-attention decode on the GPU against the fp64 oracle.

Tolerances: |out - ref| <= 1e-2 + 1e-2 |ref| per element, |lse - ref| <= 1e-3,
-inf exactly where the oracle has -inf (rows with no valid entry).
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_gqa_amd as pkv
from gpu_util import assert_lse_close, assert_out_close, bf16_to_np, to_dev
from inputs import make_config, make_mla
from oracle import ref

pytestmark = pytest.mark.gpu


def run_gpu(w, indices=None):
    idx = w.indices if indices is None else indices
    out, lse = pkv.gather_mla(to_dev(w.q), to_dev(w.kv_pool), to_dev(np.ascontiguousarray(idx)),
                              w.sm_scale, d_v=w.d_v)
    torch.cuda.synchronize()
    return bf16_to_np(out), lse.cpu().numpy().astype(np.float64)


def check(w, got, indices=None, what="mla"):
    idx = w.indices if indices is None else indices
    want = ref.mla_gather_decode(w.q, w.kv_pool, idx, w.sm_scale, w.d_v)
    assert_out_close(got[0], want[0], what + " out")
    assert_lse_close(got[1], want[1], what + " lse")


def test_mla_config():
    w = make_config("mla")
    check(w, run_gpu(w), what="mla config")


@pytest.mark.parametrize("heads", [16, 32, 48, 64, 128])
@pytest.mark.parametrize("topk", [1, 31, 32, 33, 100, 640])
def test_mla_shapes(heads, topk):
    w = make_mla(40 + topk, batch=3, num_qo_heads=heads, pool_tokens=4096, topk=topk,
                 masked_per_row=topk // 7)
    check(w, run_gpu(w), what=f"heads={heads} topk={topk}")


def test_mla_masking_rules():
    w = make_mla(51, batch=4, num_qo_heads=64, pool_tokens=1000, topk=200, masked_per_row=20)
    idx = w.indices.copy()
    idx[0, :] = -1                                  # nothing valid: zeros and -inf
    idx[1, ::3] = w.pool_tokens + 5                 # ids past the pool end are masked
    idx[2, 10:20] = idx[2, 0]                       # repeated ids each count
    idx[3, :] = -7
    idx[3, 150] = 3                                 # a single valid entry
    got = run_gpu(w, idx)
    check(w, got, idx, "masking")
    assert np.all(got[0][0] == 0.0) and np.all(np.isneginf(got[1][0]))
    single = ref.bf16_to_f64(w.kv_pool[3, :w.d_v])
    assert np.max(np.abs(got[0][3] - single)) <= 1e-2


def test_mla_unlisted_rows_are_never_read():
    """Every pool row that no valid entry lists holds NaN. Masked entries (-1,
    past the pool end, a masked tail spanning whole pieces) read nothing, so
    the output stays finite and equal to the oracle's."""
    w = make_mla(53, batch=3, num_qo_heads=128, pool_tokens=2000, topk=300, masked_per_row=40)
    idx = w.indices.copy()
    idx[1, ::5] = w.pool_tokens + 1
    idx[2, 100:] = -1
    listed = np.unique(idx[(idx >= 0) & (idx < w.pool_tokens)])
    unlisted = np.setdiff1d(np.arange(w.pool_tokens), listed)
    w.kv_pool[unlisted] = 0x7FC0                    # bf16 quiet NaN
    got = run_gpu(w, idx)
    assert np.all(np.isfinite(got[0]))
    check(w, got, idx, "unlisted rows NaN")


def test_mla_scale_and_rerun():
    w = make_mla(52, batch=2, num_qo_heads=128, pool_tokens=3000, topk=512, sm_scale=0.11)
    a = run_gpu(w)
    check(w, a, what="scale")
    b = run_gpu(w)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_mla_degenerate_shapes():
    """Empty lists, an empty pool and an empty batch: every row has no valid
    entry, so out is 0 and lse is -inf, as in the oracle."""
    w = make_mla(54, batch=2, num_qo_heads=64, pool_tokens=100, topk=8)
    empty = np.zeros((2, 0), np.int32)
    got = run_gpu(w, indices=empty)
    check(w, got, indices=empty, what="topk 0")
    assert not got[0].any() and np.all(got[1] == -np.inf)
    # pool of no rows: every id is out of range, so masked
    out, lse = pkv.gather_mla(to_dev(w.q), torch.empty((0, 576), dtype=torch.bfloat16, device="cuda"),
                              to_dev(w.indices), w.sm_scale, d_v=512)
    torch.cuda.synchronize()
    assert not bf16_to_np(out).any() and torch.all(lse == -torch.inf)
    # no rows at all
    out, lse = pkv.gather_mla(to_dev(w.q)[:0], to_dev(w.kv_pool), to_dev(w.indices)[:0],
                              w.sm_scale, d_v=512)
    torch.cuda.synchronize()
    assert out.shape == (0, 64, 512) and lse.shape == (0, 64)


def test_mla_shape_errors():
    w = make_mla(53, batch=1, num_qo_heads=16, pool_tokens=100, topk=8)
    q = to_dev(w.q)
    with pytest.raises(ValueError):
        pkv.gather_mla(q[:, :, :512].contiguous(), to_dev(w.kv_pool)[:, :512].contiguous(),
                       to_dev(w.indices), w.sm_scale, d_v=512)


def run_gpu_ex(w, attn_sink=None, topk_length=None):
    sink_t = None if attn_sink is None else to_dev(np.asarray(attn_sink, np.float32))
    len_t = None if topk_length is None else to_dev(np.asarray(topk_length, np.int32))
    out, lse = pkv.gather_mla(to_dev(w.q), to_dev(w.kv_pool), to_dev(w.indices), w.sm_scale,
                              d_v=w.d_v, attn_sink=sink_t, topk_length=len_t)
    torch.cuda.synchronize()
    return bf16_to_np(out), lse.cpu().numpy().astype(np.float64)


def check_ex(w, got, what, attn_sink=None, topk_length=None):
    want = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v,
                                 attn_sink=None if attn_sink is None else
                                 np.asarray(attn_sink, np.float32).astype(np.float64),
                                 topk_length=topk_length)
    assert_out_close(got[0], want[0], what + " out")
    assert_lse_close(got[1], want[1], what + " lse")


def test_mla_config_with_sink_and_lengths():
    """Full-size list cut into pieces (merge path) with a sink per head and a
    length per row, including 0, the whole list, and values outside [0, topk]."""
    w = make_config("mla")
    rng = np.random.default_rng(81)
    sink = rng.normal(1.0, 2.0, size=w.num_qo_heads).astype(np.float32)
    lens = rng.integers(0, w.topk + 1, size=w.batch).astype(np.int32)
    lens[:5] = [0, w.topk, w.topk + 100, -3, 1]
    check_ex(w, run_gpu_ex(w, sink, lens), "mla sink+len", sink, lens)
    check_ex(w, run_gpu_ex(w, sink, None), "mla sink", sink, None)
    check_ex(w, run_gpu_ex(w, None, lens), "mla len", None, lens)


@pytest.mark.parametrize("topk", [33, 100, 640])
def test_mla_sink_and_length_shapes(topk):
    w = make_mla(90 + topk, batch=4, num_qo_heads=64, pool_tokens=2048, topk=topk,
                 masked_per_row=topk // 9)
    rng = np.random.default_rng(topk)
    sink = rng.normal(0.0, 3.0, size=64).astype(np.float32)
    sink[:4] = [50.0, -50.0, 0.0, np.inf]            # output ~0, no effect, even, all to the sink
    lens = np.array([topk, topk // 2, 1, 0], np.int32)
    check_ex(w, run_gpu_ex(w, sink, lens), f"topk={topk}", sink, lens)


def test_mla_sink_minus_inf_is_bit_identical():
    w = make_mla(95, batch=3, num_qo_heads=128, pool_tokens=4096, topk=640)
    a = run_gpu_ex(w)
    b = run_gpu_ex(w, attn_sink=np.full(128, -np.inf, np.float32))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = run_gpu_ex(w, topk_length=np.full(3, 640, np.int32))
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])


def test_mla_hip_graph_replay_matches_eager():
    """The gather (partial kernel + merge) captured once in a HIP graph and
    replayed with eager work between replays equals the eager call bit for
    bit: the call only enqueues kernels."""
    w = make_mla(54, batch=4, num_qo_heads=128, pool_tokens=3000, topk=600, masked_per_row=30)
    q, pool, idx = to_dev(w.q), to_dev(w.kv_pool), to_dev(w.indices)
    ws = torch.empty(max(16, pkv.pkv_gather_mla_workspace_size(w.batch, 128, 576, 512, w.topk)),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((w.batch, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.batch, 128), dtype=torch.float32, device="cuda")
    pkv.pkv_gather_mla(q, pool, idx, w.sm_scale, ws, out, lse)
    torch.cuda.synchronize()
    want = (bf16_to_np(out), lse.cpu().numpy().astype(np.float64))
    check(w, want, what="eager")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            pkv.pkv_gather_mla(q, pool, idx, w.sm_scale, ws, out, lse, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (bf16_to_np(out), lse.cpu().numpy().astype(np.float64))
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), f"replay {i}"
