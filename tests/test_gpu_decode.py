"""Paged GQA decode on the GPU against the fp64 oracle, through the C ABI.

Tolerances (bf16 output, fp32 LSE): |out - ref| <= 1e-2 + 1e-2 |ref| per
element, |lse - ref| <= 1e-3, and -inf exactly where the oracle has -inf.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_gqa_amd as pkv
from gpu_util import assert_lse_close, assert_out_close, bf16_to_np, to_dev, upload_gqa
from inputs import make_config, make_gqa
from oracle import ref

pytestmark = pytest.mark.gpu

_W = {}
_REF = {}


def workload(name):
    if name not in _W:
        _W[name] = make_config(name)
    return _W[name]


def oracle(name):
    if name not in _REF:
        w = workload(name)
        _REF[name] = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices,
                                          w.sm_scale)
    return _REF[name]


def run_gpu(w, dev=None, **kw):
    dev = dev or upload_gqa(w)
    out, lse = pkv.decode(dev["q"], dev["k"], dev["v"], dev["indptr"], dev["indices"], w.sm_scale,
                          kv_indptr_host=w.kv_indptr, **kw)
    torch.cuda.synchronize()
    return bf16_to_np(out), lse.cpu().numpy().astype(np.float64)


def check(w, want, got, what):
    assert_out_close(got[0], want[0], what + " out")
    assert_lse_close(got[1], want[1], what + " lse")


@pytest.mark.parametrize("name", ["tiny", "edge", "gqa", "throughput"])
@pytest.mark.parametrize("split", [True, False], ids=["split", "nosplit"])
def test_config_vs_oracle(name, split):
    w = workload(name)
    check(w, oracle(name), run_gpu(w, allow_split=split), f"{name} split={split}")


@pytest.mark.parametrize("chunk", [32, 64, 96, 256, 1000])
def test_edge_chunk_sizes(chunk):
    w = workload("edge")
    check(w, oracle("edge"), run_gpu(w, chunk_tokens=chunk), f"edge chunk={chunk}")


@pytest.mark.parametrize("lengths", [
    [1, 31, 32, 33, 63, 64, 65, 95, 96, 97],
    [0, 0, 5, 0],
    [2047, 2048, 2049, 1],
    [0],
    [1],
])
@pytest.mark.parametrize("chunk", [0, 32, 64])
def test_ragged_small(lengths, chunk):
    w = make_gqa(200 + len(lengths), lengths, pool_pages=sum(lengths) + 37)
    want = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices, w.sm_scale)
    check(w, want, run_gpu(w, chunk_tokens=chunk), f"ragged {lengths} chunk={chunk}")


def test_empty_batch():
    """B = 0: nothing to decode; the call returns empty outputs."""
    w = make_gqa(500, [], pool_pages=5)
    for chunk in (0, 32):
        out, lse = run_gpu(w, chunk_tokens=chunk)
        assert out.shape == (0, 32, 128) and lse.shape == (0, 32)


def test_many_short_sequences_per_worker():
    """3,000 sequences of 0-4 tokens and one of 5,000: the cost-balanced plan
    packs about ten short segments into a worker, and the long sequence is
    cut across workers."""
    rng = np.random.default_rng(230)
    lengths = [int(x) for x in rng.integers(0, 5, size=3000)]
    lengths[1234] = 5000
    w = make_gqa(231, lengths, pool_pages=sum(lengths) + 11)
    plan = pkv.pkv_plan_create(w.kv_indptr, num_cus=256)
    flat = pkv.pkv_plan_export(plan)
    assert max(np.diff(flat[4:5 + flat[0]])) >= 8 and flat[3] > 1
    want = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices, w.sm_scale)
    check(w, want, run_gpu(w), "many short sequences")


def test_empty_and_single_token_exact():
    """n = 0 gives exact zeros and -inf; n = 1 gives the V row rounded to bf16."""
    w = workload("edge")
    out, lse = run_gpu(w)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    page = int(w.kv_indices[w.kv_indptr[1]])
    v = ref.bf16_to_f64(w.v_pool[page, 0])          # [4, 128]
    for h in range(32):
        assert np.array_equal(out[1, h], v[h // 8]), h


def test_uniform_v_edge():
    w = workload("edge")
    out, _ = run_gpu(w)
    assert np.max(np.abs(out[7] - 0.75)) <= 1e-2


def test_split_matches_nosplit():
    w = workload("gqa")
    dev = upload_gqa(w)
    a = run_gpu(w, dev, allow_split=False)
    b = run_gpu(w, dev, chunk_tokens=64)
    assert_out_close(a[0], b[0], "split vs nosplit")
    assert np.max(np.abs(a[1] - b[1])) <= 1e-3


def test_timing_events_leave_results_unchanged():
    """A decode launched with timing events bound to its plan gives the same
    bits as one without, the events hold a positive duration shorter than the
    whole batch's wall time, and unbinding them restores plain launches."""
    w = workload("gqa")
    dev = upload_gqa(w)
    plan = pkv.pkv_plan_create(w.kv_indptr)
    ws = torch.empty(max(pkv.pkv_plan_workspace_size(plan), 16), dtype=torch.uint8, device="cuda")
    pkv.pkv_plan_upload(plan, ws)
    stream = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with pytest.raises(ValueError):
        pkv.pkv_plan_set_timing_events(plan, a, b)   # not created yet
    a.record(stream)
    b.record(stream)
    results = []
    for timed in (False, True, False):
        out = torch.empty_like(dev["q"])
        lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
        if timed:
            pkv.pkv_plan_set_timing_events(plan, a, b)
        pkv.pkv_run(plan, dev["q"], dev["k"], dev["v"], dev["indptr"], dev["indices"],
                    w.sm_scale, ws, out, lse)
        if timed:
            pkv.pkv_plan_set_timing_events(plan)
        pkv.pkv_merge(plan, ws, out, lse)
        torch.cuda.synchronize()
        results.append((bf16_to_np(out), lse.cpu().numpy()))
        if timed:
            ms = a.elapsed_time(b)
            assert 0.0 < ms < 50.0, ms
    for r in results[1:]:
        assert np.array_equal(r[0], results[0][0]) and np.array_equal(r[1], results[0][1])
    check(w, oracle("gqa"), (results[1][0], results[1][1].astype(np.float64)), "timed run")


def test_rerun_bit_identical():
    w = workload("gqa")
    dev = upload_gqa(w)
    a = run_gpu(w, dev)
    b = run_gpu(w, dev)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_physical_page_relabel_bit_identical():
    """Moving pages in the pool (and remapping the list) leaves the GPU result bit-identical."""
    w = workload("edge")
    a = run_gpu(w)
    rng = np.random.default_rng(17)
    perm = rng.permutation(w.num_pages)
    k = np.empty_like(w.k_pool)
    v = np.empty_like(w.v_pool)
    k[perm] = w.k_pool
    v[perm] = w.v_pool
    w2 = make_gqa(3, [0])   # container; fields replaced below
    w2.q, w2.k_pool, w2.v_pool = w.q, k, v
    w2.kv_indptr, w2.kv_indices, w2.sm_scale = w.kv_indptr, perm[w.kv_indices].astype(np.int32), w.sm_scale
    b = run_gpu(w2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_unused_pages_never_read():
    """NaN in every page no sequence lists must not reach the output."""
    w = workload("tiny")
    used = np.zeros(w.num_pages, dtype=bool)
    used[w.kv_indices] = True
    dev = upload_gqa(w)
    nan_rows = torch.from_numpy(np.nonzero(~used)[0]).cuda()
    dev["k"][nan_rows] = float("nan")
    dev["v"][nan_rows] = float("nan")
    out, lse = run_gpu(w, dev)
    check(w, oracle("tiny"), (out, lse), "tiny with NaN unused pages")


def test_many_split_sequences_and_workers():
    """Over 256 split sequences and over 256 workers: the merge records that do
    not fit the kernel arguments are read from the workspace, and workers past
    the first 256 take their first segment from their record."""
    rng = np.random.default_rng(303)
    lengths = [int(x) for x in rng.integers(65, 400, size=300)]
    lengths[7] = 0
    lengths[150] = 0
    w = make_gqa(303, lengths)
    plan = pkv.pkv_plan_create(w.kv_indptr, chunk_tokens=64)
    flat = pkv.pkv_plan_export(plan)
    assert flat[0] > 256 and flat[2] > 256                # workers, merge records
    want = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices, w.sm_scale)
    check(w, want, run_gpu(w, chunk_tokens=64), "300 sequences, 64-token chunks")
    check(w, want, run_gpu(w), "300 sequences, default plan")


def test_sm_scale_argument():
    w = make_gqa(300, [50, 700], pool_pages=800, sm_scale=0.3)
    want = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices, w.sm_scale)
    check(w, want, run_gpu(w), "sm_scale=0.3")
    w0 = make_gqa(301, [50, 700], pool_pages=800, sm_scale=0.0)
    want0 = ref.gqa_paged_decode(w0.q, w0.k_pool, w0.v_pool, w0.kv_indptr, w0.kv_indices, 0.0)
    check(w0, want0, run_gpu(w0), "sm_scale=0")
    wn = make_gqa(302, [50, 700], pool_pages=800, sm_scale=-1.0 / np.sqrt(128.0))
    wantn = ref.gqa_paged_decode(wn.q, wn.k_pool, wn.v_pool, wn.kv_indptr, wn.kv_indices, wn.sm_scale)
    check(wn, wantn, run_gpu(wn), "sm_scale<0")


def test_explicit_stream():
    w = workload("tiny")
    dev = upload_gqa(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse = pkv.decode(dev["q"], dev["k"], dev["v"], dev["indptr"], dev["indices"],
                              w.sm_scale, kv_indptr_host=w.kv_indptr)
    s.synchronize()
    check(w, oracle("tiny"), (bf16_to_np(out), lse.cpu().numpy().astype(np.float64)), "stream")


def test_plan_mismatch_raises():
    w = workload("tiny")
    dev = upload_gqa(w)
    ws = torch.empty(pkv.pkv_workspace_size(w.kv_indptr, num_cus=0), dtype=torch.uint8, device="cuda")
    plan = pkv.pkv_plan_create(w.kv_indptr, workspace=ws)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    other = torch.empty_like(ws)
    with pytest.raises(ValueError):
        pkv.pkv_run(plan, dev["q"], dev["k"], dev["v"], dev["indptr"], dev["indices"], w.sm_scale,
                    other, out, lse)
    with pytest.raises(ValueError):
        pkv.pkv_run(plan, dev["q"][:1].contiguous(), dev["k"], dev["v"], dev["indptr"][:2].contiguous(),
                    dev["indices"][:17].contiguous(), w.sm_scale, ws, out[:1].contiguous(),
                    lse[:1].contiguous())


def test_prepared_calls_match():
    """prepare_run / prepare_merge enqueue the same call as pkv_run / pkv_merge."""
    w = workload("edge")
    dev = upload_gqa(w)
    ws = torch.empty(pkv.pkv_workspace_size(w.kv_indptr), dtype=torch.uint8, device="cuda")
    plan = pkv.pkv_plan_create(w.kv_indptr, workspace=ws)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    run = pkv.prepare_run(plan, dev["q"], dev["k"], dev["v"], dev["indptr"], dev["indices"],
                          w.sm_scale, ws, out, lse)
    merge = pkv.prepare_merge(plan, ws, out, lse)
    for _ in range(2):
        run()
        merge()
    torch.cuda.synchronize()
    check(w, oracle("edge"), (bf16_to_np(out), lse.cpu().numpy().astype(np.float64)), "prepared")


@pytest.mark.parametrize("engine", ["mfma", "dot2"])
def test_hip_graph_replay_matches_eager(engine):
    """run + merge captured once in a HIP graph and replayed several times, with
    eager work and synchronisations between replays: every replay equals the
    eager result bit for bit (the calls enqueue kernels only), with either
    contraction engine."""
    w = workload("edge")
    dev = upload_gqa(w)
    ws = torch.empty(pkv.pkv_workspace_size(w.kv_indptr), dtype=torch.uint8, device="cuda")
    plan = pkv.pkv_plan_create(w.kv_indptr, workspace=ws)
    pkv.pkv_plan_set_engine(plan, engine)
    out = torch.empty_like(dev["q"])
    lse = torch.empty(dev["q"].shape[:2], dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    pkv.pkv_run(plan, dev["q"], dev["k"], dev["v"], dev["indptr"], dev["indices"], w.sm_scale, ws,
                out, lse)
    pkv.pkv_merge(plan, ws, out, lse)
    torch.cuda.synchronize()
    want = (bf16_to_np(out), lse.cpu().numpy().astype(np.float64))
    check(w, oracle("edge"), want, "eager")

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        run = pkv.prepare_run(plan, dev["q"], dev["k"], dev["v"], dev["indptr"], dev["indices"],
                              w.sm_scale, ws, out, lse, stream=s.cuda_stream)
        merge = pkv.prepare_merge(plan, ws, out, lse, stream=s.cuda_stream)
        with torch.cuda.graph(graph, stream=s):
            run()
            merge()
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        lse.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (bf16_to_np(out), lse.cpu().numpy().astype(np.float64))
        assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1]), f"replay {i}"
