"""The decode kernel with its contractions on the vector ALU (PKV_ENGINE_DOT2,
v_dot2c_f32_bf16) against the fp64 oracle, through the C ABI.

Same definition and tolerances as the matrix-core engine: |out - ref| <=
1e-2 + 1e-2 |ref| per element, |lse - ref| <= 1e-3, -inf exactly where the
oracle has -inf. The engine reads the same tiles through the same plan, so
the cases below cover what differs: the score reduction across lanes, the
per-head softmax state shared between lanes, the P.V lane layout, and both
ways of addressing the pool.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_gqa_amd as pkv
from gpu_util import assert_lse_close, assert_out_close, bf16_to_np, to_dev, upload_gqa
from inputs import make_block_table, make_config, make_gqa
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
        if hasattr(w, "block_table"):
            _REF[name] = ref.gqa_block_table_decode(w.q, w.k_pool, w.v_pool, w.block_table,
                                                    w.seq_lens, w.sm_scale)
        else:
            _REF[name] = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr,
                                              w.kv_indices, w.sm_scale)
    return _REF[name]


def run_csr(w, dev=None, engine="dot2", sm_scale=None, **kw):
    dev = dev or upload_gqa(w)
    out, lse = pkv.decode(dev["q"], dev["k"], dev["v"], dev["indptr"], dev["indices"],
                          w.sm_scale if sm_scale is None else sm_scale,
                          kv_indptr_host=w.kv_indptr, engine=engine, **kw)
    torch.cuda.synchronize()
    return bf16_to_np(out), lse.cpu().numpy().astype(np.float64)


def run_table(w, engine="dot2", **kw):
    out, lse = pkv.decode_block_table(to_dev(w.q), to_dev(w.k_pool), to_dev(w.v_pool),
                                      to_dev(w.block_table), w.seq_lens, w.sm_scale,
                                      engine=engine, **kw)
    torch.cuda.synchronize()
    return bf16_to_np(out), lse.cpu().numpy().astype(np.float64)


def check(want, got, what):
    assert_out_close(got[0], want[0], what + " out")
    assert_lse_close(got[1], want[1], what + " lse")


@pytest.mark.parametrize("name", ["tiny", "edge", "gqa", "throughput"])
@pytest.mark.parametrize("split", [True, False], ids=["split", "nosplit"])
def test_config_vs_oracle(name, split):
    w = workload(name)
    check(oracle(name), run_csr(w, allow_split=split), f"dot2 {name} split={split}")


@pytest.mark.parametrize("name", ["gqa_ps16", "gqa_ps64", "edge_ps16"])
def test_block_table_vs_oracle(name):
    w = workload(name)
    check(oracle(name), run_table(w), f"dot2 {name}")


@pytest.mark.parametrize("chunk", [32, 64, 96, 1000])
def test_edge_chunk_sizes(chunk):
    w = workload("edge")
    check(oracle("edge"), run_csr(w, chunk_tokens=chunk), f"dot2 edge chunk={chunk}")


@pytest.mark.parametrize("lengths", [
    [1, 31, 32, 33, 63, 64, 65, 95, 96, 97],
    [0, 0, 5, 0],
    [2047, 2048, 2049, 1],
    [1],
])
@pytest.mark.parametrize("chunk", [0, 32])
def test_ragged_small(lengths, chunk):
    w = make_gqa(600 + len(lengths), lengths, pool_pages=sum(lengths) + 37)
    want = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices, w.sm_scale)
    check(want, run_csr(w, chunk_tokens=chunk), f"dot2 ragged {lengths} chunk={chunk}")


@pytest.mark.parametrize("ps", [1, 16, 64, 1024])
def test_block_table_partial_pages(ps):
    lengths = [1, ps - 1, ps, ps + 1, 5 * ps + 3, 0]
    w = make_block_table(610 + ps, lengths, ps)
    want = ref.gqa_block_table_decode(w.q, w.k_pool, w.v_pool, w.block_table, w.seq_lens,
                                      w.sm_scale)
    check(want, run_table(w, chunk_tokens=32), f"dot2 table ps={ps}")


def test_empty_and_single_token_exact():
    """n = 0 gives exact zeros and -inf; n = 1 gives the V row (p = 1, l = 1)."""
    w = workload("edge")
    out, lse = run_csr(w)
    assert np.all(out[0] == 0.0) and np.all(np.isneginf(lse[0]))
    page = int(w.kv_indices[w.kv_indptr[1]])
    v = ref.bf16_to_f64(w.v_pool[page, 0])
    for h in range(32):
        assert np.array_equal(out[1, h], v[h // 8]), h


def test_uniform_v_and_peaky_edge():
    """Constant V passes through; the K x 30 sequence (one score far above the
    rest) stays within tolerance (checked by the config test) and its LSE is
    finite."""
    w = workload("edge")
    out, lse = run_csr(w)
    assert np.max(np.abs(out[7] - 0.75)) <= 1e-2
    assert np.all(np.isfinite(lse[1:]))


@pytest.mark.parametrize("scale", [0.0, -0.0883883])
def test_sm_scale_zero_and_negative(scale):
    w = workload("tiny")
    want = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices, scale)
    check(want, run_csr(w, sm_scale=scale, chunk_tokens=32), f"dot2 sm_scale={scale}")


def test_engines_agree():
    """Both engines compute one definition; on the gqa workload their outputs
    stay within the oracle tolerance of each other and the plan (hence which
    outputs are merged) is the same."""
    w = workload("gqa")
    dev = upload_gqa(w)
    a = run_csr(w, dev, engine="mfma")
    b = run_csr(w, dev, engine="dot2")
    assert_out_close(b[0], a[0], "dot2 vs mfma out")
    assert_lse_close(b[1], a[1], "dot2 vs mfma lse")


def test_engine_switch_on_one_plan():
    """One plan and workspace, run with each engine in turn: the engine is a
    property of the run, and the second run overwrites the first's outputs."""
    w = make_gqa(620, [700, 3, 1500], pool_pages=2300)
    want = ref.gqa_paged_decode(w.q, w.k_pool, w.v_pool, w.kv_indptr, w.kv_indices, w.sm_scale)
    dev = upload_gqa(w)
    plan = pkv.pkv_plan_create(w.kv_indptr, chunk_tokens=128)
    ws = torch.empty(max(pkv.pkv_plan_workspace_size(plan), 16), dtype=torch.uint8,
                     device="cuda")
    pkv.pkv_plan_upload(plan, ws)
    for engine in ("dot2", "mfma", "dot2"):
        pkv.pkv_plan_set_engine(plan, engine)
        out = torch.full_like(dev["q"], float("nan"))
        lse = torch.full((3, 32), float("nan"), dtype=torch.float32, device="cuda")
        pkv.pkv_run(plan, dev["q"], dev["k"], dev["v"], dev["indptr"], dev["indices"],
                    w.sm_scale, ws, out, lse)
        pkv.pkv_merge(plan, ws, out, lse)
        torch.cuda.synchronize()
        check(want, (bf16_to_np(out), lse.cpu().numpy().astype(np.float64)), f"switch {engine}")


@pytest.mark.parametrize("chunk", [0, 64])
def test_exact_means_both_engines(chunk):
    """Inputs whose result is exact in every accumulation order: K = 0 (every
    score 0, so p = 1 and l counts the tokens), V = v0 +- 1/4 alternating over
    the tokens with v0 on a grid of 1/8 in [-4, 4] (every sum exact in fp32),
    and lengths and cuts that are multiples of 64 tokens (every piece holds as
    many + as - rows). The output is then v0 exactly, for both engines, split
    or not, through the merge's power-of-two weights."""
    lengths = [64, 128, 256, 512, 1024]
    w = make_gqa(630, lengths, pool_pages=sum(lengths) + 5)
    rng = np.random.default_rng(631)
    v0 = rng.integers(-32, 33, size=(len(lengths), 4, 128)).astype(np.float32) / 8.0
    k = np.zeros(w.k_pool.shape, dtype=np.float32)
    v = np.zeros(w.v_pool.shape, dtype=np.float32)
    for b, n in enumerate(lengths):
        for j in range(n):
            page = w.kv_indices[w.kv_indptr[b] + j]
            v[page, 0] = v0[b] + (0.25 if j % 2 == 0 else -0.25)
    from inputs.configs import bf16_bits_from_f32
    w.k_pool = bf16_bits_from_f32(k)
    w.v_pool = bf16_bits_from_f32(v)
    want = np.repeat(v0, 8, axis=1)   # query head h reads KV head h // 8
    dev = upload_gqa(w)
    outs = {}
    for engine in ("mfma", "dot2"):
        out, lse = run_csr(w, dev, engine=engine, chunk_tokens=chunk)
        assert np.array_equal(out, want), engine
        assert np.max(np.abs(lse - np.log2(np.array(lengths))[:, None])) <= 1e-6, engine
        outs[engine] = (out, lse)
    assert np.array_equal(outs["mfma"][1], outs["dot2"][1])
