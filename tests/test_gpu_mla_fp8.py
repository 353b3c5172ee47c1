"""Index-gather decode over an FP8 latent pool (656-byte tokens) on the GPU,
against the fp64 oracle, through the C ABI.

Tolerances as for the bf16 pool: |out - ref| <= 1e-2 + 1e-2 |ref|,
|lse - ref| <= 1e-3, -inf exactly where the oracle has -inf. The kernel
dequantises each value as the oracle does (fp32 product, bf16 rounding), so
its result must also equal, bit for bit, the bf16-pool kernel run on the
oracle's dequantised pool.
"""

import numpy as np
import pytest
import torch

import paged_kv_attention_gqa_amd as pkv
from gpu_util import assert_lse_close, assert_out_close, bf16_to_np, to_dev
from inputs import make_config, make_mla_fp8
from oracle import ref

pytestmark = pytest.mark.gpu


def run_fp8(w, indices=None, attn_sink=None, topk_length=None):
    idx = w.indices if indices is None else indices
    out, lse = pkv.gather_mla_fp8(
        to_dev(w.q), to_dev(w.kv_pool), to_dev(np.ascontiguousarray(idx)), w.sm_scale,
        attn_sink=None if attn_sink is None else to_dev(np.asarray(attn_sink, np.float32)),
        topk_length=None if topk_length is None else to_dev(np.asarray(topk_length, np.int32)))
    torch.cuda.synchronize()
    return bf16_to_np(out), lse.cpu().numpy().astype(np.float64)


def check(w, got, what, indices=None, attn_sink=None, topk_length=None):
    idx = w.indices if indices is None else indices
    want = ref.mla_gather_decode_fp8(
        w.q, w.kv_pool, idx, w.sm_scale,
        attn_sink=None if attn_sink is None else np.asarray(attn_sink, np.float32).astype(np.float64),
        topk_length=topk_length)
    assert_out_close(got[0], want[0], what + " out")
    assert_lse_close(got[1], want[1], what + " lse")


def test_fp8_config():
    w = make_config("mla_fp8")
    check(w, run_fp8(w), "mla_fp8 config")


def test_fp8_equals_bf16_kernel_on_dequantised_pool():
    w = make_config("mla_fp8")
    a = run_fp8(w)
    pool = ref.dequant_fp8_rows(w.kv_pool)                 # [T, 576] bf16 bits
    out, lse = pkv.gather_mla(to_dev(w.q), to_dev(pool), to_dev(w.indices), w.sm_scale)
    torch.cuda.synchronize()
    b = bf16_to_np(out), lse.cpu().numpy().astype(np.float64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("heads", [16, 64, 128])
@pytest.mark.parametrize("topk", [1, 33, 640])
def test_fp8_shapes(heads, topk):
    w = make_mla_fp8(60 + topk, batch=3, num_qo_heads=heads, pool_tokens=3000, topk=topk,
                     masked_per_row=topk // 7)
    check(w, run_fp8(w), f"fp8 heads={heads} topk={topk}")


def test_fp8_masking_with_nan_row_zero():
    """Masked entries read no pool row; NaN codes in row 0, which no entry
    lists, must not reach the output."""
    w = make_mla_fp8(65, batch=4, num_qo_heads=64, pool_tokens=900, topk=200, masked_per_row=20)
    w.kv_pool[0, :512] = 0x7F                                  # e4m3 NaN
    idx = w.indices.copy()
    idx[idx == 0] = 5                                          # nobody lists row 0 itself
    idx[0, :] = -1
    idx[1, ::3] = w.pool_tokens + 9
    idx[2, 10:20] = idx[2, 0]
    got = run_fp8(w, idx)
    check(w, got, "fp8 masking", indices=idx)
    assert np.all(got[0][0] == 0.0) and np.all(np.isneginf(got[1][0]))


def test_fp8_unlisted_rows_are_never_read():
    """Every token that no valid entry lists has NaN codes, NaN scales and a
    NaN bf16 tail; the output stays finite and equal to the oracle's."""
    w = make_mla_fp8(66, batch=3, num_qo_heads=64, pool_tokens=1500, topk=300, masked_per_row=40)
    idx = w.indices.copy()
    idx[1, ::5] = w.pool_tokens + 1
    idx[2, 100:] = -1
    listed = np.unique(idx[(idx >= 0) & (idx < w.pool_tokens)])
    unlisted = np.setdiff1d(np.arange(w.pool_tokens), listed)
    w.kv_pool[unlisted, :512] = 0x7F                              # e4m3 NaN
    w.kv_pool[unlisted, 512:528] = np.frombuffer(np.full(4, np.nan, np.float32).tobytes(), np.uint8)
    w.kv_pool[unlisted, 528:] = np.frombuffer(np.full(64, 0x7FC0, np.uint16).tobytes(), np.uint8)
    got = run_fp8(w, idx)
    assert np.all(np.isfinite(got[0]))
    check(w, got, "fp8 unlisted rows NaN", indices=idx)


def test_fp8_sink_and_lengths():
    w = make_mla_fp8(66, batch=6, num_qo_heads=128, pool_tokens=5000, topk=640)
    rng = np.random.default_rng(66)
    sink = rng.normal(0.5, 2.0, size=128).astype(np.float32)
    lens = np.array([640, 0, 1, 333, 700, -2], np.int32)
    check(w, run_fp8(w, attn_sink=sink, topk_length=lens), "fp8 sink+len", attn_sink=sink,
          topk_length=lens)
