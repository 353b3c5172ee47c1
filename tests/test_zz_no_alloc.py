"""pkv_gather_mla_noalloc (partials in the library's device scratch) against
pkv_gather_mla (partials in a caller workspace): the two share every kernel, so
their outputs must agree bit for bit; both are also checked against the oracle
within the gather tolerances. Two calls in a row, the second with a smaller
input, since the scratch keeps the previous call's contents."""

import numpy as np
import pytest
import torch

import paged_kv_attention_gqa_amd as pkv
from gpu_util import assert_lse_close, assert_out_close, bf16_to_np, to_dev
from inputs import make_mla
from oracle import ref

pytestmark = pytest.mark.gpu


def _run_both(w):
    q = to_dev(w.q)
    pool = to_dev(w.kv_pool)
    idx = to_dev(w.indices)
    ws = torch.empty(max(pkv.pkv_gather_mla_workspace_size(w.batch, w.num_qo_heads, w.d_qk,
                                                           w.d_v, w.topk), 16),
                     dtype=torch.uint8, device="cuda")
    shape = (w.batch, w.num_qo_heads, w.d_v)
    out_a = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse_a = torch.empty(shape[:2], dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    lse_b = torch.empty_like(lse_a)
    pkv.pkv_gather_mla(q, pool, idx, w.sm_scale, ws, out_a, lse_a, w.d_v)
    pkv.pkv_gather_mla_noalloc(q, pool, idx, w.sm_scale, out_b, lse_b, w.d_v)
    torch.cuda.synchronize()
    return (out_a, lse_a), (out_b, lse_b)


def _check(w, got, want, what):
    assert_out_close(bf16_to_np(got[0]), want[0], what + " out")
    assert_lse_close(got[1].cpu().numpy().astype(np.float64), want[1], what + " lse")


def test_noalloc_gather_matches_workspace_gather_twice():
    big = make_mla(900, batch=32, num_qo_heads=128, pool_tokens=20000, topk=2048)
    small = make_mla(901, batch=5, num_qo_heads=64, pool_tokens=3000, topk=512)
    for w in (big, small):
        ws_bytes = pkv.pkv_gather_mla_workspace_size(w.batch, w.num_qo_heads, w.d_qk, w.d_v,
                                                     w.topk)
        assert 0 < ws_bytes <= 48 << 20      # the scratch is really used, and fits
        (oa, la), (ob, lb) = _run_both(w)
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16)), w.batch
        assert torch.equal(la, lb), w.batch
        want = ref.mla_gather_decode(w.q, w.kv_pool, w.indices, w.sm_scale, w.d_v)
        _check(w, (ob, lb), want, f"noalloc B={w.batch}")
