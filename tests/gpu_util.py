"""Helpers for the GPU tests: uploading seeded inputs and comparing with the oracle."""

from __future__ import annotations

import numpy as np
import torch

OUT_ATOL = 1e-2
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    t = torch.from_numpy(a).cuda()
    return t if dtype is None else t.to(dtype)


def upload_gqa(w):
    return dict(q=to_dev(w.q), k=to_dev(w.k_pool), v=to_dev(w.v_pool),
                indptr=to_dev(w.kv_indptr), indices=to_dev(w.kv_indices))


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_out_close(got: np.ndarray, want: np.ndarray, what: str):
    """|got - want| <= 1e-2 + 1e-2 |want| elementwise; NaN anywhere fails."""
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    bound = OUT_ATOL + OUT_RTOL * np.abs(want)
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outputs beyond tolerance; "
                           f"max abs err {err.max():.4g}, worst excess {(err - bound).max():.4g}")


def assert_lse_close(got: np.ndarray, want: np.ndarray, what: str):
    neg = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), neg), f"{what}: -inf pattern differs"
    assert np.isfinite(got[~neg]).all(), f"{what}: non-finite LSE"
    if (~neg).any():
        err = np.abs(got[~neg] - want[~neg]).max()
        assert err <= LSE_ATOL, f"{what}: max |lse err| {err:.4g} > {LSE_ATOL}"
