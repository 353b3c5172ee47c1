"""Python binding of libpkv (paged KV-cache attention decode for MI355X).

Argument marshalling only: every function here turns torch tensors into
pointers and sizes and calls the C entry point of the same name declared in
``include/pkv.h``. All computation happens in the library's HIP kernels. The
library is loaded on first use; if it has not been built, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import numpy as np

from ._build import LIB_PATH

__all__ = [
    "PkvError", "Plan", "decode", "gather_mla", "library_path",
    "pkv_workspace_size", "pkv_plan_create", "pkv_plan_destroy", "pkv_plan_export",
    "pkv_plan_workspace_size", "pkv_plan_upload", "pkv_plan_set_engine",
    "pkv_plan_set_timing_events",
    "PKV_ENGINE_MFMA", "PKV_ENGINE_DOT2",
    "pkv_run", "pkv_merge", "pkv_gather_mla_workspace_size", "pkv_gather_mla",
    "prepare_run", "prepare_merge", "prepare_gather_mla", "prepare_append_kv",
    "pkv_block_table_workspace_size", "pkv_block_table_plan_create", "pkv_block_table_run",
    "prepare_block_table_run", "decode_block_table", "pkv_append_kv",
    "pkv_gather_mla_fp8", "gather_mla_fp8", "pkv_gather_mla_noalloc",
    "pkv_status_string", "pkv_last_error",
]

PKV_OK = 0
PKV_ERR_INVALID_ARG = 1
PKV_ERR_UNSUPPORTED = 2
PKV_ERR_WORKSPACE_TOO_SMALL = 3
PKV_ERR_PLAN_MISMATCH = 4
PKV_ERR_HIP = 5

PKV_ENGINE_MFMA = 0
PKV_ENGINE_DOT2 = 1
ENGINES = {"mfma": PKV_ENGINE_MFMA, "dot2": PKV_ENGINE_DOT2}

# Every symbol include/pkv.h declares, with (restype, argtypes).
_c = ctypes
_P = _c.c_void_p
_I32 = _c.c_int32
_I64 = _c.c_int64
_SZ = _c.c_size_t
_I32P = _c.POINTER(_c.c_int32)
SIGNATURES = {
    "pkv_workspace_size": (_I32, [_I32P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                  _c.POINTER(_SZ)]),
    "pkv_plan_create": (_I32, [_I32P, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _I32, _P, _SZ,
                               _P, _c.POINTER(_P)]),
    "pkv_plan_destroy": (None, [_P]),
    "pkv_plan_workspace_size": (_I32, [_P, _c.POINTER(_SZ)]),
    "pkv_plan_upload": (_I32, [_P, _P, _SZ, _P]),
    "pkv_plan_set_engine": (_I32, [_P, _I32]),
    "pkv_plan_set_timing_events": (_I32, [_P, _P, _P]),
    "pkv_plan_export": (_I32, [_P, _I32P, _SZ, _c.POINTER(_SZ)]),
    "pkv_run": (_I32, [_P, _P, _I32, _I32, _I32, _P, _P, _I64, _I32, _I32, _I32, _P, _I64, _P,
                       _I64, _c.c_float, _P, _SZ, _P, _P, _P]),
    "pkv_block_table_workspace_size": (_I32, [_I32P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                              _I32, _c.POINTER(_SZ)]),
    "pkv_block_table_plan_create": (_I32, [_I32P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                           _I32, _P, _SZ, _P, _c.POINTER(_P)]),
    "pkv_block_table_run": (_I32, [_P, _P, _I32, _I32, _I32, _P, _P, _I64, _I32, _I32, _I32, _P,
                                   _I32, _I32, _c.c_float, _P, _SZ, _P, _P, _P]),
    "pkv_merge": (_I32, [_P, _P, _SZ, _P, _P, _P]),
    "pkv_append_kv": (_I32, [_P, _P, _I64, _I32, _I32, _I32, _P, _P, _P, _I64, _P]),
    "pkv_gather_mla_workspace_size": (_I32, [_I32, _I32, _I32, _I32, _I32, _c.POINTER(_SZ)]),
    "pkv_gather_mla": (_I32, [_P, _P, _I64, _P, _I32, _I32, _I32, _I32, _I32, _c.c_float, _P,
                              _P, _P, _SZ, _P, _P, _P]),
    "pkv_gather_mla_noalloc": (_I32, [_P, _P, _I64, _P, _I32, _I32, _I32, _I32, _I32,
                                      _c.c_float, _P, _P, _P, _P, _P]),
    "pkv_gather_mla_fp8": (_I32, [_P, _P, _I64, _P, _I32, _I32, _I32, _I32, _I32, _c.c_float,
                                  _P, _P, _P, _SZ, _P, _P, _P]),
    "pkv_status_string": (_c.c_char_p, [_I32]),
    "pkv_last_error": (_c.c_char_p, []),
}

_LIB = None


def library_path() -> str:
    return LIB_PATH


def lib():
    """The loaded libpkv (ctypes). Raises if the library has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libpkv.so is not built ({LIB_PATH}); run "
                               "paged_kv_attention_gqa_amd._build.build() first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


class PkvError(Exception):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = lib().pkv_last_error().decode()
        text = lib().pkv_status_string(status).decode()
        super().__init__(f"{where}: {text} ({status}): {detail}")


class PkvValueError(PkvError, ValueError):
    pass


class PkvRuntimeError(PkvError, RuntimeError):
    pass


def _check(status: int, where: str):
    if status != PKV_OK:
        raise (PkvRuntimeError if status == PKV_ERR_HIP else PkvValueError)(status, where)


def pkv_status_string(status: int) -> str:
    return lib().pkv_status_string(status).decode()


def pkv_last_error() -> str:
    return lib().pkv_last_error().decode()


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _host_indptr(kv_indptr_host) -> np.ndarray:
    if hasattr(kv_indptr_host, "detach"):
        kv_indptr_host = kv_indptr_host.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(kv_indptr_host), dtype=np.int32)


def _require(t, name, dtypes, cuda=True):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if cuda and t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")


def _bf16_types():
    import torch
    return (torch.bfloat16, torch.int16, torch.uint16)


def pkv_workspace_size(kv_indptr_host, num_qo_heads=32, num_kv_heads=4, head_dim=128,
                       page_size=1, num_cus=0, allow_split=True, chunk_tokens=0) -> int:
    ind = _host_indptr(kv_indptr_host)
    out = ctypes.c_size_t(0)
    _check(lib().pkv_workspace_size(ind.ctypes.data_as(_I32P), len(ind) - 1, num_qo_heads,
                                    num_kv_heads, head_dim, page_size, num_cus,
                                    int(bool(allow_split)), chunk_tokens, ctypes.byref(out)),
           "pkv_workspace_size")
    return int(out.value)


class Plan:
    """Owns one pkv_plan handle (destroyed with the object, by the library that made it)."""

    def __init__(self, handle: int, batch: int, total_tokens: int):
        self.handle = handle
        self.batch = batch
        self.total_tokens = total_tokens
        self._lib = lib()

    def __del__(self):
        if getattr(self, "handle", None):
            self._lib.pkv_plan_destroy(self.handle)
            self.handle = None


def pkv_plan_create(kv_indptr_host, num_qo_heads=32, num_kv_heads=4, head_dim=128, page_size=1,
                    num_cus=0, allow_split=True, chunk_tokens=0, workspace=None,
                    stream=None) -> Plan:
    ind = _host_indptr(kv_indptr_host)
    if workspace is not None:
        _require(workspace, "workspace", (__import__("torch").uint8,))
    handle = ctypes.c_void_p(0)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = 0 if workspace is None else _stream(stream)
    _check(lib().pkv_plan_create(ind.ctypes.data_as(_I32P), len(ind) - 1, num_qo_heads,
                                 num_kv_heads, head_dim, page_size, num_cus,
                                 int(bool(allow_split)), chunk_tokens, _ptr(workspace), ws_bytes,
                                 st, ctypes.byref(handle)),
           "pkv_plan_create")
    return Plan(handle.value, len(ind) - 1, int(ind[-1]) if len(ind) else 0)


def pkv_plan_destroy(plan: Plan):
    if plan.handle:
        plan._lib.pkv_plan_destroy(plan.handle)
        plan.handle = None


def pkv_plan_export(plan: Plan) -> list:
    need = ctypes.c_size_t(0)
    _check(lib().pkv_plan_export(plan.handle, None, 0, ctypes.byref(need)), "pkv_plan_export")
    buf = (ctypes.c_int32 * need.value)()
    _check(lib().pkv_plan_export(plan.handle, buf, need.value, ctypes.byref(need)),
           "pkv_plan_export")
    return list(buf)


def _run_args(plan: Plan, q, k_pool, v_pool, kv_indptr, kv_indices, sm_scale, workspace, out,
              lse, stream):
    import torch
    bf = _bf16_types()
    _require(q, "q", bf)
    _require(k_pool, "k_pool", bf)
    _require(v_pool, "v_pool", bf)
    _require(kv_indptr, "kv_indptr", (torch.int32,))
    _require(kv_indices, "kv_indices", (torch.int32,))
    _require(workspace, "workspace", (torch.uint8,))
    _require(out, "out", bf)
    _require(lse, "lse", (torch.float32,))
    if q.dim() != 3 or k_pool.dim() != 4:
        raise ValueError("q must be [B, Hq, D] and the pools [pages, page_size, Hkv, D]")
    if tuple(k_pool.shape) != tuple(v_pool.shape):
        raise ValueError("k_pool and v_pool must have the same shape")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != tuple(q.shape[:2]):
        raise ValueError("out must be shaped like q and lse like q.shape[:2]")
    return (plan.handle, _ptr(q), q.shape[0], q.shape[1], q.shape[2], _ptr(k_pool), _ptr(v_pool),
            k_pool.shape[0], k_pool.shape[1], k_pool.shape[2], k_pool.shape[3], _ptr(kv_indptr),
            kv_indptr.numel(), _ptr(kv_indices), kv_indices.numel(), float(sm_scale),
            _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream(stream))


def pkv_run(plan: Plan, q, k_pool, v_pool, kv_indptr, kv_indices, sm_scale, workspace, out,
            lse, stream=None):
    _check(lib().pkv_run(*_run_args(plan, q, k_pool, v_pool, kv_indptr, kv_indices, sm_scale,
                                    workspace, out, lse, stream)),
           "pkv_run")


def prepare_run(plan: Plan, q, k_pool, v_pool, kv_indptr, kv_indices, sm_scale, workspace, out,
                lse, stream=None):
    """Marshal the arguments of pkv_run once; the returned callable enqueues the
    same call again (same tensors, same stream) with no per-call checks in Python.
    The tensors must stay alive and in place while the callable is used."""
    args = _run_args(plan, q, k_pool, v_pool, kv_indptr, kv_indices, sm_scale, workspace, out,
                     lse, stream)
    fn = plan._lib.pkv_run

    def call():
        st = fn(*args)
        if st != PKV_OK:
            _check(st, "pkv_run")
    return call


def prepare_merge(plan: Plan, workspace, out, lse, stream=None):
    """Like prepare_run, for pkv_merge."""
    args = (plan.handle, _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
            _stream(stream))
    fn = plan._lib.pkv_merge

    def call():
        st = fn(*args)
        if st != PKV_OK:
            _check(st, "pkv_merge")
    return call


def _host_lengths(seq_lens_host) -> np.ndarray:
    if hasattr(seq_lens_host, "detach"):
        seq_lens_host = seq_lens_host.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(seq_lens_host), dtype=np.int32).reshape(-1)


def pkv_block_table_workspace_size(seq_lens_host, num_qo_heads=32, num_kv_heads=4, head_dim=128,
                                   page_size=16, num_cus=0, allow_split=True,
                                   chunk_tokens=0) -> int:
    lens = _host_lengths(seq_lens_host)
    out = ctypes.c_size_t(0)
    _check(lib().pkv_block_table_workspace_size(lens.ctypes.data_as(_I32P), len(lens),
                                                num_qo_heads, num_kv_heads, head_dim, page_size,
                                                num_cus, int(bool(allow_split)), chunk_tokens,
                                                ctypes.byref(out)),
           "pkv_block_table_workspace_size")
    return int(out.value)


def pkv_block_table_plan_create(seq_lens_host, num_qo_heads=32, num_kv_heads=4, head_dim=128,
                                page_size=16, num_cus=0, allow_split=True, chunk_tokens=0,
                                workspace=None, stream=None) -> Plan:
    lens = _host_lengths(seq_lens_host)
    if workspace is not None:
        _require(workspace, "workspace", (__import__("torch").uint8,))
    handle = ctypes.c_void_p(0)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = 0 if workspace is None else _stream(stream)
    _check(lib().pkv_block_table_plan_create(lens.ctypes.data_as(_I32P), len(lens), num_qo_heads,
                                             num_kv_heads, head_dim, page_size, num_cus,
                                             int(bool(allow_split)), chunk_tokens,
                                             _ptr(workspace), ws_bytes, st, ctypes.byref(handle)),
           "pkv_block_table_plan_create")
    return Plan(handle.value, len(lens), int(lens.astype(np.int64).sum()))


def _block_table_args(plan: Plan, q, k_pool, v_pool, block_table, sm_scale, workspace, out, lse,
                      stream):
    import torch
    bf = _bf16_types()
    _require(q, "q", bf)
    _require(k_pool, "k_pool", bf)
    _require(v_pool, "v_pool", bf)
    _require(block_table, "block_table", (torch.int32,))
    _require(workspace, "workspace", (torch.uint8,))
    _require(out, "out", bf)
    _require(lse, "lse", (torch.float32,))
    if q.dim() != 3 or k_pool.dim() != 4 or block_table.dim() != 2:
        raise ValueError("q must be [B, Hq, D], the pools [pages, page_size, Hkv, D] and "
                         "block_table [B, max_pages]")
    if tuple(k_pool.shape) != tuple(v_pool.shape):
        raise ValueError("k_pool and v_pool must have the same shape")
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != tuple(q.shape[:2]):
        raise ValueError("out must be shaped like q and lse like q.shape[:2]")
    return (plan.handle, _ptr(q), q.shape[0], q.shape[1], q.shape[2], _ptr(k_pool), _ptr(v_pool),
            k_pool.shape[0], k_pool.shape[1], k_pool.shape[2], k_pool.shape[3], _ptr(block_table),
            block_table.shape[0], block_table.shape[1], float(sm_scale), _ptr(workspace),
            workspace.numel(), _ptr(out), _ptr(lse), _stream(stream))


def pkv_block_table_run(plan: Plan, q, k_pool, v_pool, block_table, sm_scale, workspace, out,
                        lse, stream=None):
    _check(lib().pkv_block_table_run(*_block_table_args(plan, q, k_pool, v_pool, block_table,
                                                        sm_scale, workspace, out, lse, stream)),
           "pkv_block_table_run")


def prepare_block_table_run(plan: Plan, q, k_pool, v_pool, block_table, sm_scale, workspace, out,
                            lse, stream=None):
    """Like prepare_run, for pkv_block_table_run."""
    args = _block_table_args(plan, q, k_pool, v_pool, block_table, sm_scale, workspace, out, lse,
                             stream)
    fn = plan._lib.pkv_block_table_run

    def call():
        st = fn(*args)
        if st != PKV_OK:
            _check(st, "pkv_block_table_run")
    return call


def pkv_merge(plan: Plan, workspace, out, lse, stream=None):
    _check(lib().pkv_merge(plan.handle, _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
                           _stream(stream)),
           "pkv_merge")


def pkv_append_kv(k_pool, v_pool, k_rows, v_rows, slot_mapping, stream=None):
    """Store k_rows / v_rows ``[n, Hkv, D]`` at the int64 ``slot_mapping`` positions
    of the pools ``[pages, page_size, Hkv, D]`` (slots outside the pool are skipped)."""
    _check(lib().pkv_append_kv(*_append_args(k_pool, v_pool, k_rows, v_rows, slot_mapping,
                                             stream)), "pkv_append_kv")


def prepare_append_kv(k_pool, v_pool, k_rows, v_rows, slot_mapping, stream=None):
    """Like prepare_run, for pkv_append_kv."""
    args = _append_args(k_pool, v_pool, k_rows, v_rows, slot_mapping, stream)
    fn = lib().pkv_append_kv

    def call():
        st = fn(*args)
        if st != PKV_OK:
            _check(st, "pkv_append_kv")
    return call


def _append_args(k_pool, v_pool, k_rows, v_rows, slot_mapping, stream):
    import torch
    bf = _bf16_types()
    for t, name in ((k_pool, "k_pool"), (v_pool, "v_pool"), (k_rows, "k_rows"),
                    (v_rows, "v_rows")):
        _require(t, name, bf)
    _require(slot_mapping, "slot_mapping", (torch.int64,))
    if k_pool.dim() != 4 or tuple(v_pool.shape) != tuple(k_pool.shape):
        raise ValueError("the pools must both be [pages, page_size, Hkv, D]")
    n = slot_mapping.numel()
    want = (n, k_pool.shape[2], k_pool.shape[3])
    if tuple(k_rows.shape) != want or tuple(v_rows.shape) != want:
        raise ValueError(f"k_rows and v_rows must be {list(want)}")
    return (_ptr(k_pool), _ptr(v_pool), k_pool.shape[0], k_pool.shape[1], k_pool.shape[2],
            k_pool.shape[3], _ptr(k_rows), _ptr(v_rows), _ptr(slot_mapping), n, _stream(stream))


def pkv_gather_mla_workspace_size(batch, num_qo_heads, d_qk, d_v, topk) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().pkv_gather_mla_workspace_size(batch, num_qo_heads, d_qk, d_v, topk,
                                               ctypes.byref(out)),
           "pkv_gather_mla_workspace_size")
    return int(out.value)


def pkv_gather_mla(q, kv_pool, indices, sm_scale, workspace, out, lse, d_v=512, stream=None,
                   attn_sink=None, topk_length=None):
    _gather(False, q, kv_pool, indices, sm_scale, workspace, out, lse, d_v, stream, attn_sink,
            topk_length)


def pkv_gather_mla_noalloc(q, kv_pool, indices, sm_scale, out, lse, d_v=512, stream=None,
                           attn_sink=None, topk_length=None):
    """pkv_gather_mla with the partials in the library's device scratch (no workspace)."""
    _gather(False, q, kv_pool, indices, sm_scale, None, out, lse, d_v, stream, attn_sink,
            topk_length, noalloc=True)


def pkv_gather_mla_fp8(q, kv_pool, indices, sm_scale, workspace, out, lse, d_v=512, stream=None,
                       attn_sink=None, topk_length=None):
    """Like pkv_gather_mla over a uint8 pool of 656-byte FP8 tokens ``[T, 656]``."""
    _gather(True, q, kv_pool, indices, sm_scale, workspace, out, lse, d_v, stream, attn_sink,
            topk_length)


def _gather(fp8, q, kv_pool, indices, sm_scale, workspace, out, lse, d_v, stream, attn_sink,
            topk_length, noalloc=False):
    fn, args, name = _gather_args(fp8, q, kv_pool, indices, sm_scale, workspace, out, lse, d_v,
                                  stream, attn_sink, topk_length, noalloc)
    _check(fn(*args), name)


def prepare_gather_mla(q, kv_pool, indices, sm_scale, workspace, out, lse, d_v=512, stream=None,
                       attn_sink=None, topk_length=None, fp8=False, noalloc=False):
    """Marshal a pkv_gather_mla (or _fp8 / _noalloc) call once; the returned
    callable enqueues the same call again with no per-call checks in Python.
    The tensors must stay alive and in place while the callable is used."""
    fn, args, name = _gather_args(fp8, q, kv_pool, indices, sm_scale, workspace, out, lse, d_v,
                                  stream, attn_sink, topk_length, noalloc)

    def call():
        st = fn(*args)
        if st != PKV_OK:
            _check(st, name)
    return call


def _gather_args(fp8, q, kv_pool, indices, sm_scale, workspace, out, lse, d_v, stream, attn_sink,
                 topk_length, noalloc=False):
    import torch
    bf = _bf16_types()
    _require(q, "q", bf)
    _require(kv_pool, "kv_pool", (torch.uint8,) if fp8 else bf)
    _require(indices, "indices", (torch.int32,))
    _require(attn_sink, "attn_sink", (torch.float32,))
    _require(topk_length, "topk_length", (torch.int32,))
    if attn_sink is not None and tuple(attn_sink.shape) != (q.shape[1],):
        raise ValueError("attn_sink must be [num_qo_heads]")
    if topk_length is not None and tuple(topk_length.shape) != (q.shape[0],):
        raise ValueError("topk_length must be [batch]")
    _require(workspace, "workspace", (torch.uint8,))
    _require(out, "out", bf)
    _require(lse, "lse", (torch.float32,))
    if q.dim() != 3 or kv_pool.dim() != 2 or indices.dim() != 2:
        raise ValueError("q must be [B, Hq, Dqk], kv_pool [T, width], indices [B, topk]")
    width = 656 if fp8 else q.shape[2]
    if kv_pool.shape[1] != width or indices.shape[0] != q.shape[0]:
        raise ValueError(f"kv_pool rows must have {width} elements and indices one row per query")
    if tuple(out.shape) != (q.shape[0], q.shape[1], d_v) or tuple(lse.shape) != tuple(q.shape[:2]):
        raise ValueError("out must be [B, Hq, d_v] and lse [B, Hq]")
    if noalloc:
        return (lib().pkv_gather_mla_noalloc,
                (_ptr(q), _ptr(kv_pool), kv_pool.shape[0], _ptr(indices), indices.shape[1],
                 q.shape[0], q.shape[1], q.shape[2], d_v, float(sm_scale), _ptr(attn_sink),
                 _ptr(topk_length), _ptr(out), _ptr(lse), _stream(stream)),
                "pkv_gather_mla_noalloc")
    ws_bytes = 0 if workspace is None else workspace.numel()
    fn = lib().pkv_gather_mla_fp8 if fp8 else lib().pkv_gather_mla
    return (fn, (_ptr(q), _ptr(kv_pool), kv_pool.shape[0], _ptr(indices), indices.shape[1],
                 q.shape[0], q.shape[1], q.shape[2], d_v, float(sm_scale), _ptr(attn_sink),
                 _ptr(topk_length), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse),
                 _stream(stream)),
            "pkv_gather_mla_fp8" if fp8 else "pkv_gather_mla")


# ------------------------------------------------------------ conveniences

def pkv_plan_workspace_size(plan: Plan) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().pkv_plan_workspace_size(plan.handle, ctypes.byref(out)), "pkv_plan_workspace_size")
    return int(out.value)


def pkv_plan_set_engine(plan: Plan, engine) -> None:
    """Pick the decode contraction engine for this plan's runs: ``"mfma"``
    (the default) or ``"dot2"``, or the integer PKV_ENGINE_* code."""
    code = ENGINES[engine] if isinstance(engine, str) else int(engine)
    _check(lib().pkv_plan_set_engine(plan.handle, code), "pkv_plan_set_engine")


def pkv_plan_set_timing_events(plan: Plan, start_event=None, stop_event=None) -> None:
    """Let the plan's decode launches record their own start/stop time into two
    torch.cuda.Event objects (already recorded once, so that they exist), or
    stop doing so with no events."""
    handles = []
    for ev in (start_event, stop_event):
        if ev is not None and not ev.cuda_event:
            raise ValueError("record the event once before binding it (torch creates it lazily)")
        handles.append(None if ev is None else ev.cuda_event)
    _check(lib().pkv_plan_set_timing_events(plan.handle, *handles), "pkv_plan_set_timing_events")


def pkv_plan_upload(plan: Plan, workspace, stream=None) -> None:
    _require(workspace, "workspace", (__import__("torch").uint8,))
    _check(lib().pkv_plan_upload(plan.handle, _ptr(workspace), workspace.numel(), _stream(stream)),
           "pkv_plan_upload")


def decode(q, k_pool, v_pool, kv_indptr, kv_indices, sm_scale: Optional[float] = None,
           kv_indptr_host=None, allow_split=True, chunk_tokens=0, num_cus=0, stream=None,
           engine="mfma"):
    """Plan, run and merge one paged GQA decode; returns ``(out, lse)`` (bf16, fp32 base 2).

    ``sm_scale`` defaults to 1/sqrt(head_dim). ``kv_indptr_host`` (a host copy
    of ``kv_indptr``) avoids a device-to-host copy when given. ``engine``
    picks the contraction units (``"mfma"`` or ``"dot2"``).
    """
    import torch
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    if kv_indptr_host is None:
        kv_indptr_host = kv_indptr.cpu()
    plan = pkv_plan_create(kv_indptr_host, q.shape[1], k_pool.shape[2], q.shape[2],
                           k_pool.shape[1], num_cus, allow_split, chunk_tokens)
    pkv_plan_set_engine(plan, engine)
    ws = torch.empty(max(pkv_plan_workspace_size(plan), 16), dtype=torch.uint8, device=q.device)
    pkv_plan_upload(plan, ws, stream)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    pkv_run(plan, q, k_pool, v_pool, kv_indptr, kv_indices, sm_scale, ws, out, lse, stream)
    pkv_merge(plan, ws, out, lse, stream)
    return out, lse


def decode_block_table(q, k_pool, v_pool, block_table, seq_lens_host,
                       sm_scale: Optional[float] = None, allow_split=True, chunk_tokens=0,
                       num_cus=0, stream=None, engine="mfma"):
    """Plan, run and merge one paged GQA decode through a block table.

    ``k_pool``/``v_pool`` are ``[pages, page_size, Hkv, D]``; ``block_table``
    is a device ``int32 [B, max_pages]``; ``seq_lens_host`` the host lengths.
    Returns ``(out, lse)`` (bf16, fp32 base 2).
    """
    import torch
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    plan = pkv_block_table_plan_create(seq_lens_host, q.shape[1], k_pool.shape[2], q.shape[2],
                                       k_pool.shape[1], num_cus, allow_split, chunk_tokens)
    pkv_plan_set_engine(plan, engine)
    ws = torch.empty(max(pkv_plan_workspace_size(plan), 16), dtype=torch.uint8, device=q.device)
    pkv_plan_upload(plan, ws, stream)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    pkv_block_table_run(plan, q, k_pool, v_pool, block_table, sm_scale, ws, out, lse, stream)
    pkv_merge(plan, ws, out, lse, stream)
    return out, lse


def gather_mla_fp8(q, kv_pool, indices, sm_scale: Optional[float] = None, d_v: int = 512,
                   stream=None, attn_sink=None, topk_length=None):
    """Index-gather latent decode over a uint8 FP8 pool ``[T, 656]``."""
    return gather_mla(q, kv_pool, indices, sm_scale, d_v, stream, attn_sink, topk_length,
                      _fp8=True)


def gather_mla(q, kv_pool, indices, sm_scale: Optional[float] = None, d_v: int = 512,
               stream=None, attn_sink=None, topk_length=None, _fp8=False):
    """Index-gather latent decode; returns ``(out [B, Hq, d_v], lse [B, Hq])``.

    ``attn_sink`` (fp32 [Hq]) and ``topk_length`` (int32 [B]) are optional
    device tensors."""
    import torch
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(q.shape[-1])
    ws_bytes = pkv_gather_mla_workspace_size(q.shape[0], q.shape[1], q.shape[2], d_v,
                                             indices.shape[1])
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    out = torch.empty((q.shape[0], q.shape[1], d_v), dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    _gather(_fp8, q, kv_pool, indices, sm_scale, ws, out, lse, d_v, stream, attn_sink,
            topk_length)
    return out, lse
