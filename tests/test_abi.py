"""The C ABI on the host: every declared symbol is exported, every argument
check returns its status before any HIP call, and the exported plan equals the
independent Python statement of the partition rule integer for integer.

No test here launches a kernel; the fake device pointers passed below are never
dereferenced because each call is rejected by a host-side check first.
"""

import ctypes
import pathlib
import re

import numpy as np
import pytest

import paged_kv_attention_gqa_amd as pkv
from inputs import lognormal_lengths
from inputs.configs import EDGE_LENGTHS
from oracle import plan_ref

HEADER = pathlib.Path(__file__).resolve().parents[1] / "include" / "pkv.h"
FAKE = 0x10000   # 16-byte aligned, never dereferenced


@pytest.fixture(scope="module")
def lib():
    try:
        return pkv.lib()
    except RuntimeError as e:
        pytest.fail(str(e))


def declared_symbols():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_symbols()
    assert len(names) == 20
    for name in names:
        assert hasattr(lib, name), name
        assert name in pkv.SIGNATURES, name


def test_status_strings(lib):
    for code in range(6):
        assert pkv.pkv_status_string(code)
    assert pkv.pkv_status_string(99) == "unknown status"


def test_set_engine_rejects_unknown_codes(lib):
    """pkv_plan_set_engine takes PKV_ENGINE_MFMA (0) and PKV_ENGINE_DOT2 (1);
    anything else, or a NULL plan, is PKV_ERR_INVALID_ARG (host only)."""
    ind = np.array([0, 5, 9], dtype=np.int32)
    plan = pkv.pkv_plan_create(ind, num_cus=8)
    for code in (pkv.PKV_ENGINE_MFMA, pkv.PKV_ENGINE_DOT2):
        assert lib.pkv_plan_set_engine(plan.handle, code) == pkv.PKV_OK
    for code in (-1, 2, 99):
        assert lib.pkv_plan_set_engine(plan.handle, code) == pkv.PKV_ERR_INVALID_ARG
        assert "engine" in pkv.pkv_last_error()
    assert lib.pkv_plan_set_engine(None, 0) == pkv.PKV_ERR_INVALID_ARG
    pkv.pkv_plan_set_engine(plan, "dot2")
    pkv.pkv_plan_set_engine(plan, "mfma")
    with pytest.raises(KeyError):
        pkv.pkv_plan_set_engine(plan, "fma")


def test_set_timing_events_arguments(lib):
    """Both events or neither; a NULL plan is rejected (host only)."""
    ind = np.array([0, 5, 9], dtype=np.int32)
    plan = pkv.pkv_plan_create(ind, num_cus=8)
    fake = ctypes.c_void_p(0x1000)
    assert lib.pkv_plan_set_timing_events(plan.handle, fake, None) == pkv.PKV_ERR_INVALID_ARG
    assert lib.pkv_plan_set_timing_events(plan.handle, None, fake) == pkv.PKV_ERR_INVALID_ARG
    assert "both" in pkv.pkv_last_error()
    assert lib.pkv_plan_set_timing_events(None, None, None) == pkv.PKV_ERR_INVALID_ARG
    assert lib.pkv_plan_set_timing_events(plan.handle, None, None) == pkv.PKV_OK


def _indptr(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def _ws(ind, **kw):
    out = ctypes.c_size_t(0)
    args = dict(hq=32, hkv=4, d=128, ps=1, cus=256, split=1, chunk=0)
    args.update(kw)
    st = pkv.lib().pkv_workspace_size(ind.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                      len(ind) - 1, args["hq"], args["hkv"], args["d"],
                                      args["ps"], args["cus"], args["split"], args["chunk"],
                                      ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw,status", [
    (dict(hq=16), pkv.PKV_ERR_UNSUPPORTED),
    (dict(hkv=8), pkv.PKV_ERR_UNSUPPORTED),
    (dict(d=64), pkv.PKV_ERR_UNSUPPORTED),
    (dict(ps=16), pkv.PKV_ERR_UNSUPPORTED),
    (dict(hq=30), pkv.PKV_ERR_INVALID_ARG),       # not a multiple of Hkv
    (dict(hq=0), pkv.PKV_ERR_INVALID_ARG),
    (dict(chunk=-1), pkv.PKV_ERR_INVALID_ARG),
    (dict(cus=-3), pkv.PKV_ERR_INVALID_ARG),
])
def test_shape_checks(lib, kw, status):
    st, _ = _ws(_indptr([3, 4]), **kw)
    assert st == status
    assert pkv.pkv_last_error()


def test_indptr_checks(lib):
    assert _ws(np.array([1, 5], np.int32))[0] == pkv.PKV_ERR_INVALID_ARG
    assert _ws(np.array([0, 5, 4], np.int32))[0] == pkv.PKV_ERR_INVALID_ARG
    out = ctypes.c_size_t(0)
    assert lib.pkv_workspace_size(None, 2, 32, 4, 128, 1, 256, 1, 0, ctypes.byref(out)) == \
        pkv.PKV_ERR_INVALID_ARG
    st, n = _ws(_indptr([]))
    assert st == pkv.PKV_OK


def test_workspace_size_formula(lib):
    ind = _indptr([1000, 10, 0, 5000])
    st, n = _ws(ind, chunk=256)
    assert st == pkv.PKV_OK
    per_worker, merges, slots = plan_ref.make_plan(ind, 256, True, 256)
    al = lambda x: -(-x // 256) * 256
    segs = sum(len(s) for s in per_worker)
    tables = 32 * len(per_worker) + 32 * segs + 16 * len(merges)
    part_o = al(tables)
    part_lse = al(part_o + slots * 32 * 128 * 4)
    assert n == al(part_lse + slots * 32 * 4)


@pytest.mark.parametrize("lengths", [[1000, 10, 0, 5000], [], [0, 0], [17, 64], [4096] * 70])
def test_plan_workspace_size_matches(lib, lengths):
    """A host-only plan reports the workspace size pkv_workspace_size gives for
    its batch, and rejects uploads into a workspace that is too small, NULL or
    misaligned before any HIP call."""
    ind = _indptr(lengths)
    st, n = _ws(ind)
    assert st == pkv.PKV_OK
    plan = pkv.pkv_plan_create(ind, num_cus=256)
    assert pkv.pkv_plan_workspace_size(plan) == n
    up = pkv.lib().pkv_plan_upload
    if n:
        assert up(plan.handle, FAKE, n - 16, 0) == pkv.PKV_ERR_WORKSPACE_TOO_SMALL
        assert up(plan.handle, FAKE + 4, n, 0) == pkv.PKV_ERR_INVALID_ARG
    assert up(plan.handle, None, n, 0) == pkv.PKV_ERR_INVALID_ARG
    assert up(None, FAKE, n, 0) == pkv.PKV_ERR_INVALID_ARG
    out = ctypes.c_size_t(0)
    assert pkv.lib().pkv_plan_workspace_size(None, ctypes.byref(out)) == pkv.PKV_ERR_INVALID_ARG


def test_noalloc_gather_rejects_a_batch_beyond_the_scratch(lib):
    """100 rows x 128 heads cut into 2 pieces need 52.5 MB of partials, more
    than the library's 48 MiB device scratch: refused before any HIP call."""
    need = pkv.pkv_gather_mla_workspace_size(100, 128, 576, 512, 2048)
    assert need > 48 << 20
    st = lib.pkv_gather_mla_noalloc(FAKE, FAKE, 1, FAKE, 2048, 100, 128, 576, 512, 0.04, None,
                                    None, FAKE, FAKE, None)
    assert st == pkv.PKV_ERR_UNSUPPORTED and "scratch" in pkv.pkv_last_error()
    assert lib.pkv_gather_mla_noalloc(FAKE, FAKE, 1, FAKE, 2048, 2, 128, 576, 500, 0.04, None,
                                      None, FAKE, FAKE, None) == pkv.PKV_ERR_UNSUPPORTED


def test_sm_scale_any_finite_value(lib):
    """Zero and negative scales pass the argument checks (the attention is
    defined for every real scale); the call then stops at the host-only plan."""
    ind = _indptr([17, 64])
    h = pkv.pkv_plan_create(ind, num_cus=256).handle
    for scale in (0.0, -0.5, -1e30, 1e30):
        assert _run_raw(h, scale=scale) == pkv.PKV_ERR_PLAN_MISMATCH


def _host_plan(ind, cus, split, chunk):
    plan = pkv.pkv_plan_create(ind, num_cus=cus, allow_split=split, chunk_tokens=chunk)
    return pkv.pkv_plan_export(plan)


PLAN_CASES = [
    ("tiny", _indptr([17, 64])),
    ("edge", _indptr(list(EDGE_LENGTHS))),
    ("gqa", _indptr(np.random.default_rng(2).integers(512, 4096, size=64, endpoint=True))),
    ("throughput", _indptr(lognormal_lengths(np.random.default_rng(4), 256))),
    ("empty_batch", _indptr([])),
    ("all_empty", _indptr([0, 0, 0])),
]


@pytest.mark.parametrize("name,ind", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
@pytest.mark.parametrize("cus,split,chunk", [(256, True, 0), (256, False, 0), (80, True, 0),
                                             (256, True, 64), (1, True, 0), (304, True, 1000),
                                             (256, True, 7)])
def test_plan_export_matches_rule(lib, name, ind, cus, split, chunk):
    assert _host_plan(ind, cus, split, chunk) == plan_ref.export(ind, cus, split, chunk)


@pytest.mark.parametrize("seed", range(25))
def test_plan_export_random(lib, seed):
    rng = np.random.default_rng(1000 + seed)
    batch = int(rng.integers(0, 400))
    lengths = rng.integers(0, 40000, size=batch) * (rng.random(batch) < 0.8)
    ind = _indptr(lengths)
    cus = int(rng.choice([1, 7, 256, 304]))
    chunk = int(rng.choice([0, 0, 0, 33, 512]))
    split = bool(rng.random() < 0.9)
    assert _host_plan(ind, cus, split, chunk) == plan_ref.export(ind, cus, split, chunk)


def _run_raw(plan_handle, **over):
    a = dict(q=FAKE, qb=2, qh=32, qd=128, k=FAKE, v=FAKE, pages=128, ps=1, hkv=4, pd=128,
             indptr=FAKE, indptr_len=3, indices=FAKE, nidx=81, scale=0.088, ws=FAKE,
             ws_bytes=1 << 20, out=FAKE, lse=FAKE, stream=0)
    a.update(over)
    return pkv.lib().pkv_run(plan_handle, a["q"], a["qb"], a["qh"], a["qd"], a["k"], a["v"],
                             a["pages"], a["ps"], a["hkv"], a["pd"], a["indptr"],
                             a["indptr_len"], a["indices"], a["nidx"], a["scale"], a["ws"],
                             a["ws_bytes"], a["out"], a["lse"], a["stream"])


def test_run_checks_before_any_hip_call(lib):
    ind = _indptr([17, 64])
    host_plan = pkv.pkv_plan_create(ind, num_cus=256)
    h = host_plan.handle
    E = pkv
    assert _run_raw(None) == E.PKV_ERR_INVALID_ARG
    assert _run_raw(h, qh=16) == E.PKV_ERR_UNSUPPORTED
    assert _run_raw(h, qd=64, pd=64) == E.PKV_ERR_UNSUPPORTED
    assert _run_raw(h, ps=2) == E.PKV_ERR_UNSUPPORTED
    assert _run_raw(h, pd=64) == E.PKV_ERR_INVALID_ARG
    assert _run_raw(h, qb=3) == E.PKV_ERR_PLAN_MISMATCH
    assert _run_raw(h, indptr_len=4) == E.PKV_ERR_INVALID_ARG
    assert _run_raw(h, nidx=80) == E.PKV_ERR_INVALID_ARG
    assert _run_raw(h, scale=float("nan")) == E.PKV_ERR_INVALID_ARG
    assert _run_raw(h, scale=float("inf")) == E.PKV_ERR_INVALID_ARG
    assert _run_raw(h, q=0) == E.PKV_ERR_INVALID_ARG
    assert _run_raw(h, k=0) == E.PKV_ERR_INVALID_ARG
    assert _run_raw(h, q=FAKE + 2) == E.PKV_ERR_INVALID_ARG      # misaligned
    assert _run_raw(h, pages=0) == E.PKV_ERR_INVALID_ARG
    # a host-only plan can be exported but never run
    assert _run_raw(h) == E.PKV_ERR_PLAN_MISMATCH
    assert pkv.lib().pkv_merge(None, FAKE, 1, FAKE, FAKE, 0) == E.PKV_ERR_INVALID_ARG


def test_plan_create_checks(lib):
    ind = _indptr([17, 64])
    handle = ctypes.c_void_p(0)
    I32P = ctypes.POINTER(ctypes.c_int32)
    st = lib.pkv_plan_create(ind.ctypes.data_as(I32P), 2, 32, 4, 128, 1, 256, 1, 0, FAKE, 16, 0,
                             ctypes.byref(handle))
    assert st == pkv.PKV_ERR_WORKSPACE_TOO_SMALL and not handle.value
    assert lib.pkv_plan_create(ind.ctypes.data_as(I32P), 2, 32, 4, 128, 1, 256, 1, 0, None, 0, 0,
                               None) == pkv.PKV_ERR_INVALID_ARG
    assert lib.pkv_plan_create(ind.ctypes.data_as(I32P), 2, 32, 4, 64, 1, 256, 1, 0, None, 0, 0,
                               ctypes.byref(handle)) == pkv.PKV_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        pkv.pkv_plan_create(ind, head_dim=64, num_cus=256)


def test_plan_export_small_buffer(lib):
    plan = pkv.pkv_plan_create(_indptr([17, 64]), num_cus=256)
    need = ctypes.c_size_t(0)
    assert lib.pkv_plan_export(plan.handle, None, 0, ctypes.byref(need)) == pkv.PKV_OK
    buf = (ctypes.c_int32 * (need.value - 1))()
    assert lib.pkv_plan_export(plan.handle, buf, need.value - 1, None) == pkv.PKV_ERR_INVALID_ARG


def test_gather_checks(lib):
    out = ctypes.c_size_t(0)
    assert lib.pkv_gather_mla_workspace_size(32, 128, 576, 512, 2048, ctypes.byref(out)) == pkv.PKV_OK
    assert lib.pkv_gather_mla_workspace_size(32, 128, 512, 512, 2048, ctypes.byref(out)) == \
        pkv.PKV_ERR_UNSUPPORTED
    assert lib.pkv_gather_mla_workspace_size(32, 100, 576, 512, 2048, ctypes.byref(out)) == \
        pkv.PKV_ERR_UNSUPPORTED
    assert lib.pkv_gather_mla_workspace_size(-1, 128, 576, 512, 2048, ctypes.byref(out)) == \
        pkv.PKV_ERR_INVALID_ARG
    g = lambda **o: lib.pkv_gather_mla(
        o.get("q", FAKE), o.get("kv", FAKE), o.get("T", 65536), o.get("idx", FAKE),
        o.get("topk", 2048), o.get("B", 32), o.get("H", 128), o.get("dqk", 576), o.get("dv", 512),
        o.get("scale", 0.04), o.get("sink", None), o.get("tlen", None), o.get("ws", FAKE),
        o.get("wsb", 1 << 30), o.get("out", FAKE), o.get("lse", FAKE), 0)
    assert g(dqk=512) == pkv.PKV_ERR_UNSUPPORTED
    assert g(scale=float("nan")) == pkv.PKV_ERR_INVALID_ARG
    assert g(q=0) == pkv.PKV_ERR_INVALID_ARG
    assert g(T=-1) == pkv.PKV_ERR_INVALID_ARG
    assert g(out=FAKE + 4) == pkv.PKV_ERR_INVALID_ARG
    assert g(sink=FAKE + 2) == pkv.PKV_ERR_INVALID_ARG
    assert g(tlen=FAKE + 1) == pkv.PKV_ERR_INVALID_ARG


# ------------------------------------------------------------ block tables

def _bt_ws(lens, **kw):
    lens = np.asarray(lens, dtype=np.int32)
    out = ctypes.c_size_t(0)
    args = dict(hq=32, hkv=4, d=128, ps=16, cus=256, split=1, chunk=0)
    args.update(kw)
    st = pkv.lib().pkv_block_table_workspace_size(
        lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), len(lens), args["hq"], args["hkv"],
        args["d"], args["ps"], args["cus"], args["split"], args["chunk"], ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw,status", [
    (dict(ps=1), pkv.PKV_OK),
    (dict(ps=16), pkv.PKV_OK),
    (dict(ps=1024), pkv.PKV_OK),
    (dict(ps=3), pkv.PKV_ERR_UNSUPPORTED),
    (dict(ps=48), pkv.PKV_ERR_UNSUPPORTED),
    (dict(ps=2048), pkv.PKV_ERR_UNSUPPORTED),
    (dict(ps=0), pkv.PKV_ERR_INVALID_ARG),
    (dict(hq=16), pkv.PKV_ERR_UNSUPPORTED),
    (dict(chunk=-1), pkv.PKV_ERR_INVALID_ARG),
])
def test_block_table_shape_checks(lib, kw, status):
    assert _bt_ws([5, 40], **kw)[0] == status


def test_block_table_length_checks(lib):
    assert _bt_ws([5, -1])[0] == pkv.PKV_ERR_INVALID_ARG
    assert _bt_ws([2 ** 30, 2 ** 30])[0] == pkv.PKV_ERR_INVALID_ARG     # 2^31 tokens
    assert _bt_ws([2 ** 30, 2 ** 30 - 1])[0] == pkv.PKV_OK
    assert _bt_ws([])[0] == pkv.PKV_OK
    out = ctypes.c_size_t(0)
    assert lib.pkv_block_table_workspace_size(None, 2, 32, 4, 128, 16, 256, 1, 0,
                                              ctypes.byref(out)) == pkv.PKV_ERR_INVALID_ARG


BT_CASES = [
    ("edge", list(EDGE_LENGTHS)),
    ("gqa", list(np.random.default_rng(6).integers(512, 4096, size=64, endpoint=True))),
    ("throughput", list(lognormal_lengths(np.random.default_rng(4), 256))),
    ("all_empty", [0, 0]),
]


@pytest.mark.parametrize("name,lens", BT_CASES, ids=[c[0] for c in BT_CASES])
@pytest.mark.parametrize("ps,cus,split,chunk", [(16, 256, True, 0), (64, 256, True, 0),
                                                (16, 256, False, 0), (128, 80, True, 96)])
def test_block_table_plan_matches_rule(lib, name, lens, ps, cus, split, chunk):
    plan = pkv.pkv_block_table_plan_create(lens, page_size=ps, num_cus=cus, allow_split=split,
                                           chunk_tokens=chunk)
    assert pkv.pkv_plan_export(plan) == plan_ref.export(_indptr(lens), cus, split, chunk)
    size = pkv.pkv_block_table_workspace_size(lens, page_size=ps, num_cus=cus,
                                              allow_split=split, chunk_tokens=chunk)
    assert size == pkv.pkv_workspace_size(_indptr(lens), num_cus=cus, allow_split=split,
                                          chunk_tokens=chunk)


def _bt_run_raw(plan_handle, **over):
    a = dict(q=FAKE, qb=2, qh=32, qd=128, k=FAKE, v=FAKE, pages=64, ps=16, hkv=4, pd=128,
             table=FAKE, rows=2, cols=3, scale=0.088, ws=FAKE, ws_bytes=1 << 20, out=FAKE,
             lse=FAKE, stream=0)
    a.update(over)
    return pkv.lib().pkv_block_table_run(plan_handle, a["q"], a["qb"], a["qh"], a["qd"], a["k"],
                                         a["v"], a["pages"], a["ps"], a["hkv"], a["pd"],
                                         a["table"], a["rows"], a["cols"], a["scale"], a["ws"],
                                         a["ws_bytes"], a["out"], a["lse"], a["stream"])


def test_block_table_run_checks_before_any_hip_call(lib):
    E = pkv
    plan = pkv.pkv_block_table_plan_create([17, 40], page_size=16, num_cus=256)   # needs 2, 3 pages
    h = plan.handle
    assert _bt_run_raw(None) == E.PKV_ERR_INVALID_ARG
    assert _bt_run_raw(h, ps=32) == E.PKV_ERR_PLAN_MISMATCH
    assert _bt_run_raw(h, ps=12) == E.PKV_ERR_UNSUPPORTED
    assert _bt_run_raw(h, rows=3) == E.PKV_ERR_INVALID_ARG
    assert _bt_run_raw(h, cols=2) == E.PKV_ERR_INVALID_ARG
    assert _bt_run_raw(h, table=0) == E.PKV_ERR_INVALID_ARG
    assert _bt_run_raw(h, pages=2 ** 27) == E.PKV_ERR_UNSUPPORTED    # 2^31 token rows
    assert _bt_run_raw(h, pages=0) == E.PKV_ERR_INVALID_ARG
    assert _bt_run_raw(h, scale=float("nan")) == E.PKV_ERR_INVALID_ARG
    assert _bt_run_raw(h, v=FAKE + 8) == E.PKV_ERR_INVALID_ARG
    assert _bt_run_raw(h) == E.PKV_ERR_PLAN_MISMATCH                 # host-only plan
    # each kind of plan is refused by the other run call
    assert _run_raw(h, ps=16) == E.PKV_ERR_PLAN_MISMATCH
    csr = pkv.pkv_plan_create(_indptr([17, 40]), num_cus=256)
    assert _bt_run_raw(csr.handle, ps=1) == E.PKV_ERR_PLAN_MISMATCH


def test_append_checks(lib):
    a = lambda **o: lib.pkv_append_kv(
        o.get("k", FAKE), o.get("v", FAKE), o.get("pages", 10), o.get("ps", 16), o.get("hkv", 4),
        o.get("d", 128), o.get("kr", FAKE), o.get("vr", FAKE), o.get("slots", FAKE),
        o.get("n", 5), 0)
    E = pkv
    assert a(n=0) == E.PKV_OK                       # nothing to store: no launch
    assert a(n=0, kr=0, vr=0, slots=0) == E.PKV_OK
    assert a(n=-1) == E.PKV_ERR_INVALID_ARG
    assert a(n=2 ** 25 + 1) == E.PKV_ERR_INVALID_ARG
    assert a(ps=0) == E.PKV_ERR_INVALID_ARG
    assert a(pages=-1) == E.PKV_ERR_INVALID_ARG
    assert a(hkv=1, d=4) == E.PKV_ERR_UNSUPPORTED   # 8-byte rows
    assert a(kr=0) == E.PKV_ERR_INVALID_ARG
    assert a(slots=0) == E.PKV_ERR_INVALID_ARG
    assert a(k=0) == E.PKV_ERR_INVALID_ARG
    assert a(vr=FAKE + 8) == E.PKV_ERR_INVALID_ARG
    assert a(slots=FAKE + 4) == E.PKV_ERR_INVALID_ARG
    assert a(pages=2 ** 62) == E.PKV_ERR_INVALID_ARG


def test_gather_fp8_checks(lib):
    g = lambda **o: lib.pkv_gather_mla_fp8(
        o.get("q", FAKE), o.get("kv", FAKE), o.get("T", 65536), o.get("idx", FAKE),
        o.get("topk", 2048), o.get("B", 32), o.get("H", 128), o.get("dqk", 576), o.get("dv", 512),
        o.get("scale", 0.04), None, None, o.get("ws", FAKE), o.get("wsb", 1 << 30),
        o.get("out", FAKE), o.get("lse", FAKE), 0)
    assert g(dqk=512) == pkv.PKV_ERR_UNSUPPORTED
    assert g(H=100) == pkv.PKV_ERR_UNSUPPORTED
    assert g(kv=FAKE + 8) == pkv.PKV_ERR_INVALID_ARG
    assert g(kv=0) == pkv.PKV_ERR_INVALID_ARG
    assert g(wsb=0) == pkv.PKV_ERR_WORKSPACE_TOO_SMALL
    assert g(B=0) == pkv.PKV_OK
