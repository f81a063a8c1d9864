"""The C-ABI library loads, exports every symbol the headers under include/ declare,
and rejects bad arguments with the documented status before any device work.

No GPU is needed: every call here fails host-side validation (or only sizes the
workspace), so nothing is enqueued.
"""
import ctypes
import glob
import os
import re

import pytest

import mla_latent_decode_absorbed_amd as mla

pytestmark = pytest.mark.cpu

HEADERS = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                        "include", "*.h")))


def declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:int|const char\*)\s+(mla_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(mla.EXPORTS)


@pytest.mark.parametrize("name", sorted(mla.EXPORTS))
def test_library_exports_symbol(name):
    lib = ctypes.CDLL(mla.LIB_PATH)
    assert hasattr(lib, name)


def test_status_strings():
    for st in (mla.OK, mla.ERR_INVALID_ARG, mla.ERR_UNSUPPORTED, mla.ERR_WORKSPACE, mla.ERR_HIP):
        assert mla.status_string(st) and "unknown" not in mla.status_string(st)
    assert "unknown" in mla.status_string(12345)


def good_desc(**kw):
    d = dict(batch=2, q_len=1, num_heads=16, num_pages=6, max_pages_per_seq=2)
    d.update(kw)
    return mla.make_desc(**d)


def test_workspace_size_is_positive_and_descriptor_only():
    a = mla.workspace_size(good_desc())
    b = mla.workspace_size(good_desc(num_pages=6000))      # pool size does not matter
    assert a > 0 and a == b
    assert mla.workspace_size(good_desc(num_splits=4)) > 0
    big = mla.workspace_size(good_desc(batch=64, num_heads=128, max_pages_per_seq=64))
    assert big > a


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, mla.ERR_INVALID_ARG),
    ("q_len", 0, mla.ERR_INVALID_ARG),
    ("num_heads", -1, mla.ERR_INVALID_ARG),
    ("num_pages", 0, mla.ERR_INVALID_ARG),
    ("max_pages_per_seq", 0, mla.ERR_INVALID_ARG),
    ("kv_dtype", 7, mla.ERR_INVALID_ARG),
    ("out_dtype", mla.FP8_E4M3, mla.ERR_INVALID_ARG),
    ("causal", 2, mla.ERR_INVALID_ARG),
    ("num_splits", -1, mla.ERR_INVALID_ARG),
    ("page_size", 32, mla.ERR_UNSUPPORTED),
    ("q_len", 17, mla.ERR_UNSUPPORTED),
])
def test_bad_descriptor_rejected(field, value, status):
    d = good_desc()
    setattr(d, field, value)
    n = ctypes.c_size_t(0)
    assert mla.lib.mla_decode_workspace_size(ctypes.byref(d), ctypes.byref(n)) == status
    rc = mla.lib.mla_decode_partial(ctypes.byref(d), 4096, 4096, None, 4096, 4096, ctypes.c_float(0.1),
                                    4096, 4096, 4096, ctypes.c_size_t(1 << 30), None)
    assert rc == status


def _call(desc, q=4096, kv=4096, kv_scale=None, bt=4096, sl=4096, scale=0.1, out=4096, lse=4096,
          ws=4096, ws_bytes=1 << 34):
    return mla.lib.mla_decode_partial(ctypes.byref(desc), q, kv, kv_scale, bt, sl, ctypes.c_float(scale),
                                      out, lse, ws, ctypes.c_size_t(ws_bytes), None)


def test_null_and_misaligned_pointers_rejected():
    d = good_desc()
    assert _call(d, q=None) == mla.ERR_INVALID_ARG
    assert _call(d, kv=None) == mla.ERR_INVALID_ARG
    assert _call(d, bt=None) == mla.ERR_INVALID_ARG
    assert _call(d, sl=None) == mla.ERR_INVALID_ARG
    assert _call(d, out=None) == mla.ERR_INVALID_ARG
    assert _call(d, lse=None) == mla.ERR_INVALID_ARG
    assert _call(d, q=4096 + 8) == mla.ERR_INVALID_ARG
    assert _call(d, kv=4096 + 4) == mla.ERR_INVALID_ARG
    assert _call(d, out=4096 + 4) == mla.ERR_INVALID_ARG
    assert _call(d, bt=4096 + 2) == mla.ERR_INVALID_ARG
    assert _call(d, scale=float("nan")) == mla.ERR_INVALID_ARG
    assert _call(d, scale=0.0) == mla.ERR_INVALID_ARG
    assert _call(d, scale=-0.1) == mla.ERR_INVALID_ARG
    assert _call(d, kv_scale=4096) == mla.ERR_INVALID_ARG          # bf16 takes no kv_scale


def test_workspace_checks():
    d = good_desc()
    need = mla.workspace_size(d)
    assert _call(d, ws=None) == mla.ERR_WORKSPACE
    assert _call(d, ws=4096 + 128) == mla.ERR_WORKSPACE              # not 256-byte aligned
    assert _call(d, ws_bytes=need - 1) == mla.ERR_WORKSPACE


def test_plan_argument_checks():
    """mla_decode_plan: the descriptor, seq_lens and workspace rules of mla_decode_partial."""
    d = good_desc()
    need = mla.workspace_size(d)

    def plan(desc, sl=4096, ws=4096, ws_bytes=1 << 34):
        return mla.lib.mla_decode_plan(ctypes.byref(desc), sl, ws, ctypes.c_size_t(ws_bytes), None)

    bad = good_desc()
    bad.batch = 0
    assert plan(bad) == mla.ERR_INVALID_ARG
    assert plan(d, sl=None) == mla.ERR_INVALID_ARG
    assert plan(d, sl=4096 + 2) == mla.ERR_INVALID_ARG
    assert plan(d, ws=None) == mla.ERR_WORKSPACE
    assert plan(d, ws=4096 + 128) == mla.ERR_WORKSPACE
    assert plan(d, ws_bytes=need - 1) == mla.ERR_WORKSPACE


def test_planned_decode_argument_checks():
    """mla_decode_partial_planned validates exactly like mla_decode_partial."""
    d = good_desc()
    need = mla.workspace_size(d)

    def call(**kw):
        a = dict(q=4096, kv=4096, kv_scale=None, bt=4096, sl=4096, scale=0.1, out=4096, lse=4096, ws=4096,
                 ws_bytes=1 << 34)
        a.update(kw)
        return mla.lib.mla_decode_partial_planned(ctypes.byref(d), a["q"], a["kv"], a["kv_scale"], a["bt"],
                                                  a["sl"], ctypes.c_float(a["scale"]), a["out"], a["lse"],
                                                  a["ws"], ctypes.c_size_t(a["ws_bytes"]), None)

    assert call(q=None) == mla.ERR_INVALID_ARG
    assert call(sl=None) == mla.ERR_INVALID_ARG
    assert call(out=4096 + 4) == mla.ERR_INVALID_ARG
    assert call(scale=0.0) == mla.ERR_INVALID_ARG
    assert call(kv_scale=4096) == mla.ERR_INVALID_ARG
    assert call(ws=None) == mla.ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == mla.ERR_WORKSPACE


def test_fp8_requires_kv_scale():
    d = good_desc(kv_dtype=mla.FP8_E4M3)
    n = ctypes.c_size_t(0)
    st = mla.lib.mla_decode_workspace_size(ctypes.byref(d), ctypes.byref(n))
    if st == mla.ERR_UNSUPPORTED:
        pytest.skip("fp8 path not built into this library")
    assert _call(d, kv_scale=None) == mla.ERR_INVALID_ARG


def test_merge_argument_checks():
    f = mla.lib.mla_merge_states
    assert f(4096, 4096, 0, 10, 4096, 4096, mla.F32, None) == mla.ERR_INVALID_ARG
    assert f(4096, 4096, 4097, 10, 4096, 4096, mla.F32, None) == mla.ERR_INVALID_ARG
    assert f(4096, 4096, 2, -1, 4096, 4096, mla.F32, None) == mla.ERR_INVALID_ARG
    assert f(4096, 4096, 2, 10, 4096, 4096, mla.FP8_E4M3, None) == mla.ERR_INVALID_ARG
    assert f(None, 4096, 2, 10, 4096, 4096, mla.F32, None) == mla.ERR_INVALID_ARG
    assert f(4096 + 4, 4096, 2, 10, 4096, 4096, mla.F32, None) == mla.ERR_INVALID_ARG
    assert f(4096, 4096, 2, 0, None, None, mla.F32, None) == mla.OK          # nothing to do


def _tensors(desc, kv_dtype_bytes=2, pages=None):
    import torch
    rows = desc.batch * desc.q_len * desc.num_heads
    dt = torch.bfloat16 if kv_dtype_bytes == 2 else torch.uint8
    return dict(
        q=torch.zeros((rows, mla.QK_DIM), dtype=dt),
        kv_cache=torch.zeros(((pages or desc.num_pages) * desc.page_size, mla.QK_DIM), dtype=dt),
        block_table=torch.zeros((desc.batch, desc.max_pages_per_seq), dtype=torch.int32),
        seq_lens=torch.zeros((desc.batch,), dtype=torch.int32),
        out=torch.zeros((rows, mla.LATENT_DIM), dtype=torch.float32),
        lse=torch.zeros((rows,), dtype=torch.float32),
    )


def test_buffer_checks_accept_matching_tensors():
    """Host-side checks pass for tensors that match the descriptor (no device call)."""
    d = mla.make_desc(3, 2, 16, 7, 5)
    t = _tensors(d)
    mla.check_decode_buffers(d, t["q"], t["kv_cache"], None, t["block_table"], t["seq_lens"], t["out"], t["lse"])


@pytest.mark.parametrize("bad", ["q", "kv_cache", "block_table", "seq_lens", "out", "lse"])
def test_buffer_checks_reject_short_or_mistyped(bad):
    """A tensor smaller than the descriptor needs (or of the wrong element size)
    raises before anything is launched: e.g. an fp8 cache passed with a bf16
    descriptor is half the bytes the kernel would read."""
    import torch
    d = mla.make_desc(3, 2, 16, 7, 5)
    t = _tensors(d)
    x = t[bad]
    t[bad] = x.flatten()[: x.numel() - 1].clone()
    with pytest.raises(ValueError):
        mla.check_decode_buffers(d, t["q"], t["kv_cache"], None, t["block_table"], t["seq_lens"], t["out"], t["lse"])
    t = _tensors(d, kv_dtype_bytes=1)       # e4m3 bytes with a bf16 descriptor
    with pytest.raises(ValueError):
        mla.check_decode_buffers(d, t["q"], t["kv_cache"], None, t["block_table"], t["seq_lens"], t["out"], t["lse"])


def test_buffer_checks_kv_scale_rules():
    import torch
    d8 = mla.make_desc(2, 1, 16, 4, 2, kv_dtype=mla.FP8_E4M3)
    t = _tensors(d8, kv_dtype_bytes=1)
    with pytest.raises(ValueError):
        mla.check_decode_buffers(d8, t["q"], t["kv_cache"], None, t["block_table"], t["seq_lens"], t["out"], t["lse"])
    mla.check_decode_buffers(d8, t["q"], t["kv_cache"], torch.ones(1), t["block_table"], t["seq_lens"],
                             t["out"], t["lse"])
    d = mla.make_desc(2, 1, 16, 4, 2)
    t = _tensors(d)
    with pytest.raises(ValueError):
        mla.check_decode_buffers(d, t["q"], t["kv_cache"], torch.ones(1), t["block_table"], t["seq_lens"],
                                 t["out"], t["lse"])


def test_merge_buffer_checks():
    import torch
    outs = torch.zeros((4, 10, mla.LATENT_DIM))
    lses = torch.zeros((4, 10))
    with pytest.raises(ValueError):
        mla.merge_states(outs, lses, 4, 11, torch.zeros((11, mla.LATENT_DIM)), torch.zeros(11))


def test_build_script_loads_without_the_package():
    """A fresh checkout has no library yet, and the package refuses to import
    without it: the build script (and the checker it runs) must therefore load
    without importing the package."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import importlib.util, os, sys\n"
        f"p = os.path.join({root!r}, 'mla_latent_decode_absorbed_amd', 'build.py')\n"
        "spec = importlib.util.spec_from_file_location('_b', p)\n"
        "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m)\n"
        "assert callable(m.build) and callable(m.check_wait_states)\n"
        "assert 'mla_latent_decode_absorbed_amd' not in sys.modules\n"
    )
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd="/")
    assert res.returncode == 0, res.stderr
    src = open(os.path.join(root, "mla_latent_decode_absorbed_amd", "build.py")).read()
    assert "from mla_latent_decode_absorbed_amd" not in src and "import mla_latent_decode_absorbed_amd" not in src


def _qdesc(**kw):
    d = dict(rows=4, num_heads=2, nope_dim=128, out_dtype=mla.BF16)
    d.update(kw)
    return mla.QueryPrepDesc(d["rows"], d["num_heads"], d["nope_dim"], d["out_dtype"])


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), mla.ERR_INVALID_ARG),
    (dict(num_heads=0), mla.ERR_INVALID_ARG),
    (dict(out_dtype=mla.F32), mla.ERR_INVALID_ARG),
    (dict(nope_dim=136), mla.ERR_UNSUPPORTED),
    (dict(nope_dim=272), mla.ERR_UNSUPPORTED),
    (dict(nope_dim=0), mla.ERR_UNSUPPORTED),
])
def test_query_prep_rejects_bad_descriptor(kw, status):
    d = _qdesc(**kw)
    assert mla.lib.mla_query_prep(ctypes.byref(d), 16, 16, 16, None, 16, None) == status


def test_query_prep_pointer_and_scale_rules():
    d = _qdesc()
    assert mla.lib.mla_query_prep(None, 16, 16, 16, None, 16, None) == mla.ERR_INVALID_ARG
    assert mla.lib.mla_query_prep(ctypes.byref(d), None, 16, 16, None, 16, None) == mla.ERR_INVALID_ARG
    assert mla.lib.mla_query_prep(ctypes.byref(d), 16, 16, 16, None, 8, None) == mla.ERR_INVALID_ARG
    assert mla.lib.mla_query_prep(ctypes.byref(d), 16, 16, 16, 16, 16, None) == mla.ERR_INVALID_ARG
    d8 = _qdesc(out_dtype=mla.FP8_E4M3)
    assert mla.lib.mla_query_prep(ctypes.byref(d8), 16, 16, 16, None, 16, None) == mla.ERR_INVALID_ARG
    # zero rows: nothing to do, no device work
    assert mla.lib.mla_query_prep(ctypes.byref(_qdesc(rows=0)), None, None, None, None, None, None) == mla.OK


def _udesc(**kw):
    d = dict(rows=4, num_heads=2, v_head_dim=128, in_dtype=mla.F32, out_dtype=mla.BF16)
    d.update(kw)
    return mla.UpProjectDesc(d["rows"], d["num_heads"], d["v_head_dim"], d["in_dtype"], d["out_dtype"])


@pytest.mark.parametrize("kw,status", [
    (dict(rows=-1), mla.ERR_INVALID_ARG),
    (dict(num_heads=0), mla.ERR_INVALID_ARG),
    (dict(in_dtype=mla.FP8_E4M3), mla.ERR_INVALID_ARG),
    (dict(out_dtype=7), mla.ERR_INVALID_ARG),
    (dict(v_head_dim=48), mla.ERR_UNSUPPORTED),
    (dict(v_head_dim=544), mla.ERR_UNSUPPORTED),
    (dict(v_head_dim=0), mla.ERR_UNSUPPORTED),
])
def test_up_project_rejects_bad_descriptor(kw, status):
    assert mla.lib.mla_up_project(ctypes.byref(_udesc(**kw)), 16, 16, 16, None) == status


def test_up_project_pointer_rules():
    d = _udesc()
    assert mla.lib.mla_up_project(None, 16, 16, 16, None) == mla.ERR_INVALID_ARG
    assert mla.lib.mla_up_project(ctypes.byref(d), None, 16, 16, None) == mla.ERR_INVALID_ARG
    assert mla.lib.mla_up_project(ctypes.byref(d), 16, 16, 8, None) == mla.ERR_INVALID_ARG
    assert mla.lib.mla_up_project(ctypes.byref(_udesc(rows=0)), None, None, None, None) == mla.OK


def test_merge_up_project_argument_rules():
    d = _udesc(in_dtype=mla.F32)
    assert mla.lib.mla_merge_up_project(16, 16, 0, ctypes.byref(d), 16, 16, None, None) == mla.ERR_INVALID_ARG
    assert mla.lib.mla_merge_up_project(16, 16, 17, ctypes.byref(d), 16, 16, None, None) == mla.ERR_INVALID_ARG
    assert mla.lib.mla_merge_up_project(16, 16, 4, ctypes.byref(_udesc(in_dtype=mla.BF16)), 16, 16, None,
                                        None) == mla.ERR_INVALID_ARG
    assert mla.lib.mla_merge_up_project(16, 16, 4, ctypes.byref(_udesc(v_head_dim=48)), 16, 16, None,
                                        None) == mla.ERR_UNSUPPORTED
    assert mla.lib.mla_merge_up_project(None, 16, 4, ctypes.byref(d), 16, 16, None, None) == mla.ERR_INVALID_ARG
    assert mla.lib.mla_merge_up_project(None, None, 4, ctypes.byref(_udesc(rows=0)), None, None, None, None) == mla.OK
