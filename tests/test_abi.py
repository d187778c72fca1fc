"""The C ABI library: it loads without a GPU, exports every symbol include/gsr.h
declares, and its host-side checks return the documented status codes before
launching anything (no compute call here)."""
import ctypes
import os
import re

import pytest

from gaussian_splatting_rasterizer_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(b.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return b.load_library()


def test_every_declared_symbol_is_exported():
    lib = _lib()
    header = open(os.path.join(ROOT, "include", "gsr.h")).read()
    declared = re.findall(r"GSR_API\s+[\w\s\*]+?\b(gs_\w+)\s*\(", header)
    assert len(declared) >= 14
    for name in declared:
        assert hasattr(lib, name), name
    assert set(b.ABI_SYMBOLS) <= set(declared)


def test_status_strings_and_defaults():
    lib = _lib()
    for code, name in [(0, "GS_OK"), (1, "GS_ERR_INVALID_ARGUMENT"), (2, "GS_ERR_WORKSPACE_TOO_SMALL"),
                       (3, "GS_ERR_STATE"), (4, "GS_ERR_HIP"), (5, "GS_ERR_UNSUPPORTED")]:
        assert lib.gs_status_string(code).decode() == name
    p = b.gs_default_params()
    assert abs(p.eps - 1e-6) < 1e-12 and abs(p.den_min - 1e-3) < 1e-9 and p.lam == 1.0
    assert abs(p.near_plane - 0.01) < 1e-8 and list(p.background) == [0.0, 0.0, 0.0]
    assert p.antialiased == 0


def _dims(**kw):
    d = dict(n_gaussians=1000, sh_degree=3, n_views=2, width=64, height=48, max_pairs=10000)
    d.update(kw)
    return b.gs_dims(d["n_gaussians"], d["sh_degree"], d["n_views"], d["width"], d["height"], d["max_pairs"])


def _size_status(**kw):
    lib = _lib()
    out = ctypes.c_size_t(0)
    return lib.gs_workspace_size(ctypes.byref(_dims(**kw)), ctypes.byref(out)), out.value


def test_workspace_size_validation():
    st, n = _size_status()
    assert st == b.GS_OK and n > 0
    assert _size_status(sh_degree=4)[0] == b.GS_ERR_INVALID_ARGUMENT
    assert _size_status(sh_degree=-1)[0] == b.GS_ERR_INVALID_ARGUMENT
    assert _size_status(n_views=0)[0] == b.GS_ERR_INVALID_ARGUMENT
    assert _size_status(n_views=33)[0] == b.GS_ERR_UNSUPPORTED
    assert _size_status(width=0)[0] == b.GS_ERR_INVALID_ARGUMENT
    assert _size_status(n_gaussians=-5)[0] == b.GS_ERR_INVALID_ARGUMENT
    assert _size_status(max_pairs=0)[0] == b.GS_ERR_INVALID_ARGUMENT
    assert _size_status(max_pairs=1 << 32)[0] == b.GS_ERR_UNSUPPORTED
    assert _size_status(max_pairs=(1 << 32) - (1 << 16) + 1)[0] == b.GS_ERR_UNSUPPORTED
    assert _size_status(n_gaussians=0)[0] == b.GS_OK
    # the size grows with the pair capacity and the image
    assert _size_status(max_pairs=20000)[1] > n and _size_status(width=128)[1] > n


def test_context_creation_checks_the_workspace():
    lib = _lib()
    st, need = _size_status()
    ctx = ctypes.c_void_p()
    d = _dims()
    assert lib.gs_context_create(ctypes.byref(d), None, need, ctypes.byref(ctx)) == b.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_context_create(ctypes.byref(d), ctypes.c_void_p(4096 + 4), need,
                                 ctypes.byref(ctx)) == b.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_context_create(ctypes.byref(d), ctypes.c_void_p(4096), need - 1,
                                 ctypes.byref(ctx)) == b.GS_ERR_WORKSPACE_TOO_SMALL
    assert "needs" in b.last_error()


def test_calls_out_of_order_are_rejected_without_launching():
    """The workspace pointer is never dereferenced on the host: a fake aligned
    address lets the state machine be exercised with no GPU."""
    lib = _lib()
    st, need = _size_status()
    ctx = ctypes.c_void_p()
    d = _dims()
    assert lib.gs_context_create(ctypes.byref(d), ctypes.c_void_p(1 << 20), need, ctypes.byref(ctx)) == b.GS_OK
    try:
        n = ctypes.c_uint64(0)
        assert lib.gs_bin_sort(ctx, None, ctypes.byref(n)) == b.GS_ERR_STATE
        assert lib.gs_render(ctx, None, None, None, None) == b.GS_ERR_STATE
        assert lib.gs_score_replay(ctx, ctypes.c_void_p(256), ctypes.c_void_p(256), None) == b.GS_ERR_STATE
        grads = b.gs_gaussian_grads(256, 256, 256, 256, 256)
        assert lib.gs_backward(ctx, ctypes.c_void_p(256), ctypes.byref(grads), None) == b.GS_ERR_STATE
        assert lib.gs_backward(None, ctypes.c_void_p(256), ctypes.byref(grads), None) == b.GS_ERR_INVALID_ARGUMENT
        assert lib.gs_render_features(ctx, ctypes.c_void_p(256), 3, None, ctypes.c_void_p(256), None) == b.GS_ERR_STATE
        assert lib.gs_attribute(ctx, ctypes.c_void_p(256), 2, ctypes.c_void_p(256), None) == b.GS_ERR_STATE
        assert lib.gs_attribute(None, ctypes.c_void_p(256), 2, ctypes.c_void_p(256), None) == b.GS_ERR_INVALID_ARGUMENT
        assert lib.gs_debug_topk(ctx, 4, ctypes.c_void_p(256), ctypes.c_void_p(256), None) == b.GS_ERR_STATE
        # mismatched scene size and null parameters: rejected before any launch
        g = b.gs_gaussians(256, 256, 256, 256, 256, 999, 3)
        cams = b.make_cameras([[1, 0, 0, 0, 1, 0, 0, 0, 1, 0, 0, 0, 64, 64, 32, 24]] * 2)
        p = b.gs_default_params()
        assert lib.gs_project(ctx, ctypes.byref(g), cams, ctypes.byref(p), None) == b.GS_ERR_INVALID_ARGUMENT
        g = b.gs_gaussians(None, 256, 256, 256, 256, 1000, 3)
        assert lib.gs_project(ctx, ctypes.byref(g), cams, ctypes.byref(p), None) == b.GS_ERR_INVALID_ARGUMENT
        g = b.gs_gaussians(258, 256, 256, 256, 256, 1000, 3)
        assert lib.gs_project(ctx, ctypes.byref(g), cams, ctypes.byref(p), None) == b.GS_ERR_INVALID_ARGUMENT
        g = b.gs_gaussians(256, 256, 256, 256, 256, 1000, 2)
        assert lib.gs_project(ctx, ctypes.byref(g), cams, ctypes.byref(p), None) == b.GS_ERR_INVALID_ARGUMENT
        bad = b.gs_default_params()
        bad.near_plane = 0.0
        g = b.gs_gaussians(256, 256, 256, 256, 256, 1000, 3)
        assert lib.gs_project(ctx, ctypes.byref(g), cams, ctypes.byref(bad), None) == b.GS_ERR_INVALID_ARGUMENT
        bad2 = b.gs_default_params()
        bad2.antialiased = 2
        assert lib.gs_project(ctx, ctypes.byref(g), cams, ctypes.byref(bad2), None) == b.GS_ERR_INVALID_ARGUMENT
        cams0 = b.make_cameras([[1, 0, 0, 0, 1, 0, 0, 0, 1, 0, 0, 0, 0, 64, 32, 24]] * 2)
        assert lib.gs_project(ctx, ctypes.byref(g), cams0, ctypes.byref(p), None) == b.GS_ERR_INVALID_ARGUMENT
        # exports before the data exists
        assert lib.gs_debug_export(ctx, b.GS_EXPORT_RECORDS, ctypes.c_void_p(256), 1 << 30, None) == b.GS_ERR_STATE
        assert lib.gs_debug_export(ctx, 99, ctypes.c_void_p(256), 16, None) == b.GS_ERR_INVALID_ARGUMENT
        # profiling with nothing recorded
        # (the read writes only as many stages as the caller's arrays hold)
        ms = (ctypes.c_double * 4)(*[-1.0] * 4)
        calls = (ctypes.c_int64 * 4)(*[-1] * 4)
        assert lib.gs_profile_enable(ctx, 1) == b.GS_OK
        assert lib.gs_profile_read(ctx, ms, calls, 3) == b.GS_OK
        assert list(calls) == [0, 0, 0, -1] and list(ms) == [0.0, 0.0, 0.0, -1.0]
        assert lib.gs_profile_read(ctx, ms, calls, -1) == b.GS_ERR_INVALID_ARGUMENT
        n = len(b.STAGES)
        ms = (ctypes.c_double * n)()
        calls = (ctypes.c_int64 * n)()
        assert lib.gs_profile_read(ctx, ms, calls, n) == b.GS_OK
        assert list(calls) == [0] * n
        # a stage mask: any subset of the stages; a bit past the last stage is rejected
        assert lib.gs_profile_stages(ctx, (1 << n) - 1) == b.GS_OK
        assert lib.gs_profile_stages(ctx, 1 << 7) == b.GS_OK
        assert lib.gs_profile_stages(ctx, 1 << n) == b.GS_ERR_INVALID_ARGUMENT
        assert lib.gs_profile_stages(ctx, 0) == b.GS_OK
        assert lib.gs_profile_stages(None, 1) == b.GS_ERR_INVALID_ARGUMENT
    finally:
        lib.gs_context_destroy(ctx)


def test_null_arguments():
    lib = _lib()
    assert lib.gs_default_params(None) == b.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_workspace_size(None, None) == b.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_project(None, None, None, None, None) == b.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_bin_sort(None, None, None) == b.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_debug_exp2(None, None, -1, None) == b.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_context_destroy(None) == b.GS_OK


def test_binding_raises_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(b, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        b.load_library(str(tmp_path / "missing.so"))
