"""The C ABI without a GPU: libtwilight.so loads, exports every function include/twilight.h
declares, and its host-side validation answers with the documented statuses before any
device work (the pointers below are never dereferenced on the host)."""
import ctypes
import os
import re
import subprocess

import pytest

import adaptive_top_sparse_amd as twl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "twilight.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|size_t|const char\*)\s+(\w+)\s*\(", text, re.M)))


def test_header_declares_the_six_stages_and_helpers():
    assert declared_functions() == sorted(twl.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = twl.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", twl.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name


def test_status_strings():
    assert twl.status_string(0) == "ok"
    for st in (-1, -2, -3, -4, -5):
        assert twl.status_string(st) and twl.status_string(st) != "unknown status"
    assert twl.status_string(12345) == "unknown status"


FAKE = 0x7f0000000000  # aligned placeholder device address, never dereferenced on the host


def layout(B=1, Hq=32, Hkv=8, d=128, ps=16, max_pages=512, phys=512):
    return twl.Layout(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=d, page_size=ps,
                      max_pages_per_seq=max_pages, num_phys_pages=phys, page_table=FAKE,
                      seq_lens=FAKE + 4096)


def test_workspace_size_is_positive_for_valid_layouts_and_zero_otherwise():
    for Hq, Hkv, d in ((32, 8, 128), (32, 32, 128), (1, 1, 64), (16, 2, 64)):
        assert twl.twilight_workspace_size(layout(Hq=Hq, Hkv=Hkv, d=d), 64) > 0
    assert twl.twilight_workspace_size(layout(d=96), 64) == 0        # head_dim
    assert twl.twilight_workspace_size(layout(Hq=24, Hkv=8), 64) == 0  # G = 3
    assert twl.twilight_workspace_size(layout(ps=32), 64) == 0       # page size
    assert twl.twilight_workspace_size(layout(), 0) == 0             # stride


def test_workspace_grows_with_the_candidate_stride():
    a = twl.twilight_workspace_size(layout(B=8, max_pages=4096, phys=32768), 512)
    b = twl.twilight_workspace_size(layout(B=8, max_pages=4096, phys=32768), 4096)
    assert b > a > 0


def _call(fn, *args):
    return getattr(twl.lib(), fn)(*args)


def test_invalid_arguments_are_rejected_on_the_host():
    L = layout()
    Lp = ctypes.byref(L)
    ws, wsn = FAKE + (1 << 20), 1 << 30
    # null required pointers
    assert _call("twilight_quantize_keys", Lp, None, None, FAKE, FAKE, None) == twl.TWL_ERR_INVALID_ARG
    assert _call("quest_page_bounds", Lp, FAKE, None, None, None) == twl.TWL_ERR_INVALID_ARG
    # misaligned vector operand
    assert _call("twilight_quantize_keys", Lp, FAKE + 2, None, FAKE, FAKE, None) == twl.TWL_ERR_INVALID_ARG
    # budget < 1
    assert _call("quest_select_pages", Lp, FAKE, FAKE, 0, FAKE, FAKE, ws, wsn, None) == twl.TWL_ERR_INVALID_ARG
    # p outside (0, 1]
    for p in (0.0, -0.5, 1.5, float("nan")):
        assert _call("twilight_topp_select", Lp, FAKE, FAKE, FAKE, 64, ctypes.c_float(p), FAKE,
                     FAKE, None, ws, wsn, None) == twl.TWL_ERR_INVALID_ARG
    # all-pages candidates need a stride covering max_pages_per_seq
    assert _call("twilight_estimate_weights", Lp, FAKE, FAKE, FAKE, None, None, 100,
                 ctypes.c_float(0.1), FAKE, ws, wsn, None) == twl.TWL_ERR_INVALID_ARG
    # workspace missing or too small
    assert _call("quest_select_pages", Lp, FAKE, FAKE, 64, FAKE, FAKE, None, 0, None) == twl.TWL_ERR_WORKSPACE
    assert _call("twilight_sparse_decode", Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 1024,
                 ctypes.c_float(0.1), FAKE, ws, 16, None) == twl.TWL_ERR_WORKSPACE
    # non-finite scale, bad stride
    assert _call("twilight_sparse_decode", Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 1024,
                 ctypes.c_float(float("inf")), FAKE, ws, wsn, None) == twl.TWL_ERR_INVALID_ARG
    assert _call("twilight_sparse_decode", Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 0,
                 ctypes.c_float(0.1), FAKE, ws, wsn, None) == twl.TWL_ERR_INVALID_ARG


def test_newer_entry_points_reject_invalid_arguments_on_the_host():
    L = layout()
    Lp = ctypes.byref(L)
    ws, wsn = FAKE + (1 << 20), 1 << 30
    f = ctypes.c_float
    # append: token_begin is required, page_minmax may be null but must be aligned
    assert _call("twilight_append_keys", Lp, FAKE, None, FAKE, FAKE, None, None) == twl.TWL_ERR_INVALID_ARG
    assert _call("twilight_append_keys", Lp, FAKE, FAKE, FAKE, FAKE, FAKE + 4, None) == twl.TWL_ERR_INVALID_ARG
    # fused estimate + top-p: required outputs, p range, scale, workspace
    for name in ("twilight_estimate_topp", "twilight_estimate_topp_headwise"):
        assert _call(name, Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 64, f(0.1), f(0.9), FAKE, None, FAKE,
                     None, ws, wsn, None) == twl.TWL_ERR_INVALID_ARG
        assert _call(name, Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 64, f(0.1), f(1.5), FAKE, FAKE, FAKE,
                     None, ws, wsn, None) == twl.TWL_ERR_INVALID_ARG
        assert _call(name, Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 64, f(float("nan")), f(0.9), FAKE,
                     FAKE, FAKE, None, ws, wsn, None) == twl.TWL_ERR_INVALID_ARG
        assert _call(name, Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 64, f(0.1), f(0.9), FAKE, FAKE, FAKE,
                     None, None, 0, None) == twl.TWL_ERR_WORKSPACE
        assert _call(name, Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 64, f(0.1), f(0.9), FAKE, FAKE, FAKE,
                     None, ws, 16, None) == twl.TWL_ERR_WORKSPACE
    # head-wise top-p and decode: same checks as the group-wise calls
    assert _call("twilight_topp_select_headwise", Lp, FAKE, FAKE, FAKE, 64, f(0.0), FAKE, FAKE,
                 None, ws, wsn, None) == twl.TWL_ERR_INVALID_ARG
    assert _call("twilight_sparse_decode_headwise", Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 1024,
                 f(0.1), FAKE, ws, 16, None) == twl.TWL_ERR_WORKSPACE
    # Quest scores and top pages on their own: required buffers, alignment, budget, size limit
    assert _call("quest_page_scores", Lp, FAKE, FAKE, None, None) == twl.TWL_ERR_INVALID_ARG
    assert _call("quest_page_scores", Lp, FAKE, FAKE, FAKE + 8, None) == twl.TWL_ERR_INVALID_ARG
    assert _call("quest_top_pages", Lp, FAKE, 0, FAKE, FAKE, None) == twl.TWL_ERR_INVALID_ARG
    assert _call("quest_top_pages", Lp, None, 64, FAKE, FAKE, None) == twl.TWL_ERR_INVALID_ARG
    assert _call("quest_top_pages", Lp, FAKE + 8, 64, FAKE, FAKE, None) == twl.TWL_ERR_INVALID_ARG
    big = layout(max_pages=40000)
    assert _call("quest_top_pages", ctypes.byref(big), FAKE, 64, FAKE, FAKE, None) == twl.TWL_ERR_UNSUPPORTED
    assert twl.quest_score_stride(1) == 64 and twl.quest_score_stride(8192) == 8192
    assert twl.quest_score_stride(8193) == 8256 and twl.quest_score_stride(0) == -1
    # key width: only 4 (or 0 for 4) and 2
    bad = layout()
    bad.key_bits = 3
    assert _call("twilight_quantize_keys", ctypes.byref(bad), FAKE, None, FAKE, FAKE, None) == twl.TWL_ERR_UNSUPPORTED
    assert twl.twilight_workspace_size(bad, 64) == 0


def test_noalloc_decode_checks_arguments_and_its_fixed_scratch_on_the_host():
    # the no-allocation decode takes no workspace: the usual argument checks, then a
    # refusal (nothing enqueued) when the partials would not fit its fixed 16 MiB buffer;
    # all of it before any device query, so it answers without a GPU
    f = ctypes.c_float
    Lp = ctypes.byref(layout())
    assert _call("twilight_sparse_decode_noalloc", Lp, None, FAKE, FAKE, FAKE, FAKE, 1024, f(0.1),
                 FAKE, None) == twl.TWL_ERR_INVALID_ARG
    assert _call("twilight_sparse_decode_noalloc", Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 0, f(0.1),
                 FAKE, None) == twl.TWL_ERR_INVALID_ARG
    assert _call("twilight_sparse_decode_noalloc", Lp, FAKE, FAKE, FAKE, FAKE, FAKE, 1024,
                 f(float("nan")), FAKE, None) == twl.TWL_ERR_INVALID_ARG
    # B = 64 sequences of 32 heads with 64k-token kept lists need far more than 16 MiB
    big = layout(B=64, Hq=32, Hkv=8, max_pages=4096, phys=64 * 4096)
    assert _call("twilight_sparse_decode_noalloc", ctypes.byref(big), FAKE, FAKE, FAKE, FAKE,
                 FAKE, 65536, f(0.1), FAKE, None) == twl.TWL_ERR_SCRATCH
    assert "16 MiB" in twl.status_string(twl.TWL_ERR_SCRATCH)
    e = layout(B=0)
    e.page_table = None
    e.seq_lens = None
    assert _call("twilight_sparse_decode_noalloc", ctypes.byref(e), FAKE, FAKE, FAKE, FAKE, FAKE,
                 1024, f(0.1), FAKE, None) == twl.TWL_OK


def test_unsupported_shapes_are_reported():
    for bad in (layout(d=256), layout(Hq=48, Hkv=8), layout(ps=8)):
        st = _call("twilight_quantize_keys", ctypes.byref(bad), FAKE, None, FAKE, FAKE, None)
        assert st == twl.TWL_ERR_UNSUPPORTED
    big = layout(max_pages=40000, phys=40000)
    st = _call("quest_select_pages", ctypes.byref(big), FAKE, FAKE, 64, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == twl.TWL_ERR_UNSUPPORTED
    st = _call("twilight_topp_select", ctypes.byref(layout()), FAKE, FAKE, FAKE, 8192,
               ctypes.c_float(0.9), FAKE, FAKE, None, FAKE, 1 << 40, None)
    assert st == twl.TWL_ERR_UNSUPPORTED


def test_empty_batch_is_a_no_op():
    L = layout(B=0)
    L.page_table = None
    L.seq_lens = None
    assert _call("twilight_quantize_keys", ctypes.byref(L), FAKE, None, FAKE, FAKE, None) == twl.TWL_OK
    assert twl.twilight_workspace_size(L, 8) > 0


def test_product_path_fails_loudly_without_the_library(monkeypatch, tmp_path):
    monkeypatch.setattr(twl, "_lib", None)
    monkeypatch.setattr(twl, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        twl.lib()
