"""Twilight hierarchical top-p sparse decode attention for MI355X (gfx950).

Thin Python binding over ``libtwilight.so``: argument marshalling only. Every step of the
path runs in the HIP kernels behind the C ABI declared in ``include/twilight.h``; the
functions below take torch tensors that live on the GPU, pass their device pointers and the
current HIP stream, and raise ``TwilightError`` on a negative status. There is no CPU
fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtwilight.so")
PAGE_SIZE = 16

TWL_OK = 0
TWL_ERR_INVALID_ARG = -1
TWL_ERR_UNSUPPORTED = -2
TWL_ERR_WORKSPACE = -3
TWL_ERR_LAUNCH = -4
TWL_ERR_SCRATCH = -5

EXPORTED = ("twilight_quantize_keys", "quest_page_bounds", "quest_select_pages",
            "twilight_estimate_weights", "twilight_topp_select", "twilight_sparse_decode",
            "twilight_append_keys", "twilight_topp_select_headwise",
            "twilight_sparse_decode_headwise", "twilight_estimate_topp",
            "twilight_estimate_topp_headwise", "quest_page_scores", "quest_top_pages",
            "twilight_sparse_decode_noalloc", "quest_score_stride",
            "twilight_workspace_size", "twilight_status_string")


class TwilightError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")
        self.status = status


class Layout(ctypes.Structure):
    """Mirror of twl_layout_t."""
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("num_phys_pages", ctypes.c_int32), ("page_table", ctypes.c_void_p),
                ("seq_lens", ctypes.c_void_p), ("key_bits", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libtwilight.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python adaptive_top_sparse_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
        LP = ctypes.POINTER(Layout)
        L.twilight_quantize_keys.argtypes = [LP, P, P, P, P, P]
        L.quest_page_bounds.argtypes = [LP, P, P, P, P]
        L.quest_select_pages.argtypes = [LP, P, P, I32, P, P, P, SZ, P]
        L.twilight_estimate_weights.argtypes = [LP, P, P, P, P, P, I32, F, P, P, SZ, P]
        L.twilight_topp_select.argtypes = [LP, P, P, P, I32, F, P, P, P, P, SZ, P]
        L.twilight_sparse_decode.argtypes = [LP, P, P, P, P, P, I32, F, P, P, SZ, P]
        L.twilight_append_keys.argtypes = [LP, P, P, P, P, P, P]
        L.twilight_topp_select_headwise.argtypes = L.twilight_topp_select.argtypes
        L.twilight_sparse_decode_headwise.argtypes = L.twilight_sparse_decode.argtypes
        L.twilight_estimate_topp.argtypes = [LP, P, P, P, P, P, I32, F, F, P, P, P, P, P, SZ, P]
        L.twilight_estimate_topp_headwise.argtypes = L.twilight_estimate_topp.argtypes
        L.quest_page_scores.argtypes = [LP, P, P, P, P]
        L.quest_top_pages.argtypes = [LP, P, I32, P, P, P]
        L.twilight_sparse_decode_noalloc.argtypes = [LP, P, P, P, P, P, I32, F, P, P]
        for name in EXPORTED[:14]:
            getattr(L, name).restype = ctypes.c_int
        L.quest_score_stride.argtypes = [I32]
        L.quest_score_stride.restype = ctypes.c_int64
        L.twilight_workspace_size.argtypes = [LP, I32]
        L.twilight_workspace_size.restype = ctypes.c_size_t
        L.twilight_status_string.argtypes = [ctypes.c_int]
        L.twilight_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().twilight_status_string(int(status)).decode()


# ---- marshalling helpers -----------------------------------------------------------------

def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous GPU tensor (None passes NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != TWL_OK:
        raise TwilightError(fn, status)


def make_layout(page_table, seq_lens, num_q_heads: int, num_kv_heads: int, head_dim: int,
                num_phys_pages: int, key_bits: int = 4) -> Layout:
    """twl_layout_t for int32 GPU tensors page_table [B, max_pages] and seq_lens [B].

    The tensors must outlive every call made with the layout."""
    import torch
    B, max_pages = page_table.shape
    return Layout(batch=B, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                  head_dim=head_dim, page_size=PAGE_SIZE, max_pages_per_seq=max_pages,
                  num_phys_pages=num_phys_pages,
                  page_table=_ptr(page_table, torch.int32, "page_table"),
                  seq_lens=_ptr(seq_lens, torch.int32, "seq_lens"), key_bits=key_bits)


# ---- the C ABI, one function each -------------------------------------------------------

def twilight_workspace_size(layout: Layout, cand_stride_pages: int) -> int:
    return int(lib().twilight_workspace_size(ctypes.byref(layout), int(cand_stride_pages)))


def twilight_quantize_keys(layout: Layout, k_cache, k_codes, k_meta, token_begin=None,
                           stream=None) -> None:
    import torch
    st = lib().twilight_quantize_keys(
        ctypes.byref(layout), _ptr(k_cache, torch.float16, "k_cache"),
        _ptr(token_begin, torch.int32, "token_begin"), _ptr(k_codes, torch.uint8, "k_codes"),
        _ptr(k_meta, torch.float16, "k_meta"), _stream(stream))
    _check("twilight_quantize_keys", st)


def quest_page_bounds(layout: Layout, k_cache, page_minmax, token_begin=None,
                      stream=None) -> None:
    import torch
    st = lib().quest_page_bounds(
        ctypes.byref(layout), _ptr(k_cache, torch.float16, "k_cache"),
        _ptr(token_begin, torch.int32, "token_begin"),
        _ptr(page_minmax, torch.float16, "page_minmax"), _stream(stream))
    _check("quest_page_bounds", st)


def twilight_append_keys(layout: Layout, k_cache, token_begin, k_codes, k_meta,
                         page_minmax=None, stream=None) -> None:
    import torch
    st = lib().twilight_append_keys(
        ctypes.byref(layout), _ptr(k_cache, torch.float16, "k_cache"),
        _ptr(token_begin, torch.int32, "token_begin"), _ptr(k_codes, torch.uint8, "k_codes"),
        _ptr(k_meta, torch.float16, "k_meta"), _ptr(page_minmax, torch.float16, "page_minmax"),
        _stream(stream))
    _check("twilight_append_keys", st)


def quest_select_pages(layout: Layout, q, page_minmax, budget_pages: int, sel_pages, sel_count,
                       workspace, stream=None) -> None:
    import torch
    st = lib().quest_select_pages(
        ctypes.byref(layout), _ptr(q, torch.float16, "q"),
        _ptr(page_minmax, torch.float16, "page_minmax"), int(budget_pages),
        _ptr(sel_pages, torch.int32, "sel_pages"), _ptr(sel_count, torch.int32, "sel_count"),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check("quest_select_pages", st)


def quest_score_stride(max_pages_per_seq: int) -> int:
    """Doubles per (sequence, KV head) row of a Quest score buffer."""
    return int(lib().quest_score_stride(int(max_pages_per_seq)))


def quest_page_scores(layout: Layout, q, page_minmax, scores, stream=None) -> None:
    import torch
    st = lib().quest_page_scores(
        ctypes.byref(layout), _ptr(q, torch.float16, "q"),
        _ptr(page_minmax, torch.float16, "page_minmax"), _ptr(scores, torch.float64, "scores"),
        _stream(stream))
    _check("quest_page_scores", st)


def quest_top_pages(layout: Layout, scores, budget_pages: int, sel_pages, sel_count,
                    stream=None) -> None:
    import torch
    st = lib().quest_top_pages(
        ctypes.byref(layout), _ptr(scores, torch.float64, "scores"), int(budget_pages),
        _ptr(sel_pages, torch.int32, "sel_pages"), _ptr(sel_count, torch.int32, "sel_count"),
        _stream(stream))
    _check("quest_top_pages", st)


def twilight_estimate_weights(layout: Layout, q, k_codes, k_meta, cand_pages, cand_count,
                              cand_stride_pages: int, sm_scale: float, weights, workspace,
                              stream=None) -> None:
    import torch
    st = lib().twilight_estimate_weights(
        ctypes.byref(layout), _ptr(q, torch.float16, "q"), _ptr(k_codes, torch.uint8, "k_codes"),
        _ptr(k_meta, torch.float16, "k_meta"), _ptr(cand_pages, torch.int32, "cand_pages"),
        _ptr(cand_count, torch.int32, "cand_count"), int(cand_stride_pages), float(sm_scale),
        _ptr(weights, torch.float32, "weights"), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check("twilight_estimate_weights", st)


def _topp_select(name: str, layout: Layout, weights, cand_pages, cand_count,
                 cand_stride_pages: int, p: float, kept, kept_count, tau, workspace,
                 stream=None) -> None:
    import torch
    st = getattr(lib(), name)(
        ctypes.byref(layout), _ptr(weights, torch.float32, "weights"),
        _ptr(cand_pages, torch.int32, "cand_pages"), _ptr(cand_count, torch.int32, "cand_count"),
        int(cand_stride_pages), float(p), _ptr(kept, torch.int32, "kept"),
        _ptr(kept_count, torch.int32, "kept_count"), _ptr(tau, torch.float32, "tau"),
        _ptr(workspace, None, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(name, st)


def _estimate_topp(name: str, layout: Layout, q, k_codes, k_meta, cand_pages, cand_count,
                   cand_stride_pages: int, sm_scale: float, p: float, weights, kept,
                   kept_count, tau, workspace, stream=None) -> None:
    import torch
    st = getattr(lib(), name)(
        ctypes.byref(layout), _ptr(q, torch.float16, "q"), _ptr(k_codes, torch.uint8, "k_codes"),
        _ptr(k_meta, torch.float16, "k_meta"), _ptr(cand_pages, torch.int32, "cand_pages"),
        _ptr(cand_count, torch.int32, "cand_count"), int(cand_stride_pages), float(sm_scale),
        float(p), _ptr(weights, torch.float32, "weights"), _ptr(kept, torch.int32, "kept"),
        _ptr(kept_count, torch.int32, "kept_count"), _ptr(tau, torch.float32, "tau"),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream))
    _check(name, st)


def twilight_estimate_topp(layout: Layout, q, k_codes, k_meta, cand_pages, cand_count,
                           cand_stride_pages: int, sm_scale: float, p: float, weights, kept,
                           kept_count, tau, workspace, stream=None) -> None:
    """Estimate and group-wise top-p in one call (weights is scratch)."""
    _estimate_topp("twilight_estimate_topp", layout, q, k_codes, k_meta, cand_pages,
                   cand_count, cand_stride_pages, sm_scale, p, weights, kept, kept_count, tau,
                   workspace, stream)


def twilight_estimate_topp_headwise(layout: Layout, q, k_codes, k_meta, cand_pages,
                                    cand_count, cand_stride_pages: int, sm_scale: float,
                                    p: float, weights, kept, kept_count, tau, workspace,
                                    stream=None) -> None:
    """Estimate and head-wise top-p in one call (weights is scratch)."""
    _estimate_topp("twilight_estimate_topp_headwise", layout, q, k_codes, k_meta, cand_pages,
                   cand_count, cand_stride_pages, sm_scale, p, weights, kept, kept_count, tau,
                   workspace, stream)


def twilight_topp_select(layout: Layout, weights, cand_pages, cand_count,
                         cand_stride_pages: int, p: float, kept, kept_count, tau, workspace,
                         stream=None) -> None:
    """Group-wise: kept [B, Hkv, stride * 16], kept_count and tau [B, Hkv]."""
    _topp_select("twilight_topp_select", layout, weights, cand_pages, cand_count,
                 cand_stride_pages, p, kept, kept_count, tau, workspace, stream)


def twilight_topp_select_headwise(layout: Layout, weights, cand_pages, cand_count,
                                  cand_stride_pages: int, p: float, kept, kept_count, tau,
                                  workspace, stream=None) -> None:
    """Head-wise: kept [B, Hq, stride * 16], kept_count and tau [B, Hq]."""
    _topp_select("twilight_topp_select_headwise", layout, weights, cand_pages, cand_count,
                 cand_stride_pages, p, kept, kept_count, tau, workspace, stream)


def _sparse_decode(name: str, layout: Layout, q, k_cache, v_cache, kept, kept_count,
                   kept_stride: int, sm_scale: float, out, workspace, stream=None) -> None:
    import torch
    st = getattr(lib(), name)(
        ctypes.byref(layout), _ptr(q, torch.float16, "q"), _ptr(k_cache, torch.float16, "k_cache"),
        _ptr(v_cache, torch.float16, "v_cache"), _ptr(kept, torch.int32, "kept"),
        _ptr(kept_count, torch.int32, "kept_count"), int(kept_stride), float(sm_scale),
        _ptr(out, torch.float16, "out"), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream))
    _check(name, st)


def twilight_sparse_decode(layout: Layout, q, k_cache, v_cache, kept, kept_count,
                           kept_stride: int, sm_scale: float, out, workspace,
                           stream=None) -> None:
    """Group-wise kept lists [B, Hkv, kept_stride]."""
    _sparse_decode("twilight_sparse_decode", layout, q, k_cache, v_cache, kept, kept_count,
                   kept_stride, sm_scale, out, workspace, stream)


def twilight_sparse_decode_noalloc(layout: Layout, q, k_cache, v_cache, kept, kept_count,
                                   kept_stride: int, sm_scale: float, out,
                                   stream=None) -> None:
    """Group-wise decode with the library's fixed device scratch (no workspace, no
    allocation; calls that overlap on one GPU race)."""
    import torch
    st = lib().twilight_sparse_decode_noalloc(
        ctypes.byref(layout), _ptr(q, torch.float16, "q"), _ptr(k_cache, torch.float16, "k_cache"),
        _ptr(v_cache, torch.float16, "v_cache"), _ptr(kept, torch.int32, "kept"),
        _ptr(kept_count, torch.int32, "kept_count"), int(kept_stride), float(sm_scale),
        _ptr(out, torch.float16, "out"), _stream(stream))
    _check("twilight_sparse_decode_noalloc", st)


def twilight_sparse_decode_headwise(layout: Layout, q, k_cache, v_cache, kept, kept_count,
                                    kept_stride: int, sm_scale: float, out, workspace,
                                    stream=None) -> None:
    """Head-wise kept lists [B, Hq, kept_stride]."""
    _sparse_decode("twilight_sparse_decode_headwise", layout, q, k_cache, v_cache, kept,
                   kept_count, kept_stride, sm_scale, out, workspace, stream)
