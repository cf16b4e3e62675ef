"""CPU oracle for Twilight hierarchical top-p sparse decode (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. It wraps ``liboracle_twilight.so`` (built from ``twilight_oracle.cpp`` by
``oracle/build.py``) with numpy-facing helpers; every computation happens in that C++
file, per (sequence, KV head) unit, in fp64.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_twilight.so")
_lib = None

_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(np.float64, flags="C_CONTIGUOUS")


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        i64, c_int, c_float = ctypes.c_int64, ctypes.c_int, ctypes.c_float
        L.orc_version.restype = c_int
        L.orc_quantize_keys.argtypes = [_u16p, i64, c_int, _u8p, _u16p, _u16p]
        L.orc_quantize_keys.restype = c_int
        L.orc_quantize_keys_bits.argtypes = [_u16p, i64, c_int, c_int, _u8p, _u16p, _u16p]
        L.orc_quantize_keys_bits.restype = c_int
        L.orc_page_bounds.argtypes = [_u16p, i64, c_int, c_int, _u16p, _u16p]
        L.orc_page_bounds.restype = c_int
        L.orc_quest_select.argtypes = [_u16p, c_int, c_int, _u16p, _u16p, i64, c_int, _i32p,
                                       ctypes.c_void_p, ctypes.POINTER(i64)]
        L.orc_quest_select.restype = c_int
        L.orc_estimate_weights.argtypes = [_u16p, c_int, c_int, _u8p, _u16p, _u16p, i64,
                                           ctypes.c_void_p, i64, c_int, c_float, _f64p, i64]
        L.orc_estimate_weights.restype = c_int
        L.orc_topp_select.argtypes = [_f64p, _u8p, c_int, i64, c_float, ctypes.c_void_p, i64,
                                      c_int, _i32p, ctypes.POINTER(ctypes.c_double)]
        L.orc_topp_select.restype = i64
        L.orc_sparse_attention.argtypes = [_u16p, c_int, c_int, _u16p, _u16p, i64, _i32p, i64,
                                           c_float, _f64p]
        L.orc_sparse_attention.restype = c_int
        L.orc_half_to_double.argtypes = [ctypes.c_uint16]
        L.orc_half_to_double.restype = ctypes.c_double
        L.orc_nearest_half_of_ratio.argtypes = [ctypes.c_double, c_int]
        L.orc_nearest_half_of_ratio.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _bits(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype == np.float16:
        return x.view(np.uint16)
    assert x.dtype == np.uint16, x.dtype
    return x


def quantize_keys(k: np.ndarray, bits: int = 4):
    """k: [n, d] fp16 -> (codes [n, d] uint8, scale [n, d/32] fp16, zero [n, d/32] fp16);
    bits 4 (the estimate's key cache) or 2 (the variant the pages ablate)."""
    k = _bits(k)
    n, d = k.shape
    codes = np.zeros((n, d), np.uint8)
    scale = np.zeros((n, d // 32), np.uint16)
    zero = np.zeros((n, d // 32), np.uint16)
    if bits == 4:
        rc = lib().orc_quantize_keys(k, n, d, codes, scale, zero)
    else:
        rc = lib().orc_quantize_keys_bits(k, n, d, int(bits), codes, scale, zero)
    if rc != 0:
        raise ValueError("orc_quantize_keys failed")
    return codes, scale.view(np.float16), zero.view(np.float16)


def page_bounds(k: np.ndarray, page_size: int = 16):
    """k: [n, d] fp16 -> (lo, hi), each [ceil(n/page_size), d] fp16."""
    k = _bits(k)
    n, d = k.shape
    P = -(-n // page_size)
    lo = np.zeros((P, d), np.uint16)
    hi = np.zeros((P, d), np.uint16)
    if lib().orc_page_bounds(k, n, d, page_size, lo, hi) != 0:
        raise ValueError("orc_page_bounds failed")
    return lo.view(np.float16), hi.view(np.float16)


def quest_select(q: np.ndarray, lo: np.ndarray, hi: np.ndarray, budget: int,
                 return_scores: bool = False):
    """q: [G, d]; lo, hi: [P, d] -> ascending selected page ids (and scores, sensitivity)."""
    q = _bits(q)
    lo = _bits(lo)
    hi = _bits(hi)
    G, d = q.shape
    P = lo.shape[0]
    sel = np.zeros(max(1, min(budget, P)), np.int32)
    scores = np.zeros(max(P, 1), np.float64)
    sens = ctypes.c_int64(0)
    m = lib().orc_quest_select(q, G, d, lo, hi, P, budget, sel,
                               scores.ctypes.data, ctypes.byref(sens))
    if m < 0:
        raise ValueError("orc_quest_select failed")
    if return_scores:
        return sel[:m].copy(), scores[:P].copy(), int(sens.value)
    return sel[:m].copy()


def estimate_weights(q, codes, scale, zero, n_tokens, cand_pages, n_slots, sm_scale,
                     page_size: int = 16):
    """Estimated softmax weights [G, n_slots] fp64 over the candidate slots.

    cand_pages: ascending int32 page ids, or None when every token is a candidate."""
    q = _bits(q)
    G, d = q.shape
    codes = np.ascontiguousarray(codes, np.uint8)
    scale = _bits(scale)
    zero = _bits(zero)
    w = np.zeros((G, max(n_slots, 1)), np.float64)
    if cand_pages is None:
        cp, ncp = None, 0
    else:
        cand_pages = np.ascontiguousarray(cand_pages, np.int32)
        cp, ncp = cand_pages.ctypes.data, cand_pages.shape[0]
    rc = lib().orc_estimate_weights(q, G, d, codes, scale, zero, n_tokens, cp, ncp, page_size,
                                    float(sm_scale), w, n_slots)
    if rc != 0:
        raise ValueError("orc_estimate_weights failed")
    return w[:, :n_slots].copy()


def topp_select(w: np.ndarray, valid: np.ndarray, p: float, cand_pages=None,
                page_size: int = 16):
    """w: [G, n_slots] fp64; valid: [n_slots] bool -> (kept token ids ascending, tau)."""
    w = np.ascontiguousarray(w, np.float64)
    G, n_slots = w.shape
    valid = np.ascontiguousarray(valid, np.uint8)
    kept = np.zeros(max(n_slots, 1), np.int32)
    tau = ctypes.c_double(0.0)
    if cand_pages is None:
        cp, ncp = None, 0
    else:
        cand_pages = np.ascontiguousarray(cand_pages, np.int32)
        cp, ncp = cand_pages.ctypes.data, cand_pages.shape[0]
    m = lib().orc_topp_select(w, valid, G, n_slots, float(np.float32(p)), cp, ncp, page_size,
                              kept, ctypes.byref(tau))
    if m < 0:
        raise ValueError("orc_topp_select failed")
    return kept[:m].copy(), float(tau.value)


def sparse_attention(q, k, v, kept, sm_scale):
    """q: [G, d]; k, v: [n, d] fp16; kept: token ids -> out [G, d] fp64."""
    q = _bits(q)
    k = _bits(k)
    v = _bits(v)
    G, d = q.shape
    kept = np.ascontiguousarray(kept, np.int32)
    if kept.size == 0:
        kept = np.zeros(1, np.int32)
        nk = 0
    else:
        nk = kept.shape[0]
    out = np.zeros((G, d), np.float64)
    rc = lib().orc_sparse_attention(q, G, d, k, v, k.shape[0], kept, nk, float(sm_scale), out)
    if rc != 0:
        raise ValueError("orc_sparse_attention failed")
    return out


def half_to_double(bits: int) -> float:
    return lib().orc_half_to_double(bits)


def nearest_half_of_ratio(num: float, den: int) -> int:
    return int(lib().orc_nearest_half_of_ratio(num, den))


def run_unit(q_group, k, v, budget, p, sm_scale, page_size: int = 16,
             headwise: bool = False, key_bits: int = 4):
    """Whole hot path for one (sequence, KV head) unit, stage by stage.

    q_group: [G, d] fp16 (the query heads sharing the KV head); k, v: [n, d] fp16 logical
    order; budget: Quest pages, or None when every token is a candidate. Returns a dict of
    every stage's output: codes/scale/zero, lo/hi, sel (ascending pages or None), weights
    [G, n_slots], valid [n_slots], kept (ascending token ids), tau, out [G, d] fp64.

    headwise: top-p per query head instead of per group (the pages name the group-wise
    budget under GQA as a limitation, atlas.scime.ai "Limitations"). Each head's kept set is
    orc_topp_select with G = 1 on that head's own weights, over the same Quest candidates,
    and its output is attention over its own kept set; kept is then a list of G arrays and
    tau a list of G floats.

    key_bits: 4, or 2 for the estimate from the 2-bit key cache (the pages' ablation).
    """
    n = k.shape[0]
    codes, scale, zero = quantize_keys(k, key_bits)
    res = {"codes": codes, "scale": scale, "zero": zero}
    P = -(-n // page_size)
    if budget is None:
        sel = None
        n_slots = P * page_size
        valid = np.arange(n_slots) < n
    else:
        lo, hi = page_bounds(k, page_size)
        res["lo"], res["hi"] = lo, hi
        sel = quest_select(q_group, lo, hi, budget) if P else np.zeros(0, np.int32)
        n_slots = budget * page_size
        tok = (np.repeat(sel.astype(np.int64), page_size) * page_size +
               np.tile(np.arange(page_size), len(sel)))
        valid = np.zeros(n_slots, bool)
        valid[:tok.size] = tok < n
    res["sel"] = sel
    res["valid"] = valid
    w = estimate_weights(q_group, codes, scale, zero, n, sel, n_slots, sm_scale, page_size)
    res["weights"] = w
    if headwise:
        per = [topp_select(w[h:h + 1], valid, p, sel, page_size) for h in range(w.shape[0])]
        res["kept"] = [kept for kept, _ in per]
        res["tau"] = [tau for _, tau in per]
        res["out"] = np.concatenate([sparse_attention(q_group[h:h + 1], k, v, per[h][0], sm_scale)
                                     for h in range(w.shape[0])])
        return res
    kept, tau = topp_select(w, valid, p, sel, page_size)
    res["kept"], res["tau"] = kept, tau
    res["out"] = sparse_attention(q_group, k, v, kept, sm_scale)
    return res
