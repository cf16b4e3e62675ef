"""Device buffers and the decode step of the Twilight hot path, driven through the C ABI.

A step is the select-then-prune pipeline of the Twilight pages (atlas.scime.ai summary,
"Approach"): Quest page selection (skipped when every token is a candidate), the int4
weight estimate, top-p thresholding with compaction, and sparse decode over the kept
tokens. torch only allocates device memory here; every stage runs in libtwilight.so.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

from . import (PAGE_SIZE, make_layout, quest_page_bounds, quest_select_pages,
               quest_page_scores, quest_top_pages, quest_score_stride,
               twilight_append_keys, twilight_estimate_topp, twilight_estimate_topp_headwise,
               twilight_estimate_weights, twilight_quantize_keys,
               twilight_sparse_decode, twilight_sparse_decode_headwise, twilight_topp_select,
               twilight_topp_select_headwise, twilight_workspace_size)


def default_sm_scale(d: int) -> float:
    """The attention scale 1/sqrt(d), rounded to fp32 as the ABI receives it."""
    return float(np.float32(1.0 / math.sqrt(d)))


@dataclasses.dataclass
class DeviceCache:
    """One layer's paged caches and tables on the GPU."""
    B: int
    Hq: int
    Hkv: int
    d: int
    budget: Optional[int]
    num_phys: int
    page_table: torch.Tensor
    seq_lens: torch.Tensor
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    k_codes: torch.Tensor
    k_meta: torch.Tensor
    page_minmax: Optional[torch.Tensor]
    last_token: torch.Tensor  # seq_len - 1 (>= 0) per sequence: the newest token
    key_bits: int = 4         # width of the estimate's key codes (4, or 2)

    def layout(self):
        return make_layout(self.page_table, self.seq_lens, self.Hq, self.Hkv, self.d,
                           self.num_phys, self.key_bits)

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def cand_stride_pages(self) -> int:
        return self.budget if self.budget is not None else self.max_pages

    def append_last_token(self, stream=None) -> None:
        """Per-step cache maintenance for the newest token of every sequence (the one at
        seq_len - 1, whose K/V row the model has written): its int4 codes and its page's
        bounds."""
        twilight_append_keys(self.layout(), self.k_cache, self.last_token, self.k_codes,
                             self.k_meta, self.page_minmax, stream=stream)

    def build_caches(self, stream=None) -> None:
        """Quantize every key and compute every page's bounds (prefill-time maintenance)."""
        lay = self.layout()
        twilight_quantize_keys(lay, self.k_cache, self.k_codes, self.k_meta, stream=stream)
        if self.page_minmax is not None:
            quest_page_bounds(lay, self.k_cache, self.page_minmax, stream=stream)

    def clone(self) -> "DeviceCache":
        """A replica at distinct addresses (for cache-defeating layer rotation)."""
        rep = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            rep[f.name] = v.clone() if isinstance(v, torch.Tensor) else v
        return DeviceCache(**rep)


def upload(w, device="cuda", with_bounds: Optional[bool] = None,
           key_bits: int = 4) -> DeviceCache:
    """Copy a workloads.Workload to the GPU (caches in the paged layout) and allocate the
    int4 key cache and the page bounds it needs."""
    s = w.spec
    dev = torch.device(device)
    budget = w.budget
    if with_bounds is None:
        with_bounds = budget is not None
    k_paged = torch.from_numpy(w.paged("k")).to(dev)
    v_paged = torch.from_numpy(w.paged("v")).to(dev)
    P = w.num_phys_pages
    return DeviceCache(
        B=s.B, Hq=s.Hq, Hkv=s.Hkv, d=s.d, budget=budget, num_phys=P,
        page_table=torch.from_numpy(w.page_table).to(dev),
        seq_lens=torch.from_numpy(w.seq_lens).to(dev),
        q=torch.from_numpy(w.q).to(dev),
        k_cache=k_paged, v_cache=v_paged,
        k_codes=torch.zeros((P, s.Hkv, PAGE_SIZE, s.d * key_bits // 8), dtype=torch.uint8,
                            device=dev),
        k_meta=torch.zeros((P, s.Hkv, PAGE_SIZE, s.d // 32, 2), dtype=torch.float16, device=dev),
        page_minmax=(torch.zeros((s.B, s.Hkv, w.max_pages, 2, s.d), dtype=torch.float16,
                                 device=dev) if with_bounds else None),
        last_token=torch.from_numpy(np.maximum(w.seq_lens.astype(np.int32) - 1, 0)).to(dev),
        key_bits=key_bits)


@dataclasses.dataclass
class StepBuffers:
    """Outputs of every stage of one step, plus the shared workspace."""
    sel_pages: Optional[torch.Tensor]
    sel_count: Optional[torch.Tensor]
    weights: torch.Tensor
    kept: torch.Tensor
    kept_count: torch.Tensor
    tau: torch.Tensor
    out: torch.Tensor
    workspace: torch.Tensor


def alloc_step(c: DeviceCache, headwise: bool = False) -> StepBuffers:
    """Step outputs; with headwise, the kept lists, counts and tau are per query head."""
    dev = c.q.device
    H = c.Hq if headwise else c.Hkv
    stride = c.cand_stride_pages
    n_slots = stride * PAGE_SIZE
    ws_bytes = twilight_workspace_size(c.layout(), stride)
    if ws_bytes == 0:
        raise ValueError("layout rejected by twilight_workspace_size")
    return StepBuffers(
        sel_pages=(torch.full((c.B, c.Hkv, stride), -1, dtype=torch.int32, device=dev)
                   if c.budget is not None else None),
        sel_count=(torch.zeros((c.B, c.Hkv), dtype=torch.int32, device=dev)
                   if c.budget is not None else None),
        weights=torch.zeros((c.B, c.Hq, n_slots), dtype=torch.float32, device=dev),
        kept=torch.full((c.B, H, n_slots), -1, dtype=torch.int32, device=dev),
        kept_count=torch.zeros((c.B, H), dtype=torch.int32, device=dev),
        tau=torch.zeros((c.B, H), dtype=torch.float32, device=dev),
        out=torch.zeros((c.B, c.Hq, c.d), dtype=torch.float16, device=dev),
        # zero-filled once; the library needs no particular contents
        workspace=torch.zeros(ws_bytes, dtype=torch.uint8, device=dev))


def quest_scores_view(c: DeviceCache, buf) -> "torch.Tensor":
    """fp64 view [B, Hkv, quest_score_stride] of the start of the step's workspace."""
    stride = quest_score_stride(c.max_pages)
    n = c.B * c.Hkv * stride
    return buf.workspace[:n * 8].view(torch.float64).view(c.B, c.Hkv, stride)


def run_step(c: DeviceCache, buf: StepBuffers, p: float, sm_scale: Optional[float] = None,
             stream=None, stages=("select", "estimate", "topp", "decode"),
             append: bool = False, headwise: bool = False, fused: bool = True) -> None:
    """One decode step of the hot path on `stream` (no host synchronization). With
    append, the step first maintains the caches for each sequence's newest token; with
    headwise (buffers from alloc_step(c, headwise=True)), top-p and decode keep one set per
    query head instead of one per KV head. With fused (the default), a step that runs both
    the estimate and top-p makes the single call that lets top-p normalise the estimate's
    logits itself; buf.weights then holds scratch, not the normalised weights."""
    if sm_scale is None:
        sm_scale = default_sm_scale(c.d)
    if append:
        c.append_last_token(stream=stream)
    lay = c.layout()
    stride = c.cand_stride_pages
    if c.budget is not None and "select" in stages:
        quest_select_pages(lay, c.q, c.page_minmax, c.budget, buf.sel_pages, buf.sel_count,
                           buf.workspace, stream=stream)
    if c.budget is not None and ("quest_scores" in stages or "quest_top" in stages):
        # the same two halves as separate calls, with the scores where the combined call
        # keeps them: the start of the workspace
        scores = quest_scores_view(c, buf)
        if "quest_scores" in stages:
            quest_page_scores(lay, c.q, c.page_minmax, scores, stream=stream)
        if "quest_top" in stages:
            quest_top_pages(lay, scores, c.budget, buf.sel_pages, buf.sel_count, stream=stream)
    cand_pages = buf.sel_pages if c.budget is not None else None
    cand_count = buf.sel_count if c.budget is not None else None
    topp = twilight_topp_select_headwise if headwise else twilight_topp_select
    decode = twilight_sparse_decode_headwise if headwise else twilight_sparse_decode
    if fused and "estimate" in stages and "topp" in stages:
        both = twilight_estimate_topp_headwise if headwise else twilight_estimate_topp
        both(lay, c.q, c.k_codes, c.k_meta, cand_pages, cand_count, stride, sm_scale, p,
             buf.weights, buf.kept, buf.kept_count, buf.tau, buf.workspace, stream=stream)
    else:
        if "estimate" in stages:
            twilight_estimate_weights(lay, c.q, c.k_codes, c.k_meta, cand_pages, cand_count,
                                      stride, sm_scale, buf.weights, buf.workspace,
                                      stream=stream)
        if "topp" in stages:
            topp(lay, buf.weights, cand_pages, cand_count, stride, p, buf.kept, buf.kept_count,
                 buf.tau, buf.workspace, stream=stream)
    if "decode" in stages:
        decode(lay, c.q, c.k_cache, c.v_cache, buf.kept, buf.kept_count, stride * PAGE_SIZE,
               sm_scale, buf.out, buf.workspace, stream=stream)


def baseline_kept(c: DeviceCache, buf: StepBuffers, mode: str):
    """Kept-token lists for the comparison steps that run on the same decode kernel:
    "dense" keeps every token of each sequence, "quest" every token of the pages the Quest
    selector chose in `buf` (a step must have run). Returns (kept [B, Hkv, stride] int32,
    kept_count [B, Hkv] int32, stride); tokens at or past a sequence's end are skipped by the
    decode itself."""
    dev = c.q.device
    if mode == "dense":
        stride = c.max_pages * PAGE_SIZE
        kept = torch.arange(stride, dtype=torch.int32, device=dev).expand(c.B, c.Hkv, stride)
        count = c.seq_lens.clamp(min=0).to(torch.int32)[:, None].expand(c.B, c.Hkv)
    elif mode == "quest":
        if c.budget is None:
            raise ValueError("the Quest-only list needs a Quest budget")
        stride = c.budget * PAGE_SIZE
        offs = torch.arange(PAGE_SIZE, dtype=torch.int32, device=dev)
        kept = (buf.sel_pages[..., None] * PAGE_SIZE + offs).reshape(c.B, c.Hkv, stride)
        count = buf.sel_count * PAGE_SIZE
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return kept.contiguous(), count.contiguous(), stride
