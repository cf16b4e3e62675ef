"""Seeded synthetic decode workloads for Twilight-style sparse decode.

This module only draws inputs and moves them between layouts. It holds none of the
method's arithmetic (no quantization, no scores, no softmax, no thresholds), so both the
fp64 oracle and the HIP path may consume what it produces.

Shapes and structure follow the five workloads the method is evaluated on (the
Twilight pages, atlas.scime.ai "Experimental setup" and "Key results": Longchat-7B-v1.5-32k
MHA layers, LLaMA-3.1-8B GQA layers at 128k context, batched decode), with planted
heavy-hitter keys standing in for the real attention structure of those models, since no
dataset or trained weight is available.

Recipe (all draws from ``numpy.random.default_rng(seed)``, PCG64):
  1. q ~ N(0,1) float32, shape [B, Hq, d], cast once to fp16 (RNE).
  2. For each sequence b in order: K_b then V_b ~ N(0,1) float32, shape [Hkv, n_b, d].
  3. For each sequence b in order: planted tokens for each KV head that carries them
     (``rng.choice`` without replacement), and key += gain * direction in float32, where
     direction is q_h / |q_h| (MHA) or unit(sum_{h in group} q_h / |q_h|) (GQA), both taken
     from the fp16 query.
  4. K_b and V_b are cast once to fp16 (RNE).
  5. Physical pages are a seeded permutation of all pages of the batch, so the page table
     is never the identity.
Tail slots of a partial last page hold a poison value (1024.0) that would visibly corrupt
any result that read them.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

PAGE_SIZE = 16
POISON = np.float16(1024.0)
BASE_SEED = 20250204


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    """One decode-layer workload.

    base: "quest" (page selector with ``budget`` pages per KV head) or None (every token is
    a candidate). plant: (kind, fraction, gain, heads_fraction, sinks) where kind is "mha"
    (per query head, direction q_h) or "gqa" (per KV head, direction the group mean).
    """
    cfg_id: int
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    n: Optional[int]                  # fixed length, or None for ragged
    n_range: Optional[tuple]          # (lo, hi) inclusive for ragged lengths
    base: Optional[str]
    budget: Optional[int]
    ps: tuple                         # top-p values
    plant_kind: Optional[str]
    plant_frac: float
    plant_gain: float
    plant_heads_frac: float           # fraction of KV heads (per sequence) that carry plants
    sinks: int                        # leading tokens that always carry a plant

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


SPECS = {
    1: WorkloadSpec(1, "tiny-1head-d64-n1k", 1, 1, 1, 64, 1024, None, None, None, (0.9,),
                    None, 0.0, 0.0, 0.0, 0),
    2: WorkloadSpec(2, "longchat7b-mha-n32k", 1, 32, 32, 128, 32768, None, "quest", 256,
                    (0.85,), "mha", 0.01, 4.0, 1.0, 4),
    3: WorkloadSpec(3, "llama31-8b-gqa-n128k", 1, 32, 8, 128, 131072, None, "quest", 512,
                    (0.9,), "gqa", 0.001, 6.0, 0.5, 0),
    4: WorkloadSpec(4, "longchat7b-mha-b32-ragged", 32, 32, 32, 128, None, (4096, 32768),
                    "quest", 256, (0.85,), "mha", 0.01, 4.0, 1.0, 0),
    5: WorkloadSpec(5, "llama31-8b-gqa-b8-n64k-full", 8, 32, 8, 128, 65536, None, None, None,
                    (0.8, 0.9, 0.95), "gqa", 0.005, 5.0, 0.6, 0),
}


@dataclasses.dataclass
class Workload:
    spec: WorkloadSpec
    seed: int
    q: np.ndarray                     # [B, Hq, d] fp16
    k: List[np.ndarray]               # per sequence [Hkv, n_b, d] fp16 (logical order)
    v: List[np.ndarray]               # per sequence [Hkv, n_b, d] fp16
    seq_lens: np.ndarray              # [B] int32
    page_table: np.ndarray            # [B, max_pages] int32 physical page ids (0 past the end)
    num_phys_pages: int
    budget: Optional[int]             # Quest pages per KV head (None: no selector)
    planted: dict                     # (b, kv_head) -> sorted planted token ids

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    def pages_of(self, b: int) -> int:
        return int(math.ceil(int(self.seq_lens[b]) / PAGE_SIZE))

    def paged(self, which: str) -> np.ndarray:
        """Scatter K or V into the paged cache layout [num_phys_pages, Hkv, 16, d] fp16."""
        src = self.k if which == "k" else self.v
        s = self.spec
        out = np.full((self.num_phys_pages, s.Hkv, PAGE_SIZE, s.d), POISON, dtype=np.float16)
        for b in range(s.B):
            n_b = int(self.seq_lens[b])
            P = self.pages_of(b)
            if P == 0:
                continue
            pad = P * PAGE_SIZE - n_b
            x = src[b]
            if pad:
                x = np.concatenate(
                    [x, np.full((s.Hkv, pad, s.d), POISON, dtype=np.float16)], axis=1)
            # [Hkv, P, 16, d] -> [P, Hkv, 16, d]
            x = x.reshape(s.Hkv, P, PAGE_SIZE, s.d).transpose(1, 0, 2, 3)
            out[self.page_table[b, :P]] = x
        return out


def _unit(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float64)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make_workload(cfg_id: int, *, n: Optional[int] = None, B: Optional[int] = None,
                  n_range: Optional[tuple] = None, budget: Optional[int] = None,
                  seed: Optional[int] = None, Hq: Optional[int] = None,
                  Hkv: Optional[int] = None, d: Optional[int] = None,
                  seq_lens: Optional[List[int]] = None) -> Workload:
    """Draw one workload. Keyword overrides shrink a configuration for fast parity runs
    while keeping its structure (head layout, planting recipe, paging)."""
    s = SPECS[cfg_id]
    over = {}
    if n is not None:
        over["n"] = n
        over["n_range"] = None
    if n_range is not None:
        over["n_range"] = n_range
        over["n"] = None
    for key, val in (("B", B), ("budget", budget), ("Hq", Hq), ("Hkv", Hkv), ("d", d)):
        if val is not None:
            over[key] = val
    if over:
        s = dataclasses.replace(s, **over)
    if s.Hq % s.Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    seed = BASE_SEED + cfg_id if seed is None else seed
    rng = np.random.default_rng(seed)

    q = rng.standard_normal((s.B, s.Hq, s.d), dtype=np.float32).astype(np.float16)
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int64)
        assert lens.shape == (s.B,)
    elif s.n is not None:
        lens = np.full(s.B, s.n, dtype=np.int64)
    else:
        lo, hi = s.n_range
        lens = rng.integers(lo, hi + 1, size=s.B)

    ks, vs = [], []
    for b in range(s.B):
        n_b = int(max(lens[b], 0))
        ks.append(rng.standard_normal((s.Hkv, n_b, s.d), dtype=np.float32))
        vs.append(rng.standard_normal((s.Hkv, n_b, s.d), dtype=np.float32))

    planted = {}
    G = s.Hq // s.Hkv
    if s.plant_kind is not None:
        qhat = _unit(q.astype(np.float32))                       # [B, Hq, d] fp64
        for b in range(s.B):
            n_b = int(max(lens[b], 0))
            if n_b == 0:
                continue
            n_heads_planted = int(round(s.plant_heads_frac * s.Hkv))
            if n_heads_planted >= s.Hkv:
                heads = np.arange(s.Hkv)
            else:
                heads = np.sort(rng.choice(s.Hkv, size=n_heads_planted, replace=False))
            m = int(round(s.plant_frac * n_b))
            for g in heads:
                g = int(g)
                toks = rng.choice(n_b, size=min(m, n_b), replace=False)
                if s.sinks:
                    toks = np.union1d(toks, np.arange(min(s.sinks, n_b)))
                toks = np.sort(toks)
                if s.plant_kind == "mha":
                    direction = qhat[b, g]
                else:
                    direction = _unit(qhat[b, g * G:(g + 1) * G].sum(axis=0))
                ks[b][g, toks, :] += (s.plant_gain * direction).astype(np.float32)
                planted[(b, g)] = toks
    ks = [x.astype(np.float16) for x in ks]
    vs = [x.astype(np.float16) for x in vs]

    pages = [int(math.ceil(int(max(L, 0)) / PAGE_SIZE)) for L in lens]
    total = int(sum(pages))
    perm = rng.permutation(total).astype(np.int32) if total else np.zeros(0, np.int32)
    max_pages = max(1, max(pages) if pages else 1)
    if s.n_range is not None:
        max_pages = max(max_pages, int(math.ceil(s.n_range[1] / PAGE_SIZE)))
    table = np.zeros((s.B, max_pages), dtype=np.int32)
    off = 0
    for b, P in enumerate(pages):
        table[b, :P] = perm[off:off + P]
        off += P
    return Workload(spec=s, seed=seed, q=q, k=ks, v=vs,
                    seq_lens=np.asarray(lens, dtype=np.int32), page_table=table,
                    num_phys_pages=max(total, 1), budget=s.budget if s.base else None,
                    planted=planted)
