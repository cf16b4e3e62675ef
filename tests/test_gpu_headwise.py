"""GPU parity of head-wise top-p under GQA (one kept set per query head; the pages name the
group-wise budget as a limitation of GQA, atlas.scime.ai "Limitations"), through the C ABI.

Quest and the weight estimate are shared with the group-wise step; top-p and decode run per
query head. Each head's kept set and output are checked against the oracle, whose head-wise
form is its top-p with G = 1 on that head's weights; with G = 1 the two modes coincide.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from adaptive_top_sparse_amd import workloads  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    "cfg3s-g4": (3, dict(n=8192 + 5, budget=64), 0.9),
    "cfg3s-g8": (3, dict(n=3000 + 1, budget=32, Hq=16, Hkv=2), 0.85),
    "cfg3s-g2-ragged": (3, dict(B=3, seq_lens=[2000 + 3, 17, 700], budget=16, Hq=4, Hkv=2),
                        0.95),
    "cfg5s-g4": (5, dict(B=2, n=4096), 0.9),
    "cfg5-n40k-g4": (5, dict(B=1, n=40000 + 3), 0.9),
    "cfg2s-mha": (2, dict(n=2048 + 7, budget=32), 0.85),
}


def _host(buf):
    return {k: (None if v is None else v.cpu().numpy().copy())
            for k, v in vars(buf).items() if k != "workspace"}


def _steps(w, p):
    from adaptive_top_sparse_amd import pipeline
    c = pipeline.upload(w)
    c.build_caches()
    group = pipeline.alloc_step(c)
    head = pipeline.alloc_step(c, headwise=True)
    head_sep = pipeline.alloc_step(c, headwise=True)
    pipeline.run_step(c, group, p, fused=False)
    pipeline.run_step(c, head, p, headwise=True)
    pipeline.run_step(c, head_sep, p, headwise=True, fused=False)
    torch.cuda.synchronize()
    hw, sep = _host(head), _host(head_sep)
    # the fused head-wise call (top-p normalising for itself) equals the separate calls
    for key in ("kept_count", "tau", "out"):
        assert np.array_equal(hw[key].view(np.uint8), sep[key].view(np.uint8)), key
    for u in np.ndindex(hw["kept_count"].shape):
        k = int(hw["kept_count"][u])
        assert np.array_equal(hw["kept"][u][:k], sep["kept"][u][:k]), u
    return _host(group), sep


@pytest.mark.parametrize("name", list(CASES))
def test_headwise_step_matches_oracle(name):
    cfg, over, p = CASES[name]
    print(f"\n[headwise] {name} cfg={cfg} {over} p={p}", flush=True)
    w = workloads.make_workload(cfg, **over)
    s = w.spec
    G = s.G
    grp, hw = _steps(w, p)
    # the stages before top-p are the group-wise ones
    for key in ("sel_pages", "sel_count", "weights"):
        if grp[key] is not None:
            assert np.array_equal(grp[key], hw[key]), key
    assert hw["kept_count"].shape == (s.B, s.Hq)
    if G == 1:
        for key in ("kept_count", "tau", "out"):
            assert np.array_equal(grp[key].view(np.uint8), hw[key].view(np.uint8)), key
        for b in range(s.B):
            for h in range(s.Hq):
                c = int(hw["kept_count"][b, h])
                assert np.array_equal(grp["kept"][b, h, :c], hw["kept"][b, h, :c])
    orc = parity.oracle_units(w, p, headwise=True)
    sm = parity.sm_scale_for(s.d)
    n_head, n_group = 0, 0
    for (b, g), res in orc.items():
        n = int(w.seq_lens[b])
        n_group += int(grp["kept_count"][b, g]) * G
        for j in range(G):
            h = g * G + j
            kc = int(hw["kept_count"][b, h])
            n_head += kc
            kept = hw["kept"][b, h, :kc]
            rv = parity.head_view(res, j)
            if n == 0:
                assert kc == 0 and np.all(hw["out"][b, h] == 0)
                continue
            parity.check_kept(kept, rv, p, n)
            parity.check_out(hw["out"][b, h:h + 1], w.q[b, h:h + 1], w.k[b][g], w.v[b][g],
                             kept, rv, sm)
    print(f"[headwise] {name}: kept token-heads head-wise {n_head}, group-wise {n_group}",
          flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", [3, 5])
def test_headwise_full_size(cfg):
    """The 128k GQA step (Quest base) and the B = 8, 64k full-attention step at full size,
    head-wise: every query head's kept set and output against the oracle."""
    from adaptive_top_sparse_amd import pipeline
    p = 0.9
    w = workloads.make_workload(cfg)
    s = w.spec
    G = s.G
    print(f"\n[headwise] {s.name} full size", flush=True)
    units = [(b, g) for b in range(s.B) for g in range(s.Hkv)]
    c = pipeline.upload(w)
    c.build_caches()
    buf = pipeline.alloc_step(c, headwise=True)
    pipeline.run_step(c, buf, p, headwise=True, fused=False)
    torch.cuda.synchronize()
    out = _host(buf)
    del c, buf
    torch.cuda.empty_cache()
    # every head, at any size: kept ids are candidates, ascending, and carry p of the mass
    for b in range(s.B):
        n = int(w.seq_lens[b])
        for h in range(s.Hq):
            g = h // G
            k = out["kept"][b, h, :out["kept_count"][b, h]]
            if out["sel_pages"] is not None:
                pages = out["sel_pages"][b, g, :out["sel_count"][b, g]]
                toks = parity.slot_tokens(pages, w.budget * 16, n)
            else:
                toks = parity.slot_tokens(None, out["weights"].shape[2], n)
            assert np.all(np.diff(k) > 0) and np.isin(k, toks[toks >= 0]).all()
            W = out["weights"][b, h].astype(np.float64)
            by_tok = dict(zip(toks[toks >= 0].tolist(), W[toks >= 0].tolist()))
            total = sum(by_tok.values())
            kept_w = np.array([by_tok[int(t)] for t in k])
            assert kept_w.sum() >= p * total - 1e-6 * total
            dropped = np.setdiff1d(toks[toks >= 0], k)
            if dropped.size and kept_w.size:
                assert max(by_tok[int(t)] for t in dropped) <= kept_w.min() * (1 + 1e-6)
    print(f"[headwise] {s.name}: oracle on all {len(units)} units", flush=True)
    orc = parity.oracle_units(w, p, units, headwise=True,
                              threads=max(1, min(16, os.cpu_count() or 1)))
    sm = parity.sm_scale_for(s.d)
    for (b, g), res in orc.items():
        n = int(w.seq_lens[b])
        if out["sel_pages"] is not None:
            assert np.array_equal(out["sel_pages"][b, g, :out["sel_count"][b, g]], res["sel"])
        parity.check_weights(out["weights"][b, g * G:(g + 1) * G], res["weights"], res["valid"])
        for j in range(G):
            h = g * G + j
            kept = out["kept"][b, h, :out["kept_count"][b, h]]
            rv = parity.head_view(res, j)
            parity.check_kept(kept, rv, p, n)
            parity.check_out(out["out"][b, h:h + 1], w.q[b, h:h + 1], w.k[b][g], w.v[b][g],
                             kept, rv, sm)
    print(f"[headwise] {s.name}: ok", flush=True)
