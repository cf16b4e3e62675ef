"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The whole step runs on the GPU for every (sequence, KV head) unit, and every unit is
checked stage by stage against the oracle (one unit per host thread; a unit takes the
oracle from a tenth of a second to a few seconds) and against properties that hold at any
size.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from adaptive_top_sparse_amd import workloads  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu

# (config, p, width of the estimate's key codes)
CASES = {
    "cfg2-longchat-mha-32k": (2, 0.85, 4),
    "cfg3-llama-gqa-128k": (3, 0.9, 4),
    "cfg3-llama-gqa-128k-2bit": (3, 0.9, 2),
    "cfg4-longchat-b32-ragged": (4, 0.85, 4),
    "cfg5-llama-gqa-b8-64k-p0.8": (5, 0.8, 4),
    "cfg5-llama-gqa-b8-64k-p0.9": (5, 0.9, 4),
    "cfg5-llama-gqa-b8-64k-p0.95": (5, 0.95, 4),
}

# oracle worker threads (at most the 16 host cores that go with one GPU), and units per
# batch of oracle results held at once
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))
ORACLE_BATCH = 64


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(CASES))
def test_full_size_step(name):
    from adaptive_top_sparse_amd import pipeline
    cfg, p, bits = CASES[name]
    print(f"\n[full size] {name}: generating", flush=True)
    w = workloads.make_workload(cfg)
    s = w.spec
    units = [(b, g) for b in range(s.B) for g in range(s.Hkv)]
    G = s.G
    c = pipeline.upload(w, key_bits=bits)
    c.build_caches()
    buf = pipeline.alloc_step(c)
    print(f"[full size] {name}: running the step", flush=True)
    pipeline.run_step(c, buf, p, fused=False)
    torch.cuda.synchronize()
    kept_count = buf.kept_count.cpu().numpy()
    kept = buf.kept.cpu().numpy()
    out = buf.out.cpu().numpy()
    weights = buf.weights.cpu().numpy()
    sel = buf.sel_pages.cpu().numpy() if buf.sel_pages is not None else None
    sel_count = buf.sel_count.cpu().numpy() if buf.sel_count is not None else None
    # the step as bench.py times it (the fused estimate + top-p call) gives the same kept
    # sets and outputs, bit for bit, on every unit
    fused = pipeline.alloc_step(c)
    pipeline.run_step(c, fused, p)
    torch.cuda.synchronize()
    assert np.array_equal(fused.kept_count.cpu().numpy(), kept_count)
    fk = fused.kept.cpu().numpy()
    for u in np.ndindex(kept_count.shape):
        assert np.array_equal(fk[u][:kept_count[u]], kept[u][:kept_count[u]]), u
    assert np.array_equal(fused.out.cpu().numpy().view(np.uint16), out.view(np.uint16))
    del fused, fk
    # the caches the GPU built (int4 codes, metadata, page bounds), read back whole
    codes_h = c.k_codes.cpu().numpy()
    meta_h = c.k_meta.cpu().numpy()
    mm_h = None if c.page_minmax is None else c.page_minmax.cpu().numpy()
    del c, buf
    torch.cuda.empty_cache()

    # properties of every unit
    assert np.isfinite(out.astype(np.float32)).all()
    for b in range(s.B):
        n = int(w.seq_lens[b])
        P = -(-n // 16)
        for g in range(s.Hkv):
            k = kept[b, g, :kept_count[b, g]]
            assert np.all(np.diff(k) > 0) and (k.size == 0 or (k[0] >= 0 and k[-1] < n))
            if sel is not None:
                m = int(sel_count[b, g])
                assert m == min(w.budget, P)
                pages = sel[b, g, :m]
                assert np.all(np.diff(pages) > 0)
                assert np.isin(k // 16, pages).all()
                n_slots = w.budget * 16
                toks = parity.slot_tokens(pages, n_slots, n)
            else:
                n_slots = weights.shape[2]
                toks = parity.slot_tokens(None, n_slots, n)
            # the GPU's own weights: kept mass reaches p of the total, and the smallest kept
            # weight is at least every dropped one (a threshold set)
            Wg = weights[b, g * G:(g + 1) * G].astype(np.float64).mean(0)
            valid = toks >= 0
            by_tok = dict(zip(toks[valid].tolist(), Wg[valid].tolist()))
            kept_w = np.array([by_tok[int(t)] for t in k])
            total = Wg[valid].sum()
            assert kept_w.sum() >= p * total - 1e-6 * total
            dropped = np.setdiff1d(toks[valid], k)
            if dropped.size and kept_w.size:
                assert max(by_tok[int(t)] for t in dropped) <= kept_w.min() * (1 + 1e-6)

    # stage-by-stage parity on every unit, in batches of oracle results
    print(f"[full size] {name}: oracle on all {len(units)} units ({len(w.planted)} planted), "
          f"{ORACLE_THREADS} threads", flush=True)
    sm = parity.sm_scale_for(s.d)
    for i0 in range(0, len(units), ORACLE_BATCH):
        orc = parity.oracle_units(w, p, units[i0:i0 + ORACLE_BATCH], key_bits=bits,
                                  threads=ORACLE_THREADS)
        for (b, g), res in orc.items():
            n = int(w.seq_lens[b])
            codes = parity.logical_rows(codes_h, w.page_table[b], n, g)
            meta = parity.logical_rows(meta_h, w.page_table[b], n, g)
            assert np.array_equal(parity.unpack_codes(codes, bits), res["codes"]), (b, g)
            assert np.array_equal(meta[..., 0].astype(np.float64),
                                  res["scale"].astype(np.float64)), (b, g)
            assert np.array_equal(meta[..., 1].astype(np.float64),
                                  res["zero"].astype(np.float64)), (b, g)
            if mm_h is not None:
                mm = mm_h[b, g, :-(-n // 16)]
                assert np.array_equal(mm[:, 0].astype(np.float64),
                                      res["lo"].astype(np.float64)), (b, g)
                assert np.array_equal(mm[:, 1].astype(np.float64),
                                      res["hi"].astype(np.float64)), (b, g)
            if sel is not None:
                m = int(sel_count[b, g])
                assert np.array_equal(sel[b, g, :m], res["sel"]), (b, g)
            parity.check_weights(weights[b, g * G:(g + 1) * G], res["weights"], res["valid"])
            k = kept[b, g, :kept_count[b, g]]
            parity.check_kept(k, res, p, n)
            parity.check_out(out[b, g * G:(g + 1) * G], w.q[b, g * G:(g + 1) * G], w.k[b][g],
                             w.v[b][g], k, res, sm)
        del orc
        print(f"[full size] {name}: {min(i0 + ORACLE_BATCH, len(units))} units match",
              flush=True)
    print(f"[full size] {name}: ok, kept {int(kept_count.sum())} token-heads", flush=True)
