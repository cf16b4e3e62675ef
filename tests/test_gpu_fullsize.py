"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The whole step runs on the GPU for every (sequence, KV head) unit; sampled units are checked
stage by stage against the oracle (which finishes one unit in seconds), and every unit is
checked against properties that hold at any size.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from adaptive_top_sparse_amd import workloads  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu

# (config, p); the units checked against the oracle are chosen by sampled_units
CASES = {
    "cfg2-longchat-mha-32k": (2, 0.85),
    "cfg3-llama-gqa-128k": (3, 0.9),
    "cfg4-longchat-b32-ragged": (4, 0.85),
    "cfg5-llama-gqa-b8-64k-p0.8": (5, 0.8),
    "cfg5-llama-gqa-b8-64k-p0.9": (5, 0.9),
    "cfg5-llama-gqa-b8-64k-p0.95": (5, 0.95),
}


def sampled_units(w, n_units=4):
    """(sequence, KV head) units for the oracle: half with planted heavy keys and half
    without when the workload has both, spread over the batch (the shortest and the longest
    sequence among them when lengths differ), seeded."""
    s = w.spec
    rng = np.random.default_rng(11 + s.cfg_id)
    planted = sorted(w.planted)
    plain = sorted((b, g) for b in range(s.B) for g in range(s.Hkv)
                   if (b, g) not in w.planted and int(w.seq_lens[b]) > 0)
    if not planted or not plain:
        pool = planted or plain
        lens = np.array([int(w.seq_lens[b]) for b, _ in pool])
        pick = {int(np.argmin(lens)), int(np.argmax(lens))}
        rest = [i for i in rng.permutation(len(pool)) if i not in pick]
        pick.update(int(i) for i in rest[:n_units - len(pick)])
        return [pool[i] for i in sorted(pick)]
    half = n_units // 2
    a = [planted[i] for i in sorted(rng.choice(len(planted), half, replace=False))]
    c = [plain[i] for i in sorted(rng.choice(len(plain), n_units - half, replace=False))]
    return a + c


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(CASES))
def test_full_size_step(name):
    from adaptive_top_sparse_amd import pipeline
    cfg, p = CASES[name]
    print(f"\n[full size] {name}: generating", flush=True)
    w = workloads.make_workload(cfg)
    units = sampled_units(w)
    s = w.spec
    G = s.G
    c = pipeline.upload(w)
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
    # the sampled units' cache rows (int4 codes, metadata, page bounds), gathered on the GPU
    cache_rows = {}
    for b, g in units:
        n = int(w.seq_lens[b])
        pages = torch.from_numpy(w.page_table[b, :-(-n // 16)].astype(np.int64)).cuda()
        cache_rows[(b, g)] = (
            c.k_codes[pages, g].cpu().numpy().reshape(-1, s.d // 2)[:n],
            c.k_meta[pages, g].cpu().numpy().reshape(-1, s.d // 32, 2)[:n],
            None if c.page_minmax is None else c.page_minmax[b, g, :pages.numel()].cpu().numpy())
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

    # stage-by-stage parity on sampled units
    print(f"[full size] {name}: oracle on {units} (planted: "
          f"{[u for u in units if u in w.planted]})", flush=True)
    orc = parity.oracle_units(w, p, units)
    sm = parity.sm_scale_for(s.d)
    for (b, g), res in orc.items():
        n = int(w.seq_lens[b])
        codes, meta, mm = cache_rows[(b, g)]
        assert np.array_equal(parity.unpack_codes(codes), res["codes"]), (b, g)
        assert np.array_equal(meta[..., 0].astype(np.float64), res["scale"].astype(np.float64))
        assert np.array_equal(meta[..., 1].astype(np.float64), res["zero"].astype(np.float64))
        if mm is not None:
            assert np.array_equal(mm[:, 0].astype(np.float64), res["lo"].astype(np.float64))
            assert np.array_equal(mm[:, 1].astype(np.float64), res["hi"].astype(np.float64))
        if sel is not None:
            m = int(sel_count[b, g])
            assert np.array_equal(sel[b, g, :m], res["sel"]), (b, g)
        parity.check_weights(weights[b, g * G:(g + 1) * G], res["weights"], res["valid"])
        k = kept[b, g, :kept_count[b, g]]
        parity.check_kept(k, res, p, n)
        parity.check_out(out[b, g * G:(g + 1) * G], w.q[b, g * G:(g + 1) * G], w.k[b][g],
                         w.v[b][g], k, res, sm)
    print(f"[full size] {name}: ok, kept {int(kept_count.sum())} token-heads", flush=True)
