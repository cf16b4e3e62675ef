"""The comparison steps on the same decode kernel: dense (every token) and Quest-only (every
token of the selected pages), through the C ABI, against the oracle's attention over the
same token sets."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import adaptive_top_sparse_amd as twl  # noqa: E402
from adaptive_top_sparse_amd import workloads  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    "cfg3s": (3, dict(n=4096 + 11, budget=64), 0.9),
    "cfg2s": (2, dict(n=2048 + 5, budget=32), 0.85),
    "cfg4s": (4, dict(B=3, n_range=(40, 3000), budget=32), 0.85),
    "cfg1": (1, {}, 0.9),
}


@pytest.mark.parametrize("name", list(CASES))
def test_dense_and_quest_only_decode_match_the_oracle(name):
    from adaptive_top_sparse_amd import pipeline
    cfg, over, p = CASES[name]
    print(f"\n[baselines] {name} cfg={cfg} {over}", flush=True)
    w = workloads.make_workload(cfg, **over)
    c = pipeline.upload(w)
    c.build_caches()
    buf = pipeline.alloc_step(c)
    pipeline.run_step(c, buf, p)
    sm = parity.sm_scale_for(w.spec.d)
    G = w.spec.G
    modes = ["dense"] + (["quest"] if c.budget is not None else [])
    for mode in modes:
        kept, count, stride = pipeline.baseline_kept(c, buf, mode)
        ws = torch.zeros(twl.twilight_workspace_size(c.layout(), stride // twl.PAGE_SIZE),
                         dtype=torch.uint8, device="cuda")
        out = torch.zeros_like(buf.out)
        twl.twilight_sparse_decode(c.layout(), c.q, c.k_cache, c.v_cache, kept, count, stride,
                                   sm, out, ws)
        torch.cuda.synchronize()
        o = out.cpu().numpy().astype(np.float64)
        kept_h = kept.cpu().numpy()
        count_h = count.cpu().numpy()
        for b in range(w.spec.B):
            n = int(w.seq_lens[b])
            for g in range(w.spec.Hkv):
                toks = kept_h[b, g, :count_h[b, g]]
                toks = toks[(toks >= 0) & (toks < n)]
                if mode == "dense":
                    assert np.array_equal(toks, np.arange(n))
                want = oracle.sparse_attention(w.q[b, g * G:(g + 1) * G], w.k[b][g], w.v[b][g],
                                               toks, sm)
                err = float(np.abs(o[b, g * G:(g + 1) * G] - want).max())
                assert err <= parity.OUT_ATOL, (mode, b, g, err)
