"""GPU parity of the two halves of the Quest selector, called on their own through the C ABI:
quest_page_scores against the oracle's exact page scores (bit for bit: the oracle sums the
products as integers and rounds once, and the kernel's fp64 sums are exact when no page is
order-sensitive, which the oracle also reports), and quest_top_pages against
quest_select_pages, which runs the same two halves with the scores in its workspace."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import adaptive_top_sparse_amd as twl  # noqa: E402
from adaptive_top_sparse_amd import pipeline, workloads  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    "gqa-d128": (3, dict(n=8192 + 5, budget=64)),
    "mha-d128-ragged": (4, dict(B=4, n_range=(40, 3000), budget=32)),
    "gqa8-d128": (3, dict(n=3000 + 1, budget=32, Hq=16, Hkv=2)),
    "gqa2-d64": (3, dict(n=2048 + 11, budget=16, Hq=8, Hkv=4, d=64)),
    "budget-covers-all": (2, dict(n=700, budget=64)),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_page_scores_exact_and_top_pages_match_the_combined_call(case):
    cfg, kw = CASES[case]
    print(f"\n[quest scores] {case}", flush=True)
    w = workloads.make_workload(cfg, **kw)
    c = pipeline.upload(w)
    c.build_caches()
    lay = c.layout()
    B, Hkv, G = len(w.seq_lens), w.spec.Hkv, w.spec.G
    stride = twl.quest_score_stride(c.max_pages)
    assert stride >= c.max_pages and stride % 64 == 0
    scores = torch.full((B, Hkv, stride), float("nan"), dtype=torch.float64, device="cuda")
    twl.quest_page_scores(lay, c.q, c.page_minmax, scores)
    sel = torch.full((B, Hkv, c.budget), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
    twl.quest_top_pages(lay, scores, c.budget, sel, cnt)
    buf = pipeline.alloc_step(c)
    buf.sel_pages.fill_(-7)
    pipeline.run_step(c, buf, 0.9, stages=("select",))
    torch.cuda.synchronize()
    sc = scores.cpu().numpy()
    sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
    assert np.array_equal(cnt_h, buf.sel_count.cpu().numpy())
    ref_sel = buf.sel_pages.cpu().numpy()
    for b in range(B):
        n = int(w.seq_lens[b])
        P = -(-n // 16)
        for g in range(Hkv):
            m = int(cnt_h[b, g])
            assert m == min(c.budget, P)
            assert np.array_equal(sel_h[b, g, :m], ref_sel[b, g, :m])
            lo, hi = oracle.page_bounds(w.k[b][g][:n])
            q_group = w.q[b, g * G:(g + 1) * G]
            o_sel, o_scores, sensitive = oracle.quest_select(q_group, lo, hi, c.budget,
                                                             return_scores=True)
            assert sensitive == 0, "no page of these workloads is order-sensitive"
            assert np.array_equal(sc[b, g, :P], o_scores), "page scores differ from the oracle"
            assert np.array_equal(sel_h[b, g, :m], o_sel)
