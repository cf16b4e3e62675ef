"""GPU edge cases of the hot path, through the C ABI: empty and tiny sequences, budgets
that cover every page, p = 1, a single kept token, exact Quest ties, graph replay,
appending one token, and host-side errors that must leave the outputs untouched."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import adaptive_top_sparse_amd as twl  # noqa: E402
from adaptive_top_sparse_amd import workloads  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def _pipeline():
    from adaptive_top_sparse_amd import pipeline
    return pipeline


def _host(buf):
    return {k: (None if v is None else v.cpu().numpy().copy())
            for k, v in vars(buf).items() if k != "workspace"}


def _check_all(w, out, p):
    orc = parity.oracle_units(w, p)
    sm = parity.sm_scale_for(w.spec.d)
    G = w.spec.G
    for (b, g), res in orc.items():
        n = int(w.seq_lens[b])
        if out["sel_pages"] is not None:
            cnt = int(out["sel_count"][b, g])
            assert cnt == len(res["sel"])
            assert np.array_equal(out["sel_pages"][b, g, :cnt], res["sel"])
        parity.check_weights(out["weights"][b, g * G:(g + 1) * G], res["weights"], res["valid"])
        kc = int(out["kept_count"][b, g])
        kept = out["kept"][b, g, :kc]
        if n == 0:
            assert kc == 0
            assert np.all(out["out"][b, g * G:(g + 1) * G] == 0)
            continue
        parity.check_kept(kept, res, p, n)
        parity.check_out(out["out"][b, g * G:(g + 1) * G], w.q[b, g * G:(g + 1) * G],
                         w.k[b][g], w.v[b][g], kept, res, sm)
    return orc


@pytest.mark.parametrize("p", [0.85, 1.0])
def test_empty_short_and_fully_covered_sequences(p):
    pl = _pipeline()
    print(f"\n[edge] empty/short sequences p={p}", flush=True)
    w = workloads.make_workload(4, B=4, seq_lens=[0, 1, 37, 700], budget=8, Hq=8, Hkv=8)
    c = pl.upload(w)
    c.build_caches()
    buf = pl.alloc_step(c)
    pl.run_step(c, buf, p)
    torch.cuda.synchronize()
    out = _host(buf)
    orc = _check_all(w, out, p)
    assert int(out["sel_count"][2, 0]) == 3                 # 37 tokens -> 3 pages, all kept
    if p == 1.0:
        for (b, g), res in orc.items():
            assert int(out["kept_count"][b, g]) == min(int(w.seq_lens[b]), 8 * 16) or b == 3


def test_gqa_group_of_eight_and_d64():
    pl = _pipeline()
    print("\n[edge] G=8, d=64", flush=True)
    w = workloads.make_workload(3, n=3000, budget=40, Hq=16, Hkv=2, d=64)
    c = pl.upload(w)
    c.build_caches()
    buf = pl.alloc_step(c)
    pl.run_step(c, buf, 0.9)
    torch.cuda.synchronize()
    _check_all(w, _host(buf), 0.9)


def test_single_kept_token_returns_v_exactly():
    pl = _pipeline()
    print("\n[edge] single kept token", flush=True)
    w = workloads.make_workload(3, n=1000, budget=16)
    c = pl.upload(w)
    buf = pl.alloc_step(c)
    rng = np.random.default_rng(3)
    picks = rng.integers(0, 1000, size=(1, w.spec.Hkv))
    kept = buf.kept.cpu().numpy()
    kept[0, :, 0] = picks[0]
    buf.kept.copy_(torch.from_numpy(kept))
    buf.kept_count.fill_(1)
    stride = c.cand_stride_pages * 16
    twl.twilight_sparse_decode(c.layout(), c.q, c.k_cache, c.v_cache, buf.kept, buf.kept_count,
                               stride, pl.default_sm_scale(w.spec.d), buf.out, buf.workspace)
    torch.cuda.synchronize()
    out = buf.out.cpu().numpy()
    G = w.spec.G
    for g in range(w.spec.Hkv):
        v = w.v[0][g][picks[0, g]]
        for h in range(G):
            assert np.array_equal(out[0, g * G + h].view(np.uint16), v.view(np.uint16))


def test_exact_quest_ties_break_by_page_index():
    pl = _pipeline()
    print("\n[edge] Quest ties", flush=True)
    w = workloads.make_workload(2, n=64 * 16, budget=10, Hq=2, Hkv=2)
    # copy page 3's keys onto pages 9, 20, 40: identical bounds, identical exact scores
    for g in range(2):
        for dst in (9, 20, 40):
            w.k[0][g][dst * 16:(dst + 1) * 16] = w.k[0][g][3 * 16:4 * 16]
    c = pl.upload(w)
    c.build_caches()
    buf = pl.alloc_step(c)
    for budget in (1, 3, 10):
        c.budget = budget
        buf = pl.alloc_step(c)
        w2 = workloads.Workload(**{**vars(w), "budget": budget})
        pl.run_step(c, buf, 0.85)
        torch.cuda.synchronize()
        _check_all(w2, _host(buf), 0.85)


def test_graph_replay_matches_eager():
    pl = _pipeline()
    print("\n[edge] graph replay", flush=True)
    w = workloads.make_workload(3, n=4096, budget=64)
    c = pl.upload(w)
    c.build_caches()
    buf = pl.alloc_step(c)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        pl.run_step(c, buf, 0.9)
    torch.cuda.synchronize()
    eager = _host(buf)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pl.run_step(c, buf, 0.9)
    for i in range(3):
        buf.out.zero_()
        buf.kept.fill_(-7)
        buf.weights.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rep = _host(buf)
        for key in ("sel_pages", "sel_count", "weights", "kept_count", "tau", "out"):
            assert np.array_equal(rep[key].view(np.uint8), eager[key].view(np.uint8)), (i, key)
        kc = rep["kept_count"]
        for b in range(kc.shape[0]):
            for h in range(kc.shape[1]):
                assert np.array_equal(rep["kept"][b, h, :kc[b, h]], eager["kept"][b, h, :kc[b, h]])


def test_append_one_token_updates_codes_and_bounds():
    pl = _pipeline()
    print("\n[edge] append one token", flush=True)
    w = workloads.make_workload(2, n=16 * 20 + 3, budget=8, Hq=4, Hkv=4)
    n0 = int(w.seq_lens[0])
    c = pl.upload(w)
    c.build_caches()
    # a new token arrives at position n0 (still inside the last page)
    rng = np.random.default_rng(11)
    new_k = rng.standard_normal((4, 128)).astype(np.float16) * np.float16(3)
    kc = c.k_cache.cpu().numpy()
    phys = w.page_table[0, n0 // 16]
    kc[phys, :, n0 % 16] = new_k
    c.k_cache.copy_(torch.from_numpy(kc))
    c.seq_lens.fill_(n0 + 1)
    begin = torch.full((1,), n0, dtype=torch.int32, device="cuda")
    lay = c.layout()
    twl.twilight_quantize_keys(lay, c.k_cache, c.k_codes, c.k_meta, token_begin=begin)
    twl.quest_page_bounds(lay, c.k_cache, c.page_minmax, token_begin=begin)
    torch.cuda.synchronize()
    codes_h = c.k_codes.cpu().numpy()
    meta_h = c.k_meta.cpu().numpy()
    mm_h = c.page_minmax.cpu().numpy()
    for g in range(4):
        k_all = np.concatenate([w.k[0][g], new_k[g:g + 1]], axis=0)
        codes, scale, zero = oracle.quantize_keys(k_all)
        got = parity.unpack_codes(parity.logical_rows(codes_h, w.page_table[0], n0 + 1, g))
        assert np.array_equal(got, codes)
        meta = parity.logical_rows(meta_h, w.page_table[0], n0 + 1, g)
        assert np.array_equal(meta[..., 0].astype(np.float64), scale.astype(np.float64))
        lo, hi = oracle.page_bounds(k_all)
        P = lo.shape[0]
        mm = mm_h[0, g, :P]
        assert np.array_equal(mm[:, 0].astype(np.float64), lo.astype(np.float64))
        assert np.array_equal(mm[:, 1].astype(np.float64), hi.astype(np.float64))


def test_host_errors_enqueue_nothing():
    pl = _pipeline()
    print("\n[edge] host-side errors", flush=True)
    w = workloads.make_workload(3, n=2048, budget=32)
    c = pl.upload(w)
    c.build_caches()
    buf = pl.alloc_step(c)
    buf.out.fill_(7)
    buf.kept_count.fill_(5)
    lay = c.layout()
    small = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(twl.TwilightError) as e:
        twl.twilight_sparse_decode(lay, c.q, c.k_cache, c.v_cache, buf.kept, buf.kept_count,
                                   32 * 16, 0.088, buf.out, small)
    assert e.value.status == twl.TWL_ERR_WORKSPACE
    with pytest.raises(twl.TwilightError) as e:
        twl.twilight_topp_select(lay, buf.weights, buf.sel_pages, buf.sel_count, 32, 1.5,
                                 buf.kept, buf.kept_count, buf.tau, buf.workspace)
    assert e.value.status == twl.TWL_ERR_INVALID_ARG
    with pytest.raises(twl.TwilightError) as e:
        twl.quest_select_pages(lay, c.q, c.page_minmax, 0, buf.sel_pages, buf.sel_count,
                               buf.workspace)
    assert e.value.status == twl.TWL_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(buf.out == 7).item() and torch.all(buf.kept_count == 5).item()
