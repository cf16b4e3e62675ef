"""GPU parity: every stage of the HIP path against the fp64 oracle, through the C ABI.

Small versions of the five workloads (same head layout, planting recipe and paging, shorter
contexts and ragged tails) are checked unit by unit and stage by stage; the acceptance
rules are in tests/parity.py. Full-size runs live in test_gpu_fullsize.py.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from adaptive_top_sparse_amd import workloads  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = {
    "cfg1": (1, {}, 0.9),
    "cfg2s": (2, dict(n=2048 + 7, budget=32), 0.85),
    "cfg3s": (3, dict(n=8192 + 5, budget=64), 0.9),
    "cfg4s": (4, dict(B=4, n_range=(40, 3000), budget=32), 0.85),
    "cfg5s-p0.8": (5, dict(B=2, n=4096), 0.8),
    "cfg5s-p0.9": (5, dict(B=2, n=4096), 0.9),
    "cfg5s-p0.95": (5, dict(B=2, n=4096), 0.95),
    # group means formed by the wide pass, then 16 slots per thread in VGPRs
    "cfg5-n16k": (5, dict(B=1, n=16384 + 9), 0.9),
    # units above 32768 slots keep half of W in LDS: GQA (wide pass) and MHA (direct)
    "cfg5-n40k": (5, dict(B=1, n=40000 + 3), 0.9),
    "cfg5-n40k-mha": (5, dict(B=1, n=40000 + 3, Hq=4, Hkv=4), 0.9),
    # long enough that the estimate takes 64-page chunks (four batches per wave: the
    # steady-state loop, then the two peeled batches; the ragged last chunk three) and the
    # decode 512-token chunks (up to eight batches each)
    "cfg5-b2-n40k": (5, dict(B=2, n=2536 * 16 - 5), 0.9),
    # the 2-bit key cache of the pages' ablation: every head dim, group size and selector
    "cfg1-2bit": (1, {}, 0.9, 2),
    "cfg3s-2bit": (3, dict(n=8192 + 5, budget=64), 0.9, 2),
    "cfg3s-2bit-g8": (3, dict(n=3000 + 1, budget=32, Hq=16, Hkv=2), 0.85, 2),
    "cfg4s-2bit": (4, dict(B=4, n_range=(40, 3000), budget=32), 0.85, 2),
    "cfg5s-2bit-g2-d64": (5, dict(B=2, n=4096 + 11, Hq=8, Hkv=4, d=64), 0.9, 2),
}


# the cases whose workload has a Quest page selector (the others build no page bounds)
QUEST_CASES = [k for k, (cfg, *_) in CASES.items() if workloads.SPECS[cfg].base is not None]


def _run(w, p, repeat=1, key_bits=4):
    """Run i uses the separate estimate and top-p calls (so that the normalised weights
    can be checked) when i is even, the single fused call when i is odd."""
    from adaptive_top_sparse_amd import pipeline
    c = pipeline.upload(w, key_bits=key_bits)
    c.build_caches()
    buf = pipeline.alloc_step(c)
    outs = []
    for i in range(repeat):
        pipeline.run_step(c, buf, p, fused=(i % 2 == 1))
        torch.cuda.synchronize()
        outs.append({k: (None if v is None else v.cpu().numpy().copy())
                     for k, v in vars(buf).items() if k != "workspace"})
    host = {
        "k_codes": c.k_codes.cpu().numpy(),
        "k_meta": c.k_meta.cpu().numpy(),
        "page_minmax": None if c.page_minmax is None else c.page_minmax.cpu().numpy(),
    }
    return c, host, outs


@pytest.fixture(scope="module", params=list(CASES))
def case(request):
    cfg, over, p, *rest = CASES[request.param]
    bits = rest[0] if rest else 4
    print(f"\n[parity case] {request.param} cfg={cfg} {over} p={p} key_bits={bits}", flush=True)
    w = workloads.make_workload(cfg, **over)
    c, host, outs = _run(w, p, repeat=2, key_bits=bits)
    orc = parity.oracle_units(w, p, key_bits=bits)
    return dict(name=request.param, w=w, p=p, host=host, out=outs[0], out2=outs[1], orc=orc,
                bits=bits)


def test_quantized_keys_bit_exact(case):
    w, host, orc = case["w"], case["host"], case["orc"]
    for (b, g), res in orc.items():
        n = int(w.seq_lens[b])
        if n == 0:
            continue
        codes = parity.unpack_codes(parity.logical_rows(host["k_codes"], w.page_table[b], n, g),
                                    case["bits"])
        assert np.array_equal(codes, res["codes"]), (b, g)
        meta = parity.logical_rows(host["k_meta"], w.page_table[b], n, g)
        assert np.array_equal(meta[..., 0].astype(np.float64), res["scale"].astype(np.float64))
        assert np.array_equal(meta[..., 1].astype(np.float64), res["zero"].astype(np.float64))


@pytest.mark.parametrize("case", QUEST_CASES, indirect=True)
def test_page_bounds_bit_exact(case):
    w, host, orc = case["w"], case["host"], case["orc"]
    assert host["page_minmax"] is not None
    for (b, g), res in orc.items():
        n = int(w.seq_lens[b])
        P = -(-n // 16)
        mm = host["page_minmax"][b, g, :P]                         # [P, 2, d]
        assert np.array_equal(mm[:, 0].astype(np.float64), res["lo"].astype(np.float64)), (b, g)
        assert np.array_equal(mm[:, 1].astype(np.float64), res["hi"].astype(np.float64)), (b, g)


@pytest.mark.parametrize("case", QUEST_CASES, indirect=True)
def test_quest_pages_bit_exact(case):
    w, out, orc = case["w"], case["out"], case["orc"]
    assert out["sel_pages"] is not None
    for (b, g), res in orc.items():
        cnt = int(out["sel_count"][b, g])
        assert cnt == len(res["sel"]), (b, g)
        assert np.array_equal(out["sel_pages"][b, g, :cnt], res["sel"]), (b, g)


def test_estimated_weights(case):
    w, out, orc = case["w"], case["out"], case["orc"]
    G = w.spec.G
    worst = 0.0
    for (b, g), res in orc.items():
        wg = out["weights"][b, g * G:(g + 1) * G]
        worst = max(worst, parity.check_weights(wg, res["weights"], res["valid"]))
    print(f"[{case['name']}] worst weight rel err {worst:.2e}")


def test_topp_kept_sets(case):
    w, out, orc, p = case["w"], case["out"], case["orc"], case["p"]
    ndiff = 0
    for (b, g), res in orc.items():
        n = int(w.seq_lens[b])
        cnt = int(out["kept_count"][b, g])
        kept = out["kept"][b, g, :cnt]
        _, d = parity.check_kept(kept, res, p, n)
        ndiff += d
    print(f"[{case['name']}] kept-set differences at tau: {ndiff}")


def test_sparse_decode(case):
    w, out, orc = case["w"], case["out"], case["orc"]
    G = w.spec.G
    sm = parity.sm_scale_for(w.spec.d)
    worst = (0.0, 0.0)
    for (b, g), res in orc.items():
        cnt = int(out["kept_count"][b, g])
        kept = out["kept"][b, g, :cnt]
        o = out["out"][b, g * G:(g + 1) * G]
        e = parity.check_out(o, w.q[b, g * G:(g + 1) * G], w.k[b][g], w.v[b][g], kept, res, sm)
        worst = (max(worst[0], e[0]), max(worst[1], e[1]))
    print(f"[{case['name']}] worst decode err {worst[0]:.2e}, end-to-end {worst[1]:.2e}")


def test_fused_estimate_topp_repeats_the_separate_calls_bit_for_bit(case):
    """The second run makes the fused estimate + top-p call, whose top-p normalises the
    logits itself: selection, kept sets, tau and outputs must equal the separate calls'."""
    a, b = case["out"], case["out2"]
    for key in a:
        if a[key] is None or key == "weights":   # the fused call leaves weights as scratch
            continue
        if key == "kept":
            for u in np.ndindex(a["kept_count"].shape):
                k = int(a["kept_count"][u])
                assert np.array_equal(a["kept"][u][:k], b["kept"][u][:k]), u
            continue
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
