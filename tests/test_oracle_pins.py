"""Pins for the CPU oracle: each check ties an oracle function to something other than
itself (brute force on tiny inputs, closed forms, invariants, textbook special cases or an
independent numpy formulation), so that a dropped term, a wrong sign or index or a
transposed operand in the oracle fails at least one of them.

Method sources (the Twilight pages): atlas.scime.ai summary "Approach" (top-p over the
estimated weights of pre-selected tokens, int4 key estimate), "Surprising findings"
(page-level top-k first, token-level top-p second) and "Limitations" (group-wise budget
under GQA).
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from adaptive_top_sparse_amd import workloads

RNG = np.random.default_rng(7)


def h_units(x):
    """Exact integer count of 2^-24 of each fp16 value (float64 holds it exactly)."""
    a = np.asarray(x, np.float16).astype(np.float64) * 2.0 ** 24
    return [int(v) for v in a.ravel()]


# ---------------------------------------------------------------- binary16 helpers ----

def test_half_decoder_matches_numpy_for_every_finite_pattern():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(vals)
    dec = np.array([oracle.half_to_double(int(b)) for b in bits[finite][::7]])
    assert np.array_equal(dec, vals[finite][::7])


def test_nearest_half_of_ratio_matches_numpy_rounding():
    # numpy converts the (correctly rounded) double quotient to binary16 with one RNE step;
    # for numerators that are fp16 differences this equals the nearest binary16 of the
    # exact ratio (a true tie is exactly representable, so no double rounding can occur).
    for _ in range(3000):
        a, b = np.float16(RNG.standard_normal() * 3), np.float16(RNG.standard_normal() * 3)
        num = abs(float(a) - float(b))
        want = np.float16(num / 15.0).view(np.uint16)
        assert oracle.nearest_half_of_ratio(num, 15) == int(want)
    # an exact tie between two binary16 neighbours goes to the even significand
    lo = np.float16(1.0)
    hi = np.nextafter(lo, np.float16(2.0))
    mid = (float(lo) + float(hi)) / 2
    assert oracle.nearest_half_of_ratio(mid * 15, 15) == int(lo.view(np.uint16))


# --------------------------------------------------------------------- c1 quantizer ----

def _numpy_quantizer(k, bits=4):
    """Independent formulation: divide and round half-to-even in fp64, then clamp."""
    L = 2 ** bits - 1
    n, d = k.shape
    x = k.astype(np.float64).reshape(n, d // 32, 32)
    mn = x.min(-1)
    mx = x.max(-1)
    scale = ((mx - mn) / L).astype(np.float16)
    s64 = scale.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        codes = np.where(s64 > 0, np.clip(np.rint((x - mn[..., None]) / s64), 0, L), 0)
    return codes.reshape(n, d).astype(np.uint8), scale, mn.astype(np.float16)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("d", [64, 128])
def test_quantizer_matches_independent_division_rounding(d, bits):
    k = RNG.standard_normal((300, d)).astype(np.float16)
    codes, scale, zero = oracle.quantize_keys(k, bits)
    c2, s2, z2 = _numpy_quantizer(k, bits)
    assert np.array_equal(codes, c2)
    assert np.array_equal(scale.astype(np.float64), s2.astype(np.float64))
    assert np.array_equal(zero.astype(np.float64), z2.astype(np.float64))


@pytest.mark.parametrize("bits", [4, 2])
def test_quantizer_nearest_code_over_all_levels(bits):
    k = (RNG.standard_normal((64, 64)) * 2).astype(np.float16)
    codes, scale, zero = oracle.quantize_keys(k, bits)
    assert codes.max() <= 2 ** bits - 1
    x = k.astype(np.float64)
    s = np.repeat(scale.astype(np.float64), 32, axis=1)
    z = np.repeat(zero.astype(np.float64), 32, axis=1)
    err_chosen = np.abs(x - (z + codes * s))
    for c in range(2 ** bits):
        assert np.all(err_chosen <= np.abs(x - (z + c * s)))


def test_two_bit_quantizer_fixed_points():
    # scale = (max - min)/3 and four levels; ties between levels go to the even code
    s_unit = 2.0 ** -2
    k = np.zeros((2, 32), np.float16)
    k[0, :] = -0.5                                 # constant: scale 0, codes 0, zero -0.5
    k[1, 1] = 3 * s_unit                           # max -> scale = s_unit exactly
    k[1, 2] = 0.5 * s_unit                         # tie 0/1 -> 0
    k[1, 3] = 1.5 * s_unit                         # tie 1/2 -> 2
    k[1, 4] = 2.5 * s_unit                         # tie 2/3 -> 2
    k[1, 5] = 1.25 * s_unit                        # nearest 1
    codes, scale, zero = oracle.quantize_keys(k, 2)
    assert scale[0, 0] == 0 and zero[0, 0] == np.float16(-0.5) and np.all(codes[0] == 0)
    assert float(scale[1, 0]) == s_unit and float(zero[1, 0]) == 0.0
    assert list(codes[1, :6]) == [0, 3, 0, 2, 2, 1]
    # (max - min)/3 is not a binary16 value: the scale is its nearest one
    k2 = np.zeros((1, 32), np.float16)
    k2[0, 7] = 1.0
    _, s2, _ = oracle.quantize_keys(k2, 2)
    assert s2[0, 0] == np.float16(1.0 / 3.0)


def test_quantizer_lossless_grid_recovers_codes():
    # keys built as zero + c*scale with a power-of-two scale, each group holding codes 0
    # and 15, dequantize exactly: the quantizer must return those codes, scale and zero.
    n, d = 40, 128
    c = RNG.integers(0, 16, size=(n, d))
    c[:, 0::32] = 0
    c[:, 1::32] = 15
    zero = -1.0
    scale = 2.0 ** -4
    k = (zero + c * scale).astype(np.float16)
    assert np.array_equal(k.astype(np.float64), zero + c * scale)
    codes, s, z = oracle.quantize_keys(k)
    assert np.array_equal(codes, c)
    assert np.all(s.astype(np.float64) == scale)
    assert np.all(z.astype(np.float64) == zero)


def test_quantizer_constant_group_and_ties():
    k = np.zeros((2, 32), np.float16)
    k[0, :] = 0.75                                  # constant group: scale 0, codes 0
    s_unit = 2.0 ** -3
    k[1, :] = 0.0
    k[1, 1] = 15 * s_unit                           # max -> scale = s_unit exactly
    k[1, 2] = 2.5 * s_unit                          # tie between 2 and 3 -> 2
    k[1, 3] = 3.5 * s_unit                          # tie between 3 and 4 -> 4
    k[1, 4] = 3.25 * s_unit                         # nearest 3
    codes, scale, zero = oracle.quantize_keys(k)
    assert scale[0, 0] == 0 and zero[0, 0] == np.float16(0.75)
    assert np.all(codes[0] == 0)
    assert float(scale[1, 0]) == s_unit and float(zero[1, 0]) == 0.0
    assert list(codes[1, :5]) == [0, 15, 2, 4, 3]


# -------------------------------------------------------------------- c2 page bounds ---

@pytest.mark.parametrize("n", [16, 37, 160, 1])
def test_page_bounds_brute_force(n):
    k = RNG.standard_normal((n, 64)).astype(np.float16)
    lo, hi = oracle.page_bounds(k, 16)
    P = -(-n // 16)
    for p in range(P):
        blk = k[p * 16:min(n, p * 16 + 16)].astype(np.float64)
        assert np.array_equal(lo[p].astype(np.float64), blk.min(0))
        assert np.array_equal(hi[p].astype(np.float64), blk.max(0))


# ------------------------------------------------------------- c3 Quest page scores ----

def _exact_score_by_corners(q, lo, hi):
    """Per head, the maximum of q_h . x over all 2^d corners of the box [lo, hi]
    (brute force, exact integers in units of 2^-48), summed over the heads."""
    G, d = q.shape
    total = 0
    for h in range(G):
        qh = h_units(q[h])
        lo_u, hi_u = h_units(lo), h_units(hi)
        best = None
        for corner in itertools.product((0, 1), repeat=d):
            v = sum(qh[c] * (hi_u[c] if corner[c] else lo_u[c]) for c in range(d))
            best = v if best is None else max(best, v)
        total += best
    return total


def test_quest_score_equals_brute_force_box_maximum():
    G, d, P = 3, 8, 6
    q = RNG.standard_normal((G, d)).astype(np.float16)
    k = RNG.standard_normal((P * 16, d)).astype(np.float16)
    lo, hi = oracle.page_bounds(k, 16)
    _, scores, _ = oracle.quest_select(q, lo, hi, budget=P, return_scores=True)
    for p in range(P):
        exact = _exact_score_by_corners(q, lo[p], hi[p])
        assert scores[p] == float(Fraction(exact, 2 ** 48))


def test_quest_score_bounds_every_token_and_is_tight_for_one_token():
    G, d = 4, 128
    n = 16 * 5 + 1                                   # last page holds a single token
    q = RNG.standard_normal((G, d)).astype(np.float16)
    k = RNG.standard_normal((n, d)).astype(np.float16)
    lo, hi = oracle.page_bounds(k, 16)
    P = lo.shape[0]
    _, scores, sens = oracle.quest_select(q, lo, hi, budget=P, return_scores=True)
    assert sens == 0
    qu = [h_units(q[h]) for h in range(G)]
    for t in range(n):
        ku = h_units(k[t])
        dot = sum(sum(qu[h][c] * ku[c] for c in range(d)) for h in range(G))
        assert Fraction(dot, 2 ** 48) <= Fraction(scores[t // 16])
    ku = h_units(k[n - 1])
    dot = sum(sum(qu[h][c] * ku[c] for c in range(d)) for h in range(G))
    assert scores[P - 1] == float(Fraction(dot, 2 ** 48))


def test_quest_group_score_is_sum_of_per_head_scores():
    G, d, P = 4, 64, 20
    q = RNG.standard_normal((G, d)).astype(np.float16)
    k = RNG.standard_normal((P * 16, d)).astype(np.float16)
    lo, hi = oracle.page_bounds(k, 16)
    _, s_all, _ = oracle.quest_select(q, lo, hi, budget=P, return_scores=True)
    parts = [oracle.quest_select(q[h:h + 1], lo, hi, budget=P, return_scores=True)[1]
             for h in range(G)]
    assert np.allclose(s_all, np.sum(parts, axis=0), rtol=0, atol=1e-9)


def test_quest_selection_matches_full_sort_with_index_ties():
    G, d, P = 2, 64, 50
    q = RNG.standard_normal((G, d)).astype(np.float16)
    k = RNG.standard_normal((P * 16, d)).astype(np.float16)
    lo, hi = oracle.page_bounds(k, 16)
    # duplicate some pages' bounds to force exact score ties
    for dst, src in ((7, 3), (31, 3), (40, 12)):
        lo[dst], hi[dst] = lo[src], hi[src]
    qu = [h_units(q[h]) for h in range(G)]
    exact = []
    for p in range(P):
        lu, hu = h_units(lo[p]), h_units(hi[p])
        exact.append(sum(max(qu[h][c] * lu[c], qu[h][c] * hu[c])
                         for h in range(G) for c in range(d)))
    for budget in (1, 5, 17, 49, 50, 80):
        order = sorted(range(P), key=lambda i: (-exact[i], i))
        want = sorted(order[:min(budget, P)])
        got = oracle.quest_select(q, lo, hi, budget)
        assert list(got) == want


def test_quest_scores_are_order_insensitive_at_workload_scale():
    w = workloads.make_workload(3, n=4096, budget=64)
    G = w.spec.G
    for g in range(w.spec.Hkv):
        lo, hi = oracle.page_bounds(w.k[0][g])
        _, _, sens = oracle.quest_select(w.q[0, g * G:(g + 1) * G], lo, hi, 64,
                                         return_scores=True)
        assert sens == 0


# ----------------------------------------------------------------- c4 the estimate ----

def _quantize(k):
    return oracle.quantize_keys(k)


def test_estimate_sums_to_one_and_invalid_slots_are_zero():
    G, d, n = 4, 128, 200                      # 13 pages, last one partial
    q = RNG.standard_normal((G, d)).astype(np.float16)
    k = RNG.standard_normal((n, d)).astype(np.float16)
    codes, scale, zero = _quantize(k)
    cand = np.array([0, 4, 12], np.int32)      # page 12 holds tokens 192..199 only
    n_slots = 5 * 16                           # two extra page slots past the list
    w = oracle.estimate_weights(q, codes, scale, zero, n, cand, n_slots, 1 / math.sqrt(d))
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
    valid = np.zeros(n_slots, bool)
    valid[:2 * 16] = True
    valid[32:32 + 8] = True
    assert np.all(w[:, ~valid] == 0.0)
    assert np.all(w[:, valid] > 0.0)


def test_estimate_is_textbook_softmax_on_lossless_keys():
    G, d, n = 2, 64, 64
    c = RNG.integers(0, 16, size=(n, d))
    c[:, 0::32], c[:, 1::32] = 0, 15
    k = (-0.5 + c * 2.0 ** -4).astype(np.float16)
    q = RNG.standard_normal((G, d)).astype(np.float16)
    codes, scale, zero = _quantize(k)
    sm = np.float32(1 / math.sqrt(d))
    w = oracle.estimate_weights(q, codes, scale, zero, n, None, n, sm)
    logits = float(sm) * (q.astype(np.float64) @ k.astype(np.float64).T)
    e = np.exp(logits - logits.max(1, keepdims=True))
    want = e / e.sum(1, keepdims=True)
    assert np.allclose(w, want, rtol=1e-12, atol=0)


def test_estimate_group_algebra_equals_direct_dequant():
    # sum_c q_c (zero + code_c * scale) == sum_groups [zero * Q_grp + scale * sum q_c code_c]
    G, d, n = 4, 128, 48
    q = RNG.standard_normal((G, d)).astype(np.float16)
    k = RNG.standard_normal((n, d)).astype(np.float16)
    codes, scale, zero = _quantize(k)
    sm = np.float32(1 / math.sqrt(d))
    w = oracle.estimate_weights(q, codes, scale, zero, n, None, n, sm)
    qf = q.astype(np.float64).reshape(G, d // 32, 32)
    cf = codes.astype(np.float64).reshape(n, d // 32, 32)
    Qg = qf.sum(-1)                                            # [G, groups]
    s = (np.einsum("gk,nk->gn", Qg, zero.astype(np.float64)) +
         np.einsum("gkc,nkc,nk->gn", qf, cf, scale.astype(np.float64))) * float(sm)
    e = np.exp(s - s.max(1, keepdims=True))
    assert np.allclose(w, e / e.sum(1, keepdims=True), rtol=1e-12, atol=0)


def test_estimate_slot_mapping_follows_the_candidate_list():
    G, d, n = 1, 64, 96
    q = RNG.standard_normal((G, d)).astype(np.float16)
    k = RNG.standard_normal((n, d)).astype(np.float16)
    codes, scale, zero = _quantize(k)
    a = oracle.estimate_weights(q, codes, scale, zero, n, np.array([1, 4], np.int32), 32, 0.125)
    b = oracle.estimate_weights(q, codes, scale, zero, n, np.array([4, 1], np.int32), 32, 0.125)
    # same tokens, same weights; only the denominator's summation order differs
    assert np.allclose(a[:, :16], b[:, 16:], rtol=1e-14, atol=0)
    assert np.allclose(a[:, 16:], b[:, :16], rtol=1e-14, atol=0)


# ------------------------------------------------------------------ c5 top-p nucleus ---

def _brute_force_min_nucleus(W, p):
    C = len(W)
    total = sum(W)
    for m in range(0, C + 1):
        best = None
        for sub in itertools.combinations(range(C), m):
            mass = sum(W[i] for i in sub)
            if mass >= p * total and (best is None or mass > best[0]):
                best = (mass, sub)
        if best is not None:
            return m, best
    return C, (total, tuple(range(C)))


@pytest.mark.parametrize("trial", range(40))
def test_topp_is_the_minimal_nucleus_by_brute_force(trial):
    C = int(RNG.integers(1, 12))
    W = RNG.dirichlet(np.ones(C) * 0.7)
    p = float(np.float32(RNG.uniform(0.05, 0.99)))
    kept, tau = oracle.topp_select(W[None, :], np.ones(C, bool), p)
    m_star, (mass_star, _) = _brute_force_min_nucleus(list(W), p)
    assert len(kept) == m_star
    mass = W[kept].sum()
    assert mass >= p * W.sum() - 1e-15
    assert math.isclose(mass, mass_star, rel_tol=1e-12)
    assert tau == W[kept].min()
    assert np.all(W[np.setdiff1d(np.arange(C), kept)] <= tau)


def test_topp_special_cases():
    W = RNG.dirichlet(np.ones(30))
    ones = np.ones(30, bool)
    kept, _ = oracle.topp_select(W[None], ones, 1.0)
    assert list(kept) == list(range(30))
    onehot = np.zeros(30)
    onehot[17] = 1.0
    for p in (1e-6, 0.5, 0.9, float(np.float32(1.0 - 2.0 ** -24))):
        kept, tau = oracle.topp_select(onehot[None], ones, p)
        assert list(kept) == [17]
        assert tau == 1.0
    kept, _ = oracle.topp_select(W[None], ones, 1e-7)
    assert list(kept) == [int(np.argmax(W))]


def test_topp_mass_exactly_at_target_stops_there():
    # mass reaches p * total exactly after two tokens (all values exact in binary): the
    # nucleus is those two, the lower slot winning the tie between the 0.25s
    W = np.array([0.5, 0.25, 0.25])
    kept, tau = oracle.topp_select(W[None], np.ones(3, bool), 0.75)
    assert list(kept) == [0, 1] and tau == 0.25
    m_star, _ = _brute_force_min_nucleus(list(W), 0.75)
    assert m_star == 2


def test_topp_at_p_one_keeps_every_valid_slot_even_zero_weights():
    # p = 1 prunes nothing: a one-hot distribution keeps all its valid slots (weights that
    # are 0, e.g. underflowed, included), and invalid slots stay out
    onehot = np.zeros(30)
    onehot[17] = 1.0
    valid = np.ones(30, bool)
    valid[25:] = False
    kept, tau = oracle.topp_select(onehot[None], valid, 1.0)
    assert list(kept) == list(range(25))
    assert tau == 0.0


def test_topp_group_mean_equals_single_head_on_the_mean():
    G, C = 4, 64
    w = RNG.dirichlet(np.ones(C), size=G)
    ones = np.ones(C, bool)
    for p in (0.3, 0.8, 0.95):
        a, ta = oracle.topp_select(w, ones, p)
        b, tb = oracle.topp_select(w.mean(0, keepdims=True), ones, p)
        assert np.array_equal(a, b) and math.isclose(ta, tb, rel_tol=1e-15)


def test_topp_maps_slots_to_tokens_ascending_and_skips_invalid():
    C = 48
    W = RNG.dirichlet(np.ones(C))
    valid = np.ones(C, bool)
    valid[40:] = False
    W[40:] = 0
    cand = np.array([9, 2, 5], np.int32)               # any page order
    kept, _ = oracle.topp_select(W[None], valid, 0.9, cand)
    assert np.all(np.diff(kept) > 0)
    slot_of = {int(cand[s // 16]) * 16 + s % 16: s for s in range(40)}
    assert all(int(t) in slot_of for t in kept)
    slots = [slot_of[int(t)] for t in kept]
    # it is the minimal nucleus over the valid slots
    kept_s, _ = oracle.topp_select(W[None], valid, 0.9)
    assert sorted(slots) == sorted(int(s) for s in kept_s)


# --------------------------------------------------------------- c7 sparse attention ---

def _dense_attention(q, k, v, sm):
    s = float(sm) * (q.astype(np.float64) @ k.astype(np.float64).T)
    e = np.exp(s - s.max(1, keepdims=True))
    return (e / e.sum(1, keepdims=True)) @ v.astype(np.float64)


def test_attention_over_all_tokens_is_dense_attention():
    G, d, n = 4, 128, 100
    q = RNG.standard_normal((G, d)).astype(np.float16)
    k = RNG.standard_normal((n, d)).astype(np.float16)
    v = RNG.standard_normal((n, d)).astype(np.float16)
    sm = np.float32(1 / math.sqrt(d))
    out = oracle.sparse_attention(q, k, v, np.arange(n, dtype=np.int32), sm)
    assert np.allclose(out, _dense_attention(q, k, v, sm), rtol=1e-12, atol=1e-14)


def test_attention_special_cases():
    G, d, n = 2, 64, 40
    q = RNG.standard_normal((G, d)).astype(np.float16)
    k = RNG.standard_normal((n, d)).astype(np.float16)
    v = RNG.standard_normal((n, d)).astype(np.float16)
    out = oracle.sparse_attention(q, k, v, np.array([13], np.int32), 0.125)
    assert np.array_equal(out, np.repeat(v[13:14].astype(np.float64), G, 0))
    out = oracle.sparse_attention(q, k, v, np.zeros(0, np.int32), 0.125)
    assert np.all(out == 0)
    k2 = k.copy()
    k2[21] = k2[5]
    out = oracle.sparse_attention(q, k2, v, np.array([5, 21], np.int32), 0.125)
    want = (v[5].astype(np.float64) + v[21].astype(np.float64)) / 2
    assert np.allclose(out, want[None], rtol=0, atol=1e-15)
    sub = np.array([3, 9, 30], np.int32)
    a = oracle.sparse_attention(q, k, v, sub, 0.125)
    assert np.allclose(a, _dense_attention(q, k[sub], v[sub], 0.125), rtol=1e-12, atol=1e-14)


# ------------------------------------------- head-wise top-p under GQA (per query head) ---

@pytest.mark.parametrize("trial", range(12))
def test_headwise_unit_is_a_nucleus_and_attention_per_head(trial):
    """Head-wise form: each query head's kept set is the minimal nucleus of its own weights
    (brute force), its output is textbook attention over that set, and two heads planted on
    different tokens keep their own planted token."""
    G, d = 2, 64
    n = int(RNG.integers(4, 12))
    p = float(np.float32(RNG.uniform(0.3, 0.95)))
    k = RNG.standard_normal((n, d)).astype(np.float16)
    v = RNG.standard_normal((n, d)).astype(np.float16)
    a, b = RNG.choice(n, 2, replace=False)
    q = RNG.standard_normal((G, d)) * 0.3
    q[0] += 0.8 * k[a].astype(np.float64)
    q[1] += 0.8 * k[b].astype(np.float64)
    q = q.astype(np.float16)
    sm = float(np.float32(1 / math.sqrt(d)))
    res = oracle.run_unit(q, k, v, None, p, sm, headwise=True)
    assert len(res["kept"]) == G and res["out"].shape == (G, d)
    for h, planted in ((0, a), (1, b)):
        W = res["weights"][h, :n]
        kept = res["kept"][h]
        m_star, (mass_star, _) = _brute_force_min_nucleus(list(W), p)
        assert len(kept) == m_star
        assert math.isclose(W[kept].sum(), mass_star, rel_tol=1e-12)
        assert res["tau"][h] == W[kept].min()
        assert planted in kept
        want = _dense_attention(q[h:h + 1], k[kept], v[kept], sm)
        assert np.allclose(res["out"][h:h + 1], want, rtol=1e-12, atol=1e-14)
    # the group-wise form on the same unit keeps the nucleus of the group mean instead
    grp = oracle.run_unit(q, k, v, None, p, sm)
    Wm = grp["weights"][:, :n].mean(0)
    m_star, (mass_star, _) = _brute_force_min_nucleus(list(Wm), p)
    assert len(grp["kept"]) == m_star


def test_headwise_equals_groupwise_for_one_head_per_group():
    d, n = 128, 70
    k = RNG.standard_normal((n, d)).astype(np.float16)
    v = RNG.standard_normal((n, d)).astype(np.float16)
    q = RNG.standard_normal((1, d)).astype(np.float16)
    sm = float(np.float32(1 / math.sqrt(d)))
    for budget in (None, 2):
        hw = oracle.run_unit(q, k, v, budget, 0.9, sm, headwise=True)
        gw = oracle.run_unit(q, k, v, budget, 0.9, sm)
        assert np.array_equal(hw["kept"][0], gw["kept"]) and hw["tau"][0] == gw["tau"]
        assert np.array_equal(hw["out"], gw["out"])
