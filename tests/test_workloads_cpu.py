"""The seeded input generator follows the recipe that its module header states.

Both the oracle and the HIP path consume these workloads, so the tests here check the
inputs themselves: the same seed gives the same arrays, the shapes and lengths of every
configuration, the page table as a permutation of the physical pages, the planting recipe
(which heads, how many tokens, sinks, and keys moved along the query direction by the
stated gain) and the paged layout with its poisoned tail slots.
"""
import numpy as np
import pytest

from adaptive_top_sparse_amd import workloads

SMALL = {
    1: dict(),
    2: dict(n=2000, budget=8),
    3: dict(n=4096 + 5, budget=16),
    4: dict(B=6, n_range=(40, 300), budget=4),
    5: dict(B=2, n=1500),
}


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_same_seed_gives_the_same_workload(cfg):
    a = workloads.make_workload(cfg, **SMALL[cfg])
    b = workloads.make_workload(cfg, **SMALL[cfg])
    assert np.array_equal(a.q, b.q)
    assert all(np.array_equal(x, y) for x, y in zip(a.k, b.k))
    assert all(np.array_equal(x, y) for x, y in zip(a.v, b.v))
    assert np.array_equal(a.page_table, b.page_table)
    assert a.planted.keys() == b.planted.keys()
    assert all(np.array_equal(a.planted[u], b.planted[u]) for u in a.planted)
    c = workloads.make_workload(cfg, seed=a.seed + 1, **SMALL[cfg])
    assert not np.array_equal(a.q, c.q)


@pytest.mark.parametrize("cfg", sorted(SMALL))
def test_shapes_dtypes_and_lengths(cfg):
    w = workloads.make_workload(cfg, **SMALL[cfg])
    s = w.spec
    assert w.q.shape == (s.B, s.Hq, s.d) and w.q.dtype == np.float16
    assert len(w.k) == len(w.v) == s.B
    for b in range(s.B):
        n_b = int(w.seq_lens[b])
        assert w.k[b].shape == w.v[b].shape == (s.Hkv, n_b, s.d)
        assert w.k[b].dtype == w.v[b].dtype == np.float16
    if s.n_range is not None:
        lo, hi = s.n_range
        assert ((w.seq_lens >= lo) & (w.seq_lens <= hi)).all()
        assert w.max_pages >= -(-hi // workloads.PAGE_SIZE)
    else:
        assert (w.seq_lens == s.n).all()
    assert w.budget == (s.budget if s.base == "quest" else None)


def test_full_size_specs_are_the_stated_workloads():
    S = workloads.SPECS
    assert (S[1].B, S[1].Hq, S[1].Hkv, S[1].d, S[1].n, S[1].base, S[1].ps) == (
        1, 1, 1, 64, 1024, None, (0.9,))
    assert (S[2].Hq, S[2].Hkv, S[2].d, S[2].n, S[2].budget, S[2].ps, S[2].sinks) == (
        32, 32, 128, 32768, 256, (0.85,), 4)
    assert (S[3].Hq, S[3].Hkv, S[3].n, S[3].budget, S[3].plant_frac, S[3].plant_gain,
            S[3].plant_heads_frac) == (32, 8, 131072, 512, 0.001, 6.0, 0.5)
    assert (S[4].B, S[4].n_range, S[4].budget, S[4].plant_frac, S[4].plant_gain) == (
        32, (4096, 32768), 256, 0.01, 4.0)
    assert (S[5].B, S[5].Hq, S[5].Hkv, S[5].n, S[5].base, S[5].ps, S[5].plant_frac,
            S[5].plant_gain, S[5].plant_heads_frac) == (
        8, 32, 8, 65536, None, (0.8, 0.9, 0.95), 0.005, 5.0, 0.6)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_page_table_is_a_permutation_of_the_physical_pages(cfg):
    w = workloads.make_workload(cfg, **SMALL[cfg])
    used = np.concatenate([w.page_table[b, :w.pages_of(b)] for b in range(w.spec.B)])
    assert used.size == w.num_phys_pages
    assert np.array_equal(np.sort(used), np.arange(w.num_phys_pages))
    assert not np.array_equal(used, np.arange(w.num_phys_pages))  # never the identity


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_planting_recipe(cfg):
    w = workloads.make_workload(cfg, **SMALL[cfg])
    s = w.spec
    per_seq_heads = int(round(s.plant_heads_frac * s.Hkv))
    for b in range(s.B):
        n_b = int(w.seq_lens[b])
        heads = sorted(g for (bb, g) in w.planted if bb == b)
        assert len(heads) == per_seq_heads
        m = int(round(s.plant_frac * n_b))
        for g in heads:
            toks = w.planted[(b, g)]
            assert np.array_equal(toks, np.unique(toks)) and toks.min() >= 0 and toks.max() < n_b
            if s.sinks:
                assert set(range(s.sinks)) <= set(toks.tolist())
                assert m <= toks.size <= m + s.sinks
            else:
                assert toks.size == m


@pytest.mark.parametrize("cfg", [2, 3])
def test_planted_keys_move_along_the_query_direction_by_the_gain(cfg):
    # k = noise + gain * u with u a unit vector and noise ~ N(0, I): u . k has mean gain on
    # planted tokens and mean 0 elsewhere (std 1 either way, plus fp16 rounding)
    w = workloads.make_workload(cfg, **SMALL[cfg])
    s = w.spec
    G = s.G
    qhat = w.q.astype(np.float64)
    qhat /= np.linalg.norm(qhat, axis=-1, keepdims=True)
    on, off = [], []
    for (b, g), toks in w.planted.items():
        u = qhat[b, g] if G == 1 else qhat[b, g * G:(g + 1) * G].sum(axis=0)
        u /= np.linalg.norm(u)
        proj = w.k[b][g].astype(np.float64) @ u
        mask = np.zeros(proj.size, dtype=bool)
        mask[toks] = True
        on.append(proj[mask])
        off.append(proj[~mask])
    on, off = np.concatenate(on), np.concatenate(off)
    assert abs(on.mean() - s.plant_gain) < 4.0 / np.sqrt(on.size) + 0.01
    assert abs(off.mean()) < 4.0 / np.sqrt(off.size) + 0.01
    assert 0.8 < off.std() < 1.2


def test_unplanted_workloads_have_no_plants():
    w = workloads.make_workload(1)
    assert w.planted == {}
    assert w.spec.plant_kind is None


@pytest.mark.parametrize("which", ["k", "v"])
def test_paged_layout_places_rows_by_the_page_table_and_poisons_tails(which):
    w = workloads.make_workload(4, **SMALL[4])
    s = w.spec
    cache = w.paged(which)
    src = w.k if which == "k" else w.v
    assert cache.shape == (w.num_phys_pages, s.Hkv, workloads.PAGE_SIZE, s.d)
    saw_tail = False
    for b in range(s.B):
        n_b = int(w.seq_lens[b])
        for p in range(w.pages_of(b)):
            phys = w.page_table[b, p]
            lo, hi = p * workloads.PAGE_SIZE, min(n_b, (p + 1) * workloads.PAGE_SIZE)
            assert np.array_equal(cache[phys, :, :hi - lo], src[b][:, lo:hi])
            if hi - lo < workloads.PAGE_SIZE:
                saw_tail = True
                assert (cache[phys, :, hi - lo:] == workloads.POISON).all()
    assert saw_tail
