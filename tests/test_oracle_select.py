"""Pins for the oracle's chunk pooling, top-B selection and compaction (CPU only)."""

import numpy as np
import pytest

import oracle
from conftest import golden


@pytest.mark.parametrize("budget", ["5", "7", "13", "100"])
def test_golden_select(budget):
    g = golden("topb_select_n20.json")
    S = np.array(g["S"], dtype=np.float64)[None]
    kept, P = oracle.topb_select(S, n_sink=g["n_sink"], w=g["w"], chunk=g["chunk"],
                                 budget=int(budget))
    assert kept[0].tolist() == g["expected_kept"][budget]
    exp_p = np.array([np.nan if x is None else x for x in g["expected_pooled"]])
    np.testing.assert_array_equal(P[0], exp_p)


def _rank_ok(P, kept, n_sink, w, n):
    """Every kept candidate outranks every dropped one under (score desc, index asc)."""
    kept_set = set(kept.tolist())
    cand = np.arange(n_sink, n - w)
    kc = [i for i in cand if i in kept_set]
    dc = [i for i in cand if i not in kept_set]
    if not kc or not dc:
        return True
    worst_kept = min(kc, key=lambda i: (P[i], -i))
    best_drop = max(dc, key=lambda i: (P[i], -i))
    return (P[worst_kept], -worst_kept) > (P[best_drop], -best_drop)


@pytest.mark.parametrize("seed", range(6))
def test_select_invariants_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(40, 300))
    n_sink = int(rng.integers(0, 4))
    w = int(rng.integers(0, 9))
    chunk = int(rng.choice([1, 2, 4, 8]))
    budget = int(rng.integers(1, n))
    S = rng.integers(0, 5, size=(3, n)).astype(np.float64)   # many exact ties
    kept, P = oracle.topb_select(S, n_sink=n_sink, w=w, chunk=chunk, budget=budget)
    n_cand = n - n_sink - w
    assert kept.shape == (3, n_sink + min(budget, n_cand) + w)
    for row in range(3):
        k = kept[row]
        assert np.all(np.diff(k) > 0)
        assert set(range(n_sink)) | set(range(n - w, n)) <= set(k.tolist())
        assert _rank_ok(P[row], k, n_sink, w, n)
        # pooled score is the chunk mean over candidate members
        for i in range(n_sink, n - w):
            c0 = (i // chunk) * chunk
            mem = [j for j in range(c0, c0 + chunk) if n_sink <= j < n - w]
            assert P[row, i] == pytest.approx(S[row, mem].mean(), rel=1e-15)


def test_compact_is_exact_gather():
    rng = np.random.default_rng(3)
    K = rng.integers(0, 2 ** 16, size=(2, 3, 50, 8), dtype=np.uint16)
    V = rng.integers(0, 2 ** 16, size=(2, 3, 50, 8), dtype=np.uint16)
    kept = np.sort(np.stack([np.stack([rng.choice(50, 11, replace=False) for _ in range(3)])
                             for _ in range(2)]), axis=-1)
    Kc, Vc = oracle.compact(K, V, kept)
    for b in range(2):
        for g in range(3):
            for r in range(11):
                assert np.array_equal(Kc[b, g, r], K[b, g, kept[b, g, r]])
                assert np.array_equal(Vc[b, g, r], V[b, g, kept[b, g, r]])


def test_retention_shift_golden():
    """Hand-worked retention-order shifts (tests/golden/retention_shift_n16.json)."""
    from conftest import golden
    g = golden("retention_shift_n16.json")
    got = oracle.retention_shift(np.array(g["kept_a"]), np.array(g["kept_b"]), n_sink=g["n_sink"],
                                 w=g["w"], n=g["n"])
    assert np.array_equal(got, np.array(g["expected_shift"]))


def test_retention_shift_properties():
    """Symmetric at equal budgets, zero against itself, blind to the protected
    tokens and to list order; a one-swap change moves it by 1/B."""
    rng = np.random.default_rng(7)
    n, n_sink, w, B = 500, 2, 16, 40
    cand = np.arange(n_sink, n - w)
    prot = np.concatenate([np.arange(n_sink), np.arange(n - w, n)])
    a = np.stack([np.sort(np.concatenate([prot, rng.choice(cand, B, replace=False)])) for _ in range(6)])
    b = np.stack([np.sort(np.concatenate([prot, rng.choice(cand, B, replace=False)])) for _ in range(6)])
    s_ab = oracle.retention_shift(a, b, n_sink=n_sink, w=w, n=n)
    assert np.allclose(s_ab, oracle.retention_shift(b, a, n_sink=n_sink, w=w, n=n))
    assert np.all(oracle.retention_shift(a, a, n_sink=n_sink, w=w, n=n) == 0)
    assert np.allclose(s_ab, oracle.retention_shift(a[:, ::-1], b, n_sink=n_sink, w=w, n=n))
    c = a.copy()
    row_cand = [i for i in range(c.shape[1]) if n_sink <= c[0, i] < n - w]
    free = np.setdiff1d(cand, c[0])
    c[0, row_cand[0]] = free[0]
    assert oracle.retention_shift(a[:1], c[:1], n_sink=n_sink, w=w, n=n)[0] == 1.0 / B
