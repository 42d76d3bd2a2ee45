"""Pins for the LORE-KV part of the oracle (CPU only).

The oracle is checked against things other than itself:
  * a hand-derived worked example (tests/golden/deletion_three_token.json);
  * literal deletion: drop token i, renormalise, recompute o_q and measure
    ||W_h (o_q - o_q^(-i))|| with the full d_model-wide W_h -- the closed form
    of the LORE-KV page (Eqs. 5-6) must reproduce it exactly at eps = 0;
  * closed forms (all-equal keys give uniform attention);
  * invariants and special cases (softmax rows sum to one, linearity in
    lambda_L, one-hot omega, MHA, duplicated GQA heads).
"""

import math

import numpy as np
import pytest

import oracle
from conftest import golden


def _softmax(s):
    s = s - s.max()
    e = np.exp(s)
    return e / e.sum()


def _visible(r, n, w):
    return np.arange(0, n - w + r + 1) if r < w else np.arange(n)


def brute_scores(Q, K, V, W_O, omega, w, m, t, lambda_l=1.0):
    """Per-query-head score by literal deletion (eps = 0), Eq. 7 with psi = mean."""
    b, h_q, nq, d = Q.shape
    h_kv, n = K.shape[1], K.shape[2]
    G = h_q // h_kv
    S_head = np.zeros((b, h_q, n))
    for bb in range(b):
        for h in range(h_q):
            g = h // G
            Wh = W_O[:, h * d:(h + 1) * d]
            E = np.zeros((nq, n))
            for r in range(nq):
                vis = _visible(r, n, w)
                s = K[bb, g, vis] @ Q[bb, h, r] / math.sqrt(d)
                o = _softmax(s) @ V[bb, g, vis]
                for j, i in enumerate(vis):
                    rest = np.delete(vis, j)
                    o_wo = _softmax(np.delete(s, j)) @ V[bb, g, rest]
                    E[r, i] = np.linalg.norm(Wh @ (o - o_wo))
            S = E[:w].mean(axis=0) if w > 0 else np.zeros(n)
            for mm in range(m):
                S = S + lambda_l * omega[bb, mm] * E[w + mm * t: w + (mm + 1) * t].mean(axis=0)
            S_head[bb, h] = S
    return S_head


def _rand_case(seed, b=2, n=37, h_q=4, h_kv=2, d=8, D=24, w=5, m=2, t=3, key_scale=1.0):
    rng = np.random.default_rng(seed)
    nq = w + m * t
    Q = rng.standard_normal((b, h_q, nq, d))
    K = rng.standard_normal((b, h_kv, n, d)) * key_scale
    V = rng.standard_normal((b, h_kv, n, d))
    W_O = rng.standard_normal((D, h_q * d)) / math.sqrt(d)
    omega = rng.dirichlet(np.ones(max(m, 1)), size=b)[:, :m]
    return Q, K, V, W_O, omega


CASES = [
    dict(seed=1),
    dict(seed=2, w=0, m=3, t=2),                 # lookahead rows only
    dict(seed=3, m=0, t=1, w=6),                 # window rows only
    dict(seed=4, h_q=3, h_kv=3, D=30),           # MHA
    dict(seed=5, key_scale=3.0, n=23, w=4),      # peaked attention
    dict(seed=6, h_q=6, h_kv=2, d=4, D=32, n=18, w=3, m=1, t=2),  # GQA 3
]


@pytest.mark.parametrize("case", CASES)
def test_closed_form_equals_literal_deletion(case):
    kw = dict(case)
    Q, K, V, W_O, omega = _rand_case(**kw)
    w = kw.get("w", 5); m = kw.get("m", 2); t = kw.get("t", 3)
    ref = brute_scores(Q, K, V, W_O, omega, w, m, t)
    got = oracle.lore_scores(Q, K, V, W_O, omega, w=w, m=m, t=t, eps=0.0, lambda_l=1.0)
    np.testing.assert_allclose(got["S_head"], ref, rtol=1e-9, atol=1e-12)
    G = Q.shape[1] // K.shape[1]
    grp = ref.reshape(ref.shape[0], K.shape[1], G, -1).mean(axis=2)
    np.testing.assert_allclose(got["S"], grp, rtol=1e-9, atol=1e-12)


def test_eps_only_shrinks_each_term():
    Q, K, V, W_O, omega = _rand_case(7)
    s0 = oracle.lore_scores(Q, K, V, W_O, omega, w=5, m=2, t=3, eps=0.0, lambda_l=1.0)
    s1 = oracle.lore_scores(Q, K, V, W_O, omega, w=5, m=2, t=3, eps=1e-6, lambda_l=1.0)
    # a/(1-a+eps) >= a/(1-a) * (1 - eps/(1-a)); with a <= 0.99 the ratio is within 1e-4
    assert np.all(s1["S_head"] <= s0["S_head"] * (1 + 1e-15))
    assert np.all(s1["S_head"] >= s0["S_head"] * (1 - 1e-4))


@pytest.mark.parametrize("lam", ["1.0", "0.5"])
def test_golden_three_token(lam):
    g = golden("deletion_three_token.json")
    Q = np.array(g["Q"])[None, None]
    K = np.array(g["K"])[None, None]
    V = np.array(g["V"])[None, None]
    W_O = np.array(g["W_O"])
    omega = np.array(g["omega"])[None]
    r = oracle.lore_scores(Q, K, V, W_O, omega, w=g["w"], m=g["m"], t=g["t"],
                           eps=g["eps"], lambda_l=float(lam))
    np.testing.assert_allclose(r["O"][0, 0], np.array(g["expected_O"]), rtol=1e-13)
    np.testing.assert_allclose(r["S"][0, 0], np.array(g["expected_S"][lam]), rtol=1e-12)


def test_projection_factor_preserves_norm():
    rng = np.random.default_rng(11)
    for D, hq, d in ((256, 4, 64), (4096, 2, 128)):
        W = rng.standard_normal((D, hq * d)) / math.sqrt(d)
        R = oracle.projection_factors(W, hq, d)
        for h in range(hq):
            assert np.allclose(np.tril(R[h], -1), 0.0)
            x = rng.standard_normal((d, 16))
            np.testing.assert_allclose(np.linalg.norm(R[h] @ x, axis=0),
                                       np.linalg.norm(W[:, h * d:(h + 1) * d] @ x, axis=0),
                                       rtol=1e-11)


def test_uniform_attention_closed_form():
    """All keys equal: a_{r,i} = 1/|visible_r|, o_r = mean of the visible values."""
    rng = np.random.default_rng(12)
    b, h_q, h_kv, n, d, D, w, m, t = 1, 2, 1, 29, 6, 20, 4, 2, 2
    eps = 1e-6
    nq = w + m * t
    Q = rng.standard_normal((b, h_q, nq, d))
    K = np.tile(rng.standard_normal(d), (b, h_kv, n, 1))
    V = rng.standard_normal((b, h_kv, n, d))
    W_O = rng.standard_normal((D, h_q * d))
    omega = np.array([[0.3, 0.7]])
    got = oracle.lore_scores(Q, K, V, W_O, omega, w=w, m=m, t=t, eps=eps, lambda_l=1.0)
    for h in range(h_q):
        Wh = W_O[:, h * d:(h + 1) * d]
        E = np.zeros((nq, n))
        for r in range(nq):
            vis = _visible(r, n, w)
            k = len(vis)
            o = V[0, 0, vis].mean(axis=0)
            c = (1.0 / k) / (1.0 - 1.0 / k + eps)
            E[r, vis] = c * np.linalg.norm((V[0, 0, vis] - o) @ Wh.T, axis=1)
        S = E[:w].mean(0) + 0.3 * E[w:w + t].mean(0) + 0.7 * E[w + t:].mean(0)
        np.testing.assert_allclose(got["S_head"][0, h], S, rtol=1e-11)


def test_softmax_rows_sum_to_one():
    Q, K, V, W_O, omega = _rand_case(13, n=50, w=6)
    m_, l_, O = oracle.lore_attention(Q, K, V, 6)
    b, h_q, nq, d = Q.shape
    G = h_q // K.shape[1]
    for bb in range(b):
        for h in range(h_q):
            for r in range(nq):
                vis = _visible(r, K.shape[2], 6)
                s = K[bb, h // G, vis] @ Q[bb, h, r] / math.sqrt(d)
                p = np.exp(s - m_[bb, h, r])
                assert abs(p.max() - 1.0) < 1e-14
                assert abs(p.sum() / l_[bb, h, r] - 1.0) < 1e-12


def test_lambda_linearity_and_window_only():
    Q, K, V, W_O, omega = _rand_case(14)
    args = dict(w=5, m=2, t=3, eps=1e-6)
    s0 = oracle.lore_scores(Q, K, V, W_O, omega, lambda_l=0.0, **args)["S_head"]
    s1 = oracle.lore_scores(Q, K, V, W_O, omega, lambda_l=1.0, **args)["S_head"]
    s2 = oracle.lore_scores(Q, K, V, W_O, omega, lambda_l=2.0, **args)["S_head"]
    np.testing.assert_allclose(s2 - s1, s1 - s0, rtol=1e-9, atol=1e-13)
    # lambda_L = 0 leaves only the window term: equal to a window-only run
    wo = oracle.lore_scores(Q[:, :, :5], K, V, W_O, omega[:, :0], w=5, m=0, t=1,
                            eps=1e-6, lambda_l=1.0)["S_head"]
    np.testing.assert_allclose(s0, wo, rtol=1e-12)


def test_one_hot_omega_ignores_other_trajectories():
    Q, K, V, W_O, _ = _rand_case(15, m=3, t=2)
    omega = np.tile(np.array([[0.0, 1.0, 0.0]]), (Q.shape[0], 1))
    args = dict(w=5, m=3, t=2, eps=1e-6, lambda_l=1.0)
    base = oracle.lore_scores(Q, K, V, W_O, omega, **args)["S_head"]
    Q2 = Q.copy()
    Q2[:, :, 5:7] += 5.0     # trajectory 0
    Q2[:, :, 9:11] -= 3.0    # trajectory 2
    moved = oracle.lore_scores(Q2, K, V, W_O, omega, **args)["S_head"]
    np.testing.assert_array_equal(base, moved)


def test_duplicated_group_heads_equal_single_head():
    Q, K, V, W_O, omega = _rand_case(16, h_q=2, h_kv=2, D=16)
    d = Q.shape[-1]
    Qg = np.repeat(Q, 3, axis=1)                       # three identical heads per KV head
    Wg = np.concatenate([W_O[:, h * d:(h + 1) * d] for h in range(2) for _ in range(3)], axis=1)
    args = dict(w=5, m=2, t=3, eps=1e-6, lambda_l=1.0)
    mha = oracle.lore_scores(Q, K, V, W_O, omega, **args)["S"]
    gqa = oracle.lore_scores(Qg, K, V, Wg, omega, **args)["S"]
    np.testing.assert_allclose(gqa, mha, rtol=1e-12)


def test_threads_do_not_change_results():
    Q, K, V, W_O, omega = _rand_case(17, n=64)
    args = dict(w=5, m=2, t=3, eps=1e-6, lambda_l=1.0)
    a = oracle.lore_scores(Q, K, V, W_O, omega, nthreads=1, **args)["S"]
    b = oracle.lore_scores(Q, K, V, W_O, omega, nthreads=4, **args)["S"]
    np.testing.assert_array_equal(a, b)


def test_probabilities_match_statistics_and_mask():
    """lore_probabilities: rows sum to 1, entries past a window row's position
    are exactly 0, and a = exp(s - row_max) / row_sum with lore_attention's
    statistics (two independent computations of the same softmax); also
    P @ V equals lore_attention's output."""
    rng = np.random.default_rng(11)
    b, hq, hk, n, d, w, nq = 2, 4, 2, 40, 16, 5, 9
    Q = rng.standard_normal((b, hq, nq, d))
    K = rng.standard_normal((b, hk, n, d))
    V = rng.standard_normal((b, hk, n, d))
    P = oracle.lore_probabilities(Q, K, w)
    assert np.allclose(P.sum(axis=-1), 1.0, atol=1e-12)
    for r in range(w):
        assert np.all(P[:, :, r, n - w + r + 1:] == 0)
    m, l, O = oracle.lore_attention(Q, K, V, w)
    G = hq // hk
    for bi in range(b):
        for h in range(hq):
            s = Q[bi, h] @ K[bi, h // G].T / np.sqrt(d)
            for r in range(nq):
                last = n - w + r if r < w else n - 1
                ref = np.exp(s[r, :last + 1] - m[bi, h, r]) / l[bi, h, r]
                assert np.allclose(P[bi, h, r, :last + 1], ref, rtol=1e-12, atol=0)
            assert np.allclose(P[bi, h] @ V[bi, h // G], O[bi, h], rtol=1e-10, atol=1e-12)
