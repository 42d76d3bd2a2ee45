"""Pins of the trajectory reliability weights in the oracle (LORE-KV page,
Method, "Reliability weights", Eqs. 2-4 and 10).

Pinned to what the definitions fix independently of the oracle's code: two
small cases solved by hand (cosines of axis-aligned queries, their z-scores in
closed form), the symmetry that makes every disagreement equal for two
trajectories, invariance of a cosine under positive scaling and under one
rotation shared by all queries of a head, equivariance under relabelling the
trajectories, the window rows playing no part, and the centered score's zero
mean under the distribution the token is drawn from (Eqs. 2-4)."""

import math

import numpy as np
import pytest

import oracle


def _q(traj_rows, w=1, d=2, heads=1, window=None):
    """Q [1][heads][w + m*t][d] from per-trajectory query lists (same on every head)."""
    m, t = len(traj_rows), len(traj_rows[0])
    Q = np.zeros((1, heads, w + m * t, d))
    if window is not None:
        Q[0, :, :w] = window
    for j, rows in enumerate(traj_rows):
        Q[0, :, w + j * t: w + (j + 1) * t] = np.asarray(rows, dtype=np.float64)
    return Q, m, t


def _softmax(x):
    e = np.exp(np.asarray(x) - np.max(x))
    return e / e.sum()


def test_hand_case_three_single_query_trajectories():
    # cos(1,2) = 1, cos(1,3) = cos(2,3) = 0  ->  D = (1/2, 1/2, 1);
    # mean 2/3, population std sqrt(1/18)  ->  Dhat = (-1/sqrt2, -1/sqrt2, sqrt2)
    Q, m, t = _q([[(1, 0)], [(2, 0)], [(0, 3)]])
    z = np.zeros((1, m, t))
    r = oracle.reliability_weights(Q, z, z, w=1, m=m, t=t, beta=1.0, gamma=1.0, lambda_d=0.3)
    assert np.allclose(r["D"][0], [0.5, 0.5, 1.0], atol=1e-15)
    s2 = math.sqrt(2.0)
    assert np.allclose(r["dhat"][0], [-1 / s2, -1 / s2, s2], atol=1e-14)
    assert np.allclose(r["omega"][0], _softmax([0.3 / s2, 0.3 / s2, -0.3 * s2]), atol=1e-15)


def test_hand_case_two_queries_each_two_heads():
    # per head: traj 1 = {e1, e2}, traj 2 = {e1, e1}, traj 3 = {e2, e2}
    # mean cos: (1,2) = 1/2, (1,3) = 1/2, (2,3) = 0  ->  D = (1/2, 3/4, 3/4)
    # mean 2/3, std 1/sqrt72  ->  Dhat = (-sqrt2, sqrt2/2, sqrt2/2)
    Q, m, t = _q([[(1, 0), (0, 1)], [(1, 0), (5, 0)], [(0, 2), (0, 1)]], heads=2)
    logp = np.array([[[-1.0, -2.0], [-0.5, -0.5], [-3.0, -1.0]]])
    ent = np.array([[[0.5, 1.5], [0.2, 0.4], [2.0, 1.0]]])
    r = oracle.reliability_weights(Q, logp, ent, w=1, m=m, t=t, beta=1.0, gamma=1.0,
                                   lambda_d=0.3)
    assert np.allclose(r["D"][0], [0.5, 0.75, 0.75], atol=1e-15)
    s2 = math.sqrt(2.0)
    assert np.allclose(r["dhat"][0], [-s2, s2 / 2, s2 / 2], atol=1e-14)
    # cbar = mean(logp + H), Hbar = mean(H) per trajectory
    cbar = np.array([(-0.5 + -0.5) / 2, (-0.3 + -0.1) / 2, (-1.0 + 0.0) / 2])
    hbar = np.array([1.0, 0.3, 1.5])
    R = cbar - hbar - 0.3 * np.array([-s2, s2 / 2, s2 / 2])
    assert np.allclose(r["R"][0], R, atol=1e-14)
    assert np.allclose(r["omega"][0], _softmax(R), atol=1e-15)


def test_two_trajectories_have_no_disagreement_spread():
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((2, 4, 3 + 2 * 5, 16))
    logp = -rng.random((2, 2, 5))
    ent = rng.random((2, 2, 5))
    r = oracle.reliability_weights(Q, logp, ent, w=3, m=2, t=5, beta=1.0, gamma=1.0,
                                   lambda_d=0.3)
    assert np.allclose(r["D"][:, 0], r["D"][:, 1], rtol=1e-14)
    assert np.all(r["dhat"] == 0.0)


def test_zero_query_has_zero_cosine():
    # traj 1 = {0}, traj 2 = {e1}, traj 3 = {e1}: cos(1,.) = 0, cos(2,3) = 1
    Q, m, t = _q([[(0, 0)], [(1, 0)], [(4, 0)]])
    z = np.zeros((1, m, t))
    r = oracle.reliability_weights(Q, z, z, w=1, m=m, t=t, beta=1.0, gamma=1.0, lambda_d=1.0)
    assert np.allclose(r["D"][0], [1.0, 0.5, 0.5], atol=1e-15)
    assert np.all(np.isfinite(r["omega"]))


def _random_case(seed, b=2, h=3, w=4, m=4, t=3, d=8):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((b, h, w + m * t, d))
    logp = -3 * rng.random((b, m, t))
    ent = 2 * rng.random((b, m, t))
    return Q, logp, ent, dict(w=w, m=m, t=t, beta=1.0, gamma=1.0, lambda_d=0.3)


def test_invariant_under_scaling_and_shared_rotation():
    Q, logp, ent, kw = _random_case(5)
    base = oracle.reliability_weights(Q, logp, ent, **kw)
    rng = np.random.default_rng(6)
    Q2 = Q * rng.uniform(0.1, 10.0, size=Q.shape[:3] + (1,))
    for h in range(Q.shape[1]):
        R, _ = np.linalg.qr(rng.standard_normal((Q.shape[3], Q.shape[3])))
        Q2[:, h] = Q2[:, h] @ R
    got = oracle.reliability_weights(Q2, logp, ent, **kw)
    assert np.allclose(got["D"], base["D"], atol=1e-13)
    assert np.allclose(got["omega"], base["omega"], atol=1e-12)


def test_relabelling_trajectories_permutes_weights():
    Q, logp, ent, kw = _random_case(7)
    w, m, t = kw["w"], kw["m"], kw["t"]
    perm = [2, 0, 3, 1]
    Qp = Q.copy()
    for j, src in enumerate(perm):
        Qp[:, :, w + j * t: w + (j + 1) * t] = Q[:, :, w + src * t: w + (src + 1) * t]
    base = oracle.reliability_weights(Q, logp, ent, **kw)
    got = oracle.reliability_weights(Qp, logp[:, perm], ent[:, perm], **kw)
    assert np.allclose(got["omega"], base["omega"][:, perm], atol=1e-14)
    assert np.allclose(got["omega"].sum(axis=1), 1.0, atol=1e-14)


def test_window_rows_play_no_part():
    Q, logp, ent, kw = _random_case(8)
    Q2 = Q.copy()
    Q2[:, :, :kw["w"]] = np.random.default_rng(9).standard_normal(Q2[:, :, :kw["w"]].shape)
    a = oracle.reliability_weights(Q, logp, ent, **kw)
    b = oracle.reliability_weights(Q2, logp, ent, **kw)
    assert np.array_equal(a["omega"], b["omega"])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_centered_score_has_zero_mean_under_its_distribution(seed):
    # Eqs. 2-4: E_{y ~ q}[log q(y) + H(q)] = -H(q) + H(q) = 0
    rng = np.random.default_rng(seed)
    p = rng.dirichlet(np.ones(50) * 0.3)
    cs = [oracle.centered_score(p, y) for y in range(50)]
    assert abs(sum(pi * c for pi, (c, _) in zip(p, cs))) < 1e-12
    H = cs[0][1]
    assert H > 0 and all(abs(h - H) < 1e-15 for _, h in cs)
    # a uniform distribution: every sampled token is exactly typical
    c, H = oracle.centered_score(np.full(8, 1 / 8), 3)
    assert abs(c) < 1e-15 and abs(H - math.log(8)) < 1e-15
