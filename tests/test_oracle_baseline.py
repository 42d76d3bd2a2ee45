"""Pins of the prompt-side baseline scores in the oracle (window attention
score of the LORE-KV page's "Prompt-side eviction", TOVA's last-query score).

They are pinned to what the definitions fix independently of the oracle's
code: every softmax row sums to one (so the window score of a KV head sums to
w over the tokens and TOVA's to 1), a brute-force double loop over scalars,
TOVA equal to the window score when w = 1, and the row statistics of the C
oracle's attention pass (a = exp(s - m) / l summed over the window rows)."""

import math

import numpy as np
import pytest

import oracle


def _inputs(seed=0, b=1, h_q=4, h_kv=2, n_q=6, n=23, d=8):
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((b, h_q, n_q, d))
    K = rng.standard_normal((b, h_kv, n, d))
    V = rng.standard_normal((b, h_kv, n, d))
    return Q, K, V


@pytest.mark.parametrize("kind,total", [("window", None), ("tova", 1.0)])
def test_row_sums(kind, total):
    Q, K, _ = _inputs(1)
    w = 4
    S = oracle.baseline_scores(Q, K, w=w, kind=kind)
    expect = float(w) if total is None else total
    assert np.allclose(S.sum(axis=-1), expect, rtol=0, atol=1e-12)
    assert np.all(S >= 0)


def test_brute_force_scalar_loops():
    Q, K, _ = _inputs(2, b=2, h_q=2, h_kv=1, n_q=5, n=9, d=3)
    w = 3
    S = oracle.baseline_scores(Q, K, w=w, kind="window")
    b, h_q, _, d = Q.shape
    n = K.shape[2]
    ref = np.zeros((b, 1, n))
    for bb in range(b):
        for h in range(h_q):
            for r in range(w):
                vis = n - w + r + 1  # keys 0 .. n-w+r
                logits = []
                for i in range(vis):
                    acc = 0.0
                    for k in range(d):
                        acc += Q[bb, h, r, k] * K[bb, 0, i, k]
                    logits.append(acc / math.sqrt(d))
                mx = max(logits)
                ex = [math.exp(x - mx) for x in logits]
                tot = sum(ex)
                for i in range(vis):
                    ref[bb, 0, i] += ex[i] / tot / h_q
    assert np.allclose(S, ref, rtol=1e-12, atol=1e-15)


def test_tova_is_window_score_of_one_row():
    Q, K, _ = _inputs(3)
    S1 = oracle.baseline_scores(Q, K, w=1, kind="window")
    T1 = oracle.baseline_scores(Q, K, w=1, kind="tova")
    assert np.array_equal(S1, T1)
    # and TOVA with w rows is the window score of the last row alone
    w = 4
    T = oracle.baseline_scores(Q, K, w=w, kind="tova")
    Qlast = Q[:, :, w - 1:w]
    Kcut = K[:, :, :K.shape[2]]  # the last window row sees every key
    assert np.allclose(T, oracle.baseline_scores(Qlast, Kcut, w=1, kind="window"), atol=1e-15)


def test_matches_attention_pass_statistics():
    Q, K, V = _inputs(4, b=1, h_q=4, h_kv=2, n_q=6, n=31, d=8)
    w = 4
    m, l, _ = oracle.lore_attention(Q, K, V, w)
    b, h_q, _, d = Q.shape
    n = K.shape[2]
    G = h_q // K.shape[1]
    ref = np.zeros((b, K.shape[1], n))
    for h in range(h_q):
        for r in range(w):
            s = K[0, h // G] @ Q[0, h, r] / math.sqrt(d)
            a = np.exp(s - m[0, h, r]) / l[0, h, r]
            a[n - w + r + 1:] = 0.0
            ref[0, h // G] += a / G
    S = oracle.baseline_scores(Q, K, w=w, kind="window")
    assert np.allclose(S, ref, rtol=1e-12, atol=1e-15)
