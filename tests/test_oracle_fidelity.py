"""Pins of the attention-output fidelity in the oracle (LORE-KV page, "Why it
works", "Output fidelity": the retained cache reproducing the full cache's
attention outputs, read as the mean cosine between the two outputs per query
head and held-out query).

Pinned to what the definition fixes independently of the oracle's code:
keeping every token (in any order) reproduces the outputs; equal keys give
uniform attention, whose outputs have a closed-form cosine; dropping tokens
whose attention underflows changes nothing; a positive scale or a rotation of
all values leaves every cosine alone; the stated zero-output conventions; and
scalar loops on a tiny GQA case."""

import math

import numpy as np
import pytest

import oracle


def _case(seed, b=2, h_q=4, h_kv=2, n_f=5, n=40, d=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, h_q, n_f, d)), rng.standard_normal((b, h_kv, n, d)),
            rng.standard_normal((b, h_kv, n, d)))


def test_keeping_everything_reproduces_the_outputs():
    Qf, K, V = _case(1)
    b, h_kv, n, _ = K.shape
    rng = np.random.default_rng(2)
    kept = np.stack([np.stack([rng.permutation(n) for _ in range(h_kv)]) for _ in range(b)])
    r = oracle.output_fidelity(Qf, K, V, kept)
    assert np.allclose(r["cos"], 1.0, atol=1e-12)
    assert np.allclose(r["fidelity"], 1.0, atol=1e-12)


@pytest.mark.parametrize("k,n", [(1, 4), (3, 10), (7, 7), (5, 20)])
def test_uniform_attention_closed_form(k, n):
    # equal keys: every token gets 1/n; kept values e1, dropped values e2
    # o_full = (k e1 + (n-k) e2)/n, o_kept = e1  ->  cos = k / sqrt(k^2 + (n-k)^2)
    d = 4
    K = np.tile(np.array([0.3, -1.0, 2.0, 0.5]), (1, 1, n, 1))
    V = np.zeros((1, 1, n, d))
    V[0, 0, :k, 0] = 1.0
    V[0, 0, k:, 1] = 1.0
    Qf = np.random.default_rng(3).standard_normal((1, 2, 3, d))
    kept = np.arange(k).reshape(1, 1, k)
    r = oracle.output_fidelity(Qf, K, V, kept)
    assert np.allclose(r["cos"], k / math.sqrt(k * k + (n - k) ** 2), atol=1e-14)


def test_dropping_tokens_without_attention_changes_nothing():
    Qf, K, V = _case(4, b=1, h_q=2, h_kv=1)
    q_dir = Qf[0].reshape(-1, Qf.shape[-1]).sum(axis=0)
    # tokens 0..9 get logits about -1e4 below the rest for every query
    K[0, 0, :10] = -1e4 * q_dir / np.linalg.norm(q_dir) ** 2 * 64
    Qf[0] = np.abs(Qf[0]) * np.sign(q_dir)  # every query points along q_dir's orthant
    kept = np.arange(10, K.shape[2]).reshape(1, 1, -1)
    r = oracle.output_fidelity(Qf, K, V, kept)
    assert np.allclose(r["cos"], 1.0, atol=1e-12)


def test_value_scale_and_rotation_leave_cosines_alone():
    Qf, K, V = _case(5)
    kept = np.sort(np.random.default_rng(6).choice(K.shape[2], size=(2, 2, 13), replace=True),
                   axis=-1)
    base = oracle.output_fidelity(Qf, K, V, kept)
    R, _ = np.linalg.qr(np.random.default_rng(7).standard_normal((8, 8)))
    got = oracle.output_fidelity(Qf, K, 3.7 * V @ R, kept)
    assert np.allclose(got["cos"], base["cos"], atol=1e-12)
    assert np.all(base["cos"] < 1.0) and np.all(base["cos"] > -1.0)


def test_zero_output_conventions():
    Qf, K, V = _case(8, b=1, h_q=1, h_kv=1, n=6)
    V[:] = 0.0
    r = oracle.output_fidelity(Qf, K, V, np.array([[[0, 3]]]))
    assert np.all(r["cos"] == 1.0)  # both outputs zero: they agree
    V[0, 0, 5] = 1.0
    r = oracle.output_fidelity(Qf, K, V, np.array([[[0, 3]]]))
    assert np.all(r["cos"] == 0.0)  # the kept output is zero, the full one is not


def test_scalar_loops_on_a_gqa_case():
    Qf, K, V = _case(9, b=1, h_q=4, h_kv=2, n_f=2, n=7, d=3)
    kept = np.array([[[0, 2, 6], [1, 3, 4]]])
    r = oracle.output_fidelity(Qf, K, V, kept)
    d = 3

    def out(q, rows):
        logits = [sum(q[c] * K[0, g, i, c] for c in range(d)) / math.sqrt(d) for i in rows]
        mx = max(logits)
        e = [math.exp(x - mx) for x in logits]
        z = sum(e)
        return [sum(e[j] / z * V[0, g, i, c] for j, i in enumerate(rows)) for c in range(d)]

    for h in range(4):
        g = h // 2
        for f in range(2):
            a = out(Qf[0, h, f], range(7))
            bk = out(Qf[0, h, f], kept[0, g])
            cos = sum(x * y for x, y in zip(a, bk)) / math.sqrt(sum(x * x for x in a) *
                                                               sum(y * y for y in bk))
            assert abs(r["cos"][0, h, f] - cos) < 1e-13
    assert abs(r["fidelity"][0] - np.mean(r["cos"])) < 1e-15
