"""Pins of the counter-causal attention and the memory refresh in the oracle
(counter-causal review "Back from the Future": 3.2 reversed mask over the
cached keys and values, Alg. 3 memory refresh, design choice 4 system-prompt
sinks, the last-token boundary rule of 3.2 Step 5).

Pinned to what the definitions fix independently of the oracle's code: scalar
loops on a tiny GQA case; the second-to-last position sees only the last key,
so its output is that value with a row sum of one; equal keys give the plain
mean of the later values; the last position sees nothing; a hand-worked
refresh; protection that no surprise value can override; J = 0 (the chunked
sliding window) and J >= n; ties to the lower position; and a refresh cycle
whose memory stays empty at J = 0."""

import math

import numpy as np
import pytest

import oracle


def _qkv(seed, b=1, h_q=4, h_kv=2, n=9, d=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((b, h_q, n, d)), rng.standard_normal((b, h_kv, n, d)),
            rng.standard_normal((b, h_kv, n, d)))


def test_scalar_loops_gqa():
    Q, K, V = _qkv(1)
    m, l, O = oracle.counter_causal_attention(Q, K, V)
    n, d = Q.shape[2], Q.shape[3]
    for h in range(4):
        g = h // 2
        for i in range(n - 1):
            logits = [sum(Q[0, h, i, c] * K[0, g, j, c] for c in range(d)) / math.sqrt(d)
                      for j in range(i + 1, n)]
            mx = max(logits)
            e = [math.exp(x - mx) for x in logits]
            z = sum(e)
            assert abs(m[0, h, i] - mx) < 1e-13 and abs(l[0, h, i] - z) < 1e-12
            for c in range(d):
                o = sum(e[k] / z * V[0, g, i + 1 + k, c] for k in range(len(e)))
                assert abs(O[0, h, i, c] - o) < 1e-13


def test_second_to_last_sees_only_the_last_key_and_last_sees_nothing():
    Q, K, V = _qkv(2, b=2)
    m, l, O = oracle.counter_causal_attention(Q, K, V)
    n, d = Q.shape[2], Q.shape[3]
    for h in range(4):
        g = h // 2
        assert np.allclose(O[:, h, n - 2], V[:, g, n - 1], atol=1e-15)
        assert np.allclose(l[:, h, n - 2], 1.0, atol=1e-15)
        assert np.allclose(m[:, h, n - 2], (Q[:, h, n - 2] * K[:, g, n - 1]).sum(-1) / math.sqrt(d))
    assert np.all(m[:, :, n - 1] == -np.inf) and np.all(l[:, :, n - 1] == 0)
    assert np.all(O[:, :, n - 1] == 0)


def test_equal_keys_average_the_later_values():
    Q, K, V = _qkv(3, n=12)
    K[:] = K[:, :, :1]  # every key equal: uniform weights over the visible keys
    _, l, O = oracle.counter_causal_attention(Q, K, V)
    for h in range(4):
        for i in range(11):
            assert np.allclose(O[0, h, i], V[0, h // 2, i + 1:].mean(axis=0), atol=1e-14)
            assert abs(l[0, h, i] - (11 - i)) < 1e-12


def test_refresh_hand_example():
    # n = 8, system prompt 2, keep J = 5: protected {0, 1, 7}; of 2..6 the two
    # largest surprises are positions 5 (0.9) and 3 (0.8)
    s = np.array([[-9.0, -9.0, 0.1, 0.8, 0.2, 0.9, 0.3, -9.0]])
    kept = oracle.refresh_select(s, n_sys=2, J=5)
    assert kept.tolist() == [[0, 1, 3, 5, 7]]


def test_protection_beats_any_surprise():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((3, 40))
    s[:, :3] = -np.inf
    s[:, -1] = -np.inf
    kept = oracle.refresh_select(s, n_sys=3, J=10)
    for row in kept:
        assert {0, 1, 2, 39} <= set(row.tolist())
        assert len(set(row.tolist())) == 10 and list(row) == sorted(row)


def test_budget_edges_and_ties():
    s = np.zeros((2, 6))
    assert oracle.refresh_select(s, n_sys=1, J=0).shape == (2, 0)       # J = 0: nothing kept
    assert oracle.refresh_select(s, n_sys=1, J=9).tolist() == [list(range(6))] * 2  # J >= n
    # all tied: the lowest candidates win
    assert oracle.refresh_select(s, n_sys=1, J=4).tolist() == [[0, 1, 2, 5]] * 2
    with pytest.raises(ValueError):
        oracle.refresh_select(s, n_sys=3, J=3)                          # no room for the last token


def test_gather_keeps_rows_and_ids_together():
    rng = np.random.default_rng(5)
    K = rng.standard_normal((2, 3, 10, 4))
    V = rng.standard_normal((2, 3, 10, 4))
    ids = rng.integers(0, 50000, size=(2, 10))
    kept = np.array([[0, 2, 9], [1, 4, 9]])
    Ko, Vo, Xo = oracle.refresh_gather(K, V, ids, kept)
    for bb in range(2):
        for r, src in enumerate(kept[bb]):
            assert np.array_equal(Ko[bb, :, r], K[bb, :, src])
            assert np.array_equal(Vo[bb, :, r], V[bb, :, src])
            assert Xo[bb, r] == ids[bb, src]


@pytest.mark.parametrize("J,h", [(0, 4), (8, 2), (12, 3)])
def test_refresh_cycle_memory(J, h):
    # the inference/refresh cycle on positions: memory J, buffer h.  At J = 0
    # nothing survives a refresh (the chunked sliding window); otherwise the
    # memory never exceeds J, the system prompt never leaves, and the newest
    # token always survives its refresh.
    rng = np.random.default_rng(6)
    n_sys = 0 if J == 0 else 2
    memory = list(range(n_sys))
    buffer = []
    for pos in range(n_sys, 60):
        buffer.append(pos)
        if len(buffer) == h:
            cache = memory + buffer
            s = rng.standard_normal((1, len(cache)))
            kept = oracle.refresh_select(s, n_sys=n_sys, J=J)[0]
            memory = [cache[k] for k in kept]
            buffer = []
            if J == 0:
                assert memory == []
            else:
                assert len(memory) == min(J, len(cache))
                assert memory[:n_sys] == list(range(n_sys)) and memory[-1] == pos
