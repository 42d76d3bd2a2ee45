"""Pins for the oracle's H2O accumulate-and-evict policy (CPU only)."""

import math

import numpy as np
import pytest

import oracle
from conftest import golden


def test_golden_uniform_keys():
    g = golden("h2o_uniform_keys.json")
    P, T = g["prompt"], g["steps"]
    L = P + T
    Q = np.ones((1, L, 1)); K = np.zeros((1, L, 1))
    V = (np.arange(L, dtype=np.float64) + 1.0).reshape(1, L, 1)
    ora = oracle.H2OOracle(Q[:, :P], K[:, :P], V[:, :P], g["heavy_frac"], g["recent_frac"], cap=8)
    np.testing.assert_allclose(ora.prefill_acc[0], g["expected_prefill_acc"], rtol=1e-14)
    assert sorted(ora.retained(0)) == g["expected_kept_prompt"]
    for s in range(T):
        o, _ = ora.attend(Q[:, P + s], K[:, P + s], V[:, P + s])
        assert o[0, 0] == pytest.approx(g["expected_o"][s], rel=1e-14)
        slot = ora.choose()
        pos = int(ora.pos[0, slot[0]]) if slot[0] >= 0 else -1
        assert pos == g["expected_evicted_pos"][s]
        ora.evict(slot)
        exp = {int(k): v for k, v in g["expected_retained_after"][s].items()}
        got = ora.retained(0)
        assert sorted(got) == sorted(exp)
        for p in exp:
            assert got[p] == pytest.approx(exp[p], rel=1e-13)


def test_golden_log_keys():
    """Non-uniform weights: keys ln(p + 1) under unit queries weigh each token
    in proportion to p + 1 (hand-derived fractions in the fixture)."""
    g = golden("h2o_log_keys.json")
    P, T = g["prompt"], g["steps"]
    L = P + T
    Q = np.ones((1, L, 1))
    K = np.log(np.arange(L, dtype=np.float64) + 1.0).reshape(1, L, 1)
    V = (np.arange(L, dtype=np.float64) + 1.0).reshape(1, L, 1)
    ora = oracle.H2OOracle(Q[:, :P], K[:, :P], V[:, :P], g["heavy_frac"], g["recent_frac"], cap=8)
    np.testing.assert_allclose(ora.prefill_acc[0], g["expected_prefill_acc"], rtol=1e-13)
    assert sorted(ora.retained(0)) == g["expected_kept_prompt"]
    for s in range(T):
        o, _ = ora.attend(Q[:, P + s], K[:, P + s], V[:, P + s])
        assert o[0, 0] == pytest.approx(g["expected_o"][s], rel=1e-13)
        slot = ora.choose()
        pos = int(ora.pos[0, slot[0]]) if slot[0] >= 0 else -1
        assert pos == g["expected_evicted_pos"][s]
        ora.evict(slot)
        exp = {int(k): v for k, v in g["expected_retained_after"][s].items()}
        got = ora.retained(0)
        assert sorted(got) == sorted(exp)
        for p in exp:
            assert got[p] == pytest.approx(exp[p], rel=1e-13)


def test_def22_zero_keys_identity():
    """H2O page, Def. 2.2: zeroing evicted keys and subtracting the spurious
    exp(0) = 1 terms gives the softmax over the retained set."""
    rng = np.random.default_rng(0)
    P, d, T = 24, 8, 6
    Qp = rng.standard_normal((2, P, d)); Kp = rng.standard_normal((2, P, d))
    Vp = rng.standard_normal((2, P, d))
    ora = oracle.H2OOracle(Qp, Kp, Vp, 0.2, 0.2, cap=16)
    for _ in range(T):
        q = rng.standard_normal((2, d)); k = rng.standard_normal((2, d)); v = rng.standard_normal((2, d))
        n_before = ora.cur_len
        # full-length key matrix over positions 0..n, evicted rows zeroed
        keys = {}
        for row in range(2):
            kk = np.zeros((n_before + 1, d))
            for s in range(ora.cap):
                if ora.pos[row, s] >= 0:
                    kk[ora.pos[row, s]] = ora.K[row, s]
            kk[n_before] = k[row]
            keys[row] = kk
        retained = [set(ora.retained(row)) | {n_before} for row in range(2)]
        _, probs = ora.attend(q, k, v)
        for row in range(2):
            ev = np.array([0.0 if p in retained[row] else 1.0 for p in range(n_before + 1)])
            num = np.exp(keys[row] @ q[row] / math.sqrt(d)) - ev
            page = num / num.sum()
            mine = np.zeros(n_before + 1)
            for s in range(ora.cap):
                if ora.pos[row, s] >= 0:
                    mine[ora.pos[row, s]] = probs[row, s]
            np.testing.assert_allclose(mine, page, rtol=1e-12, atol=1e-15)
        ora.evict(ora.choose())


def test_no_eviction_equals_one_shot_column_sums():
    """With a budget above the length nothing is evicted, and the running
    accumulators equal the column sums of the full causal attention."""
    rng = np.random.default_rng(1)
    P, T, d = 12, 7, 4
    L = P + T
    Q = rng.standard_normal((3, L, d)); K = rng.standard_normal((3, L, d)); V = rng.standard_normal((3, L, d))
    ora = oracle.H2OOracle(Q[:, :P], K[:, :P], V[:, :P], 0.6, 0.6, cap=L + 2)
    for s in range(T):
        ora.attend(Q[:, P + s], K[:, P + s], V[:, P + s])
        assert np.all(ora.choose() < 0)
    full = oracle.h2o_prefill_acc(Q, K)
    for row in range(3):
        got = ora.retained(row)
        assert sorted(got) == list(range(L))
        np.testing.assert_allclose([got[p] for p in range(L)], full[row], rtol=1e-12)


def test_decode_invariants():
    rng = np.random.default_rng(2)
    P, T, d, rows = 60, 40, 8, 4
    Qp = rng.standard_normal((rows, P, d)); Kp = rng.standard_normal((rows, P, d)) * 1.5
    Vp = rng.standard_normal((rows, P, d))
    ora = oracle.H2OOracle(Qp, Kp, Vp, 0.1, 0.1, cap=24)
    k_h, k_r = oracle.h2o_budget(P, 0.1, 0.1)
    for row in range(rows):
        kept = sorted(ora.retained(row))
        assert len(kept) == k_h + k_r
        assert set(range(P - k_r, P)) <= set(kept)
    for step in range(T):
        q = rng.standard_normal((rows, d)); k = rng.standard_normal((rows, d)); v = rng.standard_normal((rows, d))
        before = [set(ora.retained(r)) for r in range(rows)]
        ora.attend(q, k, v)
        slots = ora.choose()
        k_h, k_r = oracle.h2o_budget(ora.cur_len, 0.1, 0.1)
        for row in range(rows):
            ret = ora.retained(row)
            if slots[row] >= 0:
                p_ev = int(ora.pos[row, slots[row]])
                assert p_ev < ora.cur_len - k_r                     # recent never evicted
                others = [p for p in ret if p < ora.cur_len - k_r and p != p_ev]
                assert all((ret[p_ev], -p_ev) < (ret[p], -p) for p in others)
        ora.evict(slots)
        for row in range(rows):
            after = set(ora.retained(row))
            assert len((before[row] | {ora.cur_len - 1}) - after) <= 1   # at most one eviction
            assert len(after) <= k_h + k_r
            assert set(range(ora.cur_len - k_r, ora.cur_len)) <= after
            # accumulated mass: every query row hands out exactly 1
            mass = sum(ora.retained(row).values()) + ora.evicted_mass[row]
            dropped_at_prefill = ora.prefill_acc[row].sum() - sum(
                ora.prefill_acc[row][p] for p in ora.kept_prompt[row])
            assert mass + dropped_at_prefill == pytest.approx(P + step + 1, rel=1e-12)


def test_tie_evicts_later_position():
    ora = oracle.H2OOracle(np.zeros((1, 10, 2)), np.zeros((1, 10, 2)), np.zeros((1, 10, 2)),
                           0.2, 0.2, cap=8)
    ora.attend(np.zeros((1, 2)), np.zeros((1, 2)), np.zeros((1, 2)))
    # force a tie between two non-recent tokens
    heavy = [s for s in range(ora.cap) if 0 <= ora.pos[0, s] < ora.cur_len - 2]
    for s in heavy:
        ora.acc[0, s] = 0.5
    slot = ora.choose()[0]
    assert ora.pos[0, slot] == max(ora.pos[0, s] for s in heavy)
