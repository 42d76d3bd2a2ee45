"""GPU parity of the H2O path (prefill accumulate -> prompt reduction -> slot
load -> decode steps) against the oracle, in lockstep, through the C ABI.

Lockstep: each decode step, the GPU's evicted position must be the oracle's,
or a near-tie (oracle accumulated scores within 1e-4 relative); the oracle then
evicts what the GPU evicted, so later steps compare from the same cache."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_eviction_amd as kv
from kvsynth import OPT30B_H2O, h2o_inputs, TORCH_DTYPES

pytestmark = pytest.mark.gpu

ACC_RTOL, ACC_ATOL = 1e-3, 1e-7
TIE = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.load()
    return torch.device("cuda")


def _rows(t, rows):
    """[b][H][...] -> [len(rows)][...] for flat (b*H) row indices."""
    f = t.reshape(-1, *t.shape[2:])
    return f[rows]


def _check_prompt_kept(kept_gpu, ora, rows, k_h, k_r, P):
    for i, r in enumerate(rows):
        g = np.sort(kept_gpu[i])
        o = np.sort(ora.own_kept_prompt[i])
        if np.array_equal(g, o):
            continue
        acc = ora.prefill_acc[i]
        cand = np.arange(0, P - k_r)
        order = np.lexsort((cand, -acc[cand]))
        tau = acc[cand[order[k_h - 1]]]
        for p in np.setxor1d(g, o):
            assert abs(acc[p] - tau) <= TIE * tau, "row %d: prompt token %d outside the tie band" % (r, p)


def run_lockstep(cfg, dev, rows, steps, gen_device="cpu"):
    inp = h2o_inputs(cfg, device=gen_device)
    dt = TORCH_DTYPES[cfg.dtype]
    cache = kv.H2OCache(cfg.batch, cfg.heads, cfg.d, cfg.cap, dt, cfg.heavy_frac,
                        cfg.recent_frac, dev)
    Qp, Kp, Vp = (inp[k].to(dev) for k in ("Qp", "Kp", "Vp"))
    cache.prefill(Qp, Kp, Vp)
    torch.cuda.synchronize()
    P = cfg.prompt
    acc_ref = oracle.h2o_prefill_acc(_rows(inp["Qp"], rows).cpu(), _rows(inp["Kp"], rows).cpu())
    acc_gpu = _rows(cache.prompt_acc, rows).cpu().double().numpy()
    np.testing.assert_allclose(acc_gpu, acc_ref, rtol=ACC_RTOL, atol=ACC_ATOL)
    kept_gpu = _rows(cache.kept_prompt, rows).cpu().numpy()
    ora = oracle.H2OOracle(_rows(inp["Qp"], rows).cpu(), _rows(inp["Kp"], rows).cpu(),
                           _rows(inp["Vp"], rows).cpu(), cfg.heavy_frac, cfg.recent_frac,
                           cfg.cap, kept=kept_gpu)
    k_h, k_r = oracle.h2o_budget(P, cfg.heavy_frac, cfg.recent_frac)
    _check_prompt_kept(kept_gpu, ora, rows, k_h, k_r, P)
    ties = 0
    for s in range(steps):
        pos_before = _rows(cache.slot_pos, rows).cpu().numpy()
        q, k, v = (inp[x][s].to(dev) for x in ("q", "k", "v"))
        O, ev = cache.step(q, k, v)
        o_ref, _ = ora.attend(_rows(inp["q"][s], rows).cpu(), _rows(inp["k"][s], rows).cpu(),
                              _rows(inp["v"][s], rows).cpu())
        O = _rows(O, rows).cpu().double().numpy()
        ev = _rows(ev, rows).cpu().numpy()
        pos_after = _rows(cache.slot_pos, rows).cpu().numpy()
        acc_after = _rows(cache.acc, rows).cpu().double().numpy()
        scale = np.abs(o_ref).max(axis=1, keepdims=True)
        assert np.all(np.abs(O - o_ref) <= 2e-3 * scale + 2e-3 * np.abs(o_ref)), \
            "step %d: O err %g" % (s, (np.abs(O - o_ref) / scale).max())
        want = ora.choose()
        adopt = np.full(len(rows), -1, dtype=np.int64)
        for i in range(len(rows)):
            # the GPU wrote the new token into the lowest slot that was free
            ws = int(np.nonzero(pos_before[i] < 0)[0][0])
            gpos = -1
            if ev[i] >= 0:
                gpos = cache.cur_len - 1 if ev[i] == ws else int(pos_before[i][ev[i]])
            opos = int(ora.pos[i, want[i]]) if want[i] >= 0 else -1
            ret = ora.retained(i)
            if gpos != opos:
                assert gpos >= 0 and opos >= 0, "step %d row %d: evicted %d vs %d" % (s, i, gpos, opos)
                assert abs(ret[gpos] - ret[opos]) <= TIE * ret[opos], \
                    "step %d row %d: evicted %d (acc %r) vs oracle %d (acc %r)" % (
                        s, i, gpos, ret[gpos], opos, ret[opos])
                ties += 1
            if gpos >= 0:
                adopt[i] = int(np.nonzero(ora.pos[i] == gpos)[0][0])
            # accumulated scores of the retained cache, before the eviction
            for slot in range(cfg.cap):
                pos = cache.cur_len - 1 if slot == ws else pos_before[i][slot]
                if pos < 0:
                    continue
                assert abs(acc_after[i][slot] - ret[pos]) <= ACC_RTOL * ret[pos] + ACC_ATOL, \
                    "step %d row %d pos %d: acc %r vs %r" % (s, i, pos, acc_after[i][slot], ret[pos])
            kept_after = sorted(int(p) for p in pos_after[i] if p >= 0)
            expect = sorted(p for p in ret if p != gpos)
            assert kept_after == expect, "step %d row %d: retained sets differ" % (s, i)
        ora.evict(adopt)
    return ties


@pytest.mark.parametrize("dtype,d", [("f16", 128), ("f32", 64), ("bf16", 128), ("f16", 64), ("f32", 128)])
def test_small_lockstep(dev, dtype, d):
    cfg = OPT30B_H2O.with_(name="small", batch=2, heads=3, d=d, prompt=200, steps=60,
                           dtype=dtype, seed=31)
    rows = list(range(cfg.batch * cfg.heads))
    ties = run_lockstep(cfg, dev, rows, cfg.steps)
    print("small %s d=%d: near-tie evictions %d" % (dtype, d, ties))


def test_ragged_prompt_lockstep(dev):
    """Prompt length not a multiple of 64, wide budget fractions."""
    cfg = OPT30B_H2O.with_(name="ragged", batch=1, heads=4, prompt=333, steps=40,
                           heavy_frac=0.25, recent_frac=0.15, seed=32)
    run_lockstep(cfg, dev, list(range(4)), cfg.steps)


def test_opt30b_full_sampled_rows(dev):
    """The full 64 x 56 decode (the bench's launch shape), all 512 steps; the
    oracle follows 6 of the 3584 (sequence, head) rows in lockstep."""
    cfg = OPT30B_H2O
    rows = [0, 57, 1000, 2047, 3000, 3583]
    ties = run_lockstep(cfg, dev, rows, cfg.steps, gen_device=dev)
    print("opt30b sampled rows: near-tie evictions %d" % ties)


def test_wide_cache_two_rows_per_group(dev):
    """A slot cache wider than 1365 slots (budget 95% of the length): the
    decode groups two rows per workgroup instead of four, to keep each row's
    probabilities, accumulators and slot map in LDS; three rows leave the
    second group half empty."""
    cfg = OPT30B_H2O.with_(name="wide", batch=1, heads=3, d=64, prompt=1024, steps=440,
                           heavy_frac=0.60, recent_frac=0.35, seed=33)
    assert cfg.cap > 1365
    run_lockstep(cfg, dev, list(range(3)), cfg.steps)


@pytest.mark.parametrize("dtype,d", [("f16", 128), ("bf16", 64), ("f32", 128)])
def test_decode_without_output_keeps_the_same_cache(dev, dtype, d):
    """O is optional: a step without it must leave the slot cache, the slot
    map, the accumulators and the evictions exactly as a step with it."""
    cfg = OPT30B_H2O.with_(name="no-o", batch=2, heads=3, d=d, prompt=200, steps=40,
                           dtype=dtype, seed=34)
    inp = h2o_inputs(cfg, device="cpu")
    dt = TORCH_DTYPES[cfg.dtype]
    caches = [kv.H2OCache(cfg.batch, cfg.heads, cfg.d, cfg.cap, dt, cfg.heavy_frac,
                          cfg.recent_frac, dev) for _ in range(2)]
    Qp, Kp, Vp = (inp[k].to(dev) for k in ("Qp", "Kp", "Vp"))
    for c in caches:
        c.prefill(Qp, Kp, Vp)
    caches[1].O.fill_(7)  # never written without the output
    for s in range(cfg.steps):
        q, k, v = (inp[x][s].to(dev) for x in ("q", "k", "v"))
        caches[0].step(q, k, v, with_output=True)
        caches[1].step(q, k, v, with_output=False)
        torch.cuda.synchronize()
        for name in ("K", "V", "slot_pos", "acc", "evict_slot"):
            a, b = getattr(caches[0], name), getattr(caches[1], name)
            assert torch.equal(a, b), "step %d: %s differs without the output" % (s, name)
    assert bool((caches[1].O == 7).all())
