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


# unit roundoff of the output element type: O is stored in the cache's dtype
O_ROUND = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8, "f32": 2.0 ** -24}


def _sorted_by_pos(pos, vals):
    """Per row, the valid positions ascending and their values (empty slots,
    position -1, sort to the end)."""
    key = np.where(pos >= 0, pos, np.iinfo(np.int64).max)
    order = np.argsort(key, axis=1, kind="stable")
    return np.take_along_axis(key, order, 1), np.take_along_axis(vals, order, 1)


def run_lockstep(cfg, dev, rows, steps, gen_device="cpu", write_last_free=False):
    """Prefill, prompt reduction and `steps` decode steps on the GPU for every
    row of cfg; the oracle follows `rows` in lockstep.  Per step: O within
    1e-3 of the row's largest component plus the rounding of O's storage type
    (a half ulp of |o|), the accumulated score of every retained token within
    1e-3 relative, the evicted position equal to the oracle's (or at a near
    tie, which the oracle then adopts) and the retained sets equal.  With
    write_last_free each new token goes into the highest free slot through
    write_slot (the default is the lowest)."""
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
    R = len(rows)
    ar = np.arange(R)
    o_round = O_ROUND[cfg.dtype]
    ties = 0
    for s in range(steps):
        pos_before = _rows(cache.slot_pos, rows).cpu().numpy().astype(np.int64)
        q, k, v = (inp[x][s].to(dev) for x in ("q", "k", "v"))
        wslot = None
        if write_last_free:
            slot_idx = torch.arange(cfg.cap, device=dev, dtype=torch.int32).expand_as(cache.slot_pos)
            wslot = torch.where(cache.slot_pos < 0, slot_idx, -1).amax(dim=-1).to(torch.int32)
        O, ev = cache.step(q, k, v, write_slot=wslot)
        o_ref, _ = ora.attend(_rows(inp["q"][s], rows).cpu(), _rows(inp["k"][s], rows).cpu(),
                              _rows(inp["v"][s], rows).cpu())
        O = _rows(O, rows).cpu().double().numpy()
        ev = _rows(ev, rows).cpu().numpy().astype(np.int64)
        pos_after = _rows(cache.slot_pos, rows).cpu().numpy().astype(np.int64)
        acc_after = _rows(cache.acc, rows).cpu().double().numpy()
        scale = np.abs(o_ref).max(axis=1, keepdims=True)
        bound = 1e-3 * scale + o_round * np.abs(o_ref)
        assert np.all(np.abs(O - o_ref) <= bound), \
            "step %d: O err %g of the row max" % (s, (np.abs(O - o_ref) / scale).max())
        # the GPU wrote the new token into the lowest slot that was free (or the
        # highest, through write_slot)
        free = pos_before < 0
        assert free.any(axis=1).all(), "step %d: a row had no free slot" % s
        ws = (cfg.cap - 1 - free[:, ::-1].argmax(axis=1)) if write_last_free else free.argmax(axis=1)
        gpos_slots = pos_before.copy()
        gpos_slots[ar, ws] = cache.cur_len - 1
        # retained set and accumulated scores before the eviction
        gk, gacc = _sorted_by_pos(gpos_slots, acc_after)
        ok, oacc = _sorted_by_pos(ora.pos, ora.acc)
        assert np.array_equal(gk, ok), "step %d: retained sets differ before the eviction" % s
        valid = gk != np.iinfo(np.int64).max
        aerr = np.abs(gacc - oacc)
        assert np.all(aerr[valid] <= ACC_RTOL * oacc[valid] + ACC_ATOL), \
            "step %d: acc err %g" % (s, (aerr[valid] / np.maximum(oacc[valid], 1e-30)).max())
        # evicted positions, in lockstep
        gpos = np.where(ev >= 0, gpos_slots[ar, np.maximum(ev, 0)], -1)
        want = ora.choose()
        opos = np.where(want >= 0, ora.pos[ar, np.maximum(want, 0)], -1)
        adopt = np.full(R, -1, dtype=np.int64)
        for i in np.nonzero(gpos != opos)[0]:
            assert gpos[i] >= 0 and opos[i] >= 0, \
                "step %d row %d: evicted %d vs %d" % (s, rows[i], gpos[i], opos[i])
            ag = ora.acc[i, np.nonzero(ora.pos[i] == gpos[i])[0][0]]
            ao = ora.acc[i, want[i]]
            assert abs(ag - ao) <= TIE * ao, "step %d row %d: evicted %d (acc %r) vs oracle %d (acc %r)" % (
                s, rows[i], gpos[i], ag, opos[i], ao)
            ties += 1
        for i in np.nonzero(gpos >= 0)[0]:
            adopt[i] = np.nonzero(ora.pos[i] == gpos[i])[0][0]
        ora.evict(adopt)
        assert np.array_equal(np.sort(pos_after, axis=1), np.sort(ora.pos, axis=1)), \
            "step %d: retained sets differ after the eviction" % s
    return ties


@pytest.mark.parametrize("dtype,d", [("f16", 128), ("f32", 64), ("bf16", 128), ("f16", 64), ("f32", 128)])
def test_small_lockstep(dev, dtype, d):
    cfg = OPT30B_H2O.with_(name="small", batch=2, heads=3, d=d, prompt=200, steps=60,
                           dtype=dtype, seed=31)
    rows = list(range(cfg.batch * cfg.heads))
    ties = run_lockstep(cfg, dev, rows, cfg.steps)
    print("small %s d=%d: near-tie evictions %d" % (dtype, d, ties))


def test_write_slot_lockstep(dev):
    """The caller picks each row's slot (here the highest free one instead of
    the default lowest): the same retained sets, accumulators and evictions
    by position, in lockstep with the oracle."""
    cfg = OPT30B_H2O.with_(name="write-slot", batch=2, heads=3, prompt=200, steps=60, seed=36)
    run_lockstep(cfg, dev, list(range(cfg.batch * cfg.heads)), cfg.steps, write_last_free=True)


def test_write_slot_not_free_leaves_row_unchanged(dev):
    """A write_slot that is occupied, or outside [0, cap), leaves its row's
    cache, slot map and accumulators exactly as they were and reports -2;
    the other rows step normally."""
    cfg = OPT30B_H2O.with_(name="bad-slot", batch=1, heads=4, prompt=200, steps=2, seed=37)
    inp = h2o_inputs(cfg, device="cpu")
    cache = kv.H2OCache(cfg.batch, cfg.heads, cfg.d, cfg.cap, torch.float16, cfg.heavy_frac,
                        cfg.recent_frac, dev)
    cache.prefill(*(inp[k].to(dev) for k in ("Qp", "Kp", "Vp")))
    torch.cuda.synchronize()
    before = {n: getattr(cache, n).clone() for n in ("K", "V", "slot_pos", "acc")}
    # rows: occupied slot 0, slot cap (out of range), slot -1, a free slot
    free0 = int((before["slot_pos"][0, 3] < 0).nonzero()[0, 0])
    wslot = torch.tensor([[0, cfg.cap, -1, free0]], dtype=torch.int32, device=dev)
    q, k, v = (inp[x][0].to(dev) for x in ("q", "k", "v"))
    _, ev = cache.step(q, k, v, write_slot=wslot)
    torch.cuda.synchronize()
    assert ev[0, :3].tolist() == [-2, -2, -2]
    for n in ("K", "V", "slot_pos", "acc"):
        assert torch.equal(getattr(cache, n)[0, :3], before[n][0, :3]), n
    assert int(cache.slot_pos[0, 3, free0]) == cache.cur_len - 1
    assert int(ev[0, 3]) != -2


def test_ragged_prompt_lockstep(dev):
    """Prompt length not a multiple of 64, wide budget fractions."""
    cfg = OPT30B_H2O.with_(name="ragged", batch=1, heads=4, prompt=333, steps=40,
                           heavy_frac=0.25, recent_frac=0.15, seed=32)
    run_lockstep(cfg, dev, list(range(4)), cfg.steps)


@pytest.mark.parametrize("dtype", ["f16", "f32"])
@pytest.mark.parametrize("prompt,heavy,recent", [(2048, 0.1, 0.1), (3000, 0.2, 0.1)],
                         ids=["p2048", "p3000-ragged"])
def test_long_prompt_lockstep(dev, prompt, heavy, recent, dtype):
    """Prompts beyond 1024 tokens (the H2O page's long-sequence runs use 2048
    and more).  16-bit prompts run the paired-block rows and column-sum
    passes; fp32 prompts the general attention pass, whose column-sum pass
    then runs several head-subset launches from the last rows to the first
    while the attention pass's workgroups stop at their rows' last key.
    P = 3000 is not a multiple of 64."""
    cfg = OPT30B_H2O.with_(name="long", batch=2, heads=3, prompt=prompt, steps=48,
                           heavy_frac=heavy, recent_frac=recent, seed=35, dtype=dtype)
    run_lockstep(cfg, dev, list(range(cfg.batch * cfg.heads)), cfg.steps)


def test_opt30b_full_sampled_rows(dev):
    """The full 64 x 56 decode (the bench's launch shape), all 512 steps; the
    oracle follows 65 of the 3584 (sequence, head) rows in lockstep: one row
    of every sequence, head 23*b mod 56 of sequence b (every head once over
    the first 56 sequences), plus the first and last row."""
    cfg = OPT30B_H2O
    rows = sorted({b * cfg.heads + (23 * b) % cfg.heads for b in range(cfg.batch)} |
                  {0, cfg.batch * cfg.heads - 1})
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


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f16", 128)])
@pytest.mark.parametrize("P", [1, 2, 63, 64, 65, 127, 129, 300, 1000])
def test_prefill_accumulate_block_edges(dev, dtype, d, P):
    """The causal prompt accumulate alone at prompt lengths around the 64-row
    blocks, where the 16-bit kernels pair block p with block nb-1-p (nb = 1,
    2, 3 and ragged last blocks, odd and even nb): acc against the oracle's
    column sums, and two calls bit-identical (rows are added in a fixed
    order)."""
    b, h = 2, 3
    g = torch.Generator().manual_seed(1000 + P)
    Qp = torch.randn(b, h, P, d, generator=g)
    Kp = torch.randn(b, h, P, d, generator=g)
    Kp[:, :, ::7] *= 3.0  # a few heavy keys
    dt = TORCH_DTYPES[dtype]
    Qd, Kd = Qp.to(dt).to(dev), Kp.to(dt).to(dev)
    desc = kv.h2o_desc(batch=b, heads=h, d=d, cap=P, dtype=dt)
    ws = torch.empty(max(1, kv.kvs_h2o_workspace_bytes(desc, kv.KVS_H2O_PREFILL)), dtype=torch.uint8,
                     device=dev)
    accs = []
    for _ in range(2):
        acc = torch.full((b, h, P), float("nan"), dtype=torch.float32, device=dev)
        kv.kvscore_h2o_accumulate(desc, kv.KVS_H2O_PREFILL, Qd, Kd, acc=acc, ws=ws)
        torch.cuda.synchronize()
        accs.append(acc.cpu())
    ref = oracle.h2o_prefill_acc(Qd.cpu().double(), Kd.cpu().double())
    np.testing.assert_allclose(accs[0].double().numpy(), ref, rtol=ACC_RTOL, atol=ACC_ATOL)
    assert torch.equal(accs[0], accs[1])


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_prefill_accumulate_longest_prompt(dev, dt):
    """The longest prompt the prefill takes (16384 tokens): acc of one
    (sequence, head) row against the oracle.  16-bit prompts run 128
    row-block pairs; fp32 prompts the general attention pass and 32
    column-sum launches."""
    P, d = 16384, 128
    g = torch.Generator().manual_seed(16384)
    Qp = torch.randn(1, 1, P, d, generator=g)
    Kp = torch.randn(1, 1, P, d, generator=g)
    Kp[:, :, ::11] *= 3.0
    Qd, Kd = Qp.to(dt).to(dev), Kp.to(dt).to(dev)
    desc = kv.h2o_desc(batch=1, heads=1, d=d, cap=P, dtype=dt)
    ws = torch.empty(kv.kvs_h2o_workspace_bytes(desc, kv.KVS_H2O_PREFILL), dtype=torch.uint8, device=dev)
    acc = torch.full((1, 1, P), float("nan"), dtype=torch.float32, device=dev)
    kv.kvscore_h2o_accumulate(desc, kv.KVS_H2O_PREFILL, Qd, Kd, acc=acc, ws=ws)
    torch.cuda.synchronize()
    ref = oracle.h2o_prefill_acc(Qd.cpu().double(), Kd.cpu().double())
    np.testing.assert_allclose(acc.cpu().double().numpy(), ref, rtol=ACC_RTOL, atol=ACC_ATOL)


def test_widest_cache_lockstep(dev):
    """The widest slot cache the decode takes (2048 slots: two rows per
    workgroup, each row's arrays 24 KB of LDS), prompt 2054 tokens, budget
    95% of the length, 100 steps in lockstep."""
    cfg = OPT30B_H2O.with_(name="widest", batch=1, heads=2, d=128, prompt=2054, steps=100,
                           heavy_frac=0.50, recent_frac=0.45, seed=35)
    assert cfg.cap == 2048
    run_lockstep(cfg, dev, list(range(2)), cfg.steps)


def test_decode_on_concurrent_streams_matches_sequential(dev):
    """Two slot caches stepped on two streams at once give bit for bit what
    stepping them one after the other gives: the decode keeps no state
    outside the caller's buffers."""
    cfg = OPT30B_H2O.with_(name="streams", batch=2, heads=3, prompt=300, steps=40, seed=37)
    dt = TORCH_DTYPES[cfg.dtype]
    inps = [h2o_inputs(cfg.with_(seed=37 + i), device="cpu") for i in range(2)]

    def fresh():
        cs = [kv.H2OCache(cfg.batch, cfg.heads, cfg.d, cfg.cap, dt, cfg.heavy_frac,
                          cfg.recent_frac, dev) for _ in range(2)]
        for c, inp in zip(cs, inps):
            c.prefill(*(inp[k].to(dev) for k in ("Qp", "Kp", "Vp")))
        torch.cuda.synchronize()
        return cs

    seq, con = fresh(), fresh()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in range(cfg.steps):
        step_in = [tuple(inp[x][s].to(dev) for x in ("q", "k", "v")) for inp in inps]
        for c, (q, k, v) in zip(seq, step_in):
            c.step(q, k, v)
        outs_seq = [c.O.clone() for c in seq]
        torch.cuda.synchronize()
        for st in streams:
            st.wait_stream(torch.cuda.current_stream())
        for c, (q, k, v), st in zip(con, step_in, streams):
            with torch.cuda.stream(st):
                c.step(q, k, v, stream=st)
        torch.cuda.synchronize()
        for i in range(2):
            for name in ("K", "V", "slot_pos", "acc", "evict_slot"):
                assert torch.equal(getattr(seq[i], name), getattr(con[i], name)), \
                    "step %d cache %d: %s differs on concurrent streams" % (s, i, name)
            assert torch.equal(outs_seq[i], con[i].O), "step %d cache %d: O differs" % (s, i)
