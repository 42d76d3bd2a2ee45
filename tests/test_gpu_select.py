"""Top-B selection alone on the GPU, from given score arrays, against the
fp64 oracle (LORE-KV page, "Evict and decode", Eq. 8, chunk pooling from the
Hyperparameters table).

The selection runs in two levels (segments of 1024 chunks keep the chunks at
or above their own top-B threshold, then one workgroup per row selects among
the survivors).  These cases cover one segment, many segments, a row whose
survivors overflow the final level's LDS staging (all scores tied), budgets
covering every candidate, and protected ranges that cut chunks.
"""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_eviction_amd as kv
from parity import check_kept

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def run_select(dev, S, n_sink, w, chunk, budget):
    b, hk, n = S.shape
    desc = kv.lore_desc(batch=b, n=n, h_q=hk, h_kv=hk, d=128, d_model=1, w=w, m=0, t=0,
                        n_sink=n_sink, chunk=chunk, budget=budget)
    ws = torch.empty(kv.kvs_topb_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    kept = torch.empty(b, hk, desc.n_keep, dtype=torch.int32, device=dev)
    Sd = S.to(dev).contiguous()
    kv.kvscore_topb_select(desc, Sd, kept, None, ws)
    torch.cuda.synchronize()
    return kept.cpu().numpy()


def check(dev, S, n_sink, w, chunk, budget):
    g = run_select(dev, S, n_sink, w, chunk, budget)
    o, pooled = oracle.topb_select(S.double().numpy(), n_sink=n_sink, w=w, chunk=chunk,
                                   budget=budget)
    return check_kept(g, o, pooled, n_sink, w, budget)


def test_single_segment_random(dev):
    g = torch.Generator().manual_seed(71)
    S = torch.rand(2, 3, 2000, generator=g)
    check(dev, S, n_sink=1, w=32, chunk=4, budget=64)


def test_many_segments_heavy_tail(dev):
    """131072 tokens (32 segments of 1024 chunks), a few large scores."""
    g = torch.Generator().manual_seed(72)
    S = torch.rand(1, 4, 131072, generator=g) * 0.01
    hot = torch.randint(0, 131072, (4, 300), generator=g)
    for r in range(4):
        S[0, r, hot[r]] = torch.rand(300, generator=g) * 5
    check(dev, S, n_sink=1, w=32, chunk=4, budget=128)


def test_all_tied_overflows_final_staging(dev):
    """Equal scores everywhere: every segment keeps all its chunks (16384 >
    the 12288 the final level stages), and the answer is the lowest indices."""
    n, n_sink, w, budget = 65536, 4, 32, 300
    S = torch.full((1, 2, n), 0.5)
    kept = run_select(dev, S, n_sink, w, 4, budget)
    expect = np.concatenate([np.arange(n_sink), np.arange(n_sink, n_sink + budget),
                             np.arange(n - w, n)])
    for row in kept.reshape(-1, kept.shape[-1]):
        assert np.array_equal(row, expect)


def test_budget_covers_all_candidates(dev):
    g = torch.Generator().manual_seed(73)
    S = torch.rand(1, 2, 5000, generator=g)
    check(dev, S, n_sink=3, w=17, chunk=4, budget=5000)


@pytest.mark.parametrize("n,n_sink,w,chunk,budget", [
    (4099, 3, 5, 4, 1000),      # ragged last segment, sink and window cut chunks
    (70000, 2, 31, 4, 9000),    # large budget: survivors of many segments
    (9000, 0, 1, 1, 777),       # chunk 1 (token-level ranking)
    (20000, 1, 32, 8, 257),     # chunk 8
    (4096, 1, 32, 4, 300),      # exactly one segment (1024 chunks): selected in the first level
    (1024, 0, 205, 1, 204),     # the H2O prompt reduction's shape, one segment
    (1030, 3, 7, 5, 1),         # one segment, one candidate kept from a cut chunk
])
def test_edges(dev, n, n_sink, w, chunk, budget):
    g = torch.Generator().manual_seed(n + budget)
    S = torch.rand(1, 2, n, generator=g) ** 4
    check(dev, S, n_sink, w, chunk, budget)


def test_quantized_scores_many_ties(dev):
    """Scores on a coarse grid (multiples of 1/8): ties inside and across
    segments.  With n_sink = 4 and w = 32 on n = 40000 every chunk is whole,
    so each chunk mean (a multiple of 1/32) is exact in fp32 and fp64 alike:
    the ranking is fully determined by (pooled desc, index asc) and the kept
    sets must be identical, not merely equal up to the tie band."""
    g = torch.Generator().manual_seed(74)
    S = torch.randint(0, 8, (1, 3, 40000), generator=g).float() / 8
    kept = run_select(dev, S, 4, 32, 4, 2000)
    o, _ = oracle.topb_select(S.double().numpy(), n_sink=4, w=32, chunk=4, budget=2000)
    assert np.array_equal(kept, o)


@pytest.mark.parametrize("budget", [128, 0, 5000])
def test_retention_shift_matches_oracle(dev, budget):
    """The retention-order shift between two GPU selections over correlated
    scores (a perturbed copy), against the oracle's count on the same kept
    lists: an exact ratio of integers, so the fp32 result is the correctly
    rounded fp64 one.  budget 0 keeps no candidate (shift 0); 5000 keeps
    every candidate of both (shift 0)."""
    g = torch.Generator().manual_seed(75 + budget)
    n, n_sink, w = 4099, 1, 32
    S1 = torch.rand(2, 3, n, generator=g)
    S2 = S1 + 0.3 * torch.rand(2, 3, n, generator=g)
    k1 = run_select(dev, S1, n_sink, w, 4, budget)
    k2 = run_select(dev, S2, n_sink, w, 4, budget)
    shift = torch.empty(2, 3, device=dev)
    kv.kvscore_retention_shift(torch.from_numpy(k1).to(dev), torch.from_numpy(k2).to(dev), shift,
                               n=n, n_sink=n_sink, w=w)
    torch.cuda.synchronize()
    ref = oracle.retention_shift(k1, k2, n_sink=n_sink, w=w, n=n)
    assert np.array_equal(shift.cpu().numpy(), ref.astype(np.float32))
    if budget in (0, 5000):
        assert np.all(ref == 0)
    else:
        assert np.all(ref > 0)


@pytest.mark.parametrize("s_off,p_off", [(0, 0), (1, 0), (0, 3), (2, 1)])
def test_pooled_output_and_misaligned_buffers(dev, s_off, p_off):
    """Scores and pooled output as views that start s_off / p_off floats into
    a larger buffer (4-byte but not 16-byte aligned when nonzero): the pooling
    reads whole 4-token chunks with 16-byte loads only where both buffers
    allow it, so every alignment must give the oracle's kept set and its
    pooled scores (chunk means of the same fp32 scores, summed in token
    order, hence equal to fp32 rounding of the fp64 mean)."""
    g = torch.Generator().manual_seed(76 + 4 * s_off + p_off)
    b, hk, n, n_sink, w, chunk, budget = 1, 3, 9001, 1, 32, 4, 300
    S = torch.rand(b, hk, n, generator=g) ** 3
    desc = kv.lore_desc(batch=b, n=n, h_q=hk, h_kv=hk, d=128, d_model=1, w=w, m=0, t=0,
                        n_sink=n_sink, chunk=chunk, budget=budget)
    ws = torch.empty(kv.kvs_topb_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    kept = torch.empty(b, hk, desc.n_keep, dtype=torch.int32, device=dev)
    sbuf = torch.empty(b * hk * n + 8, device=dev)
    pbuf = torch.full((b * hk * n + 8,), 7.0, device=dev)
    Sd = sbuf[s_off:s_off + b * hk * n].view(b, hk, n)
    Pd = pbuf[p_off:p_off + b * hk * n].view(b, hk, n)
    Sd.copy_(S.to(dev))
    kv.kvscore_topb_select(desc, Sd, kept, Pd, ws)
    torch.cuda.synchronize()
    ko, po = oracle.topb_select(S.double().numpy(), n_sink=n_sink, w=w, chunk=chunk, budget=budget)
    check_kept(kept.cpu().numpy(), ko, po, n_sink, w, budget)
    pg = Pd.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(pg), np.isnan(po)), "pooled NaNs differ from the protected set"
    fin = ~np.isnan(po)
    assert np.all(np.abs(pg[fin] - po[fin]) <= 1e-6 * np.abs(po[fin]) + 1e-37)
    # nothing outside the view was written
    rest = torch.cat([pbuf[:p_off], pbuf[p_off + b * hk * n:]]).cpu()
    assert torch.all(rest == 7.0)


@pytest.mark.parametrize("n,chunk,budget", [(4000, 4, 999), (1024, 1, 205), (600, 3, 100)])
def test_one_segment_ties_exact(dev, n, chunk, budget):
    """Rows of one segment are selected in full by the first level.  Scores on
    a coarse grid with whole chunks (exact chunk means): the kept sets must
    equal the oracle's exactly, ties at the threshold going to the lower
    index, including a threshold chunk that is only partly kept."""
    g = torch.Generator().manual_seed(77 + n)
    n_sink = chunk  # whole chunks only
    w = (n - n_sink) % chunk + chunk  # the window ends the candidates on a chunk edge
    S = torch.randint(0, 6, (2, 3, n), generator=g).float() / 8
    kept = run_select(dev, S, n_sink, w, chunk, budget)
    o, _ = oracle.topb_select(S.double().numpy(), n_sink=n_sink, w=w, chunk=chunk, budget=budget)
    assert np.array_equal(kept, o)
