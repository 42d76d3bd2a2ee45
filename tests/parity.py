"""Comparison rules between the HIP path and the oracle (shared by GPU tests).

Scores: for candidate tokens |S_gpu - S_ora| <= 1e-3 |S_ora| + 1e-6 max S_ora
(fp32 accumulation; the absolute floor only covers values far below the
row's scale).  Kept sets: same size; every index in the symmetric difference
must sit at a near-tie, its oracle pooled score within 1e-4 relative of the
oracle's B-th ranked pooled score.  Compaction: bit-exact copy of the rows the
GPU selected.  Softmax statistics: 1e-5 relative; attention outputs: within
1e-3 of the row's largest component.
"""

import numpy as np
import torch

SCORE_RTOL = 1e-3
SCORE_FLOOR = 1e-6
TIE_BAND = 1e-4


def lore_desc_kwargs(cfg):
    return dict(batch=cfg.batch, n=cfg.n, h_q=cfg.h_q, h_kv=cfg.h_kv, d=cfg.d,
                d_model=cfg.d_model, w=cfg.w, m=cfg.m, t=cfg.t, n_sink=cfg.n_sink,
                chunk=cfg.chunk, budget=cfg.budget, eps=cfg.eps, lambda_l=cfg.lambda_l)


def check_stats(m_gpu, l_gpu, O_gpu, m_ora, l_ora, O_ora, o_rtol=1e-3):
    m_gpu, l_gpu, O_gpu = (np.asarray(x, dtype=np.float64) for x in (m_gpu, l_gpu, O_gpu))
    dm = np.abs(m_gpu - m_ora)
    dl = np.abs(l_gpu - l_ora) / l_ora
    assert np.all(dm <= 1e-5 * np.abs(m_ora) + 1e-6), "row_max err %g" % dm.max()
    assert dl.max() <= 1e-5, "row_sum rel err %g" % dl.max()
    scale = np.abs(O_ora).max(axis=-1, keepdims=True)
    do = np.abs(O_gpu - O_ora) / scale
    assert do.max() <= o_rtol, "O err %g (rel to row max)" % do.max()
    return dict(m=dm.max(), l=dl.max(), O=do.max())


def check_scores(S_gpu, S_ora, n_sink, w):
    S_gpu = np.asarray(S_gpu, dtype=np.float64)
    n = S_ora.shape[-1]
    cand = slice(n_sink, n - w)
    sg, so = S_gpu[..., cand], S_ora[..., cand]
    floor = SCORE_FLOOR * np.abs(S_ora).max(axis=-1, keepdims=True)
    err = np.abs(sg - so)
    bound = SCORE_RTOL * np.abs(so) + floor
    worst = (err / np.maximum(np.abs(so), 1e-300)).max() if so.size else 0.0
    assert np.all(err <= bound), "score err: %d violations, max rel %g" % (
        int((err > bound).sum()), worst)
    return worst


def check_kept(kept_gpu, kept_ora, pooled_ora, n_sink, w, budget):
    kept_gpu = np.asarray(kept_gpu)
    assert kept_gpu.shape == kept_ora.shape, (kept_gpu.shape, kept_ora.shape)
    flat_g = kept_gpu.reshape(-1, kept_gpu.shape[-1])
    flat_o = kept_ora.reshape(-1, kept_ora.shape[-1])
    flat_p = pooled_ora.reshape(-1, pooled_ora.shape[-1])
    n = flat_p.shape[-1]
    n_diff = 0
    for row in range(flat_g.shape[0]):
        g, o = flat_g[row], flat_o[row]
        assert np.all(np.diff(g) > 0), "kept not strictly ascending"
        if np.array_equal(g, o):
            continue
        cand = np.arange(n_sink, n - w)
        B = min(budget, cand.size)
        order = np.lexsort((cand, -flat_p[row, cand]))
        tau = flat_p[row, cand[order[B - 1]]]
        diff = np.setxor1d(g, o)
        for i in diff:
            assert n_sink <= i < n - w, "protected token %d differs" % i
            assert abs(flat_p[row, i] - tau) <= TIE_BAND * abs(tau), (
                "token %d (pooled %r) differs outside the tie band of tau %r" % (i, flat_p[row, i], tau))
        n_diff += diff.size
    return n_diff


def check_compaction(K, V, kept, Kc, Vc):
    K, V, Kc, Vc = (x.view(torch.int16) if x.dtype in (torch.bfloat16, torch.float16) else
                    x.view(torch.int32) for x in (K, V, Kc, Vc))
    idx = kept.long()[..., None].expand(*kept.shape, K.shape[-1])
    assert torch.equal(torch.gather(K, 2, idx), Kc)
    assert torch.equal(torch.gather(V, 2, idx), Vc)
