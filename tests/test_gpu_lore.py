"""GPU parity of the LORE-KV path (probs -> deletion -> top-B -> compaction)
against the fp64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_eviction_amd as kv
from kvsynth import (TINY, MISTRAL_16K, LLAMA_128K, QWEN_14B_BATCH, lore_inputs, TORCH_DTYPES)
from parity import (lore_desc_kwargs, check_stats, check_scores, check_kept, check_compaction)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.load()
    return torch.device("cuda")


def run_gpu(cfg, inp, dev):
    desc = kv.lore_desc(dtype=TORCH_DTYPES[cfg.dtype], **lore_desc_kwargs(cfg))
    ev = kv.LoreEviction(desc, dev)
    Q, K, V, W, om = (inp[k].to(dev).contiguous() for k in ("Q", "K", "V", "W_O", "omega"))
    ev.score(Q, K, V, W, om)
    pooled = torch.empty_like(ev.S)
    ev.select(pooled)
    b, hk, nk, d = cfg.batch, cfg.h_kv, desc.n_keep, cfg.d
    Kc = torch.empty(b, hk, nk, d, dtype=K.dtype, device=dev)
    Vc = torch.empty_like(Kc)
    pos = torch.empty(b, hk, nk, dtype=torch.int32, device=dev)
    ev.compact(K, V, Kc, Vc, pos)
    torch.cuda.synchronize()
    check_compaction(K, V, ev.kept, Kc, Vc)
    assert torch.equal(pos, ev.kept)
    return {k: getattr(ev, k).cpu().numpy() for k in ("row_max", "row_sum", "O", "S", "kept")} | \
        {"pooled": pooled.cpu().numpy()}


def run_oracle(cfg, inp):
    r = oracle.lore_scores(inp["Q"], inp["K"], inp["V"], inp["W_O"], inp["omega"], w=cfg.w,
                           m=cfg.m, t=cfg.t, eps=cfg.eps, lambda_l=cfg.lambda_l)
    kept, pooled = oracle.topb_select(r["S"], n_sink=cfg.n_sink, w=cfg.w, chunk=cfg.chunk,
                                      budget=cfg.budget)
    r["kept"], r["pooled"] = kept, pooled
    return r


def compare(cfg, g, o, o_rtol=1e-3):
    st = check_stats(g["row_max"], g["row_sum"], g["O"], o["row_max"], o["row_sum"], o["O"], o_rtol)
    worst = check_scores(g["S"], o["S"], cfg.n_sink, cfg.w)
    nd = check_kept(g["kept"], o["kept"], o["pooled"], cfg.n_sink, cfg.w, cfg.budget)
    check_pooled(cfg, g)
    print("%s: stats %s, worst score rel err %.3g, kept diffs at ties %d" % (cfg.name, st, worst, nd))


def check_pooled(cfg, g):
    """The selector's pooled scores against the oracle's pooling of the same
    (GPU) scores: NaN on exactly the protected tokens, and each candidate's
    chunk mean to fp32 rounding of a sum of at most `chunk` terms."""
    Pg = g["pooled"].astype(np.float64)
    Po = oracle.pooled_scores(g["S"].astype(np.float64), cfg.n_sink, cfg.w, cfg.chunk)
    assert np.array_equal(np.isnan(Pg), np.isnan(Po)), "pooled NaNs differ from the protected set"
    fin = ~np.isnan(Po)
    err = np.abs(Pg[fin] - Po[fin])
    assert np.all(err <= 1e-6 * np.abs(Po[fin]) + 1e-37), "pooled score error %g" % err.max()


def test_tiny_fp32(dev):
    inp = lore_inputs(TINY)
    g = run_gpu(TINY, inp, dev)
    o = run_oracle(TINY, inp)
    compare(TINY, g, o, o_rtol=1e-5)
    assert np.array_equal(g["kept"], o["kept"])


SMALL = [
    TINY.with_(name="bf16-d128-g4-n1000", dtype="bf16", d=128, h_q=8, h_kv=2, n=1000,
               d_model=512, budget=64, seed=11),
    TINY.with_(name="f16-d64-mha-n777-nq11", dtype="f16", d=64, h_q=3, h_kv=3, n=777,
               d_model=192, w=5, m=2, t=3, chunk=1, budget=50, n_sink=2, seed=12),
    TINY.with_(name="bf16-d128-g5-b2-n2085", dtype="bf16", d=128, h_q=10, h_kv=2, n=2085,
               d_model=1280, budget=100, batch=2, seed_per_seq=True, omega_per_seq=True, seed=13),
    MISTRAL_16K.with_(name="f32-d128-g2-b2-n300", dtype="f32", h_q=4, h_kv=2, n=300,
                      d_model=512, batch=2, budget=40, seed=14),
    TINY.with_(name="bf16-d64-g8-n4096", dtype="bf16", d=64, h_q=8, h_kv=1, n=4096,
               d_model=512, seed=15),
    TINY.with_(name="bf16-d128-g16-n600", dtype="bf16", d=128, h_q=16, h_kv=1, n=600,
               d_model=2048, budget=30, seed=16, window_from_facts=False),
    # one KV head over a long cache: pass 1 runs 79 (and 40) token splits, so
    # the merge holds 8 split weights per thread in registers and reads the
    # rest again, and takes the partial O in several rounds of 32
    TINY.with_(name="bf16-d128-g4-n40000-79splits", dtype="bf16", d=128, h_q=4, h_kv=1,
               n=40000, d_model=512, budget=200, seed=19),
    TINY.with_(name="f16-d64-g2-n20000-40splits", dtype="f16", d=64, h_q=2, h_kv=1, n=20000,
               d_model=128, budget=100, seed=20),
    # fp16 inputs through the 16-bit MFMA paths over many tiles and splits
    TINY.with_(name="f16-d128-g4-n16384", dtype="f16", d=128, h_q=8, h_kv=2, n=16384,
               d_model=1024, budget=256, seed=21),
    # fp32 inputs over many tiles and splits (d 64, GQA 2, a ragged tail)
    TINY.with_(name="f32-d64-g2-n9001", dtype="f32", d=64, h_q=4, h_kv=2, n=9001,
               d_model=256, budget=200, seed=22),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small_shapes(dev, cfg):
    inp = lore_inputs(cfg)
    compare(cfg, run_gpu(cfg, inp, dev), run_oracle(cfg, inp))


@pytest.mark.parametrize("lam,omega_1", [(1e-40, None), (1.0, 1e-39)],
                         ids=["subnormal-lambda", "underflowed-omega"])
def test_subnormal_row_weights(dev, lam, omega_1):
    """Row weights below FLT_MIN -- a subnormal lambda_L, or one trajectory's
    omega entry that underflowed in the softmax -- contribute nothing on the
    GPU: every score stays finite (1/w_r would overflow) and within the bar
    of the oracle, whose terms of that size lie far below the scores' own
    rounding."""
    cfg = TINY.with_(name="subnormal-w", dtype="bf16", d=128, h_q=8, h_kv=2, n=1000,
                     d_model=512, budget=64, seed=17, lambda_l=lam)
    inp = lore_inputs(cfg)
    if omega_1 is not None:
        inp["omega"][:, 1] = omega_1
    g = run_gpu(cfg, inp, dev)
    assert np.isfinite(g["S"]).all()
    compare(cfg, g, run_oracle(cfg, inp))


def test_probs_without_mask(dev):
    """KVS_MASK_NONE: every scoring row sees all n tokens, so the statistics
    are the oracle's with no causal window rows (w = 0 in its visibility);
    the window rows' statistics differ from the window-causal ones."""
    cfg = TINY.with_(name="mask-none", dtype="bf16", d=128, h_q=8, h_kv=2, n=1000, d_model=512,
                     seed=18)
    inp = lore_inputs(cfg)
    desc = kv.lore_desc(dtype=TORCH_DTYPES[cfg.dtype], **lore_desc_kwargs(cfg))
    Q, K, V = (inp[k].to(dev).contiguous() for k in ("Q", "K", "V"))
    b, hq, nq, d = Q.shape
    outs = {}
    for mask in (kv.KVS_MASK_NONE, kv.KVS_MASK_WINDOW_CAUSAL):
        m = torch.empty(b, hq, nq, device=dev)
        l = torch.empty_like(m)
        O = torch.empty(b, hq, nq, d, device=dev)
        ws = torch.empty(kv.kvs_lore_workspace_bytes(desc), dtype=torch.uint8, device=dev)
        kv.kvscore_probs(desc, Q, K, V, m, l, O, ws, mask=mask)
        torch.cuda.synchronize()
        outs[mask] = (m.cpu().numpy(), l.cpu().numpy(), O.cpu().numpy())
    m_o, l_o, O_o = oracle.lore_attention(inp["Q"], inp["K"], inp["V"], 0)
    check_stats(*outs[kv.KVS_MASK_NONE], m_o, l_o, O_o)
    assert not np.allclose(outs[kv.KVS_MASK_NONE][1][..., :cfg.w],
                           outs[kv.KVS_MASK_WINDOW_CAUSAL][1][..., :cfg.w])


PROB_CASES = [
    (TINY, 1),
    (TINY.with_(name="bf16-d128-g4-n1000", dtype="bf16", d=128, h_q=8, h_kv=2, n=1000,
                d_model=512, seed=19), 1),
    (TINY.with_(name="f16-d64-mha-n777-nq11", dtype="f16", d=64, h_q=3, h_kv=3, n=777,
                d_model=192, w=5, m=2, t=3, seed=20), 0),
    (TINY.with_(name="bf16-d64-g2-b2-n300", dtype="bf16", d=64, h_q=4, h_kv=2, n=300, batch=2,
                d_model=256, seed_per_seq=True, omega_per_seq=True, seed=21), 1),
]


@pytest.mark.parametrize("cfg,mask", PROB_CASES, ids=[c.name + "-mask%d" % m for c, m in PROB_CASES])
def test_dense_probabilities(dev, cfg, mask):
    """The optional dense probabilities P of kvscore_probs against the oracle's
    softmax written out directly: hidden tokens exactly 0, visible ones within
    5e-4 relative (the row statistics carry 1e-5 of the logit scale, and the
    exponent amplifies an absolute logit error into a relative one) plus a
    1e-9 floor for probabilities near fp32 underflow."""
    inp = lore_inputs(cfg)
    desc = kv.lore_desc(dtype=TORCH_DTYPES[cfg.dtype], **lore_desc_kwargs(cfg))
    Q, K, V = (inp[k].to(dev).contiguous() for k in ("Q", "K", "V"))
    b, hq, nq, d = Q.shape
    m = torch.empty(b, hq, nq, device=dev)
    l = torch.empty_like(m)
    O = torch.empty(b, hq, nq, d, device=dev)
    P = torch.full((b, hq, nq, cfg.n), 7.0, device=dev)
    ws = torch.empty(kv.kvs_lore_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    kv.kvscore_probs(desc, Q, K, V, m, l, O, ws, mask=mask, P=P)
    torch.cuda.synchronize()
    w = cfg.w if mask == kv.KVS_MASK_WINDOW_CAUSAL else 0
    ref = oracle.lore_probabilities(inp["Q"], inp["K"], w)
    Pg = P.cpu().double().numpy()
    hidden = np.zeros(ref.shape, dtype=bool)
    for r in range(min(w, nq)):
        hidden[:, :, r, cfg.n - w + r + 1:] = True
    assert np.all(Pg[hidden] == 0)
    err = np.abs(Pg - ref)[~hidden]
    bound = 5e-4 * ref[~hidden] + 1e-9
    assert np.all(err <= bound), "P err %g (rel)" % (err / np.maximum(ref[~hidden], 1e-30)).max()
    assert np.allclose(Pg.sum(axis=-1), 1.0, atol=1e-4)


def test_mistral_16k_full(dev):
    inp = lore_inputs(MISTRAL_16K)
    compare(MISTRAL_16K, run_gpu(MISTRAL_16K, inp, dev), run_oracle(MISTRAL_16K, inp))


@pytest.mark.parametrize("cfg,layer", [(LLAMA_128K, 0), (LLAMA_128K, 31), (QWEN_14B_BATCH, 0)],
                         ids=["llama128k-layer0", "llama128k-layer31", "qwen14b-batch"])
def test_full_size_every_head(dev, cfg, layer):
    """Full-size launch (the bench's configuration) checked completely against
    the oracle: every (sequence, KV head) unit -- all 8 KV heads of a 131072-token
    Llama layer (an early and a late layer: their inputs are drawn from
    different seeds), all 64 (sequence, KV head) units of the Qwen batch --
    with every candidate score, every kept set, the pooled scores and the
    softmax statistics and outputs of every query head."""
    inp = lore_inputs(cfg, layer=layer, device=dev)
    g = run_gpu(cfg, inp, dev)
    o = run_oracle(cfg, {k: inp[k].cpu() for k in ("Q", "K", "V", "W_O", "omega")})
    compare(cfg, g, o)


def _edge_case(dev, cfg, inp):
    g, o = run_gpu(cfg, inp, dev), run_oracle(cfg, inp)
    check_scores(g["S"], o["S"], cfg.n_sink, cfg.w)
    check_kept(g["kept"], o["kept"], o["pooled"], cfg.n_sink, cfg.w, cfg.budget)
    return g, o


@pytest.mark.parametrize("n,budget", [(33, 128), (40, 7), (100, 0), (161, 128), (162, 128)])
def test_budget_edges(dev, n, budget):
    """No candidates, fewer candidates than B, B = 0, and n = n_sink + w + B (+1)."""
    cfg = TINY.with_(name="edge-n%d-b%d" % (n, budget), n=n, budget=budget, n_facts=4,
                     dtype="bf16", seed=21)
    g, o = _edge_case(dev, cfg, lore_inputs(cfg))
    assert g["kept"].shape[-1] == cfg.n_keep
    assert np.array_equal(g["kept"], o["kept"])


def test_exact_ties_keep_lower_indices(dev):
    """Equal keys everywhere and one shared value vector on every candidate:
    all candidates score exactly alike, so the selection must be the B lowest
    candidate indices (n_sink = 4 keeps every chunk whole, so chunk means of
    equal scores stay exactly equal)."""
    cfg = TINY.with_(name="ties", n=300, dtype="bf16", budget=20, n_sink=4, seed=22)
    inp = lore_inputs(cfg)
    inp["K"][:] = 0.25
    v0 = inp["V"][:, :, 5:6, :].clone()
    inp["V"][:, :, : cfg.n - cfg.w, :] = v0
    g, o = _edge_case(dev, cfg, inp)
    expect = np.concatenate([np.arange(4), np.arange(4, 24), np.arange(300 - 32, 300)])
    for row in g["kept"].reshape(-1, g["kept"].shape[-1]):
        assert np.array_equal(row, expect)


@pytest.mark.parametrize("cfg", [MISTRAL_16K.with_(name="det", n=4096),
                                 QWEN_14B_BATCH.with_(name="det-g5", n=4096, batch=2)],
                         ids=["g4", "g5-two-launches"])
def test_deterministic(dev, cfg):
    """Bitwise identical results over three runs, also for a query-head group
    of 5, whose score pass runs as two launches (the second adding to S)."""
    inp = lore_inputs(cfg)
    runs = [run_gpu(cfg, inp, dev) for _ in range(3)]
    for r in runs[1:]:
        assert np.array_equal(r["S"], runs[0]["S"])
        assert np.array_equal(r["kept"], runs[0]["kept"])
        assert np.array_equal(r["O"], runs[0]["O"])
