"""GPU parity of the prompt-side baseline scores (window attention score,
TOVA's last-query score) and of their top-B selection, against the oracle,
through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_eviction_amd as kv
from kvsynth import TINY, MISTRAL_16K, LLAMA_128K, lore_inputs, TORCH_DTYPES
from parity import lore_desc_kwargs, check_scores, check_kept

pytestmark = pytest.mark.gpu

KINDS = {"window": kv.KVS_BASELINE_WINDOW, "tova": kv.KVS_BASELINE_TOVA}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.load()
    return torch.device("cuda")


def run_gpu(cfg, inp, dev, kind):
    desc = kv.lore_desc(dtype=TORCH_DTYPES[cfg.dtype], **lore_desc_kwargs(cfg))
    ev = kv.LoreEviction(desc, dev)
    Q, K, V = (inp[k].to(dev).contiguous() for k in ("Q", "K", "V"))
    ev.baseline(KINDS[kind], Q, K, V)
    ev.select()
    torch.cuda.synchronize()
    return ev.S.cpu().numpy(), ev.kept.cpu().numpy()


def compare(cfg, S, kept, So, name, kind):
    worst = check_scores(S, So, cfg.n_sink, cfg.w)
    kept_o, pooled_o = oracle.topb_select(So, n_sink=cfg.n_sink, w=cfg.w, chunk=cfg.chunk,
                                          budget=cfg.budget)
    nd = check_kept(kept, kept_o, pooled_o, cfg.n_sink, cfg.w, cfg.budget)
    print("%s %s: worst score rel err %.3g, kept diffs at ties %d" % (name, kind, worst, nd))


SMALL = [
    TINY,
    TINY.with_(name="bf16-d128-g4-n1000", dtype="bf16", d=128, h_q=8, h_kv=2, n=1000,
               d_model=512, budget=64, seed=11),
    TINY.with_(name="f16-d64-mha-n777-nq11", dtype="f16", d=64, h_q=3, h_kv=3, n=777,
               d_model=192, w=5, m=2, t=3, chunk=1, budget=50, n_sink=2, seed=12),
    TINY.with_(name="bf16-d128-g5-b2-n2085", dtype="bf16", d=128, h_q=10, h_kv=2, n=2085,
               d_model=1280, budget=100, batch=2, seed_per_seq=True, omega_per_seq=True, seed=13),
    TINY.with_(name="bf16-d64-g16-n600-w1", dtype="bf16", d=64, h_q=16, h_kv=1, n=600,
               d_model=1024, w=1, budget=30, seed=16, window_from_facts=False),
]


@pytest.mark.parametrize("kind", ["window", "tova"])
@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small_shapes(dev, cfg, kind):
    inp = lore_inputs(cfg)
    S, kept = run_gpu(cfg, inp, dev, kind)
    So = oracle.baseline_scores(inp["Q"], inp["K"], w=cfg.w, kind=kind)
    compare(cfg, S, kept, So, cfg.name, kind)
    # each softmax row sums to one: w per KV head (window), 1 (TOVA)
    assert np.allclose(S.sum(axis=-1), cfg.w if kind == "window" else 1.0, rtol=1e-4)


def test_mistral_16k_window(dev):
    inp = lore_inputs(MISTRAL_16K)
    S, kept = run_gpu(MISTRAL_16K, inp, dev, "window")
    So = oracle.baseline_scores(inp["Q"], inp["K"], w=MISTRAL_16K.w, kind="window")
    compare(MISTRAL_16K, S, kept, So, MISTRAL_16K.name, "window")


@pytest.mark.parametrize("kind", ["window", "tova"])
def test_llama_128k_every_head(dev, kind):
    """The full-size launch; the oracle checks every KV head of layer 0
    completely (scores of every candidate and every kept set)."""
    cfg = LLAMA_128K
    inp = lore_inputs(cfg, layer=0, device=dev)
    S, kept = run_gpu(cfg, inp, dev, kind)
    So = oracle.baseline_scores(inp["Q"].cpu(), inp["K"].cpu(), w=cfg.w, kind=kind)
    compare(cfg, S, kept, So, cfg.name, kind)
