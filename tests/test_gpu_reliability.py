"""GPU parity of the trajectory reliability weights (LORE-KV Method,
"Reliability weights", Eqs. 2-4 and 10) against the oracle, through the C ABI.

The device computes cosines, norms and every sum in fp64 from queries that
are exact in fp32, so D and Dhat agree with the fp64 oracle to rounding; the
outputs are fp32, so the bar is the fp32 rounding of each value: Dhat within
2e-6 absolute (|Dhat| <= sqrt(m - 1)), omega within 1e-6 relative."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_eviction_amd as kv
from kvsynth import (TINY, MISTRAL_16K, LLAMA_128K, QWEN_14B_BATCH, lore_inputs,
                     trajectory_token_stats, TORCH_DTYPES)
from parity import lore_desc_kwargs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.load()
    return torch.device("cuda")


def run_and_compare(desc, Q, logp, ent, coef, dev, name):
    b, m = desc.batch, desc.m
    Qd = Q.to(dev).contiguous()
    omega = torch.full((b, m), float("nan"), device=dev)
    dhat = torch.full((b, m), float("nan"), device=dev)
    ws = torch.empty(kv.kvs_lore_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    kv.kvscore_reliability_weights(desc, Qd, logp.to(dev), ent.to(dev), omega, coef, dhat=dhat,
                                   ws=ws)
    torch.cuda.synchronize()
    ref = oracle.reliability_weights(Q, logp, ent, w=desc.w, m=m, t=desc.t, beta=coef[0],
                                     gamma=coef[1], lambda_d=coef[2])
    om, dh = omega.cpu().double().numpy(), dhat.cpu().double().numpy()
    err_d = np.abs(dh - ref["dhat"]).max()
    err_w = (np.abs(om - ref["omega"]) / ref["omega"]).max()
    print("%s: max |dDhat| %.3g, max rel domega %.3g, omega %s" % (name, err_d, err_w,
                                                                   np.round(om[0], 4)))
    assert err_d <= 2e-6, name
    assert err_w <= 1e-6, name
    assert np.allclose(om.sum(axis=1), 1.0, atol=1e-6)
    # the product path without the optional output gives the same weights
    omega2 = torch.empty_like(omega)
    kv.kvscore_reliability_weights(desc, Qd, logp.to(dev), ent.to(dev), omega2, coef, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(omega, omega2)
    return ref


WORKLOADS = [
    TINY,
    TINY.with_(name="bf16-d128-b2-n1000", dtype="bf16", d=128, h_q=8, h_kv=2, n=1000,
               d_model=512, batch=2, seed_per_seq=True, omega_per_seq=True, seed=21),
    MISTRAL_16K,
    LLAMA_128K,
    QWEN_14B_BATCH,
]


@pytest.mark.parametrize("preset", ["D", "E"])
@pytest.mark.parametrize("cfg", WORKLOADS, ids=[c.name for c in WORKLOADS])
def test_workload_shapes(dev, cfg, preset):
    coef = kv.RELIABILITY_D if preset == "D" else kv.RELIABILITY_E
    desc = kv.lore_desc(dtype=TORCH_DTYPES[cfg.dtype], **lore_desc_kwargs(cfg))
    Q = lore_inputs(cfg, 0, device=dev)["Q"].cpu()
    logp, ent = trajectory_token_stats(cfg, 0)
    ref = run_and_compare(desc, Q, logp, ent, coef, dev, "%s/%s" % (cfg.name, preset))
    if preset == "D":
        assert np.abs(ref["dhat"]).max() > 0.1  # the disagreement term is exercised


def _random_q(seed, b, h_q, nq, d, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(b, h_q, nq, d, generator=g).to(dtype)


def _stats(seed, b, m, t):
    g = torch.Generator().manual_seed(seed)
    ent = 0.5 + 3.5 * torch.rand(b, m, t, generator=g)
    return torch.clamp(-ent + 0.8 * torch.randn(b, m, t, generator=g), max=0.0), ent


@pytest.mark.parametrize("shape", [
    dict(w=32, m=1, t=8, dtype=torch.bfloat16),    # one trajectory: omega = 1
    dict(w=32, m=2, t=16, dtype=torch.bfloat16),   # two: Dhat = 0 by symmetry
    dict(w=0, m=60, t=1, dtype=torch.float32),     # many single-query trajectories
    dict(w=3, m=5, t=7, dtype=torch.float16),      # odd sizes, ragged pair counts per wave
], ids=["m1", "m2", "m60-t1-w0", "f16-m5-t7"])
def test_edges(dev, shape):
    b, h_q, d = 3, 6, 64 if shape["dtype"] == torch.float16 else 128
    w, m, t = shape["w"], shape["m"], shape["t"]
    desc = kv.lore_desc(batch=b, n=4096, h_q=h_q, h_kv=2, d=d, d_model=h_q * d, w=w, m=m, t=t,
                        dtype=shape["dtype"])
    Q = _random_q(7 + m, b, h_q, w + m * t, d, shape["dtype"])
    logp, ent = _stats(8 + m, b, m, t)
    ref = run_and_compare(desc, Q, logp, ent, kv.RELIABILITY_D, dev, "edge m=%d t=%d" % (m, t))
    if m <= 2:
        assert np.all(ref["dhat"] == 0.0)
