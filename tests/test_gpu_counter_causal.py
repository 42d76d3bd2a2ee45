"""GPU parity of the counter-causal refresh (counter-causal review "Back from
the Future": 3.2 reversed-mask attention over the cache, Alg. 3 memory
refresh) against the oracle, through the C ABI.

Attention: row statistics and outputs to the bar of the LORE-KV attention pass
(m within 1e-5, l within 1e-5 relative, O within 1e-3 of the row's largest
component); the last position, which sees no key, exactly (m = -inf, l = 0,
O = 0).  Refresh: kept positions, gathered rows and token ids bit-exact."""

import numpy as np
import pytest
import torch

import oracle
import kv_cache_eviction_amd as kv
from kvsynth import QWEN7B_REFRESH, refresh_inputs, TORCH_DTYPES
from parity import check_stats

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.load()
    return torch.device("cuda")


def run_attention(cfg, inp, dev, n=None):
    n = cfg.n if n is None else n
    desc = kv.lore_desc(batch=cfg.batch, n=n, h_q=cfg.h_q, h_kv=cfg.h_kv, d=cfg.d,
                        d_model=cfg.h_q * cfg.d, w=0, m=1, t=1, n_sink=0,
                        dtype=TORCH_DTYPES[cfg.dtype])
    b, hq, d = cfg.batch, cfg.h_q, cfg.d
    m = torch.empty(b, hq, n, device=dev)
    l = torch.empty(b, hq, n, device=dev)
    O = torch.full((b, hq, n, d), float("nan"), device=dev)
    Q, K, V = (inp[k].to(dev).contiguous() for k in ("Q", "K", "V"))
    kv.kvscore_counter_causal(desc, Q, K, V, m, l, O)
    torch.cuda.synchronize()
    return m.cpu().numpy(), l.cpu().numpy(), O.cpu().numpy()


def compare_attention(cfg, inp, got, heads, name, n=None):
    m, l, O = got
    G = cfg.h_q // cfg.h_kv
    g = heads[0] // G
    mo, lo, Oo = oracle.counter_causal_attention(inp["Q"][:, heads].cpu(), inp["K"][:, g:g + 1].cpu(),
                                                 inp["V"][:, g:g + 1].cpu())
    m, l, O = m[:, heads], l[:, heads], O[:, heads]
    n = cfg.n if n is None else n
    # every position but the last sees at least one key
    if n > 1:
        check_stats(m[:, :, :n - 1], l[:, :, :n - 1], O[:, :, :n - 1], mo[:, :, :n - 1],
                    lo[:, :, :n - 1], Oo[:, :, :n - 1])
    assert np.all(m[:, :, n - 1] == -np.inf) and np.all(l[:, :, n - 1] == 0)
    assert np.all(O[:, :, n - 1] == 0)
    print("%s heads %s: counter-causal attention within the bar" % (name, heads))


SMALL = [
    QWEN7B_REFRESH.with_(name="f32-d64-g2-n100", h_q=4, h_kv=2, d=64, J=80, n_sys=4, dtype="f32",
                         seed=61),
    QWEN7B_REFRESH.with_(name="bf16-d128-g7-n640", J=512, n_sys=16, seed=62),
    QWEN7B_REFRESH.with_(name="f16-d64-mha-b2-n777", batch=2, h_q=3, h_kv=3, d=64, J=622,
                         n_sys=8, dtype="f16", seed=63),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_attention_small(dev, cfg):
    inp = refresh_inputs(cfg, device="cpu")
    got = run_attention(cfg, inp, dev)
    G = cfg.h_q // cfg.h_kv
    for g in range(cfg.h_kv):
        compare_attention(cfg, inp, got, list(range(g * G, (g + 1) * G)), cfg.name)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 129])
def test_attention_tiny_and_block_edges(dev, n):
    # one token (sees nothing), two, and caches ending just before, at and
    # just after a 64-position block boundary
    cfg = QWEN7B_REFRESH.with_(name="edge", h_q=6, h_kv=2, d=64, J=256, n_sys=0, dtype="f32",
                               seed=66)
    x = refresh_inputs(cfg, device="cpu")  # 320 positions, cut to the first n
    inp = {k: x[k][:, :, :n].contiguous() for k in ("Q", "K", "V")}
    got = run_attention(cfg, inp, dev, n=n)
    for g in range(cfg.h_kv):
        compare_attention(cfg, inp, got, [3 * g, 3 * g + 1, 3 * g + 2], "n=%d" % n, n=n)


@pytest.mark.parametrize("n,J,n_sys", [(1, 1, 0), (1, 5, 3), (2, 1, 0), (65, 40, 8)])
def test_refresh_tiny(dev, n, J, n_sys):
    cfg = QWEN7B_REFRESH.with_(batch=2, h_kv=2, d=64, dtype="f16", seed=67)
    x = refresh_inputs(cfg.with_(J=256), device="cpu")
    inp = {"K": x["K"][:, :, :n].contiguous(), "V": x["V"][:, :, :n].contiguous(),
           "surprise": x["surprise"][:, :n].contiguous(), "ids": x["ids"][:, :n].contiguous()}
    check_refresh(inp, run_refresh(inp, 2, J, n_sys, dev), J, n_sys)


def test_attention_full_size_every_head(dev):
    """The full-size launch (n = 5120 cached tokens, 28 query heads over 4 KV
    heads); the oracle checks every query head of every KV head."""
    cfg = QWEN7B_REFRESH
    inp = refresh_inputs(cfg, device=dev)
    got = run_attention(cfg, inp, dev)
    G = cfg.h_q // cfg.h_kv
    host = {k: v.cpu() for k, v in inp.items()}
    for g in range(cfg.h_kv):
        compare_attention(cfg, host, got, list(range(g * G, (g + 1) * G)), cfg.name)


def run_refresh(inp, heads_K, J, n_sys, dev, with_ids=True):
    K, V = inp["K"].to(dev).contiguous(), inp["V"].to(dev).contiguous()
    S = inp["surprise"].to(dev).contiguous()
    ids = inp["ids"].to(dev).contiguous() if with_ids else None
    b, h, n, d = K.shape
    keep = min(J, n)
    kept = torch.full((b, keep), -7, dtype=torch.int32, device=dev)
    Ko = torch.empty(b, h, keep, d, dtype=K.dtype, device=dev)
    Vo = torch.empty_like(Ko)
    ido = torch.empty(b, keep, dtype=torch.int32, device=dev) if with_ids else None
    ws = torch.empty(kv.kvs_refresh_workspace_bytes(b, n), dtype=torch.uint8, device=dev)
    kv.kvscore_refresh(S, K, V, kept, Ko, Vo, n_sys=n_sys, J=J, ids=ids, ids_out=ido, ws=ws)
    torch.cuda.synchronize()
    return kept.cpu(), Ko.cpu(), Vo.cpu(), None if ido is None else ido.cpu()


def check_refresh(inp, got, J, n_sys):
    kept, Ko, Vo, ido = got
    ko = oracle.refresh_select(inp["surprise"].cpu(), n_sys=n_sys, J=J)
    assert np.array_equal(kept.numpy(), ko)
    # fp32 widening is exact for every dtype, so equal values mean equal rows
    K_, V_, X_ = oracle.refresh_gather(inp["K"].cpu().float(), inp["V"].cpu().float(),
                                       inp["ids"].cpu(), ko)
    assert np.array_equal(Ko.float().numpy(), K_) and np.array_equal(Vo.float().numpy(), V_)
    if ido is not None:
        assert np.array_equal(ido.numpy(), X_)


@pytest.mark.parametrize("J,n_sys", [(512, 16), (17, 16), (640, 16), (2000, 0), (1, 0)],
                         ids=["J512", "only-protected", "keep-all", "no-sys-J>=n", "J1"])
def test_refresh_edges(dev, J, n_sys):
    cfg = QWEN7B_REFRESH.with_(batch=3, J=512, n_sys=16, seed=64)  # n = 640
    inp = refresh_inputs(cfg, device="cpu")
    # quantised surprise: many exact ties, broken toward the lower position
    inp["surprise"] = torch.round(inp["surprise"] * 4) / 4
    check_refresh(inp, run_refresh(inp, cfg.h_kv, J, n_sys, dev), J, n_sys)


def test_refresh_without_ids_and_at_full_size(dev):
    cfg = QWEN7B_REFRESH
    inp = refresh_inputs(cfg, device="cpu")
    check_refresh(inp, run_refresh(inp, cfg.h_kv, cfg.J, cfg.n_sys, dev), cfg.J, cfg.n_sys)
    kept, Ko, Vo, ido = run_refresh(inp, cfg.h_kv, cfg.J, cfg.n_sys, dev, with_ids=False)
    assert ido is None and kept.shape == (1, cfg.J)


@pytest.mark.parametrize("J", [0, 96])
def test_refresh_cycle_on_device(dev, J):
    # the inference/refresh cycle with the memory on the device: buffer h = 32
    # new tokens per chunk; each refresh keeps J (J = 0: the chunked sliding
    # window, nothing survives).  The kept token ids match an oracle replay.
    h, heads, d, n_sys = 32, 2, 64, 8 if J else 0
    rng = np.random.default_rng(65)
    mem_ids = np.arange(n_sys, dtype=np.int32)[None]
    Km = torch.randn(1, heads, n_sys, d, dtype=torch.float16)
    Vm = torch.randn(1, heads, n_sys, d, dtype=torch.float16)
    ref_mem = list(range(n_sys))
    pos = n_sys
    for _ in range(8):
        new_ids = np.arange(pos, pos + h, dtype=np.int32)[None]
        pos += h
        Kc = torch.cat([Km, torch.randn(1, heads, h, d, dtype=torch.float16)], dim=2)
        Vc = torch.cat([Vm, torch.randn(1, heads, h, d, dtype=torch.float16)], dim=2)
        ids = np.concatenate([mem_ids, new_ids], axis=1)
        s = torch.as_tensor(rng.standard_normal((1, ids.shape[1])), dtype=torch.float32)
        inp = {"K": Kc, "V": Vc, "surprise": s, "ids": torch.as_tensor(ids)}
        got = run_refresh(inp, heads, J, n_sys, dev)
        if J == 0:  # nothing survives the refresh
            assert all(t.numel() == 0 for t in got)
            mem_ids = np.zeros((1, 0), dtype=np.int32)
            Km, Vm = Kc[:, :, :0], Vc[:, :, :0]
            ref_mem = []
            continue
        check_refresh(inp, got, J, n_sys)
        kept, Km, Vm, ido = got
        mem_ids = ido.numpy()
        cache = ref_mem + list(range(pos - h, pos))
        ref_mem = [cache[k] for k in oracle.refresh_select(s, n_sys=n_sys, J=J)[0]]
        assert mem_ids[0].tolist() == ref_mem
        assert ref_mem[:n_sys] == list(range(n_sys)) and ref_mem[-1] == pos - 1
    assert len(ref_mem) == (0 if J == 0 else min(J, n_sys + 8 * h))
