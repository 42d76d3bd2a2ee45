"""The LORE-KV layer path captured in a HIP graph: the library enqueues only
kernel launches on the caller's stream (no memsets, allocations or
synchronisations), so one captured layer (probs, deletion, top-B, compaction)
replays to the eager result.  Each replay follows eager work of its own on
other data and a synchronisation, and each is checked bit-exactly."""

import pytest
import torch

import kv_cache_eviction_amd as kv
from kvsynth import TINY, lore_inputs, TORCH_DTYPES
from parity import lore_desc_kwargs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.load()
    return torch.device("cuda")


def test_layer_graph_replays_match_eager(dev):
    cfg = TINY.with_(name="graph-bf16", dtype="bf16", d=128, h_q=8, h_kv=2, n=3000,
                     d_model=512, budget=96, seed=71)
    desc = kv.lore_desc(dtype=TORCH_DTYPES[cfg.dtype], **lore_desc_kwargs(cfg))
    x = {k: v.to(dev).contiguous() for k, v in lore_inputs(cfg, 0, device=dev).items()}
    y = {k: v.to(dev).contiguous() for k, v in lore_inputs(cfg, 1, device=dev).items()}
    ev = kv.LoreEviction(desc, dev)
    other = kv.LoreEviction(desc, dev)
    Ko = torch.empty(cfg.batch, cfg.h_kv, desc.n_keep, cfg.d, dtype=x["K"].dtype, device=dev)
    Vo = torch.empty_like(Ko)
    Ko2, Vo2 = torch.empty_like(Ko), torch.empty_like(Vo)

    def layer():
        ev.run(x["Q"], x["K"], x["V"], x["W_O"], x["omega"], Ko, Vo)

    layer()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (ev.S, ev.kept, Ko, Vo)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work of the program's own between replays, on other buffers
        other.run(y["Q"], y["K"], y["V"], y["W_O"], y["omega"], Ko2, Vo2)
        for t in (ev.S, Ko, Vo):
            t.zero_()
        ev.kept.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((ev.S, ev.kept, Ko, Vo), ref):
            assert torch.equal(a, b), "replay %d differs from the eager run" % rep
    assert not torch.equal(other.S, ev.S)


def test_layers_on_concurrent_streams_match_sequential(dev):
    """Two layers enqueued on two streams at once, each with its own buffers
    and workspace, give bit-for-bit the results of running them one after the
    other: the library keeps no state between calls that concurrent streams
    could share (the stream argument is passed through the binding)."""
    cfg = TINY.with_(name="streams-bf16", dtype="bf16", d=128, h_q=8, h_kv=2, n=5000,
                     d_model=512, budget=120, seed=72)
    desc = kv.lore_desc(dtype=TORCH_DTYPES[cfg.dtype], **lore_desc_kwargs(cfg))
    xs = [{k: v.to(dev).contiguous() for k, v in lore_inputs(cfg, l, device=dev).items()}
          for l in range(2)]
    evs = [kv.LoreEviction(desc, dev) for _ in range(2)]
    outs = [(torch.empty(cfg.batch, cfg.h_kv, desc.n_keep, cfg.d, dtype=xs[0]["K"].dtype, device=dev),
             torch.empty(cfg.batch, cfg.h_kv, desc.n_keep, cfg.d, dtype=xs[0]["K"].dtype, device=dev))
            for _ in range(2)]

    def run(i, stream=None):
        x, (Ko, Vo) = xs[i], outs[i]
        evs[i].run(x["Q"], x["K"], x["V"], x["W_O"], x["omega"], Ko, Vo, stream=stream)

    for i in range(2):
        run(i)
    torch.cuda.synchronize()
    ref = [[t.clone() for t in (evs[i].S, evs[i].kept, *outs[i])] for i in range(2)]
    for rep in range(3):
        for i in range(2):
            for t in (evs[i].S, *outs[i]):
                t.zero_()
            evs[i].kept.fill_(-1)
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                run(i, stream=streams[i])
        torch.cuda.synchronize()
        for i in range(2):
            got = (evs[i].S, evs[i].kept, *outs[i])
            for a, b in zip(got, ref[i]):
                assert torch.equal(a, b), "rep %d: layer %d differs on concurrent streams" % (rep, i)
