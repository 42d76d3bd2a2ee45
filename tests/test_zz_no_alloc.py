"""The allocation-free top-B selection against the workspace entry point,
through the C ABI.

kvscore_topb_select_noalloc runs the kernels of kvscore_topb_select on a
scratch array the library owns on each GPU instead of a caller workspace.
Selection is index work, so the two must agree bit for bit: the same kept
sets and the same pooled scores.  Two calls run in a row, the second on a
smaller input, so the second call works over scratch the first one left
behind (the scratch is never cleared between calls).
"""

import pytest
import torch

import oracle
import kv_cache_eviction_amd as kv
from parity import check_kept

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.load()
    return torch.device("cuda:0")


def _scores(shape, seed, dev):
    """Heavy-tailed scores with a few large outliers per row."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    S = torch.rand(*shape, generator=g, device=dev) ** 4
    b, hk, n = shape
    hot = torch.randint(0, n, (b, hk, 64), generator=g, device=dev)
    S.scatter_(2, hot, 5.0 + torch.rand(b, hk, 64, generator=g, device=dev))
    return S.contiguous()


def _both(dev, S, n_sink, w, chunk, budget):
    b, hk, n = S.shape
    desc = kv.lore_desc(batch=b, n=n, h_q=hk, h_kv=hk, d=128, d_model=1, w=w, m=0, t=0,
                        n_sink=n_sink, chunk=chunk, budget=budget)
    ws = torch.empty(kv.kvs_topb_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    kept_ws = torch.empty(b, hk, desc.n_keep, dtype=torch.int32, device=dev)
    pooled_ws = torch.empty(b, hk, n, device=dev)
    kept_na = torch.full_like(kept_ws, -7)
    pooled_na = torch.full_like(pooled_ws, 3.0)
    kv.kvscore_topb_select(desc, S, kept_ws, pooled_ws, ws)
    kv.kvscore_topb_select_noalloc(desc, S, kept_na, pooled_na)
    torch.cuda.synchronize()
    assert torch.equal(kept_ws, kept_na)
    assert torch.equal(pooled_ws.view(torch.int32), pooled_na.view(torch.int32))
    return kept_na.cpu().numpy()


def test_noalloc_matches_workspace_entry_two_calls(dev):
    # first: the Llama-3.1-8B 128K layer's selection (8 KV heads, 131072
    # tokens, chunk 4: 2 MiB of scratch); second: a smaller, ragged input
    # with a larger budget over the scratch the first call left
    big = _scores((1, 8, 131072), 501, dev)
    k1 = _both(dev, big, n_sink=1, w=32, chunk=4, budget=128)
    small = _scores((2, 3, 5003), 502, dev)
    k2 = _both(dev, small, n_sink=3, w=17, chunk=4, budget=300)
    # third: rows of one segment (the H2O prompt reduction's shape), which the
    # first kernel selects in full
    tiny = _scores((3, 4, 1024), 503, dev)
    k3 = _both(dev, tiny, n_sink=0, w=205, chunk=1, budget=204)
    # and all match the oracle's selection (up to the tie band)
    for S, k, (n_sink, w, chunk, budget) in ((big, k1, (1, 32, 4, 128)), (small, k2, (3, 17, 4, 300)),
                                             (tiny, k3, (0, 205, 1, 204))):
        o, pooled = oracle.topb_select(S.double().cpu().numpy(), n_sink=n_sink, w=w, chunk=chunk,
                                       budget=budget)
        check_kept(k, o, pooled, n_sink, w, budget)


def test_noalloc_rejects_inputs_above_the_scratch(dev):
    # 64 sequences x 8 KV heads x 2^20 tokens at chunk 1 would need 4 GiB of
    # scratch: refused on the host, nothing enqueued, outputs untouched
    b, hk, n = 64, 8, 1 << 20
    desc = kv.lore_desc(batch=b, n=n, h_q=hk, h_kv=hk, d=128, d_model=1, w=32, m=0, t=0,
                        n_sink=1, chunk=1, budget=128)
    assert kv.kvs_topb_workspace_bytes(desc) > (32 << 20)
    import ctypes
    lib = kv.load()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the size check fails first
    rc = lib.kvscore_topb_select_noalloc(ctypes.byref(desc), fake, fake, None, None)
    assert rc == 2 and "maximum" in kv.last_error()
