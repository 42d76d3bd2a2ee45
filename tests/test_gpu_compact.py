"""kv_compact alone on the GPU against the oracle's gather (LORE-KV page,
Method: decoding runs on the compacted cache; H2O page, System
Implementation Details: kept rows loaded into slots), with the contract's
edges: destination rows past n_keep left untouched, pos_out -1 and score_out
0 there, and kept indices outside [0, n_src) copying nothing."""
import numpy as np
import pytest
import torch

import oracle
import kv_cache_eviction_amd as kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kv.load()
    return torch.device("cuda")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float16, 64),
                                     (torch.float32, 128), (torch.float32, 64)])
def test_gather_edges(dev, dtype, d):
    g = torch.Generator().manual_seed(d + (2 if dtype == torch.float32 else 1))
    b, h, n_src, n_keep, cap = 2, 3, 777, 90, 130
    K = torch.randn(b, h, n_src, d, generator=g).to(dtype)
    V = torch.randn(b, h, n_src, d, generator=g).to(dtype)
    score = torch.rand(b, h, n_src, generator=g)
    kept = torch.stack([torch.stack([torch.randperm(n_src, generator=g)[:n_keep].sort().values
                                     for _ in range(h)]) for _ in range(b)]).to(torch.int32)
    # a few indices outside [0, n_src): nothing is copied for them
    bad = {(0, 0, 5): -1, (1, 2, 0): n_src, (1, 1, n_keep - 1): n_src + 100}
    for (bb, hh, r), val in bad.items():
        kept[bb, hh, r] = val
    Kd, Vd, kd, sd = K.to(dev), V.to(dev), kept.to(dev), score.to(dev)
    Ko = torch.full((b, h, cap, d), 3.0, dtype=dtype, device=dev)  # a sentinel value
    Vo = torch.full_like(Ko, 3.0)
    pos = torch.full((b, h, cap), 7, dtype=torch.int32, device=dev)
    so = torch.full((b, h, cap), 9.0, device=dev)
    kv.kv_compact(Kd, Vd, kd, Ko, Vo, pos, sd, so)
    torch.cuda.synchronize()
    Ko, Vo, pos, so = Ko.cpu(), Vo.cpu(), pos.cpu(), so.cpu()
    ok = (kept >= 0) & (kept < n_src)
    safe = torch.where(ok, kept, torch.zeros_like(kept))
    Kr, Vr = oracle.compact(K.view(torch.int16 if dtype != torch.float32 else torch.int32).numpy(),
                            V.view(torch.int16 if dtype != torch.float32 else torch.int32).numpy(),
                            safe.numpy())
    iv = torch.int16 if dtype != torch.float32 else torch.int32
    Kg = Ko.view(iv).numpy()
    Vg = Vo.view(iv).numpy()
    okn = ok.numpy()
    # copied rows: bit-exact
    assert np.array_equal(Kg[:, :, :n_keep][okn], Kr[okn])
    assert np.array_equal(Vg[:, :, :n_keep][okn], Vr[okn])
    # rows of out-of-range indices and rows past n_keep: untouched
    sentinel = torch.full((d,), 3.0, dtype=dtype).view(iv).numpy()
    for arr in (Kg, Vg):
        assert (arr[:, :, :n_keep][~okn] == sentinel).all()
        assert (arr[:, :, n_keep:] == sentinel).all()
    # positions and carried scores
    exp_pos = torch.where(ok, kept, torch.full_like(kept, -1))
    assert torch.equal(pos[:, :, :n_keep], exp_pos)
    assert (pos[:, :, n_keep:] == -1).all()
    exp_s = torch.where(ok, torch.gather(score, 2, safe.long()), torch.zeros(()))
    assert torch.equal(so[:, :, :n_keep], exp_s)
    assert (so[:, :, n_keep:] == 0).all()


def test_nothing_kept_touches_only_the_maps(dev):
    """n_keep = 0: no row is copied; pos_out and score_out read -1 and 0."""
    b, h, n_src, cap, d = 1, 2, 100, 16, 128
    K = torch.randn(b, h, n_src, d, device=dev).to(torch.bfloat16)
    V = torch.randn_like(K)
    kept = torch.empty(b, h, 0, dtype=torch.int32, device=dev)
    Ko = torch.full((b, h, cap, d), 5.0, dtype=torch.bfloat16, device=dev)
    Vo = torch.full_like(Ko, 5.0)
    pos = torch.full((b, h, cap), 7, dtype=torch.int32, device=dev)
    so = torch.full((b, h, cap), 9.0, device=dev)
    kv.kv_compact(K, V, kept, Ko, Vo, pos, torch.rand(b, h, n_src, device=dev), so)
    torch.cuda.synchronize()
    assert (Ko == 5.0).all() and (Vo == 5.0).all()
    assert (pos == -1).all() and (so == 0).all()
