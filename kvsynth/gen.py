"""Seeded synthetic inputs for the scoring and eviction workloads.

This module only draws inputs.  It holds none of the scoring, selection or
eviction arithmetic: the oracle and the HIP path both take what it returns.

Every value is drawn in fp32 from a ``torch.Generator`` seeded per layer (and
per sequence where the workload says so), then rounded once (round to nearest
even) to the workload's dtype.  A CPU generator and a GPU generator give
different streams for the same seed; each caller passes the device it wants
and the data it gets is a deterministic function of (workload, layer, device).

Recipes (sizes from ``kvsynth.configs``):

``facts``  K, V ~ N(0, 1).  Token 0 is an attention sink: its key is scaled by
           8.  ``n_facts`` fact positions are drawn without replacement from
           the candidate range [1, n - w).  A scoring query is
           0.6 * k_target + 0.4 * z, z ~ N(0, I), with the target a fact drawn
           uniformly (lookahead rows always; window rows too unless
           ``window_from_facts`` is False, in which case window rows target a
           uniformly drawn non-fact candidate).
``heavy``  K, V ~ N(0, 1).  Each KV head g has a mean query mu_g ~ N(0, I);
           each query is mu_g + N(0, I).  1% of the candidates (shared by the
           heads) are heavy hitters: their key gains rho * mu_g / |mu_g| with
           rho = min(8, u^(-1/1.5)), u ~ U(0, 1], which adds about rho to the
           scaled logit and gives accumulated attention a power-law tail.

W_O ~ N(0, 1/d) of shape [d_model][h_q * d] (the linear-layer layout: head h
owns columns h*d .. h*d+d-1).  omega = softmax of M standard normals.

The H2O recipe draws prompt Q, K, V ~ N(0, 1) of shape [b][H][P][d], scales the
key of 5% of prompt positions (shared by the heads of a sequence) by 3, then
draws the per-step q, k, v ~ N(0, 1) of shape [steps][b][H][d].
"""

import torch

from .configs import LoreConfig, H2OConfig, RefreshConfig

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(gen, *shape, device):
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def _facts_sequence(cfg: LoreConfig, gen, device):
    """K, V, Q and fact positions for one sequence, 'facts' recipe."""
    h_kv, h_q, n, d, nq, w = cfg.h_kv, cfg.h_q, cfg.n, cfg.d, cfg.n_q, cfg.w
    K = _randn(gen, h_kv, n, d, device=device)
    V = _randn(gen, h_kv, n, d, device=device)
    K[:, 0, :] *= 8.0
    n_cand = n - w - 1  # candidates [1, n - w)
    # tiny caches with fewer candidates than facts draw from every non-sink token
    pool = n_cand if n_cand >= cfg.n_facts else max(n - 1, 1)
    k_facts = min(cfg.n_facts, pool)
    facts = torch.randperm(pool, generator=gen, device=device)[:k_facts] + (1 if n > 1 else 0)
    z = _randn(gen, h_q, nq, d, device=device)
    pick = torch.randint(0, k_facts, (h_q, nq), generator=gen, device=device)
    target = facts[pick]  # [h_q][nq]
    if not cfg.window_from_facts:
        is_fact = torch.zeros(n, dtype=torch.bool, device=device)
        is_fact[facts] = True
        non_fact = torch.arange(1, n - w, device=device)
        non_fact = non_fact[~is_fact[1: n - w]]
        pick_w = torch.randint(0, non_fact.numel(), (h_q, w), generator=gen, device=device)
        target[:, :w] = non_fact[pick_w]
    g_of_h = torch.arange(h_q, device=device) // cfg.group
    k_target = K[g_of_h[:, None], target]  # [h_q][nq][d]
    Q = 0.6 * k_target + 0.4 * z
    return K, V, Q, facts


def _heavy_sequence(cfg: LoreConfig, gen, device):
    """K, V, Q and heavy-hitter positions for one sequence, 'heavy' recipe."""
    h_kv, h_q, n, d, nq = cfg.h_kv, cfg.h_q, cfg.n, cfg.d, cfg.n_q
    mu = _randn(gen, h_kv, d, device=device)
    K = _randn(gen, h_kv, n, d, device=device)
    V = _randn(gen, h_kv, n, d, device=device)
    n_cand = n - cfg.n_sink - cfg.w
    n_hh = max(1, int(round(0.01 * n_cand)))
    hh = torch.randperm(n_cand, generator=gen, device=device)[:n_hh] + cfg.n_sink
    u = 1.0 - torch.rand(n_hh, generator=gen, device=device)  # (0, 1]
    rho = torch.clamp(u.pow(-1.0 / 1.5), max=8.0)
    mu_hat = mu / mu.norm(dim=1, keepdim=True)
    K[:, hh, :] += rho[None, :, None] * mu_hat[:, None, :]
    g_of_h = torch.arange(h_q, device=device) // cfg.group
    Q = mu[g_of_h][:, None, :] + _randn(gen, h_q, nq, d, device=device)
    return K, V, Q, hh


def lore_inputs(cfg: LoreConfig, layer: int = 0, device="cpu"):
    """Inputs for one layer of a LORE-KV workload.

    Returns a dict with Q [b][h_q][n_q][d], K and V [b][h_kv][n][d], W_O
    [d_model][h_q*d] (all in the workload dtype), omega [b][m] fp32 and the
    planted positions ``marks`` [b][*] int64 (facts or heavy hitters).
    """
    dt = TORCH_DTYPES[cfg.dtype]
    shared = _generator(cfg.seed + layer if not cfg.seed_per_seq else 10_000 + cfg.seed + layer,
                        device)
    W_O = _randn(shared, cfg.d_model, cfg.h_q * cfg.d, device=device) / (cfg.d ** 0.5)
    n_omega = cfg.batch if cfg.omega_per_seq else 1
    omega = torch.softmax(_randn(shared, n_omega, cfg.m, device=device), dim=1)
    omega = omega.expand(cfg.batch, cfg.m).contiguous()
    seq = _heavy_sequence if cfg.recipe == "heavy" else _facts_sequence
    Ks, Vs, Qs, marks = [], [], [], []
    for b in range(cfg.batch):
        gen = _generator(cfg.seed + layer + b, device) if cfg.seed_per_seq else shared
        K, V, Q, mk = seq(cfg, gen, device)
        Ks.append(K); Vs.append(V); Qs.append(Q); marks.append(mk)
    return {
        "Q": torch.stack(Qs).to(dt),
        "K": torch.stack(Ks).to(dt),
        "V": torch.stack(Vs).to(dt),
        "W_O": W_O.to(dt),
        "omega": omega,
        "marks": torch.stack(marks),
    }


def future_queries(cfg: LoreConfig, inputs, n_f: int, layer: int = 0, device="cpu"):
    """Held-out "future" queries [b][h_q][n_f][d] (workload dtype) for one
    layer's inputs: each is 0.6 * k_target + 0.4 * z, z ~ N(0, I), with the
    target drawn uniformly from the sequence's planted positions (facts or
    heavy hitters) and k_target its key at the query head's KV head; a stream
    of its own, separate from the scoring queries'."""
    gen = _generator(30_000 + cfg.seed + layer, device)
    K = inputs["K"].to(device=device, dtype=torch.float32)
    marks = inputs["marks"].to(device)
    g_of_h = torch.arange(cfg.h_q, device=device) // cfg.group
    out = []
    for b in range(cfg.batch):
        pick = torch.randint(0, marks.shape[1], (cfg.h_q, n_f), generator=gen, device=device)
        target = marks[b][pick]
        z = _randn(gen, cfg.h_q, n_f, cfg.d, device=device)
        out.append(0.6 * K[b][g_of_h[:, None], target] + 0.4 * z)
    return torch.stack(out).to(TORCH_DTYPES[cfg.dtype])


def refresh_inputs(cfg: RefreshConfig, device="cpu"):
    """Inputs of one counter-causal refresh: fresh queries Q [b][h_q][n][d] and
    the cache K, V [b][h_kv][n][d] ~ N(0, 1) in the workload dtype; the
    surprise [b][n] ~ N(0, 1) fp32 (what the LM head's logits would give) and
    token ids [b][n] ~ U[0, 151936) int32 (Qwen2.5's vocabulary size)."""
    gen = _generator(cfg.seed, device)
    dt = TORCH_DTYPES[cfg.dtype]
    n = cfg.n
    return {
        "Q": _randn(gen, cfg.batch, cfg.h_q, n, cfg.d, device=device).to(dt),
        "K": _randn(gen, cfg.batch, cfg.h_kv, n, cfg.d, device=device).to(dt),
        "V": _randn(gen, cfg.batch, cfg.h_kv, n, cfg.d, device=device).to(dt),
        "surprise": _randn(gen, cfg.batch, n, device=device),
        "ids": torch.randint(0, 151936, (cfg.batch, n), generator=gen, device=device,
                             dtype=torch.int32),
    }


def trajectory_token_stats(cfg: LoreConfig, layer: int = 0, device="cpu"):
    """Per-token statistics of the M sampled continuations, which a model's
    next-token distributions would give: entropy [b][m][t] ~ U(0.5, 4) nats
    and log-probability [b][m][t] = min(0, -entropy + 0.8 z), z ~ N(0, 1)
    (tokens about as likely as the distribution they came from, with noise).
    Returns (logp, entropy), fp32."""
    gen = _generator(20_000 + cfg.seed + layer, device)
    shape = (cfg.batch, cfg.m, cfg.t)
    ent = 0.5 + 3.5 * torch.rand(*shape, generator=gen, device=device, dtype=torch.float32)
    logp = torch.clamp(-ent + 0.8 * _randn(gen, *shape, device=device), max=0.0)
    return logp, ent


def h2o_inputs(cfg: H2OConfig, device="cpu"):
    """Inputs for an H2O prompt + decode run.

    Returns Qp, Kp, Vp [b][H][P][d]; q, k, v [steps][b][H][d] in the workload
    dtype, and ``boosted`` [b][n_boost] prompt positions whose key was scaled.
    """
    dt = TORCH_DTYPES[cfg.dtype]
    gen = _generator(cfg.seed, device)
    b, H, P, d = cfg.batch, cfg.heads, cfg.prompt, cfg.d
    Qp = _randn(gen, b, H, P, d, device=device)
    Kp = _randn(gen, b, H, P, d, device=device)
    Vp = _randn(gen, b, H, P, d, device=device)
    n_boost = int(cfg.boost_frac * P)
    boosted = torch.stack([torch.randperm(P, generator=gen, device=device)[:n_boost]
                           for _ in range(b)]) if n_boost > 0 else \
        torch.zeros(b, 0, dtype=torch.int64, device=device)
    for bi in range(b):
        Kp[bi][:, boosted[bi], :] *= cfg.boost
    q = _randn(gen, cfg.steps, b, H, d, device=device)
    k = _randn(gen, cfg.steps, b, H, d, device=device)
    v = _randn(gen, cfg.steps, b, H, d, device=device)
    return {"Qp": Qp.to(dt), "Kp": Kp.to(dt), "Vp": Vp.to(dt),
            "q": q.to(dt), "k": k.to(dt), "v": v.to(dt), "boosted": boosted}
