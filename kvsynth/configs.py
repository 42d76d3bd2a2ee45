"""The synthetic workloads, by shape.

Shapes and hyperparameters follow the LORE-KV project page ("Monte Carlo
Estimation for KV-Cache Eviction", Method and Hyperparameters table: w=32,
M=4, T=8, lambda_L=1, eps=1e-6, chunk=4) and the H2O summary page ("H2O:
Heavy-Hitter Oracle", 3.2 and the Evaluation Methodology budget rule).  The
model shapes (heads, head dim, d_model) are those of the public model cards
the pages evaluate on; nothing here reads a dataset or weights.
"""

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class LoreConfig:
    """One LORE-KV scoring workload: one eviction over one layer's cache.

    ``recipe`` selects the input generator in ``kvsynth.gen``:
      * ``"facts"``  - K,V ~ N(0,1), token 0 a sink with key norm x8, 16
                       planted fact tokens that the scoring queries look at;
      * ``"heavy"``  - K,V ~ N(0,1), 1% of candidates are heavy hitters whose
                       keys lean toward the head's mean query.
    ``window_from_facts`` False means the window queries target non-fact
    tokens, so the facts are reached only by lookahead queries.
    """

    name: str
    batch: int
    n: int
    h_q: int
    h_kv: int
    d: int
    d_model: int
    dtype: str  # "f32" | "bf16"
    seed: int
    recipe: str = "facts"
    w: int = 32
    m: int = 4
    t: int = 8
    n_sink: int = 1
    chunk: int = 4
    budget: int = 128
    eps: float = 1e-6
    lambda_l: float = 1.0
    layers: int = 1
    n_facts: int = 16
    window_from_facts: bool = True
    seed_per_seq: bool = False  # each sequence b gets seed + b
    omega_per_seq: bool = False

    @property
    def n_q(self) -> int:
        return self.w + self.m * self.t

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    @property
    def n_keep(self) -> int:
        return min(self.n, self.n_sink + self.budget + self.w)

    def with_(self, **kw) -> "LoreConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class H2OConfig:
    """H2O decode-time eviction: accumulated-attention heavy hitters plus a
    recent window, budget a fraction of the current length."""

    name: str
    batch: int
    heads: int
    d: int
    prompt: int
    steps: int
    dtype: str  # "f16" | "f32"
    seed: int
    heavy_frac: float = 0.10
    recent_frac: float = 0.10
    boost_frac: float = 0.05  # fraction of prompt positions whose key is scaled
    boost: float = 3.0

    def k_heavy(self, cur_len: int) -> int:
        return int(self.heavy_frac * cur_len)

    def k_recent(self, cur_len: int) -> int:
        return int(self.recent_frac * cur_len)

    @property
    def cap(self) -> int:
        """Slots needed: the largest budget plus the token being appended."""
        last = self.prompt + self.steps
        return self.k_heavy(last) + self.k_recent(last) + 2

    def with_(self, **kw) -> "H2OConfig":
        return replace(self, **kw)


# Tiny deletion-score layer, fp32: the oracle finishes it in well under a second.
TINY = LoreConfig(name="tiny-fp32-n512", batch=1, n=512, h_q=4, h_kv=2, d=64,
                  d_model=256, dtype="f32", seed=101, recipe="facts")

# Mistral-7B-shaped layer at 16K context (RULER-16K length on the LORE-KV page).
MISTRAL_16K = LoreConfig(name="mistral7b-layer-n16384", batch=1, n=16384, h_q=32,
                         h_kv=8, d=128, d_model=4096, dtype="bf16", seed=202,
                         recipe="heavy")

# Llama-3.1-8B-shaped 128K layer (RULER-128K on the LORE-KV page), 32 layers.
LLAMA_128K = LoreConfig(name="llama3.1-8b-128k-32layers", batch=1, n=131072, h_q=32,
                        h_kv=8, d=128, d_model=4096, dtype="bf16", seed=303,
                        recipe="facts", layers=32, window_from_facts=False)

# Qwen2.5-14B-shaped batched scoring: 8 sequences of 32K, GQA 5, B=512.
QWEN_14B_BATCH = LoreConfig(name="qwen2.5-14b-8x32k", batch=8, n=32768, h_q=40,
                            h_kv=8, d=128, d_model=5120, dtype="bf16", seed=404,
                            recipe="facts", budget=512, seed_per_seq=True,
                            omega_per_seq=True)

# H2O decode on an OPT-30B-shaped layer (56 heads, MHA), fp16.
OPT30B_H2O = H2OConfig(name="opt30b-h2o-b64-p1024-g512", batch=64, heads=56, d=128,
                       prompt=1024, steps=512, dtype="f16", seed=505)

@dataclass(frozen=True)
class RefreshConfig:
    """A counter-causal memory refresh: memory J, buffer h = J/4 (the review's
    Design choice 3), n = J + h cached tokens, n_sys system-prompt sinks."""
    name: str
    batch: int
    h_q: int
    h_kv: int
    d: int
    J: int
    n_sys: int
    dtype: str
    seed: int

    @property
    def h(self) -> int:
        return self.J // 4

    @property
    def n(self) -> int:
        return self.J + self.h

    def with_(self, **kw) -> "RefreshConfig":
        return replace(self, **kw)


# Qwen2.5-7B-shaped layer (28 query heads, 4 KV heads) at the largest cache
# the counter-causal review times (4096 kept tokens), bf16.
QWEN7B_REFRESH = RefreshConfig(name="qwen2.5-7b-refresh-J4096", batch=1, h_q=28, h_kv=4, d=128,
                               J=4096, n_sys=64, dtype="bf16", seed=606)

LORE_CONFIGS = {c.name: c for c in (TINY, MISTRAL_16K, LLAMA_128K, QWEN_14B_BATCH)}
H2O_CONFIGS = {OPT30B_H2O.name: OPT30B_H2O}
