"""Buffers and call order for the two eviction flows (device memory via torch).

``LoreEviction``: one LORE-KV eviction of one layer -- kvscore_probs,
kvscore_deletion, kvscore_topb_select, kv_compact on one stream, with every
intermediate preallocated on the device (LORE-KV Method: score, keep the
protected set plus the top-B per KV head, decode from the compacted cache).

``H2OCache``: H2O's preallocated slot cache (H2O page, System Implementation
Details): the prompt's accumulated attention, its reduction to the budget
(kvscore_topb_select with n_sink = 0, w = recent budget, chunk = 1), the load
into slots, then one kvscore_h2o_accumulate per decode step.
"""

import torch

from . import _lib as L


class LoreEviction:
    def __init__(self, desc: "L.LoreDesc", device="cuda"):
        self.desc = desc
        b, hq, hk, n, d, nq = desc.batch, desc.h_q, desc.h_kv, desc.n, desc.d, desc.n_q
        f32 = dict(dtype=torch.float32, device=device)
        self.row_max = torch.empty(b, hq, nq, **f32)
        self.row_sum = torch.empty(b, hq, nq, **f32)
        self.O = torch.empty(b, hq, nq, d, **f32)
        self.S = torch.empty(b, hk, n, **f32)
        self.kept = torch.empty(b, hk, desc.n_keep, dtype=torch.int32, device=device)
        self.ws = torch.empty(L.kvs_lore_workspace_bytes(desc), dtype=torch.uint8, device=device)
        self.omega = torch.empty(b, desc.m, **f32)

    def weights(self, Q, logp, entropy, coef=L.RELIABILITY_D, stream=None):
        """Trajectory weights omega (Eq. 10) from the lookahead rows of Q and the
        sampled tokens' log-probabilities and entropies [batch][m][t]."""
        L.kvscore_reliability_weights(self.desc, Q, logp, entropy, self.omega, coef, ws=self.ws,
                                      stream=stream)
        return self.omega

    def score(self, Q, K, V, W_O, omega, stream=None):
        L.kvscore_probs(self.desc, Q, K, V, self.row_max, self.row_sum, self.O, self.ws, stream)
        L.kvscore_deletion(self.desc, Q, K, V, W_O, omega, self.row_max, self.row_sum, self.O,
                           self.S, self.ws, stream)
        return self.S

    def baseline(self, kind, Q, K, V, stream=None):
        """Prompt-side baseline scores (L.KVS_BASELINE_WINDOW or L.KVS_BASELINE_TOVA)
        into S, for the same selector; runs pass 1 for the row statistics."""
        L.kvscore_probs(self.desc, Q, K, V, self.row_max, self.row_sum, self.O, self.ws, stream)
        L.kvscore_baseline_scores(self.desc, kind, Q, K, self.row_max, self.row_sum, self.S,
                                  self.ws, stream)
        return self.S

    def fidelity(self, Qf, K, V, K_keep, V_keep, stream=None):
        """Attention-output fidelity of the retained cache under held-out
        queries Qf [batch][h_q][n_f][d]: (cos [batch][h_q][n_f], mean [batch])."""
        b, hq, n_f = Qf.shape[0], Qf.shape[1], Qf.shape[2]
        dev = Qf.device
        cos = torch.empty(b, hq, n_f, dtype=torch.float32, device=dev)
        fid = torch.empty(b, dtype=torch.float32, device=dev)
        nb = L.kvs_fidelity_workspace_bytes(self.desc, n_f, K_keep.shape[2])
        ws = self.ws if self.ws.numel() >= nb else torch.empty(nb, dtype=torch.uint8, device=dev)
        L.kvscore_output_fidelity(self.desc, Qf, K, V, K_keep, V_keep, cos, fid, ws, stream)
        return cos, fid

    def select(self, pooled=None, stream=None):
        L.kvscore_topb_select(self.desc, self.S, self.kept, pooled, self.ws, stream)
        return self.kept

    def compact(self, K, V, K_out, V_out, pos_out=None, stream=None):
        L.kv_compact(K, V, self.kept, K_out, V_out, pos_out, stream=stream)

    def run(self, Q, K, V, W_O, omega, K_out, V_out, pos_out=None, stream=None):
        self.score(Q, K, V, W_O, omega, stream)
        self.select(stream=stream)
        self.compact(K, V, K_out, V_out, pos_out, stream)


class H2OCache:
    def __init__(self, batch, heads, d, cap, dtype=torch.float16, heavy_frac=0.1,
                 recent_frac=0.1, device="cuda"):
        self.batch, self.heads, self.d, self.cap, self.dtype = batch, heads, d, cap, dtype
        self.heavy_frac, self.recent_frac = heavy_frac, recent_frac
        self.K = torch.zeros(batch, heads, cap, d, dtype=dtype, device=device)
        self.V = torch.zeros(batch, heads, cap, d, dtype=dtype, device=device)
        self.slot_pos = torch.full((batch, heads, cap), -1, dtype=torch.int32, device=device)
        self.acc = torch.zeros(batch, heads, cap, dtype=torch.float32, device=device)
        self.O = torch.empty(batch, heads, d, dtype=dtype, device=device)
        self.evict_slot = torch.empty(batch, heads, dtype=torch.int32, device=device)
        self.cur_len = 0
        self.device = device

    def budget(self, cur_len):
        return int(self.heavy_frac * cur_len), int(self.recent_frac * cur_len)

    def prefill(self, Qp, Kp, Vp, stream=None):
        """Accumulate the causal prompt's attention, keep the recent budget
        plus the heaviest of the rest, and load them into slots."""
        b, h, P, d = Kp.shape
        pdesc = L.h2o_desc(batch=b, heads=h, d=d, cap=P, dtype=self.dtype)
        self.prompt_acc = torch.empty(b, h, P, dtype=torch.float32, device=self.device)
        k_h, k_r = self.budget(P)
        sdesc = L.lore_desc(batch=b, n=P, h_q=h, h_kv=h, d=d, d_model=1, w=k_r, m=0, t=0,
                            n_sink=0, chunk=1, budget=k_h, dtype=self.dtype)
        nbytes = max(L.kvs_h2o_workspace_bytes(pdesc, L.KVS_H2O_PREFILL),
                     L.kvs_topb_workspace_bytes(sdesc))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        L.kvscore_h2o_accumulate(pdesc, L.KVS_H2O_PREFILL, Qp, Kp, acc=self.prompt_acc, ws=ws,
                                 stream=stream)
        self.kept_prompt = torch.empty(b, h, sdesc.n_keep, dtype=torch.int32, device=self.device)
        L.kvscore_topb_select(sdesc, self.prompt_acc, self.kept_prompt, None, ws, stream)
        L.kv_compact(Kp, Vp, self.kept_prompt, self.K, self.V, self.slot_pos, self.prompt_acc,
                     self.acc, stream)
        self.cur_len = P

    def step(self, q, k, v, stream=None, with_output=True, write_slot=None):
        """One decode step: append, attend, accumulate, evict at most one.
        write_slot [batch][heads] int32 (optional): the free slot each row's new
        token goes into (else the lowest free slot)."""
        self.cur_len += 1
        k_h, k_r = self.budget(self.cur_len)
        desc = L.h2o_desc(batch=self.batch, heads=self.heads, d=self.d, cap=self.cap,
                          cur_len=self.cur_len, k_heavy=k_h, k_recent=k_r, dtype=self.dtype)
        L.kvscore_h2o_accumulate(desc, L.KVS_H2O_DECODE, q, self.K, self.V, k, v, self.slot_pos,
                                 self.acc, self.O if with_output else None, self.evict_slot,
                                 stream=stream, write_slot=write_slot)
        return self.O, self.evict_slot
