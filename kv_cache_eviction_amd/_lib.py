"""ctypes binding of libkvscore.so: same entry-point names as include/kvscore.h.

Argument marshalling only.  Every tensor must be a contiguous CUDA (HIP)
tensor of the stated shape and dtype; shapes are checked here, on the host,
before the C ABI is called, so a mismatched buffer never reaches a kernel.
The computation itself runs in the library's HIP kernels; there is no
fallback: if the library is missing, loading raises.
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVS_SANITIZED_BUILD=1 selects the host-sanitized debug build (build.py
# --sanitize; its runtime must be preloaded)
LIB_PATH = os.path.join(_PKG, "_build_san" if os.environ.get("KVS_SANITIZED_BUILD") == "1" else "",
                        "libkvscore.so")

KVS_F32, KVS_BF16, KVS_F16 = 0, 1, 2
KVS_H2O_PREFILL, KVS_H2O_DECODE = 0, 1
KVS_BASELINE_WINDOW, KVS_BASELINE_TOVA = 0, 1
KVS_MASK_NONE, KVS_MASK_WINDOW_CAUSAL, KVS_MASK_CAUSAL, KVS_MASK_SLOTS = 0, 1, 2, 3
DTYPE_CODE = {torch.float32: KVS_F32, torch.bfloat16: KVS_BF16, torch.float16: KVS_F16}
CODE_DTYPE = {v: k for k, v in DTYPE_CODE.items()}

EXPORTS = ("kvs_lore_workspace_bytes", "kvs_topb_workspace_bytes", "kvscore_probs", "kvscore_deletion",
           "kvscore_baseline_scores", "kvscore_reliability_weights", "kvs_fidelity_workspace_bytes",
           "kvscore_output_fidelity", "kvscore_counter_causal",
           "kvs_refresh_workspace_bytes", "kvscore_refresh", "kvscore_topb_select", "kvscore_topb_select_noalloc", "kvscore_retention_shift", "kv_compact", "kvs_h2o_workspace_bytes",
           "kvscore_h2o_accumulate", "kvs_measure_peaks", "kvs_timing_enable", "kvs_timing_count", "kvs_timing_read",
           "kvs_timing_reset", "kvs_last_error")


class KvsError(RuntimeError):
    pass


class LoreDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n", ctypes.c_int32), ("h_q", ctypes.c_int32),
                ("h_kv", ctypes.c_int32), ("d", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("w", ctypes.c_int32), ("m", ctypes.c_int32), ("t", ctypes.c_int32),
                ("n_sink", ctypes.c_int32), ("chunk", ctypes.c_int32), ("budget", ctypes.c_int32),
                ("eps", ctypes.c_float), ("lambda_l", ctypes.c_float), ("dtype", ctypes.c_int32)]

    @property
    def n_q(self):
        return self.w + self.m * self.t

    @property
    def n_keep(self):
        return self.n_sink + min(self.budget, self.n - self.n_sink - self.w) + self.w


class H2ODesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("d", ctypes.c_int32),
                ("cap", ctypes.c_int32), ("cur_len", ctypes.c_int32), ("k_heavy", ctypes.c_int32),
                ("k_recent", ctypes.c_int32), ("dtype", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkvscore.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise KvsError("%s is missing: build it with `python -m kv_cache_eviction_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    LP, HP = ctypes.POINTER(LoreDesc), ctypes.POINTER(H2ODesc)
    lib.kvs_last_error.restype = ctypes.c_char_p
    lib.kvs_last_error.argtypes = []
    lib.kvs_lore_workspace_bytes.restype = sz
    lib.kvs_lore_workspace_bytes.argtypes = [LP]
    lib.kvscore_probs.restype = i32
    lib.kvscore_probs.argtypes = [LP, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kvscore_deletion.restype = i32
    lib.kvscore_deletion.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kvscore_baseline_scores.restype = i32
    lib.kvscore_baseline_scores.argtypes = [LP, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    f32 = ctypes.c_float
    lib.kvscore_reliability_weights.restype = i32
    lib.kvscore_reliability_weights.argtypes = [LP, vp, vp, vp, f32, f32, f32, vp, vp, vp, sz, vp]
    lib.kvs_fidelity_workspace_bytes.restype = sz
    lib.kvs_fidelity_workspace_bytes.argtypes = [LP, i32, i32]
    lib.kvscore_output_fidelity.restype = i32
    lib.kvscore_output_fidelity.argtypes = [LP, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kvscore_counter_causal.restype = i32
    lib.kvscore_counter_causal.argtypes = [LP, vp, vp, vp, vp, vp, vp, vp]
    lib.kvs_refresh_workspace_bytes.restype = sz
    lib.kvs_refresh_workspace_bytes.argtypes = [i32, i32]
    lib.kvscore_refresh.restype = i32
    lib.kvscore_refresh.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                    vp, vp, sz, vp]
    lib.kvs_topb_workspace_bytes.restype = sz
    lib.kvs_topb_workspace_bytes.argtypes = [LP]
    lib.kvscore_topb_select.restype = i32
    lib.kvscore_topb_select.argtypes = [LP, vp, vp, vp, vp, sz, vp]
    lib.kvscore_retention_shift.restype = i32
    lib.kvscore_retention_shift.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp]
    lib.kvs_measure_peaks.restype = i32
    lib.kvs_measure_peaks.argtypes = [vp, sz, ctypes.POINTER(ctypes.c_float),
                                      ctypes.POINTER(ctypes.c_float), vp]
    lib.kvscore_topb_select_noalloc.restype = i32
    lib.kvscore_topb_select_noalloc.argtypes = [LP, vp, vp, vp, vp]
    lib.kv_compact.restype = i32
    lib.kv_compact.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kvs_h2o_workspace_bytes.restype = sz
    lib.kvs_h2o_workspace_bytes.argtypes = [HP, i32]
    lib.kvscore_h2o_accumulate.restype = i32
    lib.kvscore_h2o_accumulate.argtypes = [HP, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                           vp]
    lib.kvs_timing_enable.restype = i32
    lib.kvs_timing_enable.argtypes = [i32]
    lib.kvs_timing_count.restype = i32
    lib.kvs_timing_count.argtypes = []
    lib.kvs_timing_read.restype = i32
    lib.kvs_timing_read.argtypes = [i32, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)]
    lib.kvs_timing_reset.restype = None
    lib.kvs_timing_reset.argtypes = []
    _lib = lib
    return lib


def last_error() -> str:
    return load().kvs_last_error().decode()


def _check(status: int, name: str):
    if status != 0:
        raise KvsError("%s failed with status %d: %s" % (name, status, last_error()))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, shape, dtype, optional=False):
    if t is None:
        if optional:
            return
        raise KvsError("%s is required" % name)
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise KvsError("%s must be a device tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise KvsError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise KvsError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise KvsError("%s must be contiguous" % name)


def lore_desc(*, batch, n, h_q, h_kv, d, d_model, w=32, m=4, t=8, n_sink=1, chunk=4,
              budget=128, eps=1e-6, lambda_l=1.0, dtype=torch.bfloat16) -> LoreDesc:
    return LoreDesc(batch, n, h_q, h_kv, d, d_model, w, m, t, n_sink, chunk, budget, eps,
                    lambda_l, DTYPE_CODE[dtype])


def h2o_desc(*, batch, heads, d, cap, cur_len=0, k_heavy=0, k_recent=0,
             dtype=torch.float16) -> H2ODesc:
    return H2ODesc(batch, heads, d, cap, cur_len, k_heavy, k_recent, DTYPE_CODE[dtype])


def kvs_lore_workspace_bytes(desc: LoreDesc) -> int:
    nb = load().kvs_lore_workspace_bytes(ctypes.byref(desc))
    if nb == 0:
        raise KvsError("invalid descriptor: " + last_error())
    return nb


def _ws_check(ws, need):
    if need and (ws is None or ws.device.type != "cuda" or ws.numel() * ws.element_size() < need):
        raise KvsError("workspace must be a device tensor of at least %d bytes" % need)


def kvscore_probs(desc, Q, K, V, row_max, row_sum, O, ws, stream=None,
                  mask=KVS_MASK_WINDOW_CAUSAL, P=None):
    dt = CODE_DTYPE[desc.dtype]
    b, hq, hk, n, d, nq = desc.batch, desc.h_q, desc.h_kv, desc.n, desc.d, desc.n_q
    _need(Q, "Q", (b, hq, nq, d), dt)
    _need(K, "K", (b, hk, n, d), dt)
    _need(V, "V", (b, hk, n, d), dt)
    _need(row_max, "row_max", (b, hq, nq), torch.float32)
    _need(row_sum, "row_sum", (b, hq, nq), torch.float32)
    _need(O, "O", (b, hq, nq, d), torch.float32)
    _need(P, "P", (b, hq, nq, n), torch.float32, optional=True)
    need = kvs_lore_workspace_bytes(desc)
    _ws_check(ws, need)
    _check(load().kvscore_probs(ctypes.byref(desc), int(mask), _ptr(Q), _ptr(K), _ptr(V), _ptr(row_max),
                                _ptr(row_sum), _ptr(O), _ptr(P), _ptr(ws), ws.numel() * ws.element_size(),
                                _stream(stream)), "kvscore_probs")


def kvscore_deletion(desc, Q, K, V, W_O, omega, row_max, row_sum, O, S, ws, stream=None):
    dt = CODE_DTYPE[desc.dtype]
    b, hq, hk, n, d, nq = desc.batch, desc.h_q, desc.h_kv, desc.n, desc.d, desc.n_q
    _need(Q, "Q", (b, hq, nq, d), dt)
    _need(K, "K", (b, hk, n, d), dt)
    _need(V, "V", (b, hk, n, d), dt)
    _need(W_O, "W_O", (desc.d_model, hq * d), dt)
    _need(omega, "omega", (b, desc.m), torch.float32, optional=desc.m == 0)
    _need(row_max, "row_max", (b, hq, nq), torch.float32)
    _need(row_sum, "row_sum", (b, hq, nq), torch.float32)
    _need(O, "O", (b, hq, nq, d), torch.float32)
    _need(S, "S", (b, hk, n), torch.float32)
    need = kvs_lore_workspace_bytes(desc)
    _ws_check(ws, need)
    _check(load().kvscore_deletion(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V), _ptr(W_O),
                                   _ptr(omega), _ptr(row_max), _ptr(row_sum), _ptr(O), _ptr(S),
                                   _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "kvscore_deletion")


def kvscore_baseline_scores(desc, kind, Q, K, row_max, row_sum, S, ws, stream=None):
    """kind: KVS_BASELINE_WINDOW or KVS_BASELINE_TOVA; row_max, row_sum from
    kvscore_probs on the same Q, K."""
    dt = CODE_DTYPE[desc.dtype]
    b, hq, hk, n, d, nq = desc.batch, desc.h_q, desc.h_kv, desc.n, desc.d, desc.n_q
    _need(Q, "Q", (b, hq, nq, d), dt)
    _need(K, "K", (b, hk, n, d), dt)
    _need(row_max, "row_max", (b, hq, nq), torch.float32)
    _need(row_sum, "row_sum", (b, hq, nq), torch.float32)
    _need(S, "S", (b, hk, n), torch.float32)
    need = kvs_lore_workspace_bytes(desc)
    _ws_check(ws, need)
    _check(load().kvscore_baseline_scores(ctypes.byref(desc), int(kind), _ptr(Q), _ptr(K),
                                          _ptr(row_max), _ptr(row_sum), _ptr(S), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)),
           "kvscore_baseline_scores")


RELIABILITY_E = (1.0, 1.3, 0.0)  # LORE-KV /E (beta, gamma, lambda_d)
RELIABILITY_D = (1.0, 1.0, 0.3)  # LORE-KV /D


def kvscore_reliability_weights(desc, Q, logp, entropy, omega, coef=RELIABILITY_D, dhat=None,
                                ws=None, stream=None):
    """Trajectory weights omega [batch][m] from the lookahead queries in Q and
    the per-token log-probability and entropy [batch][m][t]; coef = (beta,
    gamma, lambda_d)."""
    dt = CODE_DTYPE[desc.dtype]
    b, hq, nq, d, m, t = desc.batch, desc.h_q, desc.n_q, desc.d, desc.m, desc.t
    _need(Q, "Q", (b, hq, nq, d), dt)
    _need(logp, "logp", (b, m, t), torch.float32)
    _need(entropy, "entropy", (b, m, t), torch.float32)
    _need(omega, "omega", (b, m), torch.float32)
    _need(dhat, "dhat", (b, m), torch.float32, optional=True)
    beta, gamma, lambda_d = (float(c) for c in coef)
    if ws is not None:
        _ws_check(ws, kvs_lore_workspace_bytes(desc))
    _check(load().kvscore_reliability_weights(
        ctypes.byref(desc), _ptr(Q), _ptr(logp), _ptr(entropy), beta, gamma, lambda_d,
        _ptr(omega), _ptr(dhat), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream)), "kvscore_reliability_weights")


def kvs_fidelity_workspace_bytes(desc: LoreDesc, n_f: int, n_keep: int) -> int:
    nb = load().kvs_fidelity_workspace_bytes(ctypes.byref(desc), int(n_f), int(n_keep))
    if nb == 0:
        raise KvsError("invalid fidelity arguments: " + last_error())
    return nb


def kvscore_output_fidelity(desc, Qf, K, V, K_keep, V_keep, cos_out, fidelity, ws, stream=None):
    """Cosine between each held-out query's attention output over the full
    cache (K, V) and over the retained cache (K_keep, V_keep), per query head,
    and the mean per sequence."""
    dt = CODE_DTYPE[desc.dtype]
    b, hq, hk, n, d = desc.batch, desc.h_q, desc.h_kv, desc.n, desc.d
    if Qf is None or K_keep is None:
        raise KvsError("Qf and K_keep are required")
    n_f, n_keep = Qf.shape[2], K_keep.shape[2]
    _need(Qf, "Qf", (b, hq, n_f, d), dt)
    _need(K, "K", (b, hk, n, d), dt)
    _need(V, "V", (b, hk, n, d), dt)
    _need(K_keep, "K_keep", (b, hk, n_keep, d), dt)
    _need(V_keep, "V_keep", (b, hk, n_keep, d), dt)
    _need(cos_out, "cos_out", (b, hq, n_f), torch.float32)
    _need(fidelity, "fidelity", (b,), torch.float32)
    _ws_check(ws, kvs_fidelity_workspace_bytes(desc, n_f, n_keep))
    _check(load().kvscore_output_fidelity(ctypes.byref(desc), n_f, n_keep, _ptr(Qf), _ptr(K),
                                          _ptr(V), _ptr(K_keep), _ptr(V_keep), _ptr(cos_out),
                                          _ptr(fidelity), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)),
           "kvscore_output_fidelity")


def kvscore_counter_causal(desc, Q, K, V, row_max, row_sum, O, stream=None):
    """Every cached position's fresh query attends to the keys after it."""
    dt = CODE_DTYPE[desc.dtype]
    b, hq, hk, n, d = desc.batch, desc.h_q, desc.h_kv, desc.n, desc.d
    _need(Q, "Q", (b, hq, n, d), dt)
    _need(K, "K", (b, hk, n, d), dt)
    _need(V, "V", (b, hk, n, d), dt)
    _need(row_max, "row_max", (b, hq, n), torch.float32)
    _need(row_sum, "row_sum", (b, hq, n), torch.float32)
    _need(O, "O", (b, hq, n, d), torch.float32)
    _check(load().kvscore_counter_causal(ctypes.byref(desc), _ptr(Q), _ptr(K), _ptr(V),
                                         _ptr(row_max), _ptr(row_sum), _ptr(O), _stream(stream)),
           "kvscore_counter_causal")


def kvs_refresh_workspace_bytes(batch: int, n: int) -> int:
    nb = load().kvs_refresh_workspace_bytes(int(batch), int(n))
    if nb == 0:
        raise KvsError("invalid refresh sizes: " + last_error())
    return nb


def kvscore_refresh(surprise, K, V, kept, K_out, V_out, *, n_sys, J, ids=None, ids_out=None,
                    ws=None, stream=None):
    """Keep the J most surprising of the n cached tokens per sequence (system
    prompt and last token protected) and gather K, V (and token ids)."""
    if K is None:
        raise KvsError("K is required")
    b, heads, n, d = K.shape
    keep = min(int(J), n)
    _need(surprise, "surprise", (b, n), torch.float32)
    _need(V, "V", (b, heads, n, d), K.dtype)
    _need(kept, "kept", (b, keep), torch.int32)
    _need(K_out, "K_out", (b, heads, keep, d), K.dtype)
    _need(V_out, "V_out", (b, heads, keep, d), K.dtype)
    _need(ids, "ids", (b, n), torch.int32, optional=True)
    _need(ids_out, "ids_out", (b, keep), torch.int32, optional=True)
    _ws_check(ws, kvs_refresh_workspace_bytes(b, n))
    _check(load().kvscore_refresh(b, heads, n, d, DTYPE_CODE[K.dtype], int(n_sys), int(J),
                                  _ptr(surprise), _ptr(K), _ptr(V), _ptr(ids), _ptr(kept),
                                  _ptr(K_out), _ptr(V_out), _ptr(ids_out), _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)),
           "kvscore_refresh")


def kvs_topb_workspace_bytes(desc: LoreDesc) -> int:
    nb = load().kvs_topb_workspace_bytes(ctypes.byref(desc))
    if nb == 0:
        raise KvsError("invalid descriptor: " + last_error())
    return nb


def kvscore_topb_select(desc, S, kept, pooled, ws, stream=None):
    b, hk, n = desc.batch, desc.h_kv, desc.n
    _need(S, "S", (b, hk, n), torch.float32)
    _need(kept, "kept", (b, hk, desc.n_keep), torch.int32)
    _need(pooled, "pooled", (b, hk, n), torch.float32, optional=True)
    need = kvs_topb_workspace_bytes(desc)
    _ws_check(ws, need)
    _check(load().kvscore_topb_select(ctypes.byref(desc), _ptr(S), _ptr(kept), _ptr(pooled),
                                      _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "kvscore_topb_select")


def kvscore_topb_select_noalloc(desc, S, kept, pooled=None, stream=None):
    """kvscore_topb_select on the library's own scratch (no workspace, no
    allocation); rejects inputs whose selection needs more than
    KVS_TOPB_NOALLOC_MAX_BYTES of scratch."""
    b, hk, n = desc.batch, desc.h_kv, desc.n
    _need(S, "S", (b, hk, n), torch.float32)
    _need(kept, "kept", (b, hk, desc.n_keep), torch.int32)
    _need(pooled, "pooled", (b, hk, n), torch.float32, optional=True)
    _check(load().kvscore_topb_select_noalloc(ctypes.byref(desc), _ptr(S), _ptr(kept),
                                              _ptr(pooled), _stream(stream)),
           "kvscore_topb_select_noalloc")


def kvscore_retention_shift(kept_a, kept_b, shift, *, n, n_sink, w, stream=None):
    """Per kept list, the share of kept_a's candidates [n_sink, n - w) absent
    from kept_b (ascending); kept_a, kept_b [..][n_keep] int32, shift [..] fp32."""
    if kept_a is None or kept_b is None:
        raise KvsError("kept_a and kept_b are required")
    lead, n_keep = tuple(kept_a.shape[:-1]), kept_a.shape[-1]
    _need(kept_a, "kept_a", lead + (n_keep,), torch.int32)
    _need(kept_b, "kept_b", lead + (n_keep,), torch.int32)
    _need(shift, "shift", lead, torch.float32)
    rows = 1
    for x in lead:
        rows *= x
    _check(load().kvscore_retention_shift(rows, n_keep, int(n), int(n_sink), int(w), _ptr(kept_a),
                                          _ptr(kept_b), _ptr(shift), _stream(stream)),
           "kvscore_retention_shift")


def kv_compact(K, V, kept, K_out, V_out, pos_out=None, score_in=None, score_out=None,
               stream=None):
    """K, V [b][heads][n_src][d]; kept [b][heads][n_keep] int32 (each in [0, n_src));
    K_out, V_out [b][heads][cap][d]; pos_out [b][heads][cap] int32; score_in
    [b][heads][n_src] fp32 -> score_out [b][heads][cap]."""
    if K is None or K.dim() != 4:
        raise KvsError("K must be [batch][heads][n_src][d]")
    b, h, n_src, d = K.shape
    dt = K.dtype
    _need(V, "V", K.shape, dt)
    if kept is None or kept.dim() != 3:
        raise KvsError("kept must be [batch][heads][n_keep]")
    n_keep = kept.shape[2]
    _need(kept, "kept", (b, h, n_keep), torch.int32)
    if K_out is None or K_out.dim() != 4:
        raise KvsError("K_out must be [batch][heads][cap][d]")
    cap = K_out.shape[2]
    _need(K_out, "K_out", (b, h, cap, d), dt)
    _need(V_out, "V_out", (b, h, cap, d), dt)
    _need(pos_out, "pos_out", (b, h, cap), torch.int32, optional=True)
    _need(score_in, "score_in", (b, h, n_src), torch.float32, optional=True)
    _need(score_out, "score_out", (b, h, cap), torch.float32, optional=score_in is None)
    _check(load().kv_compact(b, h, n_src, n_keep, cap, d, DTYPE_CODE[dt], _ptr(K), _ptr(V),
                             _ptr(kept), _ptr(K_out), _ptr(V_out), _ptr(pos_out), _ptr(score_in),
                             _ptr(score_out), _stream(stream)), "kv_compact")


def kvs_h2o_workspace_bytes(desc: H2ODesc, mode: int) -> int:
    return load().kvs_h2o_workspace_bytes(ctypes.byref(desc), mode)


def kvscore_h2o_accumulate(desc, mode, q, K, V=None, k_new=None, v_new=None, slot_pos=None,
                           acc=None, O=None, evict_slot=None, ws=None, stream=None,
                           write_slot=None):
    dt = CODE_DTYPE[desc.dtype]
    b, h, d, cap = desc.batch, desc.heads, desc.d, desc.cap
    if mode == KVS_H2O_PREFILL:
        _need(q, "q", (b, h, cap, d), dt)
        _need(K, "K", (b, h, cap, d), dt)
        _need(acc, "acc", (b, h, cap), torch.float32)
        need = kvs_h2o_workspace_bytes(desc, mode)
        if need == 0:
            raise KvsError("invalid descriptor: " + last_error())
        _ws_check(ws, need)
        nb = ws.numel() * ws.element_size()
    elif mode == KVS_H2O_DECODE:
        _need(q, "q", (b, h, d), dt)
        _need(K, "K", (b, h, cap, d), dt)
        _need(V, "V", (b, h, cap, d), dt)
        _need(k_new, "k_new", (b, h, d), dt)
        _need(v_new, "v_new", (b, h, d), dt)
        _need(slot_pos, "slot_pos", (b, h, cap), torch.int32)
        _need(acc, "acc", (b, h, cap), torch.float32)
        _need(O, "O", (b, h, d), dt, optional=True)
        _need(evict_slot, "evict_slot", (b, h), torch.int32, optional=True)
        _need(write_slot, "write_slot", (b, h), torch.int32, optional=True)
        nb = 0
    else:
        raise KvsError("unknown H2O mode %r" % (mode,))
    _check(load().kvscore_h2o_accumulate(ctypes.byref(desc), mode, _ptr(q), _ptr(K), _ptr(V),
                                         _ptr(k_new), _ptr(v_new), _ptr(write_slot),
                                         _ptr(slot_pos), _ptr(acc),
                                         _ptr(O), _ptr(evict_slot), _ptr(ws), nb, _stream(stream)),
           "kvscore_h2o_accumulate")


def kvs_measure_peaks(buf, stream=None):
    """Measured dense bf16 MFMA TFLOP/s and streaming HBM read GB/s on a
    caller-owned device buffer (uint8, >= 66 MiB; 1 GiB recommended)."""
    if buf is None or not buf.is_cuda or not buf.is_contiguous():
        raise KvsError("kvs_measure_peaks: buf must be a contiguous device tensor")
    tf, gb = ctypes.c_float(), ctypes.c_float()
    _check(load().kvs_measure_peaks(_ptr(buf), buf.numel() * buf.element_size(), ctypes.byref(tf),
                                    ctypes.byref(gb), _stream(stream)), "kvs_measure_peaks")
    return tf.value, gb.value


def kvs_timing_enable(on: bool = True):
    _check(load().kvs_timing_enable(1 if on else 0), "kvs_timing_enable")


def kvs_timing_reset():
    load().kvs_timing_reset()


def kvs_timing_records():
    """[(kernel name, ms)] of every launch recorded since the last reset."""
    lib = load()
    out = []
    name, ms = ctypes.c_char_p(), ctypes.c_float()
    for i in range(lib.kvs_timing_count()):
        _check(lib.kvs_timing_read(i, ctypes.byref(name), ctypes.byref(ms)), "kvs_timing_read")
        out.append((name.value.decode(), ms.value))
    return out
