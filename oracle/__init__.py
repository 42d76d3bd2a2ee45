"""Plain, slow fp64 oracle for KV-cache scoring, selection, compaction and H2O.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The HIP product path never imports
it, and it imports nothing from the product package.

Sources followed (cited per function):
  * LORE-KV project page, "Monte Carlo Estimation for KV-Cache Eviction":
    Method ("Prefill", "Projected deletion score" Eqs. 5-7, "Evict and decode"
    Eq. 8) and the Hyperparameters table (w, M, T, lambda_L, eps, chunk).
  * H2O summary page, "H2O: Heavy-Hitter Oracle": 3.4 formal problem
    formulation (Defs. 2.1-2.2), the H2O eviction algorithm (accumulated
    scores, greedy eviction, budget split), System Implementation Details.
  * LORE-KV page, Method, "Reliability weights" (Eqs. 2-4, 10): the
    trajectory weights omega; "Why it works", "Output fidelity": the
    attention-output fidelity of a retained cache.
  * counter-causal review "Back from the Future", 3.2 (reversed mask over
    the cached keys and values) and Alg. 3 (memory refresh): counter-causal
    attention and the refresh selection.
  * LORE-KV page, "The query-reference mismatch" ("Prompt-side eviction") and
    the counter-causal review "Back from the Future", "Prerequisites"
    (TOVA): the prompt-side baseline scores.

Readings taken where the pages leave a step open (each also listed in the
design notes): softmax logits carry 1/sqrt(d); window rows are causal at their
own positions; psi is the arithmetic mean; the GQA group score is the mean of
its query heads' scores; chunk pooling is the mean over a chunk's candidate
members; ties rank by lower index; H2O's budget is floor(frac * current
length) per part, the recent part is protected, and the prompt is reduced to
the budget by accumulated column sums before decoding; the prompt-side
baseline scores sum the window rows' attention (TOVA: the last window row
only) and take the GQA group mean; the trajectory disagreement D_m is the mean
(1 - cosine) between its lookahead queries and every other trajectory's, per
query head, standardized over the trajectories (zero below a spread of 1e-6); output
fidelity is the mean cosine between per-head attention outputs over the full
and the retained cache; the memory refresh keeps its survivors in position
order, protects the system prompt and the last token, and breaks ties toward
the lower position; the retention-order shift is the share of one
selection's kept candidates (protected tokens left out) that the other
selection does not keep.

Every function here is pinned by tests to what the pages and the mathematics
fix (worked examples, closed forms, invariants, brute force on tiny inputs).
The readings above are conventions no page fixes: parity on those choices is
unpinned, and they are listed with the design notes.
"""

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lore_oracle.c")
# KVS_SANITIZED_BUILD=1 selects the AddressSanitizer + UBSan build (clang,
# the same sanitizer runtime as the library's sanitized build)
_SANITIZED = os.environ.get("KVS_SANITIZED_BUILD") == "1"
_BUILD = os.path.join(_HERE, "_build_san" if _SANITIZED else "_build")
_SO = os.path.join(_BUILD, "liboracle.so")
_lib_handle = None

_DP = ctypes.POINTER(ctypes.c_double)


def build(force: bool = False) -> str:
    """Compile the C part of the oracle with gcc (IEEE fp64: no fast-math).
    With KVS_SANITIZED_BUILD=1: ROCm's clang with AddressSanitizer and
    UndefinedBehaviorSanitizer and its OpenMP runtime, into _build_san/."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        if _SANITIZED:
            llvm = "/opt/rocm/llvm"
            cmd = [llvm + "/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer",
                   "-fsanitize=address,undefined", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                   "-ffp-contract=off", _SRC, "-o", tmp, "-L" + llvm + "/lib",
                   "-Wl,-rpath," + llvm + "/lib", "-lm"]
        else:
            cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                   "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _SO)
    return _SO


def _lib():
    global _lib_handle
    if _lib_handle is None:
        lib = ctypes.CDLL(build())
        i, d = ctypes.c_int, ctypes.c_double
        lib.ora_lore_attention.argtypes = [i, i, i, i, i, i, i, _DP, _DP, _DP, _DP, _DP, _DP, i]
        lib.ora_lore_attention.restype = i
        lib.ora_lore_scores.argtypes = [i, i, i, i, i, i, i, i, d, d,
                                        _DP, _DP, _DP, _DP, _DP, _DP, _DP, _DP, _DP, i]
        lib.ora_lore_scores.restype = i
        lib.ora_max_threads.argtypes = []
        lib.ora_max_threads.restype = i
        _lib_handle = lib
    return _lib_handle


def max_threads() -> int:
    return _lib().ora_max_threads()


def _f64(x):
    """Exact widening to a contiguous fp64 numpy array (torch tensors accepted)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(_DP)


# --------------------------------------------------------------------------
# LORE-KV
# --------------------------------------------------------------------------

def lore_attention(Q, K, V, w, nthreads=0):
    """Softmax statistics and outputs of the w + M*T scoring rows.

    LORE-KV page, Method: "Prefill" keeps the window queries of the last w
    prompt tokens; Eq. 5 uses the attention output o_q.  Row r < w sees
    tokens 0..n-w+r (causal at its own position); later rows see all n.
    Returns (row_max [b][h_q][n_q], row_sum [b][h_q][n_q], O [b][h_q][n_q][d]).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    b, h_q, n_q, d = Q.shape
    _, h_kv, n, _ = K.shape
    m = np.empty((b, h_q, n_q)); l = np.empty((b, h_q, n_q)); O = np.empty((b, h_q, n_q, d))
    rc = _lib().ora_lore_attention(b, n, h_q, h_kv, d, n_q, w, _ptr(Q), _ptr(K), _ptr(V),
                                   _ptr(m), _ptr(l), _ptr(O), int(nthreads))
    if rc != 0:
        raise ValueError("ora_lore_attention: invalid shape")
    return m, l, O


def lore_probabilities(Q, K, w):
    """The attention probabilities a_{q,i} of every scoring row over the cache.

    LORE-KV page, Method (a_{q,i} of Eq. 5, softmax of q.k_i / sqrt(d)), with
    the visibility of lore_attention: row r < w sees tokens 0..n-w+r, later
    rows all n; invisible entries are exactly 0.  Written out directly
    (logits, row maximum, exponentials, row sum), not through
    lore_attention.  Returns P [b][h_q][n_q][n] fp64.
    """
    Q, K = _f64(Q), _f64(K)
    b, h_q, n_q, d = Q.shape
    _, h_kv, n, _ = K.shape
    G = h_q // h_kv
    P = np.zeros((b, h_q, n_q, n))
    for bi in range(b):
        for h in range(h_q):
            s = Q[bi, h] @ K[bi, h // G].T / math.sqrt(d)          # [n_q][n]
            for r in range(n_q):
                last = n - w + r if r < w else n - 1
                row = s[r, :last + 1]
                e = np.exp(row - row.max())
                P[bi, h, r, :last + 1] = e / e.sum()
    return P


def projection_factors(W_O, h_q, d):
    """R_h (upper triangular) with R_h^T R_h = W_h^T W_h for every query head.

    W_h is the d_model x d column slice h*d..h*d+d-1 of W_O (the head's output
    projection, LORE-KV page Eq. 6).  ||W_h x|| == ||R_h x|| for every x, so
    the oracle can take the projected norm in d dimensions.  The Cholesky
    factorisation is the library step.
    """
    W = _f64(W_O)
    R = np.empty((h_q, d, d))
    for h in range(h_q):
        Wh = W[:, h * d:(h + 1) * d]
        L = np.linalg.cholesky(Wh.T @ Wh)
        R[h] = L.T
    return R


def lore_scores(Q, K, V, W_O, omega, *, w, m, t, eps, lambda_l, nthreads=0, R=None):
    """Projected deletion score of every cached token for every KV head.

    LORE-KV page, "Projected deletion score", Eqs. 5-7, with psi the mean and
    the KV head's score the mean over its GQA group of query heads ("Evict and
    decode", Eq. 8: each KV head keeps its own top-B).
    Returns a dict: S [b][h_kv][n], S_head [b][h_q][n], row_max, row_sum, O.
    """
    Q, K, V, omega = _f64(Q), _f64(K), _f64(V), _f64(omega)
    b, h_q, n_q, d = Q.shape
    _, h_kv, n, _ = K.shape
    if n_q != w + m * t:
        raise ValueError("n_q must equal w + m*t")
    if R is None:
        R = projection_factors(W_O, h_q, d)
    R = _f64(R)
    row_max, row_sum, O = lore_attention(Q, K, V, w, nthreads)
    S_head = np.empty((b, h_q, n))
    rc = _lib().ora_lore_scores(b, n, h_q, h_kv, d, w, m, t, float(eps), float(lambda_l),
                                _ptr(Q), _ptr(K), _ptr(V), _ptr(R), _ptr(omega),
                                _ptr(row_max), _ptr(row_sum), _ptr(O), _ptr(S_head),
                                int(nthreads))
    if rc != 0:
        raise ValueError("ora_lore_scores: invalid shape (%d)" % rc)
    S = S_head.reshape(b, h_kv, h_q // h_kv, n).mean(axis=2)
    return {"S": S, "S_head": S_head, "row_max": row_max, "row_sum": row_sum, "O": O}


def baseline_scores(Q, K, *, w, kind):
    """Prompt-side attention scores of every cached token per KV head.

    kind "window": the LORE-KV page's prompt-side baseline ("The
    query-reference mismatch", "Prompt-side eviction"): a token ranks by how
    the last w prompt queries attend to it, S_i = sum_{r<w} a_{r,i}.
    kind "tova": the counter-causal review's TOVA ("Prerequisites",
    attention-based eviction): the last prompt token's attention only,
    S_i = a_{w-1,i}.  Window row r is causal at position n-w+r, as in
    lore_attention; the KV head's score is the mean over its query heads.
    Returns S [b][h_kv][n].
    """
    if kind not in ("window", "tova"):
        raise ValueError("kind must be 'window' or 'tova'")
    Q, K = _f64(Q), _f64(K)
    b, h_q, n_q, d = Q.shape
    _, h_kv, n, _ = K.shape
    G = h_q // h_kv
    rows = range(w) if kind == "window" else [w - 1]
    S = np.zeros((b, h_kv, n))
    for bb in range(b):
        for h in range(h_q):
            g = h // G
            for r in rows:
                s = K[bb, g] @ Q[bb, h, r] / math.sqrt(d)
                s[n - w + r + 1:] = -np.inf  # causal at its own position
                s = np.exp(s - s.max())
                S[bb, g] += s / s.sum() / G
    return S


def counter_causal_attention(Q, K, V):
    """Counter-causal attention over a cache (counter-causal review, 3.2
    "The approximation: reusing cached K/V with a reversed mask", Steps 1 and
    3): the fresh query of every cached position i attends only to the cached
    keys of positions j > i (a strictly upper-triangular mask) with the usual
    softmax(q k^T / sqrt(d)) weights and original positions.  The last position
    sees no key (Step 5 treats it separately): its row_max is -inf, row_sum 0
    and output 0.
    Q [b][h_q][n][d]; K, V [b][h_kv][n][d] (query head h uses KV head h // G).
    Returns (row_max [b][h_q][n] in units of q.k/sqrt(d), row_sum, O [b][h_q][n][d]).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    b, h_q, n, d = Q.shape
    G = h_q // K.shape[1]
    row_max = np.full((b, h_q, n), -np.inf)
    row_sum = np.zeros((b, h_q, n))
    O = np.zeros((b, h_q, n, d))
    for bb in range(b):
        for h in range(h_q):
            g = h // G
            s = Q[bb, h] @ K[bb, g].T / math.sqrt(d)
            for i in range(n - 1):
                row = s[i, i + 1:]
                mx = row.max()
                p = np.exp(row - mx)
                row_max[bb, h, i] = mx
                row_sum[bb, h, i] = p.sum()
                O[bb, h, i] = p @ V[bb, g, i + 1:] / p.sum()
    return row_max, row_sum, O


def refresh_select(surprise, *, n_sys, J):
    """Memory refresh selection (counter-causal review, Alg. 3 with design
    choice 4 and the boundary rule of 3.2 Step 5): of the n = J + h cached
    tokens keep the J of largest surprise; the n_sys system-prompt tokens are
    never evicted and the last token is always kept.  Ties go to the lower
    position; the kept positions are returned in ascending order (so the next
    refresh's mask still means "later positions").  J = 0 keeps nothing.
    surprise [b][n]; needs J = 0 or J >= min(n, n_sys + 1).
    Returns kept [b][min(J, n)] int64.
    """
    S = _f64(surprise)
    b, n = S.shape
    keep = min(J, n)
    if keep == 0:
        return np.zeros((b, 0), dtype=np.int64)
    protected = sorted(set(range(min(n_sys, n))) | {n - 1})
    if keep < len(protected):
        raise ValueError("J smaller than the protected set")
    kept = np.empty((b, keep), dtype=np.int64)
    for bb in range(b):
        rest = [i for i in range(n) if i not in protected]
        rest.sort(key=lambda i: (-S[bb, i], i))
        kept[bb] = sorted(protected + rest[:keep - len(protected)])
    return kept


def refresh_gather(K, V, ids, kept):
    """K' = K[kept], V' = V[kept] on every head, X' = X[kept] (Alg. 3: the kept
    entries of K, V and the token ids stay in one-to-one correspondence).
    K, V [b][h][n][d]; ids [b][n]; kept [b][J].  Returns (K', V', X')."""
    K, V = np.asarray(K), np.asarray(V)
    ids, kept = np.asarray(ids), np.asarray(kept)
    b = K.shape[0]
    Ko = np.stack([K[bb][:, kept[bb]] for bb in range(b)])
    Vo = np.stack([V[bb][:, kept[bb]] for bb in range(b)])
    Xo = np.stack([ids[bb][kept[bb]] for bb in range(b)])
    return Ko, Vo, Xo


def output_fidelity(Qf, K, V, kept):
    """Attention-output fidelity of a retained cache (LORE-KV page, "Why it
    works", "Output fidelity": how closely the retained cache reproduces the
    full cache's attention outputs).

    Read as: for every held-out query row r of query head h, the cosine between
    o_full = softmax(q K^T / sqrt(d)) V over all n tokens of the head's KV head
    and o_kept, the same over the kept tokens only (renormalised), both in the
    head's value space; the fidelity is the mean over heads and rows.  Two zero
    outputs agree (cosine 1); one zero output has cosine 0.
    Qf [b][h_q][n_f][d]; K, V [b][h_kv][n][d]; kept [b][h_kv][n_keep] indices.
    Returns dict(cos [b][h_q][n_f], fidelity [b]).
    """
    Qf, K, V = _f64(Qf), _f64(K), _f64(V)
    kept = np.asarray(kept.cpu() if hasattr(kept, "cpu") else kept).astype(np.int64)
    b, h_q, n_f, d = Qf.shape
    h_kv = K.shape[1]
    G = h_q // h_kv

    def attend(q, Kx, Vx):
        s = q @ Kx.T / math.sqrt(d)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        return (p / p.sum(axis=1, keepdims=True)) @ Vx

    cos = np.empty((b, h_q, n_f))
    for bb in range(b):
        for h in range(h_q):
            g = h // G
            idx = kept[bb, g]
            of = attend(Qf[bb, h], K[bb, g], V[bb, g])
            ok = attend(Qf[bb, h], K[bb, g][idx], V[bb, g][idx])
            nf, nk = np.linalg.norm(of, axis=1), np.linalg.norm(ok, axis=1)
            both = (nf == 0) & (nk == 0)
            one = (nf == 0) ^ (nk == 0)
            den = np.where((nf == 0) | (nk == 0), 1.0, nf * nk)
            c = (of * ok).sum(axis=1) / den
            cos[bb, h] = np.where(both, 1.0, np.where(one, 0.0, c))
    return {"cos": cos, "fidelity": cos.mean(axis=(1, 2))}


STD_FLOOR = 1e-6  # below this spread the disagreements are taken as equal


def centered_score(probs, y):
    """Centered score of one sampled token (LORE-KV "Reliability weights",
    Eqs. 2-4): c = log q(y | h) + H(q(. | h)), from the full next-token
    distribution `probs` and the sampled index `y`.  Returns (c, H)."""
    p = np.asarray(probs, dtype=np.float64)
    nz = p > 0
    H = float(-(p[nz] * np.log(p[nz])).sum())
    return float(math.log(p[y])) + H, H


def reliability_weights(Q, logp, entropy, *, w, m, t, beta, gamma, lambda_d):
    """Trajectory weights omega of Eq. 10 (LORE-KV "Reliability weights"):
    R_m = beta * cbar_m - gamma * Hbar_m - lambda_d * Dhat_m, omega = softmax(R).

    Q [b][h_q][w + m*t][d]: the scoring queries; rows w + j*t .. w + j*t + t-1
    are trajectory j's lookahead queries.  logp, entropy [b][m][t]: log q(y_u)
    of each sampled token and the entropy of the distribution it was drawn
    from, so c_u = logp_u + entropy_u (Eqs. 2-4); cbar_m and Hbar_m are the
    means over the trajectory's t tokens.

    Dhat_m, "the standardized cosine disagreement of trajectory m's queries
    with the others", is read as: D_m = mean of (1 - cos(q, q')) over every
    query head, every query q of trajectory m and every query q' of every other
    trajectory at the same head (a query of zero norm has cosine 0 with all);
    Dhat = (D - mean D) / std D over the m trajectories (population std), and
    Dhat = 0 when that std is below STD_FLOOR (all trajectories equally
    typical, e.g. m = 2, where D_1 = D_2 by symmetry).
    Returns dict(omega [b][m], dhat [b][m], D [b][m], R [b][m]).
    """
    Q, logp, entropy = _f64(Q), _f64(logp), _f64(entropy)
    b, h_q, n_q, d = Q.shape
    if n_q != w + m * t or logp.shape != (b, m, t) or entropy.shape != (b, m, t):
        raise ValueError("shape mismatch")
    D = np.zeros((b, m))
    for bb in range(b):
        for j in range(m):
            total, count = 0.0, 0
            for h in range(h_q):
                mine = Q[bb, h, w + j * t: w + (j + 1) * t]
                for jj in range(m):
                    if jj == j:
                        continue
                    other = Q[bb, h, w + jj * t: w + (jj + 1) * t]
                    for q in mine:
                        for q2 in other:
                            nq, nq2 = np.linalg.norm(q), np.linalg.norm(q2)
                            cos = 0.0 if nq == 0.0 or nq2 == 0.0 else float(q @ q2) / (nq * nq2)
                            total += 1.0 - cos
                            count += 1
            D[bb, j] = total / count if count else 0.0
    mu = D.mean(axis=1, keepdims=True)
    sd = np.sqrt(((D - mu) ** 2).mean(axis=1, keepdims=True))
    dhat = np.where(sd < STD_FLOOR, 0.0, (D - mu) / np.where(sd < STD_FLOOR, 1.0, sd))
    cbar = (logp + entropy).mean(axis=2)
    hbar = entropy.mean(axis=2)
    R = beta * cbar - gamma * hbar - lambda_d * dhat
    e = np.exp(R - R.max(axis=1, keepdims=True))
    return {"omega": e / e.sum(axis=1, keepdims=True), "dhat": dhat, "D": D, "R": R}


def pooled_scores(S, n_sink, w, chunk):
    """Chunk pooling ("adjacent-token grouping", chunk = 4 in the LORE-KV
    Hyperparameters table): each candidate gets the mean score of the
    candidates in its aligned chunk [chunk*floor(i/chunk), +chunk).
    Candidates are [n_sink, n - w); protected tokens get NaN.
    """
    S = _f64(S)
    n = S.shape[-1]
    flat = S.reshape(-1, n)
    idx = np.arange(n)
    cand = (idx >= n_sink) & (idx < n - w)
    cid = idx // chunk
    counts = np.bincount(cid[cand], minlength=cid[-1] + 1)
    P = np.full(flat.shape, np.nan)
    for row in range(flat.shape[0]):
        sums = np.bincount(cid[cand], weights=flat[row, cand], minlength=cid[-1] + 1)
        P[row, cand] = sums[cid[cand]] / counts[cid[cand]]
    return P.reshape(S.shape)


def topb_select(S, *, n_sink, w, chunk, budget):
    """Kept token indices per KV head, ascending.

    LORE-KV page, Eq. 8: each KV head keeps the protected set (the attention
    sink(s) [0, n_sink) and the window [n - w, n)) plus its top-B candidates,
    ranked by pooled score descending, ties by lower index.
    Returns (kept [..][n_keep] int64, pooled [..][n]).
    """
    S = _f64(S)
    n = S.shape[-1]
    P = pooled_scores(S, n_sink, w, chunk)
    flat = P.reshape(-1, n)
    cand = np.arange(n_sink, n - w)
    protected = np.concatenate([np.arange(n_sink), np.arange(n - w, n)])
    out = []
    for row in range(flat.shape[0]):
        order = np.lexsort((cand, -flat[row, cand]))  # last key primary: score desc, then index asc
        chosen = cand[order[:budget]]
        out.append(np.sort(np.concatenate([protected, chosen])))
    kept = np.stack(out).reshape(S.shape[:-1] + (len(out[0]),))
    return kept.astype(np.int64), P


def retention_shift(kept_a, kept_b, *, n_sink, w, n):
    """Share of the retained candidates that change between two selections.

    LORE-KV page, "More analyses", "Retention-order shift" (about 20% of the
    retained tokens change at B = 128).  Reading: for each KV head, the
    candidates [n_sink, n - w) that selection A keeps and selection B does
    not, as a fraction of A's kept candidates; the protected tokens are kept
    by both and are left out.  With equal budgets the measure is symmetric.
    kept_a, kept_b [..][n_keep] (any order); returns [..] fp64 (0 when A keeps
    no candidate).
    """
    a = np.asarray(kept_a).reshape(-1, np.asarray(kept_a).shape[-1])
    b = np.asarray(kept_b).reshape(-1, np.asarray(kept_b).shape[-1])
    out = np.empty(a.shape[0])
    for row in range(a.shape[0]):
        ca = {int(i) for i in a[row] if n_sink <= i < n - w}
        cb = {int(i) for i in b[row] if n_sink <= i < n - w}
        out[row] = len(ca - cb) / len(ca) if ca else 0.0
    return out.reshape(np.asarray(kept_a).shape[:-1])


def compact(K, V, kept):
    """Gather the kept rows: K'[..][r] = K[..][kept[r]] (decoding then runs on
    the compressed cache, LORE-KV Method).  Works on any dtype, exact copy."""
    K = np.asarray(K); V = np.asarray(V); kept = np.asarray(kept)
    idx = kept[..., None].repeat(K.shape[-1], axis=-1)
    return np.take_along_axis(K, idx, axis=-2), np.take_along_axis(V, idx, axis=-2)


# --------------------------------------------------------------------------
# H2O
# --------------------------------------------------------------------------

def h2o_prefill_acc(Qp, Kp):
    """Accumulated attention of every prompt token over the causal prompt.

    H2O page, 3.4: the accumulated score of a token is the sum of the attention
    weights it receives from the tokens after it (and itself); row r attends to
    keys 0..r with softmax(q.k / sqrt(d)).  Qp, Kp [..][P][d] -> acc [..][P].
    """
    Qp, Kp = _f64(Qp), _f64(Kp)
    P, d = Kp.shape[-2:]
    Qf = Qp.reshape(-1, P, d); Kf = Kp.reshape(-1, P, d)
    acc = np.empty((Qf.shape[0], P))
    future = np.triu(np.ones((P, P), dtype=bool), k=1)
    for row in range(Qf.shape[0]):
        s = Qf[row] @ Kf[row].T / math.sqrt(d)
        s[future] = -np.inf
        s -= s.max(axis=1, keepdims=True)
        a = np.exp(s)
        a /= a.sum(axis=1, keepdims=True)
        acc[row] = a.sum(axis=0)
    return acc.reshape(Qp.shape[:-1])


def h2o_budget(cur_len, heavy_frac, recent_frac):
    """(k_heavy, k_recent) for the current length: floor of each fraction."""
    return int(heavy_frac * cur_len), int(recent_frac * cur_len)


class H2OOracle:
    """Step-by-step H2O eviction over independent (sequence, head) rows.

    H2O page: the cache keeps the recent tokens plus the heavy hitters by
    accumulated attention (3.2); each step the new query attends over the
    retained cache and itself, its probabilities are added to the
    accumulators (o~_i = o~_{i-1} + o_i), and if the cache is over budget the
    retained non-recent token with the lowest accumulated score is evicted
    (ties: the later position goes first), at most one per step (Def. 2.1).
    The prompt is reduced to the budget by its causal column sums before the
    first decode step.

    State per row: pos [cap] (-1 = empty), acc [cap], K, V [cap][d], fp64.
    Slot order is the oracle's own and carries no meaning.
    """

    def __init__(self, Qp, Kp, Vp, heavy_frac, recent_frac, cap, kept=None):
        Qp, Kp, Vp = _f64(Qp), _f64(Kp), _f64(Vp)
        P, d = Kp.shape[-2:]
        self.rows = int(np.prod(Kp.shape[:-2]))
        self.d, self.cap = d, cap
        self.heavy_frac, self.recent_frac = heavy_frac, recent_frac
        acc = h2o_prefill_acc(Qp, Kp).reshape(self.rows, P)
        self.prefill_acc = acc.copy()
        k_h, k_r = h2o_budget(P, heavy_frac, recent_frac)
        self.own_kept_prompt, _ = topb_select(acc, n_sink=0, w=k_r, chunk=1, budget=k_h)
        # a caller running in lockstep may hand in its own prompt selection
        kept = self.own_kept_prompt if kept is None else np.asarray(kept).reshape(self.rows, -1)
        if kept.shape[1] > cap:
            raise ValueError("cap too small for the prompt budget")
        self.pos = np.full((self.rows, cap), -1, dtype=np.int64)
        self.acc = np.zeros((self.rows, cap))
        self.K = np.zeros((self.rows, cap, d)); self.V = np.zeros((self.rows, cap, d))
        Kf = Kp.reshape(self.rows, P, d); Vf = Vp.reshape(self.rows, P, d)
        nk = kept.shape[1]
        for row in range(self.rows):
            self.pos[row, :nk] = kept[row]
            self.acc[row, :nk] = acc[row, kept[row]]
            self.K[row, :nk] = Kf[row, kept[row]]
            self.V[row, :nk] = Vf[row, kept[row]]
        self.cur_len = P
        self.kept_prompt = kept
        self.evicted_mass = np.zeros(self.rows)

    def attend(self, q, k, v):
        """Append the new token and accumulate its query's attention.

        q, k, v [rows][d].  Returns (o [rows][d], probs [rows][cap]).
        """
        q, k, v = _f64(q).reshape(self.rows, self.d), _f64(k).reshape(self.rows, self.d), \
            _f64(v).reshape(self.rows, self.d)
        self.cur_len += 1
        for row in range(self.rows):
            free = np.nonzero(self.pos[row] < 0)[0]
            if free.size == 0:
                raise RuntimeError("no free slot")
            s = free[0]
            self.pos[row, s] = self.cur_len - 1
            self.acc[row, s] = 0.0
            self.K[row, s] = k[row]
            self.V[row, s] = v[row]
        valid = self.pos >= 0
        logits = np.einsum("rcd,rd->rc", self.K, q) / math.sqrt(self.d)
        logits[~valid] = -np.inf
        logits -= logits.max(axis=1, keepdims=True)
        a = np.exp(logits)
        a /= a.sum(axis=1, keepdims=True)
        self.acc += a
        o = np.einsum("rc,rcd->rd", a, self.V)
        return o, a

    def choose(self):
        """Slot each row would evict now (-1 if within budget): the lowest
        accumulated score among retained non-recent tokens, ties to the
        later position."""
        k_h, k_r = h2o_budget(self.cur_len, self.heavy_frac, self.recent_frac)
        out = np.full(self.rows, -1, dtype=np.int64)
        for row in range(self.rows):
            valid = self.pos[row] >= 0
            if valid.sum() <= k_h + k_r:
                continue
            cand = np.nonzero(valid & (self.pos[row] < self.cur_len - k_r))[0]
            order = np.lexsort((-self.pos[row, cand], self.acc[row, cand]))
            out[row] = cand[order[0]]
        return out

    def evict(self, slots):
        for row, s in enumerate(np.asarray(slots).reshape(-1)):
            if s >= 0:
                self.evicted_mass[row] += self.acc[row, s]
                self.pos[row, s] = -1
                self.acc[row, s] = 0.0

    def retained(self, row):
        """{position: accumulated score} of one row's cache."""
        sl = np.nonzero(self.pos[row] >= 0)[0]
        return {int(self.pos[row, s]): float(self.acc[row, s]) for s in sl}
