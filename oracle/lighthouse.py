"""Lighthouse Attention layer: plain CPU oracle (numpy, fp64).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this module. The HIP library never
calls it and shares no code with it.

Sources. Two pages describe the layer:
  [AIT] aitrends.kr, "Lighthouse Attention" AI summary (sections "핵심 기여",
        "방법론", "기술 상세", "한계점");
  [TLL] techllm.github.io, "lighthouse-attention-long-context-pretraining"
        review (sections "어떻게 동작하나", "핵심 수식", "한계와 주의할 점").
Each function names the passage it follows. Where the pages leave a step open
the reading taken is stated in the function and, with its reason, in the
design notes of the repository.

Everything is per head: q, k, v and dO are [N, d] arrays. Arithmetic is fp64,
except the token score, which is fp32 in a stated order (see score_ref.c) so
that selected indices can be compared bit for bit.

Parity status. Each step is pinned by the CPU tests in ``tests/test_oracle_*``
(closed forms, invariants, brute force, a library attention routine and finite
differences). What is NOT pinned by anything outside this repository: the
paper's own numbers (the pages print no worked example), the choice of
sum-of-norms as the scalar score, the stratum size and the order of entries
that end on the same token.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

# Stratum size of the stratified top-K. [TLL, "한계와 주의할 점"] says the top-K is
# not a global top-K but a stratified one in which every segment contributes a
# fixed count; the pages give no segment size. Reading: segments of 2048
# contiguous entries of the level being ranked.
STRATUM = 2048

_HERE = os.path.dirname(os.path.abspath(__file__))
_BUILD_DIR = os.path.join(_HERE, "_build")
_SCORER_SO = os.path.join(_BUILD_DIR, "libscore_ref.so")
_scorer_lib = None


# ----------------------------------------------------------------------------
# build of the C scorer (gcc only; no HIP)
# ----------------------------------------------------------------------------
def build_scorer(force: bool = False) -> str:
    """Compile oracle/score_ref.c into oracle/_build/libscore_ref.so."""
    src = os.path.join(_HERE, "score_ref.c")
    if force or not os.path.exists(_SCORER_SO) or os.path.getmtime(_SCORER_SO) < os.path.getmtime(src):
        os.makedirs(_BUILD_DIR, exist_ok=True)
        tmp = _SCORER_SO + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
            src, "-o", tmp, "-lm"])
        os.replace(tmp, _SCORER_SO)
    return _SCORER_SO


def _scorer():
    global _scorer_lib
    if _scorer_lib is None:
        lib = ctypes.CDLL(build_scorer())
        for name in ("oracle_row_norm2",):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        fn = lib.oracle_token_scores
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        fn = lib.oracle_token_scores_v
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        _scorer_lib = lib
    return _scorer_lib


# ----------------------------------------------------------------------------
# sizes
# ----------------------------------------------------------------------------
def level_sizes(N: int, L: int, p: int) -> list[int]:
    """n_l = N / p^l entries at pyramid level l = 0..L-1 [AIT, "핵심 기여": the
    pyramid holds sum_l N/p^l entries]."""
    return [N // p ** l for l in range(L)]


def subseq_len(N: int, L: int, p: int, k: int) -> int:
    """S = N/p^(L-1) + (L-1)*p*k [TLL, "핵심 수식"]: the coarsest level kept whole
    plus p*k gathered entries from each of the other L-1 levels."""
    return N // p ** (L - 1) + (L - 1) * p * k


def strata(n: int) -> int:
    """Number of strata C at a level of n entries: one stratum if n <= STRATUM,
    else n / STRATUM (n must then be a multiple of STRATUM)."""
    return 1 if n <= STRATUM else n // STRATUM


def quotas(k: int, C: int) -> list[int]:
    """Per-stratum quota: floor(k/C), plus one for the first k mod C strata."""
    base, extra = divmod(k, C)
    return [base + (1 if c < extra else 0) for c in range(C)]


def check_shape(N: int, d: int, L: int, p: int, k: int) -> None:
    """Raise ValueError on a shape the method does not define (the same rules the
    library applies)."""
    if L < 1 or N < 1 or d < 16:
        raise ValueError("need L >= 1, N >= 1, d >= 16")
    if L > 1:
        if p < 2:
            raise ValueError("need p >= 2 when L > 1")
        if N % p ** (L - 1):
            raise ValueError("N must be a multiple of p^(L-1)")
        n = level_sizes(N, L, p)
        if k < 0 or k > n[L - 1]:
            raise ValueError("need 0 <= k <= N/p^(L-1)")
        for l in range(1, L):
            if n[l] > STRATUM and n[l] % STRATUM:
                raise ValueError("level %d has %d entries: not a multiple of the stratum" % (l, n[l]))


# ----------------------------------------------------------------------------
# forward steps
# ----------------------------------------------------------------------------
def pool_level(x: np.ndarray, p: int, l: int) -> np.ndarray:
    """Level-l pooled rows: X^(l)_i = p^-l * sum of X_j over j in [i p^l, (i+1) p^l).

    [AIT, "기술 상세" item 1; TLL, "어떻게 동작하나" step 1]: Q, K and V are
    average-pooled by the same factor p, window by window, into an L-level
    pyramid. Reading: non-overlapping windows aligned at token 0, computed
    straight from level 0.
    """
    w = p ** l
    n = x.shape[0] // w
    return x.astype(np.float64).reshape(n, w, x.shape[1]).sum(axis=1) / float(w)


def row_norm2_f32(x: np.ndarray) -> np.ndarray:
    """||x_r||^2 in fp32, in the order stated in score_ref.c."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape[0], dtype=np.float32)
    if _scorer().oracle_row_norm2(x.ctypes.data, x.shape[0], x.shape[1], out.ctypes.data):
        raise ValueError("unsupported d=%d for the scorer" % x.shape[1])
    return out


# Score variants, in the numbering the library's C ABI uses.
SCORERS = ("sum", "product", "query", "key")


def token_scores(q: np.ndarray, k: np.ndarray, scorer: str = "sum") -> np.ndarray:
    """Level-0 score, fp32, from nq = sqrt(||q_j||^2) and nk = sqrt(||k_j||^2):
    "sum" nq + nk (default), "product" nq * nk, "query" nq, "key" nk.

    [AIT, "기술 상세" item 2]: level 0 is scored by the l2 norms of Q_i and K_i;
    [TLL, "어떻게 동작하나" step 2]: the score is parameter-free; [AIT, "핵심
    기여"]: the query/key scores are l2 norms of more than one kind ("QK and KQ
    l2 norms, etc."). Reading: the default adds the two norms (the plainest
    single scalar built from both); the variants are their product and either
    norm alone.
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    s = np.empty(q.shape[0], dtype=np.float32)
    if scorer == "sum":
        rc = _scorer().oracle_token_scores(q.ctypes.data, k.ctypes.data, q.shape[0], q.shape[1], s.ctypes.data)
    else:
        rc = _scorer().oracle_token_scores_v(q.ctypes.data, k.ctypes.data, q.shape[0], q.shape[1],
                                             SCORERS.index(scorer), s.ctypes.data)
    if rc:
        raise ValueError("unsupported d=%d for the scorer" % q.shape[1])
    return s


def score_pyramid(s0: np.ndarray, L: int, p: int) -> list[np.ndarray]:
    """Scores at every level: s^(l)_i = max over its p children s^(l-1)_(p i + c).

    [AIT, "기술 상세" item 2]: coarser levels receive the score by max-pooling.
    """
    levels = [np.asarray(s0, dtype=np.float32)]
    for _ in range(1, L):
        prev = levels[-1]
        levels.append(prev.reshape(prev.shape[0] // p, p).max(axis=1))
    return levels


def stratified_topk(s: np.ndarray, k: int) -> np.ndarray:
    """Stratified top-k of one level, returned in ascending index order.

    [AIT, "핵심 기여"; TLL, "어떻게 동작하나" step 2]: the best entries are picked
    by a non-differentiable top-K; [TLL, "한계와 주의할 점"]: it is stratified,
    every segment giving a fixed count. Reading: strata of STRATUM contiguous
    entries; stratum c keeps its quota of entries with the largest score, ties
    broken by the lowest index.
    """
    n = s.shape[0]
    C = strata(n)
    size = n // C
    picked = []
    for c, q in enumerate(quotas(k, C)):
        idx = np.arange(c * size, (c + 1) * size, dtype=np.int64)
        seg = s[c * size:(c + 1) * size]
        rank = np.lexsort((idx, -seg))  # score descending, then index ascending
        picked.append(np.sort(idx[rank[:q]]))
    return np.concatenate(picked) if picked else np.zeros(0, dtype=np.int64)


def select(scores: list[np.ndarray], L: int, k: int) -> dict[int, np.ndarray]:
    """Sel_l for l = 1..L-1: k parents per level, ranked by their max-pooled score.

    Reading of what k counts: the gathered sub-sequence has (L-1)*p*k entries
    besides the top level [TLL, "핵심 수식"], so each of levels 1..L-1 selects k
    parents and their p children one level down are gathered.
    """
    return {l: stratified_topk(scores[l], k) for l in range(1, L)}


def expand(sel: dict[int, np.ndarray], N: int, L: int, p: int) -> list[np.ndarray]:
    """Gathered entries per level, ascending.

    G_(L-1) is the whole coarsest level [TLL, "핵심 수식": the top level is kept
    whole]; for l < L-1, G_l holds the p children p*j + c of every j in Sel_(l+1).
    """
    n = level_sizes(N, L, p)
    G = [None] * L
    G[L - 1] = np.arange(n[L - 1], dtype=np.int64)
    for l in range(L - 1):
        parents = np.asarray(sel[l + 1], dtype=np.int64)
        G[l] = (p * parents[:, None] + np.arange(p, dtype=np.int64)[None, :]).reshape(-1)
    return G


def entry_end(level: np.ndarray, index: np.ndarray, p: int) -> np.ndarray:
    """Last token t(l, i) = (i+1) p^l - 1 covered by entry (l, i)."""
    return (index + 1) * (np.int64(p) ** level) - 1


def causal_order(G: list[np.ndarray], p: int) -> tuple[np.ndarray, np.ndarray]:
    """Levels and indices of the gathered entries in sub-sequence order.

    [TLL, "어떻게 동작하나" step 3]: the chosen entries are sorted into causal
    order to form one contiguous sub-sequence. Reading: order by the last token
    an entry covers, and for equal last tokens the coarser entry first.
    """
    lev = np.concatenate([np.full(g.shape[0], l, dtype=np.int64) for l, g in enumerate(G)])
    idx = np.concatenate(G)
    t = entry_end(lev, idx, p)
    order = np.lexsort((-lev, t))
    return lev[order], idx[order]


def gather(x: np.ndarray, ent_level: np.ndarray, ent_index: np.ndarray, p: int) -> np.ndarray:
    """Sub-sequence rows: row a is the pooled row of entry (ent_level[a], ent_index[a])."""
    out = np.empty((ent_level.shape[0], x.shape[1]), dtype=np.float64)
    for l in np.unique(ent_level):
        rows = ent_level == l
        out[rows] = pool_level(x, p, int(l))[ent_index[rows]]
    return out


def _future(S: int) -> np.ndarray:
    """Boolean [S, S] mask of the pairs (a, b) with b > a (key after query)."""
    idx = np.arange(S)
    return idx[None, :] > idx[:, None]


def attention(qt: np.ndarray, kt: np.ndarray, vt: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Dense causal softmax attention over the sub-sequence, scale 1/sqrt(d).

    [AIT, "핵심 기여" and "기술 상세" item 3]: stock FlashAttention runs on the
    gathered S entries; its default is causal scaled-dot-product attention.
    Returns the output rows and the natural-log row log-sum-exp.
    """
    S, d = qt.shape
    logits = (qt @ kt.T) / np.sqrt(d)
    logits[_future(S)] = -np.inf
    m = logits.max(axis=1, keepdims=True)
    np.subtract(logits, m, out=logits)
    np.exp(logits, out=logits)
    l = logits.sum(axis=1, keepdims=True)
    np.divide(logits, l, out=logits)
    out = logits @ vt
    lse = (m + np.log(l)).reshape(-1)
    return out, lse


def scatter_range(level: int, index: int, p: int, N: int) -> tuple[int, int]:
    """R(l, i) as a half-open token range [lo, hi).

    [AIT, "기술 상세" item 4; TLL, "어떻게 동작하나" step 4]: each output goes back
    over a shifted range R(l, i) so that causality holds. Reading: the entry's
    span shifted right by p^l - 1, i.e. from its last token t(l, i) through
    t(l, i) + p^l - 1, clipped at N.
    """
    w = p ** level
    lo = (index + 1) * w - 1
    return lo, min(lo + w, N)


def scatter(ot: np.ndarray, ent_level: np.ndarray, ent_index: np.ndarray, p: int, N: int) -> np.ndarray:
    """O_j = sum of the sub-sequence outputs whose range R(l, i) holds j (an empty
    sum is 0) [AIT, "기술 상세" item 4: summed over R(l, i) for every position]."""
    out = np.zeros((N, ot.shape[1]), dtype=np.float64)
    for a in range(ot.shape[0]):
        lo, hi = scatter_range(int(ent_level[a]), int(ent_index[a]), p, N)
        out[lo:hi] += ot[a]
    return out


def forward(q, k, v, L: int, p: int, kk: int, sel: dict | None = None, scorer: str = "sum") -> dict:
    """Whole layer for one head, with every intermediate.

    Steps in the pages' order [AIT, "방법론" and "기술 상세"]: pyramid pool,
    score and top-K, gathered-sequence attention, scatter-back. ``sel`` holds
    the selection fixed (the top-K is non-differentiable, so a caller may pass
    the indices of an earlier call); ``scorer`` names the score variant (see
    token_scores).
    """
    N, d = q.shape
    check_shape(N, d, L, p, kk)
    s0 = token_scores(q, k, scorer)
    scores = score_pyramid(s0, L, p)
    if sel is None:
        sel = select(scores, L, kk)
    G = expand(sel, N, L, p)
    ent_level, ent_index = causal_order(G, p)
    qt = gather(q, ent_level, ent_index, p)
    kt = gather(k, ent_level, ent_index, p)
    vt = gather(v, ent_level, ent_index, p)
    ot, lse = attention(qt, kt, vt)
    out = scatter(ot, ent_level, ent_index, p, N)
    return dict(scores=scores, sel=sel, G=G, ent_level=ent_level, ent_index=ent_index,
                qt=qt, kt=kt, vt=vt, ot=ot, lse=lse, out=out)


# ----------------------------------------------------------------------------
# backward (indices held fixed)
# ----------------------------------------------------------------------------
def scatter_bwd(dout: np.ndarray, ent_level: np.ndarray, ent_index: np.ndarray, p: int) -> np.ndarray:
    """Adjoint of scatter: dOt_a = sum of dO_j over j in R(l, i)."""
    N = dout.shape[0]
    dout = dout.astype(np.float64)
    dot = np.zeros((ent_level.shape[0], dout.shape[1]), dtype=np.float64)
    for a in range(ent_level.shape[0]):
        lo, hi = scatter_range(int(ent_level[a]), int(ent_index[a]), p, N)
        dot[a] = dout[lo:hi].sum(axis=0)
    return dot


def attention_bwd(qt, kt, vt, lse, dot):
    """Textbook gradients of causal softmax attention with scale 1/sqrt(d).

    P = softmax(Q K^T / sqrt(d)) (causal); dV = P^T dO; dP = dO V^T;
    dS = P * (dP - rowsum(P * dP)); dQ = dS K / sqrt(d); dK = dS^T Q / sqrt(d).
    [AIT, "방법론" item 5]: gradients flow through the attention of the
    gathered sequence.
    """
    S, d = qt.shape
    scale = 1.0 / np.sqrt(d)
    prob = (qt @ kt.T) * scale
    np.subtract(prob, lse[:, None], out=prob)
    np.exp(prob, out=prob)
    prob[_future(S)] = 0.0
    dvt = prob.T @ dot
    dprob = dot @ vt.T
    row = (prob * dprob).sum(axis=1, keepdims=True)
    np.subtract(dprob, row, out=dprob)
    np.multiply(dprob, prob, out=dprob)  # dprob now holds dS
    del prob
    dqt = (dprob @ kt) * scale
    dkt = (dprob.T @ qt) * scale
    return dqt, dkt, dvt


def pool_bwd(dxt: np.ndarray, ent_level: np.ndarray, ent_index: np.ndarray, p: int, N: int) -> np.ndarray:
    """Adjoint of gather(pool(.)): token j receives p^-l * dXt_a from every
    gathered entry (l, i) whose window [i p^l, (i+1) p^l) holds j."""
    dx = np.zeros((N, dxt.shape[1]), dtype=np.float64)
    for a in range(ent_level.shape[0]):
        w = p ** int(ent_level[a])
        i = int(ent_index[a])
        dx[i * w:(i + 1) * w] += dxt[a] / float(w)
    return dx


def backward(fwd: dict, dout: np.ndarray, p: int) -> dict:
    """Gradients of the layer output with respect to q, k and v, indices fixed.

    [AIT, "핵심 기여" and "방법론" item 5; TLL, "어떻게 동작하나" step 2]: the top-K
    is non-differentiable with no straight-through estimator; gradients flow
    through scatter-back, the attention and the gather (and so the pooling).
    Nothing flows through the scores.
    """
    N = dout.shape[0]
    lev, idx = fwd["ent_level"], fwd["ent_index"]
    dot = scatter_bwd(dout, lev, idx, p)
    dqt, dkt, dvt = attention_bwd(fwd["qt"], fwd["kt"], fwd["vt"], fwd["lse"], dot)
    return dict(dot=dot, dqt=dqt, dkt=dkt, dvt=dvt,
                dq=pool_bwd(dqt, lev, idx, p, N),
                dk=pool_bwd(dkt, lev, idx, p, N),
                dv=pool_bwd(dvt, lev, idx, p, N))


# ----------------------------------------------------------------------------
# single output rows, for sampled checks at sizes where the whole layer is slow
# ----------------------------------------------------------------------------
def attention_rows(qt, kt, vt, rows: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The attention output and LSE of the listed sub-sequence rows only."""
    d = qt.shape[1]
    out = np.empty((rows.shape[0], d), dtype=np.float64)
    lse = np.empty(rows.shape[0], dtype=np.float64)
    for r, a in enumerate(rows):
        a = int(a)
        z = (kt[:a + 1] @ qt[a]) / np.sqrt(d)
        m = z.max()
        e = np.exp(z - m)
        lsum = e.sum()
        out[r] = (e / lsum) @ vt[:a + 1]
        lse[r] = m + np.log(lsum)
    return out, lse


def attention_bwd_query_rows(qt, kt, vt, dot, rows: np.ndarray) -> np.ndarray:
    """dQ of the listed sub-sequence rows only (the textbook gradient of
    attention_bwd, one query at a time): with the query's own softmax row P,
    dP_b = dO_a . V_b, delta = sum_b P_b dP_b, dS_b = P_b (dP_b - delta),
    dQ_a = sum_(b <= a) dS_b K_b / sqrt(d)."""
    d = qt.shape[1]
    out = np.empty((rows.shape[0], d), dtype=np.float64)
    for r, a in enumerate(rows):
        a = int(a)
        z = (kt[:a + 1] @ qt[a]) / np.sqrt(d)
        P = np.exp(z - z.max())
        P /= P.sum()
        dP = vt[:a + 1] @ dot[a]
        dS = P * (dP - np.dot(P, dP))
        out[r] = (dS @ kt[:a + 1]) / np.sqrt(d)
    return out


def attention_bwd_key_rows(qt, kt, vt, dot, keys: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """dK and dV of the listed sub-sequence rows only: dV_b = sum_(a >= b) P_ab
    dO_a and dK_b = sum_(a >= b) dS_ab Q_a / sqrt(d), with each query's softmax
    row formed on its own (every query from the smallest listed key on)."""
    S, d = qt.shape
    keys = np.asarray(keys, dtype=np.int64)
    dk = np.zeros((keys.shape[0], d), dtype=np.float64)
    dv = np.zeros((keys.shape[0], d), dtype=np.float64)
    for a in range(int(keys.min()), S):
        z = (kt[:a + 1] @ qt[a]) / np.sqrt(d)
        P = np.exp(z - z.max())
        P /= P.sum()
        dP = vt[:a + 1] @ dot[a]
        dS = P * (dP - np.dot(P, dP))
        seen = keys <= a
        dv[seen] += P[keys[seen], None] * dot[a][None, :]
        dk[seen] += dS[keys[seen], None] * qt[a][None, :] / np.sqrt(d)
    return dk, dv



# ----------------------------------------------------------------------------
# the step on either side: the Q, K, V projections and their gradients
# ----------------------------------------------------------------------------
def project(x: np.ndarray, w: np.ndarray, H: int, d: int) -> np.ndarray:
    """Projected rows [3][H][N][d] (Q, K, V) of x [N][d_model] by w [d_model][3 H d]
    (columns: Q heads, K heads, V heads, d each), in fp64.

    [AIT, "방법론" item 5]: the layer's Q, K and V come from the W_Q, W_K and
    W_V projections, through which the gradients flow back.
    """
    N = x.shape[0]
    y = x.astype(np.float64) @ w.astype(np.float64)            # [N][3 H d]
    return y.reshape(N, 3, H, d).transpose(1, 2, 0, 3).copy()  # [3][H][N][d]


def project_bwd(x: np.ndarray, w: np.ndarray, dqkv: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Gradients of project() given dLoss at its output dqkv [3][H][N][d]:
    dx = dY W^T and dW = x^T dY with dY = dqkv as [N][3 H d]."""
    _, H, N, d = dqkv.shape
    dy = dqkv.transpose(2, 0, 1, 3).reshape(N, 3 * H * d)
    return dy @ w.astype(np.float64).T, x.astype(np.float64).T @ dy


def layer_forward(x, w, H: int, d: int, L: int, p: int, kk: int, qkv: np.ndarray | None = None) -> dict:
    """Projections, then the layer head by head: out [H][N][d]. ``qkv`` uses
    given projected rows instead of computing them (e.g. rows already
    rounded to the caller's storage type)."""
    qkv = project(x, w, H, d) if qkv is None else qkv
    heads = [forward(qkv[0, h], qkv[1, h], qkv[2, h], L, p, kk) for h in range(H)]
    return dict(qkv=qkv, heads=heads, out=np.stack([f["out"] for f in heads]))


def layer_backward(fwd: dict, x, w, dout: np.ndarray, p: int) -> dict:
    """dx and dW of the layer with its projections, indices held fixed:
    the layer's backward head by head, then the projections' adjoint."""
    H = len(fwd["heads"])
    g = [backward(fwd["heads"][h], dout[h], p) for h in range(H)]
    dqkv = np.stack([np.stack([gh[n] for gh in g]) for n in ("dq", "dk", "dv")])  # [3][H][N][d]
    dx, dw = project_bwd(x, w, dqkv)
    return dict(dqkv=dqkv, dx=dx, dw=dw)
