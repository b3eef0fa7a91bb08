"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a value the
pages state, a closed form, an invariant, a brute force coded from the rule
rather than from the oracle's own steps, a library routine (torch's scaled dot
product attention in fp64) or finite differences. CPU only.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synth_inputs import make_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(N, d, seed=0, n_plant=0, dtype=torch.bfloat16):
    q, k, v = make_qkv(N, 1, d, dtype, n_plant, seed)
    return (q[0].float().numpy(), k[0].float().numpy(), v[0].float().numpy())


# ---------------------------------------------------------------- sizes
def test_subseq_len_golden():
    with open(os.path.join(GOLDEN, "subseq_lengths.json")) as f:
        cases = json.load(f)["cases"]
    rng = np.random.default_rng(0)
    for c in cases:
        N, L, p, k, S = c["N"], c["L"], c["p"], c["k"], c["S"]
        assert oracle.subseq_len(N, L, p, k) == S
        # |G| of the expansion, with any valid selection, equals S.
        n = oracle.level_sizes(N, L, p)
        sel = {l: np.sort(rng.choice(n[l], size=k, replace=False)) for l in range(1, L)}
        G = oracle.expand(sel, N, L, p)
        assert sum(g.shape[0] for g in G) == S
        assert np.array_equal(G[L - 1], np.arange(n[L - 1]))  # top level kept whole


def test_expand_children_bruteforce():
    # G_l for l < L-1 is every entry of level l whose parent floor(i/p) was
    # selected at level l+1, found by scanning all of level l; the top level
    # is gathered whole. Random selections at several shapes, so a wrong
    # child map of the right size (p*j + c permuted, j*p^2, c*p + j, ...) fails.
    rng = np.random.default_rng(31)
    for N, L, p, k in [(256, 4, 2, 7), (1024, 3, 4, 16), (4096, 2, 8, 64), (512, 5, 2, 3), (64, 2, 4, 16)]:
        n = oracle.level_sizes(N, L, p)
        sel = {l: np.sort(rng.choice(n[l], size=k, replace=False)) for l in range(1, L)}
        G = oracle.expand(sel, N, L, p)
        for l in range(L - 1):
            chosen = set(sel[l + 1].tolist())
            want = [i for i in range(n[l]) if i // p in chosen]
            assert sorted(G[l].tolist()) == want, (N, L, p, k, l)
            assert len(set(G[l].tolist())) == G[l].shape[0]      # no entry twice
        assert G[L - 1].tolist() == list(range(n[L - 1]))


@pytest.mark.parametrize("N,L,p,k", [(4096, 3, 2, 256), (8192, 4, 2, 100), (16384, 3, 4, 300),
                                     (2048 * 4 * 3, 2, 4, 1000), (512, 1, 2, 0), (1024, 3, 2, 0)])
def test_selection_counts(N, L, p, k):
    rng = np.random.default_rng(N + L)
    s0 = rng.random(N).astype(np.float32)
    scores = oracle.score_pyramid(s0, L, p)
    sel = oracle.select(scores, L, k)
    n = oracle.level_sizes(N, L, p)
    for l in range(1, L):
        s = sel[l]
        assert s.shape[0] == k                       # exactly k per selected level
        assert np.all(np.diff(s) > 0)                # ascending, distinct
        C = oracle.strata(n[l])
        size = n[l] // C
        counts = np.bincount(s // size, minlength=C)
        assert counts.tolist() == oracle.quotas(k, C)  # fixed count per stratum
    G = oracle.expand(sel, N, L, p)
    assert sum(g.shape[0] for g in G) == oracle.subseq_len(N, L, p, k)


def test_quota_split():
    assert oracle.quotas(10, 4) == [3, 3, 2, 2]
    assert oracle.quotas(1536, 16) == [96] * 16
    assert oracle.quotas(7, 1) == [7]


# ---------------------------------------------------------------- pooling
def test_pool_constant_and_ramp():
    N, d, p = 256, 16, 4
    # few significant bits, so every partial sum of the window is exact
    c = np.random.default_rng(1).integers(-64, 64, d) / 8.0
    const = np.tile(c, (N, 1))
    ramp = np.tile(np.arange(N, dtype=np.float64)[:, None], (1, d))
    for l in range(4):
        w = p ** l
        pc = oracle.pool_level(const, p, l)
        assert pc.shape == (N // w, d)
        assert np.array_equal(pc, np.tile(c, (N // w, 1)))       # mean of a constant
        pr = oracle.pool_level(ramp, p, l)[:, 0]
        mid = np.arange(N // w) * w + (w - 1) / 2.0             # window midpoint
        assert np.array_equal(pr, mid)


# ---------------------------------------------------------------- scores
def test_scorer_hand_values():
    with open(os.path.join(GOLDEN, "scorer_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        row = np.zeros((1, c["d"]), dtype=np.float32)
        for col, val in c["row"].items():
            row[0, int(col)] = val
        assert oracle.row_norm2_f32(row)[0] == np.float32(c["norm2"]), c["name"]
        if "score_with_zero_key" in c:
            s = oracle.token_scores(row, np.zeros_like(row))
            assert s[0] == np.float32(c["score_with_zero_key"])


def test_scorer_variants_hand_values():
    with open(os.path.join(GOLDEN, "scorer_cases.json")) as f:
        cases = json.load(f)["variants"]["cases"]
    for c in cases:
        q = np.zeros((1, c["d"]), dtype=np.float32)
        k = np.zeros((1, c["d"]), dtype=np.float32)
        for col, val in c["q"].items():
            q[0, int(col)] = val
        for col, val in c["k"].items():
            k[0, int(col)] = val
        for name, want in c["scores"].items():
            assert oracle.token_scores(q, k, name)[0] == np.float32(want), (c["name"], name)


def test_scorer_variants_follow_the_roots():
    # every variant combines the same two correctly rounded roots; the sum
    # variant equals the default scorer bit for bit, and the variants order
    # entries as their definitions do (query-only ignores K entirely)
    q, k, _ = _inputs(512, 128, seed=21, n_plant=8, dtype=torch.float32)
    nq = np.sqrt(oracle.row_norm2_f32(q))
    nk = np.sqrt(oracle.row_norm2_f32(k))
    assert np.array_equal(oracle.token_scores(q, k, "sum"), oracle.token_scores(q, k))
    assert np.array_equal(oracle.token_scores(q, k, "sum"), (nq + nk).astype(np.float32))
    assert np.array_equal(oracle.token_scores(q, k, "product"), (nq * nk).astype(np.float32))
    assert np.array_equal(oracle.token_scores(q, k, "query"), nq)
    assert np.array_equal(oracle.token_scores(q, k, "key"), nk)
    assert np.array_equal(oracle.token_scores(q, np.zeros_like(k), "query"), nq)
    with pytest.raises(ValueError):
        oracle.token_scores(q, k, "bogus")


def test_scorer_single_nonzero_exact():
    # one nonzero bf16 element per row: ||x||^2 = x^2 exactly, sqrt exact.
    rng = np.random.default_rng(2)
    vals = torch.tensor(rng.standard_normal(64) * 8, dtype=torch.bfloat16).float().numpy()
    q = np.zeros((64, 128), np.float32)
    k = np.zeros((64, 128), np.float32)
    q[np.arange(64), rng.integers(0, 128, 64)] = vals
    k[np.arange(64), rng.integers(0, 128, 64)] = vals[::-1]
    s = oracle.token_scores(q, k)
    assert np.array_equal(s, np.abs(vals) + np.abs(vals[::-1]))


def test_scorer_error_bound():
    # fp32 result within (d/8 + log2(d/8) + 2) * 2^-24 relative of the fp64 value.
    q, k, _ = _inputs(2048, 128, seed=3, n_plant=8, dtype=torch.float32)
    s = oracle.token_scores(q, k).astype(np.float64)
    exact = np.linalg.norm(q.astype(np.float64), axis=1) + np.linalg.norm(k.astype(np.float64), axis=1)
    bound = (128 / 8 + 4 + 2) * 2.0 ** -24
    assert np.all(np.abs(s - exact) <= bound * exact)


def test_score_pyramid_is_max():
    rng = np.random.default_rng(4)
    s0 = rng.random(64).astype(np.float32)
    sc = oracle.score_pyramid(s0, 3, 2)
    for i in range(16):
        assert sc[2][i] == max(s0[4 * i:4 * i + 4])


# ---------------------------------------------------------------- top-K
def test_topk_property_bruteforce():
    # Every kept key beats every dropped key of its stratum; key = (score, -index).
    rng = np.random.default_rng(5)
    n = 2048 * 3
    s = rng.integers(0, 50, n).astype(np.float32)  # many ties
    k = 40
    sel = oracle.stratified_topk(s, k)
    kept = set(sel.tolist())
    for c in range(3):
        lo = c * 2048
        ks = [i for i in range(lo, lo + 2048) if i in kept]
        ds = [i for i in range(lo, lo + 2048) if i not in kept]
        worst_kept = min((s[i], -i) for i in ks)
        best_dropped = max((s[i], -i) for i in ds)
        assert worst_kept > best_dropped


def test_topk_tiny_exhaustive():
    # n = 6 entries, every quota: the kept set is the subset of size q whose
    # keys are all larger than the rest, found by enumerating subsets.
    rng = np.random.default_rng(6)
    s = rng.integers(0, 3, 6).astype(np.float32)
    for q in range(7):
        best = None
        for sub in itertools.combinations(range(6), q):
            rest = [i for i in range(6) if i not in sub]
            if all((s[a], -a) > (s[b], -b) for a in sub for b in rest):
                best = sub
        assert tuple(oracle.stratified_topk(s, q).tolist()) == best


def test_topk_all_equal_takes_lowest_indices():
    s = np.ones(2048 * 4, dtype=np.float32)
    sel = oracle.stratified_topk(s, 10)
    assert sel.tolist() == [0, 1, 2, 2048, 2049, 2050, 4096, 4097, 6144, 6145]


# ---------------------------------------------------------------- order / causality
def test_order_matches_pairwise_rule():
    rng = np.random.default_rng(7)
    N, L, p, k = 256, 4, 2, 5
    n = oracle.level_sizes(N, L, p)
    sel = {l: np.sort(rng.choice(n[l], k, replace=False)) for l in range(1, L)}
    G = oracle.expand(sel, N, L, p)
    lev, idx = oracle.causal_order(G, p)
    ents = [(l, int(i)) for l in range(L) for i in G[l]]

    def key(e):  # last token covered, then coarser first
        l, i = e
        return ((i + 1) * p ** l - 1, -l)
    pos = {(int(a), int(b)): r for r, (a, b) in enumerate(zip(lev, idx))}
    for e in ents:
        assert pos[e] == sum(1 for f in ents if key(f) < key(e))


def test_causality_perturbation():
    # With the selection held fixed, O_j depends on tokens <= j only.
    N, d, L, p, k = 512, 16, 3, 2, 12
    q, kk, v = _inputs(N, d, seed=8)
    base = oracle.forward(q, kk, v, L, p, k)
    rng = np.random.default_rng(9)
    for j in (0, 37, 100, 255, 256, 400, 510):
        q2, k2, v2 = q.copy(), kk.copy(), v.copy()
        for x in (q2, k2, v2):
            x[j + 1:] += rng.standard_normal((N - j - 1, d)).astype(np.float32)
        out2 = oracle.forward(q2, k2, v2, L, p, k, sel=base["sel"])["out"]
        assert np.array_equal(out2[:j + 1], base["out"][:j + 1])


# ---------------------------------------------------------------- whole-pyramid brute force
def test_everything_selected_bruteforce():
    # L = 2 with k = n_1: every entry of both levels is gathered (S = N + N/p).
    N, d, p = 64, 16, 4
    q, k, v = _inputs(N, d, seed=10)
    res = oracle.forward(q, k, v, 2, p, N // p)
    assert res["ot"].shape[0] == N + N // p
    ents = [(l, i) for l in (0, 1) for i in range(N // p ** l)]
    rows = {l: (oracle.pool_level(q, p, l), oracle.pool_level(k, p, l), oracle.pool_level(v, p, l)) for l in (0, 1)}
    end = lambda e: ((e[1] + 1) * p ** e[0] - 1, -e[0])
    out = np.zeros((N, d))
    for e in ents:
        visible = [f for f in ents if end(f) <= end(e)]  # the rule, pair by pair
        z = np.array([rows[e[0]][0][e[1]] @ rows[f[0]][1][f[1]] for f in visible]) / np.sqrt(d)
        w = np.exp(z - z.max())
        w /= w.sum()
        o = sum(wi * rows[f[0]][2][f[1]] for wi, f in zip(w, visible))
        lo = (e[1] + 1) * p ** e[0] - 1
        out[lo:min(lo + p ** e[0], N)] += o
    assert np.allclose(res["out"], out, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- dense reduction
def test_L1_is_dense_causal_attention_fwd_bwd():
    N, d = 96, 32
    q, k, v = _inputs(N, d, seed=11)
    res = oracle.forward(q, k, v, 1, 2, 0)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None],
                                                           is_causal=True)[0, 0]
    assert np.allclose(res["out"], ref.detach().numpy(), rtol=1e-12, atol=1e-12)
    dout = np.random.default_rng(12).standard_normal((N, d))
    ref.backward(torch.tensor(dout))
    g = oracle.backward(res, dout, 2)
    for name, t in (("dq", tq), ("dk", tk), ("dv", tv)):
        assert np.allclose(g[name], t.grad.numpy(), rtol=1e-10, atol=1e-12), name


# ---------------------------------------------------------------- scatter
def test_scatter_adjoint_and_coverage():
    rng = np.random.default_rng(13)
    N, L, p, k = 256, 4, 2, 6
    n = oracle.level_sizes(N, L, p)
    sel = {l: np.sort(rng.choice(n[l], k, replace=False)) for l in range(1, L)}
    lev, idx = oracle.causal_order(oracle.expand(sel, N, L, p), p)
    S = lev.shape[0]
    x = rng.standard_normal((S, 3))
    y = rng.standard_normal((N, 3))
    lhs = np.sum(oracle.scatter(x, lev, idx, p, N) * y)
    rhs = np.sum(x * oracle.scatter_bwd(y, lev, idx, p))
    assert np.isclose(lhs, rhs, rtol=1e-12)
    # With every output row equal to 1, O_j counts the levels whose entry
    # i = floor((j+1)/p^l) - 1 exists and was gathered.
    ones = oracle.scatter(np.ones((S, 1)), lev, idx, p, N)[:, 0]
    G = oracle.expand(sel, N, L, p)
    for j in range(N):
        cnt = 0
        for l in range(L):
            i = (j + 1) // p ** l - 1
            cnt += int(i >= 0 and i in set(G[l].tolist()))
        assert ones[j] == cnt


def test_pool_bwd_adjoint():
    rng = np.random.default_rng(14)
    N, L, p, k, d = 128, 3, 4, 3, 4
    n = oracle.level_sizes(N, L, p)
    sel = {l: np.sort(rng.choice(n[l], k, replace=False)) for l in range(1, L)}
    lev, idx = oracle.causal_order(oracle.expand(sel, N, L, p), p)
    x = rng.standard_normal((N, d))
    y = rng.standard_normal((lev.shape[0], d))
    lhs = np.sum(oracle.gather(x, lev, idx, p) * y)
    rhs = np.sum(x * oracle.pool_bwd(y, lev, idx, p, N))
    assert np.isclose(lhs, rhs, rtol=1e-12)


# ---------------------------------------------------------------- backward
def test_backward_finite_differences():
    N, d, L, p, k = 32, 16, 3, 2, 2
    q, kk, v = (x.astype(np.float64) for x in _inputs(N, d, seed=15))
    base = oracle.forward(q, kk, v, L, p, k)
    sel = base["sel"]
    dout = np.random.default_rng(16).standard_normal((N, d))
    g = oracle.backward(base, dout, p)
    loss = lambda a, b, c: float(np.sum(oracle.forward(a, b, c, L, p, k, sel=sel)["out"] * dout))
    rng = np.random.default_rng(17)
    h = 1e-6
    for which, grad in ((0, g["dq"]), (1, g["dk"]), (2, g["dv"])):
        for _ in range(12):
            r, c = int(rng.integers(N)), int(rng.integers(d))
            args_p = [q.copy(), kk.copy(), v.copy()]
            args_m = [q.copy(), kk.copy(), v.copy()]
            args_p[which][r, c] += h
            args_m[which][r, c] -= h
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[r, c]) <= 1e-6 * max(1.0, abs(fd)), (which, r, c, fd, grad[r, c])


def test_attention_rows_match_full():
    q, k, v = (x.astype(np.float64) for x in _inputs(200, 16, seed=18))
    o, lse = oracle.attention(q, k, v)
    rows = np.array([0, 1, 57, 199])
    o2, lse2 = oracle.attention_rows(q, k, v, rows)
    assert np.allclose(o[rows], o2, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse[rows], lse2, rtol=1e-12)


def test_backward_rows_match_full():
    # the per-row gradients used at sizes where the whole backward is slow
    # equal the whole-matrix backward (itself pinned to torch's fp64 autograd)
    q, k, v = (x.astype(np.float64) for x in _inputs(200, 16, seed=19))
    dout = np.random.default_rng(20).standard_normal((200, 16))
    o, lse = oracle.attention(q, k, v)
    dq, dk, dv = oracle.attention_bwd(q, k, v, lse, dout)
    rows = np.array([0, 1, 57, 150, 199])
    assert np.allclose(oracle.attention_bwd_query_rows(q, k, v, dout, rows), dq[rows], rtol=1e-10, atol=1e-12)
    keys = np.array([120, 121, 180, 199])
    dk2, dv2 = oracle.attention_bwd_key_rows(q, k, v, dout, keys)
    assert np.allclose(dk2, dk[keys], rtol=1e-10, atol=1e-12)
    assert np.allclose(dv2, dv[keys], rtol=1e-10, atol=1e-12)


def test_projection_adjoint_against_autograd():
    # project() and project_bwd() against torch's fp64 autograd of x @ w
    rng = np.random.default_rng(22)
    N, dm, H, d = 40, 24, 2, 8
    x = rng.standard_normal((N, dm))
    w = rng.standard_normal((dm, 3 * H * d))
    tx = torch.tensor(x, requires_grad=True)
    tw = torch.tensor(w, requires_grad=True)
    y = tx @ tw
    qkv = oracle.project(x, w, H, d)
    for t in range(3):
        for h in range(H):
            assert np.allclose(qkv[t, h], y[:, (t * H + h) * d:(t * H + h + 1) * d].detach().numpy(), rtol=1e-13)
    dqkv = rng.standard_normal((3, H, N, d))
    dy = torch.tensor(np.concatenate([dqkv[t, h] for t in range(3) for h in range(H)], axis=1))
    y.backward(dy)
    dx, dw = oracle.project_bwd(x, w, dqkv)
    assert np.allclose(dx, tx.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dw, tw.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_layer_with_projections_finite_differences():
    # the whole step (projections, layer) with the selection held fixed:
    # central differences of sum(out * dout) in x and in W
    rng = np.random.default_rng(23)
    N, dm, H, d, L, p, k = 32, 16, 2, 16, 3, 2, 2
    x = rng.standard_normal((N, dm))
    w = rng.standard_normal((dm, 3 * H * d)) / 4.0
    base = oracle.layer_forward(x, w, H, d, L, p, k)
    sels = [f["sel"] for f in base["heads"]]
    dout = rng.standard_normal((H, N, d))
    g = oracle.layer_backward(base, x, w, dout, p)

    def loss(xx, ww):
        qkv = oracle.project(xx, ww, H, d)
        out = np.stack([oracle.forward(qkv[0, h], qkv[1, h], qkv[2, h], L, p, k, sel=sels[h])["out"]
                        for h in range(H)])
        return float(np.sum(out * dout))
    eps = 1e-6
    for _ in range(8):
        r, c = int(rng.integers(N)), int(rng.integers(dm))
        xp, xm = x.copy(), x.copy()
        xp[r, c] += eps
        xm[r, c] -= eps
        fd = (loss(xp, w) - loss(xm, w)) / (2 * eps)
        assert abs(fd - g["dx"][r, c]) <= 1e-6 * max(1.0, abs(fd))
        r, c = int(rng.integers(dm)), int(rng.integers(3 * H * d))
        wp, wm = w.copy(), w.copy()
        wp[r, c] += eps
        wm[r, c] -= eps
        fd = (loss(x, wp) - loss(x, wm)) / (2 * eps)
        assert abs(fd - g["dw"][r, c]) <= 1e-6 * max(1.0, abs(fd))


def test_shape_rules():
    with pytest.raises(ValueError):
        oracle.check_shape(102, 64, 3, 2, 4)       # N not a multiple of p^(L-1)
    with pytest.raises(ValueError):
        oracle.check_shape(4096, 64, 3, 2, 1025)   # k above the top level
    with pytest.raises(ValueError):
        oracle.check_shape(2 * 7168, 64, 2, 2, 4)  # n_1 = 7168 > 2048, not a multiple
    oracle.check_shape(4096, 64, 3, 2, 1024)
