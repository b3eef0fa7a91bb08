"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it, head by head, with the CPU oracle on the same seeded inputs.

Bars:
  * scores (every level), selected indices, sub-sequence order and slot maps:
    bit-exact;
  * gathered rows: the fp16 pair hi + lo of a query / key row equals the exact
    pooled mean to 2^-18 relative; a value row is one fp16 rounding of it;
  * attention output, log-sum-exp, layer output, dO_sub, dV_sub and dv,
    element by element:
        |g - r| <= 2e-2 + 2^-7 |r|,
    and over the whole tensor sum|g - r| / sum|r| <= 1e-2. The stated bound is
    max-abs 2e-2 and mean-relative 1e-2 in bf16; the relative term 2^-7 |r|
    is one bf16 ulp of the reference (bf16 has 8 significant bits, so the
    output rounding alone is up to 2^-9 |r|, above 2e-2 once |r| > 10);
  * dQ_sub, dK_sub, dq and dk (the products of dS = P (dP - delta)), element
    by element against the largest |r| of the element's token row:
        |g - r| <= 2e-2 + 2^-7 max_row |r|,
    and the same mean-relative bound. An element of these four that is small
    by cancellation (a sum of terms dS_ij K_j or dS_ij Q_i far larger than
    itself) carries the rounding of those terms: the fp16 operands of the
    gradient products, and dS itself, which is the difference of two large
    numbers when |dO_sub| is large. The element-wise count of each such
    tensor against the strict bound is reported beside it.
Every comparison also reports the literal max-abs error and, for tensors the
library stores in bf16, the max-abs error left after the output's own rounding
(|g - r| minus half a bf16 ulp of r).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_long_context_lh_amd as lh

ATOL, RTOL, MEAN_REL = 2e-2, 2.0 ** -7, 1e-2
# the gradients formed from dS (see the module docstring)
ROW_SCALED = ("dqsub", "dksub", "dq", "dk")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_half_ulp(r: np.ndarray) -> np.ndarray:
    """Half a unit in the last place of |r| in bf16 (8 significant bits)."""
    a = np.abs(r)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.where(a > 0, np.exp2(e - 8.0), 2.0 ** -134)


def error_stats(got, ref, stored_bf16=False) -> dict:
    """Literal max-abs error, mean relative error, and (bf16 storage) the
    max-abs error beyond the rounding of the reference to bf16."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    st = {"max_abs": float(err.max()) if err.size else 0.0,
          "mean_rel": float(err.sum() / max(np.abs(ref).sum(), 1e-30))}
    if stored_bf16 and err.size:
        st["max_abs_beyond_rounding"] = float(np.maximum(err - bf16_half_ulp(ref), 0.0).max())
    return st


def assert_close(got, ref, name, atol=ATOL, rtol=RTOL, mean_rel=MEAN_REL, stored_bf16=False, row_scaled=False):
    """Element-wise |g - r| <= atol + rtol |r| (row_scaled: rtol times the
    largest |r| of the element's row, the last axis) and mean-relative <=
    mean_rel. Returns the error statistics (see error_stats); a row-scaled
    comparison also counts the elements over the strict element-wise bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % name
    st = error_stats(got, ref, stored_bf16)
    err = np.abs(got - ref)
    tol = atol + rtol * np.abs(ref)
    if row_scaled and ref.ndim >= 2:
        st["over_elementwise"] = int((err > tol).sum())
        tol = atol + rtol * np.abs(ref).max(axis=-1, keepdims=True)
    bad = err > tol
    if bad.any():
        idx = np.unravel_index(np.argmax(err / tol), err.shape)
        row = np.abs(ref[idx[:-1]]).max() if ref.ndim >= 2 else abs(ref[idx])
        raise AssertionError("%s: %d of %d out of tolerance; worst at %s got %r ref %r (row max |r| %.4g); "
                             "stats %s" % (name, int(bad.sum()), err.size, idx, got[idx], ref[idx], row, st))
    assert st["mean_rel"] <= mean_rel, "%s: mean relative error %.3g > %.3g" % (name, st["mean_rel"], mean_rel)
    return st


def fmt_stats(st: dict) -> str:
    s = "max %.3g rel %.2g" % (st["max_abs"], st["mean_rel"])
    if "max_abs_beyond_rounding" in st:
        s += " beyond-rounding %.3g" % st["max_abs_beyond_rounding"]
    if "over_elementwise" in st:
        s += " (row-scaled; %d over the element-wise bound)" % st["over_elementwise"]
    return s


class GpuRun:
    """One forward (and optionally backward) through the C ABI, with views of
    the intermediates it leaves in the workspace."""

    def __init__(self, q, k, v, L, p, kk, dout=None, scorer="sum", nograd=False):
        self.H, self.N, self.d = q.shape
        self.L, self.p, self.k, self.dtype = L, p, kk, q.dtype
        if nograd:  # lh_forward_nograd: the forward no backward follows
            assert dout is None and scorer == "sum"
            self.out, self.ws = lh.forward_nograd(q, k, v, L, p, kk)
        else:
            self.out, self.ws = lh.forward(q, k, v, L, p, kk, scorer=scorer)
        self.grads = None
        if dout is not None:
            self.grads = lh.backward(dout, L, p, kk, self.ws)
        torch.cuda.synchronize()
        self.S = lh.subseq_len(self.N, L, p, kk)
        self.S_pad = lh.padded_subseq_len(self.N, L, p, kk)

    def region(self, name):
        return lh.region(self.ws, name, self.N, self.H, self.d, self.L, self.p, self.k, self.dtype)

    def head(self, name, h):
        """Region `name` of head h, as a CPU tensor in its natural shape."""
        r = self.region(name)
        S, Sp, d, H = self.S, self.S_pad, self.d, self.H
        if name in ("scores", "slot"):
            return r.view(H, -1)[h].cpu()
        if name == "sel":
            return r.view(self.L - 1, H, self.k)[:, h].cpu()
        if name in ("ent", "lse"):
            return r.view(H, Sp)[h].cpu()
        if name.endswith("_t"):
            return r.view(H, d, Sp)[h].cpu()
        return r.view(H, Sp, d)[h].cpu()


def head_inputs(x, h):
    return x[h].float().cpu().numpy()


def compare_selection(run: GpuRun, h: int, ref: dict) -> None:
    """Scores at every level, selection, order and slot maps: bit-exact."""
    L, p = run.L, run.p
    n = oracle.level_sizes(run.N, L, p)
    if L > 1:
        sc = run.head("scores", h).numpy()
        off = 0
        for l in range(L):
            g = sc[off:off + n[l]]
            r = ref["scores"][l]
            if not np.array_equal(g.view(np.uint32), r.view(np.uint32)):
                bad = np.nonzero(g.view(np.uint32) != r.view(np.uint32))[0]
                raise AssertionError("head %d level %d scores differ at %d entries, first %d: %r vs %r"
                                     % (h, l, bad.size, bad[0], g[bad[0]], r[bad[0]]))
            off += n[l]
        sel = run.head("sel", h).numpy()
        for l in range(1, L):
            assert np.array_equal(sel[l - 1], ref["sel"][l]), "head %d: selection of level %d differs" % (h, l)
    ent = run.head("ent", h).numpy()
    S = run.S
    assert np.array_equal(ent[:S] & 7, ref["ent_level"]), "head %d: order (levels) differs" % h
    assert np.array_equal(ent[:S] >> 3, ref["ent_index"]), "head %d: order (indices) differs" % h
    assert np.all(ent[S:] == -1)
    slot = run.head("slot", h).numpy()
    off = 0
    for l in range(L):
        want = np.full(n[l], -1, dtype=np.int64)
        rows = np.nonzero(ref["ent_level"] == l)[0]
        want[ref["ent_index"][rows]] = rows
        assert np.array_equal(slot[off:off + n[l]], want), "head %d: slot map of level %d differs" % (h, l)
        off += n[l]


class Failures:
    """Runs every comparison of a case and raises once at the end with all of
    the failures, so a report names every tensor out of tolerance."""

    def __init__(self):
        self.msgs = []

    def check(self, stats, key, *args, **kw):
        try:
            stats[key] = assert_close(*args, **kw)
        except AssertionError as e:
            self.msgs.append(str(e))
            say("  FAIL " + str(e))

    def raise_if_any(self):
        if self.msgs:
            raise AssertionError("%d comparison(s) failed:\n" % len(self.msgs) + "\n".join(self.msgs))


def compare_forward(run: GpuRun, h: int, ref: dict, tag: str = "", fails: Failures | None = None,
                    scale: dict | None = None) -> dict:
    """``scale`` (per tensor name) multiplies the absolute term of the bound:
    for inputs that are a unit-scale problem times known powers of two, whose
    outputs are then that problem's outputs times known powers of two."""
    S = run.S
    scale = scale or {}
    own = fails is None
    fails = Failures() if own else fails
    stats = {}
    # the gathered rows are staged times per-head powers of two (Q, K, V)
    ex = run.region("exp").view(4, run.H)[:, h].cpu().numpy()
    pair = run.dtype == torch.float32  # bf16 inputs: the lo parts stay in the library's e4m3 tiles
    for t, (pre, key) in enumerate((("q", "qt"), ("k", "kt"))):
        hi = run.head(pre + "hi", h)[:S].double().numpy()
        lo = run.head(pre + "lo", h)[:S].double().numpy() if pair else 0.0
        r = ref[key] * 2.0 ** int(ex[t])
        # the pair: 2^-18 relative (its 22 bits); hi alone: 2^-11 (fp16's
        # rounding) and a little more for the fp32 rounding of a pooled mean
        # before it; 2^-22 (before the staging scale): the fp32 rounding of a
        # pooled sum whose terms cancel, and the fp16 subnormal quanta where
        # the lo part of a small value lands
        rel = 2.0 ** -18 if pair else 2.0 ** -11 * (1.0 + 2.0 ** -10)
        bad = np.abs(hi + lo - r) > rel * np.abs(r) + 2.0 ** (int(ex[t]) - 22)
        if bad.any():
            i, c = np.argwhere(bad)[0]
            raise AssertionError("%s head %d: gathered %s rows (staged times 2^%d): %d elements off, first [%d, %d] "
                                 "(level %d): exact %r hi %r lo %r" % (tag, h, pre, int(ex[t]), bad.sum(), i, c,
                                                                       ref["ent_level"][i], r[i, c], hi[i, c],
                                                                       lo[i, c]))
        if pre == "k":  # the transposes of K hi and V (no kernel needs Q hi's)
            assert np.array_equal(run.head(pre + "hi_t", h)[:, :S].numpy(), run.head(pre + "hi", h)[:S].numpy().T)
    v = run.head("v", h)[:S].double().numpy()
    vr = ref["vt"] * 2.0 ** int(ex[2])
    assert np.all(np.abs(v - vr) <= 2.0 ** -11 * np.abs(vr) + 2.0 ** -24), "%s head %d: gathered v rows" % (tag, h)
    assert np.array_equal(run.head("v_t", h)[:, :S].numpy(), run.head("v", h)[:S].numpy().T)
    bf = run.dtype == torch.bfloat16
    fails.check(stats, "osub", run.head("osub", h)[:S].numpy(), ref["ot"], "%s head %d O_sub" % (tag, h),
                atol=ATOL * scale.get("out", 1.0))
    # the library keeps the log-sum-exp in the log2 domain
    fails.check(stats, "lse", run.head("lse", h)[:S].numpy(), ref["lse"] / np.log(2.0), "%s head %d LSE" % (tag, h))
    fails.check(stats, "out", run.out[h].float().cpu().numpy(), ref["out"], "%s head %d output" % (tag, h),
                stored_bf16=bf, atol=ATOL * scale.get("out", 1.0))
    if own:
        fails.raise_if_any()
    return stats


def compare_backward(run: GpuRun, h: int, ref: dict, gref: dict, tag: str = "",
                     fails: Failures | None = None, scale: dict | None = None) -> dict:
    S = run.S
    scale = scale or {}
    own = fails is None
    fails = Failures() if own else fails
    stats = {}
    bf = run.dtype == torch.bfloat16
    fails.check(stats, "dosub", run.head("dosub", h)[:S].numpy(), gref["dot"], "%s head %d dO_sub" % (tag, h),
                atol=1e-4 * scale.get("dout", 1.0), rtol=1e-5, mean_rel=1e-6)
    for name, key in (("dqsub", "dqt"), ("dksub", "dkt"), ("dvsub", "dvt")):
        fails.check(stats, name, run.head(name, h)[:S].numpy(), gref[key], "%s head %d %s" % (tag, h, name),
                    row_scaled=name in ROW_SCALED, atol=ATOL * scale.get(name[:2], 1.0))
    for i, key in enumerate(("dq", "dk", "dv")):
        fails.check(stats, key, run.grads[i][h].float().cpu().numpy(), gref[key], "%s head %d %s" % (tag, h, key),
                    stored_bf16=bf, row_scaled=key in ROW_SCALED, atol=ATOL * scale.get(key, 1.0))
    if own:
        fails.raise_if_any()
    return stats


def check_case(q, k, v, L, p, kk, dout=None, heads=None, tag="", scorer="sum", scales=None, nograd=False):
    """Whole-path parity of one case on the listed heads (default: all);
    ``scales(h)`` gives head h's absolute-term factors (see compare_forward)."""
    run = GpuRun(q, k, v, L, p, kk, dout, scorer=scorer, nograd=nograd)
    heads = range(run.H) if heads is None else heads
    out = {}
    fails = Failures()
    for h in heads:
        qh, kh, vh = head_inputs(q, h), head_inputs(k, h), head_inputs(v, h)
        ref = oracle.forward(qh, kh, vh, L, p, kk, scorer=scorer)
        compare_selection(run, h, ref)
        sc = scales(h) if scales is not None else None
        out[h] = compare_forward(run, h, ref, tag, fails, scale=sc)
        if dout is not None:
            gref = oracle.backward(ref, head_inputs(dout, h), p)
            out[h].update(compare_backward(run, h, ref, gref, tag, fails, scale=sc))
        say("  %s head %d: %s" % (tag, h, "; ".join("%s %s" % (k2, fmt_stats(v2)) for k2, v2 in out[h].items())))
    fails.raise_if_any()
    return run, out


def selection_ref(q, k, h, L, p, kk):
    """The oracle's scores, selection and causal order of head h."""
    qh, kh = head_inputs(q, h), head_inputs(k, h)
    sc = oracle.score_pyramid(oracle.token_scores(qh, kh), L, p)
    sel = oracle.select(sc, L, kk)
    lev, idx = oracle.causal_order(oracle.expand(sel, q.shape[1], L, p), p)
    return dict(scores=sc, sel=sel, ent_level=lev, ent_index=idx)


def check_sampled_tokens(run: GpuRun, q, k, v, dout, h: int, tokens, last: int, tag: str = "") -> dict:
    """Full-size check of one head on sampled tokens, where the whole oracle
    would be slow: the oracle builds the selection, causal order and gathered
    rows of the head, then only the sub-sequence rows the sampled tokens need.
    Layer output and dq of `tokens`; dk and dv of the `last` final tokens
    (their entries end at the sequence's end, so the key rows of the oracle's
    backward need only the last few queries)."""
    N, L, p = run.N, run.L, run.p
    ref = selection_ref(q, k, h, L, p, run.k)
    lev, idx = ref["ent_level"], ref["ent_index"]
    S = lev.shape[0]
    pos = [np.full(N // p ** l, -1, dtype=np.int64) for l in range(L)]
    for l in range(L):
        rows = np.nonzero(lev == l)[0]
        pos[l][idx[rows]] = rows
    xs = [head_inputs(x, h).astype(np.float64) for x in (q, k, v)]
    qt, kt, vt = (oracle.gather(x, lev, idx, p) for x in xs)
    tokens = np.asarray(sorted(set(int(t) for t in tokens)), dtype=np.int64)
    # layer output: O_j = sum over l of O_sub of entry (l, (j+1)/p^l - 1) when gathered
    cover_o = [[pos[l][(j + 1) // p ** l - 1] for l in range(L) if (j + 1) // p ** l - 1 >= 0] for j in tokens]
    need = np.unique(np.array([a for c in cover_o for a in c if a >= 0], dtype=np.int64))
    o_rows, _ = oracle.attention_rows(qt, kt, vt, need)
    o_of = {int(a): o_rows[r] for r, a in enumerate(need)}
    out_ref = np.array([sum((o_of[int(a)] for a in c if a >= 0), np.zeros(run.d)) for c in cover_o])
    # gradients: dX_j = sum over l of p^-l dX_sub of entry (l, j / p^l) when gathered
    dot = oracle.scatter_bwd(head_inputs(dout, h).astype(np.float64), lev, idx, p)

    def pulled(rows_of, toks):
        out = np.zeros((len(toks), run.d))
        for r, j in enumerate(toks):
            for l in range(L):
                a = int(pos[l][j // p ** l])
                if a >= 0:
                    out[r] += rows_of[a] / float(p ** l)
        return out
    cover_g = np.unique(np.array([pos[l][j // p ** l] for j in tokens for l in range(L)], dtype=np.int64))
    cover_g = cover_g[cover_g >= 0]
    dq_rows = oracle.attention_bwd_query_rows(qt, kt, vt, dot, cover_g)
    dq_ref = pulled({int(a): dq_rows[r] for r, a in enumerate(cover_g)}, tokens)
    late = np.arange(N - last, N)
    cover_l = np.unique(np.array([pos[l][j // p ** l] for j in late for l in range(L)], dtype=np.int64))
    cover_l = cover_l[cover_l >= 0]
    dk_rows, dv_rows = oracle.attention_bwd_key_rows(qt, kt, vt, dot, cover_l)
    dk_ref = pulled({int(a): dk_rows[r] for r, a in enumerate(cover_l)}, late)
    dv_ref = pulled({int(a): dv_rows[r] for r, a in enumerate(cover_l)}, late)
    bf = run.dtype == torch.bfloat16
    out = run.out[h].float().cpu().numpy()
    dq, dk, dv = (g[h].float().cpu().numpy() for g in run.grads)
    fails = Failures()
    st = {}
    fails.check(st, "out", out[tokens], out_ref, "%s head %d out" % (tag, h), stored_bf16=bf)
    fails.check(st, "dq", dq[tokens], dq_ref, "%s head %d dq" % (tag, h), stored_bf16=bf, row_scaled=True)
    fails.check(st, "dk", dk[late], dk_ref, "%s head %d dk" % (tag, h), stored_bf16=bf, row_scaled=True)
    fails.check(st, "dv", dv[late], dv_ref, "%s head %d dv" % (tag, h), stored_bf16=bf)
    say("  %s head %d (%d tokens, last %d; S = %d): %s" % (tag, h, len(tokens), last, S,
                                                         "; ".join("%s %s" % (n, fmt_stats(x)) for n, x in st.items())))
    fails.raise_if_any()
    return st
