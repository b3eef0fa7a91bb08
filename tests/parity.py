"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
compare it, head by head, with the CPU oracle on the same seeded inputs.

Bars:
  * scores (every level), selected indices, sub-sequence order and slot maps:
    bit-exact;
  * gathered rows: the fp16 pair hi + lo of a query / key row equals the exact
    pooled mean to 2^-18 relative; a value row is one fp16 rounding of it;
  * attention outputs, layer outputs and gradients (row = one token's d-vector):
    every element |g - r| <= 2e-2 + 2^-7 * max|r over its row|, and
    sum|g - r| / sum|r| <= 1e-2. The row scale replaces |r| because outputs are
    rounded to bf16 (half an ulp is 2^-9 |r|, far above 2e-2 once |r| > 10) and
    because a gradient element that is small by cancellation inside a large row
    can only be as accurate as the terms that cancel.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import sparse_long_context_lh_amd as lh

ATOL, RTOL, MEAN_REL = 2e-2, 2.0 ** -7, 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(got, ref, name, atol=ATOL, rtol=RTOL, mean_rel=MEAN_REL):
    """Row-scaled bound (see the module docstring); rows are the last axis."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % name
    err = np.abs(got - ref)
    scale = np.abs(ref) if ref.ndim < 2 else np.abs(ref).max(axis=-1, keepdims=True)
    tol = atol + rtol * scale
    bad = err > tol
    denom = max(np.abs(ref).sum(), 1e-30)
    rel = err.sum() / denom
    if bad.any():
        idx = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError("%s: %d of %d out of tolerance; worst at %s got %r ref %r; max err %.3g; mean rel %.3g"
                             % (name, int(bad.sum()), err.size, idx, got[idx], ref[idx], err.max(), rel))
    assert rel <= mean_rel, "%s: mean relative error %.3g > %.3g" % (name, rel, mean_rel)
    return float(err.max()), float(rel)


class GpuRun:
    """One forward (and optionally backward) through the C ABI, with views of
    the intermediates it leaves in the workspace."""

    def __init__(self, q, k, v, L, p, kk, dout=None):
        self.H, self.N, self.d = q.shape
        self.L, self.p, self.k, self.dtype = L, p, kk, q.dtype
        self.out, self.ws = lh.forward(q, k, v, L, p, kk)
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
            return r.view(H, self.L - 1, self.k)[h].cpu()
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


def compare_forward(run: GpuRun, h: int, ref: dict, tag: str = "") -> dict:
    S = run.S
    stats = {}
    for pre, key in (("q", "qt"), ("k", "kt")):
        hi = run.head(pre + "hi", h)[:S].double().numpy()
        lo = run.head(pre + "lo", h)[:S].double().numpy()
        r = ref[key]
        # 2^-22: a few quanta of the fp16 subnormal range, where lo of a small value lands
        bad = np.abs(hi + lo - r) > 2.0 ** -18 * np.abs(r) + 2.0 ** -22
        if bad.any():
            i, c = np.argwhere(bad)[0]
            raise AssertionError("%s head %d: gathered %s rows: %d elements off, first [%d, %d] (level %d): "
                                 "exact %r hi %r lo %r" % (tag, h, pre, bad.sum(), i, c, ref["ent_level"][i],
                                                           r[i, c], hi[i, c], lo[i, c]))
        assert np.array_equal(run.head(pre + "hi_t", h)[:, :S].numpy(), run.head(pre + "hi", h)[:S].numpy().T)
    v = run.head("v", h)[:S].double().numpy()
    assert np.all(np.abs(v - ref["vt"]) <= 2.0 ** -11 * np.abs(ref["vt"]) + 2.0 ** -24), \
        "%s head %d: gathered v rows" % (tag, h)
    assert np.array_equal(run.head("v_t", h)[:, :S].numpy(), run.head("v", h)[:S].numpy().T)
    stats["osub"] = assert_close(run.head("osub", h)[:S].numpy(), ref["ot"], "%s head %d O_sub" % (tag, h))
    # the library keeps the log-sum-exp in the log2 domain
    stats["lse"] = assert_close(run.head("lse", h)[:S].numpy(), ref["lse"] / np.log(2.0), "%s head %d LSE" % (tag, h))
    stats["out"] = assert_close(run.out[h].float().cpu().numpy(), ref["out"], "%s head %d output" % (tag, h))
    return stats


def compare_backward(run: GpuRun, h: int, ref: dict, gref: dict, tag: str = "") -> dict:
    S = run.S
    stats = {}
    stats["dosub"] = assert_close(run.head("dosub", h)[:S].numpy(), gref["dot"], "%s head %d dO_sub" % (tag, h),
                                  atol=1e-4, rtol=1e-5, mean_rel=1e-6)
    for name, key in (("dqsub", "dqt"), ("dksub", "dkt"), ("dvsub", "dvt")):
        stats[name] = assert_close(run.head(name, h)[:S].numpy(), gref[key], "%s head %d %s" % (tag, h, name))
    for i, key in enumerate(("dq", "dk", "dv")):
        stats[key] = assert_close(run.grads[i][h].float().cpu().numpy(), gref[key], "%s head %d %s" % (tag, h, key))
    return stats


def check_case(q, k, v, L, p, kk, dout=None, heads=None, tag=""):
    """Whole-path parity of one case on the listed heads (default: all)."""
    run = GpuRun(q, k, v, L, p, kk, dout)
    heads = range(run.H) if heads is None else heads
    out = {}
    for h in heads:
        qh, kh, vh = head_inputs(q, h), head_inputs(k, h), head_inputs(v, h)
        ref = oracle.forward(qh, kh, vh, L, p, kk)
        compare_selection(run, h, ref)
        out[h] = compare_forward(run, h, ref, tag)
        if dout is not None:
            gref = oracle.backward(ref, head_inputs(dout, h), p)
            out[h].update(compare_backward(run, h, ref, gref, tag))
        say("  %s head %d ok: %s" % (tag, h, {k2: "%.2g/%.2g" % v2 for k2, v2 in out[h].items()}))
    return run, out
