"""Precision study of the attention kernels' operand roundings.

Test infrastructure (CPU only, not collected by pytest: run it by name). The
attention kernels form their products from fp16 and e4m3 operands and add them
in fp32. This script repeats those roundings in numpy on the gathered
sub-sequence of one head of a workload, for a sample of query rows, and
compares O_sub and dQ_sub with the oracle's exact (fp64) values, for the
scheme the kernels use and for variants that drop one correction term:

  shipped    logits from the query's fp16 pair (its lo part as a block-scaled
             e4m3 copy) against the fp16 key row; P.V with an fp16 pair of
             P * 2^15; dP from dO_sub's fp16 pair (its lo part as an e4m3
             copy, against an e4m3 copy of V); dS and the key row of dQ in fp16
  no-P-lo    P.V with P * 2^15 rounded once to fp16 (O_sub, and with it
             delta = rowsum(dO_sub * O_sub), no longer carry the P the
             backward recomputes)
  rounded-l  as no-P-lo, but the normaliser sums the fp16 values themselves,
             so the weights that form O_sub sum to one and delta stays
             consistent with them
  no-dO-lo   dP from dO_sub rounded once to fp16
  no-Q-lo    logits from the query row rounded once to fp16 (forward and
             backward, which share the logits)

Staging follows the kernels: per-head powers of two bring the largest |q| and
|k| element into [2^11, 2^12), the largest V row norm into [2^4, 2^5) and the
largest dO_sub row norm into [2^8, 2^9); each e4m3 copy holds x * 2^-e with
one fixed e per tensor (FP8_EXP), which takes the bound the staging puts on
that tensor to 256, inside e4m3's largest value 448; conversions round to
nearest even. Left out: the fp32 summation order
(products are added in fp64 here) and the bf16 rounding of the layer's outputs.

--shared-v A replaces every value row by A c + v / 8, c one fixed N(0, 1)
row (shared by all tokens): the attended values then nearly agree, so dP -
delta, dS and dQ are small by cancellation while |delta| is not, and the
element-wise bound is mostly its absolute term. --v-scale F multiplies the
value rows by F (a power of two: exact); the errors of P's rounding grow with
them, the bound's absolute term does not.

Rows: the R rows with the largest |dO_sub| (the entries whose dS = P (dP -
delta) cancels most) and R rows drawn at random. Per variant the script prints
the largest error over those rows as a fraction of the parity tests' bounds,
    O_sub:  |g - r| <= 2e-2 + 2^-7 |r|
    dQ_sub: |g - r| <= 2e-2 + 2^-7 max_row |r|
(a fraction above 1 fails the bound), and the number of elements above it.

    python tests/precision_study.py [--workload lh-fwdbwd-1m] [--head 0] [--rows 256] [--shared-v A] [--v-scale F]
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
from parity import ATOL, RTOL  # noqa: E402
from synth_inputs import by_name, make_dout, make_qkv  # noqa: E402

VARIANTS = {
    "shipped": dict(q_lo=True, p_lo=True, do_lo=True),
    "no-P-lo": dict(q_lo=True, p_lo=False, do_lo=True),
    "rounded-l": dict(q_lo=True, p_lo=False, do_lo=True, l_rounded=True),
    "no-dO-lo": dict(q_lo=True, p_lo=True, do_lo=False),
    "no-Q-lo": dict(q_lo=False, p_lo=True, do_lo=True),
}


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def f16(x):
    """Round (fp32 values) to fp16, nearest even."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)


def e4m3(x):
    """Round to OCP e4m3 (3 stored mantissa bits, exponents -6..8, subnormal
    spacing 2^-9), nearest even; the inputs here stay within +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    q = np.exp2(e - 3.0)
    return np.sign(x) * np.minimum(np.round(a / q) * q, 448.0)  # np.round: half to even


def stage_exp(m: float, target: int) -> int:
    """Power of two that brings m into [2^(target-1), 2^target)."""
    return (target - 1) - int(np.floor(np.log2(m)))


# Fixed scale exponents of the e4m3 copies. After staging, a query element is
# below 2^12, so the lo part of its fp16 pair is at most half an fp16 ulp
# there, 2^0; key elements are below 2^12; value elements below 2^5 (their row
# norm is); dO_sub elements below 2^9, so its lo part is at most 2^-3. Each e
# takes that bound to 2^8.
FP8_EXP = {"q_lo": 0 - 8, "k": 12 - 8, "v": 5 - 8, "do_lo": -3 - 8}


def head_inputs(w, h: int, shared_v: float = 0.0, v_scale: float = 1.0):
    q, k, v = make_qkv(w.N, w.H, w.d, w.dtype, w.n_plant, seed=0)
    dout = make_dout(w.N, w.H, w.d, w.dtype, seed=1)
    if shared_v:
        import torch
        c = torch.randn(w.d, generator=torch.Generator().manual_seed(7))
        v = (shared_v * c[None, None, :] + v.float() / 8).to(w.dtype)
    f = lambda t: t[h].float().numpy().astype(np.float64)  # noqa: E731
    return f(q), f(k), f(v) * v_scale, f(dout)


def subsequence(q, k, v, dout, w):
    """The oracle's steps up to the gathered rows and dO_sub (no attention)."""
    scores = oracle.score_pyramid(oracle.token_scores(q, k), w.L, w.p)
    sel = oracle.select(scores, w.L, w.k)
    G = oracle.expand(sel, w.N, w.L, w.p)
    lev, idx = oracle.causal_order(G, w.p)
    qt, kt, vt = (oracle.gather(x, lev, idx, w.p) for x in (q, k, v))
    dot = oracle.scatter_bwd(dout, lev, idx, w.p)
    return qt, kt, vt, dot


class Emulation:
    """The kernels' staged operands of one head's sub-sequence."""

    def __init__(self, q, k, v, qt, kt, vt, dot):
        d = qt.shape[1]
        self.d = d
        self.exq = stage_exp(np.abs(q).max(), 12)
        self.exk = stage_exp(np.abs(k).max(), 12)
        self.exv = stage_exp(np.linalg.norm(v, axis=1).max(), 5)
        self.exd = stage_exp(np.linalg.norm(dot, axis=1).max(), 9)
        qs = f32(qt * 2.0 ** self.exq)
        self.q_hi = f16(qs)
        q_lo = f16(qs - self.q_hi)
        self.sq = FP8_EXP["q_lo"]
        self.q_lo8 = e4m3(q_lo / 2.0 ** self.sq)
        self.k16 = f16(f32(kt * 2.0 ** self.exk))
        self.sk = FP8_EXP["k"]
        self.k8 = e4m3(self.k16 / 2.0 ** self.sk)
        self.v16 = f16(f32(vt * 2.0 ** self.exv))
        self.sv = FP8_EXP["v"]
        self.v8 = e4m3(self.v16 / 2.0 ** self.sv)
        ds = f32(dot * 2.0 ** self.exd)
        self.do_hi = f16(ds)
        do_lo = f16(ds - self.do_hi)
        self.sd = FP8_EXP["do_lo"]
        self.do_lo8 = e4m3(do_lo / 2.0 ** self.sd)
        self.dot = dot
        # the bounds above hold: no e4m3 copy reaches its largest value
        self.fp8_peak = max(np.abs(x).max() for x in (self.q_lo8, self.k8, self.v8, self.do_lo8))

    def row(self, a: int, q_lo: bool, p_lo: bool, do_lo: bool, l_rounded: bool = False):
        """O_sub and dQ_sub of sub-sequence row a under one variant."""
        n = a + 1
        z = self.k16[:n] @ self.q_hi[a]
        if q_lo:
            z = z + (self.k8[:n] @ self.q_lo8[a]) * 2.0 ** (self.sq + self.sk)
        z = z * 2.0 ** -(self.exq + self.exk) / np.sqrt(self.d)
        m = z.max()
        p15 = f32(np.exp(z - m) * 2.0 ** 15)
        p_hi = f16(p15)
        lsum = p_hi.sum() if l_rounded else p15.sum()
        pv = p_hi + (f16(p15 - p_hi) if p_lo else 0.0)
        o = (pv @ self.v16[:n]) / lsum * 2.0 ** -self.exv
        lse = m + np.log(lsum * 2.0 ** -15)
        # backward: P again from the same logits and the forward's LSE
        P = f32(np.exp(z - lse))
        dp = self.v16[:n] @ self.do_hi[a]
        if do_lo:
            dp = dp + (self.v8[:n] @ self.do_lo8[a]) * 2.0 ** (self.sd + self.sv)
        delta = float(self.dot[a] @ o) * 2.0 ** (self.exd + self.exv)
        ds = f16(f32(P * (dp - delta)))
        dq = (ds @ self.k16[:n]) * 2.0 ** -(self.exd + self.exv + self.exk) / np.sqrt(self.d)
        return o, dq


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--workload", default="lh-fwdbwd-1m")
    ap.add_argument("--head", type=int, default=0)
    ap.add_argument("--rows", type=int, default=256, help="rows of each kind (largest |dO_sub|, random)")
    ap.add_argument("--shared-v", type=float, default=0.0, help="value rows A c + v / 8 (see above)")
    ap.add_argument("--v-scale", type=float, default=1.0, help="value rows times F (see above)")
    args = ap.parse_args()
    w = by_name(args.workload)
    t0 = time.time()
    q, k, v, dout = head_inputs(w, args.head, args.shared_v, args.v_scale)
    qt, kt, vt, dot = subsequence(q, k, v, dout, w)
    S = qt.shape[0]
    em = Emulation(q, k, v, qt, kt, vt, dot)
    del q, k, v, dout
    rng = np.random.default_rng(0)
    big = np.argsort(-np.linalg.norm(dot, axis=1))[: args.rows]
    rnd = rng.choice(S, size=min(args.rows, S), replace=False)
    rows = np.unique(np.concatenate([big, rnd]))
    o_ref, _ = oracle.attention_rows(qt, kt, vt, rows)
    dq_ref = oracle.attention_bwd_query_rows(qt, kt, vt, dot, rows)
    print("%s%s%s, head %d: S = %d, %d rows (the %d of largest |dO_sub|, max %.0f, and %d random); staging 2^%d 2^%d 2^%d 2^%d"
          % (w.name, ", value rows %g c + v / 8" % args.shared_v if args.shared_v else "",
             ", value rows times %g" % args.v_scale if args.v_scale != 1.0 else "", args.head, S, rows.shape[0], big.shape[0], np.linalg.norm(dot, axis=1).max(), rnd.shape[0],
             em.exq, em.exk, em.exv, em.exd))
    o_bound = ATOL + RTOL * np.abs(o_ref)
    dq_bound = ATOL + RTOL * np.abs(dq_ref).max(axis=1, keepdims=True)
    print("%-9s %22s %22s" % ("variant", "O_sub: worst / bound", "dQ_sub: worst / bound"))
    for name, flags in VARIANTS.items():
        o = np.empty_like(o_ref)
        dq = np.empty_like(dq_ref)
        for r, a in enumerate(rows):
            o[r], dq[r] = em.row(int(a), **flags)
        ro = np.abs(o - o_ref) / o_bound
        rq = np.abs(dq - dq_ref) / dq_bound
        print("%-9s %14.3f (%5d over) %14.3f (%5d over)" % (name, ro.max(), int((ro > 1).sum()), rq.max(), int((rq > 1).sum())),
              flush=True)
    print("%.0f s" % (time.time() - t0))


if __name__ == "__main__":
    main()
