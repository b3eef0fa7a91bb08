"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: scores, selection, order and slot maps bit-exact on EVERY
head; attention output, layer output and (for the forward + backward
workloads) gradients against the CPU oracle on one sampled head, whose
fp64 attention over S ~ 10-22K entries takes the oracle well under a minute.
Inputs are drawn on the device and copied to the host for the oracle."""
import numpy as np
import pytest
import torch

import oracle
from parity import GpuRun, compare_backward, compare_forward, compare_selection, head_inputs, say
from synth_inputs import WORKLOADS, make_dout, make_qkv

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("w", WORKLOADS[1:], ids=lambda w: w.name)
def test_full_size_workload(w):
    say("workload %s: N=%d H=%d d=%d L=%d p=%d k=%d S=%d bwd=%s"
        % (w.name, w.N, w.H, w.d, w.L, w.p, w.k, oracle.subseq_len(w.N, w.L, w.p, w.k), w.backward))
    q, k, v = make_qkv(w.N, w.H, w.d, w.dtype, w.n_plant, seed=0, device="cuda")
    dout = make_dout(w.N, w.H, w.d, w.dtype, seed=1, device="cuda") if w.backward else None
    run = GpuRun(q, k, v, w.L, w.p, w.k, dout)
    for h in range(w.H):
        qh, kh = head_inputs(q, h), head_inputs(k, h)
        sc = oracle.score_pyramid(oracle.token_scores(qh, kh), w.L, w.p)
        sel = oracle.select(sc, w.L, w.k)
        lev, idx = oracle.causal_order(oracle.expand(sel, w.N, w.L, w.p), w.p)
        compare_selection(run, h, dict(scores=sc, sel=sel, ent_level=lev, ent_index=idx))
    say("  selection of all %d heads bit-exact" % w.H)
    h = w.H // 2  # one sampled head, full numerics
    ref = oracle.forward(head_inputs(q, h), head_inputs(k, h), head_inputs(v, h), w.L, w.p, w.k)
    stats = compare_forward(run, h, ref, w.name)
    if w.backward:
        gref = oracle.backward(ref, head_inputs(dout, h), w.p)
        stats.update(compare_backward(run, h, ref, gref, w.name))
    say("  head %d: %s" % (h, {n: "%.2g/%.2g" % s for n, s in stats.items()}))
    assert np.all(np.isfinite(run.out.float().cpu().numpy()))
