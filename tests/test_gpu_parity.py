"""GPU parity of the whole Lighthouse path against the CPU oracle, at sizes the
oracle finishes in seconds: several tiles per kernel, ragged sub-sequence
tails, every dtype / head size, and the method's degenerate cases. Calls go
through the C ABI (liblh.so via ctypes)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_long_context_lh_amd as lh
from parity import ATOL, RTOL, GpuRun, assert_close, check_case, compare_selection, head_inputs, say, selection_ref
from synth_inputs import make_dout, make_qkv

pytestmark = pytest.mark.gpu


def _case(N, H, d, L, p, k, dtype=torch.bfloat16, n_plant=8, seed=0, bwd=False, heads=None, tag="", scorer="sum"):
    say("case %s: N=%d H=%d d=%d L=%d p=%d k=%d dtype=%s S=%d bwd=%s scorer=%s"
        % (tag, N, H, d, L, p, k, dtype, oracle.subseq_len(N, L, p, k), bwd, scorer))
    q, kk, v = (x.cuda() for x in make_qkv(N, H, d, dtype, n_plant, seed))
    dout = make_dout(N, H, d, dtype, seed + 1).cuda() if bwd else None
    return check_case(q, kk, v, L, p, k, dout, heads=heads, tag=tag, scorer=scorer)


def test_sqrt_correctly_rounded_all_positive_floats():
    # every positive finite fp32 value, in two launches
    bad = lh.selftest_sqrt(1, 0x40000000) + lh.selftest_sqrt(0x40000001, 0x7f800000 - 0x40000001)
    assert bad == 0


def test_fp32_d64_small_workload():
    # the 4K fp32 workload itself: N=4096, H=4, d=64, L=3, p=2, k=256 (S=2048)
    _case(4096, 4, 64, 3, 2, 256, torch.float32, n_plant=0, tag="fp32-4k")


def test_bf16_d128_p2_strata_ragged():
    # level 1 has 4 strata, level 2 has 2; S = 4096 + 2*2*300 = 5296 (ragged tail)
    _case(16384, 2, 128, 3, 2, 300, tag="p2-strata")


def test_bf16_d128_p4_L4_ragged():
    _case(32768, 2, 128, 4, 4, 100, n_plant=32, tag="p4-L4")


def test_bf16_d64_p8():
    _case(8192, 2, 64, 3, 8, 100, tag="p8")


def test_backward_p4_L3():
    _case(8192, 2, 128, 3, 4, 50, bwd=True, tag="bwd-p4")


def test_backward_p2_d64_fp32():
    _case(4096, 2, 64, 3, 2, 200, torch.float32, n_plant=0, bwd=True, tag="bwd-fp32")


def test_backward_fp32_d128():
    # fp32 inputs at d = 128: the logits take the key's lo part as well
    _case(4096, 2, 128, 3, 2, 128, torch.float32, n_plant=4, bwd=True, tag="bwd-fp32-d128")


def test_backward_L5_p4_shape_of_512k():
    # the 512K workload's pyramid (L=5, p=4) at N=32K: S = 128 + 4*4*32 = 640
    _case(32768, 2, 128, 5, 4, 32, n_plant=32, bwd=True, tag="bwd-L5")


def test_upper_levels_p4_L6():
    # levels 4 and 5 lie above the row tiles of the front pass and of the
    # scatter-back adjoint: they are built from the window sums of the level below
    _case(8192, 2, 128, 6, 4, 4, n_plant=4, bwd=True, tag="up-p4-L6")


def test_upper_levels_p8_L4_d64():
    _case(8192, 2, 64, 4, 8, 8, n_plant=4, bwd=True, tag="up-p8-L4")


def test_upper_levels_p2_L8():
    _case(8192, 2, 128, 8, 2, 16, n_plant=4, bwd=True, tag="up-p2-L8")


def test_dense_L1_fwd_bwd_ragged():
    # L = 1: S = N, dense causal attention; N = 1000 is not a multiple of any tile
    _case(1000, 2, 64, 1, 2, 0, bwd=True, tag="L1")


def test_k0_only_top_level():
    _case(4096, 2, 128, 3, 2, 0, bwd=True, tag="k0")


def test_everything_selected():
    # L = 2, k = n_1: the whole pyramid is gathered (S = N + N/p)
    _case(2048, 2, 64, 2, 2, 1024, bwd=True, tag="all")


def test_ties_take_lowest_index():
    # every row equal: all scores tie, each stratum keeps its lowest indices
    N, H, d, L, p, k = 16384, 1, 128, 3, 2, 77
    row = torch.randn(d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    q = row.expand(H, N, d).contiguous().cuda()
    run = GpuRun(q, q, q, L, p, k)
    sel = run.head("sel", 0).numpy()
    for l in (1, 2):
        want = oracle.stratified_topk(np.ones(N // p ** l, dtype=np.float32), k)
        assert np.array_equal(sel[l - 1], want)
    res = oracle.forward(q[0].float().cpu().numpy(), q[0].float().cpu().numpy(), q[0].float().cpu().numpy(), L, p, k)
    assert np.array_equal(sel[0], res["sel"][1]) and np.array_equal(sel[1], res["sel"][2])


@pytest.mark.parametrize("p_two", [0.1, 0.02])
def test_partial_ties_across_a_stratum(p_two):
    # Rows are c_j times one fixed row (c_j = 2 with probability p_two, else
    # 1), so every score takes one of two values and a stratum of 2048
    # entries holds hundreds of equal ones. With p_two = 0.1 the quota-th
    # largest score is the larger value and the kept ties (the first r in
    # index order) run across several waves and chunks of the stratum; with
    # 0.02 fewer than the quota hold the larger value and the threshold is the
    # smaller one, most of the stratum tying with it.
    N, H, d, L, p, k = 65536, 2, 64, 3, 2, 3000
    g = torch.Generator().manual_seed(11)
    u, w = torch.randn(d, generator=g), torch.randn(d, generator=g)
    c = torch.where(torch.rand(H, N, 1, generator=g) < p_two, 2.0, 1.0)  # one factor per token
    q, kk, v = ((c * row).to(torch.bfloat16).cuda() for row in (u, w, torch.randn(d, generator=g)))
    run = GpuRun(q, kk, v, L, p, k)
    for h in range(H):
        ref = selection_ref(q, kk, h, L, p, k)
        compare_selection(run, h, ref)
        sc1 = ref["scores"][1]
        say("  p_two=%.2f head %d: level 1 holds %d entries at the larger score" % (p_two, h, int((sc1 == sc1.max()).sum())))


def test_deterministic_bitwise():
    N, H, d, L, p, k = 16384, 2, 128, 3, 4, 200
    q, kk, v = (x.cuda() for x in make_qkv(N, H, d, torch.bfloat16, 8, 5))
    dout = make_dout(N, H, d, torch.bfloat16, 6).cuda()
    a = GpuRun(q, kk, v, L, p, k, dout)
    b = GpuRun(q, kk, v, L, p, k, dout)
    assert torch.equal(a.out, b.out)
    for x, y in zip(a.grads, b.grads):
        assert torch.equal(x, y)


def test_heads_are_independent():
    # head h of an H-head call equals a 1-head call on head h alone
    N, H, d, L, p, k = 8192, 3, 128, 3, 2, 64
    q, kk, v = (x.cuda() for x in make_qkv(N, H, d, torch.bfloat16, 8, 7))
    full = GpuRun(q, kk, v, L, p, k)
    one = GpuRun(q[1:2].contiguous(), kk[1:2].contiguous(), v[1:2].contiguous(), L, p, k)
    assert torch.equal(full.out[1], one.out[0])


def test_heads_of_very_different_magnitudes():
    # the fp8 copies of the lo products take one scale per head and tensor:
    # head 0 has Q and V 32 times larger, K 32 times smaller and dO 8 times
    # larger than the seeded inputs, head 1 the reverse (logits unchanged;
    # dP, and with it dS, stays well inside the fp16 range)
    N, H, d, L, p, k = 16384, 2, 128, 3, 4, 64
    q, kk, v = make_qkv(N, H, d, torch.bfloat16, 8, 11)
    dout = make_dout(N, H, d, torch.bfloat16, 12)
    f = torch.tensor([32.0, 1.0 / 32.0]).view(H, 1, 1)  # powers of two: exact in bf16
    g = torch.tensor([8.0, 1.0 / 8.0]).view(H, 1, 1)
    q, kk, v, dout = ((x.float() * s).to(torch.bfloat16) for x, s in ((q, f), (kk, 1.0 / f), (v, f), (dout, g)))
    say("case scaled heads: N=%d H=%d d=%d L=%d p=%d k=%d" % (N, H, d, L, p, k))
    check_case(q.cuda(), kk.cuda(), v.cuda(), L, p, k, dout.cuda(), tag="scaled-heads")


def test_zero_upstream_gradient():
    # dO = 0: every lo part and tile maximum is zero (the fp8 scales take
    # their smallest exponent); all gradients must be exactly zero
    N, H, d, L, p, k = 8192, 2, 128, 3, 4, 50
    q, kk, v = (x.cuda() for x in make_qkv(N, H, d, torch.bfloat16, 8, 13))
    run = GpuRun(q, kk, v, L, p, k, torch.zeros(H, N, d, dtype=torch.bfloat16, device="cuda"))
    for g in run.grads:
        assert torch.count_nonzero(g).item() == 0
    assert torch.all(torch.isfinite(run.out.float()))


def test_kept_sums_of_a_level_not_materialised():
    # fp32, k = 1: level 3 (256 entries, the last one finished in the front
    # pass's tiles at d = 64) is cheaper to re-average in the gather than to
    # write, so the level above it is built from the kept window sums rather
    # than from pooled means
    _case(16384, 1, 64, 5, 4, 1, torch.float32, n_plant=0, bwd=True, tag="kept-sums")


@pytest.mark.parametrize("N,H,d,L,p,k,dtype", [
    (4, 1, 64, 3, 2, 1, torch.float32),    # levels of 4, 2 and 1 entries; S = 1 + 2*2*1 = 5
    (8, 2, 64, 2, 4, 2, torch.bfloat16),   # everything of level 1 selected; S = 2 + 4*2 = 10
    (64, 1, 128, 3, 2, 3, torch.bfloat16), # one row tile, odd k
])
def test_tiny_pyramids(N, H, d, L, p, k, dtype):
    # far smaller than any tile of any kernel: every load and store is a tail
    _case(N, H, d, L, p, k, dtype, n_plant=0, bwd=True, tag="tiny")


def test_single_token():
    # N = 1, L = 1: the softmax has one term, so the output is the value row
    # itself and dV = dO; dQ and dK are zero up to the rounding of dP - delta
    N, H, d = 1, 2, 128
    q, kk, v = (x.cuda() for x in make_qkv(N, H, d, torch.bfloat16, 0, 17))
    dout = make_dout(N, H, d, torch.bfloat16, 18).cuda()
    say("case single token: N=1 H=2 d=128 L=1")
    check_case(q, kk, v, 1, 2, 0, dout, tag="single-token")
    run = GpuRun(q, kk, v, 1, 2, 0, dout)
    assert torch.equal(run.out, v)
    assert torch.equal(run.grads[2], dout)


@pytest.mark.parametrize("N,H,d,L,p,k,dtype", [
    (8192, 2, 128, 3, 2, 300, torch.bfloat16),   # ragged tail, strata
    (16384, 2, 128, 4, 4, 40, torch.bfloat16),
    (4096, 2, 64, 3, 2, 256, torch.float32),      # fp32: the K lo product stays
    (3000, 2, 128, 1, 2, 0, torch.bfloat16),      # dense, ragged
    (2048, 1, 64, 3, 8, 0, torch.bfloat16),       # top level only
])
def test_forward_nograd(N, H, d, L, p, k, dtype):
    # the forward no backward follows: whole-path parity with the oracle, and
    # the same selection, order, staged rows and log-sum-exp as lh_forward
    # bit for bit (only O_sub differs)
    tag = "nograd N=%d L=%d p=%d k=%d %s d=%d" % (N, L, p, k, dtype, d)
    say("case %s" % tag)
    q, kk, v = (x.cuda() for x in make_qkv(N, H, d, dtype, 8, 5))
    run, _ = check_case(q, kk, v, L, p, k, tag=tag, nograd=True)
    full = GpuRun(q, kk, v, L, p, k)
    names = ["ent", "qhi", "khi", "v", "lse"] + (["qlo", "klo"] if dtype == torch.float32 else []) \
        + (["scores", "sel", "slot"] if L > 1 else [])
    for h in range(H):
        for name in names:
            a, b = run.head(name, h), full.head(name, h)
            if name in ("ent", "lse", "qhi", "qlo", "khi", "klo", "v"):
                a, b = a[:run.S], b[:run.S]
            assert torch.equal(a, b), (name, h)
    # both outputs are within the element-wise bound of the oracle's, so
    # within twice that bound of each other
    a, b = run.out.float(), full.out.float()
    say("  nograd vs lh_forward: max |out difference| %.3g" % (a - b).abs().max().item())
    assert bool(((a - b).abs() <= 2 * (ATOL + RTOL * b.abs())).all())


def test_forward_nograd_large_values():
    # lh_forward_nograd forms P.V from each probability rounded once to fp16
    # (relative error at most 2^-11), so an element (row, c) of one level's
    # O_sub moves by at most 2^-11 times the largest |v[:, c]| among the rows
    # it attends, and out (a sum over at most L levels) by L times that. With
    # value rows 32 times the seeded inputs (head 0; head 1: 1/32) that term
    # is larger than the bound's absolute part, so the check adds it to the
    # bound; the count over the plain bound is reported beside it.
    N, H, d, L, p, k = 16384, 2, 128, 3, 4, 64
    q, kk, v = make_qkv(N, H, d, torch.bfloat16, 8, 11)
    f = torch.tensor([32.0, 1.0 / 32.0]).view(H, 1, 1)  # powers of two: exact in bf16
    v = (v.float() * f).to(torch.bfloat16)
    say("case nograd, value rows times 32 and 1/32: N=%d H=%d d=%d L=%d p=%d k=%d" % (N, H, d, L, p, k))
    run = GpuRun(q.cuda(), kk.cuda(), v.cuda(), L, p, k, nograd=True)
    for h in range(H):
        qh, kh, vh = head_inputs(q, h), head_inputs(kk, h), head_inputs(v, h)
        ref = oracle.forward(qh, kh, vh, L, p, k)
        extra = 2.0 ** -11 * np.abs(vh).max(axis=0, keepdims=True)  # per column c
        osub = run.head("osub", h)[:run.S].numpy()
        out = run.out[h].float().cpu().numpy()
        st_o = assert_close(osub, ref["ot"], "nograd head %d O_sub" % h, atol=ATOL + extra)
        st = assert_close(out, ref["out"], "nograd head %d output" % h, atol=ATOL + L * extra, stored_bf16=True)
        plain = int((np.abs(out - ref["out"]) > ATOL + RTOL * np.abs(ref["out"])).sum())
        say("  head %d: O_sub max-abs %.3g, out max-abs %.3g (largest |v| %.3g); %d outputs over the plain bound"
            % (h, st_o["max_abs"], st["max_abs"], float(np.abs(vh).max()), plain))


def test_selection_hook_and_forward_only_workspace():
    # lh_selection points at the selection lh_forward made (level by level,
    # [H, k], equal to the oracle's); a forward given only the forward's
    # prefix of the workspace writes the same output bit for bit
    N, H, d, L, p, k = 32768, 2, 128, 4, 4, 40
    q, kk, v = (x.cuda() for x in make_qkv(N, H, d, torch.bfloat16, 8, 21))
    say("case selection hook: N=%d H=%d d=%d L=%d p=%d k=%d" % (N, H, d, L, p, k))
    full = GpuRun(q, kk, v, L, p, k)
    ws_fwd = lh.alloc_workspace(N, H, d, L, p, k, torch.bfloat16, forward_only=True)
    assert ws_fwd.numel() == lh.forward_workspace_bytes(N, H, d, L, p, k, torch.bfloat16)
    assert ws_fwd.numel() < full.ws.numel()
    out2, _ = lh.forward(q, kk, v, L, p, k, ws=ws_fwd)
    torch.cuda.synchronize()
    assert torch.equal(out2, full.out)
    for h in range(H):
        ref = oracle.forward(q[h].float().cpu().numpy(), kk[h].float().cpu().numpy(), v[h].float().cpu().numpy(),
                             L, p, k)
        for l in range(1, L):
            a = lh.selection(full.ws, N, H, d, L, p, k, l)[h].cpu().numpy()
            b = lh.selection(ws_fwd, N, H, d, L, p, k, l)[h].cpu().numpy()
            assert np.array_equal(a, ref["sel"][l]) and np.array_equal(b, ref["sel"][l])
            assert np.array_equal(a, full.head("sel", h)[l - 1].numpy())


@pytest.fixture
def recompute_dq():
    """Plans without stored dS tiles: the dQ kernel recomputes S and dP."""
    old = lh.ds_tile_budget()
    lh.set_ds_tile_budget(0)
    yield
    lh.set_ds_tile_budget(old)


@pytest.mark.parametrize("N,H,d,L,p,k,dtype,n_plant", [
    (32768, 2, 128, 5, 4, 32, torch.bfloat16, 32),   # the 512K workload's pyramid
    (8192, 2, 128, 3, 4, 50, torch.bfloat16, 8),
    (4096, 2, 64, 3, 2, 200, torch.float32, 0),
    (4096, 2, 128, 3, 2, 128, torch.float32, 4),
    (1000, 2, 64, 1, 2, 0, torch.bfloat16, 8),       # dense, ragged
    (64, 1, 128, 3, 2, 3, torch.bfloat16, 0),        # one tile, all tail
])
def test_recomputed_dq(recompute_dq, N, H, d, L, p, k, dtype, n_plant):
    _case(N, H, d, L, p, k, dtype, n_plant=n_plant, bwd=True, tag="dq-recompute")


def test_recomputed_dq_against_stored_tiles():
    # same dK and dV bit for bit (the dK/dV kernel only skips its dS store);
    # dQ from recomputed S and dP within the tolerance of the stored tiles' dQ
    N, H, d, L, p, k = 16384, 2, 128, 4, 4, 60
    q, kk, v = (x.cuda() for x in make_qkv(N, H, d, torch.bfloat16, 8, 41))
    dout = make_dout(N, H, d, torch.bfloat16, 42).cuda()
    a = GpuRun(q, kk, v, L, p, k, dout)
    old = lh.ds_tile_budget()
    lh.set_ds_tile_budget(0)
    try:
        b = GpuRun(q, kk, v, L, p, k, dout)
    finally:
        lh.set_ds_tile_budget(old)
    assert b.ws.numel() < a.ws.numel()
    assert torch.equal(a.out, b.out)
    assert torch.equal(a.grads[1], b.grads[1]) and torch.equal(a.grads[2], b.grads[2])
    for h in range(H):
        x, y = a.head("dqsub", h)[:a.S].numpy(), b.head("dqsub", h)[:a.S].numpy()
        err = np.abs(x.astype(np.float64) - y)
        assert np.all(err <= 2e-2 + 2.0 ** -7 * np.abs(x).max(axis=-1, keepdims=True))
        say("  head %d: dQ_sub recomputed vs stored tiles: max %.3g" % (h, err.max()))


@pytest.mark.parametrize("scorer", ["product", "query", "key", "sum"])
@pytest.mark.parametrize("N,H,d,L,p,k,dtype", [
    (16384, 2, 128, 3, 2, 300, torch.bfloat16),   # level 1 in 4 strata
    (32768, 2, 64, 4, 4, 100, torch.float32),
])
def test_scorer_variants(scorer, N, H, d, L, p, k, dtype):
    # each score variant: scores at every level and the selection bit-exact,
    # the whole layer (forward and backward) within tolerance
    _case(N, H, d, L, p, k, dtype, n_plant=16, bwd=True, tag="score-" + scorer, scorer=scorer)


def test_scorers_select_differently():
    # the variants are really different rankings on these inputs (per-token
    # scales shared by Q and K make them close, so K gets its own scale here)
    N, H, d, L, p, k = 16384, 1, 128, 3, 2, 200
    q, kk, v = make_qkv(N, H, d, torch.bfloat16, 8, 51)
    kk = (kk.float() * torch.exp(torch.randn(N, generator=torch.Generator().manual_seed(52)))[None, :, None]).to(
        torch.bfloat16)
    q, kk, v = q.cuda(), kk.cuda(), v.cuda()
    sels = {}
    for scorer in ("sum", "product", "query", "key"):
        run = GpuRun(q, kk, v, L, p, k, scorer=scorer)
        sels[scorer] = run.head("sel", 0).numpy().copy()
        ref = oracle.forward(q[0].float().cpu().numpy(), kk[0].float().cpu().numpy(), v[0].float().cpu().numpy(),
                             L, p, k, scorer=scorer)
        for l in range(1, L):
            assert np.array_equal(sels[scorer][l - 1], ref["sel"][l]), (scorer, l)
    names = list(sels)
    for i in range(len(names)):
        for j in range(i + 1, len(names)):
            assert not np.array_equal(sels[names[i]], sels[names[j]]), (names[i], names[j])



@pytest.mark.parametrize("N,H,d,dm,L,p,k,dtype", [
    (8192, 2, 128, 256, 3, 4, 50, torch.bfloat16),
    (4096, 2, 64, 96, 3, 2, 100, torch.float32),
    (1000, 2, 64, 64, 1, 2, 0, torch.bfloat16),    # dense, ragged
])
def test_layer_with_projections(N, H, d, dm, L, p, k, dtype):
    # the step around the layer: projections in (rocBLAS GEMMs), the layer,
    # and the backward to x and W. The projected rows equal x W to within
    # their rounding to the storage type; from those rows on, the oracle runs
    # the layer (selection bit-exact, outputs within tolerance) and its
    # backward, then the projections' adjoint in fp64.
    from parity import Failures, assert_close, compare_selection, fmt_stats
    from synth_inputs import make_layer_inputs
    say("case layer: N=%d H=%d d=%d d_model=%d L=%d p=%d k=%d dtype=%s" % (N, H, d, dm, L, p, k, dtype))
    x, w = make_layer_inputs(N, dm, H, d, dtype, n_plant=8, seed=61)
    dout = make_dout(N, H, d, dtype, 62)
    xc, wc, dc = x.cuda(), w.cuda(), dout.cuda()
    out, ws = lh.layer_forward(xc, wc, H, d, L, p, k)
    qkv = lh.layer_qkv(ws, N, H, d, dtype).float().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    xd, wd = x.double().numpy(), w.double().numpy()
    ref_qkv = oracle.project(xd, wd, H, d)
    # one rounding to the storage type (at most an ulp, whatever the GEMM's
    # rounding mode) plus fp32 accumulation over d_model terms
    ulp = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -23
    acc = oracle.project(np.abs(xd), np.abs(wd), H, d)
    ratio = np.abs(qkv - ref_qkv) / (ulp * np.abs(ref_qkv) + 2.0 ** -20 * acc)
    say("  projections: max |g - r| %.3g, worst fraction of the bound %.3g" % (np.abs(qkv - ref_qkv).max(),
                                                                          ratio.max()))
    assert ratio.max() <= 1.0
    fwd = oracle.layer_forward(xd, wd, H, d, L, p, k, qkv=qkv)
    bf = dtype == torch.bfloat16
    fails = Failures()
    st = {}
    # the layer's own workspace follows the projected rows (next 256 bytes)
    lh_ws = ws[(3 * H * N * d * (2 if bf else 4) + 255) // 256 * 256:]
    for h in range(H):
        for l in range(1, L):
            got = lh.selection(lh_ws, N, H, d, L, p, k, l)[h].cpu().numpy()
            assert np.array_equal(got, fwd["heads"][h]["sel"][l]), (h, l)
        fails.check(st, "out%d" % h, out[h].float().cpu().numpy(), fwd["out"][h], "layer head %d out" % h,
                    stored_bf16=bf)
    dx, dw = lh.layer_backward(xc, wc, dc, H, d, L, p, k, ws)
    torch.cuda.synchronize()
    g = oracle.layer_backward(fwd, xd, wd, dout.double().numpy(), p)
    fails.check(st, "dx", dx.float().cpu().numpy(), g["dx"], "layer dx", stored_bf16=bf, row_scaled=True)
    fails.check(st, "dw", dw.float().cpu().numpy(), g["dw"], "layer dw", stored_bf16=bf, row_scaled=True)
    say("  layer: " + "; ".join("%s %s" % (n, fmt_stats(x_)) for n, x_ in st.items()))
    fails.raise_if_any()


def test_values_sharing_one_direction():
    # Every value row is 16 c + v / 8 for one fixed row c: the values a query
    # attends to nearly agree, so dP - delta, dS and dq are small by
    # cancellation while |delta| is not, and the dq bound is mostly its
    # absolute term. What P's fp16 rounding leaves in O_sub, and so in delta,
    # is then what that bound sees: the precision study
    # (tests/precision_study.py, emulating every row of this case) puts dQ_sub
    # at 0.34-0.48 of the bound with the fp16 pair of P in the forward and at
    # 1.4-1.9, 12-36 elements over, without its lo half. Top-level windows of
    # 256 tokens, so dO_sub rows sum up to 256 rows of dO.
    N, H, d, L, p, k = 65536, 2, 128, 5, 4, 256
    q, kk, v = make_qkv(N, H, d, torch.bfloat16, 8, 81)
    c = torch.randn(d, generator=torch.Generator().manual_seed(7))
    v = (16.0 * c + v.float() / 8).to(torch.bfloat16)
    dout = make_dout(N, H, d, torch.bfloat16, 82)
    say("case values sharing one direction: N=%d H=%d d=%d L=%d p=%d k=%d S=%d"
        % (N, H, d, L, p, k, oracle.subseq_len(N, L, p, k)))
    check_case(q.cuda(), kk.cuda(), v.cuda(), L, p, k, dout.cuda(), tag="shared-v")


@pytest.mark.parametrize("N,L,p,k", [(16384, 3, 4, 64), (1000, 1, 2, 0)])
def test_heads_scaled_far_outside_fp16(N, L, p, k):
    # head 0 has Q, V and dO times 2^12 and K times 2^-12, head 1 the reverse
    # (powers of two: exact in bf16; the logits q.k are those of the seeded
    # inputs). Without per-head staging scales the fp16 rows of head 0 (|q|,
    # |v| up to 7e4, dO_sub sums beyond 1e6) would overflow and those of head 1
    # (|q|, |v|, |dO| around 1e-4) would lose their low bits to fp16's
    # subnormals. For any fixed selection such a head is the unit-scale
    # problem with its outputs multiplied by powers of two: out and dv by f,
    # dq by f_do f_v f_k = f, dk by f_do f_v f_q = f^3 (f = 2^12 or 2^-12);
    # the bound's absolute term is carried over by the same factors.
    H, d = 2, 128
    q, kk, v = make_qkv(N, H, d, torch.bfloat16, 8, 71)
    dout = make_dout(N, H, d, torch.bfloat16, 72)
    f = torch.tensor([2.0 ** 12, 2.0 ** -12]).view(H, 1, 1)
    q, v, dout = ((x.float() * f).to(torch.bfloat16) for x in (q, v, dout))
    kk = (kk.float() / f).to(torch.bfloat16)
    say("case heads scaled by 2^12 and 2^-12: N=%d H=%d d=%d L=%d p=%d k=%d" % (N, H, d, L, p, k))

    def factors(h):
        fh = float(f[h])
        return {"out": fh, "dout": fh, "dq": fh, "dv": fh, "dk": fh ** 3}
    check_case(q.cuda(), kk.cuda(), v.cuda(), L, p, k, dout.cuda(), tag="scaled-2^12", scales=factors)
