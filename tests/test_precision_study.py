"""Checks of the precision study's own arithmetic (CPU): its e4m3 and fp16
roundings on values whose results are fixed by the formats, and its emulation
of the shipped operand scheme against the oracle on a small workload."""
import numpy as np
import torch

import precision_study as ps
from synth_inputs import Workload


def test_e4m3_rounding_fixed_points():
    # OCP e4m3: 3 stored mantissa bits, normal exponents -6..8 (largest 448),
    # subnormal spacing 2^-9; ties to even
    x = np.array([448.0, 1.0, 0.3, 1.0625, 1.1875, 2.0 ** -6, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, -5.3])
    want = np.array([448.0, 1.0, 0.3125, 1.0, 1.25, 2.0 ** -6, 2.0 ** -9, 0.0, 2.0 ** -8, -5.5])
    assert np.array_equal(ps.e4m3(x), want)


def test_f16_rounding_fixed_points():
    # fp16: 10 stored mantissa bits; 1 + 2^-11 is a tie that goes to 1 (even),
    # 1 + 3 * 2^-11 a tie that goes to 1 + 2^-9
    x = np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 65504.0, 2.0 ** -24])
    assert np.array_equal(ps.f16(x), np.array([1.0, 1.0 + 2.0 ** -9, 65504.0, 2.0 ** -24]))


def test_scale_exponents():
    assert ps.stage_exp(3.0, 12) == 10          # 3 * 2^10 in [2^11, 2^12)
    assert ps.stage_exp(2048.0, 12) == 0
    # the largest staged magnitude of each e4m3 operand lands on 2^8 <= 448
    assert ps.FP8_EXP == {"q_lo": -8, "k": 4, "v": -3, "do_lo": -11}
    big = np.nextafter(np.float32(4096.0), np.float32(0.0))   # largest staged |q| below 2^12
    q_lo = float(np.float32(big) - np.float32(ps.f16(big)))
    assert abs(q_lo) <= 1.0 and abs(q_lo) / 2.0 ** ps.FP8_EXP["q_lo"] <= 256.0


def test_emulated_scheme_small_workload():
    # the shipped scheme stays inside the parity bounds on a small bf16 case,
    # and dropping dO_sub's lo part is never better than keeping it
    w = Workload("study-small", 1, 64, 4096, 3, 4, 64, torch.bfloat16, 4, True)
    q, k, v, dout = ps.head_inputs(w, 0)
    qt, kt, vt, dot = ps.subsequence(q, k, v, dout, w)
    em = ps.Emulation(q, k, v, qt, kt, vt, dot)
    rows = np.arange(qt.shape[0])
    o_ref, _ = ps.oracle.attention_rows(qt, kt, vt, rows)
    dq_ref = ps.oracle.attention_bwd_query_rows(qt, kt, vt, dot, rows)
    o_bound = ps.ATOL + ps.RTOL * np.abs(o_ref)
    dq_bound = ps.ATOL + ps.RTOL * np.abs(dq_ref).max(axis=1, keepdims=True)
    worst = {}
    for name, flags in ps.VARIANTS.items():
        o = np.empty_like(o_ref)
        dq = np.empty_like(dq_ref)
        for r, a in enumerate(rows):
            o[r], dq[r] = em.row(int(a), **flags)
        worst[name] = (np.max(np.abs(o - o_ref) / o_bound), np.max(np.abs(dq - dq_ref) / dq_bound))
    assert em.fp8_peak <= 256.0
    assert worst["shipped"][0] < 1.0 and worst["shipped"][1] < 1.0
    assert worst["no-dO-lo"][1] >= worst["shipped"][1]
