"""Throughput of the Lighthouse layer (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-extra] [--copy-calibration]
    python bench.py --sweep [--steps K] [--warmup W]   ((L, p, k) sweep at 512K tokens)
    python bench.py --summarize-stats DIR              (rocprofv3 --stats output -> markdown)
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR [--workload NAME]

A step is one lh_forward + lh_backward over the whole workload (every stage
of the path, all heads), inputs resident in HBM. The default workload is the
512K-token forward + backward shape (H=16, d=128, L=5, p=4, k=512, S=10240),
the single-layer setting at which the layer's forward and forward+backward
speedups are quoted. Prints one JSON line.

With the default workload the same JSON line also carries the rest of the
metric's range ("workloads": 1M tokens forward + backward, 128K and 64K
forward, each with its dominant stage's roofline) and dense causal attention
over the same 512K tokens ("dense_512k": L = 1, S = N, one warmup and one
timed step), with the layer's speedup over it, forward and forward+backward,
and the step around the layer ("projection_layer_512k": Q/K/V projections of
an input with d_model = 2048 in, the backward to the input and the weights;
the projections' share is that step minus the layer's own).

Per-kernel timing: the library records caller-created HIP events between its
stages on the launch stream (lh_forward_timed / lh_backward_timed), so every
stage's average launch duration is measured inside the timed region. The
roofline object describes the stage with the largest share of the step.

HBM traffic: two rocprofv3 counter runs of this script with
--copy-calibration (one with --pmc FETCH_SIZE, one with --pmc WRITE_SIZE)
see, besides the layer's kernels, one elementwise kernel that reads and
writes exactly 1 GiB; the ratio of those bytes to what the counters report
for it scales the layer's kernels. --summarize-traffic writes the scaled
bytes per launch of every stage to profiles/traffic_<stage>_<workload>.json,
tagged with the digest of the kernel sources, and the "traffic" field of
the roofline object is read from there only while the sources still match.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Lighthouse layer tokens/s fwd & fwd+bwd at 128K–1M; % HBM / MFMA peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, datasheet
MFMA_F16_PEAK_TFS = 2500.0   # MI355X dense fp16 / bf16 matrix, datasheet

MFMA_STAGES = {"attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq"}

# rocprofv3 kernel names -> stages of the path
KERNEL_STAGES = [
    (r"lh::k_(front(_up)?|absmax)<", "front"),
    (r"lh::k_head_exp\(", "head_exp"),      # once in the forward, once in the backward
    (r"lh::k_topk\(", "topk"),
    (r"lh::k_index\(", "index"),
    (r"lh::k_gather<", "gather"),
    (r"lh::k_attn_fwd<", "attn_fwd"),
    (r"lh::k_pull<\d+, [^,]+, 1, 1,", "scatter"),
    (r"lh::k_scatter_bwd(_up)?<", "scatter_bwd"),
    (r"lh::k_(bwd_prep<|rowmax<)", "bwd_prep"),
    (r"lh::k_attn_bwd_dkdv<", "attn_bwd_dkdv"),
    (r"lh::k_attn_bwd_dq(_rc)?<", "attn_bwd_dq"),
    (r"lh::k_pull<\d+, [^,]+, 3, 0,", "pool_bwd"),
]
CALIB_BYTES = 1 << 30        # the calibration kernel reads and writes this many bytes
CALIB_PATTERN = r"neg_kernel"


def stage_of(kernel_name: str):
    import re
    for pat, stage in KERNEL_STAGES:
        if re.search(pat, kernel_name):
            return stage
    return None


def ds_tiles_kept(w, S: int) -> bool:
    """Whether the library's plan stores the backward's dS tiles for this shape
    (the causal half of S x S per head in fp16, within the dS tile budget);
    otherwise its dQ kernel recomputes S and dP."""
    import sparse_long_context_lh_amd as lh
    T = (S + 255) // 256 * 256 // 32
    return 2 * w.H * (T * (T + 1) // 2) * 1024 <= lh.ds_tile_budget()


def mfma_factor(stage: str, dtype_name: str, nograd: bool, ds_kept: bool = True) -> float:
    """Matrix-core cycles the attention kernels execute per algorithmic one:
    the precision scheme's extra products per 32x32 tile pair (fp16 32x32x16
    products take 32 cycles, block-scaled fp8 32x32x64 ones 64). bf16 inputs:
    forward 24 fp16 + 2 fp8 (without the backward's context 16 + 2) against
    16; dK/dV 32 + 4 fp8 against 32; dQ from stored tiles 8 against 8, dQ
    recomputing S and dP 24 + 4 fp8 against 24. fp32 inputs: forward 40 (32
    without the context), dK/dV 56, recomputing dQ 48."""
    bf16 = dtype_name == "bf16"
    if stage == "attn_fwd":
        return ((16 if nograd else 24) * 32 + 2 * 64) / 512.0 if bf16 else (32.0 if nograd else 40.0) / 16.0
    if stage == "attn_bwd_dkdv":
        return (32 * 32 + 4 * 64) / 1024.0 if bf16 else 56.0 / 32.0
    if stage == "attn_bwd_dq" and not ds_kept:
        return (24 * 32 + 4 * 64) / 768.0 if bf16 else 48.0 / 24.0
    return 1.0


def algorithmic(stage: str, w, S: int) -> float:
    """Algorithmic work of one launch of `stage` over the whole workload:
    flops for the attention stages, HBM bytes for the others (the least
    traffic the stage's definition needs: each listed array read or written
    once)."""
    N, H, d = w.N, w.H, w.d
    s_io = 2 if w.dtype_name == "bf16" else 4
    lvl = sum(N // w.p ** l for l in range(w.L))
    sub = S * d * H
    if stage == "attn_fwd":        # Q K^T and P V, causal: 2 * (S^2/2) * d * 2
        return 2.0 * S * S * d * H
    if stage == "attn_bwd_dkdv":   # S, dP, dV, dK: four causal products
        return 4.0 * S * S * d * H
    if stage == "attn_bwd_dq":     # dQ: one causal product (three when S and dP are recomputed)
        return (1.0 if ds_tiles_kept(w, S) else 3.0) * S * S * d * H
    if stage == "front":           # read Q, K, V; write the score pyramid
        return 3.0 * N * d * H * s_io + 4.0 * lvl * H
    if stage == "topk":            # read levels 1.. of the scores; write the selection
        return 4.0 * (lvl - N) * H + 4.0 * (w.L - 1) * w.k * H
    if stage == "index":           # read the selection; write order and slots of S entries
        return 4.0 * (w.L - 1) * w.k * H + 8.0 * S * H
    if stage == "gather":          # read the gathered rows once; write the fp16 operands (Q, K, V rows;
        # K, V transposed) and the lo parts: fp32 inputs as fp16 (Q, K), bf16 as e4m3 tiles beside
        # e4m3 copies of K and V
        return sub * s_io * 3.0 + sub * 2.0 * 5 + (sub * 3.0 if w.dtype_name == "bf16" else sub * 2.0 * 2)
    if stage == "scatter":         # read O_sub, write O
        return sub * 4.0 + N * d * H * s_io
    if stage == "scatter_bwd":     # read dO, write dO_sub
        return N * d * H * s_io + sub * 4.0
    if stage == "bwd_prep":        # read dO_sub, O_sub and the LSE; write dO_sub's fp16 hi part, its lo
        # part (fp32 inputs: fp16; bf16: an e4m3 tile), delta and LSE - 15
        return sub * 8.0 + sub * 2.0 + (sub * 1.0 if w.dtype_name == "bf16" else sub * 2.0) + 12.0 * S * H
    if stage == "pool_bwd":        # read dQ/dK/dV_sub, write dq, dk, dv
        return sub * 4.0 * 3 + 3.0 * N * d * H * s_io
    raise KeyError(stage)


class Hip:
    """HIP event helpers (the runtime torch already loaded)."""

    def __init__(self):
        import torch
        path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.lib = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def events(self, n):
        out = (ctypes.c_void_p * n)()
        for i in range(n):
            e = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out[i] = e.value
        return out

    def elapsed(self, a, b) -> float:
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def cpu_baseline(q, k, v, dout, w, min_seconds=10.0):
    """The CPU oracle, as it stands, on the same inputs (forward + backward),
    head after head until at least min_seconds of work (or every head);
    scaled to the whole workload by the share of heads run."""
    import threadpoolctl
    import oracle

    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    heads, dt = 0, 0.0
    while heads < w.H and dt < min_seconds:
        qh, kh, vh, dh = (x[heads].float().cpu().numpy() for x in (q, k, v, dout))
        t0 = time.perf_counter()
        ref = oracle.forward(qh, kh, vh, w.L, w.p, w.k)
        oracle.backward(ref, dh, w.p)
        dt += time.perf_counter() - t0
        del ref
        heads += 1
    try:
        host = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        host = os.cpu_count() or 1
    return {"value": w.N * heads / (dt * w.H), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "heads 0-%d of %d (forward + backward, %.1f s of oracle time), scaled by the share of heads"
                      % (heads - 1, w.H, dt),
            "host_cores": host,
            "threads": "cores = the BLAS threads of the oracle's matrix products; its per-entry scatter, "
                       "scatter-adjoint and pool-adjoint loops run on one thread"}


def load_traffic(stage: str, workload: str):
    """HBM bytes per launch of `stage` from committed rocprofv3 counter runs,
    if they were taken on the kernel source that is built now; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (stage, workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from sparse_long_context_lh_amd.build import source_digest
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("bytes_per_launch")


def summarize_stats(d: str) -> None:
    """Markdown table of a rocprofv3 --stats run: per stage of the path, the
    kernels, their launches and average duration."""
    import csv
    path = os.path.join(d, "run_kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    print("| stage | kernel | calls | avg us | total ms |")
    print("|---|---|---:|---:|---:|")
    for r in rows:
        st = stage_of(r["Name"])
        if st is None:
            continue
        print("| %s | `%s` | %s | %.1f | %.2f |" % (st, r["Name"].replace("void ", "")[:70], r["Calls"],
                                                 float(r["AverageNs"]) / 1e3, float(r["TotalDurationNs"]) / 1e6))


def summarize_traffic(fetch_dir: str, write_dir: str, workload: str) -> None:
    """Per-stage HBM bytes per step from two counter runs (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch), scaled by the calibration kernel's known
    1 GiB read and write; writes profiles/traffic_<stage>_<workload>.json."""
    import csv
    import re
    from collections import defaultdict
    from sparse_long_context_lh_amd.build import source_digest

    def per_stage(d, counter):
        tot, calls, calib = defaultdict(float), defaultdict(set), []
        for r in csv.DictReader(open(os.path.join(d, "run_counter_collection.csv"))):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"]) * 1024.0
            if re.search(CALIB_PATTERN, r["Kernel_Name"]):
                calib.append(v)
                continue
            st = stage_of(r["Kernel_Name"])
            if st is not None:
                tot[st] += v
                calls[(st, r["Kernel_Name"])].add(r["Dispatch_Id"])
        if not calib:
            raise SystemExit("no calibration kernel in %s (run bench.py with --copy-calibration)" % d)
        # launches of each stage = launches of its least launched kernel (every
        # kernel of a stage runs at least once per step; the per-level kernels
        # of the front pass run several times at deep pyramids)
        n = {}
        for (st, _), ids in calls.items():
            n[st] = min(n.get(st, len(ids)), len(ids))
        scale = CALIB_BYTES / (sum(calib) / len(calib))
        return {st: tot[st] / n[st] * scale for st in tot}, scale

    fetch, fs = per_stage(fetch_dir, "FETCH_SIZE")
    write, wsc = per_stage(write_dir, "WRITE_SIZE")
    digest = source_digest()
    print("calibration: FETCH_SIZE x %.4f, WRITE_SIZE x %.4f" % (fs, wsc))
    print("| stage | read MB / step | written MB / step | total MB |")
    print("|---|---:|---:|---:|")
    for st in sorted(fetch, key=lambda x: -(fetch[x] + write.get(x, 0.0))):
        total = fetch[st] + write.get(st, 0.0)
        print("| %s | %.1f | %.1f | %.1f |" % (st, fetch[st] / 1e6, write.get(st, 0.0) / 1e6, total / 1e6))
        rec = {"stage": st, "workload": workload, "bytes_per_launch": round(total), "read_bytes": round(fetch[st]),
               "written_bytes": round(write.get(st, 0.0)), "fetch_scale": fs, "write_scale": wsc,
               "source_digest": digest}
        with open(os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (st, workload)), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")


def measure(lh, hip, w0, steps, warmup, backward=True, nograd=False):
    """Time `steps` calls of the layer on workload w0 (forward + backward, or
    forward alone; nograd: lh_forward_nograd, the forward no backward follows)
    after `warmup` untimed ones; per-stage times from the HIP events the
    library records between its kernels on the launch stream."""
    import torch
    from synth_inputs import make_dout, make_qkv

    class W:  # workload fields used by algorithmic()
        pass
    w = W()
    w.N, w.H, w.d, w.L, w.p, w.k = w0.N, w0.H, w0.d, w0.L, w0.p, w0.k
    w.dtype_name = "bf16" if w0.dtype == torch.bfloat16 else "fp32"
    q, k, v = make_qkv(w.N, w.H, w.d, w0.dtype, w0.n_plant, seed=0, device="cuda")
    dout = make_dout(w.N, w.H, w.d, w0.dtype, seed=1, device="cuda") if backward else None
    S = lh.subseq_len(w.N, w.L, w.p, w.k)
    ws = lh.alloc_workspace(w.N, w.H, w.d, w.L, w.p, w.k, w0.dtype, forward_only=not backward)
    out = torch.empty_like(q)
    grads = tuple(torch.empty_like(q) for _ in range(3)) if backward else None
    stream = torch.cuda.current_stream()

    assert not (backward and nograd)
    fwd = lh.forward_nograd if nograd else lh.forward

    def step(evf=None, evb=None):
        fwd(q, k, v, w.L, w.p, w.k, ws=ws, out=out, stream=stream, events=evf)
        if backward:
            lh.backward(dout, w.L, w.p, w.k, ws, *grads, stream=stream, events=evb)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    fnames, bnames = lh.stage_names(False), (lh.stage_names(True) if backward else [])
    evf = [hip.events(len(fnames) + 1) for _ in range(steps)]
    evb = [hip.events(len(bnames) + 1) for _ in range(steps)] if backward else [None] * steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evf[i], evb[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage_ms = {}
    for names, evs in ((fnames, evf), (bnames, evb)):
        for j, name in enumerate(names):
            stage_ms[name] = sum(hip.elapsed(e[j], e[j + 1]) for e in evs) / steps
    fwd_ms = sum(hip.elapsed(e[0], e[len(fnames)]) for e in evf) / steps
    bwd_ms = sum(hip.elapsed(e[0], e[len(bnames)]) for e in evb) / steps if backward else 0.0
    for e in evf + (evb if backward else []):
        hip.destroy(e)

    stages = {}
    for name, ms in stage_ms.items():
        a = algorithmic(name, w, S) / (ms / 1000.0) if ms > 0 else 0.0
        if name in MFMA_STAGES:
            f = mfma_factor(name, w.dtype_name, nograd, ds_tiles_kept(w, S))
            stages[name] = {"ms": round(ms, 4), "TFLOP/s": round(a / 1e12, 1), "frac": round(a / 1e12 / MFMA_F16_PEAK_TFS, 4),
                            "executed_TFLOP/s": round(a * f / 1e12, 1), "mfma_factor": f}
        else:
            stages[name] = {"ms": round(ms, 4), "GB/s": round(a / 1e9, 1), "frac": round(a / 1e9 / HBM_PEAK_GBS, 4)}
    dom = max(stage_ms, key=stage_ms.get)
    work = algorithmic(dom, w, S)
    sec = stage_ms[dom] / 1000.0
    if dom in MFMA_STAGES:
        achieved, peak, unit, bound = work / sec / 1e12, MFMA_F16_PEAK_TFS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = work / sec / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    res = {"w": w, "S": S, "ms_per_step": wall * 1000.0 / steps, "fwd_ms": fwd_ms, "bwd_ms": bwd_ms,
           "stages": stages,
           "roofline": {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                        "frac": round(achieved / peak, 4), "traffic": load_traffic(dom, w0.name)},
           "inputs": (q, k, v, dout)}
    del ws, out, grads
    return res


def summary(r, steps, warmup, backward):
    """The record of one extra workload in the JSON line."""
    w = r["w"]
    d = {"N": w.N, "H": w.H, "d": w.d, "L": w.L, "p": w.p, "k": w.k, "S": r["S"], "steps": steps, "warmup": warmup,
         "fwd_ms": round(r["fwd_ms"], 4), "fwd_tokens_per_s": round(w.N / (r["fwd_ms"] / 1000.0), 1),
         "roofline": r["roofline"]}
    if backward:
        d.update({"fwdbwd_ms": round(r["ms_per_step"], 4),
                  "fwdbwd_tokens_per_s": round(w.N / (r["ms_per_step"] / 1000.0), 1),
                  "bwd_ms": round(r["bwd_ms"], 4)})
    return d


def measure_ceilings():
    """What library kernels reach on this GPU right now, as context for the
    roofline fractions (which are taken against the datasheet peaks): an fp16
    GEMM of 8192^3 (torch.mm, hipBLASLt) under sustained load, where the chip
    lowers its clock, and a 2 GiB device copy and read (torch). torch's own
    stream and events time torch's own kernels."""
    import torch

    def timed(fn, n):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n  # ms

    out = {}
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.float16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.float16)
    c = torch.empty_like(a)
    ms = timed(lambda: torch.mm(a, b, out=c), 20)
    out["gemm_fp16_8192_tflops"] = round(2.0 * 8192 ** 3 / (ms / 1e3) / 1e12, 1)
    del a, b, c
    src = torch.ones(1 << 29, device="cuda", dtype=torch.float32)  # 2 GiB
    dst = torch.empty_like(src)
    nbytes = src.numel() * 4
    out["copy_2gib_gbs"] = round(2.0 * nbytes / (timed(lambda: dst.copy_(src), 5) / 1e3) / 1e9, 1)
    out["read_2gib_gbs"] = round(nbytes / (timed(lambda: src.sum(), 5) / 1e3) / 1e9, 1)
    del src, dst
    out["note"] = "copy counts bytes read + written; roofline fractions are against the datasheet peaks"
    return out


def measure_layer(lh, steps=3, warmup=1, d_model=2048):
    """The step around the layer at the headline shape (N = 512K, H = 16,
    d = 128, L = 5, p = 4, k = 512): Q/K/V projections of x [N, d_model] by
    W [d_model, 3 H d] (rocBLAS), the layer, and the backward to x and W;
    wall time of `steps` calls after `warmup`, bracketed by synchronisations."""
    import torch
    from synth_inputs import make_dout, make_layer_inputs, by_name
    w = by_name("lh-fwdbwd-512k")
    x, W = make_layer_inputs(w.N, d_model, w.H, w.d, w.dtype, w.n_plant, seed=0, device="cuda")
    dout = make_dout(w.N, w.H, w.d, w.dtype, seed=1, device="cuda")
    n = lh.layer_workspace_bytes(w.N, w.H, w.d, d_model, w.L, w.p, w.k, w.dtype)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out = torch.empty(w.H, w.N, w.d, dtype=w.dtype, device="cuda")
    dx, dW = torch.empty_like(x), torch.empty_like(W)

    def fwd():
        lh.layer_forward(x, W, w.H, w.d, w.L, w.p, w.k, ws=ws, out=out)

    def bwd():
        lh.layer_backward(x, W, dout, w.H, w.d, w.L, w.p, w.k, ws, dx=dx, dw=dW)

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    t_f = (time.perf_counter() - t0) / steps
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
        bwd()
    torch.cuda.synchronize()
    t_fb = (time.perf_counter() - t0) / steps
    gemm_fwd = 2.0 * w.N * d_model * 3 * w.H * w.d  # x W
    del ws, x, W, dout, out, dx, dW
    return {"N": w.N, "H": w.H, "d": w.d, "d_model": d_model, "L": w.L, "p": w.p, "k": w.k, "steps": steps,
            "warmup": warmup, "fwd_ms": round(t_f * 1e3, 3), "fwd_tokens_per_s": round(w.N / t_f, 1),
            "fwdbwd_ms": round(t_fb * 1e3, 3), "fwdbwd_tokens_per_s": round(w.N / t_fb, 1),
            "gemm_tflop_fwd": round(gemm_fwd / 1e12, 2), "gemm_tflop_fwdbwd": round(3 * gemm_fwd / 1e12, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lh-fwdbwd-512k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--nograd", action="store_true",
                    help="forward workloads: time lh_forward_nograd (the forward no backward follows)")
    ap.add_argument("--no-extra", action="store_true",
                    help="time the headline workload only (no other sizes, no dense denominator)")
    ap.add_argument("--sweep", action="store_true",
                    help="time the (L, p, k) sweep at 512K tokens instead: one JSON line per shape")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 1 GiB read + 1 GiB write elementwise kernel before the warmup")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.summarize_stats:
        summarize_stats(args.summarize_stats)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, workload=args.workload)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer here has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_long_context_lh_amd as lh
    from synth_inputs import by_name

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.full((CALIB_BYTES // 4,), 7, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    hip = Hip()
    if args.sweep:
        from synth_inputs import SWEEP_WORKLOADS
        for w0 in SWEEP_WORKLOADS:
            r = measure(lh, hip, w0, args.steps, args.warmup, backward=True)
            r.pop("inputs")
            rec = {"workload": w0.name, **summary(r, args.steps, args.warmup, True),
                   "ds_tiles": ds_tiles_kept(r["w"], r["S"]),
                   "stages_ms": {n: x["ms"] for n, x in r["stages"].items()}}
            print(json.dumps(rec), flush=True)
            torch.cuda.empty_cache()
        return
    w0 = by_name(args.workload)
    if args.nograd and w0.backward:
        raise SystemExit("--nograd applies to forward workloads")
    head = measure(lh, hip, w0, args.steps, args.warmup, backward=w0.backward, nograd=args.nograd)
    w = head["w"]
    res = {
        "metric": METRIC,
        "value": round(w.N / (head["ms_per_step"] / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w0.dtype == torch.bfloat16 else "fp32",
        "data": "synthetic",
        "config": {"workload": w0.name, "N": w.N, "H": w.H, "d": w.d, "L": w.L, "p": w.p, "k": w.k, "S": head["S"],
                   "step": "forward+backward" if w0.backward else ("forward (nograd)" if args.nograd else "forward"),
                   "parallelism": "none (1 GPU)"},
        "fwd_tokens_per_s": round(w.N / (head["fwd_ms"] / 1000.0), 1),
        "fwd_ms": round(head["fwd_ms"], 4),
        "bwd_ms": round(head["bwd_ms"], 4),
        "roofline": head["roofline"],
        "stages": head["stages"],
    }
    if not args.no_extra and w0.backward:
        # the forward alone, as a call no backward follows (lh_forward_nograd)
        r = measure(lh, hip, w0, args.steps, args.warmup, backward=False, nograd=True)
        r.pop("inputs")
        res["nograd_fwd_ms"] = round(r["fwd_ms"], 4)
        res["nograd_fwd_tokens_per_s"] = round(w.N / (r["fwd_ms"] / 1000.0), 1)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        q, k, v, dout = head["inputs"]
        res["cpu_baseline"] = cpu_baseline(q, k, v, dout, w)
    head.pop("inputs")
    torch.cuda.empty_cache()
    if not args.no_extra and w0.name == "lh-fwdbwd-512k":
        # the rest of the metric's range (1M forward + backward, 128K and 64K
        # forward), then dense causal attention over the same 512K tokens: the
        # denominator of the layer's speedup
        extra = {}
        for name, steps, warm, bwd in (("lh-fwdbwd-1m", 5, 2, True), ("lh-fwd-128k", 5, 2, False),
                                       ("lh-fwd-64k", 5, 2, False)):
            r = measure(lh, hip, by_name(name), steps, warm, backward=bwd)
            r.pop("inputs")
            extra[name] = summary(r, steps, warm, bwd)
            torch.cuda.empty_cache()
            if not bwd:  # and as a call no backward follows
                r = measure(lh, hip, by_name(name), steps, warm, backward=False, nograd=True)
                r.pop("inputs")
                extra[name]["nograd"] = summary(r, steps, warm, False)
                torch.cuda.empty_cache()
        res["workloads"] = extra
        r = measure(lh, hip, by_name("dense-fwdbwd-512k"), 1, 1, backward=True)
        r.pop("inputs")
        dense = summary(r, 1, 1, True)
        dense["speedup_fwd"] = round(r["fwd_ms"] / head["fwd_ms"], 2)
        dense["speedup_fwdbwd"] = round(r["ms_per_step"] / head["ms_per_step"], 2)
        res["dense_512k"] = dense
        torch.cuda.empty_cache()
        lay = measure_layer(lh)
        # the projections' share: the step minus the layer's own step above
        g_f = lay["fwd_ms"] - head["fwd_ms"]
        g_fb = lay["fwdbwd_ms"] - head["ms_per_step"]
        lay["gemm_ms_fwd"] = round(g_f, 3)
        lay["gemm_ms_fwdbwd"] = round(g_fb, 3)
        lay["gemm_tflops_fwdbwd"] = round(lay["gemm_tflop_fwdbwd"] / (g_fb / 1e3), 1) if g_fb > 0 else None
        res["projection_layer_512k"] = lay
        torch.cuda.empty_cache()
        res["ceilings"] = measure_ceilings()
        torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
