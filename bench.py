"""Throughput of the Lighthouse layer (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--copy-calibration]
    python bench.py --summarize-stats DIR              (rocprofv3 --stats output -> markdown)
    python bench.py --summarize-traffic FETCH_DIR WRITE_DIR [--workload NAME]

A step is one lh_forward + lh_backward over the whole workload (every stage
of the path, all heads), inputs resident in HBM. The default workload is the
512K-token forward + backward shape (H=16, d=128, L=5, p=4, k=512, S=10240),
the single-layer setting at which the layer's forward and forward+backward
speedups are quoted. Prints one JSON line.

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
    (r"lh::k_front(_up)?<", "front"),
    (r"lh::k_topk\(", "topk"),
    (r"lh::k_index\(", "index"),
    (r"lh::k_(gather<|lo8<\d+, 0>)", "gather"),
    (r"lh::k_attn_fwd<", "attn_fwd"),
    (r"lh::k_pull<\d+, [^,]+, 1, 1,", "scatter"),
    (r"lh::k_scatter_bwd(_up)?<", "scatter_bwd"),
    (r"lh::k_(bwd_prep<|lo8<\d+, 1>)", "bwd_prep"),
    (r"lh::k_attn_bwd_dkdv<", "attn_bwd_dkdv"),
    (r"lh::k_attn_bwd_dq<", "attn_bwd_dq"),
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
    if stage == "attn_bwd_dq":     # dQ: one causal product
        return 1.0 * S * S * d * H
    if stage == "front":           # read Q, K, V; write the score pyramid
        return 3.0 * N * d * H * s_io + 4.0 * lvl * H
    if stage == "topk":            # read levels 1.. of the scores; write the selection
        return 4.0 * (lvl - N) * H + 4.0 * (w.L - 1) * w.k * H
    if stage == "index":           # read the selection; write order and slots of S entries
        return 4.0 * (w.L - 1) * w.k * H + 8.0 * S * H
    if stage == "gather":          # read the gathered rows once, write the fp16 operands
        return sub * s_io * 3.0 + sub * 2.0 * 8
    if stage == "scatter":         # read O_sub, write O
        return sub * 4.0 + N * d * H * s_io
    if stage == "scatter_bwd":     # read dO, write dO_sub
        return N * d * H * s_io + sub * 4.0
    if stage == "bwd_prep":        # read dO_sub and O_sub, write the fp16 operands
        return sub * 8.0 + sub * 2.0 * 3
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
    return {"value": w.N * heads / (dt * w.H), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": "heads 0-%d of %d (forward + backward, %.1f s of oracle time), scaled by the share of heads"
                      % (heads - 1, w.H, dt)}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lh-fwdbwd-512k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    from synth_inputs import by_name, make_dout, make_qkv

    w0 = by_name(args.workload)

    class W:  # workload fields used by algorithmic()
        pass
    w = W()
    w.N, w.H, w.d, w.L, w.p, w.k = w0.N, w0.H, w0.d, w0.L, w0.p, w0.k
    w.dtype_name = "bf16" if w0.dtype == torch.bfloat16 else "fp32"
    torch.cuda.set_device(0)
    dev = "cuda"
    q, k, v = make_qkv(w.N, w.H, w.d, w0.dtype, w0.n_plant, seed=0, device=dev)
    dout = make_dout(w.N, w.H, w.d, w0.dtype, seed=1, device=dev)
    S = lh.subseq_len(w.N, w.L, w.p, w.k)
    ws = lh.alloc_workspace(w.N, w.H, w.d, w.L, w.p, w.k, w0.dtype)
    out = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(evf=None, evb=None):
        lh.forward(q, k, v, w.L, w.p, w.k, ws=ws, out=out, stream=stream, events=evf)
        lh.backward(dout, w.L, w.p, w.k, ws, dq, dk, dv, stream=stream, events=evb)

    if args.copy_calibration:
        src = torch.full((CALIB_BYTES // 4,), 7, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hip = Hip()
    fnames, bnames = lh.stage_names(False), lh.stage_names(True)
    evf = [hip.events(len(fnames) + 1) for _ in range(args.steps)]
    evb = [hip.events(len(bnames) + 1) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evf[i], evb[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage_ms = {}
    for names, evs in ((fnames, evf), (bnames, evb)):
        for j, name in enumerate(names):
            stage_ms[name] = sum(hip.elapsed(e[j], e[j + 1]) for e in evs) / args.steps
    fwd_ms = sum(hip.elapsed(e[0], e[len(fnames)]) for e in evf) / args.steps
    bwd_ms = sum(hip.elapsed(e[0], e[len(bnames)]) for e in evb) / args.steps
    for e in evf + evb:
        hip.destroy(e)

    ms_per_step = wall * 1000.0 / args.steps
    dom = max(stage_ms, key=stage_ms.get)
    work = algorithmic(dom, w, S)
    sec = stage_ms[dom] / 1000.0
    if dom in MFMA_STAGES:
        achieved, peak, unit, bound = work / sec / 1e12, MFMA_F16_PEAK_TFS, "TFLOP/s", "mfma"
    else:
        achieved, peak, unit, bound = work / sec / 1e9, HBM_PEAK_GBS, "GB/s", "hbm"
    stages = {}
    for name, ms in stage_ms.items():
        a = algorithmic(name, w, S) / (ms / 1000.0) if ms > 0 else 0.0
        if name in MFMA_STAGES:
            stages[name] = {"ms": round(ms, 4), "TFLOP/s": round(a / 1e12, 1), "frac": round(a / 1e12 / MFMA_F16_PEAK_TFS, 4)}
        else:
            stages[name] = {"ms": round(ms, 4), "GB/s": round(a / 1e9, 1), "frac": round(a / 1e9 / HBM_PEAK_GBS, 4)}

    res = {
        "metric": METRIC,
        "value": round(w.N / (ms_per_step / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w0.name, "N": w.N, "H": w.H, "d": w.d, "L": w.L, "p": w.p, "k": w.k, "S": S,
                   "step": "forward+backward", "parallelism": "none (1 GPU)"},
        "fwd_tokens_per_s": round(w.N / (fwd_ms / 1000.0), 1),
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "roofline": {"kernel": dom, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": load_traffic(dom, w0.name)},
        "stages": stages,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(q, k, v, dout, w)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
