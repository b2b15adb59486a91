"""Throughput of the block-scaled FP4 quantize-dequantize path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path over the fp32 4096 x 4096
block-size-sweep workload (the numerical study of "Finer is Better (with the
Right Scaling)": N(0,1) and Laplace(0,1) tensors, each also scaled by 1e-4):
  * 128 fp4q_quantize calls: 4 tensors x block {4, 8, 16, 32} x
    {abs-max, prevent-zero, 4-over-6, brute force} x {tensor-amax, none},
    every output (packed codes, E4M3 scales, fp32 dequant, block MSE);
  * block-wise Hadamard rotation fused into quantization (H = 16 NVFP4,
    H = 32 MXFP4) on the N(0,1) tensor;
  * FOCUS relaxed fake-quant forward (+ codes) and STE backward on the
    N(0,1) tensor (MXFP4 and NVFP4, sub-blocks of 8, fp16 c ~ U[0.8, 1.25],
    upstream gradient N(0,1));
  * stand-alone dequantize and block MSE of one NVFP4 result.
Calls cycle through the four tensors so consecutive calls touch different
256 MB of data (the 256 MB last-level cache cannot serve a whole tensor from
one call to the next).

All inputs are generated once and are resident in HBM before timing; every
output buffer is preallocated; the timed region holds only library calls.
value = algorithmic bytes of the step (each input read once, each output
written once) / step time.  Per-call HIP events over the timed steps give
the per-strategy rates and the roofline of the dominant kernel.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E, published
VALU_PEAK_TOPS = 256 * 128 * 2.4e9 / 1e12   # 256 CUs x 128 fp32 lanes/clock x 2.4 GHz = 157.3 TFLOP/s / 2
BF_INSTR_PER_EVAL = 13.25                   # VALU instructions of one candidate-element evaluation (B=16 loop)
BF_CANDIDATES = 126                         # positive finite E4M3 scales an exhaustive search evaluates
CSRC = os.path.join(ROOT, "microscaling_fp4_block_fp4q_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

STRATS = {0: "absmax", 1: "prevent-zero", 2: "4-over-6", 3: "brute-force"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements outside the step (scale search, UE5M3, histogram, GEMM)")
    ap.add_argument("--cpu-rows", type=int, default=48, help="rows per tensor in the oracle sample")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--calls-out", default=None, help="write every call's mean time (ms) and bytes to this file")
    ap.add_argument("--summarize", nargs="+", default=None, metavar="DIR",
                    help="summarise rocprofv3 csv output directories into --label under profiles/ and exit")
    ap.add_argument("--label", default=None)
    ap.add_argument("--command", default="", help="the command that produced the --summarize directories")
    ap.add_argument("--only", default=None,
                    help="profiling mode: run only the calls whose name contains one of these "
                         "'|'-separated texts, --steps times, and print no result line")
    ap.add_argument("--profile-gemm", action="store_true",
                    help="profiling mode: run only the 8192^3 MXFP4 GEMM, --steps times, and print no result line")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="profiling mode: also run a device-to-device copy of this many MiB "
                         "(calibrates the HBM byte counters)")
    return ap.parse_args()


class Call:
    """One preallocated library call of the step."""

    def __init__(self, name, fn, args, nbytes, elems, kind, meta):
        self.name, self.fn, self.args = name, fn, args
        self.nbytes, self.elems, self.kind, self.meta = nbytes, elems, kind, meta
        self.times = []

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError(f"{self.name}: status {st}")


GEMM_SOURCES = ("gemm.hip",)


def source_digest(gemm: bool = False) -> str:
    """sha256 over the HIP sources and headers (ties counter profiles to a
    kernel version): the GEMM's own source for gemm=True, else every other
    one (the quantize path)."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".hpp")) and (f in GEMM_SOURCES) == gemm:
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def summarize(dirs, label, command):
    """Aggregate rocprofv3 csv output (kernel stats and counter collections)
    into profiles/<label>.json (numbers) and profiles/<label>.md (table)."""
    import csv
    import glob
    gemm = "gemm" in label
    out = {"label": label, "command": command, "source_digest": source_digest(gemm), "kernels": {}, "counters": {}}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                out["kernels"][r["Name"]] = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                                             "min_us": float(r["MinNs"]) / 1e3,
                                             "total_ms": float(r["TotalDurationNs"]) / 1e6,
                                             "percent": float(r["Percentage"])}
        # The trace splits each kernel's dispatches by whether the abs-max
        # pre-pass ran right before it (TENSOR_AMAX calls) or not; the bench's
        # roofline averages the launches without it.
        for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
            trace = sorted(csv.DictReader(open(f)), key=lambda r: int(r["Start_Timestamp"]))
            split, prev = {}, ""
            for r in trace:
                us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                key = "after_amax" if "k_amax" in prev else "without_amax"
                split.setdefault(r["Kernel_Name"], {"without_amax": [], "after_amax": []})[key].append(us)
                prev = r["Kernel_Name"]
            for k, v in split.items():
                out.setdefault("split", {})[k] = {
                    key: {"dispatches": len(ds), "avg_us": sum(ds) / len(ds)} for key, ds in v.items() if ds}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            acc = {}
            for r in csv.DictReader(open(f)):
                acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            for k, cs in acc.items():
                dst = out["counters"].setdefault(k, {})
                for c, v in cs.items():
                    dst[c] = {"mean": sum(v) / len(v), "dispatches": len(v)}
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, label + ".json"), "w") as f:
        json.dump(out, f, indent=1)
    lines = [f"# {label}", "", f"Command: `{command}`", "", f"Kernel sources digest: `{out['source_digest']}`", ""]
    if out["kernels"]:
        lines += ["| kernel | calls | avg us | min us | total ms | % |", "|---|---|---|---|---|---|"]
        for k, v in sorted(out["kernels"].items(), key=lambda kv: -kv[1]["total_ms"])[:25]:
            lines.append(f"| `{k[:90]}` | {v['calls']} | {v['avg_us']:.2f} | {v['min_us']:.2f} | "
                         f"{v['total_ms']:.3f} | {v['percent']:.2f} |")
        lines.append("")
    if out.get("split") and out["kernels"]:
        lines += ["Dispatches split by whether the abs-max pre-pass ran right before them (from the kernel trace):", "",
                  "| kernel | without pre-pass: dispatches | avg us | after pre-pass: dispatches | avg us |",
                  "|---|---|---|---|---|"]
        top = [k for k, _ in sorted(out["kernels"].items(), key=lambda kv: -kv[1]["total_ms"])[:25]]
        for k in top:
            v = out["split"].get(k, {})
            a, b = v.get("without_amax"), v.get("after_amax")
            if not a or not b:
                continue
            lines.append(f"| `{k[:90]}` | {a['dispatches']} | {a['avg_us']:.2f} | {b['dispatches']} | {b['avg_us']:.2f} |")
        lines.append("")
    if out["counters"]:
        lines += ["| kernel | counter | mean per dispatch | dispatches |", "|---|---|---|---|"]
        for k, cs in out["counters"].items():
            for c, v in sorted(cs.items()):
                lines.append(f"| `{k[:90]}` | {c} | {v['mean']:.1f} | {v['dispatches']} |")
    with open(os.path.join(PROFILES, label + ".md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote profiles/{label}.json and .md")


def dominant_profile(kernel_name: str):
    """Counters of kernel_name from the committed profile, or None when the
    profile is missing or was taken on other kernel sources."""
    path = os.path.join(PROFILES, "counters_bench_dominant.json")
    if not os.path.exists(path):
        return None
    prof = json.load(open(path))
    if prof.get("source_digest") != source_digest():
        return None
    return next((v for k, v in prof["counters"].items() if kernel_name in k), None)


def counter_traffic(kernel_name: str):
    """HBM bytes per launch of kernel_name from the committed counter profile,
    scaled by a plain copy of known size; None if the profile is missing or
    was taken on other kernel sources."""
    path = os.path.join(PROFILES, "counters_bench_dominant.json")
    if not os.path.exists(path):
        return None
    prof = json.load(open(path))
    if prof.get("source_digest") != source_digest():
        return None
    cnt = prof["counters"]
    copy = next((v for k, v in cnt.items() if "copyBuffer" in k), None)
    kern = next((v for k, v in cnt.items() if kernel_name in k), None)
    if not copy or not kern or "FETCH_SIZE" not in kern or "WRITE_SIZE" not in kern:
        return None
    copy_kib = prof.get("copy_mib", 256) * 1024.0
    f_scale = copy_kib / copy["FETCH_SIZE"]["mean"]
    w_scale = copy_kib / copy["WRITE_SIZE"]["mean"]
    return 1024.0 * (kern["FETCH_SIZE"]["mean"] * f_scale + kern["WRITE_SIZE"]["mean"] * w_scale)


def gemm_profile():
    """The committed kernel-stat and counter profiles of the 8192^3 GEMM, if
    they were taken on the current GEMM source."""
    out = {}
    for label in ("kernel_stats_mxfp4_gemm_8192", "counters_mxfp4_gemm_8192"):
        path = os.path.join(PROFILES, label + ".json")
        if not os.path.exists(path):
            continue
        prof = json.load(open(path))
        if prof.get("source_digest") != source_digest(gemm=True):
            continue
        for k, v in prof.get("kernels", {}).items():
            if "k_mxfp4_gemm" in k:
                out["avg_kernel_us"] = v["avg_us"]
            elif "shuffle_scales" in k:
                out["avg_shuffle_us"] = v["avg_us"]
        for k, cs in prof.get("counters", {}).items():
            if "k_mxfp4_gemm" in k:
                out.update({c: v["mean"] for c, v in cs.items()})
            elif "copyBuffer" in k:
                out.update({"copy_" + c: v["mean"] for c, v in cs.items()})
        if "copy_mib" in prof:
            out["copy_mib"] = prof["copy_mib"]
    return out


def quant_bytes(rows, cols, B, in_es=4, dq_es=4, mse=True, dq=True):
    n = rows * cols
    return n * in_es + n // 2 + n // B + (n * dq_es if dq else 0) + (4 * n // B if mse else 0)


def build_step(F, S, torch, dev):
    """Generate the workload on the host, upload it, preallocate every output."""
    L = F.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    host = S.config2()
    names = ["normal", "laplace", "normal_1e-4", "laplace_1e-4"]
    R, C = host["normal"].shape
    X = {k: S.to_torch(host[k], S.F32, dev) for k in names}
    keep = list(X.values())                      # keep tensors and configs alive

    def t_empty(shape, dtype):
        t = torch.empty(shape, dtype=dtype, device=dev)
        keep.append(t)
        return t

    def ptr(t):
        return ctypes.c_void_p(t.data_ptr()) if t is not None else None

    calls = []
    combos = [(B, st, gm) for B in (4, 8, 16, 32) for st in (0, 1, 2, 3) for gm in (1, 0)]
    for ci, (B, st, gm) in enumerate(combos):
        for ti in range(4):
            tname = names[(ti + ci) % 4]       # every combo on all four tensors, rotated per combo
            x = X[tname]
            cfg = F.config(F.E4M3, B, st, gm)
            keep.append(cfg)
            codes = t_empty((R, C // 2), torch.uint8)
            scales = t_empty((R, C // B), torch.uint8)
            g = t_empty((1,), torch.float32)
            dq = t_empty((R, C), torch.float32)
            mse = t_empty((R, C // B), torch.float32)
            ws = t_empty((max(F.workspace_bytes(cfg, R, C), 16),), torch.uint8)
            args = (ctypes.byref(cfg), ptr(x), F.F32, R, C, C, ptr(codes), ptr(scales), ptr(g), ptr(dq),
                    F.F32, C, ptr(mse), ptr(ws), stream)
            calls.append(Call(f"quantize B={B} {STRATS[st]} {'amax' if gm else 'none'}", L.fp4q_quantize, args,
                              quant_bytes(R, C, B), R * C, "quantize",
                              dict(B=B, strategy=STRATS[st], global_mode="tensor-amax" if gm else "none",
                                   tensor=tname)))

    xn = X["normal"]
    # block Hadamard fused before quantization
    for H, cfg in ((16, F.nvfp4(0, hadamard=16)), (32, F.mxfp4(0, hadamard=32))):
        keep.append(cfg)
        codes = t_empty((R, C // 2), torch.uint8)
        scales = t_empty((R, C // cfg.block), torch.uint8)
        g = t_empty((1,), torch.float32)
        dq = t_empty((R, C), torch.float32)
        mse = t_empty((R, C // cfg.block), torch.float32)
        ws = t_empty((max(F.workspace_bytes(cfg, R, C), 16),), torch.uint8)
        args = (ctypes.byref(cfg), ptr(xn), F.F32, R, C, C, ptr(codes), ptr(scales), ptr(g), ptr(dq), F.F32, C,
                ptr(mse), ptr(ws), stream)
        calls.append(Call(f"quantize hadamard={H} {'nvfp4' if H == 16 else 'mxfp4'}", L.fp4q_quantize, args,
                          quant_bytes(R, C, cfg.block), R * C, "rotate+quantize", dict(H=H)))
        if H == 16:
            nv_codes, nv_scales, nv_g, nv_cfg = codes, scales, g, cfg

    # stand-alone dequantize and block MSE of the NVFP4 (rotated) result
    out = t_empty((R, C), torch.float32)
    calls.append(Call("dequantize nvfp4", L.fp4q_dequantize,
                      (ctypes.byref(nv_cfg), ptr(nv_codes), ptr(nv_scales), ptr(nv_g), R, C, ptr(out), F.F32, C, stream),
                      R * C // 2 + R * C // 16 + 4 * R * C, R * C, "dequantize", {}))
    mse = t_empty((R, C // 16), torch.float32)
    calls.append(Call("block_mse nvfp4", L.fp4q_block_mse,
                      (ctypes.byref(nv_cfg), ptr(xn), F.F32, R, C, C, ptr(nv_codes), ptr(nv_scales), ptr(nv_g),
                       ptr(mse), stream),
                      4 * R * C + R * C // 2 + R * C // 16 + 4 * R * C // 16, R * C, "block_mse", {}))

    # FOCUS relaxed fake-quant forward / backward, sub-blocks of 8
    K = 8
    rng = np.random.default_rng(7)
    c16 = S.cast(rng.uniform(0.8, 1.25, (R, C // K)), S.F16)
    ct = S.to_torch(c16, S.F16, dev)
    gt = S.to_torch(S.normal(R, C, 8, S.F32), S.F32, dev)
    keep += [ct, gt]
    for cfg in (F.mxfp4(), F.nvfp4(0, F.GLOBAL_USER, 2.0 ** -12)):
        keep.append(cfg)
        B = cfg.block
        scales = t_empty((R, C // B), torch.uint8)
        gq = t_empty((1,), torch.float32)
        codes = t_empty((R, C // 2), torch.uint8)
        ws = t_empty((16,), torch.uint8)
        # S_dq from abs-max quantization (outside the timed step)
        st = L.fp4q_quantize(ctypes.byref(cfg), ptr(xn), F.F32, R, C, C, ptr(codes), ptr(scales), ptr(gq),
                             None, F.F32, C, None, ptr(ws), stream)
        assert st == 0, st
        g_in = None if cfg.scale_fmt == F.E8M0 else gq
        w_hat = t_empty((R, C), torch.float32)
        fcodes = t_empty((R, C // 2), torch.uint8)
        grad_c = t_empty((R, C // K), torch.float32)
        fmt = "mxfp4" if B == 32 else "nvfp4"
        calls.append(Call(f"focus fwd {fmt}", L.fp4q_relaxed_fakequant_fwd,
                          (ctypes.byref(cfg), ptr(xn), F.F32, R, C, C, ptr(scales), ptr(g_in), ptr(ct), K,
                           ptr(w_hat), F.F32, C, ptr(fcodes), stream),
                          4 * R * C + 2 * R * C // K + R * C // B + 4 * R * C + R * C // 2, R * C, "focus_fwd", {}))
        calls.append(Call(f"focus bwd {fmt}", L.fp4q_relaxed_fakequant_bwd,
                          (ctypes.byref(cfg), ptr(xn), F.F32, R, C, C, ptr(scales), ptr(g_in), ptr(ct), K, ptr(gt),
                           F.F32, C, ptr(grad_c), stream),
                          8 * R * C + 2 * R * C // K + R * C // B + 4 * R * C // K, R * C, "focus_bwd", {}))
    torch.cuda.synchronize()
    return calls, keep, host, X


def time_quantize_configs(F, torch, x, cfgs, reps=5):
    """Quantize calls outside the step (widenings of the path): each config on
    one 4096 x 4096 fp32 input with every output, timed per call with HIP
    events on the library's stream; GB/s of the call's algorithmic bytes."""
    L = F.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    R, C = x.shape
    out = {}
    for name, cfg in cfgs:
        B = cfg.block
        codes = torch.empty((R, C // 2), dtype=torch.uint8, device=x.device)
        scales = torch.empty((R, C // B), dtype=torch.uint8, device=x.device)
        g = torch.empty(1, dtype=torch.float32, device=x.device)
        dq = torch.empty((R, C), dtype=torch.float32, device=x.device)
        mse = torch.empty((R, C // B), dtype=torch.float32, device=x.device)
        ws = torch.empty(max(F.workspace_bytes(cfg, R, C), 16), dtype=torch.uint8, device=x.device)
        args = (ctypes.byref(cfg), ctypes.c_void_p(x.data_ptr()), F.F32, R, C, C, ctypes.c_void_p(codes.data_ptr()),
                ctypes.c_void_p(scales.data_ptr()), ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(dq.data_ptr()),
                F.F32, C, ctypes.c_void_p(mse.data_ptr()), ctypes.c_void_p(ws.data_ptr()), stream)
        ev = []
        for i in range(reps + 1):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            st_ = L.fp4q_quantize(*args)
            e1.record()
            if st_ != 0:
                raise RuntimeError(f"{name}: status {st_}")
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev[1:]]))
        nb = quant_bytes(R, C, B)
        out[name] = {"ms": round(ms, 4), "GB/s": round(nb / (ms * 1e6), 1),
                     "Gelem/s": round(R * C / (ms * 1e6), 2), "g": float(g.item())}
    return out


def time_histogram(F, torch, x, reps=10):
    """Codebook-occupancy histogram (outside the step) of the NVFP4 codes of
    one 4096 x 4096 input: HBM-bound over rows * cols / 2 code bytes."""
    L = F.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    R, C = x.shape
    codes = F.quantize(x, F.config(F.E4M3, 16, F.ABSMAX, F.GLOBAL_NONE), want_mse=False)["codes"]
    counts = torch.zeros(16, dtype=torch.int64, device=x.device)
    ev = []
    for _ in range(reps + 1):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        st_ = L.fp4q_code_histogram(ctypes.c_void_p(codes.data_ptr()), R, C, ctypes.c_void_p(counts.data_ptr()),
                                    stream)
        e1.record()
        if st_ != 0:
            raise RuntimeError(f"histogram: status {st_}")
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev[1:]]))
    h = counts.cpu().numpy() / (reps + 1)                 # the calls accumulate
    return {"ms": round(ms, 4), "GB/s": round(R * C / 2 / (ms * 1e6), 1),
            "zero_code_fraction": round(float(h[0] + h[8]) / (R * C), 4),
            "what": "not part of the step: counts of the 16 nibble codes of the NVFP4 (block 16, no per-tensor "
                    "scale) codes of the 4096x4096 N(0,1) input, 8 MiB of code bytes"}


MFMA_FP4_PEAK_TFLOPS = 10100.0              # MI355X dense FP4 matrix peak, published


def time_gemm(F, torch, dev, warm=30, reps=10, rounds=3):
    """MXFP4 GEMM (outside the step): C = dq(A) dq(B)^T with A the MXFP4
    quantization of N(0,1) activations [tokens, in] and B that of N(0, 0.02^2)
    weights [out, in], bf16 C.  Each call also rearranges both scale tensors
    for the matrix cores.  Mean over rounds x reps calls after a warm-up, HIP
    events on the library's stream; 2 M N K flops per call."""
    out = {}
    gen = torch.Generator(device=dev).manual_seed(11)
    for M, N, K in ((8192, 8192, 8192), (8192, 14336, 4096), (8192, 4096, 14336)):
        qa = F.quantize(torch.randn((M, K), generator=gen, device=dev), F.mxfp4(), want_mse=False)
        qb = F.quantize(torch.randn((N, K), generator=gen, device=dev) * 0.02, F.mxfp4(), want_mse=False)
        c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = F.gemm_workspace(M, N, K, dev)
        args = (qa["codes"], qa["scales"], qb["codes"], qb["scales"], c, ws)
        for _ in range(warm):
            F.fp4q_mxfp4_gemm(*args)
        ev = []
        for _ in range(rounds * reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            F.fp4q_mxfp4_gemm(*args)
            e1.record()
            ev.append((e0, e1))
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out[f"{M}x{N}x{K}"] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                               "mfma_frac": round(tf / MFMA_FP4_PEAK_TFLOPS, 4)}
        if M == N == K == 8192:
            alg = M * K // 2 + N * K // 2 + (M + N) * K // 32 + M * N * 2
            prof = gemm_profile()
            roof = {"bound": "mfma", "kernel": "k_mxfp4_gemm<0> (+ 2 k_gemm_shuffle_scales)",
                    "achieved": round(tf, 1), "peak": MFMA_FP4_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / MFMA_FP4_PEAK_TFLOPS, 4), "avg_launch_ms": round(ms, 4),
                    "algorithmic_MB_per_launch": round(alg / 1e6, 2), "traffic": None}
            if "avg_kernel_us" in prof:
                roof["profile_kernel_only_us"] = prof["avg_kernel_us"]
                roof["profile_shuffle_us"] = prof.get("avg_shuffle_us")
            if "FETCH_SIZE" in prof and "WRITE_SIZE" in prof and "copy_FETCH_SIZE" in prof:
                kib = prof.get("copy_mib", 256) * 1024.0
                t = 1024.0 * (prof["FETCH_SIZE"] * kib / prof["copy_FETCH_SIZE"] +
                              prof["WRITE_SIZE"] * kib / prof["copy_WRITE_SIZE"])
                roof["traffic"] = round(t / 1e6, 2)
                roof["traffic_unit"] = "MB per launch of the GEMM kernel (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
            if "SQ_VALU_MFMA_BUSY_CYCLES" in prof and "GRBM_GUI_ACTIVE" in prof:
                # busy cycles summed over the 1024 SIMDs; GRBM_GUI_ACTIVE summed over the 8 XCDs
                roof["mfma_busy_frac"] = round(prof["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 /
                                               (prof["GRBM_GUI_ACTIVE"] / 8), 4)
            out["roofline_8192"] = roof
        del qa, qb, c, ws, args
    out["peak"] = {"TFLOP/s": MFMA_FP4_PEAK_TFLOPS, "what": "MI355X dense FP4 matrix-core peak"}
    out["what"] = ("not part of the step: MXFP4 GEMM (M x N x K) of MXFP4-quantized N(0,1) activations and "
                   "N(0,0.02^2) weights on the block-scaled 32x32x64 matrix cores, bf16 output, including the "
                   "per-call scale rearrangement; mean of 30 calls after 30 warm-up calls")
    return out


def cpu_baseline(O, S, host, rows_per_tensor):
    """The oracle (single thread) on the first rows of every tensor, over the
    same call list as one GPU step."""
    names = ["normal", "laplace", "normal_1e-4", "laplace_1e-4"]
    nbytes = 0
    t0 = time.perf_counter()
    for B in (4, 8, 16, 32):
        for st in (0, 1, 2, 3):
            for gm in (1, 0):
                for name in names:
                    x = np.ascontiguousarray(host[name][:rows_per_tensor])
                    O.quantize(x, fmt=1, block=B, strategy=st, global_mode=gm)
                    nbytes += quant_bytes(x.shape[0], x.shape[1], B)
    x = np.ascontiguousarray(host["normal"][:rows_per_tensor])
    r, c = x.shape
    for H, fmt, B, gm in ((16, 1, 16, 1), (32, 0, 32, 0)):
        q = O.quantize(x, fmt=fmt, block=B, strategy=0, global_mode=gm, hadamard=H)
        nbytes += quant_bytes(r, c, B)
    O.dequantize(q["codes"], q["scales"], 1.0, fmt=0, block=32, rows=r, cols=c)
    nbytes += r * c // 2 + r * c // 32 + 4 * r * c
    O.block_mse(x, q["codes"], q["scales"], 1.0, fmt=0, block=32, hadamard=32)
    nbytes += 4 * r * c + r * c // 2 + r * c // 32 + 4 * r * c // 32
    c16 = S.cast(np.random.default_rng(7).uniform(0.8, 1.25, (r, c // 8)), S.F16)
    gr = S.normal(r, c, 8, S.F32)
    for fmt, B, g in ((0, 32, 1.0), (1, 16, 2.0 ** -12)):
        q = O.quantize(x, fmt=fmt, block=B, strategy=0, global_mode=2 if fmt else 0, user_g=g, dq_dt=None)
        O.relaxed_fwd(x, q["scales"], g, c16, fmt=fmt, block=B, sub_block=8)
        O.relaxed_bwd(x, q["scales"], g, c16, gr, fmt=fmt, block=B, sub_block=8)
        nbytes += 8 * r * c + r * c // 4 + r * c // B + r * c // 2
        nbytes += 8 * r * c + r * c // 4 + r * c // B + r * c // 2
    dt = time.perf_counter() - t0
    return nbytes, dt


def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.label or "profile", args.command)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path has no multi-GPU "
              "code: each GPU would quantize its own row shard independently).", file=sys.stderr)
        sys.exit(2)

    import torch

    from microscaling_fp4_block_fp4q_amd import fp4q as F
    from microscaling_fp4_block_fp4q_amd import synth as S

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile_gemm:
        gen = torch.Generator(device=dev).manual_seed(11)
        M = N = K = 8192
        qa = F.quantize(torch.randn((M, K), generator=gen, device=dev), F.mxfp4(), want_mse=False)
        qb = F.quantize(torch.randn((N, K), generator=gen, device=dev) * 0.02, F.mxfp4(), want_mse=False)
        c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = F.gemm_workspace(M, N, K, dev)
        torch.cuda.synchronize()
        if args.copy_mb:
            src = torch.empty(args.copy_mb << 18, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            src.fill_(1.0)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            F.fp4q_mxfp4_gemm(qa["codes"], qa["scales"], qb["codes"], qb["scales"], c, ws)
            if args.copy_mb:
                dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] profiling run done", file=sys.stderr, flush=True)
        return
    print("[bench] generating and uploading the workload", file=sys.stderr, flush=True)
    calls, keep, host, X = build_step(F, S, torch, dev)
    step_bytes = sum(c.nbytes for c in calls)

    def step(record=False):
        for c in calls:
            if record:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                c()
                e1.record()
                c.times.append((e0, e1))
            else:
                c()

    if args.only is not None or args.copy_mb:
        pats = [] if args.only is None else args.only.split("|")
        sel = [c for c in calls if any(pt in c.name for pt in pats)]
        print(f"[bench] profiling {len(sel)} calls x {args.steps}: {[c.name for c in sel][:4]}", file=sys.stderr,
              flush=True)
        if args.copy_mb:
            src = torch.empty(args.copy_mb << 18, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            src.fill_(1.0)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            for c in sel:
                c()
            if args.copy_mb:
                dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] profiling run done", file=sys.stderr, flush=True)
        return

    print(f"[bench] {len(calls)} calls per step, warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps bracketed by device synchronisation
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(record=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    per_call = []
    for c in calls:
        ms = float(np.mean([a.elapsed_time(b) for a, b in c.times]))
        per_call.append((c, ms))

    # per-strategy aggregates (quantize calls)
    groups = {}
    for c, ms in per_call:
        key = c.meta.get("strategy", c.kind)
        g = groups.setdefault(key, [0, 0, 0.0])
        g[0] += c.nbytes
        g[1] += c.elems
        g[2] += ms
    breakdown = {k: {"GB/s": round(b / (ms * 1e6), 1), "Gelem/s": round(e / (ms * 1e6), 2),
                     "hbm_frac": round(b / (ms * 1e6) / HBM_PEAK_GBS, 4), "ms_per_step": round(ms, 4)}
                 for k, (b, e, ms) in groups.items()}

    # dominant kernel: the kernel family (strategy, block) with the largest share of the step
    fam = {}
    for c, ms in per_call:
        key = (c.meta.get("strategy", c.kind), c.meta.get("B"))
        fam.setdefault(key, []).append((c, ms))
    dom_key = max(fam, key=lambda k: sum(ms for _, ms in fam[k]))
    dom = fam[dom_key]
    solo = [(c, ms) for c, ms in dom if c.meta.get("global_mode") != "tensor-amax"] or dom
    dom_ms = float(np.mean([ms for _, ms in solo]))    # launches without the abs-max pre-pass
    dom_elems = dom[0][0].elems
    strategy, B = dom_key
    if strategy == "brute-force":
        kname = f"k_quant_bf<float, {B}, 0, 1>"
        work = BF_CANDIDATES * BF_INSTR_PER_EVAL * dom_elems          # exhaustive-search VALU work per launch
        achieved = work / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "alu", "kernel": kname, "achieved": round(achieved, 2),
                    "peak": round(VALU_PEAK_TOPS, 1), "unit": "T VALU instr/s",
                    "frac": round(achieved / VALU_PEAK_TOPS, 4),
                    "work_per_launch": f"{BF_CANDIDATES} candidates x {BF_INSTR_PER_EVAL} VALU instructions x "
                                       f"{dom_elems} elements (the exhaustive search; the exact branch and bound "
                                       "evaluates a fraction of the candidates, so frac > 1 is pruning)",
                    "avg_launch_ms": round(dom_ms, 4)}
        prof = dominant_profile(kname)
        if prof and "SQ_INSTS_VALU" in prof:
            executed = prof["SQ_INSTS_VALU"]["mean"] * 64            # lane-instructions actually issued
            roofline["executed_valu_instr_per_launch"] = round(executed)
            roofline["executed_valu_frac"] = round(executed / (dom_ms * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4)
    else:
        kname = f"k_quant<float, {B}" if B else dom[0][0].kind
        nbytes = dom[0][0].nbytes
        achieved = nbytes / (dom_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "avg_launch_ms": round(dom_ms, 4)}
    traffic = counter_traffic(kname)
    roofline["traffic"] = None if traffic is None else round(traffic / 1e6, 2)
    roofline["traffic_unit"] = "MB per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    roofline["algorithmic_MB_per_launch"] = round(dom[0][0].nbytes / 1e6, 2)
    # the practical HBM ceiling of this access pattern: device copies of the same
    # four 64 MiB inputs, in the same rotation, into four 64 MiB buffers
    names = list(X)
    dsts = [torch.empty_like(X[n]) for n in names]
    copy_ms = []
    for i in range(32 + 4):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        dsts[(i + 1) % 4].copy_(X[names[i % 4]])
        e1.record()
        copy_ms.append((e0, e1))
    torch.cuda.synchronize()
    cms = float(np.mean([a.elapsed_time(b) for a, b in copy_ms[4:]]))
    copy_gbs = 2 * X[names[0]].numel() * 4 / (cms * 1e6)
    del dsts
    for k, v in breakdown.items():
        v["frac_of_copy"] = round(v["GB/s"] / copy_gbs, 4)
    if args.no_extras:
        search = ue5m3 = hist = gemm = {"what": "not measured (--no-extras)"}
    else:
        search = time_quantize_configs(F, torch, X["normal"], [
            ("absmax", F.config(F.E4M3, 16, F.ABSMAX, F.GLOBAL_SEARCH)),
            ("4-over-6", F.config(F.E4M3, 16, F.FOUR_OVER_SIX, F.GLOBAL_SEARCH)),
            ("brute-force", F.config(F.E4M3, 16, F.BRUTE_FORCE, F.GLOBAL_SEARCH))])
        ue5m3 = time_quantize_configs(F, torch, X["normal"], [
            (f"B={B} {STRATS[st]}", F.config(F.UE5M3, B, st)) for B in (16, 4) for st in (0, 2, 3)])
        hist = time_histogram(F, torch, X["normal"])
        gemm = time_gemm(F, torch, dev)
    stream_quant = [(c, ms) for c, ms in per_call if c.meta.get("strategy") in ("absmax", "4-over-6")]
    sb = sum(c.nbytes for c, _ in stream_quant)
    sms = sum(ms for _, ms in stream_quant)

    result = {
        "metric": "FP4 quantize+dequant GB/s and Gelem/s per strategy; % of HBM/VALU peak",
        "value": round(step_bytes / (ms_per_step * 1e6), 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "fp32 4096x4096 N(0,1) and Laplace(0,1), each also x1e-4; E4M3-scaled FP4, "
                               "block 4/8/16/32 x {abs-max, prevent-zero, 4-over-6, brute-force} x "
                               "{tensor-amax, none}, all outputs; + block-Hadamard 16/32 fused quantize, "
                               "FOCUS fwd/bwd (sub-block 8), dequantize, block MSE",
                   "calls_per_step": len(calls), "algorithmic_bytes_per_step": step_bytes},
        "roofline": roofline,
        "streaming_absmax_4over6": {"GB/s": round(sb / (sms * 1e6), 1),
                                    "hbm_frac": round(sb / (sms * 1e6) / HBM_PEAK_GBS, 4),
                                    "frac_of_copy": round(sb / (sms * 1e6) / copy_gbs, 4)},
        "per_strategy": breakdown,
        "global_scale_search": dict({"what": "not part of the step: NVFP4 block 16 quantize of the 4096x4096 "
                                             "N(0,1) input with the per-tensor scale searched over 32 "
                                             "candidates (abs-max pre-pass, 32-candidate scoring, tree "
                                             "reduction, pick, quantize at the winner); GB/s of the "
                                             "quantize call's algorithmic bytes"}, **search),
        "ue5m3_scales": dict({"what": "not part of the step: quantize of the 4096x4096 N(0,1) input with "
                                      "UE5M3 block scales (no per-tensor scale), every output"}, **ue5m3),
        "code_histogram": hist,
        "mxfp4_gemm": gemm,
        "copy_reference": {"GB/s": round(copy_gbs, 1), "hbm_frac": round(copy_gbs / HBM_PEAK_GBS, 4),
                           "what": "device copy (read + write bytes) of the four 64 MiB inputs in rotation, "
                                   "the same access pattern as the quantize calls; per_strategy frac_of_copy "
                                   "is GB/s relative to it"},
    }

    if not args.no_cpu_baseline:
        from oracle import oracle as O
        O.build()
        print(f"[bench] oracle on {args.cpu_rows} rows per tensor (1 thread)", file=sys.stderr, flush=True)
        nb, dt = cpu_baseline(O, S, host, args.cpu_rows)
        result["cpu_baseline"] = {"value": round(nb / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                                  "sample": f"the step's call list on the first {args.cpu_rows} rows of each "
                                            f"4096x4096 tensor ({nb / 1e6:.1f} MB algorithmic, {dt:.1f} s)"}
    if args.calls_out:
        with open(args.calls_out, "w") as f:
            json.dump([{"name": c.name, "tensor": c.meta.get("tensor"), "ms": ms, "bytes": c.nbytes}
                       for c, ms in per_call], f, indent=0)
    line = json.dumps(result)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")
    per = sorted(per_call, key=lambda t: -t[1])
    for c, ms in per[:12]:
        print(f"[bench] {c.name:40s} {ms:9.4f} ms  {c.nbytes / (ms * 1e6):8.1f} GB/s", file=sys.stderr)


if __name__ == "__main__":
    main()
