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
written once) / step time.  Inside the timed steps HIP events bracket only
the launches of the dominant kernel family (found in the warm-up), whose
live launch times give the roofline; the per-strategy rates come from the
same steps run again afterwards with every call bracketed by events.  A
cold leg times every call once more with the caches flushed before it
(1 GiB of reads on the same stream, outside the events).

Beside the step, the other workloads are timed per call, warm and cold:
fp32 1024 x 1024 (launch-bound, reported only), the Llama-3.1-8B-shaped
bf16 MLP weights, bf16 8192 x 4096 activations with the fused rotation, and
the bf16 4096 x 12288 FOCUS fake-quant.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0                       # MI355X HBM3E, published
# fp32 vector peak: 256 CUs x 128 fp32 lanes/clock x 2.4 GHz = 78.6 T lane-instructions/s
# (the published 157.3 TFLOP/s counts an FMA as two flops)
VALU_PEAK_TOPS = 256 * 128 * 2.4e9 / 1e12
BF_INSTR_PER_EVAL = 13.25                   # VALU instructions of one candidate-element evaluation (B=16 loop)
BF_CANDIDATES = 126                         # positive finite E4M3 scales an exhaustive search evaluates
CSRC = os.path.join(ROOT, "microscaling_fp4_block_fp4q_amd", "csrc")
PROBE_LIB = os.path.join(ROOT, "microscaling_fp4_block_fp4q_amd", "libfp4q_probe.so")
PROFILES = os.path.join(ROOT, "profiles")
FLUSH_MIB = 1024                            # the cold leg reads 1 GiB before each call

STRATS = {0: "absmax", 1: "prevent-zero", 2: "4-over-6", 3: "brute-force"}
VALU_PROBES = {0: "v_add_f32", 1: "v_mul_f32", 2: "v_fma_f32", 3: "integer add/xor/shift",
               4: "fp32 min/max/add", 5: "brute-force candidate evaluation (block of 16)",
               6: "brute-force candidate evaluation, rounding by the FP4 pair converts"}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the measurements outside the step (scale search, UE5M3, histogram, GEMM)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-config lines of the other workloads (C1, C3, C4, C5)")
    ap.add_argument("--cpu-rows", type=int, default=48, help="rows per tensor in the oracle sample")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--calls-out", default=None, help="write every call's mean time (ms) and bytes to this file")
    ap.add_argument("--summarize", nargs="+", default=None, metavar="DIR",
                    help="summarise rocprofv3 csv output directories into --label under profiles/ and exit")
    ap.add_argument("--label", default=None)
    ap.add_argument("--command", default="", help="the command that produced the --summarize directories")
    ap.add_argument("--probe-json", default=None,
                    help="with --summarize: the --probe result line whose VALU probe times the counters divide")
    ap.add_argument("--only", default=None,
                    help="profiling mode: run only the calls whose name contains one of these "
                         "'|'-separated texts, --steps times, and print no result line")
    ap.add_argument("--configs-only", default=None,
                    help="profiling mode: run only the per-config calls whose name contains one of these "
                         "'|'-separated texts, --steps times, and print no result line")
    ap.add_argument("--profile-gemm", action="store_true",
                    help="profiling mode: run only the 8192^3 MXFP4 GEMM, --steps times, and print no result line")
    ap.add_argument("--probe", action="store_true",
                    help="run the HBM stream and VALU rate probes, print their JSON line and exit")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="profiling mode: also run a device-to-device copy of this many MiB "
                         "(calibrates the HBM byte counters)")
    return ap.parse_args(argv)


class Call:
    """One preallocated library call."""

    def __init__(self, name, fn, args, nbytes, elems, kind, meta):
        self.name, self.fn, self.args = name, fn, args
        self.nbytes, self.elems, self.kind, self.meta = nbytes, elems, kind, meta
        self.times = []
        self.cold = []

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


def summarize(dirs, label, command, probe_json=None):
    """Aggregate rocprofv3 csv output (kernel stats and counter collections)
    into profiles/<label>.json (numbers) and profiles/<label>.md (table).
    With probe_json (the line bench.py --probe printed in the same command),
    the VALU probes' executed lane-instruction rates are derived: SQ_INSTS_VALU
    x 64 per dispatch over the probe's mean launch time."""
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
        # pre-pass ran right before it (TENSOR_AMAX calls) or not.
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
            rows = list(csv.DictReader(open(f)))
            key_of = (lambda r: int(r["Dispatch_Id"])) if rows and "Dispatch_Id" in rows[0] else None
            if key_of:
                rows.sort(key=key_of)
            acc = {}
            for r in rows:
                acc.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            for k, cs in acc.items():
                dst = out["counters"].setdefault(k, {})
                for c, v in cs.items():
                    dst[c] = {"mean": sum(v) / len(v), "dispatches": len(v), "values": v}
    rate_lines = []
    if probe_json:
        probe = json.loads(open(probe_json).read().strip().splitlines()[-1])
        out["probe"] = probe
        out["rates"] = {}
        rate_lines = ["VALU probes: executed lane-instructions (SQ_INSTS_VALU x 64) over the mean launch time "
                      "(HIP events, same command):", "",
                      "| probe | lanes | ms | SQ_INSTS_VALU per dispatch | T lane-instr/s | of 78.6 T |",
                      "|---|---|---|---|---|---|"]
        for name, v in probe["valu"].items():
            kc = next((c for k, c in out["counters"].items() if f"k_valu<{v['kind']}>" in k), None)
            if not kc or "SQ_INSTS_VALU" not in kc:
                continue
            ins = kc["SQ_INSTS_VALU"]["mean"]
            rate = ins * 64 / (v["ms"] * 1e-3) / 1e12
            out["rates"][name] = round(rate, 2)
            rate_lines.append(f"| {name} | {v['lanes']} | {v['ms']:.4f} | {ins:.0f} | {rate:.2f} | "
                              f"{rate / VALU_PEAK_TOPS:.3f} |")
        rate_lines += ["", "HBM stream probes (same command):", "", "| stream | GB/s | of 8 TB/s | workgroups |",
                       "|---|---|---|---|"]
        for name, v in probe["hbm"].items():
            rate_lines.append(f"| {name} | {v['GB/s']} | {v['hbm_frac']} | {v['workgroups']} |")
        rate_lines.append("")
    os.makedirs(PROFILES, exist_ok=True)
    with open(os.path.join(PROFILES, label + ".json"), "w") as f:
        json.dump(out, f, indent=1)
    lines = [f"# {label}", "", f"Command: `{command}`", "", f"Kernel sources digest: `{out['source_digest']}`", ""]
    lines += rate_lines
    if out["kernels"]:
        lines += ["| kernel | calls | avg us | min us | total ms | % |", "|---|---|---|---|---|---|"]
        for k, v in sorted(out["kernels"].items(), key=lambda kv: -kv[1]["total_ms"])[:30]:
            lines.append(f"| `{k[:90]}` | {v['calls']} | {v['avg_us']:.2f} | {v['min_us']:.2f} | "
                         f"{v['total_ms']:.3f} | {v['percent']:.2f} |")
        lines.append("")
    if out.get("split") and out["kernels"]:
        lines += ["Dispatches split by whether the abs-max pre-pass ran right before them (from the kernel trace):", "",
                  "| kernel | without pre-pass: dispatches | avg us | after pre-pass: dispatches | avg us |",
                  "|---|---|---|---|---|"]
        top = [k for k, _ in sorted(out["kernels"].items(), key=lambda kv: -kv[1]["total_ms"])[:30]]
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


def load_profile(label: str, gemm: bool = False):
    """A committed profile summary, or None when it is missing or was taken
    on other kernel sources."""
    path = os.path.join(PROFILES, label + ".json")
    if not os.path.exists(path):
        return None
    prof = json.load(open(path))
    if prof.get("source_digest") != source_digest(gemm):
        return None
    return prof


def kernel_counters(prof, kernel_name: str):
    if not prof:
        return None
    return next((v for k, v in prof["counters"].items() if kernel_name in k), None)


def copy_scaled_traffic(prof, kern):
    """HBM bytes per dispatch (list) of a kernel's FETCH_SIZE / WRITE_SIZE
    counters, scaled by what the same counters read for a plain device copy
    of known size in the same runs; None without both."""
    cnt = prof["counters"] if prof else {}
    copy = next((v for k, v in cnt.items() if "copyBuffer" in k or "k_copy" in k), None)
    if not copy or not kern or "FETCH_SIZE" not in kern or "WRITE_SIZE" not in kern:
        return None
    copy_kib = prof.get("copy_mib", 256) * 1024.0
    f_scale = copy_kib / copy["FETCH_SIZE"]["mean"]
    w_scale = copy_kib / copy["WRITE_SIZE"]["mean"]
    fs, ws = kern["FETCH_SIZE"].get("values"), kern["WRITE_SIZE"].get("values")
    if not fs or not ws or len(fs) != len(ws):
        fs, ws = [kern["FETCH_SIZE"]["mean"]], [kern["WRITE_SIZE"]["mean"]]
    return [1024.0 * (f * f_scale + w * w_scale) for f, w in zip(fs, ws)]


def gemm_profile():
    """The committed kernel-stat and counter profiles of the 8192^3 GEMM, if
    they were taken on the current GEMM source."""
    out = {}
    for label in ("kernel_stats_mxfp4_gemm_8192", "counters_mxfp4_gemm_8192"):
        prof = load_profile(label, gemm=True)
        if not prof:
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


# --------------------------------------------------------------------------
# probes: HBM streams and VALU issue rates (libfp4q_probe.so)
# --------------------------------------------------------------------------

_probe = None


def probe_lib():
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError(f"{PROBE_LIB} is missing: build it with `python -m microscaling_fp4_block_fp4q_amd.build`")
        L = ctypes.CDLL(PROBE_LIB)
        L.fp4q_probe_stream.restype = ctypes.c_int
        L.fp4q_probe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_void_p]
        L.fp4q_probe_valu.restype = ctypes.c_int
        L.fp4q_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        _probe = L
    return _probe


def cu_count(torch):
    return torch.cuda.get_device_properties(0).multi_processor_count


class Flusher:
    """Evicts L2 and the last-level cache without leaving dirty lines behind:
    a read of 1 GiB (8 loads in flight per lane) on the library's stream."""

    def __init__(self, torch, dev):
        self.src = torch.ones(FLUSH_MIB << 18, dtype=torch.float32, device=dev)
        self.grid = 8 * cu_count(torch)
        self.dst = torch.empty(self.grid * 256, dtype=torch.int32, device=dev)
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def __call__(self):
        st = probe_lib().fp4q_probe_stream(4, ctypes.c_void_p(self.src.data_ptr()), ctypes.c_void_p(self.dst.data_ptr()),
                                           self.src.numel() // 4, self.grid, self.stream)
        if st != 0:
            raise RuntimeError("cache flush read failed")


def events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def time_fn(torch, fn, reps, flush=None):
    """Mean ms of fn over reps calls, each bracketed by HIP events on the
    current stream (after one untimed call); with flush, the caches are
    flushed before every call, outside the events."""
    fn()
    ev = []
    for _ in range(reps):
        if flush:
            flush()
        e0, e1 = events(torch)
        e0.record()
        fn()
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev]))


def run_probes(torch, dev, reps=10):
    """HBM stream ceilings (read, write, copy: 1 GiB cold, and the step's
    access pattern of four 64 MiB tensors in rotation) and VALU issue rates."""
    L = probe_lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cus = cu_count(torch)
    out = {"hbm": {}, "valu": {}}
    n = 1 << 30
    a = torch.ones(n // 4, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    small = torch.empty(64 * cus * 256, dtype=torch.int32, device=dev)
    flush = Flusher(torch, dev)

    def stream_call(kind, src, dst, nbytes, grid):
        def fn():
            if L.fp4q_probe_stream(kind, ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                                   nbytes // 16, grid, stream) != 0:
                raise RuntimeError("probe stream failed")
        return fn

    for name, kind, moved in (("read, 4 loads in flight", 0, 1), ("read, 8 loads in flight", 4, 1),
                              ("read, 16 loads in flight", 5, 1), ("read, 8 non-temporal loads in flight", 6, 1),
                              ("write (streaming stores)", 1, 1), ("write (plain stores)", 7, 1),
                              ("copy (streaming stores)", 2, 2), ("copy (streaming stores, 8 loads in flight)", 8, 2),
                              ("copy (plain stores)", 3, 2)):
        best = None
        for wpc in (4, 8, 16, 32):
            grid = wpc * cus
            dst = small if kind in (0, 4, 5, 6) else b
            ms = time_fn(torch, stream_call(kind, a, dst, n, grid), reps, flush)
            gbs = moved * n / (ms * 1e6)
            if best is None or gbs > best["GB/s"]:
                best = {"GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "ms": round(ms, 4),
                        "workgroups": grid}
        out["hbm"][f"{name}, 1 GiB, cold"] = best
    # the step's pattern: four 64 MiB inputs in rotation, copied into four outputs
    xs = [torch.ones(16 << 20, dtype=torch.float32, device=dev) for _ in range(4)]
    ys = [torch.empty_like(x) for x in xs]
    grid = 8 * cus
    ev = []
    for i in range(36):
        e0, e1 = events(torch)
        e0.record()
        if L.fp4q_probe_stream(2, ctypes.c_void_p(xs[i % 4].data_ptr()), ctypes.c_void_p(ys[(i + 1) % 4].data_ptr()),
                               (64 << 20) // 16, grid, stream) != 0:
            raise RuntimeError("probe stream failed")
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    ms = float(np.mean([p.elapsed_time(q) for p, q in ev[4:]]))
    gbs = 2 * (64 << 20) / (ms * 1e6)
    out["hbm"]["copy (streaming stores), four 64 MiB tensors in rotation, warm"] = {
        "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "ms": round(ms, 4), "workgroups": grid}
    del a, b, xs, ys, flush

    o = torch.empty(32 * cus * 256, dtype=torch.float32, device=dev)
    for kind, name in VALU_PROBES.items():
        iters = 4096 if kind < 5 else 1024
        grid = 32 * cus

        def fn(kind=kind, iters=iters, grid=grid):
            if L.fp4q_probe_valu(kind, iters, grid, ctypes.c_void_p(o.data_ptr()), stream) != 0:
                raise RuntimeError("probe valu failed")
        ms = time_fn(torch, fn, reps)
        out["valu"][name] = {"kind": kind, "iters": iters, "workgroups": grid, "ms": round(ms, 5),
                             "lanes": grid * 256}
    return out


# --------------------------------------------------------------------------
# the step: the fp32 4096 x 4096 block-size sweep
# --------------------------------------------------------------------------

class Builder:
    """Preallocated outputs of library calls (kept alive with the inputs)."""

    def __init__(self, F, torch, dev):
        self.F, self.torch, self.dev = F, torch, dev
        self.keep = []
        self.stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def empty(self, shape, dtype):
        t = self.torch.empty(shape, dtype=dtype, device=self.dev)
        self.keep.append(t)
        return t

    @staticmethod
    def ptr(t):
        return ctypes.c_void_p(t.data_ptr()) if t is not None else None

    def quantize_call(self, name, cfg, x, x_dt, kind, meta, dq_dt=None, mse=True):
        """fp4q_quantize of x [R, C] with every requested output preallocated."""
        F, torch = self.F, self.torch
        self.keep.append(cfg)
        R, C = x.shape
        B = cfg.block
        codes = self.empty((R, C // 2), torch.uint8)
        scales = self.empty((R, C // B), torch.uint8)
        g = self.empty((1,), torch.float32)
        dq = None if dq_dt is None else self.empty((R, C), {F.F32: torch.float32, F.BF16: torch.bfloat16}[dq_dt])
        m = self.empty((R, C // B), torch.float32) if mse else None
        ws = self.empty((max(F.workspace_bytes(cfg, R, C), 16),), torch.uint8)
        args = (ctypes.byref(cfg), self.ptr(x), x_dt, R, C, C, self.ptr(codes), self.ptr(scales), self.ptr(g),
                self.ptr(dq), dq_dt if dq_dt is not None else F.F32, C, self.ptr(m), self.ptr(ws), self.stream)
        in_es = 4 if x_dt == F.F32 else 2
        dq_es = 0 if dq_dt is None else (4 if dq_dt == F.F32 else 2)
        nbytes = quant_bytes(R, C, B, in_es, dq_es, mse=mse, dq=dq_dt is not None)
        c = Call(name, F.lib().fp4q_quantize, args, nbytes, R * C, kind, meta)
        c.outputs = dict(codes=codes, scales=scales, g=g)
        return c


def build_step(F, S, torch, dev):
    """Generate the workload on the host, upload it, preallocate every output."""
    L = F.lib()
    bld = Builder(F, torch, dev)
    host = S.config2()
    names = ["normal", "laplace", "normal_1e-4", "laplace_1e-4"]
    R, C = host["normal"].shape
    X = {k: S.to_torch(host[k], S.F32, dev) for k in names}
    bld.keep += list(X.values())
    ptr = bld.ptr

    calls = []
    combos = [(B, st, gm) for B in (4, 8, 16, 32) for st in (0, 1, 2, 3) for gm in (1, 0)]
    for ci, (B, st, gm) in enumerate(combos):
        for ti in range(4):
            tname = names[(ti + ci) % 4]       # every combo on all four tensors, rotated per combo
            cfg = F.config(F.E4M3, B, st, gm)
            calls.append(bld.quantize_call(f"quantize B={B} {STRATS[st]} {'amax' if gm else 'none'}", cfg, X[tname],
                                           F.F32, "quantize",
                                           dict(B=B, strategy=STRATS[st], global_mode="tensor-amax" if gm else "none",
                                                tensor=tname), dq_dt=F.F32))

    xn = X["normal"]
    # block Hadamard fused before quantization
    for H, cfg in ((16, F.nvfp4(0, hadamard=16)), (32, F.mxfp4(0, hadamard=32))):
        c = bld.quantize_call(f"quantize hadamard={H} {'nvfp4' if H == 16 else 'mxfp4'}", cfg, xn, F.F32,
                              "rotate+quantize", dict(H=H), dq_dt=F.F32)
        calls.append(c)
        if H == 16:
            nv, nv_cfg = c.outputs, cfg

    # stand-alone dequantize and block MSE of the NVFP4 (rotated) result
    out = bld.empty((R, C), torch.float32)
    calls.append(Call("dequantize nvfp4", L.fp4q_dequantize,
                      (ctypes.byref(nv_cfg), ptr(nv["codes"]), ptr(nv["scales"]), ptr(nv["g"]), R, C, ptr(out), F.F32,
                       C, bld.stream),
                      R * C // 2 + R * C // 16 + 4 * R * C, R * C, "dequantize", {}))
    mse = bld.empty((R, C // 16), torch.float32)
    calls.append(Call("block_mse nvfp4", L.fp4q_block_mse,
                      (ctypes.byref(nv_cfg), ptr(xn), F.F32, R, C, C, ptr(nv["codes"]), ptr(nv["scales"]),
                       ptr(nv["g"]), ptr(mse), bld.stream),
                      4 * R * C + R * C // 2 + R * C // 16 + 4 * R * C // 16, R * C, "block_mse", {}))

    # FOCUS relaxed fake-quant forward / backward, sub-blocks of 8
    K = 8
    rng = np.random.default_rng(7)
    c16 = S.cast(rng.uniform(0.8, 1.25, (R, C // K)), S.F16)
    ct = S.to_torch(c16, S.F16, dev)
    gt = S.to_torch(S.normal(R, C, 8, S.F32), S.F32, dev)
    bld.keep += [ct, gt]
    for cfg in (F.mxfp4(), F.nvfp4(0, F.GLOBAL_USER, 2.0 ** -12)):
        calls += focus_calls(F, bld, cfg, xn, F.F32, ct, gt, F.F32, K, F.F32, "", codes=True)
    torch.cuda.synchronize()
    return calls, bld, host, X


def focus_calls(F, bld, cfg, w, w_dt, ct, gt, g_dt, K, out_dt, tag, codes=True):
    """FOCUS forward (+ codes) and backward calls with S_dq from an abs-max
    quantization of w (made here, outside any timing)."""
    torch = bld.torch
    L = F.lib()
    ptr = bld.ptr
    bld.keep.append(cfg)
    R, C = w.shape
    B = cfg.block
    scales = bld.empty((R, C // B), torch.uint8)
    gq = bld.empty((1,), torch.float32)
    qc = bld.empty((R, C // 2), torch.uint8)
    ws = bld.empty((max(F.workspace_bytes(cfg, R, C), 16),), torch.uint8)
    st = L.fp4q_quantize(ctypes.byref(cfg), ptr(w), w_dt, R, C, C, ptr(qc), ptr(scales), ptr(gq), None, F.F32, C,
                         None, ptr(ws), bld.stream)
    assert st == 0, st
    g_in = None if cfg.scale_fmt == F.E8M0 else gq
    es = 4 if w_dt == F.F32 else 2
    oes = 4 if out_dt == F.F32 else 2
    w_hat = bld.empty((R, C), torch.float32 if out_dt == F.F32 else torch.bfloat16)
    fcodes = bld.empty((R, C // 2), torch.uint8) if codes else None
    grad_c = bld.empty((R, C // K), torch.float32)
    fmt = "mxfp4" if B == 32 else "nvfp4"
    fwd_bytes = es * R * C + 2 * R * C // K + R * C // B + oes * R * C + (R * C // 2 if codes else 0)
    bwd_bytes = es * R * C + (4 if g_dt == F.F32 else 2) * R * C + 2 * R * C // K + R * C // B + 4 * R * C // K
    return [Call(f"focus fwd {fmt}{tag}", L.fp4q_relaxed_fakequant_fwd,
                 (ctypes.byref(cfg), ptr(w), w_dt, R, C, C, ptr(scales), ptr(g_in), ptr(ct), K,
                  ptr(w_hat), out_dt, C, ptr(fcodes), bld.stream), fwd_bytes, R * C, "focus_fwd", {"fmt": fmt}),
            Call(f"focus bwd {fmt}{tag}", L.fp4q_relaxed_fakequant_bwd,
                 (ctypes.byref(cfg), ptr(w), w_dt, R, C, C, ptr(scales), ptr(g_in), ptr(ct), K, ptr(gt),
                  g_dt, C, ptr(grad_c), bld.stream), bwd_bytes, R * C, "focus_bwd", {"fmt": fmt})]


# --------------------------------------------------------------------------
# the other workloads, per call
# --------------------------------------------------------------------------

def build_configs(F, S, torch, dev):
    """Preallocated calls of the fp32 1024^2, Llama-shaped weight, activation
    and FOCUS workloads: {config label: (description, [calls])}."""
    bld = Builder(F, torch, dev)
    out = {}

    x1 = S.to_torch(S.config1(), S.F32, dev)
    bld.keep.append(x1)
    out["C1"] = ("fp32 1024x1024 N(0,1): MXFP4 and NVFP4 abs-max, every output (launch-bound; reported, not "
                 "judged against the roofline)",
                 [bld.quantize_call("C1 mxfp4 absmax", F.mxfp4(), x1, F.F32, "quantize", {}, dq_dt=F.F32),
                  bld.quantize_call("C1 nvfp4 absmax amax", F.nvfp4(), x1, F.F32, "quantize", {}, dq_dt=F.F32)])

    c3 = S.config3()
    calls = []
    for wname in ("w_down", "w_up"):
        w = S.to_torch(c3[wname], S.BF16, dev)
        bld.keep.append(w)
        shape = "x".join(map(str, w.shape))
        for fname, mk in (("nvfp4 4-over-6 amax", lambda: F.nvfp4(F.FOUR_OVER_SIX)), ("mxfp4 absmax", F.mxfp4)):
            for full in (False, True):
                mode = "full" if full else "packed"
                calls.append(bld.quantize_call(f"C3 {wname} {shape} {fname} {mode}", mk(), w, F.BF16, "quantize",
                                               {"mode": mode}, dq_dt=F.BF16 if full else None, mse=full))
    del c3
    out["C3"] = ("Llama-3.1-8B-shaped bf16 MLP weights (W_down 4096x14336, W_gate/up 14336x4096; 0.02 Student-t "
                 "df=3, 0.5% of columns x20): NVFP4 4-over-6 + tensor-amax and MXFP4 abs-max; packed-only "
                 "(codes + scales) and full (+ bf16 dequant + block MSE)", calls)

    a = S.to_torch(S.config4(), S.BF16, dev)
    bld.keep.append(a)
    calls = []
    acts = (("mxfp4 absmax", lambda H: F.mxfp4(hadamard=H)),
            ("nvfp4 absmax amax", lambda H: F.nvfp4(hadamard=H)),
            ("nvfp4 absmax user-g", lambda H: F.nvfp4(global_mode=F.GLOBAL_USER, global_scale=0.015625, hadamard=H)),
            ("nvfp4 4-over-6 amax", lambda H: F.nvfp4(F.FOUR_OVER_SIX, hadamard=H)))
    for H in (0, 16, 32):
        for fname, mk in acts:
            for full in (False, True):
                mode = "full" if full else "packed"
                calls.append(bld.quantize_call(f"C4 H={H} {fname} {mode}", mk(H), a, F.BF16, "quantize",
                                               {"H": H, "mode": mode}, dq_dt=F.BF16 if full else None, mse=full))
    out["C4"] = ("bf16 activations 8192x4096 (Laplace(0,1), 0.1% of channels x50), block Hadamard H in {0, 16, 32} "
                 "fused before MXFP4 / NVFP4 (tensor-amax pre-pass over the rotated rows, or a user g) quantization; "
                 "packed-only and full outputs", calls)

    K = 8
    w5, c5, g5 = S.config5(K)
    wt, ct, gt = S.to_torch(w5, S.BF16, dev), S.to_torch(c5, S.F16, dev), S.to_torch(g5, S.BF16, dev)
    bld.keep += [wt, ct, gt]
    calls = []
    for cfg in (F.mxfp4(), F.nvfp4()):
        calls += focus_calls(F, bld, cfg, wt, F.BF16, ct, gt, F.BF16, K, F.BF16, "", codes=False)
        calls += focus_calls(F, bld, cfg, wt, F.BF16, ct, gt, F.BF16, K, F.BF16, " +codes", codes=True)[:1]
    out["C5"] = ("FOCUS fake-quant of bf16 4096x12288 N(0,0.02) weights, sub-blocks of 8, fp16 c ~ U[0.8,1.25], "
                 "bf16 upstream gradient N(0,1); S_dq from MXFP4 / NVFP4 abs-max; forward (bf16 W_hat, with and "
                 "without codes) and STE backward (fp32 grad_c)", calls)
    torch.cuda.synchronize()
    return out, bld


def time_configs(torch, configs, flush, reps_warm=10, reps_cold=5):
    res = {}
    for label, (what, calls) in configs.items():
        rows = {}
        tb = tw = tc = 0.0
        for c in calls:
            mw = time_fn(torch, c, reps_warm)
            mc = time_fn(torch, c, reps_cold, flush)
            gw, gc = c.nbytes / (mw * 1e6), c.nbytes / (mc * 1e6)
            rows[c.name] = {"bytes": c.nbytes, "ms_warm": round(mw, 4), "GB/s_warm": round(gw, 1),
                            "hbm_frac_warm": round(gw / HBM_PEAK_GBS, 4), "ms_cold": round(mc, 4),
                            "GB/s_cold": round(gc, 1), "hbm_frac_cold": round(gc / HBM_PEAK_GBS, 4),
                            "Gelem/s_cold": round(c.elems / (mc * 1e6), 2)}
            tb += c.nbytes
            tw += mw
            tc += mc
        res[label] = {"what": what, "GB/s_warm": round(tb / (tw * 1e6), 1),
                      "hbm_frac_warm": round(tb / (tw * 1e6) / HBM_PEAK_GBS, 4),
                      "GB/s_cold": round(tb / (tc * 1e6), 1), "hbm_frac_cold": round(tb / (tc * 1e6) / HBM_PEAK_GBS, 4),
                      "calls": rows}
    return res


def time_quantize_configs(F, torch, x, cfgs, reps=5):
    """Quantize calls outside the step (widenings of the path): each config on
    one 4096 x 4096 fp32 input with every output, timed per call with HIP
    events on the library's stream; GB/s of the call's algorithmic bytes."""
    bld = Builder(F, torch, x.device)
    R, C = x.shape
    out = {}
    for name, cfg in cfgs:
        c = bld.quantize_call(name, cfg, x, F.F32, "quantize", {}, dq_dt=F.F32)
        ms = time_fn(torch, c, reps)
        out[name] = {"ms": round(ms, 4), "GB/s": round(c.nbytes / (ms * 1e6), 1),
                     "Gelem/s": round(R * C / (ms * 1e6), 2), "g": float(c.outputs["g"].item())}
    return out


def time_histogram(F, torch, x, reps=10):
    """Codebook-occupancy histogram (outside the step) of the NVFP4 codes of
    one 4096 x 4096 input: HBM-bound over rows * cols / 2 code bytes."""
    L = F.lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    R, C = x.shape
    codes = F.quantize(x, F.config(F.E4M3, 16, F.ABSMAX, F.GLOBAL_NONE), want_mse=False)["codes"]
    counts = torch.zeros(16, dtype=torch.int64, device=x.device)

    def fn():
        st_ = L.fp4q_code_histogram(ctypes.c_void_p(codes.data_ptr()), R, C, ctypes.c_void_p(counts.data_ptr()),
                                    stream)
        if st_ != 0:
            raise RuntimeError(f"histogram: status {st_}")
    ms = time_fn(torch, fn, reps)
    h = counts.cpu().numpy() / (reps + 1)                 # the calls accumulate
    return {"ms": round(ms, 4), "GB/s": round(R * C / 2 / (ms * 1e6), 1),
            "zero_code_fraction": round(float(h[0] + h[8]) / (R * C), 4),
            "what": "not part of the step: counts of the 16 nibble codes of the NVFP4 (block 16, no per-tensor "
                    "scale) codes of the 4096x4096 N(0,1) input, 8 MiB of code bytes (stand-alone pass)",
            "fused": time_fused_counts(F, torch, x)}


def time_fused_counts(F, torch, x, reps=20, rounds=3):
    """Cost of counting the code occupancy inside the quantize kernels
    (fp4q_quantize_histogram) against the same quantize call without it, on
    one 4096 x 4096 fp32 input: best of `rounds` interleaved means."""
    R, C = x.shape
    dev = x.device
    out = {}
    for name, cfg in (("mxfp4 abs-max", F.mxfp4()),
                      ("nvfp4 4-over-6 tensor-amax", F.config(F.E4M3, 16, F.FOUR_OVER_SIX, F.GLOBAL_TENSOR_AMAX)),
                      ("brute-force block 4", F.config(F.E4M3, 4, F.BRUTE_FORCE, F.GLOBAL_NONE))):
        codes = torch.empty((R, C // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((R, C // cfg.block), dtype=torch.uint8, device=dev)
        g = torch.empty(1, dtype=torch.float32, device=dev)
        n = F.workspace_bytes(cfg, R, C)
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev) if n else None
        counts = F.counts_buffer(dev)
        plain = lambda: F.fp4q_quantize(cfg, x, codes, scales, g, None, None, ws)
        counted = lambda: F.fp4q_quantize_histogram(cfg, x, codes, scales, counts, g, None, None, ws)
        r = 5 if cfg.strategy == F.BRUTE_FORCE else reps
        tp, tc = [], []
        for _ in range(rounds):
            tp.append(time_fn(torch, plain, r))
            tc.append(time_fn(torch, counted, r))
        p_ms, c_ms = min(tp), min(tc)
        out[name] = {"ms": round(p_ms, 4), "ms_with_counts": round(c_ms, 4), "overhead": round(c_ms / p_ms - 1, 4)}
    out["what"] = ("the same quantize call (codes + scales) with and without the fused 16-code occupancy count "
                   "(fp4q_quantize_histogram: per-thread counters, one atomic per code per workgroup into 64 "
                   "replica rows)")
    return out


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
        ms = time_fn(torch, lambda: F.fp4q_mxfp4_gemm(*args), rounds * reps)
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


MFMA_FP16_PEAK_TFLOPS = 2500.0              # MI355X dense fp16 matrix peak, published


def time_gemm_nvfp4(F, torch, dev, warm=10, reps=10, rounds=2):
    """NVFP4 GEMM (outside the step): the same shapes with NVFP4 operands
    (E4M3 scales per 16, tensor-amax g per operand; 4-over-6 for the
    weights).  The matrix cores take only power-of-two block scales, so the
    operands are decoded to fp16 and run on the fp16 matrix cores: the peak
    that bounds it is the dense fp16 one; the FP4 peak is given beside it."""
    out = {}
    gen = torch.Generator(device=dev).manual_seed(12)
    for M, N, K in ((8192, 8192, 8192), (8192, 14336, 4096), (8192, 4096, 14336)):
        qa = F.quantize(torch.randn((M, K), generator=gen, device=dev), F.nvfp4(), want_mse=False)
        qb = F.quantize(torch.randn((N, K), generator=gen, device=dev) * 0.02, F.nvfp4(F.FOUR_OVER_SIX),
                        want_mse=False)
        c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(max(F.nvfp4_gemm_workspace_bytes(M, N, K), 256), dtype=torch.uint8, device=dev)
        args = (qa["codes"], qa["scales"], qa["g"], qb["codes"], qb["scales"], qb["g"], c, ws)
        for _ in range(warm):
            F.fp4q_nvfp4_gemm(*args)
        ms = time_fn(torch, lambda: F.fp4q_nvfp4_gemm(*args), rounds * reps)
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out[f"{M}x{N}x{K}"] = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1),
                               "mfma_frac": round(tf / MFMA_FP16_PEAK_TFLOPS, 4),
                               "of_fp4_peak": round(tf / MFMA_FP4_PEAK_TFLOPS, 4)}
        del qa, qb, c, ws, args
    out["peak"] = {"TFLOP/s": MFMA_FP16_PEAK_TFLOPS, "what": "MI355X dense fp16 matrix-core peak (the operands "
                                                              "run decoded to fp16)"}
    out["what"] = ("not part of the step: NVFP4 GEMM (M x N x K) of NVFP4-quantized N(0,1) activations and "
                   "N(0,0.02^2) weights (E4M3 scales per 16 values, tensor-amax g), decoded to fp16 on the way "
                   "to the 32x32x16 fp16 matrix cores, bf16 output, including the per-call scale rearrangement; "
                   "mean of 20 calls after 10 warm-up calls")
    return out


# --------------------------------------------------------------------------
# the oracle on the host cores
# --------------------------------------------------------------------------

def cpu_step_sample(O, S, host, r0, r1):
    """The step's call list on rows [r0, r1) of every tensor, through the
    single-threaded oracle; returns the algorithmic bytes."""
    names = ["normal", "laplace", "normal_1e-4", "laplace_1e-4"]
    nbytes = 0
    for B in (4, 8, 16, 32):
        for st in (0, 1, 2, 3):
            for gm in (1, 0):
                for name in names:
                    x = np.ascontiguousarray(host[name][r0:r1])
                    O.quantize(x, fmt=1, block=B, strategy=st, global_mode=gm)
                    nbytes += quant_bytes(x.shape[0], x.shape[1], B)
    x = np.ascontiguousarray(host["normal"][r0:r1])
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
    return nbytes


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(O, S, host, rows):
    """The oracle (its plain single-threaded C) over the step's call list on a
    bounded row sample: (i) one thread pinned to one core on rows [0, rows);
    (ii) every core of this process's CPU set (at most 16), each thread on its
    own rows of the same tensors, concurrently (ctypes releases the GIL)."""
    cores = sorted(os.sched_getaffinity(0))
    O.lib()
    os.sched_setaffinity(0, {cores[0]})
    try:
        t0 = time.perf_counter()
        nb1 = cpu_step_sample(O, S, host, 0, rows)
        dt1 = time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, set(cores))
    n = min(len(cores), 16)
    per = max(1, rows // 4)
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(n) as ex:
        nbn = sum(ex.map(lambda i: cpu_step_sample(O, S, host, rows + i * per, rows + (i + 1) * per), range(n)))
    dtn = time.perf_counter() - t0
    return {"value": round(nb1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"the step's call list on the first {rows} rows of each 4096x4096 tensor "
                      f"({nb1 / 1e6:.1f} MB algorithmic, {dt1:.1f} s, one thread pinned to one core)",
            "all_cores": {"value": round(nbn / dtn / 1e9, 4), "unit": "GB/s", "cores": n,
                          "sample": f"{n} threads, each the step's call list on its own {per} rows "
                                    f"({nbn / 1e6:.1f} MB algorithmic, {dtn:.1f} s)"},
            "cpu_model": cpu_model(), "host_cpus_visible": len(cores),
            "compiler": "gcc " + " ".join(O.CFLAGS)}


# --------------------------------------------------------------------------
# roofline of the dominant kernel
# --------------------------------------------------------------------------

def profiled_calls(calls, prof):
    """The calls a bench.py --only profiling run made, in dispatch order (its
    pattern is read from the command recorded with the profile)."""
    import re
    m = re.search(r"--only '([^']*)'", prof.get("command", "")) if prof else None
    pats = m.group(1).split("|") if m else []
    return [c for c in calls if any(p in c.name for p in pats)]


def bf_roofline(calls, per_call, dom, B, valu_probe):
    """Roofline of the brute-force quantize kernel over its launches without
    the abs-max pre-pass (their HIP events hold the kernel alone): executed
    VALU lane-instructions (SQ_INSTS_VALU x 64 per dispatch, from the
    committed counter profile of the same calls on the same sources) over
    the live mean launch time, against the fp32 vector peak."""
    kname = f"k_quant_bf<float, {B}, 0, 1, false>"
    prof = load_profile("counters_bench_dominant")
    kc = kernel_counters(prof, kname)
    solo = [(c, ms) for c, ms in dom if c.meta.get("global_mode") == "none"]
    ms_solo = float(np.mean([ms for _, ms in solo]))
    roof = {"bound": "alu", "kernel": kname, "achieved": None, "peak": round(VALU_PEAK_TOPS, 1),
            "unit": "T VALU lane-instructions/s", "frac": None, "traffic": None,
            "avg_launch_ms": round(ms_solo, 4), "launches": f"{len(solo)} per step (the calls without the "
                                                           "per-tensor pre-pass, whose events time this kernel alone)",
            "work": "executed VALU lane-instructions per launch = SQ_INSTS_VALU x 64 (rocprofv3 counters of the "
                    "same calls on the same kernel sources, profiles/counters_bench_dominant)",
            "algorithmic_MB_per_launch": round(dom[0][0].nbytes / 1e6, 2)}
    elems = dom[0][0].elems
    exhaustive = BF_CANDIDATES * BF_INSTR_PER_EVAL * elems
    roof["exhaustive_equivalent"] = {
        "value": round(exhaustive / (ms_solo * 1e-3) / 1e12, 2), "unit": "T lane-instructions/s",
        "what": f"{BF_CANDIDATES} candidates x {BF_INSTR_PER_EVAL} VALU instructions x {elems} elements per launch "
                "(an exhaustive search) / time; the exact branch and bound evaluates a fraction of the candidates"}
    if valu_probe:
        roof["valu_probe"] = valu_probe
    if not kc or "SQ_INSTS_VALU" not in kc or "values" not in kc["SQ_INSTS_VALU"]:
        roof["why_null"] = "no per-dispatch counter profile on the current kernel sources"
        return roof
    seq = [c for c in profiled_calls(calls, prof) if c.meta.get("strategy") == "brute-force" and c.meta.get("B") == B]
    vals = kc["SQ_INSTS_VALU"]["values"]
    if not seq or len(vals) % len(seq):
        roof["why_null"] = "the counter profile's dispatches do not match its calls"
        return roof
    ins_of = {id(c): 64.0 * float(np.mean(vals[k::len(seq)])) for k, c in enumerate(seq)}
    if any(id(c) not in ins_of for c, _ in solo):
        roof["why_null"] = "the counter profile does not cover every launch"
        return roof
    total_instr = sum(ins_of[id(c)] for c, _ in solo)
    total_ms = sum(ms for _, ms in solo)
    achieved = total_instr / (total_ms * 1e-3) / 1e12
    roof["achieved"] = round(achieved, 2)
    roof["frac"] = round(achieved / VALU_PEAK_TOPS, 4)
    roof["executed_valu_lane_instr_per_launch"] = round(total_instr / len(solo))
    groups = {}
    for c, ms in solo:
        key = "x1e-4 tensors (no per-tensor scale: block scales underflow, short searches)" \
            if c.meta.get("tensor", "").endswith("1e-4") else "N(0,1) and Laplace(0,1) tensors"
        g = groups.setdefault(key, [0.0, 0.0, 0])
        g[0] += ins_of[id(c)]
        g[1] += ms
        g[2] += 1
    roof["by_input"] = {k: {"launches": v[2], "avg_launch_ms": round(v[1] / v[2], 4),
                            "executed_lane_instr_per_launch": round(v[0] / v[2]),
                            "achieved": round(v[0] / (v[1] * 1e-3) / 1e12, 2),
                            "frac": round(v[0] / (v[1] * 1e-3) / 1e12 / VALU_PEAK_TOPS, 4)}
                        for k, v in groups.items()}
    tr = copy_scaled_traffic(prof, kc)
    if tr:
        roof["traffic"] = round(float(np.mean(tr)) / 1e6, 2)
        roof["traffic_unit"] = "MB per launch (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size)"
    return roof


def valu_probe_summary():
    """Executed-instruction rates of the VALU probes from the committed probe
    profile (kernel time and SQ_INSTS_VALU of the same run)."""
    prof = json.load(open(os.path.join(PROFILES, "valu_probe.json"))) if os.path.exists(
        os.path.join(PROFILES, "valu_probe.json")) else None
    if not prof or "rates" not in prof:
        return None
    return {"measured_T_lane_instr_per_s": prof["rates"], "source": "profiles/valu_probe.md"}


# --------------------------------------------------------------------------

def main():
    args = parse()
    if args.summarize:
        summarize(args.summarize, args.label or "profile", args.command, args.probe_json)
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
    if args.probe:
        print("[bench] probes", file=sys.stderr, flush=True)
        res = run_probes(torch, dev)
        print(json.dumps(res), flush=True)
        if args.json_out:
            with open(args.json_out, "w") as f:
                f.write(json.dumps(res) + "\n")
        return
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
    if args.configs_only is not None:
        configs, _cbld = build_configs(F, S, torch, dev)
        pats = args.configs_only.split("|")
        sel = [c for _, calls in configs.values() for c in calls if any(pt in c.name for pt in pats)]
        print(f"[bench] profiling {len(sel)} calls x {args.steps}: {[c.name for c in sel][:6]}", file=sys.stderr,
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
    print("[bench] generating and uploading the workload", file=sys.stderr, flush=True)
    calls, bld, host, X = build_step(F, S, torch, dev)
    step_bytes = sum(c.nbytes for c in calls)

    if args.only is not None or args.copy_mb:
        pats = [] if args.only is None else args.only.split("|")
        sel = [c for c in calls if any(pt in c.name for pt in pats)]
        print(f"[bench] profiling {len(sel)} calls x {args.steps}: {[(c.name, c.meta.get('tensor')) for c in sel][:8]}",
              file=sys.stderr, flush=True)
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

    def step(record=None):
        """One pass over the calls; record = None (no events), "all", or
        the ids of the calls to bracket with HIP events."""
        for c in calls:
            if record is not None and (record == "all" or id(c) in record):
                e0, e1 = events(torch)
                e0.record()
                c()
                e1.record()
                c.times.append((e0, e1))
            else:
                c()

    def family(c):
        return (c.meta.get("strategy", c.kind), c.meta.get("B"))

    def mean_ms(c):
        return float(np.mean([a.elapsed_time(b) for a, b in c.times]))

    # Warm-up.  Its last step (an extra untimed step with --warmup 0) brackets
    # every call with events to find the dominant kernel family: the
    # (strategy, block) family with the largest share of the step.
    print(f"[bench] {len(calls)} calls per step, warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(max(args.warmup - 1, 0)):
        step()
    step(record="all")
    torch.cuda.synchronize()
    fam_ms = {}
    for c in calls:
        fam_ms[family(c)] = fam_ms.get(family(c), 0.0) + mean_ms(c)
        c.times = []
    dom_key = max(fam_ms, key=fam_ms.get)
    dom_ids = {id(c) for c in calls if family(c) == dom_key}

    # Timed region: K steps bracketed by device synchronisation.  Events
    # bracket only the dominant family's launches (the roofline's live
    # launch times): an event pair around every call adds about 1 ms to a
    # 7 ms step (measured), which is measurement, not work.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(record=dom_ids)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = 1e3 * elapsed / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)
    dom_live = {id(c): mean_ms(c) for c in calls if id(c) in dom_ids}
    for c in calls:
        c.times = []

    # Per-call times for the per-strategy table: the same steps again after
    # the timed region, every call bracketed by events.
    for _ in range(args.steps):
        step(record="all")
    torch.cuda.synchronize()
    per_call = [(c, mean_ms(c)) for c in calls]

    # cold leg: every call once more, each after a cache flush outside its events
    flush = Flusher(torch, dev)
    for c in calls:
        flush()
        e0, e1 = events(torch)
        e0.record()
        c()
        e1.record()
        c.cold.append((e0, e1))
    torch.cuda.synchronize()
    cold_ms = {id(c): float(np.mean([a.elapsed_time(b) for a, b in c.cold])) for c in calls}
    print(f"[bench] cold leg: {sum(cold_ms.values()):.3f} ms of calls", file=sys.stderr, flush=True)

    # per-strategy aggregates
    groups = {}
    for c, ms in per_call:
        key = c.meta.get("strategy", c.kind)
        g = groups.setdefault(key, [0, 0, 0.0, 0.0])
        g[0] += c.nbytes
        g[1] += c.elems
        g[2] += ms
        g[3] += cold_ms[id(c)]
    breakdown = {k: {"GB/s": round(b / (ms * 1e6), 1), "Gelem/s": round(e / (ms * 1e6), 2),
                     "hbm_frac": round(b / (ms * 1e6) / HBM_PEAK_GBS, 4), "ms_per_step": round(ms, 4),
                     "GB/s_cold": round(b / (cms * 1e6), 1), "hbm_frac_cold": round(b / (cms * 1e6) / HBM_PEAK_GBS, 4)}
                 for k, (b, e, ms, cms) in groups.items()}

    # dominant kernel family (found in the warm-up) with its launch times from the timed region
    dom = [(c, dom_live[id(c)]) for c in calls if id(c) in dom_ids]
    strategy, B = dom_key
    vprobe = valu_probe_summary()
    if strategy == "brute-force":
        roofline = bf_roofline(calls, per_call, dom, B, vprobe)
    else:
        dom_ms = float(np.mean([ms for _, ms in dom]))
        nbytes = dom[0][0].nbytes
        achieved = nbytes / (dom_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": f"k_quant<float, {B}" if B else dom[0][0].kind,
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "avg_launch_ms": round(dom_ms, 4), "traffic": None}

    del flush
    print("[bench] probes (HBM stream ceilings, VALU rates)", file=sys.stderr, flush=True)
    probes = run_probes(torch, dev, reps=5)
    rot = probes["hbm"]["copy (streaming stores), four 64 MiB tensors in rotation, warm"]["GB/s"]
    for v in breakdown.values():
        v["frac_of_copy"] = round(v["GB/s"] / rot, 4)

    configs = None
    if not args.no_configs:
        print("[bench] per-config lines (C1, C3, C4, C5)", file=sys.stderr, flush=True)
        cfgs, cbld = build_configs(F, S, torch, dev)
        flush = Flusher(torch, dev)
        configs = time_configs(torch, cfgs, flush)
        del cfgs, cbld, flush
        torch.cuda.empty_cache()
    if args.no_extras:
        search = ue5m3 = hist = gemm = gemm_nv = {"what": "not measured (--no-extras)"}
    else:
        print("[bench] widenings (scale search, UE5M3, histogram, GEMM)", file=sys.stderr, flush=True)
        search = time_quantize_configs(F, torch, X["normal"], [
            ("absmax", F.config(F.E4M3, 16, F.ABSMAX, F.GLOBAL_SEARCH)),
            ("4-over-6", F.config(F.E4M3, 16, F.FOUR_OVER_SIX, F.GLOBAL_SEARCH)),
            ("brute-force", F.config(F.E4M3, 16, F.BRUTE_FORCE, F.GLOBAL_SEARCH))])
        ue5m3 = time_quantize_configs(F, torch, X["normal"], [
            (f"B={B} {STRATS[st]}", F.config(F.UE5M3, B, st)) for B in (16, 4) for st in (0, 2, 3)])
        hist = time_histogram(F, torch, X["normal"])
        gemm = time_gemm(F, torch, dev)
        gemm_nv = time_gemm_nvfp4(F, torch, dev)
    stream_quant = [(c, ms) for c, ms in per_call if c.meta.get("strategy") in ("absmax", "4-over-6")]
    sb = sum(c.nbytes for c, _ in stream_quant)
    sms = sum(ms for _, ms in stream_quant)
    scms = sum(cold_ms[id(c)] for c, _ in stream_quant)

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
                                    "GB/s_cold": round(sb / (scms * 1e6), 1),
                                    "hbm_frac_cold": round(sb / (scms * 1e6) / HBM_PEAK_GBS, 4),
                                    "frac_of_copy": round(sb / (sms * 1e6) / rot, 4)},
        "cold_step": {"GB/s": round(step_bytes / (sum(cold_ms.values()) * 1e6), 1),
                      "what": "the step's calls each timed once after a cache flush (1 GiB read on the same "
                              "stream, outside the events); GB/s of the step's algorithmic bytes over the sum of "
                              "the call times"},
        "per_strategy": breakdown,
        "configs": configs,
        "hbm_reference": dict(probes["hbm"], what="hand-written stream kernels (libfp4q_probe.so): 16-byte "
                                                  "accesses, best over 4-32 workgroups per CU; cold = after a "
                                                  "1 GiB read"),
        "global_scale_search": dict({"what": "not part of the step: NVFP4 block 16 quantize of the 4096x4096 "
                                             "N(0,1) input with the per-tensor scale searched over 32 "
                                             "candidates (abs-max pre-pass, 32-candidate scoring, tree "
                                             "reduction, pick, quantize at the winner); GB/s of the "
                                             "quantize call's algorithmic bytes"}, **search),
        "ue5m3_scales": dict({"what": "not part of the step: quantize of the 4096x4096 N(0,1) input with "
                                      "UE5M3 block scales (no per-tensor scale), every output"}, **ue5m3),
        "code_histogram": hist,
        "mxfp4_gemm": gemm,
        "nvfp4_gemm": gemm_nv,
    }

    if not args.no_cpu_baseline:
        from oracle import oracle as O
        O.build()
        print(f"[bench] oracle on {args.cpu_rows} rows per tensor (1 thread, then all cores)", file=sys.stderr,
              flush=True)
        result["cpu_baseline"] = cpu_baseline(O, S, host, args.cpu_rows)
    if args.calls_out:
        with open(args.calls_out, "w") as f:
            json.dump([{"name": c.name, "tensor": c.meta.get("tensor"), "ms": ms, "ms_cold": cold_ms[id(c)],
                        "bytes": c.nbytes} for c, ms in per_call], f, indent=0)
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
