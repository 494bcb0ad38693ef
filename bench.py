#!/usr/bin/env python3
"""Benchmark: useful TFLOP/s of fused masked attention forward + JVP on one
MI355X, and its fraction of the bf16 dense MFMA peak.

One step = one call of the whole operation (attn_jvp_fwd: scores, score
tangents, masked online softmax, both products with V and tV, epilogue) over
one batch of seeded synthetic inputs already resident in HBM.  Default
workload: frame-wise teacher forcing, B=1, H=12, d=128, 21 clean + 21 noisy
frames of 1560 tokens (N = 65520), bf16.

Useful FLOPs = 12 d x (allowed query-key pairs) x B x H: 2 flops per
multiply-add over q.k, tq.k, q.tk, p.v, p.tv and (p ts).v, masked pairs not
counted (partial tiles included), exp and other vector work not counted.
With --clean-tangent-zero: 4 d per clean-row pair, 8 d per noisy-row /
clean-key pair, 12 d per noisy-row / noisy-key pair (attn_jvp_plan_flops).

--ranges runs the workload's mask as a range list (query groups x key
intervals, attn_jvp_fwd_table); --config 6, the c1-4 teacher-forcing
workload (a one-frame first chunk, then four-frame chunks), exists only as a
range list.

--primal measures the forward without tangents (attn_jvp_fwd_primal: o and
lse only; useful FLOPs = 4 d x allowed pairs x B x H, for q.k and p.v).

--backward measures the backward instead (attn_jvp_bwd: the dq kernel, then
the dk/dv kernel, from q, k, v, o, lse and dO on the same plan); useful
FLOPs = 10 d x (allowed pairs) x B x H (q.k, dO.v, dS k, dS q, P dO).

Prints one JSON line.  --gpus above 1 is refused: the benchmark measures one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4 SIMD x 1024 bf16 flop/clk x 2.4 GHz (dense)
METRIC = "useful TFLOP/s of masked attn fwd+JVP and % of bf16 MFMA peak, 1 GPU"
METRIC_BWD = "useful TFLOP/s of masked attn backward (dq, dk, dv) and % of bf16 MFMA peak, 1 GPU"
METRIC_PRIMAL = "useful TFLOP/s of masked attn forward without tangents and % of bf16 MFMA peak, 1 GPU"
_CSRC = os.path.join(ROOT, "masked_attention_jvp_amd", "csrc")
KERNEL_SRCS = {
    "fwd": [os.path.join(_CSRC, f) for f in ("attn_jvp_kernels.hip", "kernel_common.h", "attn_jvp_launch.h",
                                               "mask_index.h")],
    "bwd": [os.path.join(_CSRC, f) for f in ("attn_jvp_bwd_kernels.hip", "kernel_common.h", "attn_jvp_launch.h",
                                               "mask_index.h")],
}
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3, help="workload id (2..5; 6 = c1-4, range list)")
    ap.add_argument("--ranges", action="store_true",
                    help="run the mask as a range list through the schedule-table kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-heads", type=int, default=1 << 30,
                    help="at most this many (b, h) slices for the CPU baseline, which stops once "
                         "10 s of oracle time are spent")
    ap.add_argument("--heads", type=int, default=0,
                    help="override the workload's head count, e.g. 3 = one GPU's share of the 12-head "
                         "workload under 4-way head (Ulysses) sharding")
    ap.add_argument("--clean-tangent-zero", action="store_true",
                    help="teacher-forcing plans whose clean tokens carry no tangent (useful FLOPs counted "
                         "for that case: about half the general work)")
    ap.add_argument("--primal", action="store_true",
                    help="time the forward without tangents (o and lse) instead of the forward + JVP")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (dq, dk, dv) on the same plan instead of the forward + JVP")
    ap.add_argument("--no-smi", action="store_true",
                    help="skip the amd-smi power / clock samples (for runs under a profiler, whose "
                         "preloaded library should not follow bench.py into the amd-smi child process)")
    ap.add_argument("--mode", choices=["attn", "copy"], default="attn",
                    help="copy: a plain 1 GiB device copy, the reference for HBM byte counters")
    return ap.parse_args()


def copy_reference(steps):
    """A plain device-to-device copy of 1 GiB, timed, for calibrating the
    FETCH_SIZE / WRITE_SIZE counters against bytes known to move."""
    import torch
    n = 1 << 29  # bf16 elements = 1 GiB
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"mode": "copy", "bytes_read_per_copy": 2 * n, "bytes_written_per_copy": 2 * n,
                      "ms_per_copy": round(dt * 1e3, 4), "GB_per_s": round(4 * n / dt / 1e9, 1)}), flush=True)


SMI_ENABLED = True


def smi_sample():
    """(socket power W, GFX clock MHz) from amd-smi, or None where unavailable
    or switched off."""
    if not SMI_ENABLED:
        return None
    try:
        out = subprocess.run(["amd-smi", "metric", "-p", "-c"], capture_output=True, text=True, timeout=10).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    pw = re.search(r"SOCKET_POWER:\s*([\d.]+)\s*W", out)
    ck = re.search(r"GFX_0:\s*CLK:\s*([\d.]+)\s*MHz", out)
    if not pw or not ck:
        return None
    return float(pw.group(1)), float(ck.group(1))


class SmiSampler(threading.Thread):
    """Samples power and clock while the timed launches run."""

    def __init__(self):
        super().__init__(daemon=True)
        self.samples, self.stop = [], threading.Event()

    def run(self):
        while not self.stop.is_set():
            v = smi_sample()
            if v is None:
                return
            self.samples.append(v)

    def summary(self):
        if not self.samples:
            return None
        return {"samples": len(self.samples),
                "power_w_median": statistics.median(v[0] for v in self.samples),
                "sclk_mhz_median": statistics.median(v[1] for v in self.samples),
                "sclk_mhz_min": min(v[1] for v in self.samples)}


def kernel_hash(part="fwd"):
    """Hash of the code the kernels of one part (fwd, bwd) are built from
    (comments and blank lines removed), so that counters stay attached to an
    unchanged kernel.  The shared launch header enters without the other
    part's parameter struct, which its kernels never see."""
    other = {"fwd": "BwdParams", "bwd": "FwdParams"}[part]
    h = hashlib.sha256()
    for path in KERNEL_SRCS[part]:
        with open(path) as f:
            code = re.sub(r"//[^\n]*", "", f.read())
        if path.endswith("attn_jvp_launch.h"):
            code = re.sub(r"struct " + other + r" \{.*?\n\};", "", code, flags=re.S)
        h.update("\n".join(l.rstrip() for l in code.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def traffic_for(workload_name, part="fwd"):
    """HBM bytes per launch from committed rocprofv3 counters, if they were
    taken on the current kernel source; else None."""
    try:
        with open(os.path.join(PROFILES, f"traffic_{workload_name}.json")) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_code_sha256_16") != kernel_hash(part) or t.get("workload") != workload_name:
        return None
    return t.get("hbm_bytes_per_launch")


# The CPU baseline times whole (b, h) slices of batch 0 until at least this
# much oracle time is spent (or the slices run out).
CPU_SAMPLE_MIN_S = 10.0


def host_info():
    """CPU model (from /proc/cpuinfo) and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cores = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        cores = os.cpu_count()
    return {"cpu_model": model, "cores_available": cores}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        return 1


def _time_oracle(w, max_heads, tensors, run, flops_per_slice, what):
    """run(args) is the oracle on one slice's host values; returns the
    cpu_baseline record over the slices timed."""
    import seeded_inputs as si
    flops, elapsed, n = 0, 0.0, 0
    for h in range(min(max_heads, w.heads)):
        args = [si.slice_values(w, t, 0, h) for t in tensors]
        t0 = time.perf_counter()
        run(args)
        elapsed += time.perf_counter() - t0
        flops += flops_per_slice
        n += 1
        if elapsed >= CPU_SAMPLE_MIN_S:
            break
    hi = host_info()
    return {
        "value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
        "sample": f"{n} of {w.batch * w.heads} (b,h) slices of {w.name} ({what}), fp64 NumPy, {elapsed:.1f} s",
        "threads": "one process, NumPy fp64 with its BLAS on `cores` threads",
        "cores_available": hi["cores_available"], "cpu_model": hi["cpu_model"],
    }


def cpu_baseline_bwd(w, max_heads, ranges=False):
    """The oracle's backward, untuned, on (b, h) slices of the same workload."""
    import oracle
    mask = oracle.RangeMask(*w.mask_ranges()) if ranges else w.desc
    return _time_oracle(w, max_heads, ("q", "k", "v", "do"), lambda a: oracle.masked_attention_bwd_slice(*a, mask),
                        oracle.backward_useful_flops(mask, w.head_dim),
                        "all rows, backward" + (", range-list mask" if ranges else ""))


def cpu_baseline_primal(w, max_heads, ranges=False):
    """The oracle (which forms o together with the tangent) on (b, h) slices;
    only the primal's 4 d flops per pair are counted."""
    import oracle
    import seeded_inputs as si
    mask = oracle.RangeMask(*w.mask_ranges()) if ranges else w.desc
    return _time_oracle(w, max_heads, si.TENSORS, lambda a: oracle.masked_attention_jvp_slice(*a, mask),
                        4 * w.head_dim * oracle.pair_count(mask),
                        "all rows; the oracle forms o with its tangent, 4 d flops per pair counted")


def cpu_baseline_ranges(w, max_heads):
    """The oracle on the range-list mask, untuned, on (b, h) slices."""
    import oracle
    import seeded_inputs as si
    rm = oracle.RangeMask(*w.mask_ranges())
    return _time_oracle(w, max_heads, si.TENSORS, lambda a: oracle.masked_attention_jvp_slice(*a, rm),
                        12 * w.head_dim * oracle.pair_count(rm), "all rows, range-list mask")


def cpu_baseline(w, max_heads, clean_tangent_zero=False):
    """The oracle, untuned, on (b, h) slices of the same workload."""
    import oracle
    import seeded_inputs as si
    fn = oracle.masked_attention_jvp_slice_ctz if clean_tangent_zero else oracle.masked_attention_jvp_slice
    return _time_oracle(w, max_heads, si.TENSORS, lambda a: fn(*a, w.desc),
                        oracle.useful_flops(w.desc, w.head_dim, clean_tangent_zero), "all rows")


def main():
    global SMI_ENABLED
    args = parse()
    SMI_ENABLED = not args.no_smi
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only; run with --gpus 1"}))
        sys.exit(2)
    if args.mode == "copy":
        copy_reference(args.steps)
        return

    import numpy as np
    import torch
    import masked_attention_jvp_amd as aj
    import seeded_inputs as si

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    w = si.WORKLOADS.get(args.config) or si.RANGE_WORKLOADS.get(args.config)
    if w is None:
        print(json.dumps({"error": f"unknown workload {args.config}"}))
        sys.exit(2)
    use_ranges = args.ranges or args.config in si.RANGE_WORKLOADS
    if args.primal and (args.backward or args.clean_tangent_zero):
        print(json.dumps({"error": "--primal is the forward alone: no --backward, no --clean-tangent-zero"}))
        sys.exit(2)
    if use_ranges and args.clean_tangent_zero:
        print(json.dumps({"error": "range-list plans have no clean-tangent-zero option"}))
        sys.exit(2)
    if args.ranges and args.config not in si.RANGE_WORKLOADS:
        w = w.with_(name=f"{w.name}_ranges")
    if args.heads > 0 and args.heads != w.heads:
        w = w.with_(heads=args.heads, name=f"{w.name}_h{args.heads}")
    flags = 0
    if args.clean_tangent_zero and args.backward:
        print(json.dumps({"error": "--clean-tangent-zero concerns the forward + JVP only"}))
        sys.exit(2)
    if args.clean_tangent_zero:
        flags = aj.ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO
        w = w.with_(name=f"{w.name}_ctz")
    if args.backward:
        w = w.with_(name=f"{w.name}_bwd")
    if args.primal:
        w = w.with_(name=f"{w.name}_primal")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    x = {}
    for t in si.TENSORS + (si.GRAD_TENSORS if args.backward else ()):
        bits = si.full_tensor_bits(w, t)
        x[t] = torch.from_numpy(bits.view(np.int16)).to(dev).view(torch.bfloat16)
        del bits
    if use_ranges:
        n_tok, groups = w.mask_ranges()
        plan = aj.attn_jvp_create_ranges(n_tok, groups, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16)
        table = torch.from_numpy(aj.attn_jvp_plan_table(plan)).to(dev)
    else:
        plan = aj.attn_jvp_create_ex(w.desc, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16, 0.0, flags)
    o = torch.empty_like(x["q"])
    to = torch.empty_like(x["q"])
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
    if use_ranges and args.primal:
        call = lambda: aj.attn_jvp_fwd_primal_table(plan, table, x["q"], x["k"], x["v"], o, lse)
    elif use_ranges and not args.backward:
        call = lambda: aj.attn_jvp_fwd_table(plan, table, *(x[t] for t in si.TENSORS), o, to, lse)
    elif args.primal:
        call = lambda: aj.attn_jvp_fwd_primal(plan, x["q"], x["k"], x["v"], o, lse)
    elif not args.backward:
        call = lambda: aj.attn_jvp_fwd(plan, *(x[t] for t in si.TENSORS), o, to, lse)
    else:
        # o and lse of these inputs, once, outside the timed region
        if use_ranges:
            aj.attn_jvp_fwd_table(plan, table, *(x[t] for t in si.TENSORS), o, to, lse)
        else:
            aj.attn_jvp_fwd(plan, *(x[t] for t in si.TENSORS), o, to, lse)
        del to, x["tq"], x["tk"], x["tv"]
        dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))
        ws = torch.empty(aj.attn_jvp_bwd_workspace_size(plan) // 4, dtype=torch.float32, device=dev)
        if use_ranges:
            call = lambda: aj.attn_jvp_bwd_table(plan, table, x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, ws)
        else:
            call = lambda: aj.attn_jvp_bwd(plan, x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    # shader clock of every XCD over the timed launches: one clock sample
    # right before the first and one right after the last, on the same stream
    clk = torch.zeros(64, dtype=torch.int64, device=dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    smi_before = smi_sample()
    sampler = SmiSampler()
    torch.cuda.synchronize()
    sampler.start()
    t0 = time.perf_counter()
    aj.attn_jvp_clock_sample(clk[:32], stream)
    for i in range(args.steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    aj.attn_jvp_clock_sample(clk[32:], stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sampler.stop.set()
    sampler.join(timeout=15)
    smi_after = smi_sample()
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_ms = float(np.mean(per_launch_ms))
    total_ms = starts[0].elapsed_time(ends[-1])
    ms_per_step = total_ms / args.steps

    c = clk.cpu().numpy()
    sclk = aj.shader_clock_mhz(c[:32], c[32:])
    sclk_mean = float(np.mean(list(sclk.values()))) if sclk else None
    props = torch.cuda.get_device_properties(dev)

    info = plan.info
    useful = (aj.attn_jvp_plan_bwd_flops(plan) if args.backward
              else 4 * w.head_dim * info["allowed_pairs_per_head"] * w.batch * w.heads if args.primal
              else aj.attn_jvp_plan_flops(plan))
    value = useful / (ms_per_step * 1e-3) / 1e12
    achieved = useful / (avg_ms * 1e-3) / 1e12
    part = "bwd" if args.backward else "fwd"
    traffic = traffic_for(w.name, part)
    nw = info["block_q"] // 32
    tb = "true" if use_ranges else "false"
    dq_kernel = f"bwd_dq_bf16_kernel<{w.head_dim},{nw}>" if use_ranges else f"bwd_dq2_bf16_kernel<{w.head_dim},{nw}>"
    kernel = (f"{dq_kernel} + bwd_dkdv_bf16_kernel<{w.head_dim},{nw},{tb}>"
              if args.backward
              else (f"fwd_bf16_kernel<{w.head_dim},{nw},true,true,true> (primal-only)" if int(table[4]) <= 3968  # entry limit
                    else f"fwd_bf16_kernel<{w.head_dim},{nw},true,true> (primal tile mode)") if args.primal and use_ranges
              else f"fwd_bf16_kernel<{w.head_dim},{nw},true,false,true> (primal-only)" if args.primal
              else (f"fwd_bf16_kernel<{w.head_dim},{nw},true,false,true> (clean side) + "
                    f"fwd_bf16_kernel<{w.head_dim},{nw},true,false> (noisy side)") if flags
              else f"fwd_bf16_kernel<{w.head_dim},{nw},false,{'true' if use_ranges else 'false'}>")

    out = {
        "metric": METRIC_BWD if args.backward else METRIC_PRIMAL if args.primal else METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": ("synthetic (seeded; q,k RMS-normalised N(0,1), v N(0,1), dO N(0,1); o, lse from the forward)"
                 if args.backward else
                 "synthetic (seeded; q,k RMS-normalised N(0,1), v N(0,1), tangents N(0,%g^2))" % w.tangent_std),
        "config": {
            "workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
            "head_dim": w.head_dim, "tokens_per_frame": w.tokens_per_frame, "n_frames": w.n_frames,
            "frames_per_chunk": w.frames_per_chunk, "tf_layout": w.tf_layout,
            "clean_tangent_zero": bool(flags),
            "pass": "backward" if args.backward else "forward" if args.primal else "forward+jvp",
            "mask": "range list" if use_ranges else "descriptor",
            "chunk_frames": list(w.chunks),
        },
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "useful_tflop_per_step": round(useful / 1e12, 4),
        "launch_ms": {"mean": round(avg_ms, 4), "median": round(float(np.median(per_launch_ms)), 4),
                      "min": round(float(np.min(per_launch_ms)), 4)},
        # amd-smi's power and clock readings trail the load by about a second:
        # samples during the timed launches are kept only for runs of 2 s or more.
        "gpu_power_clock": {"before": smi_before, "after": smi_after,
                            "during": sampler.summary() if wall >= 2.0 else None},
        "wall_s_timed": round(wall, 3),
        "gpu": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                "compute_units": props.multi_processor_count,
                # average shader clock per XCD over the timed launches (s_memtime
                # against the 100 MHz real-time counter)
                "sclk_mhz_timed": {str(k): round(v, 1) for k, v in sorted(sclk.items())},
                "sclk_mhz_timed_mean": round(sclk_mean, 1) if sclk_mean else None},
        "host": host_info(),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "avg_launch_ms": round(avg_ms, 4),
            # the same peak at the clock measured over the timed launches
            "peak_at_timed_sclk": round(PEAK_BF16_TFLOPS * sclk_mean / 2400.0, 1) if sclk_mean else None,
            "frac_at_timed_sclk": round(achieved / (PEAK_BF16_TFLOPS * sclk_mean / 2400.0), 4) if sclk_mean else None,
        },
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = (cpu_baseline_bwd(w, args.cpu_sample_heads, use_ranges) if args.backward
                               else cpu_baseline_primal(w, args.cpu_sample_heads, use_ranges) if args.primal
                               else cpu_baseline_ranges(w, args.cpu_sample_heads) if use_ranges
                               else cpu_baseline(w, args.cpu_sample_heads, bool(flags)))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
