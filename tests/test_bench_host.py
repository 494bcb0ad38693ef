"""Host-side logic of bench.py, no GPU: the one-GPU refusal, the kernel-code
hash that ties committed traffic counters to the kernel source, and the
lookup of those counters."""
import json
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_json_line():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def _copy_sources(tmp_path, monkeypatch):
    srcs = {}
    for part, paths in bench.KERNEL_SRCS.items():
        srcs[part] = []
        for p in paths:
            q = tmp_path / os.path.basename(p)
            if not q.exists():
                shutil.copy(p, q)
            srcs[part].append(str(q))
    monkeypatch.setattr(bench, "KERNEL_SRCS", srcs)
    return tmp_path


def _edit(path, old, new):
    s = path.read_text()
    assert s.count(old) == 1
    path.write_text(s.replace(old, new))


def test_kernel_hash_follows_each_part_s_own_code(tmp_path, monkeypatch):
    d = _copy_sources(tmp_path, monkeypatch)
    fwd0, bwd0 = bench.kernel_hash("fwd"), bench.kernel_hash("bwd")
    # comments and blank lines do not count
    _edit(d / "attn_jvp_kernels.hip", "namespace attn_jvp {", "namespace attn_jvp {\n\n// a note\n")
    assert bench.kernel_hash("fwd") == fwd0
    # the backward's parameter struct is not part of the forward's code, and the reverse
    _edit(d / "attn_jvp_launch.h", "  float* ws;", "  float* ws;\n  int32_t extra_bwd_field;")
    assert bench.kernel_hash("fwd") == fwd0 and bench.kernel_hash("bwd") != bwd0
    bwd1 = bench.kernel_hash("bwd")
    _edit(d / "attn_jvp_launch.h", "  int32_t primal;", "  int32_t primal;\n  int32_t extra_fwd_field;")
    assert bench.kernel_hash("fwd") != fwd0 and bench.kernel_hash("bwd") == bwd1
    # a code change in a shared header changes both
    fwd2 = bench.kernel_hash("fwd")
    _edit(d / "kernel_common.h", "namespace attn_jvp {", "namespace attn_jvp {\nconstexpr int kUnused = 1;")
    assert bench.kernel_hash("fwd") != fwd2 and bench.kernel_hash("bwd") != bwd1


def test_traffic_is_reported_only_for_the_recorded_kernel_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    name = "some_workload"
    rec = {"workload": name, "kernel_code_sha256_16": bench.kernel_hash("fwd"), "hbm_bytes_per_launch": 123}
    (tmp_path / f"traffic_{name}.json").write_text(json.dumps(rec))
    assert bench.traffic_for(name, "fwd") == 123
    assert bench.traffic_for(name, "bwd") is None          # other part's code
    assert bench.traffic_for("other_workload", "fwd") is None  # no record
    rec["kernel_code_sha256_16"] = "0" * 16
    (tmp_path / f"traffic_{name}.json").write_text(json.dumps(rec))
    assert bench.traffic_for(name, "fwd") is None          # stale record


def test_no_smi_switches_the_power_samples_off(monkeypatch):
    calls = []
    monkeypatch.setattr(bench.subprocess, "run", lambda *a, **k: calls.append(a) or None)
    monkeypatch.setattr(bench, "SMI_ENABLED", False)
    assert bench.smi_sample() is None and calls == []
    s = bench.SmiSampler()
    s.start()
    s.join(timeout=5)
    assert not s.is_alive() and s.summary() is None and calls == []


def test_cpu_baseline_times_slices_until_its_time_floor(monkeypatch):
    import seeded_inputs as si
    w = si.WORKLOADS[1]  # 2 heads
    monkeypatch.setattr(bench, "CPU_SAMPLE_MIN_S", 0.0)  # the first slice already reaches it
    rec = bench.cpu_baseline(w, 1 << 30)
    assert rec["kind"] == "oracle" and rec["value"] > 0 and rec["sample"].startswith("1 of 2 ")
    monkeypatch.setattr(bench, "CPU_SAMPLE_MIN_S", 1e9)  # never reached: every slice of batch 0
    assert bench.cpu_baseline(w, 1 << 30)["sample"].startswith("2 of 2 ")
    assert bench.cpu_baseline_bwd(w, 1)["sample"].startswith("1 of 2 ")  # the cap
