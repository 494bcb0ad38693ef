"""Helpers shared by the GPU tests: seeded device inputs and error norms."""
import sys

import numpy as np
import torch

import seeded_inputs as si
from seeded_inputs import TENSORS, Workload, WORKLOADS


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def small_workload(cfg_id, tokens_per_frame, n_frames, frames_per_chunk, tf, heads=2, batch=1, d=128,
                   dtype="bf16", tangent_std=0.1):
    return Workload(f"small_{cfg_id}", cfg_id, batch, heads, d, tokens_per_frame, n_frames, frames_per_chunk, tf,
                    dtype, tangent_std, dtype == "bf16")


def to_device(w: Workload, bits: np.ndarray, device="cuda"):
    if w.dtype == "bf16":
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(bits).to(device)


def device_inputs(w: Workload, device="cuda"):
    return {t: to_device(w, si.full_tensor_bits(w, t), device) for t in TENSORS}


def host_values(w: Workload, b: int, h: int):
    return [si.slice_values(w, t, b, h) for t in TENSORS]


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    return float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))


def sample_rows(desc, n_random=16, seed=0):
    """Rows at the start, middle and end of chunks 0, 1, C/2 and C-1 on every
    side, around 128-row block edges, and a few random ones."""
    tpf, f, c, tf = desc
    T, C, nh = tpf * c, f // c, tpf * f
    n = nh * (2 if tf else 1)
    rows = set()
    for side in range(2 if tf else 1):
        for ch in sorted({0, 1 % C, C // 2, C - 1}):
            lo = side * nh + ch * T
            rows.update([lo, lo + T // 2, lo + T - 1])
        for b in (127, 128, 255, 256):
            if b < nh:
                rows.add(side * nh + b)
        rows.add(side * nh + nh - 1)
    rng = np.random.default_rng(seed)
    rows.update(int(x) for x in rng.choice(n, n_random, replace=False))
    return np.array(sorted(rows))
