"""attn_jvp_bwd_noalloc: the backward with the library's fixed device
workspace, for callers that cannot allocate.  Through the C ABI, it must give
the same dq, dk, dv as attn_jvp_bwd with a caller workspace, bit for bit
(same kernels), on two calls in a row, the second with a smaller input (the
fixed workspace keeps the first call's contents, which no call reads).
Plans above its fixed size are refused before any device work.
"""
import ctypes

import numpy as np
import pytest
import torch

import masked_attention_jvp_amd as aj
import seeded_inputs as si
from gpu_util import log, small_workload, device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _case(w):
    x = device_inputs(w)
    x["do"] = torch.from_numpy(si.full_tensor_bits(w, "do").view(np.int16 if w.dtype == "bf16" else np.float32)) \
        .to("cuda")
    if w.dtype == "bf16":
        x["do"] = x["do"].view(torch.bfloat16)
    dt = aj.ATTN_JVP_BF16 if w.dtype == "bf16" else aj.ATTN_JVP_FP32
    plan = aj.attn_jvp_create_ex(w.desc, w.batch, w.heads, w.head_dim, dt, 0.0, 0)
    o, to = torch.empty_like(x["q"]), torch.empty_like(x["q"])
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device="cuda")
    aj.attn_jvp_fwd(plan, *(x[t] for t in si.TENSORS), o, to, lse)
    return plan, x, o, lse


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _compare(w):
    plan, x, o, lse = _case(w)
    ref = [torch.empty_like(x["q"]) for _ in range(3)]
    ws = torch.empty(aj.attn_jvp_bwd_workspace_size(plan) // 4, dtype=torch.float32, device="cuda")
    aj.attn_jvp_bwd(plan, x["q"], x["k"], x["v"], o, lse, x["do"], *ref, ws)
    got = [torch.full_like(x["q"], float("nan")) for _ in range(3)]
    aj.attn_jvp_bwd_noalloc(plan, x["q"], x["k"], x["v"], o, lse, x["do"], *got)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(_bits(g), _bits(r)), f"{w.name}: {name} differs from attn_jvp_bwd"
    log(f"[noalloc] {w.name} B={w.batch} H={w.heads} N={w.seq_len} d={w.head_dim} {w.dtype}: "
        f"dq, dk, dv bit-identical to attn_jvp_bwd")


def test_noalloc_matches_bwd_on_two_calls_second_smaller():
    _compare(small_workload(701, 400, 6, 1, 1, heads=3, batch=2, d=128))  # 4800 tokens, 6 slices
    _compare(small_workload(702, 50, 5, 1, 1, heads=2, batch=1, d=64))    # 500 tokens, 2 slices
    _compare(small_workload(703, 37, 4, 2, 0, heads=1, batch=1, d=128, dtype="fp32"))


def test_noalloc_refuses_plans_above_its_workspace():
    """8 B H N > 32 MiB: refused with ATTN_JVP_E_OVERFLOW before any device
    work (dummy, aligned pointers are never dereferenced)."""
    plan = aj.attn_jvp_create_ex((1560, 21, 1, 1), 1, 65, 128, aj.ATTN_JVP_BF16, 0.0, 0)  # 65 x 65520 rows
    lib = aj._load()
    p = ctypes.c_void_p(1 << 20)
    code = lib.attn_jvp_bwd_noalloc(plan.handle, p, p, p, p, p, p, p, p, p, None)
    assert code == 7, aj.attn_jvp_last_error_detail()
    assert "33554432" in aj.attn_jvp_last_error_detail()
