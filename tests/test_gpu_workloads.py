"""Whole (b, h) slices of the four full-size bf16 workloads against the oracle.

Each workload runs once, in the launch configuration bench.py times (one
plan over all B x H slices, every output in caller memory), with o, t_o and
lse prefilled with NaN: every element of every slice must be written and
finite afterwards, so a query block that the grid never computed cannot go
unnoticed.  Then the first and the last (b, h) slice are compared with the
fp64 oracle over all their rows (the definition: Causal-rCM Appendix B,
eqs. 42-45), normwise relative error below 1e-2 on o and t_o, lse within
2e-2.  The clean-tangent-zero plans (section 3.1.2, after eq. 17) get the
same on both teacher-forcing layouts, against the oracle's definition with
the clean tangents zeroed.

The backward (dq, dk, dv; section 3.2.1: the student's FlashAttention-2
based masked attention trains through it) gets the same treatment at the
four workloads: o and lse from the forward, then the backward through the
plan entry points bench.py --backward times, with dq, dk, dv and the
workspace prefilled with NaN and required finite everywhere, and the first
and last (b, h) slice against the oracle's backward over all rows and keys
(normwise 1e-2 on dq, dk, dv and delta).  The range-list workload c1-4
(Appendix B's query groups x key intervals; section 4's chunk pattern with a
first chunk of one frame) gets both checks through the table entry points.

The oracle takes about 8 s per slice of 65520 tokens on a 16-thread host.
"""
import numpy as np
import pytest
import torch

import oracle
import masked_attention_jvp_amd as aj
import seeded_inputs as si
from seeded_inputs import WORKLOADS, TENSORS
from oracle import RangeMask
from gpu_util import log, device_inputs, host_values, to_device, to_f64, rel_err

pytestmark = pytest.mark.gpu

TOL = 1e-2
LSE_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _run_prefilled(w, x, flags):
    plan = aj.attn_jvp_create_ex(w.desc, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16, 0.0, flags)
    nan = float("nan")
    o = torch.full_like(x["q"], nan)
    to = torch.full_like(x["q"], nan)
    lse = torch.full(w.shape[:3], nan, dtype=torch.float32, device=x["q"].device)
    aj.attn_jvp_fwd(plan, *(x[t] for t in TENSORS), o, to, lse)
    torch.cuda.synchronize()
    for name, t in (("o", o), ("t_o", to), ("lse", lse)):
        assert torch.isfinite(t).all().item(), f"{w.name}: {name} has elements not written (NaN) or not finite"
    return o, to, lse


def _whole_slices(w, flags, oracle_fn):
    log(f"[whole slices] {w.name} B={w.batch} H={w.heads} flags={flags}")
    x = device_inputs(w)
    o, to, lse = _run_prefilled(w, x, flags)
    for b, h in sorted({(0, 0), (w.batch - 1, w.heads - 1)}):
        ro, rto, rl = oracle_fn(*host_values(w, b, h), w.desc)
        eo, eto = rel_err(to_f64(o[b, h]), ro), rel_err(to_f64(to[b, h]), rto)
        el = float(np.max(np.abs(to_f64(lse[b, h]) - rl)))
        log(f"    (b={b}, h={h}) all {w.seq_len} rows: rel err o={eo:.3e} to={eto:.3e} max |dlse|={el:.3e}")
        assert eo < TOL and eto < TOL and el < LSE_TOL


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_workload_whole_slices(cfg):
    _whole_slices(WORKLOADS[cfg], 0, oracle.masked_attention_jvp_slice)


@pytest.mark.parametrize("cfg", [3, 4])
def test_workload_whole_slices_clean_tangent_zero(cfg):
    _whole_slices(WORKLOADS[cfg], aj.ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO, oracle.masked_attention_jvp_slice_ctz)


def _whole_slices_bwd(w):
    log(f"[whole slices, backward] {w.name} B={w.batch} H={w.heads}")
    x = device_inputs(w)
    x["do"] = to_device(w, si.full_tensor_bits(w, "do"))
    plan = aj.attn_jvp_create_ex(w.desc, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16, 0.0, 0)
    o = torch.empty_like(x["q"])
    to = torch.empty_like(x["q"])
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device=x["q"].device)
    aj.attn_jvp_fwd(plan, *(x[t] for t in TENSORS), o, to, lse)
    del to, x["tq"], x["tk"], x["tv"]
    nan = float("nan")
    dq, dk, dv = (torch.full_like(x["q"], nan) for _ in range(3))
    ws = torch.full((aj.attn_jvp_bwd_workspace_size(plan) // 4,), nan, dtype=torch.float32, device=x["q"].device)
    aj.attn_jvp_bwd(plan, x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, ws)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("workspace", ws)):
        assert torch.isfinite(t).all().item(), f"{w.name}: {name} has elements not written (NaN) or not finite"
    ws = ws.view(w.batch, w.heads, 2, w.seq_len)
    for b, h in sorted({(0, 0), (w.batch - 1, w.heads - 1)}):
        q, k, v = host_values(w, b, h)[:3]
        rq, rk, rv, rd = oracle.masked_attention_bwd_slice(q, k, v, si.slice_values(w, "do", b, h), w.desc)
        e = [rel_err(to_f64(t[b, h]), r) for t, r in ((dq, rq), (dk, rk), (dv, rv))]
        ed = rel_err(-to_f64(ws[b, h, 0]), rd)
        log(f"    (b={b}, h={h}) all {w.seq_len} rows and keys: rel err dq={e[0]:.3e} dk={e[1]:.3e} "
            f"dv={e[2]:.3e} delta={ed:.3e}")
        assert max(e) < TOL and ed < TOL


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_workload_whole_slices_backward(cfg):
    _whole_slices_bwd(WORKLOADS[cfg])


def _range_plan(w):
    n, groups = w.mask_ranges()
    plan = aj.attn_jvp_create_ranges(n, groups, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16)
    table = torch.from_numpy(aj.attn_jvp_plan_table(plan)).to("cuda")
    return plan, table, RangeMask(n, groups)


def test_range_workload_whole_slices():
    w = si.RANGE_WORKLOADS[6]
    log(f"[whole slices, range list] {w.name} B={w.batch} H={w.heads}")
    plan, table, rm = _range_plan(w)
    x = device_inputs(w)
    nan = float("nan")
    o = torch.full_like(x["q"], nan)
    to = torch.full_like(x["q"], nan)
    lse = torch.full(w.shape[:3], nan, dtype=torch.float32, device=x["q"].device)
    aj.attn_jvp_fwd_table(plan, table, *(x[t] for t in TENSORS), o, to, lse)
    torch.cuda.synchronize()
    for name, t in (("o", o), ("t_o", to), ("lse", lse)):  # every row of c1-4 is in a group
        assert torch.isfinite(t).all().item(), f"{w.name}: {name} has elements not written (NaN) or not finite"
    for b, h in sorted({(0, 0), (w.batch - 1, w.heads - 1)}):
        ro, rto, rl = oracle.masked_attention_jvp_slice(*host_values(w, b, h), rm)
        eo, eto = rel_err(to_f64(o[b, h]), ro), rel_err(to_f64(to[b, h]), rto)
        el = float(np.max(np.abs(to_f64(lse[b, h]) - rl)))
        log(f"    (b={b}, h={h}) all {w.seq_len} rows: rel err o={eo:.3e} to={eto:.3e} max |dlse|={el:.3e}")
        assert eo < TOL and eto < TOL and el < LSE_TOL


def test_range_workload_whole_slices_backward():
    w = si.RANGE_WORKLOADS[6]
    log(f"[whole slices, range list, backward] {w.name} B={w.batch} H={w.heads}")
    plan, table, rm = _range_plan(w)
    x = device_inputs(w)
    x["do"] = to_device(w, si.full_tensor_bits(w, "do"))
    o = torch.empty_like(x["q"])
    to = torch.empty_like(x["q"])
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device=x["q"].device)
    aj.attn_jvp_fwd_table(plan, table, *(x[t] for t in TENSORS), o, to, lse)
    del to, x["tq"], x["tk"], x["tv"]
    nan = float("nan")
    dq, dk, dv = (torch.full_like(x["q"], nan) for _ in range(3))
    ws = torch.full((aj.attn_jvp_bwd_workspace_size(plan) // 4,), nan, dtype=torch.float32, device=x["q"].device)
    aj.attn_jvp_bwd_table(plan, table, x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, ws)
    torch.cuda.synchronize()
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv), ("workspace", ws)):
        assert torch.isfinite(t).all().item(), f"{w.name}: {name} has elements not written (NaN) or not finite"
    ws = ws.view(w.batch, w.heads, 2, w.seq_len)
    for b, h in sorted({(0, 0), (w.batch - 1, w.heads - 1)}):
        q, k, v = host_values(w, b, h)[:3]
        rq, rk, rv, rd = oracle.masked_attention_bwd_slice(q, k, v, si.slice_values(w, "do", b, h), rm)
        e = [rel_err(to_f64(t[b, h]), r) for t, r in ((dq, rq), (dk, rk), (dv, rv))]
        ed = rel_err(-to_f64(ws[b, h, 0]), rd)
        log(f"    (b={b}, h={h}) all {w.seq_len} rows and keys: rel err dq={e[0]:.3e} dk={e[1]:.3e} "
            f"dv={e[2]:.3e} delta={ed:.3e}")
        assert max(e) < TOL and ed < TOL


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_full_workload_forward_and_backward_are_deterministic():
    # No result is accumulated by atomics, and a task's arithmetic does not
    # depend on which workgroup takes it from the work queues: repeated calls
    # at the full size, where thousands of workgroups stream long tile runs
    # through the DMA ring (the backward with one workgroup barrier per two
    # steps) and take their tasks in a different interleaving every time,
    # give the same bits every time.
    w = WORKLOADS[3]
    log(f"[full-size determinism] {w.name}")
    x = device_inputs(w)
    x["do"] = to_device(w, si.full_tensor_bits(w, "do"))
    plan = aj.attn_jvp_create_ex(w.desc, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16, 0.0, 0)
    dev = x["q"].device
    fwd_ref = bwd_ref = None
    for it in range(5):
        o, to = torch.empty_like(x["q"]), torch.empty_like(x["q"])
        lse = torch.empty(w.shape[:3], dtype=torch.float32, device=dev)
        aj.attn_jvp_fwd(plan, *(x[t] for t in TENSORS), o, to, lse)
        dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))
        ws = torch.empty(aj.attn_jvp_bwd_workspace_size(plan) // 4, dtype=torch.float32, device=dev)
        aj.attn_jvp_bwd(plan, x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, ws)
        torch.cuda.synchronize()
        fwd, bwd = (o, to, lse), (dq, dk, dv, ws)
        if fwd_ref is None:
            fwd_ref, bwd_ref = fwd, bwd
            continue
        for a, b in zip(fwd_ref + bwd_ref, fwd + bwd):
            assert torch.equal(_bits(a), _bits(b)), f"call {it} differs from call 0"
