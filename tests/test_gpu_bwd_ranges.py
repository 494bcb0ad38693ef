"""GPU parity of the backward on range-list plans (attn_jvp_bwd_table)
against the fp64 oracle, through the C ABI.

o and lse come from the library's own range-list forward on the same inputs
(zero tangents); the oracle computes the backward from q, k, v and dO alone.
Tolerances as for descriptor plans (normwise relative error per slice):
bf16 1e-2, fp32 1e-4; the workspace's -delta plane against the oracle's
delta, its second plane against -lse log2(e) (the most negative finite float
for rows in no group).
Rows in no group get dq = 0 exactly and leave no trace in dk, dv.

A chunked mask given as a range list walks, for every row and every key,
the same tiles in the same order as the descriptor path (tiles a row or key
does not see add exact zeros), so dq, dk, dv and the workspace must be
bit-identical to attn_jvp_bwd -- at small ragged sizes and at the full
65520-token workload.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import masked_attention_jvp_amd as aj
from oracle import RangeMask
from seeded_inputs import TENSORS, WORKLOADS
from gpu_util import log, small_workload, device_inputs, host_values, to_device, to_f64, rel_err, sample_rows

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp32": 1e-4}
DELTA_TOL = {"bf16": 1e-2, "fp32": 1e-5}
LOG2E = 1.4426950408889634

GAPS = (40, ((0, 6, ((0, 3), (10, 14))), (9, 15, ((0, 40),)), (15, 33, ((5, 6), (20, 33))), (35, 40, ((1, 2),))))
MULTI = (170, ((0, 60, ((0, 3), (37, 39), (72, 100), (133, 140))), (60, 170, ((0, 170),))))
STRIPES = (300, ((0, 40, ((0, 70),)), (60, 100, ((0, 70), (150, 300))), (130, 170, ((0, 70),)),
                 (200, 300, ((150, 300),))))
MASKS = {
    "tf_c1_2_t16": si.chunked_mask_ranges(16, (1, 2, 2), 1),
    "tf_c1_4_t50": si.chunked_mask_ranges(50, (1, 4, 4), 1),
    "bc_c2_1_t37": si.chunked_mask_ranges(37, (2, 1, 1, 3), 0),
    "und_gen": si.und_gen_ranges(20, 5, 30),
    "dense_150": (150, ((0, 150, ((0, 150),)),)),
    "gaps": GAPS,
    "multi": MULTI,        # rows with four key intervals
    "stripes": STRIPES,    # keys seen by three separate row intervals
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _inputs(w):
    x = device_inputs(w)
    x["do"] = to_device(w, si.full_tensor_bits(w, "do"))
    return x


def _run_ranges(x, groups):
    z = torch.zeros_like(x["q"])
    o, _, lse = aj.masked_attention_jvp_ranges(x["q"], x["k"], x["v"], z, z, z, groups, return_lse=True)
    dq, dk, dv, ws = aj.masked_attention_bwd_ranges(x["q"], x["k"], x["v"], o, lse, x["do"], groups,
                                                    return_workspace=True)
    torch.cuda.synchronize()
    b, h, n, _ = x["q"].shape
    return dq, dk, dv, ws.view(b, h, 2, n), lse


def _run_desc(w, x):
    z = torch.zeros_like(x["q"])
    o, _, lse = aj.masked_attention_jvp(x["q"], x["k"], x["v"], z, z, z, w.desc, return_lse=True)
    dq, dk, dv, ws = aj.masked_attention_bwd(x["q"], x["k"], x["v"], o, lse, x["do"], w.desc, return_workspace=True)
    torch.cuda.synchronize()
    return dq, dk, dv, ws.view(w.batch, w.heads, 2, w.seq_len), lse


def _slices(w, b, h):
    q, k, v = host_values(w, b, h)[:3]
    return q, k, v, si.slice_values(w, "do", b, h)


def _parity(cid, name, d=128, dtype="bf16", heads=2):
    n, groups = MASKS[name]
    w = small_workload(cid, n, 1, 1, 0, heads=heads, d=d, dtype=dtype)
    log(f"[range bwd parity] {name} N={n} d={d} {dtype}")
    x = _inputs(w)
    dq, dk, dv, ws, lse = (to_f64(t) for t in _run_ranges(x, groups))
    rm = RangeMask(n, groups)
    covered = oracle.mask_dense(rm).any(axis=1)
    worst = np.zeros(4)
    for h in range(w.heads):
        rq, rk, rv, rd = oracle.masked_attention_bwd_slice(*_slices(w, 0, h), rm)
        worst = np.maximum(worst, [rel_err(dq[0, h], rq), rel_err(dk[0, h], rk), rel_err(dv[0, h], rv),
                                   rel_err(-ws[0, h, 0], rd)])
        for t in (dq, dk, dv):
            assert np.isfinite(t[0, h]).all()
        assert np.all(dq[0, h, ~covered] == 0) and np.all(ws[0, h, 0, ~covered] == 0)
        assert np.all(ws[0, h, 1, ~covered] == np.finfo(np.float32).min)
        nl = -lse[0, h, covered].astype(np.float32) * np.float32(LOG2E)
        assert np.max(np.abs(ws[0, h, 1, covered] - nl) / np.maximum(np.abs(nl), 1.0)) < 1e-6
    log(f"    max rel err dq={worst[0]:.3e} dk={worst[1]:.3e} dv={worst[2]:.3e} delta={worst[3]:.3e}")
    tol = TOL[dtype]
    assert worst[0] < tol and worst[1] < tol and worst[2] < tol and worst[3] < DELTA_TOL[dtype]


@pytest.mark.parametrize("name", sorted(MASKS))
def test_bf16_range_bwd_parity(name):
    _parity(500 + sorted(MASKS).index(name), name)


@pytest.mark.parametrize("name", ["gaps", "tf_c1_4_t50", "stripes"])
def test_bf16_range_bwd_parity_d64(name):
    _parity(510, name, d=64)


@pytest.mark.parametrize("name", ["gaps", "tf_c1_2_t16", "multi", "stripes"])
def test_fp32_range_bwd_parity(name):
    _parity(520, name, d=64, dtype="fp32")


def _same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("desc", [(50, 5, 1, 1), (160, 9, 3, 1), (37, 7, 1, 0), (1, 5, 1, 1), (64, 4, 1, 1)])
@pytest.mark.parametrize("d, dtype", [(128, "bf16"), (64, "bf16"), (64, "fp32")])
def test_chunked_mask_as_ranges_bwd_is_bit_identical_to_descriptor(desc, d, dtype):
    tpf, f, c, tf = desc
    w = small_workload(530, tpf, f, c, tf, heads=2, d=d, dtype=dtype)
    x = _inputs(w)
    ref = _run_desc(w, x)
    n, groups = si.chunked_mask_ranges(tpf, (c,) * (f // c), tf)
    got = _run_ranges(x, groups)
    for a, b in zip(ref[:4], got[:4]):
        assert _same_bits(a, b)


def test_full_workload_as_ranges_bwd_is_bit_identical_to_descriptor():
    w = WORKLOADS[3]
    log(f"[range bwd equivalence] {w.name}")
    x = _inputs(w)
    ref = _run_desc(w, x)
    n, groups = w.mask_ranges()
    got = _run_ranges(x, groups)
    for a, b in zip(ref[:4], got[:4]):
        assert _same_bits(a, b)


def test_c1_4_workload_bwd_sampled():
    """Full c1-4 workload: dq and delta on sampled rows; dk and dv of the keys
    of the last chunk of each side, whose attending rows all lie in that
    chunk (the oracle takes those rows whole)."""
    w = si.RANGE_WORKLOADS[6]
    n, groups = w.mask_ranges()
    rm = RangeMask(n, groups)
    log(f"[range bwd sampled] {w.name}")
    x = _inputs(w)
    dq, dk, dv, ws, _ = _run_ranges(x, groups)
    assert torch.isfinite(dq).all().item() and torch.isfinite(dk).all().item() and torch.isfinite(dv).all().item()
    T, nh = w.tokens_per_frame, w.tokens_per_side
    rows = set(sample_rows((T, 21, 1, 1), n_random=8, seed=6).tolist())
    for side in (0, 1):  # chunk edges at 0, 1, 5, 9, 13, 17 frames
        for fr in (0, 1, 5, 17):
            rows.update([side * nh + fr * T, side * nh + fr * T + T - 1])
    rows = np.array(sorted(r for r in rows if r < n))
    b, h = 0, w.heads - 1
    sl = _slices(w, b, h)
    rq, _, _, rd = oracle.masked_attention_bwd_rows(*sl, rm, rows)
    e_q = rel_err(to_f64(dq[b, h, rows]), rq)
    e_d = rel_err(-to_f64(ws[b, h, 0, rows]), rd)
    log(f"    {len(rows)} rows: dq {e_q:.3e} delta {e_d:.3e}")
    assert e_q < TOL["bf16"] and e_d < DELTA_TOL["bf16"]
    last = 4 * T  # the last chunk holds four frames
    for side in (0, 1):
        chunk = np.arange(side * nh + nh - last, side * nh + nh)
        _, rk, rv, _ = oracle.masked_attention_bwd_rows(*sl, rm, chunk)
        e_k = rel_err(to_f64(dk[b, h, chunk]), rk[chunk])
        e_v = rel_err(to_f64(dv[b, h, chunk]), rv[chunk])
        log(f"    side {side} last-chunk keys: dk {e_k:.3e} dv {e_v:.3e}")
        assert e_k < TOL["bf16"] and e_v < TOL["bf16"]


def test_range_bwd_run_to_run_bitwise_determinism():
    n, groups = MASKS["multi"]
    x = _inputs(small_workload(540, n, 1, 1, 0, heads=2))
    runs = [_run_ranges(x, groups)[:4] for _ in range(3)]
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert _same_bits(a, b)


def test_range_bwd_gpu_error_paths():
    n, groups = MASKS["gaps"]
    w = small_workload(550, n, 1, 1, 0)
    x = _inputs(w)
    plan = aj.attn_jvp_create_ranges(n, groups, w.batch, w.heads, w.head_dim)
    table = torch.from_numpy(aj.attn_jvp_plan_table(plan)).cuda()
    o = torch.empty_like(x["q"])
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device="cuda")
    ws = torch.empty(aj.attn_jvp_bwd_workspace_size(plan) // 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))
    with pytest.raises(aj.AttnJvpError):  # descriptor entry point on a range plan
        aj.attn_jvp_bwd(plan, x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, ws)
    with pytest.raises(aj.AttnJvpError) as e:  # dk aliases dq
        aj.attn_jvp_bwd_table(plan, table, x["q"], x["k"], x["v"], o, lse, x["do"], dq, dq, dv, ws)
    assert e.value.code == 1
    with pytest.raises(aj.AttnJvpError):  # table too short
        aj.attn_jvp_bwd_table(plan, table[:4], x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, ws)


@pytest.mark.parametrize("name, dtype, d", [("gaps", "bf16", 128), ("tf_c1_4_t50", "bf16", 64), ("stripes", "fp32", 64)])
def test_range_batch_and_heads_are_independent(name, dtype, d):
    # B = 2, H = 3: the table kernels map workgroups to (b, h) slices through
    # the XCD-grouped order over the whole grid; every slice against the oracle
    n, groups = MASKS[name]
    w = small_workload(560, n, 1, 1, 0, heads=3, batch=2, d=d, dtype=dtype)
    log(f"[range batch x heads] {name} N={n} d={d} {dtype}")
    x = _inputs(w)
    o, to, lse = (to_f64(t) for t in aj.masked_attention_jvp_ranges(*(x[t] for t in TENSORS), groups,
                                                                       return_lse=True))
    po = to_f64(aj.masked_attention_fwd_ranges(x["q"], x["k"], x["v"], groups))
    dq, dk, dv, _, _ = (to_f64(t) for t in _run_ranges(x, groups))
    rm = RangeMask(n, groups)
    tol = TOL[dtype]
    for b in range(w.batch):
        for h in range(w.heads):
            sl = host_values(w, b, h)
            ro, rto, _ = oracle.masked_attention_jvp_slice(*sl, rm)
            rq, rk, rv, _ = oracle.masked_attention_bwd_slice(*sl[:3], si.slice_values(w, "do", b, h), rm)
            assert np.array_equal(po[b, h], o[b, h])  # the primal forward gives the same o
            for got, ref in ((o, ro), (to, rto), (dq, rq), (dk, rk), (dv, rv)):
                assert rel_err(got[b, h], ref) < tol, (b, h)
