"""GPU parity of range-list plans (query groups x key intervals) through the
C ABI (attn_jvp_fwd_table).

* against the fp64 oracle on the same RangeMask: normwise relative error
  1e-2 (bf16) / 1e-4 (fp32) on o and t_o, lse max abs 2e-2 / 1e-5; rows in
  no group give o = t_o = 0 exactly and lse = -inf;
* a chunked mask given as a range list runs the same arithmetic per row as
  the descriptor path (same key tiles in the same order; tiles a row does not
  see add exact zeros), so o, t_o and lse must be bit-identical to it -- at
  small ragged sizes and at the full 65520-token workload;
* the c1-4 workload (initial chunk of one frame, then four-frame chunks) at
  full size on sampled rows; determinism; an exact-zero probe on masks whose
  rows have up to four key intervals.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from oracle import RangeMask
import masked_attention_jvp_amd as aj
from seeded_inputs import TENSORS, WORKLOADS
from gpu_util import log, small_workload, device_inputs, host_values, to_f64, rel_err, sample_rows

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp32": 1e-4}
LSE_TOL = {"bf16": 2e-2, "fp32": 1e-5}

GAPS = (40, ((0, 6, ((0, 3), (10, 14))), (9, 15, ((0, 40),)), (15, 33, ((5, 6), (20, 33))), (35, 40, ((1, 2),))))
MULTI = (170, ((0, 60, ((0, 3), (37, 39), (72, 100), (133, 140))), (60, 170, ((0, 170),))))
MASKS = {
    "tf_c1_2_t16": si.chunked_mask_ranges(16, (1, 2, 2), 1),
    "tf_c1_4_t50": si.chunked_mask_ranges(50, (1, 4, 4), 1),
    "bc_c2_1_t37": si.chunked_mask_ranges(37, (2, 1, 1, 3), 0),
    "und_gen": si.und_gen_ranges(20, 5, 30),
    "dense_150": (150, ((0, 150, ((0, 150),)),)),
    "gaps": GAPS,
    "multi": MULTI,
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _workload_for(cid, n, heads=2, d=128, dtype="bf16", batch=1):
    # value recipe of a sequence of n tokens (the mask comes from the range list)
    return small_workload(cid, n, 1, 1, 0, heads=heads, batch=batch, d=d, dtype=dtype)


def _run(x, groups, return_lse=True):
    out = aj.masked_attention_jvp_ranges(*(x[t] for t in TENSORS), groups, return_lse=return_lse)
    torch.cuda.synchronize()
    return out


def _parity(cid, name, d=128, dtype="bf16"):
    n, groups = MASKS[name]
    w = _workload_for(cid, n, d=d, dtype=dtype)
    log(f"[range parity] {name} N={n} d={d} {dtype}")
    x = device_inputs(w)
    o, to, lse = (to_f64(t) for t in _run(x, groups))
    rm = RangeMask(n, groups)
    covered = oracle.mask_dense(rm).any(axis=1)
    worst = [0.0, 0.0, 0.0]
    for h in range(w.heads):
        ro, rto, rl = oracle.masked_attention_jvp_slice(*host_values(w, 0, h), rm)
        worst = [max(worst[0], rel_err(o[0, h], ro)), max(worst[1], rel_err(to[0, h], rto)),
                 max(worst[2], float(np.max(np.abs(lse[0, h, covered] - rl[covered]))))]
        assert np.all(o[0, h, ~covered] == 0) and np.all(to[0, h, ~covered] == 0)
        assert np.all(np.isneginf(lse[0, h, ~covered]))
    log(f"    rel err o={worst[0]:.3e} to={worst[1]:.3e} |dlse|={worst[2]:.3e}")
    assert worst[0] < TOL[dtype] and worst[1] < TOL[dtype] and worst[2] < LSE_TOL[dtype]


@pytest.mark.parametrize("name", sorted(MASKS))
def test_bf16_range_parity(name):
    _parity(300 + sorted(MASKS).index(name), name)


@pytest.mark.parametrize("name, d", [("gaps", 64), ("tf_c1_4_t50", 64)])
def test_bf16_range_parity_d64(name, d):
    _parity(310, name, d=d)


@pytest.mark.parametrize("name", ["gaps", "tf_c1_2_t16", "multi"])
def test_fp32_range_parity(name):
    _parity(320, name, d=64, dtype="fp32")


def _same_bits(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("desc", [(50, 5, 1, 1), (160, 9, 3, 1), (37, 7, 1, 0), (1, 5, 1, 1), (64, 4, 1, 1)])
@pytest.mark.parametrize("d, dtype", [(128, "bf16"), (64, "bf16"), (64, "fp32")])
def test_chunked_mask_as_ranges_is_bit_identical_to_descriptor(desc, d, dtype):
    tpf, f, c, tf = desc
    w = small_workload(330, tpf, f, c, tf, heads=2, d=d, dtype=dtype)
    x = device_inputs(w)
    ref = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc, return_lse=True)
    n, groups = si.chunked_mask_ranges(tpf, (c,) * (f // c), tf)
    got = _run(x, groups)
    for a, b in zip(ref, got):
        assert _same_bits(a, b)


def test_full_workload_as_ranges_is_bit_identical_to_descriptor():
    w = WORKLOADS[3]
    log(f"[range equivalence] {w.name}")
    x = device_inputs(w)
    ref = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc, return_lse=True)
    n, groups = w.mask_ranges()
    got = _run(x, groups)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert _same_bits(a, b)


def test_c1_4_workload_sampled_rows():
    w = si.RANGE_WORKLOADS[6]
    n, groups = w.mask_ranges()
    rm = RangeMask(n, groups)
    log(f"[range sampled] {w.name}")
    x = device_inputs(w)
    o, to, lse = _run(x, groups)
    assert torch.isfinite(o).all().item() and torch.isfinite(to).all().item()
    T = w.tokens_per_frame
    rows = set(sample_rows((T, 21, 1, 1), n_random=12, seed=6).tolist())
    for side in (0, 1):  # the first chunk (one frame) and the chunk edges at 1, 5, 9, ... frames
        for fr in (0, 1, 5, 9, 17, 20):
            rows.update([side * 21 * T + fr * T, side * 21 * T + fr * T + T - 1])
    rows = np.array(sorted(r for r in rows if r < n))
    go, gto, ro_, rto_ = [], [], [], []
    for b, h in [(0, 0), (0, w.heads - 1)]:
        ro, rto, rl = oracle.masked_attention_jvp_rows(host_values(w, b, h), rm, rows)
        go.append(to_f64(o[b, h, rows]))
        gto.append(to_f64(to[b, h, rows]))
        ro_.append(ro)
        rto_.append(rto)
        assert np.max(np.abs(to_f64(lse[b, h, rows]) - rl)) < LSE_TOL["bf16"]
    eo, eto = rel_err(np.stack(go), np.stack(ro_)), rel_err(np.stack(gto), np.stack(rto_))
    log(f"    {len(rows)} rows: rel err o={eo:.3e} to={eto:.3e}")
    assert eo < TOL["bf16"] and eto < TOL["bf16"]


def test_range_run_to_run_bitwise_determinism():
    n, groups = MASKS["multi"]
    x = device_inputs(_workload_for(340, n))
    runs = [_run(x, groups) for _ in range(3)]
    for r in runs[1:]:
        for a, b in zip(runs[0], r):
            assert _same_bits(a, b)


@pytest.mark.parametrize("name", ["gaps", "multi", "und_gen"])
def test_range_exact_zero_probe(name):
    # q = tq = tk = tv = 0 and v = one-hot key indicators: o[i, c] = p(i, key0 + c),
    # exactly 0 where the range list forbids the pair
    n, groups = MASKS[name]
    rm = RangeMask(n, groups)
    m = oracle.mask_dense(rm)
    d = 128
    z = torch.zeros((1, 1, n, d), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((1, 1, n, d), generator=torch.Generator().manual_seed(2)).to("cuda", torch.bfloat16)
    for key0 in range(0, n, d):
        v = torch.zeros_like(z)
        cols = torch.arange(d, device="cuda")
        keys = key0 + cols
        ok = keys < n
        v[0, 0, keys[ok], cols[ok]] = 1.0
        o, _ = aj.masked_attention_jvp_ranges(z, k, v, z, z, z, groups)
        torch.cuda.synchronize()
        nk = int(ok.sum())
        got = to_f64(o[0, 0])[:, :nk]
        want = m[:, key0:key0 + nk]
        assert np.all(got[~want] == 0.0)
        assert np.all(got[want] > 0.0)


def test_range_gpu_error_paths():
    n, groups = MASKS["gaps"]
    w = _workload_for(350, n)
    x = device_inputs(w)
    plan = aj.attn_jvp_create_ranges(n, groups, w.batch, w.heads, w.head_dim)
    table = torch.from_numpy(aj.attn_jvp_plan_table(plan)).cuda()
    o, to = torch.empty_like(x["q"]), torch.empty_like(x["q"])
    with pytest.raises(aj.AttnJvpError):  # descriptor entry point on a range plan
        aj.attn_jvp_fwd(plan, *(x[t] for t in TENSORS), o, to)
    with pytest.raises(aj.AttnJvpError) as e:  # output aliasing an input
        aj.attn_jvp_fwd_table(plan, table, *(x[t] for t in TENSORS), x["q"], to)
    assert e.value.code == 1
    with pytest.raises(aj.AttnJvpError):  # table too short
        aj.attn_jvp_fwd_table(plan, table[:4], *(x[t] for t in TENSORS), o, to)
