"""Edge cases on the GPU, through the C ABI: the degenerate sizes and masks
of the method and the largest sequence the kernels' 32-bit buffer offsets
allow.

* single-key rows: N = 1 (one block-causal chunk) and N = 2 (teacher
  forcing with one frame per side), where every row sees one key, so o = v
  of that key exactly, in bf16 and fp32, and t_o and lse match the oracle;
  in the backward P = 1 and dS = 0: dv = dO up to one rounding and dq, dk
  vanish up to the rounding of dO.v - delta (exactly in fp32, where both
  sums run in the same order);
* a range-list plan with no group at all: every row is excluded, so the
  forward gives o = t_o = 0 and lse = -inf and the backward all zeros;
* the largest bf16 head at d = 128, N = 8388607 tokens (N d 2 bytes just
  under 2^31), as a block-diagonal range list of 4096-token groups (the last
  one ragged): the forward, the JVP and the backward of the first, a middle
  and the last two groups against the oracle.  A block-diagonal mask makes
  each group an independent dense problem, so the oracle runs on the
  group's rows and keys alone.
"""
import numpy as np
import pytest
import torch

import oracle
import masked_attention_jvp_amd as aj
from oracle import RangeMask
from gpu_util import log, small_workload, device_inputs, to_f64, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("desc", [(1, 1, 1, 0), (1, 1, 1, 1)])
@pytest.mark.parametrize("d, dtype", [(128, "bf16"), (64, "bf16"), (64, "fp32")])
def test_single_key_rows(desc, d, dtype):
    w = small_workload(600, *desc, heads=2, d=d, dtype=dtype)
    x = device_inputs(w)
    o, to, lse = aj.masked_attention_jvp(*(x[t] for t in ("q", "k", "v", "tq", "tk", "tv")), w.desc, return_lse=True)
    torch.cuda.synchronize()
    # row i sees key i only (N = 2: the noisy row sees its own token)
    assert torch.equal(_bits(o), _bits(x["v"]))
    tol = 1e-2 if dtype == "bf16" else 1e-4
    rto = np.empty(o.shape)
    rl = np.empty(lse.shape)
    for h in range(w.heads):
        sl = [to_f64(x[t][0, h]) for t in ("q", "k", "v", "tq", "tk", "tv")]
        _, rto[0, h], rl[0, h] = oracle.masked_attention_jvp_slice(*sl, w.desc)
    assert rel_err(to_f64(to), rto) < tol
    assert np.max(np.abs(to_f64(lse) - rl)) < (2e-2 if dtype == "bf16" else 1e-5)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(601)
    do = torch.randn(x["q"].shape, device="cuda", generator=gen).to(x["q"].dtype)
    dq, dk, dv = aj.masked_attention_bwd(x["q"], x["k"], x["v"], o, lse, do, w.desc)
    torch.cuda.synchronize()
    assert rel_err(to_f64(dv), to_f64(do)) < tol
    if dtype == "fp32":
        assert torch.count_nonzero(dq).item() == 0 and torch.count_nonzero(dk).item() == 0
    else:
        assert float(dq.abs().max()) < 1e-3 and float(dk.abs().max()) < 1e-3


def test_range_plan_without_groups_gives_zeros():
    n = 300
    w = small_workload(610, n, 1, 1, 0, heads=2)
    x = device_inputs(w)
    o, to, lse = aj.masked_attention_jvp_ranges(*(x[t] for t in ("q", "k", "v", "tq", "tk", "tv")), [],
                                                return_lse=True)
    do = torch.ones_like(x["q"])
    dq, dk, dv, ws = aj.masked_attention_bwd_ranges(x["q"], x["k"], x["v"], o, lse, do, [], return_workspace=True)
    torch.cuda.synchronize()
    for t in (o, to, dq, dk, dv):
        assert torch.count_nonzero(t).item() == 0
    assert torch.all(torch.isneginf(lse)).item()
    ws = ws.view(1, 2, 2, n)
    assert torch.count_nonzero(ws[:, :, 0]).item() == 0
    assert torch.all(ws[:, :, 1] == torch.finfo(torch.float32).min).item()


N_MAX = (2 ** 31 - 1) // (2 * 128)  # 8388607 tokens: one bf16 head of d = 128 just under 2^31 bytes
T_GROUP = 4096


def _big_inputs(n, d, seed):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    out = {}
    for name, std in (("q", 1.0), ("k", 1.0), ("v", 1.0), ("tq", 0.1), ("tk", 0.1), ("tv", 0.1), ("do", 1.0)):
        t = torch.randn((1, 1, n, d), device="cuda", generator=gen, dtype=torch.float32)
        out[name] = (t * std).to(torch.bfloat16)
        del t
    return out


def test_largest_sequence_block_diagonal():
    n, d = N_MAX, 128
    assert n * d * 2 < 2 ** 31 <= (n + 1) * d * 2 + 255
    n_groups = -(-n // T_GROUP)
    groups = [(g * T_GROUP, min((g + 1) * T_GROUP, n), [(g * T_GROUP, min((g + 1) * T_GROUP, n))])
              for g in range(n_groups)]
    log(f"[largest sequence] N={n} d={d}, {n_groups} block-diagonal groups of {T_GROUP}")
    x = _big_inputs(n, d, 20261203)
    plan = aj.attn_jvp_create_ranges(n, groups, 1, 1, d)
    table = torch.from_numpy(aj.attn_jvp_plan_table(plan)).cuda()
    o, to, dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(5))
    lse = torch.empty((1, 1, n), dtype=torch.float32, device="cuda")
    ws = torch.empty(aj.attn_jvp_bwd_workspace_size(plan) // 4, dtype=torch.float32, device="cuda")
    aj.attn_jvp_fwd_table(plan, table, *(x[t] for t in ("q", "k", "v", "tq", "tk", "tv")), o, to, lse)
    aj.attn_jvp_bwd_table(plan, table, x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, ws)
    torch.cuda.synchronize()
    dense = lambda m: RangeMask(m, [(0, m, [(0, m)])])
    for g in (0, n_groups // 2, n_groups - 2, n_groups - 1):
        lo, hi = groups[g][0], groups[g][1]
        sl = [to_f64(x[t][0, 0, lo:hi]) for t in ("q", "k", "v", "tq", "tk", "tv", "do")]
        ro, rto, rl = oracle.masked_attention_jvp_slice(*sl[:6], dense(hi - lo))
        rq, rk, rv, _ = oracle.masked_attention_bwd_slice(*sl[:3], sl[6], dense(hi - lo))
        errs = [rel_err(to_f64(o[0, 0, lo:hi]), ro), rel_err(to_f64(to[0, 0, lo:hi]), rto),
                rel_err(to_f64(dq[0, 0, lo:hi]), rq), rel_err(to_f64(dk[0, 0, lo:hi]), rk),
                rel_err(to_f64(dv[0, 0, lo:hi]), rv)]
        dl = float(np.max(np.abs(to_f64(lse[0, 0, lo:hi]) - rl)))
        log(f"    group {g} rows [{lo}, {hi}): o {errs[0]:.2e} to {errs[1]:.2e} dq {errs[2]:.2e} dk {errs[3]:.2e} "
            f"dv {errs[4]:.2e} |dlse| {dl:.2e}")
        assert max(errs) < 1e-2 and dl < 2e-2
