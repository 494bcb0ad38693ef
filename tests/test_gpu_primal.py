"""GPU checks of the forward without tangents (attn_jvp_fwd_primal) through
the C ABI: o and lse must be bit-identical to those of the forward + JVP
(same products, same online softmax), which the oracle parity tests cover;
plus direct oracle parity at full workload size on sampled rows, the
backward fed from it, and error paths."""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import masked_attention_jvp_amd as aj
from seeded_inputs import TENSORS, WORKLOADS
from gpu_util import log, small_workload, device_inputs, host_values, to_device, to_f64, rel_err, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("geom", [(50, 5, 1, 1, 128, "bf16"), (40, 6, 3, 1, 128, "bf16"), (37, 7, 1, 0, 128, "bf16"),
                                  (130, 3, 1, 1, 64, "bf16"), (1, 5, 1, 1, 128, "bf16"), (48, 4, 2, 1, 128, "fp32"),
                                  (33, 5, 5, 0, 64, "fp32")])
def test_primal_is_bit_identical_to_the_jvp_forward(geom):
    tpf, f, c, tf, d, dtype = geom
    w = small_workload(400, tpf, f, c, tf, heads=2, d=d, dtype=dtype)
    x = device_inputs(w)
    o_ref, _, lse_ref = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc, return_lse=True)
    o, lse = aj.masked_attention_fwd(x["q"], x["k"], x["v"], w.desc, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(o_ref)) and torch.equal(_bits(lse), _bits(lse_ref))


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_primal_workload(cfg):
    w = WORKLOADS[cfg]
    log(f"[primal] {w.name}")
    x = device_inputs(w)
    o, lse = aj.masked_attention_fwd(x["q"], x["k"], x["v"], w.desc, return_lse=True)
    torch.cuda.synchronize()
    if cfg == 3:  # bit-identical to the forward + JVP at full size
        o_ref, _, lse_ref = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(_bits(o), _bits(o_ref)) and torch.equal(_bits(lse), _bits(lse_ref))
    rows = sample_rows(w.desc, seed=40 + cfg)
    b, h = w.batch - 1, w.heads - 1
    ro, _, rl = oracle.masked_attention_jvp_rows(host_values(w, b, h), w.desc, rows)
    e = rel_err(to_f64(o[b, h, rows]), ro)
    log(f"    {len(rows)} rows: rel err o={e:.3e}")
    assert e < 1e-2 and np.max(np.abs(to_f64(lse[b, h, rows]) - rl)) < 2e-2


def test_backward_from_the_primal_forward():
    # the backward needs o and lse only: feeding it the primal forward's gives the same bits
    w = small_workload(410, 160, 9, 3, 1, heads=2)
    x = device_inputs(w)
    do = to_device(w, si.full_tensor_bits(w, "do"))
    o, lse = aj.masked_attention_fwd(x["q"], x["k"], x["v"], w.desc, return_lse=True)
    g1 = aj.masked_attention_bwd(x["q"], x["k"], x["v"], o, lse, do, w.desc)
    z = torch.zeros_like(x["q"])
    o2, _, lse2 = aj.masked_attention_jvp(x["q"], x["k"], x["v"], z, z, z, w.desc, return_lse=True)
    g2 = aj.masked_attention_bwd(x["q"], x["k"], x["v"], o2, lse2, do, w.desc)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(_bits(a), _bits(b))


def test_primal_error_paths():
    w = small_workload(420, 16, 3, 1, 1)
    x = device_inputs(w)
    plan = aj.attn_jvp_create(w.desc, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16)
    with pytest.raises(aj.AttnJvpError) as e:  # o aliasing k
        aj.attn_jvp_fwd_primal(plan, x["q"], x["k"], x["v"], x["k"])
    assert e.value.code == 1
    big = torch.empty(x["q"].numel() + 8, dtype=torch.bfloat16, device="cuda")
    mis = big[1:1 + x["q"].numel()].view(x["q"].shape)
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_fwd_primal(plan, x["q"], x["k"], x["v"], mis)
    assert e.value.code == 3


RANGE_MASKS = {
    "tf_c1_4_t50": si.chunked_mask_ranges(50, (1, 4, 4), 1),
    "und_gen": si.und_gen_ranges(20, 5, 30),
    "gaps": (40, ((0, 6, ((0, 3), (10, 14))), (9, 15, ((0, 40),)), (15, 33, ((5, 6), (20, 33))),
                  (35, 40, ((1, 2),)))),
    "multi": (170, ((0, 60, ((0, 3), (37, 39), (72, 100), (133, 140))), (60, 170, ((0, 170),)))),
}


@pytest.mark.parametrize("name", sorted(RANGE_MASKS))
@pytest.mark.parametrize("d, dtype", [(128, "bf16"), (64, "bf16"), (64, "fp32")])
def test_range_primal_is_bit_identical_to_the_range_jvp_forward(name, d, dtype):
    n, groups = RANGE_MASKS[name]
    w = small_workload(430, n, 1, 1, 0, heads=2, d=d, dtype=dtype)
    x = device_inputs(w)
    o_ref, _, lse_ref = aj.masked_attention_jvp_ranges(*(x[t] for t in TENSORS), groups, return_lse=True)
    o, lse = aj.masked_attention_fwd_ranges(x["q"], x["k"], x["v"], groups, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(o_ref)) and torch.equal(_bits(lse), _bits(lse_ref))


def test_range_primal_c1_4_workload():
    w = si.RANGE_WORKLOADS[6]
    n, groups = w.mask_ranges()
    log(f"[range primal] {w.name}")
    x = device_inputs(w)
    o_ref, _, lse_ref = aj.masked_attention_jvp_ranges(*(x[t] for t in TENSORS), groups, return_lse=True)
    o, lse = aj.masked_attention_fwd_ranges(x["q"], x["k"], x["v"], groups, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(o_ref)) and torch.equal(_bits(lse), _bits(lse_ref))


def test_range_primal_error_paths():
    n, groups = RANGE_MASKS["gaps"]
    w = small_workload(440, n, 1, 1, 0)
    x = device_inputs(w)
    plan = aj.attn_jvp_create_ranges(n, groups, w.batch, w.heads, w.head_dim)
    table = torch.from_numpy(aj.attn_jvp_plan_table(plan)).cuda()
    o = torch.empty_like(x["q"])
    with pytest.raises(aj.AttnJvpError):  # the descriptor entry point on a range plan
        aj.attn_jvp_fwd_primal(plan, x["q"], x["k"], x["v"], o)
    with pytest.raises(aj.AttnJvpError) as e:  # o aliasing v
        aj.attn_jvp_fwd_primal_table(plan, table, x["q"], x["k"], x["v"], x["v"])
    assert e.value.code == 1
    with pytest.raises(aj.AttnJvpError):  # table too short
        aj.attn_jvp_fwd_primal_table(plan, table[:4], x["q"], x["k"], x["v"], o)


@pytest.mark.parametrize("n_tiles", [3968, 3969])
def test_range_primal_at_the_two_workgroup_entry_limit(n_tiles):
    """Range-list plans run the primal-only forward at two workgroups per CU
    when no query block streams more than 3968 key tiles, and the
    one-workgroup instance otherwise: one block of 128 rows sees all keys,
    the others one tile.  Both sides of the limit give o and lse of the
    forward + JVP bit for bit."""
    n = 32 * n_tiles
    groups = ((0, 128, ((0, n),)), (128, n, ((0, 32),)))
    w = small_workload(431, n, 1, 1, 0, heads=1, d=64)
    log(f"[range primal] entry limit: {n} tokens, {n_tiles} tiles in the first block")
    x = device_inputs(w)
    o_ref, _, lse_ref = aj.masked_attention_jvp_ranges(*(x[t] for t in TENSORS), groups, return_lse=True)
    o, lse = aj.masked_attention_fwd_ranges(x["q"], x["k"], x["v"], groups, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(_bits(o), _bits(o_ref)) and torch.equal(_bits(lse), _bits(lse_ref))
    assert not torch.isnan(o.float()).any()
