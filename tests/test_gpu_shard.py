"""One GPU's share under head sharding, through the C ABI.

Sharding by head leaves each GPU the full sequence and H / P heads: 3 of the
12 heads of the 65520-token teacher-forcing workload at P = 4.  That grid
(1536 query blocks) is too small for XCD-grouped rounds, so the kernels take
the blocks heavy first across the (b, h) slices instead, while the 12-head
grid keeps the grouped order (6 rounds).  Every block computes its own rows
(forward, dq) or keys (dk, dv) in a fixed order whatever the launch order,
so the 3-head results must equal the first 3 heads of the 12-head run bit
for bit; sampled rows of the last shard head are also checked against the
oracle.  The block-causal 32760-token workload (at 12 heads 3 rounds of
1024 workgroups: 2 grouped, the third in index order) gets the same check
on its forward.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import masked_attention_jvp_amd as aj
from seeded_inputs import TENSORS, WORKLOADS
from gpu_util import log, device_inputs, host_values, to_device, to_f64, rel_err, sample_rows

pytestmark = pytest.mark.gpu

SHARD_HEADS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _fwd(w, x):
    o, to, lse = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc, return_lse=True)
    torch.cuda.synchronize()
    return o, to, lse


@pytest.mark.parametrize("cfg", [3, 2])
def test_shard_forward_equals_the_full_grid_bitwise(cfg):
    full = WORKLOADS[cfg]
    shard = full.with_(heads=SHARD_HEADS)
    log(f"[shard] {full.name}: {SHARD_HEADS} of {full.heads} heads")
    x = device_inputs(full)
    o, to, lse = _fwd(full, x)
    xs = {t: x[t][:, :SHARD_HEADS].contiguous() for t in TENSORS}
    so, sto, slse = _fwd(shard, xs)
    for a, b in ((so, o), (sto, to), (slse, lse)):
        assert torch.equal(_bits(a), _bits(b[:, :SHARD_HEADS].contiguous()))
    if cfg == 3:
        # the primal-only kernel (two workgroups per CU) on the shard
        po, plse = aj.masked_attention_fwd(xs["q"], xs["k"], xs["v"], shard.desc, return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(_bits(po), _bits(so)) and torch.equal(_bits(plse), _bits(slse))
    h = SHARD_HEADS - 1
    rows = sample_rows(shard.desc, seed=70 + cfg)
    ro, rto, rl = oracle.masked_attention_jvp_rows(host_values(shard, 0, h), shard.desc, rows)
    eo, eto = rel_err(to_f64(so[0, h, rows]), ro), rel_err(to_f64(sto[0, h, rows]), rto)
    log(f"    head {h}, {len(rows)} rows: rel err o={eo:.3e} to={eto:.3e}")
    assert eo < 1e-2 and eto < 1e-2 and np.max(np.abs(to_f64(slse[0, h, rows]) - rl)) < 2e-2


def test_shard_backward_equals_the_full_grid_bitwise():
    full = WORKLOADS[3]
    shard = full.with_(heads=SHARD_HEADS)
    log(f"[shard bwd] {full.name}: {SHARD_HEADS} of {full.heads} heads")
    x = device_inputs(full)
    x["do"] = to_device(full, si.full_tensor_bits(full, "do"))
    o, _, lse = _fwd(full, x)
    grads = aj.masked_attention_bwd(x["q"], x["k"], x["v"], o, lse, x["do"], full.desc)
    torch.cuda.synchronize()
    sl = lambda t: t[:, :SHARD_HEADS].contiguous()
    sgrads = aj.masked_attention_bwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(o), sl(lse), sl(x["do"]), shard.desc)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), sgrads, grads):
        assert torch.equal(_bits(a), _bits(sl(b))), name


def test_shard_clean_tangent_zero_equals_the_full_grid_bitwise():
    """The clean-tangent-zero plan: XCD-grouped at 12 heads, index order at 3."""
    full = WORKLOADS[3]
    shard = full.with_(heads=SHARD_HEADS)
    x = device_inputs(full)
    args = [x[t] for t in TENSORS]
    o, to, lse = aj.masked_attention_jvp(*args, full.desc, return_lse=True, clean_tangent_zero=True)
    torch.cuda.synchronize()
    so, sto, slse = aj.masked_attention_jvp(*(a[:, :SHARD_HEADS].contiguous() for a in args), shard.desc,
                                            return_lse=True, clean_tangent_zero=True)
    torch.cuda.synchronize()
    for a, b in ((so, o), (sto, to), (slse, lse)):
        assert torch.equal(_bits(a), _bits(b[:, :SHARD_HEADS].contiguous()))
