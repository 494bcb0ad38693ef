"""An explicit softmax scale, through the C ABI (attn_jvp_create's
softmax_scale; reading 1: the scale multiplies the scores and their tangent
alike).  The default 1/sqrt(d) is what every other test uses; here the
forward + JVP, the forward without tangents, the backward and a range-list
plan run with two other scales against the oracle given the same scale, and
the plan built with scale 1/sqrt(d) spelled out equals the default bit for
bit.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
import masked_attention_jvp_amd as aj
from seeded_inputs import TENSORS
from gpu_util import log, small_workload, device_inputs, host_values, to_device, to_f64, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


TOL = {"bf16": 1e-2, "fp32": 1e-4}
LSE_TOL = {"bf16": 2e-2, "fp32": 1e-5}


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("scale", [0.3, 0.02])
@pytest.mark.parametrize("dtype, d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_explicit_scale(scale, dtype, d):
    w = small_workload(960, 40, 6, 2, 1, heads=2, d=d, dtype=dtype)
    x = device_inputs(w)
    x["do"] = to_device(w, si.full_tensor_bits(w, "do"))
    o, to, lse = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc, scale=scale, return_lse=True)
    po, plse = aj.masked_attention_fwd(x["q"], x["k"], x["v"], w.desc, scale=scale, return_lse=True)
    dq, dk, dv = aj.masked_attention_bwd(x["q"], x["k"], x["v"], o, lse, x["do"], w.desc, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(_bits(po), _bits(o)) and torch.equal(plse, lse)
    for h in range(w.heads):
        sl = host_values(w, 0, h)
        ro, rto, rl = oracle.masked_attention_jvp_slice(*sl, w.desc, scale=scale)
        rq, rk, rv, _ = oracle.masked_attention_bwd_slice(*sl[:3], si.slice_values(w, "do", 0, h), w.desc,
                                                          scale=scale)
        errs = {"o": rel_err(to_f64(o[0, h]), ro), "to": rel_err(to_f64(to[0, h]), rto),
                "dq": rel_err(to_f64(dq[0, h]), rq), "dk": rel_err(to_f64(dk[0, h]), rk),
                "dv": rel_err(to_f64(dv[0, h]), rv)}
        dl = float(np.max(np.abs(to_f64(lse[0, h]) - rl)))
        log(f"[scale {scale} {dtype} d={d} h={h}] " + " ".join(f"{k} {e:.2e}" for k, e in errs.items())
            + f" |dlse| {dl:.2e}")
        assert max(errs.values()) < TOL[dtype] and dl < LSE_TOL[dtype], errs


@pytest.mark.parametrize("dtype, d", [("bf16", 128), ("fp32", 64)])
def test_explicit_scale_range_list(dtype, d):
    n, groups = si.chunked_mask_ranges(40, (1, 2, 3), 1)
    w = small_workload(961, n, 1, 1, 0, heads=2, d=d, dtype=dtype)
    x = device_inputs(w)
    scale = 0.3
    o, to, lse = aj.masked_attention_jvp_ranges(*(x[t] for t in TENSORS), groups, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    rm = oracle.RangeMask(n, groups)
    for h in range(w.heads):
        ro, rto, rl = oracle.masked_attention_jvp_slice(*host_values(w, 0, h), rm, scale=scale)
        eo, eto = rel_err(to_f64(o[0, h]), ro), rel_err(to_f64(to[0, h]), rto)
        log(f"[range scale {scale} {dtype} h={h}] o {eo:.2e} to {eto:.2e}")
        assert eo < TOL[dtype] and eto < TOL[dtype]
        assert np.max(np.abs(to_f64(lse[0, h]) - rl)) < LSE_TOL[dtype]


def test_default_scale_spelled_out_is_bitwise_the_default():
    w = small_workload(962, 40, 6, 2, 1, heads=2, d=128)
    x = device_inputs(w)
    a = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc, return_lse=True)
    b = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc, scale=1.0 / np.sqrt(128.0), return_lse=True)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(_bits(u), _bits(v))
