"""Large scores, through the C ABI: the online softmax's rescaling.

The kernels keep a per-row reference max and rescale l, r and the output
accumulators only when a tile's max passes it by more than 2^8 (exp2 units),
and the backward recomputes P from the forward's lse.  The seeded workloads
(RMS-normalised q, k) hardly ever move the reference after the first tile,
so these cases drive it on purpose:

* scaled queries: q ~ N(0, 8^2) per element, so scores are N(0, 64) and the
  row maxima jump by more than 2^8 between tiles now and then;
* a ramp along the keys: q and every key share a direction e, with k_j . e
  growing linearly in j, so that each 32-key tile's scores pass the previous
  tile's by more than 2^8 (after the softmax scale and log2(e)): the
  reference moves on every tile of every row, and p concentrates on the
  last keys a row sees.  tq and tk keep their components along e, so tq.k
  carries a ramp too: over the few keys a row weighs most, the (scaled)
  score tangents share a part of up to about 6.5 (d = 128, last rows) next
  to a spread of about 0.1 among them.  t_o is the p-weighted spread of ts
  times v (eq. 45: the shared part cancels between acc_tsv / l and (r / l) o),
  so this is the case where rounding p~ ts to bf16 as an MFMA operand would
  lose t_o; the kernels round p~ (ts - c) with a per-row centre c instead
  (exact in eq. 45).

A third case isolates that cancellation: every key's tangent shares one
large component (tk_j = tk0_j + g u for a unit vector u, g = 64 and 1024), so
the score tangents of row i share sigma g (q_i . u), of order 90 at g = 1024,
a part that contributes exactly nothing to t_o.

Forward + JVP, the forward without tangents and the backward are compared
with the fp64 oracle on the same rounded values (bf16 within 1e-2, fp32
within 1e-4 normwise).  lse is held to atol + rtol |lse|: an fp32 score of
magnitude |s| carries rounding of order 1e-7 |s| from each operation that
forms it, so at |lse| near 265 (the ramp) an fp32 evaluation of the plain
definition is already 8e-5 off; fp32: 1e-5 + 1e-6 |lse|, bf16: 2e-2 +
1e-4 |lse|.

One exception, bf16 dq on the ramp.  Each row of dS = P (dP - delta) sums
to zero exactly, and dq_i = scale sum_j dS_ij k_j; with the ramp every key
carries a large common component along e (up to about 740), so dq lives on
that cancellation.  Rounding dS to bf16 for the dS k product (unit roundoff
2^-9) breaks it and moves dq_i by up to 2^-9 scale sum_j |dS_ij| |k_j|,
about a tenth of |dq| here, for any kernel that feeds dS to the matrix unit
in bf16.  That dq is held to twice this rounding bound (Frobenius norms)
instead, and the fp32 plan to the normwise 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
import masked_attention_jvp_amd as aj
from gpu_util import log, to_f64, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


DESC = (96, 7, 1, 1)  # teacher forcing, 7 frames of 96 tokens: N = 1344, partial tiles on both sides
TOL = {"bf16": 1e-2, "fp32": 1e-4}
LSE_TOL = {"bf16": (2e-2, 1e-4), "fp32": (1e-5, 1e-6)}  # (atol, rtol)


def _dq_rounding_bound(q, k, v, do, lse, desc):
    """Frobenius norm of 2^-9 scale |dS| |K| (the definition's dS, fp64)."""
    d = q.shape[1]
    scale = 1.0 / np.sqrt(d)
    allowed = oracle.mask_dense(desc)
    p = np.where(allowed, np.exp(scale * (q @ k.T) - lse[:, None]), 0.0)
    dp = do @ v.T
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    return float(np.linalg.norm(2.0 ** -9 * scale * (np.abs(ds) @ np.abs(k))))


def _inputs(kind, n, d, heads, dtype, seed, common=0.0):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    q, k, v = f(heads, n, d), f(heads, n, d), f(heads, n, d)
    tq, tk, tv = (0.1 * f(heads, n, d) for _ in range(3))
    do = f(heads, n, d)
    if kind == "scaled":
        q *= 8.0
    elif kind == "ramp":  # along e = first axis, q . e = 4 and k_j . e = slope * j
        # per key the score grows by 4 slope / sqrt(d); 9 exp2 units per 32 keys
        slope = 9.0 / 32 / np.log2(np.e) * np.sqrt(d) / 4.0
        q[:, :, 0] = 4.0
        k[:, :, 0] = slope * np.arange(n, dtype=np.float32)
    else:  # common: every key tangent shares common * u (per head, unit u)
        u = f(heads, 1, d)
        u /= np.linalg.norm(u, axis=2, keepdims=True)
        tk += np.float32(common) * u
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = {name: torch.from_numpy(a[None]).to(tdt) for name, a in
           (("q", q), ("k", k), ("v", v), ("tq", tq), ("tk", tk), ("tv", tv), ("do", do))}
    host = {name: t[0].double().numpy() for name, t in dev.items()}  # the rounded values
    return {name: t.cuda() for name, t in dev.items()}, host


@pytest.mark.parametrize("kind", ["scaled", "ramp"])
@pytest.mark.parametrize("dtype, d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_large_scores_forward_jvp_primal_backward(kind, dtype, d):
    tpf, f, c, tf = DESC
    n = tpf * f * (1 + tf)
    heads = 2
    x, hv = _inputs(kind, n, d, heads, dtype, seed=900 + d + (kind == "ramp"))
    o, to, lse = aj.masked_attention_jvp(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], DESC, return_lse=True)
    po, plse = aj.masked_attention_fwd(x["q"], x["k"], x["v"], DESC, return_lse=True)
    dq, dk, dv = aj.masked_attention_bwd(x["q"], x["k"], x["v"], o, lse, x["do"], DESC)
    torch.cuda.synchronize()
    bits = (lambda t: t.view(torch.int16)) if dtype == "bf16" else (lambda t: t.view(torch.int32))
    assert torch.equal(bits(po), bits(o)) and torch.equal(plse, lse)
    for h in range(heads):
        sl = [hv[t][h] for t in ("q", "k", "v", "tq", "tk", "tv")]
        ro, rto, rl = oracle.masked_attention_jvp_slice(*sl, DESC)
        rq, rk, rv, _ = oracle.masked_attention_bwd_slice(*sl[:3], hv["do"][h], DESC)
        errs = {"o": rel_err(to_f64(o[0, h]), ro), "to": rel_err(to_f64(to[0, h]), rto),
                "dq": rel_err(to_f64(dq[0, h]), rq), "dk": rel_err(to_f64(dk[0, h]), rk),
                "dv": rel_err(to_f64(dv[0, h]), rv)}
        atol, rtol = LSE_TOL[dtype]
        dl = float(np.max(np.abs(to_f64(lse[0, h]) - rl) / (atol + rtol * np.abs(rl))))
        log(f"[{kind} {dtype} d={d} h={h}] max |lse| {np.max(np.abs(rl)):.1f}; "
            + " ".join(f"{k} {e:.2e}" for k, e in errs.items()) + f" lse error / bound {dl:.2f}")
        if dtype == "bf16" and kind == "ramp":
            bound = _dq_rounding_bound(*sl[:3], hv["do"][h], rl, DESC)
            adq = float(np.linalg.norm(to_f64(dq[0, h]) - rq))
            log(f"    dq: |error| {adq:.3e} against the bf16 rounding bound {bound:.3e} (|dq| {np.linalg.norm(rq):.3e})")
            assert adq < 2.0 * bound
            del errs["dq"]
        assert max(errs.values()) < TOL[dtype], errs
        assert dl < 1.0
        assert all(torch.isfinite(t).all().item() for t in (o, to, lse, dq, dk, dv))


def test_large_scores_range_list_ramp():
    """The ramp on a range-list mask (teacher forcing with a one-frame first
    chunk, then chunks of 3 frames): the schedule-table kernels share the
    rescaling but stage their tiles and masks from the table."""
    import seeded_inputs as si
    n, groups = si.chunked_mask_ranges(96, (1, 3, 3), 1)
    rm = oracle.RangeMask(n, groups)
    d, heads = 128, 2
    x, hv = _inputs("ramp", n, d, heads, "bf16", seed=950)
    o, to, lse = aj.masked_attention_jvp_ranges(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], groups,
                                                return_lse=True)
    po, plse = aj.masked_attention_fwd_ranges(x["q"], x["k"], x["v"], groups, return_lse=True)
    dq, dk, dv = aj.masked_attention_bwd_ranges(x["q"], x["k"], x["v"], o, lse, x["do"], groups)
    torch.cuda.synchronize()
    assert torch.equal(po.view(torch.int16), o.view(torch.int16)) and torch.equal(plse, lse)
    atol, rtol = LSE_TOL["bf16"]
    for h in range(heads):
        sl = [hv[t][h] for t in ("q", "k", "v", "tq", "tk", "tv")]
        ro, rto, rl = oracle.masked_attention_jvp_slice(*sl, rm)
        rq, rk, rv, _ = oracle.masked_attention_bwd_slice(*sl[:3], hv["do"][h], rm)
        errs = {"o": rel_err(to_f64(o[0, h]), ro), "to": rel_err(to_f64(to[0, h]), rto),
                "dk": rel_err(to_f64(dk[0, h]), rk), "dv": rel_err(to_f64(dv[0, h]), rv)}
        adq = float(np.linalg.norm(to_f64(dq[0, h]) - rq))
        bound = _dq_rounding_bound(*sl[:3], hv["do"][h], rl, rm)
        dl = float(np.max(np.abs(to_f64(lse[0, h]) - rl) / (atol + rtol * np.abs(rl))))
        log(f"[range ramp h={h}] max |lse| {np.max(np.abs(rl)):.1f}; "
            + " ".join(f"{k} {e:.2e}" for k, e in errs.items())
            + f" dq |error| {adq:.3e} (bound {bound:.3e}) lse error / bound {dl:.2f}")
        assert max(errs.values()) < TOL["bf16"], errs
        assert adq < 2.0 * bound and dl < 1.0


@pytest.mark.parametrize("common", [64.0, 1024.0])
@pytest.mark.parametrize("dtype, d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_common_key_tangent_cancels(common, dtype, d):
    """tk_j = tk0_j + g u: the score tangents of row i share sigma g (q_i . u),
    which drops out of t_o (eq. 45); t_o must still match the oracle."""
    tpf, f, c, tf = DESC
    n = tpf * f * (1 + tf)
    heads = 2
    x, hv = _inputs("common", n, d, heads, dtype, seed=970 + d, common=common)
    o, to, lse = aj.masked_attention_jvp(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], DESC, return_lse=True)
    to_ctz = aj.masked_attention_jvp(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], DESC,
                                     clean_tangent_zero=True)[1]
    torch.cuda.synchronize()
    for h in range(heads):
        sl = [hv[t][h] for t in ("q", "k", "v", "tq", "tk", "tv")]
        ro, rto, _ = oracle.masked_attention_jvp_slice(*sl, DESC)
        _, rto_ctz, _ = oracle.masked_attention_jvp_slice_ctz(*sl, DESC)
        eo, eto = rel_err(to_f64(o[0, h]), ro), rel_err(to_f64(to[0, h]), rto)
        eto_ctz = rel_err(to_f64(to_ctz[0, h]), rto_ctz)
        log(f"[common {common:g} {dtype} d={d} h={h}] rel err o {eo:.2e} to {eto:.2e} to (clean tangent zero) "
            f"{eto_ctz:.2e}")
        assert eo < TOL[dtype] and eto < TOL[dtype] and eto_ctz < TOL[dtype]
