"""GPU parity of clean-tangent-zero plans (Causal-rCM section 3.1.2, text
after eq. 17: the clean context carries zero tangent).

* against the oracle (the general definition with the clean tangents zeroed),
  to the same tolerances as the general path;
* against the general HIP path run on inputs whose clean tangents are zero:
  o and lse bit for bit, t_o value for value (only the sign of an exact zero
  may differ, as the general path adds zero products);
* the clean halves of tq, tk, tv are never read: NaN there changes nothing;
* clean rows get t_o exactly zero.
"""
import numpy as np
import pytest
import torch

import oracle
import masked_attention_jvp_amd as aj
from seeded_inputs import WORKLOADS, TENSORS
from gpu_util import (log, small_workload, device_inputs, host_values, to_f64, rel_err, sample_rows)

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp32": 1e-4}
LSE_TOL = {"bf16": 2e-2, "fp32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _run(w, x, ctz):
    o, to, lse = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc, return_lse=True, clean_tangent_zero=ctz)
    torch.cuda.synchronize()
    return o, to, lse


def _with_clean_tangents(w, x, value):
    y = dict(x)
    for t in ("tq", "tk", "tv"):
        y[t] = x[t].clone()
        y[t][:, :, : w.tokens_per_side] = value
    return y


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


SMALL = [
    # id, tokens_per_frame, n_frames, frames_per_chunk, d
    (201, 50, 5, 1, 128),   # ragged blocks and tiles, frame-wise
    (202, 40, 6, 3, 128),   # chunk-wise
    (203, 130, 3, 1, 64),   # head_dim 64
    (204, 1, 5, 1, 128),    # 10 tokens: far smaller than one block
    (205, 64, 4, 1, 128),   # frame == one tile: the halves meet on a tile edge
    (206, 160, 9, 3, 128),  # several chunks per side, many tiles
    (207, 37, 6, 1, 128),   # a tile straddles the clean / noisy boundary
]


@pytest.mark.parametrize("cid, tpf, f, c, d", SMALL, ids=[str(s[0]) for s in SMALL])
def test_ctz_small_parity_and_equivalences(cid, tpf, f, c, d):
    w = small_workload(cid, tpf, f, c, 1, heads=2, d=d)
    log(f"[ctz parity] {w.name} desc={w.desc} d={d}")
    x = device_inputs(w)
    o, to, lse = _run(w, x, True)
    nh = w.tokens_per_side
    # clean rows: exactly zero tangent output
    assert torch.count_nonzero(to[:, :, :nh].float()).item() == 0
    errs = []
    for b in range(w.batch):
        for h in range(w.heads):
            ro, rto, rl = oracle.masked_attention_jvp_slice_ctz(*host_values(w, b, h), w.desc)
            errs.append((rel_err(to_f64(o[b, h]), ro), rel_err(to_f64(to[b, h]), rto),
                         float(np.max(np.abs(to_f64(lse[b, h]) - rl)))))
    eo, eto, el = (max(e[i] for e in errs) for i in range(3))
    log(f"    max rel err o={eo:.3e} to={eto:.3e}  max |dlse|={el:.3e}")
    assert eo < TOL["bf16"] and eto < TOL["bf16"] and el < LSE_TOL["bf16"]
    # the general path on zeroed clean tangents
    g_o, g_to, g_lse = _run(w, _with_clean_tangents(w, x, 0.0), False)
    assert torch.equal(_bits(o), _bits(g_o)) and torch.equal(_bits(lse), _bits(g_lse))
    assert torch.equal(to.float(), g_to.float())
    # NaN in the clean halves is never read
    n_o, n_to, n_lse = _run(w, _with_clean_tangents(w, x, float("nan")), True)
    for a, b_ in ((o, n_o), (to, n_to), (lse, n_lse)):
        assert torch.equal(_bits(a), _bits(b_))


@pytest.mark.parametrize("cid, tpf, f, c, d", [(210, 48, 4, 2, 128), (211, 33, 5, 1, 64)])
def test_ctz_fp32_small_parity(cid, tpf, f, c, d):
    w = small_workload(cid, tpf, f, c, 1, heads=2, d=d, dtype="fp32")
    x = device_inputs(w)
    o, to, lse = _run(w, x, True)
    assert torch.count_nonzero(to[:, :, : w.tokens_per_side]).item() == 0
    for b in range(w.batch):
        for h in range(w.heads):
            ro, rto, rl = oracle.masked_attention_jvp_slice_ctz(*host_values(w, b, h), w.desc)
            assert rel_err(to_f64(o[b, h]), ro) < TOL["fp32"]
            assert rel_err(to_f64(to[b, h]), rto) < TOL["fp32"]
            assert np.max(np.abs(to_f64(lse[b, h]) - rl)) < LSE_TOL["fp32"]
    n_o, n_to, n_lse = _run(w, _with_clean_tangents(w, x, float("nan")), True)
    for a, b_ in ((o, n_o), (to, n_to), (lse, n_lse)):
        assert torch.equal(_bits(a), _bits(b_))


@pytest.mark.parametrize("cfg", [3, 4])
def test_ctz_workload_sampled_rows(cfg):
    w = WORKLOADS[cfg]
    log(f"[ctz sampled parity] {w.name}")
    x = device_inputs(w)
    o, to, lse = _run(w, x, True)
    assert torch.isfinite(o).all().item() and torch.isfinite(to).all().item()
    assert torch.count_nonzero(to[:, :, : w.tokens_per_side].float()).item() == 0
    rows = sample_rows(w.desc, seed=100 + cfg)
    go, gto, rgo, rgto = [], [], [], []
    for b, h in [(0, 0), (w.batch - 1, w.heads - 1)]:
        ro, rto, rl = oracle.masked_attention_jvp_slice_ctz(*host_values(w, b, h), w.desc, rows=rows)
        go.append(to_f64(o[b, h, rows]))
        gto.append(to_f64(to[b, h, rows]))
        rgo.append(ro)
        rgto.append(rto)
        assert np.max(np.abs(to_f64(lse[b, h, rows]) - rl)) < LSE_TOL["bf16"]
    eo, eto = rel_err(np.stack(go), np.stack(rgo)), rel_err(np.stack(gto), np.stack(rgto))
    log(f"    {len(rows)} rows: rel err o={eo:.3e} to={eto:.3e}")
    assert eo < TOL["bf16"] and eto < TOL["bf16"]


def test_ctz_run_to_run_bitwise_determinism():
    w = small_workload(212, 160, 9, 3, 1, heads=2)
    x = device_inputs(w)
    runs = [_run(w, x, True) for _ in range(3)]
    for r in runs[1:]:
        for a, b_ in zip(runs[0], r):
            assert torch.equal(_bits(a), _bits(b_))
