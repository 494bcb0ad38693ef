"""GPU parity of the masked-attention backward (dq, dk, dv) against the fp64
oracle, through the C ABI.

o and lse come from the library's own forward on the same inputs (the
forward is checked against the oracle elsewhere); the oracle computes the
backward from q, k, v and dO alone.  Tolerances (normwise relative error
over a slice): bf16 1e-2 -- inputs, P and dS enter the matrix cores rounded
to bf16 (relative 2^-9 each) and o is the forward's bf16 output, which
enters delta; fp32 1e-4.  The workspace's first plane (-delta) is compared
with the oracle's delta (bf16: 1e-2 normwise; fp32: 1e-5) and its second
plane with -lse log2(e) of the library's own lse (exact up to one rounding).
"""
import numpy as np
import pytest
import torch

import oracle
import masked_attention_jvp_amd as aj
import seeded_inputs as si
from seeded_inputs import WORKLOADS
from gpu_util import log, small_workload, device_inputs, host_values, to_device, to_f64, rel_err, sample_rows

pytestmark = pytest.mark.gpu

TOL = {"bf16": 1e-2, "fp32": 1e-4}
DELTA_TOL = {"bf16": 1e-2, "fp32": 1e-5}
LOG2E = 1.4426950408889634


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    aj._load()


def _inputs(w):
    x = device_inputs(w)
    x["do"] = to_device(w, si.full_tensor_bits(w, "do"))
    return x


def _run(w, x):
    z = torch.zeros_like(x["q"])
    o, _, lse = aj.masked_attention_jvp(x["q"], x["k"], x["v"], z, z, z, w.desc, return_lse=True)
    dq, dk, dv, ws = aj.masked_attention_bwd(x["q"], x["k"], x["v"], o, lse, x["do"], w.desc, return_workspace=True)
    torch.cuda.synchronize()
    return dq, dk, dv, ws.view(w.batch, w.heads, 2, w.seq_len), lse


def _slices(w, b, h):
    q, k, v = host_values(w, b, h)[:3]
    return q, k, v, si.slice_values(w, "do", b, h)


def _full_parity(w):
    log(f"[bwd parity] {w.name} desc={w.desc} B={w.batch} H={w.heads} d={w.head_dim} {w.dtype}")
    x = _inputs(w)
    dq, dk, dv, ws, lse = _run(w, x)
    dq, dk, dv, ws, lse = (to_f64(t) for t in (dq, dk, dv, ws, lse))
    worst = np.zeros(4)
    for b in range(w.batch):
        for h in range(w.heads):
            rq, rk, rv, rd = oracle.masked_attention_bwd_slice(*_slices(w, b, h), w.desc)
            e = [rel_err(dq[b, h], rq), rel_err(dk[b, h], rk), rel_err(dv[b, h], rv), rel_err(-ws[b, h, 0], rd)]
            worst = np.maximum(worst, e)
            assert np.isfinite(dq[b, h]).all() and np.isfinite(dk[b, h]).all() and np.isfinite(dv[b, h]).all()
            nl = -lse[b, h].astype(np.float32) * np.float32(LOG2E)
            assert np.max(np.abs(ws[b, h, 1] - nl) / np.maximum(np.abs(nl), 1.0)) < 1e-6
    log(f"    max rel err dq={worst[0]:.3e} dk={worst[1]:.3e} dv={worst[2]:.3e} delta={worst[3]:.3e}")
    tol = TOL[w.dtype]
    assert worst[0] < tol and worst[1] < tol and worst[2] < tol and worst[3] < DELTA_TOL[w.dtype]


SMALL_BF16 = [
    # id, tokens_per_frame, n_frames, frames_per_chunk, tf_layout, d
    (201, 50, 5, 1, 1, 128),   # ragged blocks and tiles, frame-wise teacher forcing
    (202, 40, 6, 3, 1, 128),   # chunk-wise teacher forcing
    (203, 37, 7, 1, 0, 128),   # block-causal, odd frame size
    (204, 100, 2, 2, 0, 128),  # one chunk: dense bidirectional attention
    (205, 1, 5, 1, 1, 128),    # 10 tokens: far smaller than one block
    (206, 130, 3, 1, 1, 64),   # head_dim 64
    (207, 64, 4, 1, 1, 128),   # frame == two tiles: aligned edges
    (208, 16, 3, 1, 1, 64),    # the tiny workload's geometry in bf16
    (209, 160, 9, 3, 1, 128),  # several chunks per side, many tiles and key blocks
    (210, 300, 5, 1, 1, 64),   # key blocks straddling chunk edges, d = 64
]


@pytest.mark.parametrize("cid, tpf, f, c, tf, d", SMALL_BF16, ids=[str(s[0]) for s in SMALL_BF16])
def test_bf16_small_bwd_parity(cid, tpf, f, c, tf, d):
    _full_parity(small_workload(cid, tpf, f, c, tf, heads=2, d=d))


@pytest.mark.parametrize("cid, tpf, f, c, tf, d", [(220, 48, 4, 2, 1, 128), (221, 33, 5, 5, 0, 64),
                                                   (222, 16, 3, 1, 1, 64)])
def test_fp32_small_bwd_parity(cid, tpf, f, c, tf, d):
    _full_parity(small_workload(cid, tpf, f, c, tf, heads=2, d=d, dtype="fp32"))


def test_bwd_batch_and_heads_are_independent():
    _full_parity(small_workload(230, 50, 4, 2, 1, heads=3, batch=2))


def test_bwd_medium_sequence_full_parity():
    # 6720 tokens: ~50 key blocks per side, 200+ query tiles per block
    _full_parity(small_workload(231, 160, 21, 1, 1, heads=1))


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_bwd_workload_sampled(cfg):
    """Full workload size: dq and delta on sampled rows; dk and dv, exactly,
    of the keys of the last chunk of each side, whose attending rows all lie
    in that chunk (the oracle takes those rows whole)."""
    w = WORKLOADS[cfg]
    log(f"[bwd sampled] {w.name}")
    x = _inputs(w)
    dq, dk, dv, ws, _ = _run(w, x)
    assert torch.isfinite(dq).all().item() and torch.isfinite(dk).all().item() and torch.isfinite(dv).all().item()
    T = w.tokens_per_frame * w.frames_per_chunk
    nh = w.tokens_per_side
    rows = sample_rows(w.desc, n_random=8, seed=cfg)
    # (the chunk-wise workload's chunks hold 4680 rows: one slice keeps the oracle within seconds)
    for b, h in ([(0, 0), (w.batch - 1, w.heads - 1)] if T < 4000 else [(w.batch - 1, w.heads - 1)]):
        sl = _slices(w, b, h)
        rq, _, _, rd = oracle.masked_attention_bwd_rows(*sl, w.desc, rows)
        e_q = rel_err(to_f64(dq[b, h, rows]), rq)
        e_d = rel_err(-to_f64(ws[b, h, 0, rows]), rd)
        log(f"    ({b},{h}) {len(rows)} rows: dq {e_q:.3e} delta {e_d:.3e}")
        assert e_q < TOL["bf16"] and e_d < DELTA_TOL["bf16"]
        for side in range(2 if w.tf_layout else 1):
            chunk = np.arange(side * nh + nh - T, side * nh + nh)
            _, rk, rv, _ = oracle.masked_attention_bwd_rows(*sl, w.desc, chunk)
            e_k = rel_err(to_f64(dk[b, h, chunk]), rk[chunk])
            e_v = rel_err(to_f64(dv[b, h, chunk]), rv[chunk])
            log(f"    ({b},{h}) side {side} last-chunk keys: dk {e_k:.3e} dv {e_v:.3e}")
            assert e_k < TOL["bf16"] and e_v < TOL["bf16"]


@pytest.mark.parametrize("geom", [(160, 9, 3, 1, 128), (96, 7, 1, 0, 64)])
def test_bwd_run_to_run_bitwise_determinism(geom):
    # no result accumulated by atomics: the same call repeated gives the same bits
    tpf, nf, fpc, tf, d = geom
    w = small_workload(240, tpf, nf, fpc, tf, heads=2, d=d)
    x = _inputs(w)
    runs = [_run(w, x)[:4] for _ in range(3)]
    for r in runs[1:]:
        for u, v in zip(runs[0], r):
            assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                               v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


def test_bwd_zero_output_gradient_gives_zero():
    w = small_workload(250, 50, 5, 1, 1)
    x = _inputs(w)
    x["do"] = torch.zeros_like(x["q"])
    dq, dk, dv, ws, _ = _run(w, x)
    assert torch.count_nonzero(dq).item() == 0
    assert torch.count_nonzero(dk).item() == 0
    assert torch.count_nonzero(dv).item() == 0
    assert torch.count_nonzero(ws[:, :, 0]).item() == 0


def test_bwd_value_gradient_of_uniform_attention():
    # q = 0: every allowed key gets weight 1 / (number of keys of the row), so
    # dv_j = sum over the rows i that see j of dO_i / n_i, and dq = dk = 0
    # when dO is constant along each row's keys' v (here v = 0 gives dP = 0)
    w = small_workload(251, 40, 6, 3, 1, heads=1)
    x = _inputs(w)
    x["q"] = torch.zeros_like(x["q"])
    x["v"] = torch.zeros_like(x["v"])
    dq, dk, dv, _, _ = _run(w, x)
    m = oracle.mask_dense(w.desc).astype(np.float64)
    p = m / m.sum(axis=1, keepdims=True)
    do = si.slice_values(w, "do", 0, 0)
    assert rel_err(to_f64(dv[0, 0]), p.T @ do) < TOL["bf16"]
    assert torch.count_nonzero(dq).item() == 0
    assert torch.count_nonzero(dk).item() == 0


def test_bwd_gpu_error_paths():
    w = small_workload(260, 16, 3, 1, 1)
    x = _inputs(w)
    plan = aj.attn_jvp_create(w.desc, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16)
    o = torch.empty_like(x["q"])
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device="cuda")
    ws = torch.empty(aj.attn_jvp_bwd_workspace_size(plan) // 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(x["q"]) for _ in range(3))
    with pytest.raises(aj.AttnJvpError) as e:  # dk aliases dq
        aj.attn_jvp_bwd(plan, x["q"], x["k"], x["v"], o, lse, x["do"], dq, dq, dv, ws)
    assert e.value.code == 1
    with pytest.raises(aj.AttnJvpError):  # workspace too small
        aj.attn_jvp_bwd(plan, x["q"], x["k"], x["v"], o, lse, x["do"], dq, dk, dv, ws[:8])
