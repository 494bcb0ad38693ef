"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Tolerances (normwise relative error ||X - X*||_F / ||X*||_F over the
compared outputs): 1e-2 for bf16 inputs, 1e-4 for fp32 inputs; lse is
compared by max absolute error (bf16: 2e-2, fp32: 1e-5).
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
    aj._load()  # fail loudly if the HIP library is missing


def _run(w, x):
    o, to, lse = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc, return_lse=True)
    torch.cuda.synchronize()
    return o, to, lse


def _full_parity(w, x=None):
    log(f"[parity] {w.name} desc={w.desc} B={w.batch} H={w.heads} d={w.head_dim} {w.dtype}")
    x = x or device_inputs(w)
    o, to, lse = _run(w, x)
    o, to, lse = to_f64(o), to_f64(to), to_f64(lse)
    errs = []
    for b in range(w.batch):
        for h in range(w.heads):
            ro, rto, rl = oracle.masked_attention_jvp_slice(*host_values(w, b, h), w.desc)
            errs.append((rel_err(o[b, h], ro), rel_err(to[b, h], rto), float(np.max(np.abs(lse[b, h] - rl)))))
            assert np.isfinite(o[b, h]).all() and np.isfinite(to[b, h]).all()
    eo, eto, el = (max(e[i] for e in errs) for i in range(3))
    log(f"    max rel err o={eo:.3e} to={eto:.3e}  max |dlse|={el:.3e}")
    assert eo < TOL[w.dtype] and eto < TOL[w.dtype] and el < LSE_TOL[w.dtype]
    return eo, eto


def test_fp32_tiny_teacher_forcing_workload():
    _full_parity(WORKLOADS[1])


SMALL_BF16 = [
    # id, tokens_per_frame, n_frames, frames_per_chunk, tf_layout, d
    (101, 50, 5, 1, 1, 128),   # ragged blocks and tiles, frame-wise TF
    (102, 40, 6, 3, 1, 128),   # chunk-wise TF
    (103, 37, 7, 1, 0, 128),   # block-causal, odd frame size
    (104, 100, 2, 2, 0, 128),  # one chunk: dense bidirectional attention
    (105, 1, 5, 1, 1, 128),    # 10 tokens: far smaller than one block
    (106, 130, 3, 1, 1, 64),   # head_dim 64
    (107, 64, 4, 1, 1, 128),   # frame == one tile: aligned edges
    (108, 16, 3, 1, 1, 64),    # the tiny workload's geometry in bf16
    (109, 160, 9, 3, 1, 128),  # several chunks per side, many tiles
]


@pytest.mark.parametrize("cid, tpf, f, c, tf, d", SMALL_BF16, ids=[str(s[0]) for s in SMALL_BF16])
def test_bf16_small_parity(cid, tpf, f, c, tf, d):
    _full_parity(small_workload(cid, tpf, f, c, tf, heads=2, d=d))


@pytest.mark.parametrize("cid, tpf, f, c, tf, d", [(110, 48, 4, 2, 1, 128), (111, 33, 5, 5, 0, 64)])
def test_fp32_small_parity(cid, tpf, f, c, tf, d):
    _full_parity(small_workload(cid, tpf, f, c, tf, heads=2, d=d, dtype="fp32"))


def test_batch_and_heads_are_independent():
    w = small_workload(120, 50, 4, 2, 1, heads=3, batch=2)
    _full_parity(w)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_workload_sampled_rows(cfg):
    w = WORKLOADS[cfg]
    log(f"[sampled parity] {w.name}")
    x = device_inputs(w)
    o, to, lse = _run(w, x)
    bh = [(0, 0), (w.batch - 1, w.heads - 1), (0, w.heads // 2)]
    rows = sample_rows(w.desc, seed=cfg)
    go, gto, rgo, rgto = [], [], [], []
    for b, h in bh:
        ro, rto, rl = oracle.masked_attention_jvp_rows(host_values(w, b, h), w.desc, rows)
        go.append(to_f64(o[b, h, rows]))
        gto.append(to_f64(to[b, h, rows]))
        rgo.append(ro)
        rgto.append(rto)
        assert np.max(np.abs(to_f64(lse[b, h, rows]) - rl)) < LSE_TOL["bf16"]
    eo, eto = rel_err(np.stack(go), np.stack(rgo)), rel_err(np.stack(gto), np.stack(rgto))
    log(f"    {len(rows)} rows x {len(bh)} heads: rel err o={eo:.3e} to={eto:.3e}")
    assert eo < TOL["bf16"] and eto < TOL["bf16"]
    # all outputs finite
    assert torch.isfinite(o).all().item() and torch.isfinite(to).all().item()


def _probe(w, key0, device="cuda"):
    """q = tq = tk = tv = 0 and v = one-hot key indicators for keys key0..key0+d-1:
    o[i, c] is then exactly p(i, key0 + c), zero where the mask forbids it."""
    B, H, N, d = w.shape
    z = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device=device)
    k = torch.randn((B, H, N, d), generator=torch.Generator().manual_seed(1)).to(device, torch.bfloat16)
    v = torch.zeros_like(z)
    cols = torch.arange(d, device=device)
    keys = key0 + cols
    ok = keys < N
    v[:, :, keys[ok], cols[ok]] = 1.0
    o, _ = aj.masked_attention_jvp(z, k, v, z, z, z, w.desc)
    torch.cuda.synchronize()
    return o, keys[ok].cpu().numpy(), int(ok.sum())


def test_exact_zero_probe_full_small():
    w = small_workload(130, 50, 5, 1, 1, heads=1)
    m = oracle.mask_dense(w.desc)
    for key0 in range(0, w.seq_len, w.head_dim):
        o, keys, nk = _probe(w, key0)
        got = to_f64(o[0, 0])[:, :nk]
        want = m[:, keys]
        assert np.all(got[~want] == 0.0), f"masked probability not exactly zero (key0={key0})"
        assert np.all(got[want] > 0.0)


@pytest.mark.parametrize("cfg", [2, 3, 4])  # config 5 has config 3's mask
def test_exact_zero_probe_workload_windows(cfg):
    w = WORKLOADS[cfg].with_(batch=1, heads=1)
    nh, T = w.tokens_per_side, w.tokens_per_frame * w.frames_per_chunk
    rows = sample_rows(w.desc, seed=cfg)
    # key windows across the first chunk edge, the side boundary, the first
    # noisy chunk edge and the end (windows past the end of a block-causal
    # sequence dropped)
    for key0 in sorted({k for k in (0, T - 64, nh - 64, nh + T - 64, w.seq_len - 128) if k + 64 <= w.seq_len}):
        o, keys, nk = _probe(w, key0)
        got = to_f64(o[0, 0, rows])[:, :nk]
        want = np.stack([oracle.allowed_row(w.desc, int(i))[keys] for i in rows])
        assert np.all(got[~want] == 0.0)
        assert np.all(got[want] > 0.0)


@pytest.mark.parametrize("geom", [(160, 9, 3, 1, 128), (96, 7, 1, 0, 64)])
def test_run_to_run_bitwise_determinism(geom):
    # Every result (o, t_o, lse) is a fixed function of the inputs: the same
    # launch repeated must agree bit for bit, whatever other work ran between.
    tpf, nf, fpc, tf, d = geom
    w = small_workload(140, tpf, nf, fpc, tf, heads=2, d=d)
    x = device_inputs(w)
    runs = [_run(w, x) for _ in range(4)]
    for r in runs[1:]:
        for u, v in zip(runs[0], r):
            assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                               v.view(torch.int16) if v.dtype == torch.bfloat16 else v)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_value_direction_gives_output_exactly(cfg):
    # tangent (0, 0, v): the scores do not move, so t_o = o bit for bit
    w = WORKLOADS[cfg]
    x = device_inputs(w)
    z = torch.zeros_like(x["q"])
    o, to = aj.masked_attention_jvp(x["q"], x["k"], x["v"], z, z, x["v"], w.desc)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), to.view(torch.int16))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_value_tangent_alone_gives_the_output_of_tv(cfg):
    # tangent (0, 0, tv): the scores do not move, so t_o = sum_j p_ij tv_j,
    # which is o with v replaced by tv -- the same bf16 packs of p~ meet tV
    # in the same order as they meet V, so the two agree bit for bit
    w = WORKLOADS[cfg]
    x = device_inputs(w)
    z = torch.zeros_like(x["q"])
    _, to = aj.masked_attention_jvp(x["q"], x["k"], x["v"], z, z, x["tv"], w.desc)
    o_tv, _ = aj.masked_attention_jvp(x["q"], x["k"], x["tv"], z, z, z, w.desc)
    torch.cuda.synchronize()
    assert torch.count_nonzero(to).item() > 0
    assert torch.equal(to.view(torch.int16), o_tv.view(torch.int16))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_tangent_linearity_is_exact(cfg):
    # every step of the tangent is linear in (tq, tk, tv), and scaling by 2
    # commutes with each rounding (fp32 sums, the bf16 packs of p~ ts and the
    # bf16 outputs), so doubling the tangents doubles t_o bit for bit and
    # leaves o unchanged -- at the full workload sizes, without the oracle
    w = WORKLOADS[cfg]
    log(f"[linearity] {w.name}")
    x = device_inputs(w)
    o1, to1 = aj.masked_attention_jvp(*(x[t] for t in TENSORS), w.desc)
    t2 = [x[t] * 2 for t in ("tq", "tk", "tv")]
    o2, to2 = aj.masked_attention_jvp(x["q"], x["k"], x["v"], *t2, w.desc)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal((to1 * 2).view(torch.int16), to2.view(torch.int16))


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_query_and_key_tangents_are_symmetric(cfg):
    # the directions (q, 0, 0) and (0, k, 0) give the same score tangent
    # sigma q.k for every pair, accumulated in the same order (the other
    # product adds exact zeros), hence the same t_o bit for bit
    w = WORKLOADS[cfg]
    x = device_inputs(w)
    z = torch.zeros_like(x["q"])
    _, ta = aj.masked_attention_jvp(x["q"], x["k"], x["v"], x["q"], z, z, w.desc)
    _, tb = aj.masked_attention_jvp(x["q"], x["k"], x["v"], z, x["k"], z, w.desc)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ta).item() > 0
    assert torch.equal(ta.view(torch.int16), tb.view(torch.int16))


def test_zero_tangent_gives_zero():
    w = small_workload(150, 50, 5, 1, 1)
    x = device_inputs(w)
    z = torch.zeros_like(x["q"])
    _, to = aj.masked_attention_jvp(x["q"], x["k"], x["v"], z, z, z, w.desc)
    torch.cuda.synchronize()
    assert torch.count_nonzero(to).item() == 0


def test_gpu_error_paths():
    w = small_workload(160, 16, 3, 1, 1)
    x = device_inputs(w)
    plan = aj.attn_jvp_create(w.desc, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16)
    o = torch.empty_like(x["q"])
    to = torch.empty_like(x["q"])
    # o aliasing an input
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_fwd(plan, x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], x["q"], to)
    assert e.value.code == 1
    # misaligned pointer (offset by one element)
    big = torch.empty(x["q"].numel() + 8, dtype=torch.bfloat16, device="cuda")
    mis = big[1:1 + x["q"].numel()].view(x["q"].shape)
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_fwd(plan, mis, x["k"], x["v"], x["tq"], x["tk"], x["tv"], o, to)
    assert e.value.code == 3
    # python-side shape and dtype checks
    with pytest.raises(aj.AttnJvpError):
        aj.attn_jvp_fwd(plan, x["q"].float(), x["k"], x["v"], x["tq"], x["tk"], x["tv"], o, to)
    with pytest.raises(aj.AttnJvpError):
        aj.masked_attention_jvp(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], (16, 4, 1, 1))
