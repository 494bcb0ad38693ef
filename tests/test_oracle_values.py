"""Pins for the oracle's attention output, log-sum-exp and tangent.

Each check reaches the oracle by a route of its own: finite differences of
the forward map, torch.func.jvp through dense masked attention (the generic
route Causal-rCM section 3.2.1 names), closed forms, scalar brute force, and
the invariants of softmax and its tangent.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import MaskDesc, mask_dense, masked_attention_jvp_slice, masked_attention_jvp_scalar
from seeded_inputs import WORKLOADS, full_values

DESCS = [MaskDesc(16, 3, 1, 1), MaskDesc(2, 6, 3, 1), MaskDesc(3, 5, 1, 0), MaskDesc(4, 4, 2, 1)]


def _rand(desc, d, seed, tstd=0.3):
    rng = np.random.default_rng(seed)
    n = desc.seq_len
    x = [rng.standard_normal((n, d)) for _ in range(3)]
    t = [tstd * rng.standard_normal((n, d)) for _ in range(3)]
    return x + t


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("desc", DESCS[:3])
def test_scalar_bruteforce_matches_vectorised(desc):
    args = _rand(desc, 8, 1)
    o, to, lse = masked_attention_jvp_slice(*args, desc)
    o2, to2, lse2 = masked_attention_jvp_scalar(*args, desc)
    assert _rel(o, o2) < 1e-13 and _rel(to, to2) < 1e-13 and np.max(np.abs(lse - lse2)) < 1e-12


@pytest.mark.parametrize("desc", DESCS)
@pytest.mark.parametrize("scale", [None, 0.7])
def test_tangent_matches_central_differences(desc, scale):
    q, k, v, tq, tk, tv = _rand(desc, 8, 2)
    h = 1e-5
    op, _, lp = masked_attention_jvp_slice(q + h * tq, k + h * tk, v + h * tv, tq, tk, tv, desc, scale)
    om, _, lm = masked_attention_jvp_slice(q - h * tq, k - h * tk, v - h * tv, tq, tk, tv, desc, scale)
    _, to, _ = masked_attention_jvp_slice(q, k, v, tq, tk, tv, desc, scale)
    fd = (op - om) / (2 * h)
    assert _rel(to, fd) < 1e-8


def _torch_dense(q, k, v, mask, scale):
    s = scale * (q @ k.transpose(-1, -2))
    s = s.masked_fill(~mask, float("-inf"))
    return torch.softmax(s, dim=-1) @ v


@pytest.mark.parametrize("desc", DESCS)
def test_matches_torch_func_jvp_dense(desc):
    d = 8
    args = _rand(desc, d, 3)
    mask = torch.from_numpy(mask_dense(desc))
    T = [torch.from_numpy(a) for a in args]
    scale = 1 / math.sqrt(d)
    o_t, to_t = torch.func.jvp(lambda q, k, v: _torch_dense(q, k, v, mask, scale), tuple(T[:3]), tuple(T[3:]))
    o, to, lse = masked_attention_jvp_slice(*args, desc)
    assert _rel(o, o_t.numpy()) < 1e-13
    assert _rel(to, to_t.numpy()) < 1e-12
    s = scale * (T[0] @ T[1].T)
    lse_t = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
    assert np.max(np.abs(lse - lse_t.numpy())) < 1e-12


def test_zero_queries_give_uniform_weights():
    # q = 0 => every allowed key has the same score: o = mean of allowed v,
    # lse = ln(number of allowed keys)
    desc = MaskDesc(3, 4, 2, 1)
    q, k, v, tq, tk, tv = _rand(desc, 6, 4)
    q[:] = 0
    o, _, lse = masked_attention_jvp_slice(q, k, v, tq, tk, tv, desc)
    m = mask_dense(desc)
    for i in range(desc.seq_len):
        keys = np.nonzero(m[i])[0]
        assert np.allclose(o[i], v[keys].mean(axis=0), rtol=0, atol=1e-14)
        assert abs(lse[i] - math.log(len(keys))) < 1e-14


def test_two_key_rows_closed_form():
    # tokens_per_frame=2, frame-wise TF: noisy rows of chunk 0 see exactly two
    # keys (their own noisy frame).  For two keys, p1 = 1/(1+exp(s2-s1)), and
    # to = p1 p2 (ts1 - ts2)(v1 - v2) + p1 tv1 + p2 tv2.
    desc = MaskDesc(2, 3, 1, 1)
    q, k, v, tq, tk, tv = _rand(desc, 5, 5)
    o, to, lse = masked_attention_jvp_slice(q, k, v, tq, tk, tv, desc)
    sc = 1 / math.sqrt(5)
    j1, j2 = 6, 7
    for i in (6, 7):
        s1, s2 = sc * q[i] @ k[j1], sc * q[i] @ k[j2]
        t1 = sc * (tq[i] @ k[j1] + q[i] @ tk[j1])
        t2 = sc * (tq[i] @ k[j2] + q[i] @ tk[j2])
        p1 = 1 / (1 + math.exp(s2 - s1))
        p2 = 1 - p1
        assert np.allclose(o[i], p1 * v[j1] + p2 * v[j2], atol=1e-14)
        want = p1 * p2 * (t1 - t2) * (v[j1] - v[j2]) + p1 * tv[j1] + p2 * tv[j2]
        assert np.allclose(to[i], want, atol=1e-14)
        assert abs(lse[i] - (max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2))))) < 1e-13


def test_single_key_rows_pass_values_through():
    # tokens_per_frame=1, frame-wise TF: the noisy row of chunk 0 sees only
    # itself, so o = v_self and to = tv_self exactly.
    desc = MaskDesc(1, 4, 1, 1)
    q, k, v, tq, tk, tv = _rand(desc, 4, 6)
    o, to, lse = masked_attention_jvp_slice(q, k, v, tq, tk, tv, desc)
    i = desc.side_len
    assert np.array_equal(o[i], v[i]) and np.array_equal(to[i], tv[i])
    assert lse[i] == pytest.approx(q[i] @ k[i] / 2, abs=1e-15)


def test_masked_probabilities_are_exactly_zero_and_rows_sum_to_one():
    # v = identity makes o the probability matrix itself
    desc = MaskDesc(3, 4, 2, 1)
    n = desc.seq_len
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal((n, 6)), rng.standard_normal((n, 6))
    eye = np.eye(n)
    zeros = np.zeros((n, 6))
    p, _, _ = masked_attention_jvp_slice(q, k, eye, zeros, zeros, np.zeros((n, n)), desc)
    m = mask_dense(desc)
    assert np.all(p[~m] == 0.0)
    assert np.all(p[m] > 0.0)
    assert np.max(np.abs(p.sum(axis=1) - 1)) < 1e-14


def test_tangent_invariants():
    desc = MaskDesc(3, 4, 2, 1)
    q, k, v, tq, tk, tv = _rand(desc, 6, 8)
    z = np.zeros_like(q)
    f = lambda a, b, c: masked_attention_jvp_slice(q, k, v, a, b, c, desc)[1]
    o = masked_attention_jvp_slice(q, k, v, z, z, z, desc)[0]
    # all-zero tangent
    assert np.all(f(z, z, z) == 0)
    # linearity in (tq, tk, tv)
    assert _rel(f(2 * tq, 2 * tk, 2 * tv) - f(tq, tk, tv), f(tq, tk, tv)) < 1e-14
    assert _rel(f(tq, tk, tv), f(tq, z, z) + f(z, tk, z) + f(z, z, tv)) < 1e-13
    # direction (0, 0, v) scales v only: to = o
    assert _rel(f(z, z, v), o) < 1e-14
    # scores are bilinear: tangents (q,0,0) and (0,k,0) both give d/de of s(1+e)
    assert _rel(f(q, z, z), f(z, k, z)) < 1e-13
    # tq = tk = 0: to = P tv (P from torch's dense softmax)
    mask = torch.from_numpy(mask_dense(desc))
    s = (torch.from_numpy(q) @ torch.from_numpy(k).T) / math.sqrt(6)
    P = torch.softmax(s.masked_fill(~mask, float("-inf")), -1).numpy()
    assert _rel(f(z, z, tv), P @ tv) < 1e-13
    # constant v: tangent rows sum to zero, so to = P tv
    vc = np.ones_like(v) * 3.0
    to_c = masked_attention_jvp_slice(q, k, vc, tq, tk, tv, desc)[1]
    assert _rel(to_c, P @ tv) < 1e-13
    oc = masked_attention_jvp_slice(q, k, vc, tq, tk, tv, desc)[0]
    assert np.max(np.abs(oc - 3.0)) < 1e-14


def test_rows_subset_matches_full():
    desc = MaskDesc(4, 5, 1, 1)
    args = _rand(desc, 8, 9)
    o, to, lse = masked_attention_jvp_slice(*args, desc)
    rows = np.array([0, 3, 17, 20, 21, 39])
    o2, to2, lse2 = oracle.masked_attention_jvp_rows(args, desc, rows)
    # same arithmetic on fewer rows; BLAS may block differently, so allow rounding
    assert _rel(o2, o[rows]) < 1e-14 and _rel(to2, to[rows]) < 1e-14
    assert np.max(np.abs(lse2 - lse[rows])) < 1e-14


def test_tiny_fp32_workload_runs_and_is_finite():
    w = WORKLOADS[1]
    args = [full_values(w, t) for t in ("q", "k", "v", "tq", "tk", "tv")]
    o, to, lse = oracle.masked_attention_jvp(*args, w.desc)
    assert o.shape == w.shape and np.isfinite(o).all() and np.isfinite(to).all()
    o2, to2, lse2 = masked_attention_jvp_scalar(*[a[0, 1] for a in args], w.desc)
    assert _rel(o[0, 1], o2) < 1e-13 and _rel(to[0, 1], to2) < 1e-13


# --- the pins have teeth: plant plausible mistakes in a copy of the oracle's
# row kernel and check that the pins above reject each one --------------------

def _planted(kind):
    from oracle import masked_attention as ma

    def rows_forward(q, k, v, tq, tk, tv, keys, scale):
        kk, vv, tkk, tvv = k[keys], v[keys], tk[keys], tv[keys]
        s = scale * (q @ kk.T)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        ts = scale * (tq @ kk.T + q @ tkk.T)
        if kind == "no_key_tangent":
            ts = scale * (tq @ kk.T)
        if kind == "unscaled_tangent":
            ts = tq @ kk.T + q @ tkk.T
        rbar = (p * ts).sum(axis=1, keepdims=True)
        if kind == "sign":
            rbar = -rbar
        tp = p * (ts - rbar)
        to = tp @ vv + (0 if kind == "no_tv" else p @ tvv)
        lse = (s.max(axis=1, keepdims=True) + np.log(e.sum(axis=1, keepdims=True)))[:, 0]
        return p @ vv, to, lse
    return ma, rows_forward


@pytest.mark.parametrize("kind", ["no_key_tangent", "unscaled_tangent", "sign", "no_tv"])
def test_finite_difference_pin_rejects_planted_mistakes(kind, monkeypatch):
    ma, bad = _planted(kind)
    monkeypatch.setattr(ma, "_rows_forward", bad)
    desc = DESCS[0]
    q, k, v, tq, tk, tv = _rand(desc, 8, 2)
    h = 1e-5
    op = ma.masked_attention_jvp_slice(q + h * tq, k + h * tk, v + h * tv, tq, tk, tv, desc)[0]
    om = ma.masked_attention_jvp_slice(q - h * tq, k - h * tk, v - h * tv, tq, tk, tv, desc)[0]
    to = ma.masked_attention_jvp_slice(q, k, v, tq, tk, tv, desc)[1]
    assert _rel(to, (op - om) / (2 * h)) > 1e-3
