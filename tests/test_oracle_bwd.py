"""Pins for the oracle's masked-attention backward.

Reached by independent routes: torch autograd through dense masked
attention in float64, central differences of the scalar loss <do, o>, and
the invariants of the softmax gradient.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import MaskDesc, masked_attention_bwd_slice, masked_attention_jvp_slice, mask_dense

DESCS = [MaskDesc(16, 3, 1, 1), MaskDesc(2, 6, 3, 1), MaskDesc(3, 5, 1, 0), MaskDesc(4, 4, 2, 1)]


def _rand(desc, d, seed):
    rng = np.random.default_rng(seed)
    n = desc.seq_len
    return [rng.standard_normal((n, d)) for _ in range(4)]


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("desc", DESCS)
@pytest.mark.parametrize("scale", [None, 0.7])
def test_matches_torch_autograd_dense(desc, scale):
    q, k, v, do = _rand(desc, 8, 21)
    sc = 1 / np.sqrt(8) if scale is None else scale
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    mask = torch.tensor(mask_dense(desc))
    s = sc * (t[0] @ t[1].T)
    s = s.masked_fill(~mask, float("-inf"))
    o = torch.softmax(s, dim=-1) @ t[2]
    o.backward(torch.tensor(do))
    dq, dk, dv, delta = masked_attention_bwd_slice(q, k, v, do, desc, scale)
    assert _rel(dq, t[0].grad.numpy()) < 1e-12
    assert _rel(dk, t[1].grad.numpy()) < 1e-12
    assert _rel(dv, t[2].grad.numpy()) < 1e-12
    assert np.max(np.abs(delta - (do * o.detach().numpy()).sum(axis=1))) < 1e-12


@pytest.mark.parametrize("desc", DESCS)
def test_matches_central_differences_of_the_loss(desc):
    q, k, v, do = _rand(desc, 8, 22)
    dq, dk, dv, _ = masked_attention_bwd_slice(q, k, v, do, desc)
    rng = np.random.default_rng(23)
    z = np.zeros_like(q)

    def loss(q_, k_, v_):
        o, _, _ = masked_attention_jvp_slice(q_, k_, v_, z, z, z, desc)
        return float((o * do).sum())

    h = 1e-5
    for grad, which in ((dq, 0), (dk, 1), (dv, 2)):
        u = rng.standard_normal(q.shape)
        args_p = [q, k, v]
        args_m = [q, k, v]
        args_p = [a + h * u if i == which else a for i, a in enumerate(args_p)]
        args_m = [a - h * u if i == which else a for i, a in enumerate(args_m)]
        fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
        assert abs(fd - float((grad * u).sum())) < 1e-7 * max(1.0, abs(fd))


@pytest.mark.parametrize("desc", DESCS)
def test_backward_invariants(desc):
    q, k, v, do = _rand(desc, 8, 24)
    dq, dk, dv, delta = masked_attention_bwd_slice(q, k, v, do, desc)
    # rows of p sum to one: the value gradients sum to the output cotangents
    assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12)
    # shifting every key by the same vector leaves the scores of a row shifted
    # by a constant: the key gradients sum to zero
    assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    # constant values: o does not depend on q or k
    vc = np.tile(v[:1], (v.shape[0], 1))
    dq2, dk2, _, _ = masked_attention_bwd_slice(q, k, vc, do, desc)
    assert np.max(np.abs(dq2)) < 1e-12 and np.max(np.abs(dk2)) < 1e-12


def test_backward_useful_flops():
    desc = MaskDesc(1560, 21, 1, 1)
    assert oracle.backward_useful_flops(desc, 128) == 10 * 128 * 1_124_323_200


@pytest.mark.parametrize("desc", DESCS + [MaskDesc(5, 6, 2, 1), MaskDesc(7, 4, 1, 0)])
def test_rows_variant_matches_torch_autograd(desc):
    # the row-restricted backward against autograd through the dense masked
    # attention with the gradient confined to the chosen rows (dO = 0 on the
    # other rows): dq on those rows, dk and dv in full, delta on those rows
    q, k, v, do = _rand(desc, 8, 31)
    n = desc.seq_len
    rng = np.random.default_rng(32)
    rows = np.sort(rng.choice(n, max(1, n // 3), replace=False))
    do_r = np.zeros_like(do)
    do_r[rows] = do[rows]
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    sc = 1 / np.sqrt(8)
    s = (sc * (t[0] @ t[1].T)).masked_fill(~torch.tensor(mask_dense(desc)), float("-inf"))
    o = torch.softmax(s, dim=-1) @ t[2]
    o.backward(torch.tensor(do_r))
    dq, dk, dv, delta = oracle.masked_attention_bwd_rows(q, k, v, do, desc, rows, batch_rows=3)
    assert _rel(dq, t[0].grad.numpy()[rows]) < 1e-12
    assert _rel(dk, t[1].grad.numpy()) < 1e-12
    assert _rel(dv, t[2].grad.numpy()) < 1e-12
    assert np.max(np.abs(delta - (do[rows] * o.detach().numpy()[rows]).sum(axis=1))) < 1e-12


def test_rows_variant_gives_full_gradients_of_keys_seen_only_by_those_rows():
    # noisy keys of chunk c are seen only by the noisy rows of chunk c
    desc = MaskDesc(6, 4, 1, 1)
    q, k, v, do = _rand(desc, 8, 33)
    full = masked_attention_bwd_slice(q, k, v, do, desc)
    T, nh = desc.chunk_len, desc.side_len
    c = 2
    rows = np.arange(nh + c * T, nh + (c + 1) * T)
    _, dk, dv, _ = oracle.masked_attention_bwd_rows(q, k, v, do, desc, rows)
    assert _rel(dk[rows], full[1][rows]) < 1e-12
    assert _rel(dv[rows], full[2][rows]) < 1e-12
