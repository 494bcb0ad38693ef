"""Pins for the oracle's clean-tangent-zero functions (Causal-rCM, section
3.1.2, text after eq. 17: the clean context carries zero tangent, only the
noisy tokens move).

The tangent is checked against central differences of the forward map along
directions that move noisy tokens only; the pair classes against their
closed forms; and the clean rows against the exact zero they must give.
"""
import numpy as np
import pytest

import oracle
from oracle import MaskDesc, masked_attention_jvp_slice, masked_attention_jvp_slice_ctz

DESCS = [MaskDesc(16, 3, 1, 1), MaskDesc(2, 6, 3, 1), MaskDesc(4, 4, 2, 1), MaskDesc(5, 3, 1, 1)]


def _rand(desc, d, seed):
    rng = np.random.default_rng(seed)
    n = desc.seq_len
    return [rng.standard_normal((n, d)) for _ in range(3)] + [0.3 * rng.standard_normal((n, d)) for _ in range(3)]


def _rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


@pytest.mark.parametrize("desc", DESCS)
def test_ctz_tangent_is_the_derivative_along_noisy_only_directions(desc):
    q, k, v, tq, tk, tv = _rand(desc, 8, 11)
    nh = desc.side_len
    # the direction the flag describes: clean tokens do not move
    dq, dk, dv = (t.copy() for t in (tq, tk, tv))
    for t in (dq, dk, dv):
        t[:nh] = 0.0
    h = 1e-5
    op, _, _ = masked_attention_jvp_slice(q + h * dq, k + h * dk, v + h * dv, dq, dk, dv, desc)
    om, _, _ = masked_attention_jvp_slice(q - h * dq, k - h * dk, v - h * dv, dq, dk, dv, desc)
    fd = (op - om) / (2 * h)
    # the ctz function is handed the *unzeroed* tangents: it must ignore the clean halves
    _, to, _ = masked_attention_jvp_slice_ctz(q, k, v, tq, tk, tv, desc)
    assert _rel(to, fd) < 1e-8


@pytest.mark.parametrize("desc", DESCS)
def test_ctz_clean_rows_exact_zero_and_nan_in_clean_halves_ignored(desc):
    q, k, v, tq, tk, tv = _rand(desc, 8, 12)
    nh = desc.side_len
    o, to, lse = masked_attention_jvp_slice_ctz(q, k, v, tq, tk, tv, desc)
    assert np.all(to[:nh] == 0.0)
    bad = [t.copy() for t in (tq, tk, tv)]
    for t in bad:
        t[:nh] = np.nan
    o2, to2, lse2 = masked_attention_jvp_slice_ctz(q, k, v, *bad, desc)
    assert np.array_equal(o, o2) and np.array_equal(to, to2) and np.array_equal(lse, lse2)
    # the primal outputs do not depend on the tangents at all
    o3, _, lse3 = masked_attention_jvp_slice(q, k, v, tq, tk, tv, desc)
    assert np.array_equal(o, o3) and np.array_equal(lse, lse3)


def test_ctz_needs_teacher_forcing_layout():
    desc = MaskDesc(4, 3, 1, 0)
    args = _rand(desc, 8, 13)
    with pytest.raises(ValueError):
        masked_attention_jvp_slice_ctz(*args, desc)


@pytest.mark.parametrize("desc", [MaskDesc(16, 3, 1, 1), MaskDesc(2, 6, 3, 1), MaskDesc(1560, 21, 1, 1),
                                  MaskDesc(1560, 21, 3, 1), MaskDesc(7, 5, 1, 0)])
def test_pair_classes_closed_forms(desc):
    T, C = desc.chunk_len, desc.n_chunks
    cc, nc, nn = oracle.pair_counts_by_class(desc)
    assert cc + nc + nn == oracle.pair_count(desc)
    assert cc == T * T * C * (C + 1) // 2  # clean rows: block-causal incl. own chunk
    if desc.tf_layout:
        assert nc == T * T * C * (C - 1) // 2  # noisy chunk c sees c earlier clean chunks
        assert nn == C * T * T  # and its own noisy chunk
    else:
        assert nc == 0 and nn == 0


def test_useful_flops_counts():
    desc = MaskDesc(1560, 21, 1, 1)
    cc, nc, nn = oracle.pair_counts_by_class(desc)
    assert oracle.useful_flops(desc, 128) == 12 * 128 * (cc + nc + nn)
    assert oracle.useful_flops(desc, 128, True) == 128 * (4 * cc + 8 * nc + 12 * nn)
    # about half the general work on the 21-frame teacher-forcing sequence
    r = oracle.useful_flops(desc, 128, True) / oracle.useful_flops(desc, 128)
    assert abs(r - 0.5152) < 1e-3
