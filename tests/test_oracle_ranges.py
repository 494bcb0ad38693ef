"""Pins for the oracle's range-list masks (query groups x key intervals) and
for the range lists the workloads are built from.

* ``ChunkListDesc`` (chunked teacher forcing with chunks of any size) against
  hand-written golden masks and against ``MaskDesc`` when all chunks are equal;
* ``RangeMask`` membership: the generated range lists reproduce the chunked
  definition (an independent construction: rectangles vs chunk arithmetic)
  and the hand-written understanding / generation mask;
* masked attention and its JVP on range masks against ``torch.func.jvp``
  through dense masked attention, rows in no group giving zero output;
* the backward on range masks against autograd; tile classes against a brute
  force over the dense mask.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from conftest import read_golden
from oracle import ChunkListDesc, MaskDesc, RangeMask, mask_dense


def test_chunk_list_matches_hand_written_golden():
    meta, rows = read_golden("mask_tf_c1_2_tpf1.txt")
    lens = tuple(meta["tpf"][0] * c for c in meta["chunks"])
    got = mask_dense(ChunkListDesc(lens, meta["tf"][0]))
    assert np.array_equal(got, np.array(rows, dtype=bool))


def test_generated_ranges_match_hand_written_golden():
    meta, rows = read_golden("mask_tf_c1_2_tpf1.txt")
    n, groups = si.chunked_mask_ranges(meta["tpf"][0], meta["chunks"], meta["tf"][0])
    assert np.array_equal(mask_dense(RangeMask(n, groups)), np.array(rows, dtype=bool))
    meta, rows = read_golden("mask_und_gen_u3_f2_s2.txt")
    n, groups = si.und_gen_ranges(meta["und"][0], meta["frames"][0], meta["tpf"][0])
    assert np.array_equal(mask_dense(RangeMask(n, groups)), np.array(rows, dtype=bool))


@pytest.mark.parametrize("desc", [(16, 3, 1, 1), (5, 6, 3, 1), (7, 5, 1, 0), (3, 4, 2, 0), (1, 5, 1, 1)])
def test_equal_chunk_lists_are_the_descriptor_masks(desc):
    tpf, f, c, tf = desc
    want = mask_dense(MaskDesc(*desc))
    assert np.array_equal(mask_dense(ChunkListDesc((tpf * c,) * (f // c), tf)), want)
    n, groups = si.chunked_mask_ranges(tpf, (c,) * (f // c), tf)
    assert np.array_equal(mask_dense(RangeMask(n, groups)), want)


@pytest.mark.parametrize("tpf, chunks, tf", [(3, (1, 4, 4), 1), (2, (3, 1, 2, 5), 1), (4, (1, 2, 2), 0),
                                             (1, (2,), 1), (5, (1, 1, 3), 1)])
def test_generated_ranges_match_chunk_list_definition(tpf, chunks, tf):
    n, groups = si.chunked_mask_ranges(tpf, chunks, tf)
    cl = ChunkListDesc(tuple(tpf * c for c in chunks), tf)
    assert n == cl.seq_len
    assert np.array_equal(mask_dense(RangeMask(n, groups)), mask_dense(cl))


def test_c1_4_workload_ranges_match_definition_on_sampled_rows():
    w = si.RANGE_WORKLOADS[6]
    n, groups = w.mask_ranges()
    assert n == w.seq_len == 65520
    rm, cl = RangeMask(n, groups), ChunkListDesc(tuple(w.tokens_per_frame * c for c in w.chunks), w.tf_layout)
    rng = np.random.default_rng(6)
    for i in list(rng.choice(n, 24, replace=False)) + [0, 1559, 1560, 32759, 32760, 34319, 34320, 65519]:
        assert np.array_equal(oracle.allowed_row(rm, int(i)), oracle.allowed_row(cl, int(i)))


def test_range_mask_membership_rules():
    # rows 2..3 in no group; group (4, 6) with two intervals, one touching the end
    rm = RangeMask(8, ((0, 2, ((0, 1), (3, 5))), (4, 6, ((2, 3), (6, 8)))))
    m = mask_dense(rm)
    assert not m[2].any() and not m[3].any() and not m[6].any() and not m[7].any()
    assert m[0].tolist() == [1, 0, 0, 1, 1, 0, 0, 0] and m[1].tolist() == m[0].tolist()
    assert m[4].tolist() == [0, 0, 1, 0, 0, 0, 1, 1] and m[5].tolist() == m[4].tolist()
    assert oracle.pair_count(rm) == 2 * 3 + 2 * 3
    assert oracle.row_groups(rm) == [(0, 2), (2, 4), (4, 6), (6, 8)]


def _dense_jvp(q, k, v, tq, tk, tv, mask, sc):
    t = lambda x: torch.tensor(x, dtype=torch.float64)
    m = torch.tensor(mask)

    def f(q_, k_, v_):
        s = (sc * (q_ @ k_.T)).masked_fill(~m, float("-inf"))
        return torch.softmax(s, dim=-1) @ v_

    return [x.numpy() for x in torch.func.jvp(f, (t(q), t(k), t(v)), (t(tq), t(tk), t(tv)))]


@pytest.mark.parametrize("case", ["tf_c1_2", "und_gen", "gaps"])
def test_range_mask_jvp_matches_torch_func_jvp(case):
    if case == "tf_c1_2":
        n, groups = si.chunked_mask_ranges(3, (1, 2, 2), 1)
    elif case == "und_gen":
        n, groups = si.und_gen_ranges(5, 3, 4)
    else:
        n, groups = 20, ((0, 6, ((0, 3), (10, 14))), (9, 15, ((0, 20),)), (15, 20, ((5, 6),)))
    rm = RangeMask(n, groups)
    rng = np.random.default_rng(41)
    q, k, v, tq, tk, tv = (rng.standard_normal((n, 8)) for _ in range(6))
    mask = mask_dense(rm)
    o, to, lse = oracle.masked_attention_jvp_slice(q, k, v, tq, tk, tv, rm)
    covered = mask.any(axis=1)
    ro, rto = _dense_jvp(q, k, v, tq, tk, tv, mask, 1 / np.sqrt(8))
    assert np.max(np.abs(o[covered] - ro[covered])) < 1e-12
    assert np.max(np.abs(to[covered] - rto[covered])) < 1e-12
    assert np.all(o[~covered] == 0) and np.all(to[~covered] == 0) and np.all(np.isneginf(lse[~covered]))


def test_range_mask_backward_matches_autograd():
    n, groups = 20, ((0, 6, ((0, 3), (10, 14))), (9, 15, ((0, 20),)), (15, 20, ((5, 6),)))
    rm = RangeMask(n, groups)
    rng = np.random.default_rng(42)
    q, k, v, do = (rng.standard_normal((n, 8)) for _ in range(4))
    mask = torch.tensor(mask_dense(rm))
    covered = mask.any(dim=1)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    s = ((t[0] @ t[1].T) / np.sqrt(8)).masked_fill(~mask, float("-inf"))
    p = torch.softmax(s, dim=-1)
    p = torch.where(covered[:, None], p, torch.zeros_like(p))  # rows in no group: no output
    (p @ t[2]).backward(torch.tensor(do))
    dq, dk, dv, _ = oracle.masked_attention_bwd_slice(q, k, v, do, rm)
    for a, b in ((dq, t[0].grad), (dk, t[1].grad), (dv, t[2].grad)):
        assert np.max(np.abs(a - b.numpy())) < 1e-12


def test_range_mask_rows_backward_matches_autograd_with_rows_in_no_group():
    # rows 6-8 and 15-19 lie in no group; dO is confined to the chosen rows
    n, groups = 24, ((0, 6, ((0, 3), (10, 14))), (9, 15, ((0, 24),)), (20, 24, ((5, 6), (18, 24))))
    rm = RangeMask(n, groups)
    rng = np.random.default_rng(7)
    q, k, v, do = (rng.standard_normal((n, 8)) for _ in range(4))
    rows = np.array([21, 0, 7, 16, 12, 5, 23])
    mask = torch.tensor(mask_dense(rm))
    covered = mask.any(dim=1)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v)]
    s = ((t[0] @ t[1].T) / np.sqrt(8)).masked_fill(~mask, float("-inf"))
    p = torch.where(covered[:, None], torch.softmax(s, dim=-1), torch.zeros(n, n, dtype=torch.float64))
    do_rows = np.zeros_like(do)
    do_rows[rows] = do[rows]
    (p @ t[2]).backward(torch.tensor(do_rows))
    dq, dk, dv, delta = oracle.masked_attention_bwd_rows(q, k, v, do, rm, rows)
    assert np.max(np.abs(dq - t[0].grad.numpy()[rows])) < 1e-12
    assert np.max(np.abs(dk - t[1].grad.numpy())) < 1e-12
    assert np.max(np.abs(dv - t[2].grad.numpy())) < 1e-12
    po = (p @ t[2]).detach().numpy()
    assert np.max(np.abs(delta - (do[rows] * po[rows]).sum(axis=1))) < 1e-12
    assert np.all(dq[[2, 3]] == 0) and np.all(delta[[2, 3]] == 0)  # rows 7 and 16: no key


@pytest.mark.parametrize("bq, bk", [(4, 4), (8, 4), (3, 5)])
def test_range_tile_classes_by_brute_force(bq, bk):
    n, groups = si.und_gen_ranges(5, 3, 4)
    rm = RangeMask(n, groups)
    m = mask_dense(rm)
    got = oracle.tile_classes(rm, bq, bk)
    for bi, (lo, hi) in enumerate(oracle.query_blocks(rm, bq)):
        assert (lo, hi) == (bi * bq, min(bi * bq + bq, n))
        for ti, (k0, k1) in enumerate(oracle.key_tiles(rm, bk)):
            cnt = int(m[lo:hi, k0:k1].sum())
            assert got[bi, ti] == (0 if cnt == 0 else (1 if cnt == (hi - lo) * (k1 - k0) else 2))
