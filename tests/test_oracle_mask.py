"""Pins for the oracle's mask, pair counts and tile classification.

The mask is checked against hand-written golden matrices (tests/golden,
each citing the passage it follows), against closed-form pair counts, and
against structural identities of the teacher-forcing layout.
"""
import numpy as np
import pytest

from conftest import read_golden
from oracle import MaskDesc, mask_dense, pair_count, tile_classes, query_blocks, key_tiles, row_groups


@pytest.mark.parametrize("name", [
    "mask_tf_tf1_f4_c2.txt",
    "mask_blockcausal_tf2_f3_c1.txt",
    "mask_tf_tf2_f3_c1.txt",
])
def test_mask_matches_hand_written_golden(name):
    meta, rows = read_golden(name)
    desc = MaskDesc(*meta["desc"])
    want = np.array(rows, dtype=bool)
    got = mask_dense(desc)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_tile_classes_match_hand_written_golden():
    meta, rows = read_golden("tiles_tf_tf2_f3_c1_bq4_bk4.txt")
    desc = MaskDesc(*meta["desc"])
    bq, bk = meta["blocks"]
    assert np.array_equal(tile_classes(desc, bq, bk), np.array(rows, dtype=np.uint8))


def _closed_form_pairs(desc):
    # tf=0: chunk c rows see (c+1) chunks: T^2 * C(C+1)/2.
    # tf=1: the clean half gives the same; noisy chunk c sees c clean chunks
    # plus itself: another T^2 * C(C+1)/2.
    T, C = desc.chunk_len, desc.n_chunks
    half = T * T * C * (C + 1) // 2
    return half * (2 if desc.tf_layout else 1)


@pytest.mark.parametrize("desc", [
    MaskDesc(16, 3, 1, 1), MaskDesc(2, 6, 3, 1), MaskDesc(5, 4, 2, 0), MaskDesc(3, 5, 5, 1),
    MaskDesc(1560, 21, 1, 0), MaskDesc(1560, 21, 1, 1), MaskDesc(1560, 21, 3, 1),
])
def test_pair_count_closed_form(desc):
    assert pair_count(desc) == _closed_form_pairs(desc)


@pytest.mark.parametrize("desc", [MaskDesc(16, 3, 1, 1), MaskDesc(3, 6, 2, 1), MaskDesc(4, 4, 4, 0)])
def test_dense_mask_sum_matches_pair_count(desc):
    assert int(mask_dense(desc).sum()) == pair_count(desc) == _closed_form_pairs(desc)


def test_workload_pair_counts():
    # allowed pairs per (b, h) of the four large workloads
    assert pair_count(MaskDesc(1560, 21, 1, 0)) == 562_161_600
    assert pair_count(MaskDesc(1560, 21, 1, 1)) == 1_124_323_200
    assert pair_count(MaskDesc(1560, 21, 3, 1)) == 1_226_534_400


@pytest.mark.parametrize("tf, f, c", [(3, 4, 1), (2, 6, 3), (5, 3, 3)])
def test_clean_half_nests_block_causal(tf, f, c):
    # The clean half of the teacher-forcing mask is the plain block-causal
    # mask on the clean tokens, and clean rows never see noisy keys.
    m1 = mask_dense(MaskDesc(tf, f, c, 1))
    m0 = mask_dense(MaskDesc(tf, f, c, 0))
    nh = tf * f
    assert np.array_equal(m1[:nh, :nh], m0)
    assert not m1[:nh, nh:].any()


@pytest.mark.parametrize("tf, f, c", [(3, 4, 1), (2, 6, 3)])
def test_noisy_rows_structure(tf, f, c):
    d = MaskDesc(tf, f, c, 1)
    m = mask_dense(d)
    nh, T = d.side_len, d.chunk_len
    for i in range(nh, 2 * nh):
        ch = (i - nh) // T
        # strictly earlier clean chunks
        assert m[i, :ch * T].all() and not m[i, ch * T:nh].any()
        # its own noisy chunk only
        own = np.zeros(nh, bool)
        own[ch * T:(ch + 1) * T] = True
        assert np.array_equal(m[i, nh:], own)
        # every row sees itself
        assert m[i, i]


def test_single_chunk_is_dense():
    # one chunk without teacher forcing is full bidirectional attention
    assert mask_dense(MaskDesc(7, 3, 3, 0)).all()


def test_row_groups_partition_and_share_keys():
    d = MaskDesc(3, 4, 2, 1)
    m = mask_dense(d)
    covered = []
    for lo, hi in row_groups(d):
        covered.extend(range(lo, hi))
        for i in range(lo, hi):
            assert np.array_equal(m[i], m[lo])
    assert covered == list(range(d.seq_len))


@pytest.mark.parametrize("desc, bq, bk", [
    (MaskDesc(16, 3, 1, 1), 32, 32), (MaskDesc(16, 3, 1, 1), 16, 8), (MaskDesc(5, 7, 1, 1), 8, 6),
    (MaskDesc(5, 6, 3, 0), 4, 16), (MaskDesc(3, 9, 3, 1), 5, 7),
])
def test_tile_classes_against_dense_mask(desc, bq, bk):
    # brute force over the dense mask: the tile-wise counts define the classes
    m = mask_dense(desc)
    got = tile_classes(desc, bq, bk)
    qb, kt = query_blocks(desc, bq), key_tiles(desc, bk)
    assert got.shape == (len(qb), len(kt))
    for a, (q0, q1) in enumerate(qb):
        for b, (k0, k1) in enumerate(kt):
            blk = m[q0:q1, k0:k1]
            want = 0 if not blk.any() else (1 if blk.all() else 2)
            assert got[a, b] == want
    # blocks never straddle the clean/noisy boundary and cover every row once
    rows = [i for q0, q1 in qb for i in range(q0, q1)]
    assert rows == list(range(desc.seq_len))
    for q0, q1 in qb:
        assert (q0 < desc.side_len) == (q1 - 1 < desc.side_len)
