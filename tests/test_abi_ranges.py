"""Host-side checks of range-list plans (query groups x key intervals), no GPU.

* argument validation before anything is built;
* the plan's tile map (which key tiles each query block streams, and whether
  every pair of a tile is allowed) equals the oracle's tile classification of
  the same RangeMask bit for bit, for bf16 and fp32 block sizes, at small
  ragged sizes and at the full c1-4 workload;
* per-row key intervals equal the oracle mask; pair counts and useful FLOPs;
* the serialised table: header, heavy-first launch order, per-wave whole bits
  against the oracle mask;
* the table's column sections, which the backward's dk/dv kernel walks: per
  key block exactly the 32-row query tiles with an allowed pair, per-wave
  whole bits, and per key the row intervals that see it, all against the
  columns of the oracle mask; key ranges, launch order and argument errors
  of the backward on range-list plans.
"""
import ctypes
import os

import numpy as np
import pytest

import oracle
import seeded_inputs as si
from conftest import check_launch_rule
from oracle import RangeMask
import masked_attention_jvp_amd as aj

pytestmark = pytest.mark.skipif(not os.path.exists(aj.library_path), reason="libattn_jvp.so not built")

GAPS = (40, ((0, 6, ((0, 3), (10, 14))), (9, 15, ((0, 40),)), (15, 33, ((5, 6), (20, 33))), (35, 40, ((1, 2),))))
MULTI = (70, ((0, 30, ((0, 3), (7, 9), (12, 20), (33, 40))), (30, 70, ((0, 70),))))  # rows with four intervals
# keys 0-19 are seen by three separate row intervals, keys 60-99 by two
STRIPES = (100, ((0, 10, ((0, 20),)), (20, 30, ((0, 20), (60, 100))), (40, 50, ((0, 20),)), (70, 100, ((60, 100),))))

MASKS = {
    "tf_c1_2": si.chunked_mask_ranges(16, (1, 2, 2), 1),
    "tf_c1_4_t50": si.chunked_mask_ranges(50, (1, 4, 4), 1),
    "bc_c2_1_t37": si.chunked_mask_ranges(37, (2, 1, 1, 3), 0),
    "und_gen": si.und_gen_ranges(20, 5, 30),
    "dense": (150, ((0, 150, ((0, 150),)),)),
    "gaps": GAPS,
    "multi": MULTI,
    "stripes": STRIPES,
    "tf_eq_as_ranges": si.chunked_mask_ranges(50, (1,) * 5, 1),
}


def _plan(name, dtype=aj.ATTN_JVP_BF16, d=128, b=1, h=1):
    n, groups = MASKS[name]
    return aj.attn_jvp_create_ranges(n, groups, b, h, d, dtype), RangeMask(n, groups)


@pytest.mark.parametrize("name", sorted(MASKS))
@pytest.mark.parametrize("dtype, d", [(aj.ATTN_JVP_BF16, 128), (aj.ATTN_JVP_BF16, 64), (aj.ATTN_JVP_FP32, 64)])
def test_range_tile_map_matches_oracle(name, dtype, d):
    p, rm = _plan(name, dtype, d)
    info = p.info
    want = oracle.tile_classes(rm, info["block_q"], info["block_k"])
    got = aj.attn_jvp_tile_map(p)
    assert got.shape == want.shape
    assert np.array_equal(got, want)
    assert info["visited_tiles_per_head"] == int((want > 0).sum())
    assert info["allowed_pairs_per_head"] == oracle.pair_count(rm)


@pytest.mark.parametrize("name", sorted(set(MASKS) - {"multi"}))
def test_range_row_ranges_match_oracle(name):
    p, rm = _plan(name)
    rr = aj.attn_jvp_row_ranges(p)
    keys = np.arange(p.seq_len)
    lo1, hi1, lo2, hi2 = (rr[:, i:i + 1] for i in range(4))
    got = ((keys >= lo1) & (keys < hi1)) | ((keys >= lo2) & (keys < hi2))
    assert np.array_equal(got, oracle.mask_dense(rm))


def test_row_ranges_refuse_rows_with_more_than_two_intervals():
    p, _ = _plan("multi")
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_row_ranges(p)
    assert e.value.code == 1


@pytest.mark.parametrize("name", sorted(MASKS))
def test_range_table_order_and_whole_bits(name):
    p, rm = _plan(name)
    t = aj.attn_jvp_plan_table(p)
    nq = p.info["n_query_blocks"]
    assert t[0] == 0x314a5441 and t[1] == nq
    blk = t[8:8 + nq + 1]
    order = t[8 + nq + 1:8 + 2 * nq + 1]
    ent = t[8 + 2 * nq + 1:8 + 2 * nq + 1 + t[2]]
    assert blk[0] == 0 and blk[-1] == t[2] == len(ent) and np.all(np.diff(blk) >= 0)
    assert sorted(order.tolist()) == list(range(nq))
    assert np.array_equal(order, aj.attn_jvp_launch_order(p))
    counts = np.diff(blk)[order]
    assert np.all(np.diff(counts) <= 0)  # heavy (more tiles) first
    m = oracle.mask_dense(rm)
    n = p.seq_len
    for qb in range(nq):
        tiles = ent[blk[qb]:blk[qb + 1]] & 0xffffff
        assert np.all(np.diff(tiles) > 0)  # ascending key order
        for e in ent[blk[qb]:blk[qb + 1]]:
            tile = int(e) & 0xffffff
            k0 = 32 * tile
            for w in range(4):
                r0, r1 = 128 * qb + 32 * w, min(128 * qb + 32 * w + 32, 128 * qb + 128, n)
                whole = bool((int(e) >> (24 + w)) & 1)
                if r0 >= r1:
                    assert whole  # no valid rows in this wave
                else:
                    assert whole == bool(k0 + 32 <= n and m[r0:r1, k0:k0 + 32].all())


def test_c1_4_workload_tile_map_matches_oracle():
    w = si.RANGE_WORKLOADS[6]
    n, groups = w.mask_ranges()
    p = aj.attn_jvp_create_ranges(n, groups, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16)
    rm = RangeMask(n, groups)
    info = p.info
    assert np.array_equal(aj.attn_jvp_tile_map(p), oracle.tile_classes(rm, info["block_q"], info["block_k"]))
    assert info["allowed_pairs_per_head"] == oracle.pair_count(rm)
    assert aj.attn_jvp_plan_flops(p) == 12 * 128 * 12 * oracle.pair_count(rm)


def test_equal_chunks_as_ranges_count_like_the_descriptor():
    for desc in [(1560, 21, 1, 1), (1560, 21, 3, 1), (1560, 21, 1, 0)]:
        tpf, f, c, tf = desc
        n, groups = si.chunked_mask_ranges(tpf, (c,) * (f // c), tf)
        pr = aj.attn_jvp_create_ranges(n, groups, 1, 12, 128)
        pd = aj.attn_jvp_create(desc, 1, 12, 128)
        assert pr.info["allowed_pairs_per_head"] == pd.info["allowed_pairs_per_head"]
        assert aj.attn_jvp_plan_flops(pr) == aj.attn_jvp_plan_flops(pd)


def test_overlapping_and_unsorted_intervals_are_merged():
    p = aj.attn_jvp_create_ranges(64, [(0, 64, [(40, 50), (0, 10), (5, 20), (20, 25), (30, 30)])], 1, 1, 128)
    rr = aj.attn_jvp_row_ranges(p)
    assert rr[0].tolist() == [0, 25, 40, 50]
    assert p.info["allowed_pairs_per_head"] == 64 * 35


@pytest.mark.parametrize("n, groups", [
    (0, [(0, 1, [(0, 1)])]),                       # no tokens
    (10, [(0, 5, [(0, 5)]), (3, 8, [(0, 5)])]),     # overlapping groups
    (10, [(5, 8, [(0, 5)]), (0, 3, [(0, 5)])]),     # unsorted groups
    (10, [(0, 11, [(0, 5)])]),                      # rows past the end
    (10, [(4, 4, [(0, 5)])]),                       # empty group
    (10, [(0, 5, [(0, 11)])]),                      # interval past the end
    (10, [(0, 5, [(6, 3)])]),                       # reversed interval
    (2000, [(0, 5, [(2 * i, 2 * i + 1) for i in range(300)])]),  # 300 disjoint intervals in one group
])
def test_create_ranges_rejects_bad_input(n, groups):
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_create_ranges(n, groups, 1, 1, 128)
    assert e.value.code == 1
    assert aj.attn_jvp_last_error_detail()


def test_range_plan_entry_points_refuse_the_wrong_plan_kind():
    lib = aj._load()
    pr, _ = _plan("gaps")
    pd = aj.attn_jvp_create((4, 3, 1, 1), 1, 1, 64, aj.ATTN_JVP_BF16)
    good = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(9)]  # table + 8 tensors
    assert lib.attn_jvp_fwd(pr.handle, *good[1:], None, None) == 1
    assert "attn_jvp_fwd_table" in aj.attn_jvp_last_error_detail()
    assert lib.attn_jvp_fwd_table(pd.handle, *good, None, None) == 1
    assert lib.attn_jvp_fwd_table(pr.handle, None, *good[1:], None, None) == 2
    assert lib.attn_jvp_fwd_table(pr.handle, ctypes.c_void_p(0x100002), *good[1:], None, None) == 3
    bwd = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(10)]
    assert lib.attn_jvp_bwd(pr.handle, *bwd, None) == 1
    assert aj.attn_jvp_plan_table_size(pd) == 0
    # the forward without tangents: q k v o (+ lse), table first for range plans
    prim = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(4)]
    table = ctypes.c_void_p(0x2000000)
    assert lib.attn_jvp_fwd_primal(pr.handle, *prim, None, None) == 1
    assert "attn_jvp_fwd_primal_table" in aj.attn_jvp_last_error_detail()
    assert lib.attn_jvp_fwd_primal_table(pd.handle, table, *prim, None, None) == 1
    assert lib.attn_jvp_fwd_primal_table(None, table, *prim, None, None) == 2
    assert lib.attn_jvp_fwd_primal_table(pr.handle, None, *prim, None, None) == 2
    assert lib.attn_jvp_fwd_primal_table(pr.handle, ctypes.c_void_p(0x2000002), *prim, None, None) == 3
    for i in range(4):
        bad = list(prim)
        bad[i] = ctypes.c_void_p(0)
        assert lib.attn_jvp_fwd_primal_table(pr.handle, table, *bad, None, None) == 2
    bad = list(prim)
    bad[3] = bad[0]  # o aliases q
    assert lib.attn_jvp_fwd_primal_table(pr.handle, table, *bad, None, None) == 1


def _sections(p):
    """The table's column sections: cblk, corder, centries, cols, cintervals."""
    t = aj.attn_jvp_plan_table(p)
    nq, ne, niv, nkb, nce, nciv = (int(t[i]) for i in (1, 2, 3, 5, 6, 7))
    n = p.seq_len
    o = 8 + (nq + 1) + nq + ne + n + 2 * niv
    out = []
    for size in (nkb + 1, nkb, nce, n, 2 * nciv):
        out.append(t[o:o + size])
        o += size
    assert o == len(t)
    return out


@pytest.mark.parametrize("name", sorted(MASKS))
@pytest.mark.parametrize("dtype", [aj.ATTN_JVP_BF16, aj.ATTN_JVP_FP32])
def test_column_tiles_and_whole_bits_match_the_mask_columns(name, dtype):
    p, rm = _plan(name, dtype, 64)
    cblk, corder, cent, _, _ = _sections(p)
    info = aj.attn_jvp_plan_bwd_info(p)
    bk = info["block_kv"]
    assert bk == (128 if dtype == aj.ATTN_JVP_BF16 else 32)
    m = oracle.mask_dense(rm)
    n = p.seq_len
    nkb = -(-n // bk)
    assert info["n_key_blocks"] == nkb == len(corder)
    assert info["n_query_blocks"] == p.info["n_query_blocks"]
    assert sorted(corder.tolist()) == list(range(nkb))
    counts = np.diff(cblk)[corder]
    assert np.all(np.diff(counts) <= 0)  # heavy (more query tiles) first
    for kb in range(nkb):
        k0, k1 = kb * bk, min(kb * bk + bk, n)
        tiles = cent[cblk[kb]:cblk[kb + 1]] & 0xffffff
        want = [t for t in range(-(-n // 32)) if m[32 * t:32 * t + 32, k0:k1].any()]
        assert tiles.tolist() == want  # ascending, exactly the tiles with an allowed pair
        for e in cent[cblk[kb]:cblk[kb + 1]]:
            q0 = 32 * (int(e) & 0xffffff)
            for w in range(bk // 32):
                a, z = k0 + 32 * w, min(k0 + 32 * w + 32, k1)
                whole = bool((int(e) >> (24 + w)) & 1)
                if a >= z:
                    assert whole  # no valid keys in this wave
                else:
                    assert whole == bool(q0 + 32 <= n and m[q0:q0 + 32, a:z].all())


@pytest.mark.parametrize("name", sorted(MASKS))
def test_column_intervals_are_the_mask_columns(name):
    p, rm = _plan(name)
    _, _, _, cols, civ = _sections(p)
    m = oracle.mask_dense(rm)
    rows = np.arange(p.seq_len)
    over_two = False
    for j in range(p.seq_len):
        off, cnt = int(cols[j]) >> 8, int(cols[j]) & 255
        iv = civ[2 * off:2 * off + 2 * cnt].reshape(-1, 2)
        assert np.all(iv[:, 0] < iv[:, 1]) and np.all(iv[1:, 0] > iv[:-1, 1])  # sorted, disjoint, not touching
        got = np.zeros(p.seq_len, bool)
        for lo, hi in iv:
            got |= (rows >= lo) & (rows < hi)
        assert np.array_equal(got, m[:, j])
        over_two = over_two or cnt > 2
    if over_two:
        with pytest.raises(aj.AttnJvpError) as e:
            aj.attn_jvp_key_ranges(p)
        assert e.value.code == 1
    else:  # the first two row intervals of each key, as the descriptor plans export them
        kr = aj.attn_jvp_key_ranges(p)
        lo1, hi1, lo2, hi2 = (kr[:, i:i + 1] for i in range(4))
        got = ((rows >= lo1) & (rows < hi1)) | ((rows >= lo2) & (rows < hi2))
        assert np.array_equal(got, m.T)


def test_range_bwd_flops_and_workspace():
    p, rm = _plan("und_gen", b=2, h=3)
    assert aj.attn_jvp_plan_bwd_flops(p) == 10 * 128 * 6 * oracle.pair_count(rm)
    assert aj.attn_jvp_bwd_workspace_size(p) == 8 * 6 * p.seq_len


@pytest.mark.parametrize("name, b, h, regime", [("tf_c1_4_t50", 3, 40, "interleaved"), ("und_gen", 2, 7, "interleaved"),
                                                ("tf_c1_4_t50", 4, 66, "grouped")])
def test_range_bwd_launch_order_is_the_table_order_under_the_xcd_rule(name, b, h, regime):
    p, _ = _plan(name, b=b, h=h)
    _, corder, _, _, _ = _sections(p)
    nk = len(corder)
    order = aj.attn_jvp_bwd_launch_order(p)
    total = b * h * nk
    assert sorted(order.tolist()) == list(range(total))
    # back to task numbers: (b, h) slice times n_key_blocks plus the block's rank in the table order
    rank = np.empty(nk, np.int64)
    rank[corder] = np.arange(nk)
    tasks = (order // nk) * nk + rank[order % nk]
    assert check_launch_rule(tasks, total, nk, 32) == regime  # kDkdvXcdGroup


def test_bwd_table_argument_errors_before_any_device_call():
    lib = aj._load()
    pr, _ = _plan("gaps")
    pd = aj.attn_jvp_create((4, 3, 1, 1), 1, 1, 64, aj.ATTN_JVP_BF16)
    bwd = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(10)]  # q k v o lse d_o dq dk dv ws
    table = ctypes.c_void_p(0x2000000)
    assert lib.attn_jvp_bwd(pr.handle, *bwd, None) == 1
    assert "attn_jvp_bwd_table" in aj.attn_jvp_last_error_detail()
    assert lib.attn_jvp_bwd_table(None, table, *bwd, None) == 2
    assert lib.attn_jvp_bwd_table(pd.handle, table, *bwd, None) == 1
    assert lib.attn_jvp_bwd_table(pr.handle, None, *bwd, None) == 2
    assert lib.attn_jvp_bwd_table(pr.handle, ctypes.c_void_p(0x2000002), *bwd, None) == 3
    for i in range(10):
        bad = list(bwd)
        bad[i] = ctypes.c_void_p(0)
        assert lib.attn_jvp_bwd_table(pr.handle, table, *bad, None) == 2
    bad = list(bwd)
    bad[7] = bad[6]  # dk aliases dq
    assert lib.attn_jvp_bwd_table(pr.handle, table, *bad, None) == 1
    bad = list(bwd)
    bad[0] = ctypes.c_void_p(0x100008)  # q misaligned
    assert lib.attn_jvp_bwd_table(pr.handle, table, *bad, None) == 3


def test_plan_whose_columns_do_not_fit_has_a_forward_but_no_backward():
    # 300 one-row groups with gaps between them all see key 0: 300 separate row intervals
    n = 600
    groups = [(2 * i, 2 * i + 1, [(0, 1)]) for i in range(300)]
    p = aj.attn_jvp_create_ranges(n, groups, 1, 1, 128)
    t = aj.attn_jvp_plan_table(p)
    assert t[5] == 0 and t[6] == 0 and t[7] == 0  # no column sections
    assert p.info["allowed_pairs_per_head"] == 300
    lib = aj._load()
    bwd = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(10)]
    assert lib.attn_jvp_bwd_table(p.handle, ctypes.c_void_p(0x2000000), *bwd, None) == 1
    assert "255" in aj.attn_jvp_last_error_detail()
    for call in (aj.attn_jvp_key_ranges, aj.attn_jvp_bwd_launch_order):
        with pytest.raises(aj.AttnJvpError) as e:
            call(p)
        assert e.value.code == 1
