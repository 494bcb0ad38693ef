"""Host-side checks of the C-ABI library (no GPU needed, no compute calls).

* the library loads and exports every function include/attn_jvp.h declares;
* plan creation validates its arguments and reports errors by code;
* the plan's per-row key ranges equal the oracle's mask bit for bit;
* the plan's tile map (what the kernel streams and masks) equals the
  oracle's tile classification bit for bit, at small sizes with ragged tails
  and at the full workload sizes;
* pair and tile counts agree with the oracle and with closed forms;
* the backward's per-key query ranges are the mask's columns bit for bit,
  its workspace size and useful FLOPs follow their definitions, and its
  argument errors come before any device call.
"""
import ctypes
import os
import re

import numpy as np
import pytest

from conftest import check_launch_rule

import oracle
from oracle import MaskDesc
import masked_attention_jvp_amd as aj
from seeded_inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_jvp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(aj.library_path), reason="libattn_jvp.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_jvp_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert len(names) == 26
    lib = ctypes.CDLL(aj.library_path)
    for name in names:
        assert hasattr(lib, name), name


def test_clock_sample_argument_errors():
    """attn_jvp_clock_sample rejects a null or misaligned buffer before any
    device work (raw pointers through the C ABI)."""
    lib = aj._load()
    assert lib.attn_jvp_clock_sample(None, None) == 2  # ATTN_JVP_E_NULL
    assert lib.attn_jvp_clock_sample(ctypes.c_void_p(0x1004), None) == 3  # ATTN_JVP_E_ALIGN


def test_bwd_noalloc_argument_errors():
    """attn_jvp_bwd_noalloc refuses null pointers, range-list plans and plans
    whose 8 B H N workspace exceeds its fixed 32 MiB, before any device work
    (dummy, aligned pointers are never dereferenced)."""
    lib = aj._load()
    p = ctypes.c_void_p(1 << 20)
    plan = aj.attn_jvp_create_ex((1560, 21, 1, 1), 1, 12, 128, aj.ATTN_JVP_BF16, 0.0, 0)
    assert lib.attn_jvp_bwd_noalloc(None, p, p, p, p, p, p, p, p, p, None) == 2
    assert lib.attn_jvp_bwd_noalloc(plan.handle, p, p, p, p, None, p, p, p, p, None) == 2
    assert "lse" in aj.attn_jvp_last_error_detail()
    big = aj.attn_jvp_create_ex((1560, 21, 1, 1), 1, 65, 128, aj.ATTN_JVP_BF16, 0.0, 0)  # 4,258,800 rows
    assert lib.attn_jvp_bwd_noalloc(big.handle, p, p, p, p, p, p, p, p, p, None) == 7
    assert "33554432" in aj.attn_jvp_last_error_detail()
    n, groups = 64, [(0, 64, [(0, 64)])]
    rp = aj.attn_jvp_create_ranges(n, groups, 1, 1, 128, aj.ATTN_JVP_BF16)
    assert lib.attn_jvp_bwd_noalloc(rp.handle, p, p, p, p, p, p, p, p, p, None) == 1


def test_shader_clock_from_two_samples():
    """Per XCD: 100 MHz x (shader counter change) / (real-time counter
    change), pairing the two samples by XCD number in any order."""
    before = np.array([[x, 1000 * x, 500, 0] for x in range(8)], dtype=np.int64)
    after = np.array([[x, 1000 * x + 2000 * (10 + x), 500 + 100 * 10, 0] for x in reversed(range(8))],
                     dtype=np.int64)
    mhz = aj.shader_clock_mhz(before.ravel(), after.ravel())
    assert sorted(mhz) == list(range(8))
    for x in range(8):
        assert mhz[x] == pytest.approx(100.0 * 2000 * (10 + x) / 1000)


def test_error_strings():
    assert aj.attn_jvp_error_string(0) == "ok"
    assert "null" in aj.attn_jvp_error_string(2)
    assert aj.attn_jvp_error_string(99) == "unknown error code"


@pytest.mark.parametrize("desc, b, h, d, dt, code", [
    ((0, 3, 1, 1), 1, 1, 64, 0, 1),        # tokens_per_frame < 1
    ((4, 3, 2, 1), 1, 1, 64, 0, 1),        # n_frames not a multiple of frames_per_chunk
    ((4, 3, 1, 2), 1, 1, 64, 0, 1),        # tf_layout not in {0, 1}
    ((4, 3, 1, 1), 0, 1, 64, 0, 1),        # batch < 1
    ((4, 3, 1, 1), 1, 1, 96, 0, 1),        # unsupported head_dim
    ((4, 3, 1, 1), 1, 1, 64, 7, 1),        # unknown dtype
    ((1 << 20, 1 << 11, 1, 1), 1, 1, 64, 0, 7),  # sequence too long
    ((1 << 12, 1 << 11, 1, 0), 1, 1, 128, 0, 7),  # bf16: N d 2 = 2^31 bytes per head
    ((1 << 13, 1 << 11, 1, 0), 1, 1, 128, 1, 7),  # fp32: N d = 2^31 elements per head
])
def test_create_rejects_bad_arguments(desc, b, h, d, dt, code):
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_create(desc, b, h, d, dt)
    assert e.value.code == code
    assert aj.attn_jvp_last_error_detail()


def test_per_head_size_limits_by_dtype():
    # bf16 byte offsets are 32-bit: N d 2 < 2^31; the fp32 kernel indexes elements with 64 bits: N d < 2^31
    n = 1 << 23  # d = 128: bf16 needs exactly 2^31 bytes per head, fp32 2^30 elements
    aj.attn_jvp_create((n, 1, 1, 0), 1, 1, 128, aj.ATTN_JVP_FP32)
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_create((n, 1, 1, 0), 1, 1, 128, aj.ATTN_JVP_BF16)
    assert e.value.code == 7
    aj.attn_jvp_create((n - 1, 1, 1, 0), 1, 1, 128, aj.ATTN_JVP_BF16)
    aj.attn_jvp_create((n, 1, 1, 0), 1, 1, 64, aj.ATTN_JVP_BF16)


@pytest.mark.parametrize("desc, flags", [((4, 3, 1, 0), 1), ((4, 3, 1, 1), 2), ((4, 3, 1, 1), 0x80000000)])
def test_create_ex_rejects_bad_flags(desc, flags):
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_create_ex(desc, 1, 1, 64, aj.ATTN_JVP_BF16, 0.0, flags)
    assert e.value.code == 1
    assert aj.attn_jvp_last_error_detail()


@pytest.mark.parametrize("desc", [(16, 3, 1, 1), (2, 6, 3, 1), (160, 9, 3, 1), (7, 5, 1, 0), (1560, 21, 1, 1),
                                  (1560, 21, 3, 1), (1560, 21, 1, 0)])
@pytest.mark.parametrize("d", [64, 128])
def test_plan_flops_match_oracle_counts(desc, d):
    b, h = 2, 3
    p = aj.attn_jvp_create(desc, b, h, d, aj.ATTN_JVP_BF16)
    assert aj.attn_jvp_plan_flops(p) == b * h * oracle.useful_flops(MaskDesc(*desc), d)
    p0 = aj.attn_jvp_create_ex(desc, b, h, d, aj.ATTN_JVP_BF16, 0.0, 0)
    assert aj.attn_jvp_plan_flops(p0) == aj.attn_jvp_plan_flops(p)
    if desc[3] == 1:
        pz = aj.attn_jvp_create_ex(desc, b, h, d, aj.ATTN_JVP_FP32, 0.0, aj.ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO)
        assert aj.attn_jvp_plan_flops(pz) == b * h * oracle.useful_flops(MaskDesc(*desc), d, True)


@pytest.mark.parametrize("desc", [(16, 3, 1, 1), (50, 5, 1, 1), (1, 5, 1, 1), (160, 9, 3, 1), (37, 7, 1, 0),
                                  (1560, 21, 1, 1), (1560, 21, 3, 1), (1560, 21, 1, 0), (100, 40, 1, 1)])
@pytest.mark.parametrize("ctz", [0, 1])
def test_launch_order_is_a_heavy_first_permutation(desc, ctz):
    if ctz and desc[3] == 0:
        pytest.skip("clean-tangent-zero needs teacher forcing")
    p = aj.attn_jvp_create_ex(desc, 1, 1, 128, aj.ATTN_JVP_BF16, 0.0, ctz)
    order = aj.attn_jvp_launch_order(p)
    nq = p.info["n_query_blocks"]
    assert sorted(order.tolist()) == list(range(nq))  # every block exactly once
    # a block's work grows with its last chunk: latest blocks of each side first
    if desc[3] == 0:
        assert np.all(np.diff(order) < 0)
    else:
        nbs = nq // 2
        side = (order >= nbs).astype(int)
        for sd in (0, 1):
            assert np.all(np.diff(order[side == sd]) < 0)
        if not ctz:  # sides alternate block by block
            assert np.all(side == np.arange(nq) % 2)
        else:  # two launches: the clean side's blocks, then the noisy side's
            assert np.all(side[:nbs] == 0) and np.all(side[nbs:] == 1)


def test_create_rejects_non_finite_scale():
    with pytest.raises(aj.AttnJvpError) as e:
        aj.attn_jvp_create((4, 3, 1, 1), 1, 1, 64, 0, float("nan"))
    assert e.value.code == 1


def test_fwd_argument_errors_before_any_device_call():
    lib = aj._load()
    p = aj.attn_jvp_create((4, 3, 1, 1), 1, 1, 64, aj.ATTN_JVP_BF16)
    good = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(8)]
    null = list(good)
    null[2] = ctypes.c_void_p(0)
    assert lib.attn_jvp_fwd(p.handle, *null, None, None) == 2
    assert lib.attn_jvp_fwd(None, *good, None, None) == 2
    mis = list(good)
    mis[4] = ctypes.c_void_p(0x10008)
    assert lib.attn_jvp_fwd(p.handle, *mis, None, None) == 3
    alias = list(good)
    alias[6] = alias[0]  # o aliases q
    assert lib.attn_jvp_fwd(p.handle, *alias, None, None) == 1
    assert "overlaps" in aj.attn_jvp_last_error_detail()


def _ranges_to_mask(rr, n):
    keys = np.arange(n)
    lo1, hi1, lo2, hi2 = (rr[:, i:i + 1] for i in range(4))
    return ((keys >= lo1) & (keys < hi1)) | ((keys >= lo2) & (keys < hi2))


SMALL = [(16, 3, 1, 1), (50, 5, 1, 1), (40, 6, 3, 1), (37, 7, 1, 0), (100, 2, 2, 0), (1, 5, 1, 1),
         (3, 9, 3, 1), (130, 3, 1, 1), (64, 4, 2, 1)]


@pytest.mark.parametrize("desc", SMALL)
@pytest.mark.parametrize("dtype", [aj.ATTN_JVP_BF16, aj.ATTN_JVP_FP32])
def test_row_ranges_match_oracle_mask(desc, dtype):
    p = aj.attn_jvp_create(desc, 1, 1, 64, dtype)
    n = p.seq_len
    assert n == MaskDesc(*desc).seq_len
    assert np.array_equal(_ranges_to_mask(aj.attn_jvp_row_ranges(p), n), oracle.mask_dense(desc))


@pytest.mark.parametrize("desc", SMALL)
@pytest.mark.parametrize("dtype, d", [(aj.ATTN_JVP_BF16, 128), (aj.ATTN_JVP_BF16, 64), (aj.ATTN_JVP_FP32, 64)])
def test_tile_map_matches_oracle(desc, dtype, d):
    p = aj.attn_jvp_create(desc, 1, 1, d, dtype)
    info = p.info
    want = oracle.tile_classes(desc, info["block_q"], info["block_k"])
    got = aj.attn_jvp_tile_map(p)
    assert got.shape == want.shape
    assert np.array_equal(got, want)
    assert info["visited_tiles_per_head"] == int((got > 0).sum())
    assert info["allowed_pairs_per_head"] == oracle.pair_count(desc)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_tile_map_matches_oracle_at_workload_size(cfg):
    w = WORKLOADS[cfg]
    p = aj.attn_jvp_create(w.desc, w.batch, w.heads, w.head_dim, aj.ATTN_JVP_BF16)
    info = p.info
    got = aj.attn_jvp_tile_map(p)
    want = oracle.tile_classes(w.desc, info["block_q"], info["block_k"])
    assert np.array_equal(got, want)
    assert info["allowed_pairs_per_head"] == oracle.pair_count(w.desc)
    assert info["visited_tiles_per_head"] == int((want > 0).sum())
    # rows of every query block: the kernel's row ranges agree with the mask on sampled rows
    rr = aj.attn_jvp_row_ranges(p)
    rng = np.random.default_rng(cfg)
    for i in rng.choice(p.seq_len, 64, replace=False):
        keys = np.arange(p.seq_len)
        mine = ((keys >= rr[i, 0]) & (keys < rr[i, 1])) | ((keys >= rr[i, 2]) & (keys < rr[i, 3]))
        assert np.array_equal(mine, oracle.allowed_row(w.desc, int(i)))


def test_plan_info_geometry():
    p = aj.attn_jvp_create((1560, 21, 1, 1), 1, 12, 128, aj.ATTN_JVP_BF16)
    info = p.info
    assert info["seq_len"] == 65520
    bq, bk = info["block_q"], info["block_k"]
    assert info["n_query_blocks"] == 2 * -(-32760 // bq)
    assert info["n_key_tiles"] == -(-65520 // bk)
    assert info["allowed_pairs_per_head"] == 1_124_323_200


@pytest.mark.parametrize("desc", SMALL)
def test_key_ranges_match_oracle_mask_columns(desc):
    p = aj.attn_jvp_create(desc, 1, 1, 64, aj.ATTN_JVP_BF16)
    n = p.seq_len
    assert np.array_equal(_ranges_to_mask(aj.attn_jvp_key_ranges(p), n), oracle.mask_dense(desc).T)


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_key_ranges_match_oracle_at_workload_size(cfg):
    # for sampled rows i: the keys whose query ranges hold i are the row's allowed keys
    w = WORKLOADS[cfg]
    p = aj.attn_jvp_create(w.desc, 1, 1, w.head_dim, aj.ATTN_JVP_BF16)
    kr = aj.attn_jvp_key_ranges(p)
    rng = np.random.default_rng(100 + cfg)
    for i in rng.choice(p.seq_len, 48, replace=False):
        sees = ((i >= kr[:, 0]) & (i < kr[:, 1])) | ((i >= kr[:, 2]) & (i < kr[:, 3]))
        assert np.array_equal(sees, oracle.allowed_row(w.desc, int(i)))


@pytest.mark.parametrize("desc", [(16, 3, 1, 1), (160, 9, 3, 1), (7, 5, 1, 0), (1560, 21, 1, 1), (1560, 21, 3, 1)])
@pytest.mark.parametrize("dtype, d", [(aj.ATTN_JVP_BF16, 128), (aj.ATTN_JVP_FP32, 64)])
def test_bwd_workspace_and_flops(desc, dtype, d):
    b, h = 2, 3
    p = aj.attn_jvp_create(desc, b, h, d, dtype)
    assert aj.attn_jvp_bwd_workspace_size(p) == 8 * b * h * p.seq_len
    assert aj.attn_jvp_plan_bwd_flops(p) == b * h * oracle.backward_useful_flops(MaskDesc(*desc), d)


def test_bwd_argument_errors_before_any_device_call():
    lib = aj._load()
    p = aj.attn_jvp_create((4, 3, 1, 1), 1, 1, 64, aj.ATTN_JVP_BF16)
    # q k v o lse d_o dq dk dv workspace: disjoint, aligned fake addresses
    good = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(10)]
    assert lib.attn_jvp_bwd(None, *good, None) == 2
    for i in range(10):
        bad = list(good)
        bad[i] = ctypes.c_void_p(0)
        assert lib.attn_jvp_bwd(p.handle, *bad, None) == 2
    for i, off in ((0, 8), (5, 2), (9, 2), (7, 4)):
        bad = list(good)
        bad[i] = ctypes.c_void_p(good[i].value + off)
        assert lib.attn_jvp_bwd(p.handle, *bad, None) == 3, i
    for out, inp in ((6, 0), (8, 5), (9, 4), (7, 8), (9, 6)):
        bad = list(good)
        bad[out] = bad[inp]
        assert lib.attn_jvp_bwd(p.handle, *bad, None) == 1, (out, inp)
        assert "overlaps" in aj.attn_jvp_last_error_detail()


@pytest.mark.parametrize("desc, b, h, regime", [
    ((1560, 21, 1, 1), 1, 12, "grouped"), ((1560, 21, 3, 1), 2, 12, "grouped"), ((1560, 21, 1, 0), 1, 12, "grouped"),
    ((1560, 21, 1, 1), 1, 40, "grouped"),
    ((100, 40, 1, 1), 1, 37, "grouped"),       # 9 full rounds of 256: 8 grouped, the rest in sequence order
    ((50, 5, 1, 1), 1, 3, "interleaved"),      # 12 workgroups
    ((1560, 21, 1, 1), 1, 3, "interleaved")])  # 1536 workgroups, under 8 per CU
def test_bwd_launch_order_follows_the_xcd_rule(desc, b, h, regime):
    p = aj.attn_jvp_create(desc, b, h, 128, aj.ATTN_JVP_BF16)
    info = aj.attn_jvp_plan_bwd_info(p)
    nk = info["n_key_blocks"]
    assert nk == p.info["n_query_blocks"]  # key blocks are cut like query blocks
    order = aj.attn_jvp_bwd_launch_order(p)
    assert check_launch_rule(order, b * h * nk, nk, 32) == regime  # kDkdvXcdGroup


def test_primal_argument_errors_before_any_device_call():
    lib = aj._load()
    p = aj.attn_jvp_create((4, 3, 1, 1), 1, 1, 64, aj.ATTN_JVP_BF16)
    good = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(4)]  # q k v o
    assert lib.attn_jvp_fwd_primal(None, *good, None, None) == 2
    for i in range(4):
        bad = list(good)
        bad[i] = ctypes.c_void_p(0)
        assert lib.attn_jvp_fwd_primal(p.handle, *bad, None, None) == 2
    bad = list(good)
    bad[2] = ctypes.c_void_p(good[2].value + 8)
    assert lib.attn_jvp_fwd_primal(p.handle, *bad, None, None) == 3
    bad = list(good)
    bad[3] = bad[1]  # o aliases k
    assert lib.attn_jvp_fwd_primal(p.handle, *bad, None, None) == 1
    pr = aj.attn_jvp_create_ranges(16, [(0, 16, [(0, 16)])], 1, 1, 64)
    assert lib.attn_jvp_fwd_primal(pr.handle, *good, None, None) == 1


def test_plan_cache_is_bounded_lru():
    """The convenience functions' plan cache keeps at most PLAN_CACHE_SIZE
    plans, evicting the least recently used."""
    import torch
    saved = dict(aj._plan_cache)
    aj._plan_cache.clear()
    try:
        n = aj.PLAN_CACHE_SIZE
        first = aj._cached_plan((4, 3, 1, 1), (1, 1, 24, 64), aj.ATTN_JVP_BF16, None)
        for i in range(n + 5):
            aj._cached_plan((4, 3, 1, 1), (1, 2 + i, 24, 64), aj.ATTN_JVP_BF16, None)
            if i == 0:  # a hit moves the first plan to the back
                assert aj._cached_plan((4, 3, 1, 1), (1, 1, 24, 64), aj.ATTN_JVP_BF16, None) is first
        assert len(aj._plan_cache) == n
        keys = list(aj._plan_cache)
        assert all(k[1][1] >= 2 for k in keys), "the oldest plans are evicted"
    finally:
        aj._plan_cache.clear()
        aj._plan_cache.update(saved)
