"""The workgroup -> task mapping of the kernels' grids (launch_task in
csrc/mask_index.h), compiled for the host with g++ and checked on the CPU.

Every kernel takes its task from launch_task(blockIdx, gridDim, per_slice,
G, small): if the mapping missed a task, a query or key block would never be
computed, and if it repeated one, two workgroups would write the same
outputs.  So for every regime (grouped large grids; small grids in index
order, heavy first across slices, and rank-major groups of 32 tasks of one
slice) it must be a permutation of 0 .. total-1, including grids with
partial groups and tails (per_slice not a multiple of 32, a number of groups
not a multiple of 8).  The tests also pin the documented structure of each
regime.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "masked_attention_jvp_amd", "csrc")

HARNESS = r"""
#include <cstdio>
#include <cstdlib>
#include "mask_index.h"
int main(int argc, char** argv) {
  const int total = atoi(argv[1]), per_slice = atoi(argv[2]), G = atoi(argv[3]), small = atoi(argv[4]);
  for (int b = 0; b < total; ++b) printf("%d\n", attn_jvp::launch_task(b, total, per_slice, G, small));
  return 0;
}
"""

SMALL_INDEX, SMALL_ACROSS, SMALL_RANK_GROUPS = 0, 1, 2  # kSmallIndex, kSmallAcross, kSmallRankGroups
GROUP = 32                                            # kSmallGroup


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    d = tmp_path_factory.mktemp("launch_task")
    src, exe = d / "lt.cpp", d / "lt"
    src.write_text(HARNESS)
    subprocess.run([gxx, "-O1", "-std=c++17", f"-I{CSRC}", str(src), "-o", str(exe)], check=True)

    def run(total, per_slice, G, small):
        out = subprocess.run([str(exe), str(total), str(per_slice), str(G), str(small)],
                             capture_output=True, text=True, check=True).stdout
        return np.array([int(x) for x in out.split()], dtype=np.int64)
    return run


def _is_grouped(total, G):
    return total >= 2048 and total // (8 * G) >= 2


# (slices, per_slice, G): small and large grids, per_slice not a multiple of
# 32, numbers of 32-task groups not a multiple of 8, single slices
GRIDS = [
    (1, 1, 128), (1, 7, 128), (3, 5, 128), (1, 33, 128), (2, 31, 128), (3, 512, 128), (3, 513, 128),
    (5, 100, 128), (6, 512, 128), (12, 512, 128), (24, 1024, 128), (40, 512, 128), (7, 97, 16),
    (13, 300, 64), (12, 171, 16), (3, 1537, 128), (16, 65, 128), (9, 64, 128),
]


@pytest.mark.parametrize("small", [SMALL_INDEX, SMALL_ACROSS, SMALL_RANK_GROUPS])
@pytest.mark.parametrize("slices, per_slice, G", GRIDS)
def test_launch_task_is_a_permutation(harness, slices, per_slice, G, small):
    total = slices * per_slice
    tasks = harness(total, per_slice, G, small)
    assert tasks.shape == (total,)
    assert np.array_equal(np.sort(tasks), np.arange(total)), "not a permutation"


def _sequence_task(t, slices, per_slice, G):
    """Task at position t of the grouped regime's sequence: rank-major where G
    divides per_slice (group k = ranks (k // slices) G .. + G - 1 of slice
    k % slices), else the index itself."""
    t = np.asarray(t)
    if per_slice % G:
        return t
    k = t // G
    return (k % slices) * per_slice + (k // slices) * G + t % G


@pytest.mark.parametrize("slices, per_slice, G", [g for g in GRIDS if _is_grouped(g[0] * g[1], g[2])])
def test_grouped_regime_is_independent_of_the_small_rule(harness, slices, per_slice, G):
    total = slices * per_slice
    ref = harness(total, per_slice, G, SMALL_ACROSS)
    for small in (SMALL_INDEX, SMALL_RANK_GROUPS):
        assert np.array_equal(harness(total, per_slice, G, small), ref)
    # XCD x (positions b = x mod 8) holds sequence group x of each round, then
    # group 7 - x in the next; the odd last round and the rest keep their
    # sequence positions
    rounds = total // (8 * G)
    even = rounds - rounds % 2
    for r in range(even):
        seg = ref[8 * G * r: 8 * G * (r + 1)]
        for x in range(8):
            xs = seg[x::8]
            g = x if r % 2 == 0 else 7 - x
            assert np.array_equal(xs, _sequence_task(8 * G * r + g * G + np.arange(G), slices, per_slice, G))
    assert np.array_equal(ref[8 * G * even:], _sequence_task(np.arange(8 * G * even, total), slices, per_slice, G))


@pytest.mark.parametrize("slices, per_slice, G", [g for g in GRIDS if _is_grouped(g[0] * g[1], g[2]) and g[1] % g[2] == 0])
def test_grouped_regime_is_heavy_first_across_slices(harness, slices, per_slice, G):
    """Where G divides per_slice, the rounds take the slices' rank groups in
    order: no position holds a rank group later than any position of a later
    round, so the lightest blocks of every slice come last."""
    total = slices * per_slice
    tasks = harness(total, per_slice, G, SMALL_ACROSS)
    rank_group = (tasks % per_slice) // G
    rounds = total // (8 * G)
    for r in range(rounds - 1):
        assert rank_group[8 * G * r: 8 * G * (r + 1)].max() <= rank_group[8 * G * (r + 1):].min()


@pytest.mark.parametrize("slices, per_slice", [(s, p) for s, p, G in GRIDS if not _is_grouped(s * p, 128)])
def test_small_index_and_across(harness, slices, per_slice):
    total = slices * per_slice
    assert np.array_equal(harness(total, per_slice, 128, SMALL_INDEX), np.arange(total))
    b = np.arange(total)
    across = harness(total, per_slice, 128, SMALL_ACROSS)
    assert np.array_equal(across, (b % slices) * per_slice + b // slices)


@pytest.mark.parametrize("slices, per_slice", [(s, p) for s, p, G in GRIDS if not _is_grouped(s * p, 128)])
def test_small_rank_groups_structure(harness, slices, per_slice):
    """Groups of 32 consecutive tasks of one slice; group g is rank g // slices
    of slice g % slices; whole rounds of 8 groups go one group per XCD,
    snaking; then the leftover whole groups in order, then the tasks past each
    slice's last whole group, heavy first across slices."""
    total = slices * per_slice
    tasks = harness(total, per_slice, 128, SMALL_RANK_GROUPS)
    per_groups = per_slice // GROUP
    n_groups = slices * per_groups
    full = n_groups // 8
    slice_of, rank = tasks // per_slice, tasks % per_slice

    def group_tasks(g):
        s, k = g % slices, g // slices
        return s * per_slice + k * GROUP + np.arange(GROUP)

    for r in range(full):
        seg = tasks[8 * GROUP * r: 8 * GROUP * (r + 1)]
        for x in range(8):
            g = r * 8 + (7 - x if r % 2 else x)
            assert np.array_equal(seg[x::8], group_tasks(g))
    pos = 8 * GROUP * full
    for g in range(full * 8, n_groups):
        assert np.array_equal(tasks[pos: pos + GROUP], group_tasks(g))
        pos += GROUP
    tail = tasks[pos:]
    assert np.all(rank[pos:] >= per_groups * GROUP)
    k = np.arange(len(tail))
    assert np.array_equal(slice_of[pos:], k % slices)
    assert np.array_equal(rank[pos:], per_groups * GROUP + k // slices)


BALANCED = r"""
#include <cstdio>
#include <cstdlib>
#include "mask_index.h"
int main(int argc, char** argv) {
  attn_jvp::MaskGeom g{};
  g.tf = 1;
  g.chunk_len = atoi(argv[1]);
  g.side_len = atoi(argv[2]);
  g.seq_len = 2 * g.side_len;
  const int bq = atoi(argv[3]);
  const int nq = attn_jvp::n_query_blocks(g, bq);
  for (int t = 0; t < nq; ++t) printf("%d\n", attn_jvp::heavy_first_qblock(g, bq, t, true));
  return 0;
}
"""


@pytest.mark.parametrize("chunk, side", [(1560, 32760), (4680, 32760), (50, 250), (16, 48), (100, 4000)])
def test_balanced_order_of_the_forward_without_tangents(tmp_path, chunk, side):
    """attn_jvp_fwd_primal (descriptor plans) takes heavy_first_qblock's
    balanced order: every block once, each side heaviest first, and aligned
    groups of 16 positions holding 8 clean then 8 noisy blocks, so that the
    round-robin hand-out gives every XCD both sides."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    src, exe = tmp_path / "bal.cpp", tmp_path / "bal"
    src.write_text(BALANCED)
    subprocess.run([gxx, "-O1", "-std=c++17", f"-I{CSRC}", str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe), str(chunk), str(side), "128"], capture_output=True, text=True, check=True).stdout
    order = np.array([int(x) for x in out.split()])
    nq = len(order)
    nbs = nq // 2
    assert sorted(order.tolist()) == list(range(nq))
    sd = (order >= nbs).astype(int)
    for s in (0, 1):
        assert np.all(np.diff(order[sd == s]) < 0)
    full = (nbs // 8) * 16
    for g0 in range(0, full, 16):
        assert sd[g0:g0 + 8].sum() == 0 and sd[g0 + 8:g0 + 16].sum() == 8
    for x in range(8):
        sl = sd[:full][x::8]
        assert int(sl.sum()) * 2 == len(sl)
