"""Host model of the LDS rings of the backward kernels and of the forward +
JVP kernel (no GPU).

Both backward kernels stream 32-row tiles through an S-stage LDS ring: step j
reads tiles j, j+1 and (after its barrier slot) j+2, and issues the DMA of
tile j+A into the stage of tile j+A-S; every P-th step has a workgroup
barrier, before which each wave waits for its own LDS reads and for its DMA
shares of the tiles up to j+P+1.  This test writes that event order out per
step, as the kernels issue it, and checks on it, for the constants in the
kernel source:
* read after DMA: every read of a tile comes after a barrier at which all
  waves had waited for that tile's DMA;
* DMA after read: a stage is refilled only after a barrier that follows the
  last read of the tile it held (reads may be in flight until the wait
  before the next barrier);
and that the compile-time conditions in the source (A >= P+2, S >= A+P,
S % P == 0) admit exactly the settings for which the model finds no hazard
and every tile's DMA is issued at least one step before the barrier that
certifies it.
"""
import os
import re

import pytest

SRC = os.path.join(os.path.dirname(__file__), "..", "masked_attention_jvp_amd", "csrc", "attn_jvp_bwd_kernels.hip")


def _constants():
    text = open(SRC).read()
    get = lambda name: int(re.search(r"constexpr int %s = (\d+);" % name, text).group(1))
    return get("kBwdStages"), get("kBwdAhead"), get("kBwdBarrierEvery")


def _events(S, A, P, n_steps):
    """Program-order events of one wave (all waves run the same order)."""
    ev = []
    for j in range(n_steps):
        # phase 1: K/V (Q/dO) fragments of tile j+1, the DMA share of tile
        # j+A, the transposed reads of tile j
        ev.append(("read", j + 1))
        ev.append(("dma", j + A))
        ev.append(("read", j))
        # phase 2: barrier slot, then the first fragments of tile j+2
        if j % P == 0:
            ev.append(("barrier", j + P + 1))  # tiles up to j+P+1 waited for
        ev.append(("read", j + 2))
    return ev


def _hazards(S, A, P, n_steps=40):
    ev = _events(S, A, P, n_steps)
    first_tiles = range(A)  # issued by the prologue, certified by its barrier
    certified = set(t for t in range(2))  # the prologue waits for tiles 0, 1
    issued_at = {t: -1 for t in first_tiles}
    pending_reads = []  # tiles with reads not yet known complete
    completed_reads = {}  # tile -> index of the last barrier behind its reads
    stage_tile = {t % S: t for t in first_tiles}
    last_read = {}
    problems = []
    barriers = 0
    for i, (kind, t) in enumerate(ev):
        if kind == "read":
            if t not in certified:
                problems.append(f"read of tile {t} before its DMA was certified")
            last_read[t] = i
            pending_reads.append(t)
        elif kind == "dma":
            old = stage_tile.get(t % S)
            if old is not None and old != t:
                if last_read.get(old, -1) > completed_reads.get(old, -2):
                    problems.append(f"DMA of tile {t} into the stage of tile {old} before its reads completed")
            stage_tile[t % S] = t
            issued_at[t] = i
        elif kind == "barrier":
            barriers += 1
            for u in pending_reads:
                completed_reads[u] = i
            pending_reads = []
            for u in range(t + 1):
                if u not in issued_at:
                    problems.append(f"barrier certifies tile {u}, whose DMA was not issued")
                certified.add(u)
    return problems


def _lead_ok(A, P):
    # tile b+P+1, certified at the barrier of step b, was issued in step
    # b+P+1-A: at least one step before
    return A >= P + 2


def test_source_constants_are_hazard_free():
    S, A, P = _constants()
    assert _hazards(S, A, P) == []
    assert _lead_ok(A, P)


def test_static_assert_matches_the_model():
    text = open(SRC).read()
    assert "kBwdAhead >= kBwdBarrierEvery + 2" in text and "kBwdStages >= kBwdAhead + kBwdBarrierEvery" in text
    for S in range(2, 13):
        for P in (1, 2, 3, 4):
            for A in range(1, S + 1):
                if S % P or S % 2:
                    continue  # the unrolled steps need these (barrier slots, score-buffer alternation)
                model_ok = not _hazards(S, A, P) and _lead_ok(A, P)
                assert_ok = A >= P + 2 and S >= A + P
                assert model_ok == assert_ok, (S, A, P, _hazards(S, A, P)[:2])


@pytest.mark.parametrize("S, A, P", [(6, 5, 2), (4, 4, 1), (6, 3, 2)])
def test_the_model_finds_planted_mistakes(S, A, P):
    # a refill of the stage still being read (A = S - P + 1, A = S), and a
    # read of a tile not yet waited for (A < P + 2 with barriers every P)
    assert _hazards(S, A, P) or not _lead_ok(A, P)


def test_forward_ring_is_hazard_free():
    # The forward + JVP kernel's ring has the same event order: K (and tK)
    # fragments of tile j+1 in phase 1 with the DMA of tile j+3, the V reads
    # of tile j, a barrier in every step after the wait for tile j+2, then
    # the first K reads of tile j+2.
    fwd = os.path.join(os.path.dirname(SRC), "attn_jvp_kernels.hip")
    text = open(fwd).read()
    kernel = text[text.index("fwd_bf16_kernel(FwdParams p)"):text.index("fwd_fp32_kernel(FwdParams p)")]
    S = int(re.search(r"constexpr int STAGES = (\d+);", kernel).group(1))
    A = int(re.search(r"using AH = std::integral_constant<int, \(ST \+ (\d+)\) % STAGES>;", kernel).group(1))
    assert (S, A) == (4, 3)
    assert _hazards(S, A, 1) == [] and _lead_ok(A, 1)
