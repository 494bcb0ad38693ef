// mask_index.h -- index arithmetic of the teacher-forcing / block-causal mask
// and of the tile schedule, shared by the host planner and the device kernels.
//
// Mask (Causal-rCM, arXiv 2606.25473, section 2.3 and section 3.1.1 eq. 8;
// chunking from section 4): with T tokens per chunk and N_h tokens per side,
//   clean row of chunk c  -> keys [0, (c+1) T)
//   noisy row of chunk c  -> keys [0, c T)  and  [N_h + c T, N_h + (c+1) T)
// so every row's key set is at most two half-open intervals.
//
// Schedule (Appendix B, "sparse custom mask representation" and Algorithm 1:
// one task per query block, streaming only the key blocks that intersect the
// task's key ranges, with the same schedule for scores and score tangents):
// query blocks are cut per side, key tiles from key 0 over the whole
// sequence.  The rows of one block lie on one side and in consecutive
// chunks, so the union of their key sets is again at most two intervals,
// which the kernel walks tile by tile.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define AJ_HD __host__ __device__ __forceinline__
#else
#define AJ_HD inline
#endif

namespace attn_jvp {

struct MaskGeom {
  int32_t side_len;   // N_h
  int32_t chunk_len;  // T
  int32_t tf;         // 0 block-causal, 1 teacher-forcing [clean | noisy]
  int32_t seq_len;    // N = N_h * (1 + tf)
};

// Half-open key intervals [lo1, hi1) and [lo2, hi2); empty when lo >= hi.
struct Ranges {
  int32_t lo1, hi1, lo2, hi2;
};

// Tile-index intervals [a0, a1) and [b0, b1), disjoint, in walking order.
struct TileSpans {
  int32_t a0, a1, b0, b1;
};

AJ_HD int32_t cdiv(int32_t a, int32_t b) { return (a + b - 1) / b; }

AJ_HD bool is_noisy(const MaskGeom& g, int32_t i) { return g.tf != 0 && i >= g.side_len; }

AJ_HD int32_t chunk_of(const MaskGeom& g, int32_t i) {
  return (is_noisy(g, i) ? i - g.side_len : i) / g.chunk_len;
}

// Allowed keys of query row i.
AJ_HD Ranges row_ranges(const MaskGeom& g, int32_t i) {
  const int32_t c = chunk_of(g, i);
  if (!is_noisy(g, i)) return Ranges{0, (c + 1) * g.chunk_len, 0, 0};
  return Ranges{0, c * g.chunk_len, g.side_len + c * g.chunk_len, g.side_len + (c + 1) * g.chunk_len};
}

// Query rows that attend to key j (the transpose of row_ranges):
//   clean key of chunk c -> clean rows [c T, N_h) and noisy rows [N_h + (c+1) T, N)
//   noisy key of chunk c -> noisy rows [N_h + c T, N_h + (c+1) T)
//   block-causal key of chunk c -> rows [c T, N)
AJ_HD Ranges col_ranges(const MaskGeom& g, int32_t j) {
  const int32_t c = chunk_of(g, j);
  if (!g.tf) return Ranges{c * g.chunk_len, g.seq_len, 0, 0};
  if (is_noisy(g, j)) return Ranges{g.side_len + c * g.chunk_len, g.side_len + (c + 1) * g.chunk_len, 0, 0};
  return Ranges{c * g.chunk_len, g.side_len, g.side_len + (c + 1) * g.chunk_len, g.seq_len};
}

AJ_HD bool in_ranges(const Ranges& r, int32_t j) {
  return (j >= r.lo1 && j < r.hi1) || (j >= r.lo2 && j < r.hi2);
}

// Does one interval of r contain all of [k0, k1)?
AJ_HD bool covers(const Ranges& r, int32_t k0, int32_t k1) {
  return (k0 >= r.lo1 && k1 <= r.hi1) || (k0 >= r.lo2 && k1 <= r.hi2);
}

AJ_HD bool meets(const Ranges& r, int32_t k0, int32_t k1) {
  const bool a = r.lo1 < r.hi1 && k0 < r.hi1 && r.lo1 < k1;
  const bool b = r.lo2 < r.hi2 && k0 < r.hi2 && r.lo2 < k1;
  return a || b;
}

AJ_HD int32_t blocks_per_side(const MaskGeom& g, int32_t block_q) { return cdiv(g.side_len, block_q); }

AJ_HD int32_t n_query_blocks(const MaskGeom& g, int32_t block_q) {
  return blocks_per_side(g, block_q) * (g.tf ? 2 : 1);
}

AJ_HD int32_t n_key_tiles(const MaskGeom& g, int32_t block_k) { return cdiv(g.seq_len, block_k); }

// Rows [*r0, *r1) of query block qb (clean-side blocks first).
AJ_HD void qblock_rows(const MaskGeom& g, int32_t block_q, int32_t qb, int32_t* r0, int32_t* r1) {
  const int32_t nbs = blocks_per_side(g, block_q);
  const int32_t side = qb / nbs, k = qb - side * nbs;
  const int32_t base = side * g.side_len;
  const int32_t end = (k + 1) * block_q < g.side_len ? (k + 1) * block_q : g.side_len;
  *r0 = base + k * block_q;
  *r1 = base + end;
}

// Heavy-first launch order within one (b, h): query block handled by
// workgroup t.  A block's work grows with its last chunk, so k walks down.
// Workgroups are handed to the 8 XCDs round robin.
// * default: the sides alternate (clean block k, noisy block k, ...): clean
//   and noisy block k carry the same work, and each XCD streams one side's
//   key ranges;
// * balanced (for plans whose sides carry different work, clean-tangent-
//   zero): slots come in groups of 2 P, the P clean blocks k .. k-P+1 then
//   the P noisy blocks of the same k, so every XCD gets one block of each
//   side per group; the last nbs mod P blocks of each side alternate.
AJ_HD int32_t heavy_first_qblock(const MaskGeom& g, int32_t block_q, int32_t t, bool balanced = false) {
  const int32_t nbs = blocks_per_side(g, block_q);
  if (!g.tf) return nbs - 1 - t;
  if (!balanced) return (t & 1) * nbs + (nbs - 1 - (t >> 1));
  constexpr int32_t P = 8;
  const int32_t full = nbs / P;
  if (t < 2 * P * full) {
    const int32_t grp = t / (2 * P), r = t - grp * 2 * P;
    const int32_t side = r / P;
    return side * nbs + (nbs - 1 - (grp * P + r - side * P));
  }
  const int32_t u = t - 2 * P * full, rem = nbs - P * full;
  return (u & 1) * nbs + (rem - 1 - (u >> 1));
}

// XCD-aware launch order.  Position b of the order over total = n_slices *
// per_slice tasks is logical task launch_task(b, ...): (b, h) slice task /
// per_slice, heavy-first rank task mod per_slice.  Workgroups are handed to
// the 8 XCDs round robin (workgroup b to XCD b mod 8), each XCD runs its
// share in order of arrival on its 32 CUs and has its own L2, so position b
// is meant for XCD b mod 8.  (Kernels with a static grid run position
// blockIdx; the bf16 forward + JVP and backward kernels take positions from
// per-XCD work queues, take_task, which keeps this split and lets an XCD that
// has finished its share take the rest of another's.)
// * Large grids (at least kMinGroupedTasks workgroups and kMinGroupedRounds
//   rounds of 8 G): every round gives each XCD a group of G consecutive
//   positions, so that tasks streaming the same tiles (neighbouring blocks of
//   one chunk) share an L2.  The direction alternates from round to round
//   (XCD x takes group x, then group 7 - x), so the falling heavy-first
//   weights even out over each pair of rounds; only an even number of rounds
//   is grouped and the rest keeps its index.  Where G divides per_slice,
//   positions are rank-major: group k of the sequence holds ranks
//   (k / n_slices) G .. + G - 1 of slice k mod n_slices, so the whole grid
//   runs heavy first across slices, with the lightest blocks of every slice
//   at the end.  (Slice-major, the last round held one slice's heaviest
//   blocks next to another's lightest, and the XCDs that took the heavy ones
//   finished late.)
// * Smaller grids, by `small`: kSmallAcross, heavy first across all slices
//   (the heaviest block of every slice, then the next, ...); kSmallRankGroups,
//   the same across groups of kSmallGroup consecutive tasks of one slice
//   (rank-major over the slices, then the round snake above), which keeps
//   some L2 locality and balances as well where a slice's weights fall
//   slowly along its order (teacher forcing, whose order alternates sides);
//   kSmallIndex, the index order.  A lone unpaired round would load some
//   XCDs far more than others (in a single round of 8 groups of 128, the
//   first group carries about 7 times the work of the fourth), and with few
//   tasks per CU a slice-by-slice order would leave the last slice's heavy
//   blocks to the end.
constexpr int32_t kMinGroupedRounds = 2;
constexpr int32_t kMinGroupedTasks = 2048;  // 8 per CU
constexpr int32_t kSmallIndex = 0, kSmallAcross = 1, kSmallRankGroups = 2;
constexpr int32_t kSmallGroup = 32;
AJ_HD int32_t launch_task(int32_t b, int32_t total, int32_t per_slice, int32_t G, int32_t small = kSmallAcross) {
  const int32_t round = 8 * G;
  const int32_t rounds = total / round;
  if (total >= kMinGroupedTasks && rounds >= kMinGroupedRounds) {
    const int32_t r = b / round;
    int32_t t = b;
    if (r < (rounds & ~1)) {
      const int32_t u = b - r * round;
      const int32_t x = (r & 1) ? 7 - (u & 7) : (u & 7);
      t = r * round + x * G + (u >> 3);
    }
    if (per_slice % G != 0) return t;
    const int32_t n_slices = total / per_slice;
    const int32_t grp = t / G, rg = grp / n_slices, s = grp - rg * n_slices;
    return s * per_slice + rg * G + (t - grp * G);
  }
  if (small == kSmallIndex) return b;
  const int32_t n_slices = total / per_slice;
  if (small == kSmallRankGroups) {
    // groups of kSmallGroup tasks of one slice, group g = rank g / n_slices
    // of slice g mod n_slices; full rounds of 8 groups snake over the XCDs,
    // then the remaining groups and the tasks past the last whole group of
    // each slice follow in that order
    constexpr int32_t GS = kSmallGroup;
    const int32_t per_groups = per_slice / GS;
    const int32_t n_groups = n_slices * per_groups;
    const int32_t full = n_groups / 8;
    if (b < full * 8 * GS) {
      const int32_t r = b / (8 * GS), u = b - r * 8 * GS;
      const int32_t grp = r * 8 + ((r & 1) ? 7 - (u & 7) : (u & 7));
      const int32_t rank = grp / n_slices;
      return (grp - rank * n_slices) * per_slice + rank * GS + (u >> 3);
    }
    int32_t rest = b - full * 8 * GS;
    if (rest < (n_groups - full * 8) * GS) {
      const int32_t grp = full * 8 + rest / GS;
      const int32_t rank = grp / n_slices;
      return (grp - rank * n_slices) * per_slice + rank * GS + (rest - (rest / GS) * GS);
    }
    rest -= (n_groups - full * 8) * GS;
    const int32_t k = rest / n_slices;
    return (rest - k * n_slices) * per_slice + per_groups * GS + k;
  }
  const int32_t k = b / n_slices;
  return (b - k * n_slices) * per_slice + k;
}

// Union of the key sets of rows [r0, r1) (one side, consecutive chunks).
AJ_HD Ranges block_ranges(const MaskGeom& g, int32_t r0, int32_t r1) {
  const Ranges first = row_ranges(g, r0);
  const Ranges last = row_ranges(g, r1 - 1);
  if (!is_noisy(g, r0)) return Ranges{0, last.hi1, 0, 0};
  return Ranges{0, last.hi1, first.lo2, last.hi2};
}

// Union of the query sets of keys [k0, k1) (one side, consecutive chunks):
// along one side both ends of each interval are non-decreasing in the key,
// so the first key's lower ends and the last key's upper ends bound it.
AJ_HD Ranges block_col_ranges(const MaskGeom& g, int32_t k0, int32_t k1) {
  const Ranges first = col_ranges(g, k0);
  const Ranges last = col_ranges(g, k1 - 1);
  return Ranges{first.lo1, last.hi1, first.lo2, last.hi2};
}

// Is [x0, x1) inside one interval of the ranges of every position of a run
// of consecutive positions on one side (row ranges or column ranges), given
// the run's first and last ranges?  Both ends of each interval are
// non-decreasing along the run, so the intersection of the first intervals
// over the run is [last.lo1, first.hi1), and likewise for the second.
AJ_HD bool run_covers(const Ranges& first, const Ranges& last, int32_t x0, int32_t x1) {
  return (x0 >= last.lo1 && x1 <= first.hi1) || (x0 >= last.lo2 && x1 <= first.hi2);
}

AJ_HD TileSpans block_tiles(const Ranges& u, int32_t block_k) {
  TileSpans s{0, 0, 0, 0};
  if (u.hi1 > u.lo1) {
    s.a0 = u.lo1 / block_k;
    s.a1 = cdiv(u.hi1, block_k);
  }
  if (u.hi2 > u.lo2) {
    s.b0 = u.lo2 / block_k;
    s.b1 = cdiv(u.hi2, block_k);
    if (s.b0 < s.a1) s.b0 = s.a1;
    if (s.b1 < s.b0) s.b1 = s.b0;
  }
  return s;
}

AJ_HD int32_t span_count(const TileSpans& s) { return (s.a1 - s.a0) + (s.b1 - s.b0); }

// Tile index of the it-th streamed tile.
AJ_HD int32_t span_tile(const TileSpans& s, int32_t it) {
  const int32_t na = s.a1 - s.a0;
  return it < na ? s.a0 + it : s.b0 + (it - na);
}

// Streamed tiles with index below x (the span's tiles increase with the
// step index, range a before range b).
AJ_HD int32_t span_count_below(const TileSpans& s, int32_t x) {
  const int32_t na = s.a1 - s.a0, nb = s.b1 - s.b0;
  const int32_t ca = x - s.a0 < 0 ? 0 : (x - s.a0 > na ? na : x - s.a0);
  const int32_t cb = x - s.b0 < 0 ? 0 : (x - s.b0 > nb ? nb : x - s.b0);
  return ca + cb;
}

// Steps t of a span whose tile index lies in [lo, hi): t in the set iff
// (unsigned)(t - first) < (unsigned)count (count 0: no step).  Since the
// span's tiles increase with t, such steps are consecutive.
struct StepRange {
  int32_t first, count;
};
AJ_HD StepRange span_steps_in(const TileSpans& s, int32_t lo, int32_t hi) {
  const int32_t a = span_count_below(s, lo), b = span_count_below(s, hi);
  return StepRange{a, b > a ? b - a : 0};
}
AJ_HD bool in_steps(const StepRange& r, int32_t t) { return (uint32_t)(t - r.first) < (uint32_t)r.count; }

// Tiles of `block` keys (or rows) that lie whole inside [x0, x1): indices
// ceil(x0 / block) .. floor(x1 / block) - 1 (x0, x1 >= 0; empty if x1 <= x0).
AJ_HD int32_t first_whole_tile(int32_t x0, int32_t block) { return cdiv(x0, block); }
AJ_HD int32_t end_whole_tile(int32_t x1, int32_t block) { return x1 / block; }

}  // namespace attn_jvp
