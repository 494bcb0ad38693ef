// attn_jvp_kernels.hip -- gfx950 kernels for block-causal / teacher-forcing
// masked attention forward + forward-mode JVP.
//
// What is computed (Causal-rCM, arXiv 2606.25473, Appendix B, eqs. 42-45 and
// Algorithm 1): one online-softmax pass per query block that keeps, beside
// the FlashAttention-2 accumulators (row max m, row sum l, sum p~ v), the JVP
// accumulators sum p~ tv, sum p~ ts v and the row term r = sum p~ ts, all
// rescaled by the same online factor; the epilogue forms
//   o = acc_o / l,   to = (acc_tv + acc_tsv) / l - (r / l) o
// with the normalised o.  All accumulators take the same rescale and the
// same 1/l; the fp32 kernel carries acc_tv + acc_tsv as one sum, the bf16
// kernel keeps them apart (acc_tsv with the unscaled score tangent, the
// scale applied once in the epilogue).
//
// bf16 kernel (one workgroup = one query block of 32*NW rows, one wave = 32
// query rows, 64-wide wavefronts, v_mfma_f32_32x32x16_bf16 with fp32
// accumulation):
// * scores are formed transposed, S^T = K Q^T, so lane l owns query l%32 and
//   16 of the 32 keys of a tile; row max and row sums stay in-lane plus one
//   permlane32 swap with the partner lane l^32;
// * the S^T accumulator, rounded to bf16, is directly the B operand of
//   O^T += V^T P^T: its 8 values per 16-key chunk are keys {4h..4h+3} and
//   {8+4h..8+4h+3}, and V^T is fetched in exactly that key order with the
//   gfx950 transposing LDS read (ds_read_b64_tr_b16), so V stays row-major;
// * the score MFMAs write vector registers directly (VGPR form), so the
//   softmax reads them with no accumulator-to-vector copies;
// * K, tK, V, tV tiles of 32 keys go HBM -> LDS by buffer_load ... lds (no
//   registers, no VALU), into a ring of 4 stages; rows are XOR-swizzled in
//   16-byte groups so the fragment reads are bank-conflict free; loads past
//   the end of the sequence return zeros;
// * software pipelining: the score MFMAs of tile j+1 sit in the same basic
//   block as the softmax of tile j and the P.V MFMAs of tile j, one MFMA per
//   scheduling slot with a share of the vector work, so the matrix cores and
//   the vector ALUs of one wave overlap;
// * rescaling is lazy: the stored row max only moves when a tile's max
//   exceeds it by more than 2^8 (in exp2 units), which keeps every p~ <= 256
//   and is exact in real arithmetic because l, r and the accumulators all
//   share the stored max;
// * whole key tiles outside the block's key ranges are never visited; the
//   element mask is applied only when some row of the wave does not cover
//   the whole tile;
// * calls without tangents, and the clean side of clean-tangent-zero plans,
//   run a primal-only instance that holds K and V only, at two workgroups
//   per CU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "attn_jvp_launch.h"
#include "kernel_common.h"
#include "mask_index.h"

namespace attn_jvp {

constexpr float kLazyRescaleLog2 = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

// Tile modes of the bf16 kernel.  kFull: the general operation.  With the
// clean-tangent-zero option (teacher forcing, clean tokens carry no tangent):
// kCleanKeys for noisy rows against clean keys (tk = tv = 0 there, so
// ts' = tq.k and there is no p~ tv term), kPrimal for clean rows (tq = 0 and
// every key they see is clean, so t_o = 0 and only o and lse are formed).
enum : int { kFull = 0, kCleanKeys = 1, kPrimal = 2 };

template <int D, int NW, bool CTZ, bool TABLE, bool PO = false>
__global__ void __launch_bounds__(NW * 64, PO ? 2 : 1) fwd_bf16_kernel(FwdParams p) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  // Range-list plans have no clean-tangent-zero option: with a table, the
  // CTZ instance is the primal-only kernel (o and lse, every tile in kPrimal).
  // PO: the primal-only kernel at two workgroups per CU (calls without
  // tangents, and the clean side of a clean-tangent-zero plan; with a table,
  // range-list blocks of at most kPoMaxTableEntries tiles).  Its ring holds K
  // and V only (64 KB) and it fits 256 registers, so two workgroups share a
  // CU and each SIMD holds two waves: the hardware issues one wave's MFMAs
  // under the other's softmax.  Every row's arithmetic is the primal tile
  // mode's.
  static_assert(!PO || CTZ, "PO is a primal-only instance");
  constexpr int BC = kBf16BlockK;            // keys per tile (= one MFMA subtile)
  static_assert(BC == 32, "one 32-key subtile per tile");
  constexpr int STAGES = 4;                  // LDS ring depth; tiles j..j+3 resident or in flight
  constexpr int BR = NW * 32;
  constexpr int KS = D / 16;                 // k-steps of the score products
  constexpr int DC = D / 32;                 // 32-wide column blocks of the outputs
  constexpr int NG = 2 * DC;                 // P.V groups per tile (two 16-key halves x DC)
  constexpr int CPR = D / 8;                 // 16-byte groups per row
  constexpr int TILE = BC * D;               // elements per tensor per stage
  constexpr int LOADS = TILE * 2 / 1024 / NW;  // 1 KB DMA loads per wave per tensor
  static_assert(LOADS * NW * 1024 == TILE * 2, "DMA split");

  // The four ring stages are separate objects so that the compiler can tell
  // a read of one stage from a DMA into another (one shared object would make
  // it wait for every DMA in flight before each transposing read).
  // A stage holds K, tK, V, tV (PO: K, V); plane kV is V's.
  constexpr int PLANES = PO ? 2 : 4, kV = PO ? 1 : 2;
  __shared__ __attribute__((aligned(1024))) uint16_t ring0[PLANES * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t ring1[PLANES * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t ring2[PLANES * TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t ring3[PLANES * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int n = lane & 31, h = lane >> 5;

  const MaskGeom g = p.g;
  const int N = g.seq_len;
  // Workgroups take the positions of the heavy-first order, in XCD groups of
  // kFwdXcdGroup (launch_task; the noisy-side launch of a clean-tangent-zero
  // plan: kCtzNoisyXcdGroup), from the per-XCD work queues (take_task):
  // neighbouring blocks of that order, which stream nearly the same key tiles,
  // share an XCD's L2, and an XCD that finishes its share early takes the
  // rest of another's.  The clean-tangent-zero instances (one side per
  // launch; the primal call over both sides in the balanced order, 8 clean
  // and 8 noisy blocks in turn) keep the index order on small grids, where
  // that was 3 % faster than heavy first across heads.  On small grids
  // general teacher-forcing plans take rank-major groups of 32 (3 % faster
  // at 3 heads than heavy first across heads, which the other plans keep).
  const int32_t small = (CTZ && !TABLE) ? kSmallIndex
                        : (!TABLE && p.g.tf) ? kSmallRankGroups : kSmallAcross;
  const int pos = workgroup_task(p.queues, p.n_tasks);
  if (pos < 0) return;  // the queues were empty: no task for this workgroup
  constexpr int32_t kGroup = (CTZ && !PO && !TABLE) ? kCtzNoisyXcdGroup : kFwdXcdGroup;
  const int task = launch_task(pos, p.n_tasks, p.n_qblocks, kGroup, small);
  const int bh = task / p.n_qblocks;
  int qb, r0, r1, ntiles, e0 = 0;
  TileSpans sp{0, 0, 0, 0};
  if constexpr (TABLE) {
    // range-list plan: block, rows and tile list from the schedule table
    qb = p.tb_order[task - bh * p.n_qblocks];
    r0 = qb * BR;
    r1 = r0 + BR < N ? r0 + BR : N;
    e0 = p.tb_blk[qb];
    ntiles = p.tb_blk[qb + 1] - e0;
  } else {
    // one side's blocks (p.n_qblocks of them per slice), heavy first
    if (p.side >= 0) qb = p.side * p.n_qblocks + (p.n_qblocks - 1 - (task - bh * p.n_qblocks));
    else if constexpr (CTZ) qb = heavy_first_qblock(g, BR, task - bh * p.n_qblocks, true);
    else qb = heavy_first_qblock(g, BR, task - bh * p.n_qblocks, false);
    qblock_rows(g, BR, qb, &r0, &r1);
    sp = block_tiles(block_ranges(g, r0, r1), BC);
    ntiles = span_count(sp);
  }
  // Range-list plans: the block's tile entries (tile | whole bit of wave w
  // << (24 + w)) staged in LDS for the whole task.
  int32_t* ent = nullptr;
  if constexpr (TABLE) {
    __shared__ int32_t ent_buf[PO ? kPoMaxTableEntries : kMaxTableEntries];
    for (int i = tid; i < ntiles; i += NW * 64) ent_buf[i] = p.tb_ent[e0 + i];
    __syncthreads();
    ent = ent_buf;
  }
  // tile index of the t-th streamed tile (t < ntiles)
  auto tile_at = [&](int t) -> int {
    if constexpr (TABLE) return __builtin_amdgcn_readfirstlane(ent[t] & 0xffffff);
    else return span_tile(sp, t);
  };
  // Range-list plans: the raw entries a step needs (its DMA tile's and the
  // next tile's) are read from LDS one step ahead, so that the step's top
  // takes them without waiting for an LDS read.
  int pf_dma = 0, pf_next = 0;
  auto prefetch_entries = [&](int j, int t_end) {
    if constexpr (TABLE) {
      pf_dma = ent[j + 3 < t_end ? j + 3 : t_end - 1];
      pf_next = ent[j + 1 < ntiles ? j + 1 : ntiles - 1];
    }
  };
  // clean-side blocks of a clean-tangent-zero plan, and every block of a
  // primal call (o and lse only)
  const bool primal_only = PO || (CTZ && TABLE) || (CTZ && (p.primal != 0 || !is_noisy(g, r0)));
  // Clean-tangent-zero, noisy block: the leading tiles whose keys all lie on
  // the clean side (below N_h) need no key tangents.  A tile that reaches N_h
  // (for short sides the two key intervals can even share one) runs in the
  // general mode, whose tk, tv loads give zeros on the clean side.
  int n_clean_tiles = g.side_len / BC - sp.a0;
  n_clean_tiles = n_clean_tiles < 0 ? 0 : (n_clean_tiles > sp.a1 - sp.a0 ? sp.a1 - sp.a0 : n_clean_tiles);

  const size_t base = (size_t)bh * (size_t)N * D;
  const int slice_bytes = N * D * 2;
  // DMA descriptors of k, tk, v, tv over this (b, h) slice.
  const i32x4_t desc[4] = {make_desc((const uint16_t*)p.k + base, slice_bytes),
                           make_desc((const uint16_t*)p.tk + base, slice_bytes),
                           make_desc((const uint16_t*)p.v + base, slice_bytes),
                           make_desc((const uint16_t*)p.tv + base, slice_bytes)};
  // Clean-tangent-zero: tk and tv are read only through descriptors over the
  // noisy half, with per-lane offsets relative to its start; a clean key's
  // offset is negative, i.e. a huge unsigned offset, which the range check
  // turns into zeros.  So no clean-side tangent is ever read, and the one
  // tile that straddles the two halves gets zeros for its clean keys.
  const size_t half = (size_t)g.side_len * D;
  const int half_bytes = g.side_len * D * 2;
  const i32x4_t desc_tn[2] = {make_desc((const uint16_t*)p.tk + base + half, half_bytes),
                              make_desc((const uint16_t*)p.tv + base + half, half_bytes)};

  const int row = r0 + wave * 32 + n;
  const bool row_ok = row < r1;
  // Range-list plans: the row's first two intervals here, any further ones
  // read in the (rare) mask branch; n_iv = 0 for rows in no group.
  int n_iv = 0, iv_off = 0;
  const Ranges rr = [&]() -> Ranges {
    if constexpr (TABLE) {
      Ranges r{0, 0, 0, 0};
      if (row_ok) {
        const int info = p.tb_rows[row];
        n_iv = info & 255;
        iv_off = info >> 8;
        if (n_iv >= 1) {
          r.lo1 = p.tb_iv[2 * iv_off];
          r.hi1 = p.tb_iv[2 * iv_off + 1];
        }
        if (n_iv >= 2) {
          r.lo2 = p.tb_iv[2 * iv_off + 2];
          r.hi2 = p.tb_iv[2 * iv_off + 3];
        }
      }
      return r;
    } else {
      return row_ok ? row_ranges(g, row) : Ranges{0, 0, 0, 0};
    }
  }();
  int max_iv = 0;  // wave-uniform: the most intervals any row of the wave has
  if constexpr (TABLE) {
    int m = n_iv;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o));
    max_iv = __builtin_amdgcn_readfirstlane(m);
  }

  // Q and tQ fragments stay in registers for the whole task (B operands).
  u32x4 qf[KS], tqf[KS];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t*)p.q + base, slice_bytes);
    const __amdgpu_buffer_rsrc_t rtq = make_rsrc((const uint16_t*)p.tq + base, slice_bytes);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = load16(rq, (row * D + 16 * s + 8 * h) * 2);
      tqf[s] = u32x4{0, 0, 0, 0};
    }
    if (!primal_only) {  // clean rows of a clean-tangent-zero plan: no tq read
#pragma unroll
      for (int s = 0; s < KS; ++s) tqf[s] = load16(rtq, (row * D + 16 * s + 8 * h) * 2);
    }
    // tq stays in accumulation registers as a B operand, which leaves vector
    // registers for the score-tangent start tile below
#pragma unroll
    for (int s = 0; s < KS; ++s) keep_in_acc(tqf[s]);
  }

  auto stage = [&](auto st) -> uint16_t* {
    constexpr int S = decltype(st)::value;
    if constexpr (S == 0) return ring0;
    else if constexpr (S == 1) return ring1;
    else if constexpr (S == 2) return ring2;
    else return ring3;
  };
  // DMA of tile t into stage `dst`.  Lane L of 1 KB block `blk` fills LDS
  // group (row, pc) and fetches global group pc ^ row_swz(row) of that row.
  // The per-lane part of the source offset is fixed; the tile's key offset
  // rides in the scalar offset.
  int dma_voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int blk = wave * LOADS + i;
    const int rw = blk * (64 / CPR) + lane / CPR;
    dma_voff[i] = (rw * D + (((lane % CPR) ^ row_swz<D>(rw)) << 3)) * 2;
  }
  // DMA instructions per wave and tile: all four tensors in kFull, K and V
  // otherwise.
  auto lpt = [](auto mode) { return decltype(mode)::value == kFull ? 4 * LOADS : 2 * LOADS; };
  // The q-th DMA instruction of tile t.  Every step issues all of them,
  // branch-free: past the run's last tile that tile is loaded again into the
  // stage that just became free, which nothing reads, so the ring always has
  // the same number of loads in flight.
  // (range-list plans pass the tile index, read once per step: tile_pre)
  auto issue_part = [&](auto mode, uint16_t* dst, int t, int q, int t_end, int tile_pre) {
    int tile;
    if constexpr (TABLE) tile = tile_pre;
    else tile = span_tile(sp, t < t_end ? t : t_end - 1);
    const int soff = tile * BC * D * 2;
    if constexpr (decltype(mode)::value == kFull) {
      const int i = q >> 2, tt = q & 3;
      uint16_t* lds = dst + tt * TILE + (wave * LOADS + i) * 512;
      if (CTZ && (tt & 1)) load16_lds_asm(desc_tn[tt >> 1], lds, dma_voff[i] + (tile * BC - g.side_len) * D * 2, 0);
      else load16_lds_asm(desc[tt], lds, dma_voff[i], soff);
    } else {
      const int i = q >> 1, tt = q & 1;
      load16_lds_asm(desc[2 * tt], dst + tt * kV * TILE + (wave * LOADS + i) * 512, dma_voff[i], soff);
    }
  };
  auto issue = [&](auto mode, uint16_t* dst, int t, int t_end) {
    int tile_pre = 0;
    if constexpr (TABLE) tile_pre = tile_at(t < t_end ? t : t_end - 1);
#pragma unroll
    for (int q = 0; q < lpt(mode); ++q) issue_part(mode, dst, t, q, t_end, tile_pre);
  };

  // accO = sum p~ v, accV = sum p~ tv, accS = sum (p~ ts') v with the
  // unscaled score tangent ts' (the scale is applied once, in the epilogue).
  // Three separate tiles keep each MFMA accumulation chain a few MFMAs apart.
  f32x16 accO[DC], accV[DC], accS[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      accO[c][i] = 0.f;
      accV[c][i] = 0.f;
      accS[c][i] = 0.f;
    }
  }
  // m: reference max of l, r and the accumulators; mn: reference of the
  // latest exponentiated tile (exp2 units).  r = sum p~ (ts' - c) (unscaled).
  float m = -INFINITY, mn = -INFINITY, l = 0.f, r = 0.f;
  const float sl2 = p.score_log2;
  const float scale = p.scale;
  // Shift of the score tangent.  The accumulators take ts' - c for a per-row
  // constant c, not ts': r holds sum p~ (ts' - c) and accS sum p~ (ts' - c) v.
  // Eq. 45 is unchanged by it, since sum p~ (ts' - c) v / l - (sum p~ (ts' - c)
  // / l) o = sum p~ ts' v / l - (r / l) o exactly (o = acc_o / l).  It keeps
  // the bf16 rounding of p~ (ts' - c), the MFMA operand, relative to the
  // spread of ts' around c rather than to ts' itself: when the score tangents
  // of a row share a large part (a key component common to all keys, met by
  // tq), t_o is a small difference of two large terms, and rounding p~ ts'
  // would lose it.  c starts at 0 and moves to the p~-weighted mean of the
  // current tile's ts' whenever the row's reference max moves: first when it
  // becomes finite (the row's first tile with an allowed key), then whenever
  // a tile's max passes it (the earlier tiles then weigh 2^-8 or less).
  // Moving c by dc takes accS -= dc acc_o and r -= dc l.  Every score-tangent
  // MFMA chain starts from -c (negc), so the hot loop does no extra work, and
  // a row's arithmetic depends only on the tiles it sees, in their order (not
  // on how blocks and runs are cut).
  float c_ts = 0.f;
  f32x16 negc;
#pragma unroll
  for (int i = 0; i < 16; ++i) negc[i] = 0.f;
  opaque(negc);

  // transposing-read addresses (element offsets inside a V tile): a lane
  // group of 16 covers 16 columns; its lane L names key 4h + L/4 (and +8),
  // columns 4 (L % 4) .. +3 of the group's 16.
  const int tr_key = 4 * h + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using MFull = std::integral_constant<int, kFull>;
  using MCleanKeys = std::integral_constant<int, kCleanKeys>;
  using MPrimal = std::integral_constant<int, kPrimal>;

  // Per-lane key window of this row: key k is allowed iff
  // (unsigned)(k - lo1) < len1 or (unsigned)(k - lo2) < len2.
  const int len1 = rr.hi1 - rr.lo1, len2 = rr.hi2 - rr.lo2;

  // Tiles that every valid row of this wave sees whole: the wave's rows are
  // consecutive and on one side, so (range 1 of each row starts at key 0 and
  // grows with the row; range 2 slides with the row's chunk) a tile is whole
  // for all of them iff it lies in [0, f1) or in [g0, g1): f1 and g1 from the
  // wave's first valid row, g0 from its last.  Scalar values.
  // In step indices: the tiles lie in [0, f1) or [g0, g1) at steps w1, w2.
  StepRange w1{0, 1 << 30}, w2{0, 0};
  if constexpr (!TABLE) {
    const int wa = r0 + wave * 32;
    const int wb = wa + 32 < r1 ? wa + 32 : r1;
    if (wa < wb) {
      const Ranges first = row_ranges(g, wa), last = row_ranges(g, wb - 1);
      w1 = span_steps_in(sp, 0, end_whole_tile(first.hi1, BC));
      w2 = span_steps_in(sp, first_whole_tile(last.lo2, BC), end_whole_tile(first.hi2, BC));
    }
  }

  // Mask tile t's scores where some row of the wave does not cover the whole
  // tile (S -> -inf, TS -> 0 outside the row's ranges).  The test is scalar;
  // the masking itself runs on partial tiles only.
  // (t may run one past the last tile on a run's last step; range-list
  // plans clamp it, its result is not used)
  auto tile_whole = [&](int t) {
    if constexpr (TABLE) {
      const int e = __builtin_amdgcn_readfirstlane(ent[t < ntiles ? t : ntiles - 1]);
      return ((e >> (24 + wave)) & 1) != 0;
    } else {
      return in_steps(w1, t) || in_steps(w2, t);
    }
  };
  auto mask_tile = [&](int t, f32x16& S, f32x16& TS) {
    if constexpr (TABLE) {
      const int k0 = tile_at(t < ntiles ? t : ntiles - 1) * BC;
      const int b1 = k0 + 4 * h - rr.lo1, b2 = k0 + 4 * h - rr.lo2;
      uint32_t okm = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = 8 * (i >> 2) + (i & 3);
        if ((unsigned)(b1 + off) < (unsigned)len1 || (unsigned)(b2 + off) < (unsigned)len2) okm |= 1u << i;
      }
      for (int k = 2; k < max_iv; ++k) {  // rows with more than two intervals (rare)
        int lo = 0, len = 0;
        if (k < n_iv) {
          lo = p.tb_iv[2 * (iv_off + k)];
          len = p.tb_iv[2 * (iv_off + k) + 1] - lo;
        }
        const int b3 = k0 + 4 * h - lo;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((unsigned)(b3 + 8 * (i >> 2) + (i & 3)) < (unsigned)len) okm |= 1u << i;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool ok = (okm >> i) & 1u;
        S[i] = ok ? S[i] : -INFINITY;
        TS[i] = ok ? TS[i] : 0.f;
      }
    } else {
      const int k0 = span_tile(sp, t) * BC;
      const int b1 = k0 + 4 * h - rr.lo1, b2 = k0 + 4 * h - rr.lo2;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = 8 * (i >> 2) + (i & 3);
        const bool ok = (unsigned)(b1 + off) < (unsigned)len1 || (unsigned)(b2 + off) < (unsigned)len2;
        S[i] = ok ? S[i] : -INFINITY;
        TS[i] = ok ? TS[i] : 0.f;
      }
    }
  };
  // New reference max of a row after a tile with row max tmx (exp2 units):
  // it moves only when the tile exceeds it by more than 2^8.
  auto next_ref = [&](float ref, float tmx) {
    return tmx > ref + kLazyRescaleLog2 ? fmaxf(ref, tmx) : ref;
  };
  // p~ = exp2(s * sl2 - ref), with nref = -ref (0 for ref = -inf: no allowed
  // key yet, every score of the row is -inf).
  auto neg_ref = [](float ref) { return ref == -INFINITY ? 0.f : -ref; };
  auto exp_elem = [&](float x, float nref) { return __builtin_amdgcn_exp2f(fmaf(x, sl2, nref)); };

  // K and tK fragments of the tile whose scores are formed next; the first
  // two k-steps are read at the end of the previous step (loop-carried).
  u32x4 kf[KS], tkf[KS];
  auto kread = [&](auto mode, const uint16_t* src, int s) {
    const int off = n * D + (((2 * s + h) ^ row_swz<D>(n)) << 3);
    kf[s] = *(const u32x4*)(src + off);
    if constexpr (decltype(mode)::value == kFull) tkf[s] = *(const u32x4*)(src + TILE + off);
  };

  // Scores of two consecutive tiles in vector registers: the current tile's
  // p~ (read by phase 1) and the next one's scores (written by the MFMAs,
  // exponentiated in phase 2); the roles alternate from step to step.
  f32x16 SA, TSA, SB, TSB;

  // Step j of a run over tiles [., t_end).  On entry P holds tile j's p~
  // (already exponentiated against the reference mn) and TS its unscaled
  // score tangents; Sn, TSn receive tile j+1's scores.
  // * top: if some row's reference moved (mn != m), rescale l, r and the
  //   accumulators to mn (rare after the first tile);
  // * phase 1 (score MFMAs of tile j+1): p~ ts', the bf16 packs and the sums
  //   l, r of tile j;
  // * phase 2 (P.V MFMAs of tile j): tile j+1's element mask (partial tiles
  //   only), row max, new reference and exponentials, in place in Sn.
  // The exponentials thus run under the P.V MFMAs and the rest of the
  // softmax under the score MFMAs, which balances the vector work of the
  // two phases.
  // Ring use: tile t sits in stage (t - run start) % 4; step j reads K of
  // tile j+1 and V of tile j, and issues the DMA of tile j+3 into the stage
  // of tile j-1, freed by the previous step's barrier.  The barrier sits in
  // phase 2, right after the last read of tile j's stage; before it each wave
  // waits for its share of tile j+2, which the next step's first K reads
  // (issued right after the barrier) need.  The last P.V MFMAs and the next
  // step's top run while the waves meet.
  // Scheduling unit: one MFMA followed by a share of vector / LDS / DMA work,
  // fenced by sched_barrier on both sides of the MFMA, so that each MFMA's
  // execution covers its own share and no vector work piles up behind
  // back-to-back MFMAs (with one wave per SIMD nothing else fills the matrix
  // unit).
  auto step = [&](auto mode, auto st, int j, int t_end, f32x16& P, f32x16& TS, f32x16& Sn, f32x16& TSn) {
    constexpr int MODE = decltype(mode)::value;
    constexpr bool HAS_TS = MODE != kPrimal;  // score tangents (tq != 0)
    constexpr bool HAS_TKV = MODE == kFull;   // key tangents (tk, tv != 0)
    constexpr int ST = decltype(st)::value;
    using NX = std::integral_constant<int, (ST + 1) % STAGES>;
    using N2 = std::integral_constant<int, (ST + 2) % STAGES>;
    using AH = std::integral_constant<int, (ST + 3) % STAGES>;
    constexpr int LPTM = HAS_TKV ? 4 * LOADS : 2 * LOADS;

    // Rare after the first tile.
    if (__builtin_expect(__any(mn != m), 0)) {
      const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m - mn);
      // rows whose reference moved: the score-tangent shift moves by dc to the
      // p~-weighted mean of this tile's ts' (TS holds ts' - c); others keep it
      float dc = 0.f;
      if constexpr (HAS_TS) {
        float sp = 0.f, spt = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          sp += P[i];
          spt = fmaf(P[i], TS[i], spt);
        }
        sp = pair_sum(sp);
        spt = pair_sum(spt);
        dc = (mn != m && sp > 0.f) ? spt / sp : 0.f;
        c_ts += dc;
        r -= dc * l;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          TS[i] -= dc;
          negc[i] = -c_ts;
        }
        opaque(negc);
      }
      m = mn;
      l *= alpha;
      r *= alpha;
      acc_hazard_wait();
#pragma unroll
      for (int c = 0; c < DC; ++c) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float ao = acc_read(accO[c][i]);
          accO[c][i] = acc_write(ao * alpha);
          if constexpr (HAS_TKV) accV[c][i] = acc_write(acc_read(accV[c][i]) * alpha);
          if constexpr (HAS_TS) accS[c][i] = acc_write(fmaf(-dc, ao, acc_read(accS[c][i])) * alpha);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // range-list plans: the tile of this step's DMA and whether tile j+1 is
    // whole, from the entries the previous step read
    int dma_tile = 0;
    bool next_whole = false;
    if constexpr (TABLE) {
      dma_tile = __builtin_amdgcn_readfirstlane(pf_dma) & 0xffffff;
      next_whole = ((__builtin_amdgcn_readfirstlane(pf_next) >> (24 + wave)) & 1) != 0;
    }

    const uint16_t* nx = stage(NX{});  // on the last tile a stale stage; unused
    const uint16_t* cur = stage(st);
    float wv[16];
    u32x4 PK[2], W[2];
    u32x4 vfr[NG], tvfr[NG];
    // transposed fragment of group gidx from tensor plane `plane` of tile j's
    // stage (kV: V, 3: tV)
    auto tr_frag = [&](int plane, int gidx) {
      const int c2 = gidx / DC, c = gidx % DC;
      const int col = 32 * c + tr_col;
      const int k1 = 16 * c2 + tr_key, k2 = k1 + 8;
      const int o1 = k1 * D + (((col >> 3) ^ row_swz<D>(k1)) << 3) + (col & 7);
      const int o2 = k2 * D + (((col >> 3) ^ row_swz<D>(k2)) << 3) + (col & 7);
      const u32x2 a = read_tr16(cur + plane * TILE + o1), b = read_tr16(cur + plane * TILE + o2);
      return u32x4{a[0], a[1], b[0], b[1]};
    };
    auto vread = [&](int gidx) {
      vfr[gidx] = tr_frag(kV, gidx);
      if constexpr (HAS_TKV) tvfr[gidx] = tr_frag(3, gidx);
    };
    // pieces of tile j's softmax back half, per element pair jj, jj+1
    auto w_mul = [&](int jj) {
      wv[jj] = P[jj] * TS[jj];
      wv[jj + 1] = P[jj + 1] * TS[jj + 1];
      pin(wv[jj]);
      pin(wv[jj + 1]);
    };
    auto pack_p = [&](int jj) {
      PK[jj >> 3][(jj & 7) >> 1] = pack_bf16(P[jj], P[jj + 1]);
      l += P[jj] + P[jj + 1];
      pin(PK[jj >> 3][(jj & 7) >> 1]);
      pin(l);
    };
    auto pack_w = [&](int jj) {
      W[jj >> 3][(jj & 7) >> 1] = pack_bf16(wv[jj], wv[jj + 1]);
      r += wv[jj] + wv[jj + 1];
      pin(W[jj >> 3][(jj & 7) >> 1]);
      pin(r);
    };
    auto dma = [&](int s) {  // this k-step's share of tile j+3's DMA
#pragma unroll
      for (int q = s * LPTM / KS; q < (s + 1) * LPTM / KS; ++q)
        issue_part(mode, stage(AH{}), j + 3, q, t_end, dma_tile);
    };

    // phase 1: scores of tile j+1 under the back half of tile j's softmax.
    // Per k-step, kFull: TS += k.tq | S += k.q | TS += tk.q with
    // p~ ts', DMA | K reads two k-steps ahead, pack p~, l | pack p~ ts', r;
    // kCleanKeys: TS += k.tq | S += k.q; kPrimal: S += k.q.  The DMA share
    // goes to the lightest slot: next to the fragment reads and the p~ pack
    // it cost 1.3 % of the launch (alternated kernel traces).
    constexpr int PAIRS_PER_STEP = 8 / KS;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int jj0 = 2 * s * PAIRS_PER_STEP;
      if constexpr (HAS_TS) {
        if (s == 0) mfma_v_init_ba(TSn, kf[s], tqf[s], negc);
        else mfma_v_acc_ba(TSn, kf[s], tqf[s]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < PAIRS_PER_STEP; ++u) w_mul(jj0 + 2 * u);
        if constexpr (!HAS_TKV) {
          if (s + 2 < KS) kread(mode, nx, s + 2);
        }
        dma(s);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (s == 0) mfma_v_first(Sn, kf[s], qf[s]);
      else mfma_v_acc(Sn, kf[s], qf[s]);
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0) prefetch_entries(j + 1, t_end);
      // (not in the first slot, so that the first MFMA of the k-step never
      // waits for it)
      if constexpr (HAS_TKV || !HAS_TS) {
        if (s + 2 < KS) kread(mode, nx, s + 2);
      }
      if constexpr (!HAS_TS) dma(s);
#pragma unroll
      for (int u = 0; u < PAIRS_PER_STEP; ++u) pack_p(jj0 + 2 * u);
      if constexpr (HAS_TKV) {
        __builtin_amdgcn_sched_barrier(0);
        mfma_v_acc(TSn, tkf[s], qf[s]);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (s == KS - 2) vread(0);
      if (s == KS - 1) vread(1);
      if constexpr (HAS_TS) {
#pragma unroll
        for (int u = 0; u < PAIRS_PER_STEP; ++u) pack_w(jj0 + 2 * u);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // phase 2: P.V of tile j under tile j+1's softmax front half.  Per group
    // NS2 MFMAs (kFull: p~.tv, p~.v, (p~ ts').v; kCleanKeys: the last two;
    // kPrimal: p~.v).  Group 0 carries no vector work on Sn (two MFMAs must
    // pass after its last score product); then the mask of a partial tile,
    // the row max over MAX_GROUPS groups, the new reference, and the
    // exponentials spread over all slots of the remaining groups.
    constexpr int NS2 = HAS_TKV ? 3 : HAS_TS ? 2 : 1;
    constexpr int MAX_GROUPS = NG >= 8 ? 2 : 1;
    constexpr int RM_PER_GROUP = NS2 >= 2 ? NS2 - 1 : 1;  // row-max slots per group
    constexpr int MAX_SLOTS = RM_PER_GROUP * MAX_GROUPS;
    constexpr int MAX_PER_SLOT = 16 / MAX_SLOTS;
    constexpr int EXP_SLOTS = NS2 * (NG - 1 - MAX_GROUPS);
    static_assert(MAX_PER_SLOT * MAX_SLOTS == 16 && EXP_SLOTS > 0, "phase-2 split");
    float tmax = -INFINITY, ref = mn, nref = 0.f;
    auto row_max = [&](int slot) {
#pragma unroll
      for (int e = 0; e < MAX_PER_SLOT; ++e) tmax = fmaxf(tmax, Sn[slot * MAX_PER_SLOT + e]);
      pin(tmax);
      if (slot == MAX_SLOTS - 1) {
        ref = next_ref(mn, pair_max(tmax) * sl2);
        nref = neg_ref(ref);
        pin(nref);
      }
    };
    auto exps = [&](int slot) {  // elements k with k * EXP_SLOTS / 16 == slot
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k * EXP_SLOTS / 16 == slot) {
          Sn[k] = exp_elem(Sn[k], nref);
          pin(Sn[k]);
        }
      }
    };
    // the vector / LDS work of slot sl (0 .. NS2-1) of group gidx
    constexpr int UB = (NG - 2) * NS2;  // linear slot of the barrier
    auto slot_work = [&](int gidx, int sl) {
      const int u = gidx * NS2 + sl;
      // (after group 1's first MFMA: two MFMAs past the last score product in every mode)
      if (gidx == 1 && sl == 0 && !(TABLE ? next_whole : tile_whole(j + 1))) mask_tile(j + 1, Sn, TSn);  // rare
      // V fragments two groups ahead; in full mode the tV ones a slot later,
      // which spreads the transposed reads next to the exponentials (0.9 %
      // faster than all four reads in the group's first slot)
      if (gidx + 2 < NG) {
        if (sl == 0) vfr[gidx + 2] = tr_frag(kV, gidx + 2);
        if constexpr (HAS_TKV) {
          if (sl == 1) tvfr[gidx + 2] = tr_frag(3, gidx + 2);
        }
      }
      if (u == UB) {
        // every read of tile j's stage is done; tile j+2 has landed here
        wait_lgkmcnt<0>();
        wait_vmcnt<LPTM>();
        barrier_nofence();
      }
      if (gidx >= 1 && gidx <= MAX_GROUPS) {
        if (NS2 == 1) row_max(gidx - 1);
        else if (sl >= 1) row_max((gidx - 1) * RM_PER_GROUP + sl - 1);
      }
      if (gidx > MAX_GROUPS) exps((gidx - 1 - MAX_GROUPS) * NS2 + sl);
      // first K reads of tile j+2, behind the barrier
      if (u == (UB + 1 < NG * NS2 ? UB + 1 : NG * NS2 - 1)) kread(mode, stage(N2{}), 0);
      if (u == (UB + 2 < NG * NS2 ? UB + 2 : NG * NS2 - 1)) kread(mode, stage(N2{}), 1);
    };
#pragma unroll
    for (int gidx = 0; gidx < NG; ++gidx) {
      const int c2 = gidx / DC, c = gidx % DC;
      int sl = 0;
      if constexpr (HAS_TKV) {
        accV[c] = mfma_bf16(tvfr[gidx], PK[c2], accV[c]);
        __builtin_amdgcn_sched_barrier(0);
        slot_work(gidx, sl++);
        __builtin_amdgcn_sched_barrier(0);
      }
      accO[c] = mfma_bf16(vfr[gidx], PK[c2], accO[c]);
      __builtin_amdgcn_sched_barrier(0);
      slot_work(gidx, sl++);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (HAS_TS) {
        accS[c] = mfma_bf16(vfr[gidx], W[c2], accS[c]);
        __builtin_amdgcn_sched_barrier(0);
        slot_work(gidx, sl++);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mn = ref;
  };

  // First tile of a run: DMA of its first three tiles, its scores, mask, row
  // max, reference and exponentials, and the first K reads of the next tile.
  auto first_tile = [&](auto mode, int t_begin, int t_end) {
    constexpr int MODE = decltype(mode)::value;
    issue(mode, ring0, t_begin, t_end);
    issue(mode, ring1, t_begin + 1, t_end);
    issue(mode, ring2, t_begin + 2, t_end);
    if constexpr (MODE == kFull) wait_vmcnt<4 * LOADS>();  // first two tiles
    else wait_vmcnt<2 * LOADS>();
    barrier_nofence();
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kread(mode, ring0, s);
      if (s == 0) mfma_v_first(SA, kf[s], qf[s]);
      else mfma_v_acc(SA, kf[s], qf[s]);
      if constexpr (MODE != kPrimal) {
        if (s == 0) mfma_v_init_ba(TSA, kf[s], tqf[s], negc);
        else mfma_v_acc_ba(TSA, kf[s], tqf[s]);
      }
      if constexpr (MODE == kFull) mfma_v_acc(TSA, tkf[s], qf[s]);
    }
    // fenced: the compiler would otherwise move the reads of SA above the wait
    __builtin_amdgcn_sched_barrier(0);
    acc_hazard_wait();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MODE == kPrimal) {
#pragma unroll
      for (int i = 0; i < 16; ++i) TSA[i] = 0.f;
    }
    if (!tile_whole(t_begin)) mask_tile(t_begin, SA, TSA);
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, SA[i]);
    mn = next_ref(mn, pair_max(tmax) * sl2);
    const float nref = neg_ref(mn);
#pragma unroll
    for (int i = 0; i < 16; ++i) SA[i] = exp_elem(SA[i], nref);
    kread(mode, ring1, 0);
    kread(mode, ring1, 1);
  };

  // One pipelined pass over tiles [t_begin, t_end) in one mode; the ring is
  // drained at the end, so runs in different modes can follow each other.
  auto run = [&](auto mode, int t_begin, int t_end) {
    if (t_begin >= t_end) return;
    first_tile(mode, t_begin, t_end);
    prefetch_entries(t_begin, t_end);
    for (int j = t_begin; j < t_end; j += 4) {
      step(mode, I0{}, j, t_end, SA, TSA, SB, TSB);
      if (j + 1 >= t_end) break;
      step(mode, I1{}, j + 1, t_end, SB, TSB, SA, TSA);
      if (j + 2 >= t_end) break;
      step(mode, I2{}, j + 2, t_end, SA, TSA, SB, TSB);
      if (j + 3 >= t_end) break;
      step(mode, I3{}, j + 3, t_end, SB, TSB, SA, TSA);
    }
    // the last step exponentiated scores of no tile: drop that reference
    mn = m;
    // DMAs of tiles past the end, and the last K reads, may be in flight
    wait_vmcnt<0>();
    wait_lgkmcnt<0>();
    barrier_nofence();
  };

  if constexpr (PO || (CTZ && TABLE)) {
    run(MPrimal{}, 0, ntiles);
  } else if constexpr (CTZ) {
    if (primal_only) {
      run(MPrimal{}, 0, ntiles);
    } else {
      run(MCleanKeys{}, 0, n_clean_tiles);  // clean keys of earlier chunks
      run(MFull{}, n_clean_tiles, ntiles);  // the block's own noisy chunks
    }
  } else {
    run(MFull{}, 0, ntiles);
  }

  // ---- epilogue: o = acc_o / l ; to = (acc_tv + scale acc_tsv) / l - (r / l) o
  acc_hazard_wait();
  const float lt = pair_sum(l);
  const float rt = pair_sum(r) * scale;
  if (row_ok) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float rb = rt * inv;
    uint16_t* Og = (uint16_t*)p.o + base + (size_t)row * D;
    uint16_t* tOg = (uint16_t*)p.to + base + (size_t)row * D;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * c + 8 * g4 + 4 * h;
        float o4[4], t4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          o4[e] = acc_read(accO[c][i]) * inv;
          t4[e] = primal_only ? 0.f
                              : fmaf(acc_read(accS[c][i]), scale, acc_read(accV[c][i])) * inv - rb * o4[e];
        }
        u32x2 ov = {pack_bf16(o4[0], o4[1]), pack_bf16(o4[2], o4[3])};
        u32x2 tv = {pack_bf16(t4[0], t4[1]), pack_bf16(t4[2], t4[3])};
        *(u32x2*)(Og + d0) = ov;
        if (!CTZ || p.to != nullptr) *(u32x2*)(tOg + d0) = tv;
      }
    }
    // one explicit fma: every instantiation rounds lse the same way
    if (h == 0 && p.lse != nullptr)
      p.lse[(size_t)bh * N + row] = lt > 0.f ? fmaf(m, kLn2, logf(lt)) : -INFINITY;
  }
}

// fp32 kernel: 32 query rows per workgroup, 8 lanes per row, each lane owning
// D/8 consecutive columns.  Keys are taken one at a time from the same tile
// schedule as the bf16 kernel, with the exact per-row mask; the online
// softmax is the plain FlashAttention-2 recurrence in fp32 (no lazy scaling).
// Range-list plans (TABLE) take each row's key intervals from the table, in
// ascending order.
template <int D, bool TABLE>
__global__ void __launch_bounds__(256) fwd_fp32_kernel(FwdParams p) {
  constexpr int BR = 32, BC = 32, E = D / 8;
  const MaskGeom g = p.g;
  const int N = g.seq_len;
  const int slice = threadIdx.x & 7, lr = threadIdx.x >> 3;
  const int bh = blockIdx.x / p.n_qblocks;
  int qb, r0, r1, ntiles = 0;
  TileSpans sp{0, 0, 0, 0};
  if constexpr (TABLE) {
    qb = p.tb_order[blockIdx.x - bh * p.n_qblocks];
    r0 = qb * BR;
    r1 = r0 + BR < N ? r0 + BR : N;
  } else {
    qb = heavy_first_qblock(g, BR, blockIdx.x - bh * p.n_qblocks, p.ctz != 0);
    qblock_rows(g, BR, qb, &r0, &r1);
    sp = block_tiles(block_ranges(g, r0, r1), BC);
    ntiles = span_count(sp);
  }
  const int row = r0 + lr;
  const bool row_ok = row < r1;
  const Ranges rr = TABLE ? Ranges{0, 0, 0, 0} : (row_ok ? row_ranges(g, row) : Ranges{0, 0, 0, 0});

  const size_t base = (size_t)bh * (size_t)N * D;
  const float* __restrict__ K = (const float*)p.k + base + slice * E;
  const float* __restrict__ V = (const float*)p.v + base + slice * E;
  const float* __restrict__ tK = (const float*)p.tk + base + slice * E;
  const float* __restrict__ tV = (const float*)p.tv + base + slice * E;
  // clean-tangent-zero: clean rows and clean keys carry no tangent and their
  // tangent rows are never read
  const bool ctz = p.ctz != 0;
  const bool row_tangent = !(ctz && (p.primal != 0 || !is_noisy(g, r0)));  // the block's rows are on one side
  float q[E], tq[E], ao[E], at[E];
  const int qrow = row_ok ? row : r0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = ((const float*)p.q)[base + (size_t)qrow * D + slice * E + e];
    tq[e] = 0.f;
    ao[e] = 0.f;
    at[e] = 0.f;
  }
  if (row_tangent) {
#pragma unroll
    for (int e = 0; e < E; ++e) tq[e] = ((const float*)p.tq)[base + (size_t)qrow * D + slice * E + e];
  }
  float m = -INFINITY, l = 0.f, r = 0.f;
  // Score-tangent shift, as in fwd_bf16_kernel: r and at take ts - c, with c
  // the (scaled) ts of the row's first allowed key, which leaves eq. 45's
  // t_o unchanged and keeps a part shared by all of the row's score tangents
  // out of the sums (in fp32 a fixed c suffices).
  float c_ts = 0.f;
  bool c_set = false;  // uniform across the row's 8 lanes
  auto key_step = [&](int j) {
      const float* kj = K + (size_t)j * D;
      const float* tkj = tK + (size_t)j * D;
      const bool key_tangent = !(ctz && (p.primal != 0 || j < g.side_len));
      float s = 0.f, ts = 0.f;
      if (key_tangent) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          s = fmaf(q[e], kj[e], s);
          ts = fmaf(tq[e], kj[e], fmaf(q[e], tkj[e], ts));
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          s = fmaf(q[e], kj[e], s);
          ts = fmaf(tq[e], kj[e], ts);
        }
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        s += __shfl_xor(s, o, 8);
        ts += __shfl_xor(ts, o, 8);
      }
      s *= p.scale;
      ts *= p.scale;
      if (!c_set) {
        c_ts = ts;
        c_set = true;
      }
      ts -= c_ts;
      const float mn = fmaxf(m, s);
      const float alpha = expf(m - mn);
      const float pj = expf(s - mn);
      l = l * alpha + pj;
      r = r * alpha + pj * ts;
      const float* vj = V + (size_t)j * D;
      const float* tvj = tV + (size_t)j * D;
      if (key_tangent) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          ao[e] = ao[e] * alpha + pj * vj[e];
          at[e] = at[e] * alpha + pj * tvj[e] + (pj * ts) * vj[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          ao[e] = ao[e] * alpha + pj * vj[e];
          at[e] = at[e] * alpha + (pj * ts) * vj[e];
        }
      }
      m = mn;
  };
  if constexpr (TABLE) {
    if (row_ok) {  // uniform across the row's 8 lanes
      const int info = p.tb_rows[row];
      const int n_iv = info & 255, iv_off = info >> 8;
      for (int k = 0; k < n_iv; ++k)
        for (int j = p.tb_iv[2 * (iv_off + k)], j1 = p.tb_iv[2 * (iv_off + k) + 1]; j < j1; ++j) key_step(j);
    }
  } else {
    for (int it = 0; it < ntiles; ++it) {
      const int k0 = span_tile(sp, it) * BC;
      const int k1 = k0 + BC < N ? k0 + BC : N;
      for (int j = k0; j < k1; ++j) {
        if (!in_ranges(rr, j)) continue;  // uniform across the row's 8 lanes
        key_step(j);
      }
    }
  }
  if (!row_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float rb = r * inv;
  float* O = (float*)p.o + base + (size_t)row * D + slice * E;
  float* tO = (float*)p.to + base + (size_t)row * D + slice * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float o = ao[e] * inv;
    O[e] = o;
    if (p.to != nullptr) tO[e] = row_tangent ? at[e] * inv - rb * o : 0.f;
  }
  if (slice == 0 && p.lse != nullptr) p.lse[(size_t)bh * N + row] = l > 0.f ? m + logf(l) : -INFINITY;
}

// ---------------------------------------------------------------------------
void block_sizes(int dtype, int head_dim, int* block_q, int* block_k) {
  (void)head_dim;
  if (dtype == kBf16) {
    *block_q = kBf16Waves * 32;
    *block_k = kBf16BlockK;
  } else {
    *block_q = 32;
    *block_k = 32;
  }
}

hipError_t launch_fwd(int dtype, int head_dim, int grid, const FwdParams& p0, hipStream_t stream) {
  const dim3 block(kBf16Waves * 64);
  const bool table = p0.tb_ent != nullptr;
  FwdParams p = p0;
  p.n_tasks = grid;
  // grid of fwd_bf16_kernel, which takes its tasks from the work queues
  const dim3 qgrid((unsigned)queue_grid(grid));
  if (dtype == kBf16 && p.primal && !table) {  // descriptor plans without tangents: the primal-only instance
    if (head_dim == 128) hipLaunchKernelGGL((fwd_bf16_kernel<128, kBf16Waves, true, false, true>), qgrid, block, 0, stream, p);
    else hipLaunchKernelGGL((fwd_bf16_kernel<64, kBf16Waves, true, false, true>), qgrid, block, 0, stream, p);
    return hipGetLastError();
  }
  if (dtype == kBf16 && table && p.primal) {  // range-list plans without tangents
    if (p.tb_max_entries <= kPoMaxTableEntries) {
      if (head_dim == 128) hipLaunchKernelGGL((fwd_bf16_kernel<128, kBf16Waves, true, true, true>), qgrid, block, 0, stream, p);
      else hipLaunchKernelGGL((fwd_bf16_kernel<64, kBf16Waves, true, true, true>), qgrid, block, 0, stream, p);
    } else {
      if (head_dim == 128) hipLaunchKernelGGL((fwd_bf16_kernel<128, kBf16Waves, true, true>), qgrid, block, 0, stream, p);
      else hipLaunchKernelGGL((fwd_bf16_kernel<64, kBf16Waves, true, true>), qgrid, block, 0, stream, p);
    }
    return hipGetLastError();
  }
  if (dtype == kBf16 && p.ctz && !table) {
    // clean-tangent-zero plans: the clean side's blocks (o and lse only) in
    // the primal-only instance at two workgroups per CU, then the noisy
    // side's in the clean-tangent-zero instance; the two launches take the
    // call's work queues one after the other
    FwdParams pc = p, pn = p;
    pc.side = 0;
    pn.side = 1;
    pc.n_qblocks = pn.n_qblocks = p.n_qblocks / 2;
    pc.n_tasks = pn.n_tasks = grid / 2;
    const dim3 hgrid((unsigned)queue_grid(grid / 2));
    if (head_dim == 128) {
      hipLaunchKernelGGL((fwd_bf16_kernel<128, kBf16Waves, true, false, true>), hgrid, block, 0, stream, pc);
      hipLaunchKernelGGL((fwd_bf16_kernel<128, kBf16Waves, true, false>), hgrid, block, 0, stream, pn);
    } else {
      hipLaunchKernelGGL((fwd_bf16_kernel<64, kBf16Waves, true, false, true>), hgrid, block, 0, stream, pc);
      hipLaunchKernelGGL((fwd_bf16_kernel<64, kBf16Waves, true, false>), hgrid, block, 0, stream, pn);
    }
    return hipGetLastError();
  }
  if (dtype == kBf16) {
    if (head_dim == 128) {
      if (table) hipLaunchKernelGGL((fwd_bf16_kernel<128, kBf16Waves, false, true>), qgrid, block, 0, stream, p);
      else hipLaunchKernelGGL((fwd_bf16_kernel<128, kBf16Waves, false, false>), qgrid, block, 0, stream, p);
    } else {
      if (table) hipLaunchKernelGGL((fwd_bf16_kernel<64, kBf16Waves, false, true>), qgrid, block, 0, stream, p);
      else hipLaunchKernelGGL((fwd_bf16_kernel<64, kBf16Waves, false, false>), qgrid, block, 0, stream, p);
    }
  } else {
    if (head_dim == 128) {
      if (table) hipLaunchKernelGGL((fwd_fp32_kernel<128, true>), dim3(grid), dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((fwd_fp32_kernel<128, false>), dim3(grid), dim3(256), 0, stream, p);
    } else {
      if (table) hipLaunchKernelGGL((fwd_fp32_kernel<64, true>), dim3(grid), dim3(256), 0, stream, p);
      else hipLaunchKernelGGL((fwd_fp32_kernel<64, false>), dim3(grid), dim3(256), 0, stream, p);
    }
  }
  return hipGetLastError();
}

}  // namespace attn_jvp
