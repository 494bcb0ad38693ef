// attn_jvp_bwd_kernels.hip -- gfx950 kernels for the backward of block-causal /
// teacher-forcing masked attention: dq, dk, dv from q, k, v, o, lse and dO.
//
// What is computed (Causal-rCM, arXiv 2606.25473, section 3.2.1: the
// FlashAttention-2 based masked attention of the student also runs its
// backward; section 2.3 and section 3.1.1 eq. 8 for the mask): with P the
// masked softmax of the scaled scores, recomputed from the forward's lse,
//   dP = dO V^T,   delta_i = sum_d dO_id O_id  (= sum_j P_ij dP_ij),
//   dS = P o (dP - delta),   dQ = scale dS K,   dK = scale dS^T Q,   dV = P^T dO,
// where masked pairs have P = 0 and hence dS = 0.
//
// Two kernels per call, which accumulate no result through atomics (their
// workgroups take tasks from work queues, but a task's arithmetic does not
// depend on the workgroup that runs it), so every result is a fixed function
// of the inputs:
// * dq kernel: one workgroup per query block with the forward's key-tile
//   schedule; lane = query.  It also writes -delta and -lse log2(e) of its
//   rows to the workspace.  Per 32-key tile: S^T = K Q^T and dP^T - delta =
//   V dO^T - delta (score products in vector-register form, the second one
//   started from -delta instead of 0), P^T = exp2(S^T scale log2(e) -
//   lse log2(e)), dS^T = P^T o (dP^T - delta), then dQ^T += K^T dS^T with K^T
//   from the transposing LDS read of the K tile.  Two versions with the same
//   arithmetic: descriptor plans run bwd_dq2_bf16_kernel, two workgroups per
//   CU; range-list plans, whose tile entries take another 30 KB of LDS, run
//   bwd_dq_bf16_kernel, one workgroup per CU with a cross-tile pipeline.
// * dk/dv kernel: one workgroup per block of 32 NW keys, cut per side like
//   the query blocks, over the 32-row query tiles of the rows that attend to
//   any of its keys (at most two intervals); lane = key.  Per query tile:
//   X = Q K^T and dP = dO V^T, P, dS, then dV^T += dO^T P and dK^T += Q^T dS
//   with dO^T and Q^T from the transposing LDS read; -delta (the start of
//   the dP product) and -lse log2(e) of the tile's rows come from the
//   workspace, staged in LDS with the tile.
// Both follow the forward kernel's structure: 32-row tiles go HBM -> LDS by
// DMA into a 6-stage ring (XOR-swizzled rows, zeros past the end), the score
// products of tile j+1 run under the elementwise work of tile j and the
// output products of tile j under the exponentials of tile j+1, one MFMA per
// scheduling slot; whole tiles outside the key (query) ranges are never
// visited and the element mask runs only on partial tiles.
#include <hip/hip_runtime.h>
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "attn_jvp_launch.h"
#include "kernel_common.h"
#include "mask_index.h"

namespace attn_jvp {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// The LDS ring.  Step j reads tiles j .. j+2 (tile j+2 only after its
// mid-step barrier slot) and issues the DMA of tile j+A into the stage of
// tile j+A-S.  Workgroup barriers sit in every P-th step; the one in step b
// follows each wave's wait for its shares of tiles up to b+P+1, the tiles
// read before the next barrier, and a wait for its own LDS reads, so every
// read of tiles up to b is complete behind it.  Hence
//   A >= P+2: tile b+P+1 was issued at least one step before barrier b;
//   S >= A+P: a stage is refilled only after a barrier behind its last read;
//   S % P == 0: the unrolled steps keep their barrier slots.
// S = 6 stages of 16 KB (the dk/dv kernel's 1 KB more), A = 4, P = 2: one
// barrier per two steps.
constexpr int kBwdStages = 6;
constexpr int kBwdAhead = 4;
constexpr int kBwdBarrierEvery = 2;
static_assert(kBwdAhead >= kBwdBarrierEvery + 2 && kBwdStages >= kBwdAhead + kBwdBarrierEvery &&
                  kBwdStages % kBwdBarrierEvery == 0 && kBwdStages % 2 == 0,
              "ring depth, prefetch distance and barrier period");

template <int V>
using IC = std::integral_constant<int, V>;

// f(IC<S>{}) for S = 0, 1, .. N-1 while it returns true; false if one did.
template <int S, int N, class F>
__device__ __forceinline__ bool unrolled_while(F&& f) {
  if constexpr (S == N) return true;
  else return f(IC<S>{}) && unrolled_while<S + 1, N>(f);
}

// Per-lane addressing shared by the two bf16 kernels.
template <int D, int NW>
struct TileGeom {
  static constexpr int ROWS = 32;                     // rows per streamed tile
  static constexpr int KS = D / 16;                   // k-steps of a score product
  static constexpr int DC = D / 32;                   // 32-wide column blocks of an output
  static constexpr int NG = 2 * DC;                   // output products per tile and accumulator
  static constexpr int CPR = D / 8;                   // 16-byte groups per row
  static constexpr int TILE = ROWS * D;               // elements per tensor per stage
  static constexpr int LOADS = TILE * 2 / 1024 / NW;  // 1 KB DMA loads per wave per tensor
  static_assert(LOADS * NW * 1024 == TILE * 2, "DMA split");

  // DMA source offset of this lane for its i-th 1 KB block: lane L of block
  // `blk` fills LDS group (row, pc) and fetches global group pc ^ swz(row).
  __device__ static int dma_voff(int wave, int lane, int i) {
    const int blk = wave * LOADS + i;
    const int rw = blk * (64 / CPR) + lane / CPR;
    return (rw * D + (((lane % CPR) ^ row_swz<D>(rw)) << 3)) * 2;
  }
  // Fragment of row n (16 bytes at k-step s, half h) of a swizzled tile: the
  // A operand of a product contracting over d.
  __device__ static u32x4 row_frag(const uint16_t* tile, int n, int h, int s) {
    return *(const u32x4*)(tile + n * D + (((2 * s + h) ^ row_swz<D>(n)) << 3));
  }
  // Transposed fragment for output group gidx (16-row half c2, 32-column
  // block c): the A operand of a product contracting over the tile's rows,
  // rows {4h .. 4h+3, 8+4h .. 8+4h+3} of the half, matching the order in
  // which a score accumulator holds them.
  __device__ static u32x4 tr_frag(const uint16_t* tile, int lane, int gidx) {
    const int h = lane >> 5;
    const int tr_row = 4 * h + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    const int c2 = gidx / DC, c = gidx % DC;
    const int col = 32 * c + tr_col;
    const int k1 = 16 * c2 + tr_row, k2 = k1 + 8;
    const int o1 = k1 * D + (((col >> 3) ^ row_swz<D>(k1)) << 3) + (col & 7);
    const int o2 = k2 * D + (((col >> 3) ^ row_swz<D>(k2)) << 3) + (col & 7);
    const u32x2 a = read_tr16(tile + o1), b = read_tr16(tile + o2);
    return u32x4{a[0], a[1], b[0], b[1]};
  }
};

// Element i of a score accumulator of lane (n, h) belongs to tile row
// 8 (i / 4) + 4 h + i % 4; mask the elements whose row is outside the lane's
// ranges r (scores -> -inf).
__device__ __forceinline__ void mask_scores(f32x16& S, int x0, int h, const Ranges& r) {
  const int len1 = r.hi1 - r.lo1, len2 = r.hi2 - r.lo2;
  const int b1 = x0 + 4 * h - r.lo1, b2 = x0 + 4 * h - r.lo2;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int off = 8 * (i >> 2) + (i & 3);
    const bool ok = (unsigned)(b1 + off) < (unsigned)len1 || (unsigned)(b2 + off) < (unsigned)len2;
    S[i] = ok ? S[i] : -INFINITY;
  }
}

// Range-list plans: an item's (a query row's, or a key's) intervals on the
// other axis, from the table's info word ((first interval << 8) | count) and
// interval list.  The first two are held as Ranges; further ones are read in
// the mask branch.  Items in no group, and items past the end, have none.
struct ItemIntervals {
  Ranges r;
  int n_iv, off;
};

__device__ __forceinline__ ItemIntervals item_intervals(const int32_t* info, const int32_t* iv, int item, bool ok) {
  ItemIntervals it{{0, 0, 0, 0}, 0, 0};
  if (ok) {
    const int w = info[item];
    it.n_iv = w & 255;
    it.off = w >> 8;
    if (it.n_iv >= 1) {
      it.r.lo1 = iv[2 * it.off];
      it.r.hi1 = iv[2 * it.off + 1];
    }
    if (it.n_iv >= 2) {
      it.r.lo2 = iv[2 * it.off + 2];
      it.r.hi2 = iv[2 * it.off + 3];
    }
  }
  return it;
}

// The most intervals any lane's item has (wave-uniform).
__device__ __forceinline__ int wave_max_intervals(int n_iv) {
  int m = n_iv;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o));
  return __builtin_amdgcn_readfirstlane(m);
}

// mask_scores with all of the item's intervals (max_iv: wave maximum).
__device__ __forceinline__ void mask_scores_iv(f32x16& S, int x0, int h, const ItemIntervals& it, int max_iv,
                                               const int32_t* iv) {
  const int len1 = it.r.hi1 - it.r.lo1, len2 = it.r.hi2 - it.r.lo2;
  const int b1 = x0 + 4 * h - it.r.lo1, b2 = x0 + 4 * h - it.r.lo2;
  uint32_t okm = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int off = 8 * (i >> 2) + (i & 3);
    if ((unsigned)(b1 + off) < (unsigned)len1 || (unsigned)(b2 + off) < (unsigned)len2) okm |= 1u << i;
  }
  for (int k = 2; k < max_iv; ++k) {  // items with more than two intervals (rare)
    int lo = 0, len = 0;
    if (k < it.n_iv) {
      lo = iv[2 * (it.off + k)];
      len = iv[2 * (it.off + k) + 1] - lo;
    }
    const int b3 = x0 + 4 * h - lo;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int off = 8 * (i >> 2) + (i & 3);
      if ((unsigned)(b3 + off) < (unsigned)len) okm |= 1u << i;
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) S[i] = ((okm >> i) & 1) ? S[i] : -INFINITY;
}

}  // namespace

// ---------------------------------------------------------------------------
// dq kernel (bf16) of range-list plans, one workgroup per CU with a
// cross-tile pipeline (the two-workgroup kernel below, given the tile
// entries of a table, was not faster on these plans).  One wave = 32 query
// rows; the K and V tiles of 32 keys stream through the LDS
// ring; the forward's block order, tile lists and row intervals come from
// the table.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 1) bwd_dq_bf16_kernel(BwdParams p) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  using TG = TileGeom<D, NW>;
  constexpr int BC = TG::ROWS;  // keys per tile
  constexpr int BR = NW * 32;   // query rows per block
  constexpr int KS = TG::KS, DC = TG::DC, NG = TG::NG, TILE = TG::TILE, LOADS = TG::LOADS;
  constexpr int LPT = 2 * LOADS;  // DMA instructions per wave and tile: K, V
  constexpr int STAGES = kBwdStages, AHEAD = kBwdAhead, BAR = kBwdBarrierEvery;

  __shared__ __attribute__((aligned(1024))) uint16_t ring[STAGES][2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;

  const MaskGeom g = p.g;
  const int N = g.seq_len;
  // Workgroups take the table's heavy-first order in XCD groups of
  // kFwdXcdGroup from the per-XCD work queues, as the forward does.
  const int n_tasks = p.n_slices * p.n_qblocks;
  const int pos = workgroup_task(p.queues, n_tasks);
  if (pos < 0) return;  // the queues were empty: no task for this workgroup
  const int task = launch_task(pos, n_tasks, p.n_qblocks, kFwdXcdGroup, kSmallAcross);
  const int bh = task / p.n_qblocks;
  const int qb = p.tb_order[task - bh * p.n_qblocks];
  const int r0 = qb * BR;
  const int r1 = r0 + BR < N ? r0 + BR : N;
  const int e0 = p.tb_blk[qb];
  const int ntiles = p.tb_blk[qb + 1] - e0;
  // the block's tile entries (tile | whole bit of wave w << (24 + w)),
  // staged in LDS for the whole task
  __shared__ int32_t ent[kMaxTableEntries];
  for (int i = tid; i < ntiles; i += NW * 64) ent[i] = p.tb_ent[e0 + i];
  __syncthreads();
  auto entry = [&](int t) { return __builtin_amdgcn_readfirstlane(ent[t < ntiles ? t : ntiles - 1]); };
  // The raw entries a step needs (its DMA tile's and the next tile's) are
  // read from LDS one step ahead, so that the step's top takes them without
  // waiting for an LDS read.
  int pf_dma = 0, pf_next = 0;
  auto prefetch_entries = [&](int j) {
    pf_dma = ent[j + kBwdAhead < ntiles ? j + kBwdAhead : ntiles - 1];
    pf_next = ent[j + 1 < ntiles ? j + 1 : ntiles - 1];
  };

  const size_t base = (size_t)bh * (size_t)N * D;
  const int slice_bytes = N * D * 2;
  const i32x4_t desc_k = make_desc((const uint16_t*)p.k + base, slice_bytes);
  const i32x4_t desc_v = make_desc((const uint16_t*)p.v + base, slice_bytes);

  const int row = r0 + wave * 32 + n;
  const bool row_ok = row < r1;
  const ItemIntervals riv = item_intervals(p.tb_rows, p.tb_iv, row, row_ok);
  const int max_iv = wave_max_intervals(riv.n_iv);

  // Q and dO fragments (B operands) stay in accumulation registers; -delta
  // = -dO . O and -lse log2(e) of the row go to the workspace for the dk/dv
  // kernel.
  u32x4 qf[KS], dof[KS];
  float ndelta, nl;
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t*)p.q + base, slice_bytes);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const uint16_t*)p.dout + base, slice_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((const uint16_t*)p.o + base, slice_bytes);
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int off = (row * D + 16 * s + 8 * h) * 2;
      qf[s] = load16(rq, off);
      dof[s] = load16(rdo, off);
      const u32x4 of = load16(ro, off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = fmaf(bf16_lo(dof[s][e]), bf16_lo(of[e]), part);
        part = fmaf(bf16_hi(dof[s][e]), bf16_hi(of[e]), part);
      }
    }
    ndelta = -pair_sum(part);
    const float lse = row_ok ? p.lse[(size_t)bh * N + row] : 0.f;
    nl = -lse * kLog2e;
    // range-list plans: a row in no group has lse = -inf and no allowed key.
    // The most negative finite float keeps its (masked) P at 0, where +inf
    // would give exp2(-inf + inf); finite, because the dk/dv kernel's delta
    // lanes read this plane past the last row, where 0 * -inf would be NaN.
    nl = lse == -INFINITY ? -FLT_MAX : nl;
    if (row_ok) p.ws[(size_t)bh * 2 * N + (size_t)h * N + row] = h ? nl : ndelta;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      keep_in_acc(qf[s]);
      keep_in_acc(dof[s]);
    }
  }
  f32x16 negd;  // start of the dP^T product: every element of the lane is its row's
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = ndelta;

  auto stage = [&](auto st) -> uint16_t* { return ring[decltype(st)::value]; };
  int dma_voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) dma_voff[i] = TG::dma_voff(wave, lane, i);
  // The q-th DMA instruction of tile `tile` (the step's tile from the table,
  // read once per step; past the last tile that tile again, into a stage
  // nothing reads, so every step issues the same number).
  auto issue_part = [&](uint16_t* dst, int q, int tile) {
    const int soff = tile * BC * D * 2;
    const int i = q >> 1, tt = q & 1;
    load16_lds_asm(tt ? desc_v : desc_k, dst + tt * TILE + (wave * LOADS + i) * 512, dma_voff[i], soff);
  };
  auto issue = [&](uint16_t* dst, int t) {
    const int tile = entry(t) & 0xffffff;
#pragma unroll
    for (int q = 0; q < LPT; ++q) issue_part(dst, q, tile);
  };

  f32x16 accQ[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) accQ[c][i] = 0.f;
  }
  const float sl2 = p.score_log2;

  // A tile every valid row of the wave sees whole has this wave's bit set in
  // its entry; the others take the partial-tile mask of scores of the tile
  // at key k0.
  auto mask_tile = [&](f32x16& S, int k0) { mask_scores_iv(S, k0, h, riv, max_iv, p.tb_iv); };
  auto exp_elem = [&](float x) { return __builtin_amdgcn_exp2f(fmaf(x, sl2, nl)); };

  u32x4 kf[KS], vf[KS];
  auto kvread = [&](const uint16_t* src, int s) {
    kf[s] = TG::row_frag(src, n, h, s);
    vf[s] = TG::row_frag(src + TILE, n, h, s);
  };

  // S^T and dP^T of two consecutive tiles (vector registers): the current
  // tile's P (exponentiated) and dP, the next tile's scores being formed.
  f32x16 SA, DA, SB, DB;

  // Step j.  Phase 1: S^T, dP^T of tile j+1 under dS of tile j and its
  // packs, and all transposed K reads of tile j; each k-step's DMA share
  // follows its dP^T MFMA, next to the transposed reads, so that it does not
  // pile onto the fragment reads and packs after the score MFMA.  Phase 2: dQ^T += K^T dS^T
  // of tile j under the mask (partial tiles) and exponentials of tile j+1.
  // (Half of the exponentials moved to the next phase 1 was 0.9 % slower.)
  // Ring: step j reads K, V of tile j+1 and K^T of tile j, and issues the DMA
  // of tile j+AHEAD; phase 2 opens with the barrier slot (every read of tile
  // j's stage is then issued), after which come the first K, V reads of tile
  // j+2, seven MFMAs ahead of their use.
  auto step = [&](auto st, int j, f32x16& P, f32x16& DP, f32x16& Sn, f32x16& DPn) {
    constexpr int ST = decltype(st)::value;
    using NX = IC<(ST + 1) % STAGES>;
    using N2 = IC<(ST + 2) % STAGES>;
    using AH = IC<(ST + AHEAD) % STAGES>;
#pragma unroll
    for (int c = 0; c < DC; ++c) keep_in_acc(accQ[c]);
    const uint16_t* nx = stage(NX{});
    const uint16_t* cur = stage(st);
    u32x4 DS[2];
    u32x4 ktf[NG];
    auto ds_pair = [&](int jj) {  // DP holds dP - delta
      DS[jj >> 3][(jj & 7) >> 1] = pack_bf16(P[jj] * DP[jj], P[jj + 1] * DP[jj + 1]);
      pin(DS[jj >> 3][(jj & 7) >> 1]);
    };
    // this step's DMA tile and the next tile's entry, prefetched by the
    // previous step
    const int dma_tile = __builtin_amdgcn_readfirstlane(pf_dma) & 0xffffff;
    const int next_e = __builtin_amdgcn_readfirstlane(pf_next);
    auto dma = [&](int s) {
#pragma unroll
      for (int q = s * LPT / KS; q < (s + 1) * LPT / KS; ++q) issue_part(stage(AH{}), q, dma_tile);
    };

    constexpr int PAIRS = 8 / KS;  // dS element pairs per k-step
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s == 0) mfma_v_first_ba(Sn, kf[s], qf[s]);
      else mfma_v_acc_ba(Sn, kf[s], qf[s]);
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0) prefetch_entries(j + 1);
      if (s + 2 < KS) kvread(nx, s + 2);
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) ds_pair(2 * (s * PAIRS + u));
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0) mfma_v_init_ba(DPn, vf[s], dof[s], negd);
      else mfma_v_acc_ba(DPn, vf[s], dof[s]);
      __builtin_amdgcn_sched_barrier(0);
      dma(s);
#pragma unroll
      for (int gq = 0; gq < NG; ++gq)
        if (gq * KS / NG == s) ktf[gq] = TG::tr_frag(cur, lane, gq);
      __builtin_amdgcn_sched_barrier(0);
    }

    // phase 2 (the last score product is two MFMAs back at the first slot)
#pragma unroll
    for (int gidx = 0; gidx < NG; ++gidx) {
      const int c2 = gidx / DC, c = gidx % DC;
      accQ[c] = mfma_bf16(ktf[gidx], DS[c2], accQ[c]);
      __builtin_amdgcn_sched_barrier(0);
      if (gidx == 0 && !((next_e >> (24 + wave)) & 1)) mask_tile(Sn, (next_e & 0xffffff) * BC);  // rare
      if (gidx == 0 && ST % BAR == 0) {
        // tiles up to j+BAR+1 have landed; reads up to tile j are complete
        wait_lgkmcnt<0>();
        wait_vmcnt<(AHEAD - BAR - 1) * LPT>();
        barrier_nofence();
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k * NG / 16 == gidx) {
          Sn[k] = exp_elem(Sn[k]);
          pin(Sn[k]);
        }
      }
      if (gidx == 1) kvread(stage(N2{}), 0);
      if (gidx == 2) kvread(stage(N2{}), 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto first_tile = [&](int t_begin) {
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) issue(ring[i], t_begin + i);
    wait_vmcnt<(AHEAD - 2) * LPT>();  // first two tiles
    barrier_nofence();
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kvread(ring[0], s);
      if (s == 0) {
        mfma_v_first_ba(SA, kf[s], qf[s]);
        mfma_v_init_ba(DA, vf[s], dof[s], negd);
      } else {
        mfma_v_acc_ba(SA, kf[s], qf[s]);
        mfma_v_acc_ba(DA, vf[s], dof[s]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    acc_hazard_wait();
    __builtin_amdgcn_sched_barrier(0);
    const int e = entry(t_begin);
    if (!((e >> (24 + wave)) & 1)) mask_tile(SA, (e & 0xffffff) * BC);
#pragma unroll
    for (int i = 0; i < 16; ++i) SA[i] = exp_elem(SA[i]);
    kvread(ring[1], 0);
    kvread(ring[1], 1);
  };

  if (ntiles > 0) {
    first_tile(0);
    prefetch_entries(0);
    for (int j = 0; j < ntiles; j += STAGES) {
      const bool more = unrolled_while<0, STAGES>([&](auto st) {
        constexpr int S = decltype(st)::value;
        if constexpr (S % 2 == 0) step(st, j + S, SA, DA, SB, DB);
        else step(st, j + S, SB, DB, SA, DA);
        return j + S + 1 < ntiles;
      });
      if (!more) break;
    }
    // DMAs past the last tile and the last K, V reads may be in flight
    wait_vmcnt<0>();
    wait_lgkmcnt<0>();
    barrier_nofence();
  }

  // ---- epilogue: dq = scale acc
  acc_hazard_wait();
  if (row_ok) {
    const float scale = p.scale;
    uint16_t* Qg = (uint16_t*)p.dq + base + (size_t)row * D;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * c + 8 * g4 + 4 * h;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc_read(accQ[c][4 * g4 + e]) * scale;
        *(u32x2*)(Qg + d0) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dq kernel (bf16) at two workgroups per CU.  The work, the tile order and
// the order of every sum are those of bwd_dq_bf16_kernel above, so its dq is
// bit-identical; the schedule differs.  With at most 256 registers per lane
// and a 4-stage ring (64 KB), two workgroups share a CU and each SIMD holds
// two waves, so the SIMD issues one wave's MFMAs while the other wave runs
// its exponentials, waits or LDS reads: the hardware interleaving takes the
// place of the cross-tile software pipeline above, which needs 328 registers.
// Step j: barrier (tile j has landed, every read of tile j-1 is complete),
// DMA of tile j+3 into tile j-1's stage under S^T and dP^T of tile j, then
// the mask, exponentials and dS^T, then dQ^T += K^T dS^T.  A wave raises
// its issue priority over its two MFMA phases, so that the SIMD keeps
// feeding the matrix core from the wave that has products ready while the
// other one runs its exponentials.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 2) bwd_dq2_bf16_kernel(BwdParams p) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  using TG = TileGeom<D, NW>;
  constexpr int BC = TG::ROWS;  // keys per tile
  constexpr int BR = NW * 32;   // query rows per block
  constexpr int KS = TG::KS, DC = TG::DC, NG = TG::NG, TILE = TG::TILE, LOADS = TG::LOADS;
  constexpr int LPT = 2 * LOADS;  // DMA instructions per wave and tile: K, V
  // Ring: tile t in stage t % STAGES, issued AHEAD steps before its use.  The
  // barrier at the top of step j follows each wave's wait for its share of
  // tile j and the MFMAs that consumed all its reads of tile j-1, whose
  // stage the step then refills with tile j + AHEAD.
  constexpr int STAGES = 4, AHEAD = 3;
  static_assert(AHEAD == STAGES - 1, "the refilled stage is the previous tile's");

  __shared__ __attribute__((aligned(1024))) uint16_t ring[STAGES][2 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;

  const MaskGeom g = p.g;
  const int N = g.seq_len;
  const int n_tasks = p.n_slices * p.n_qblocks;
  const int pos = workgroup_task(p.queues, n_tasks);
  if (pos < 0) return;  // the queues were empty: no task for this workgroup
  const int task = launch_task(pos, n_tasks, p.n_qblocks, kFwdXcdGroup, g.tf ? kSmallRankGroups : kSmallAcross);
  const int bh = task / p.n_qblocks;
  int r0, r1;
  const int qb = heavy_first_qblock(g, BR, task - bh * p.n_qblocks);
  qblock_rows(g, BR, qb, &r0, &r1);
  const TileSpans sp = block_tiles(block_ranges(g, r0, r1), BC);
  const int ntiles = span_count(sp);

  const size_t base = (size_t)bh * (size_t)N * D;
  const int slice_bytes = N * D * 2;
  const i32x4_t desc_k = make_desc((const uint16_t*)p.k + base, slice_bytes);
  const i32x4_t desc_v = make_desc((const uint16_t*)p.v + base, slice_bytes);

  const int row = r0 + wave * 32 + n;
  const bool row_ok = row < r1;
  const Ranges rr = row_ok ? row_ranges(g, row) : Ranges{0, 0, 0, 0};

  u32x4 qf[KS], dof[KS];
  float ndelta, nl;
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t*)p.q + base, slice_bytes);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc((const uint16_t*)p.dout + base, slice_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc((const uint16_t*)p.o + base, slice_bytes);
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int off = (row * D + 16 * s + 8 * h) * 2;
      qf[s] = load16(rq, off);
      dof[s] = load16(rdo, off);
      const u32x4 of = load16(ro, off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part = fmaf(bf16_lo(dof[s][e]), bf16_lo(of[e]), part);
        part = fmaf(bf16_hi(dof[s][e]), bf16_hi(of[e]), part);
      }
    }
    ndelta = -pair_sum(part);
    const float lse = row_ok ? p.lse[(size_t)bh * N + row] : 0.f;
    nl = -lse * kLog2e;
    if (row_ok) p.ws[(size_t)bh * 2 * N + (size_t)h * N + row] = h ? nl : ndelta;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      keep_in_acc(qf[s]);
      keep_in_acc(dof[s]);
    }
  }
  f32x16 negd;
#pragma unroll
  for (int i = 0; i < 16; ++i) negd[i] = ndelta;

  auto stage = [&](auto st) -> uint16_t* { return ring[decltype(st)::value]; };
  int dma_voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) dma_voff[i] = TG::dma_voff(wave, lane, i);
  // LDS byte address of this wave's first DMA block in stage 0 (scalar)
  const int lds_wave = __builtin_amdgcn_readfirstlane(lds_addr(&ring[0][0])) + wave * LOADS * 1024;
  auto issue_part = [&](int stg, int t, int q, int t_end) {
    const int tile = span_tile(sp, t < t_end ? t : t_end - 1);
    const int soff = tile * BC * D * 2;
    const int i = q >> 1, tt = q & 1;
    load16_lds_at(tt ? desc_v : desc_k, lds_wave + stg * 4 * TILE + tt * 2 * TILE + i * 1024, dma_voff[i], soff);
  };

  f32x16 accQ[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) accQ[c][i] = 0.f;
  }
  const float sl2 = p.score_log2;

  Ranges wfirst{0, 0, 0, 0}, wlast{0, 0, 0, 0};
  {
    const int wa = r0 + wave * 32;
    const int wb = wa + 32 < r1 ? wa + 32 : r1;
    if (wa < wb) {
      wfirst = row_ranges(g, wa);
      wlast = row_ranges(g, wb - 1);
    }
  }
  const StepRange w1 = span_steps_in(sp, first_whole_tile(wlast.lo1, BC), end_whole_tile(wfirst.hi1, BC));
  const StepRange w2 = span_steps_in(sp, first_whole_tile(wlast.lo2, BC), end_whole_tile(wfirst.hi2, BC));
  auto tile_whole = [&](int t) { return in_steps(w1, t) || in_steps(w2, t); };

  auto step = [&](auto st, int j) {
    constexpr int ST = decltype(st)::value;
    using AH = IC<(ST + AHEAD) % STAGES>;
#pragma unroll
    for (int c = 0; c < DC; ++c) keep_in_acc(accQ[c]);
    // this wave's share of tile j has landed (tiles j+1, j+2 may be in
    // flight); behind the barrier every wave's share has, and every read of
    // tile j-1, whose stage is refilled below, is complete
    wait_vmcnt<(AHEAD - 1) * LPT>();
    barrier_nofence();
    const uint16_t* cur = stage(st);
    u32x4 kf[KS], vf[KS];
    auto kvread = [&](int s) {
      kf[s] = TG::row_frag(cur, n, h, s);
      vf[s] = TG::row_frag(cur + TILE, n, h, s);
    };
    f32x16 S, DP;
    kvread(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s + 1 < KS) kvread(s + 1);
      if (s == 0) mfma_v_first_ba(S, kf[s], qf[s]);
      else mfma_v_acc_ba(S, kf[s], qf[s]);
      if (s == 0) mfma_v_init_ba(DP, vf[s], dof[s], negd);
      else mfma_v_acc_ba(DP, vf[s], dof[s]);
#pragma unroll
      for (int q = s * LPT / KS; q < (s + 1) * LPT / KS; ++q) issue_part(AH::value, j + AHEAD, q, ntiles);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
    u32x4 ktf[NG];
    ktf[0] = TG::tr_frag(cur, lane, 0);
    __builtin_amdgcn_sched_barrier(0);
    acc_hazard_wait();
    __builtin_amdgcn_sched_barrier(0);
    if (!tile_whole(j)) mask_scores(S, span_tile(sp, j) * BC, h, rr);  // partial tiles only
    u32x4 DS[2];
#pragma unroll
    for (int jj = 0; jj < 16; jj += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(S[jj], sl2, nl));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(S[jj + 1], sl2, nl));
      DS[jj >> 3][(jj & 7) >> 1] = pack_bf16(p0 * DP[jj], p1 * DP[jj + 1]);
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int gidx = 0; gidx < NG; ++gidx) {
      if (gidx + 1 < NG) ktf[gidx + 1] = TG::tr_frag(cur, lane, gidx + 1);
      const int c2 = gidx / DC, c = gidx % DC;
      accQ[c] = mfma_bf16(ktf[gidx], DS[c2], accQ[c]);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  if (ntiles > 0) {
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) {
#pragma unroll
      for (int q = 0; q < LPT; ++q) issue_part(i, i, q, ntiles);
    }
    for (int j = 0; j < ntiles; j += STAGES) {
      const bool more = unrolled_while<0, STAGES>([&](auto st) {
        constexpr int S = decltype(st)::value;
        step(st, j + S);
        return j + S + 1 < ntiles;
      });
      if (!more) break;
    }
    // DMAs past the last tile may be in flight
    wait_vmcnt<0>();
    wait_lgkmcnt<0>();
    barrier_nofence();
  }

  // ---- epilogue: dq = scale acc
  acc_hazard_wait();
  if (row_ok) {
    const float scale = p.scale;
    uint16_t* Qg = (uint16_t*)p.dq + base + (size_t)row * D;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * c + 8 * g4 + 4 * h;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc_read(accQ[c][4 * g4 + e]) * scale;
        *(u32x2*)(Qg + d0) = u32x2{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dk/dv kernel (bf16).  One wave = 32 keys; the Q and dO tiles of 32 rows
// and the rows' delta and -lse log2(e) stream through the LDS ring.  TABLE:
// range-list plans, with key blocks cut from key 0, their order, query-tile
// lists and per-key row intervals from the table's column sections.
template <int D, int NW, bool TABLE>
__global__ void __launch_bounds__(NW * 64, 1) bwd_dkdv_bf16_kernel(BwdParams p) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  using TG = TileGeom<D, NW>;
  constexpr int BQ = TG::ROWS;  // query rows per tile
  constexpr int BK = NW * 32;   // keys per block
  constexpr int KS = TG::KS, DC = TG::DC, NG = TG::NG, TILE = TG::TILE, LOADS = TG::LOADS;
  constexpr int LPT = 2 * LOADS + 1;  // DMA instructions per wave and tile: Q, dO, row terms
  constexpr int STAGES = kBwdStages, AHEAD = kBwdAhead, BAR = kBwdBarrierEvery;

  __shared__ __attribute__((aligned(1024))) uint16_t ring[STAGES][2 * TILE];
  // per stage and wave: -delta of the tile's 32 rows, then their -lse log2(e)
  __shared__ __attribute__((aligned(256))) float rows[STAGES][NW * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, h = lane >> 5;

  const MaskGeom g = p.g;
  const int N = g.seq_len;
  // Key blocks are cut per side like query blocks; index order is heavy
  // first (the earliest keys of a side are seen by the most rows).  Groups of
  // 32 neighbouring key blocks, which stream nearly the same query tiles, run
  // on one XCD (a quarter of the fetches past L2 of plain round robin); the
  // workgroups take them from the per-XCD work queues.
  const int n_tasks = p.n_slices * p.n_kblocks;
  const int pos = workgroup_task(p.queues, n_tasks);
  if (pos < 0) return;  // the queues were empty: no task for this workgroup
  const int task = launch_task(pos, n_tasks, p.n_kblocks, kDkdvXcdGroup);
  const int bh = task / p.n_kblocks;
  int k0, k1, ntiles, e0 = 0;
  TileSpans sp{0, 0, 0, 0};
  if constexpr (TABLE) {
    const int kb = p.cb_order[task - bh * p.n_kblocks];
    k0 = kb * BK;
    k1 = k0 + BK < N ? k0 + BK : N;
    e0 = p.cb_blk[kb];
    ntiles = p.cb_blk[kb + 1] - e0;
  } else {
    const int kb = task - bh * p.n_kblocks;
    qblock_rows(g, BK, kb, &k0, &k1);
    sp = block_tiles(block_col_ranges(g, k0, k1), BQ);
    ntiles = span_count(sp);
  }
  // range-list plans: the block's query-tile entries (tile | whole bit of
  // wave w << (24 + w)), staged in LDS for the whole task
  int32_t* ent = nullptr;
  if constexpr (TABLE) {
    __shared__ int32_t ent_buf[kMaxTableEntries];
    for (int i = tid; i < ntiles; i += NW * 64) ent_buf[i] = p.cb_ent[e0 + i];
    __syncthreads();
    ent = ent_buf;
  }
  auto entry = [&](int t) { return __builtin_amdgcn_readfirstlane(ent[t < ntiles ? t : ntiles - 1]); };
  // Range-list plans: the raw entries a step needs (its DMA tile's and the
  // next tile's) are read from LDS one step ahead, so that the step's top
  // takes them without waiting for an LDS read.
  int pf_dma = 0, pf_next = 0;
  auto prefetch_entries = [&](int j) {
    if constexpr (TABLE) {
      pf_dma = ent[j + kBwdAhead < ntiles ? j + kBwdAhead : ntiles - 1];
      pf_next = ent[j + 1 < ntiles ? j + 1 : ntiles - 1];
    }
  };

  const size_t base = (size_t)bh * (size_t)N * D;
  const int slice_bytes = N * D * 2;
  const i32x4_t desc_q = make_desc((const uint16_t*)p.q + base, slice_bytes);
  const i32x4_t desc_do = make_desc((const uint16_t*)p.dout + base, slice_bytes);
  // the row terms: lanes 0-31 fetch -delta, lanes 32-63 -lse log2(e); past
  // the end a delta lane reads the next plane (masked rows only) and an
  // lse lane reads zeros
  const i32x4_t desc_ws = make_desc(p.ws + (size_t)bh * 2 * N, N * 8);
  const int ws_voff = (lane & 31) * 4 + (lane >> 5) * N * 4;

  const int key = k0 + wave * 32 + n;
  const bool key_ok = key < k1;
  ItemIntervals civ{{0, 0, 0, 0}, 0, 0};
  int max_iv = 0;
  if constexpr (TABLE) {
    civ = item_intervals(p.cb_cols, p.cb_iv, key, key_ok);
    max_iv = wave_max_intervals(civ.n_iv);
  }
  const Ranges cr = TABLE ? civ.r : (key_ok ? col_ranges(g, key) : Ranges{0, 0, 0, 0});

  // K and V fragments (B operands) stay in accumulation registers for the
  // whole task (zeros for keys past the block).
  u32x4 kf[KS], vf[KS];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t*)p.k + base, slice_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t*)p.v + base, slice_bytes);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int off = (key * D + 16 * s + 8 * h) * 2;
      kf[s] = load16(rk, off);
      vf[s] = load16(rv, off);
      if (!key_ok) {
        kf[s] = u32x4{0, 0, 0, 0};
        vf[s] = u32x4{0, 0, 0, 0};
      }
      keep_in_acc(kf[s]);
      keep_in_acc(vf[s]);
    }
  }

  auto stage = [&](auto st) -> uint16_t* { return ring[decltype(st)::value]; };
  auto rstage = [&](auto st) -> float* { return rows[decltype(st)::value] + wave * 64; };
  int dma_voff[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) dma_voff[i] = TG::dma_voff(wave, lane, i);
  // (range-list plans pass the tile index, read once per step: tile_pre)
  auto issue_part = [&](uint16_t* dst, float* rdst, int t, int q, int t_end, int tile_pre) {
    int tile;
    if constexpr (TABLE) tile = tile_pre;
    else tile = span_tile(sp, t < t_end ? t : t_end - 1);
    if (q < 2 * LOADS) {
      const int i = q >> 1, tt = q & 1;
      load16_lds_asm(tt ? desc_do : desc_q, dst + tt * TILE + (wave * LOADS + i) * 512, dma_voff[i],
                     tile * BQ * D * 2);
    } else {
      load4_lds_asm(desc_ws, rdst, ws_voff, tile * BQ * 4);
    }
  };
  auto issue = [&](auto st, int t, int t_end) {
    int tile_pre = 0;
    if constexpr (TABLE) tile_pre = entry(t) & 0xffffff;
#pragma unroll
    for (int q = 0; q < LPT; ++q) issue_part(stage(st), rstage(st), t, q, t_end, tile_pre);
  };

  f32x16 accV[DC], accK[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      accV[c][i] = 0.f;
      accK[c][i] = 0.f;
    }
  }
  const float sl2 = p.score_log2;

  // Query tiles that every valid key of the wave sees whole (range-list
  // plans: the entry's bit of this wave).
  Ranges wfirst{0, 0, 0, 0}, wlast{0, 0, 0, 0};
  if constexpr (!TABLE) {
    const int wa = k0 + wave * 32;
    const int wb = wa + 32 < k1 ? wa + 32 : k1;
    if (wa < wb) {
      wfirst = col_ranges(g, wa);
      wlast = col_ranges(g, wb - 1);
    }
  }
  // as step ranges: query tiles inside [wlast.lo1, wfirst.hi1) or
  // [wlast.lo2, wfirst.hi2), the rows that see every valid key of the wave
  const StepRange w1 = span_steps_in(sp, first_whole_tile(wlast.lo1, BQ), end_whole_tile(wfirst.hi1, BQ));
  const StepRange w2 = span_steps_in(sp, first_whole_tile(wlast.lo2, BQ), end_whole_tile(wfirst.hi2, BQ));
  auto tile_whole = [&](int t) { return in_steps(w1, t) || in_steps(w2, t); };
  // the partial-tile mask of scores of the query tile at row q0
  auto mask_tile = [&](f32x16& X, int q0) {
    if constexpr (TABLE) mask_scores_iv(X, q0, h, civ, max_iv, p.cb_iv);
    else mask_scores(X, q0, h, cr);
  };
  // Row terms of the lane's elements 4 q4 .. 4 q4 + 3 (rows 8 q4 + 4h + 0..3):
  // plane 0 -delta, plane 1 -lse log2(e).  Read a quad at a time, shortly
  // before use, to keep few of them live.
  auto rows_read = [&](const float* src, int plane, int q4, float* dst) {
    const float4 v = *(const float4*)(src + 32 * plane + 8 * q4 + 4 * h);
    dst[4 * q4 + 0] = v.x;
    dst[4 * q4 + 1] = v.y;
    dst[4 * q4 + 2] = v.z;
    dst[4 * q4 + 3] = v.w;
  };

  u32x4 qf[KS], dof[KS];
  auto qdread = [&](const uint16_t* src, int s) {
    qf[s] = TG::row_frag(src, n, h, s);
    dof[s] = TG::row_frag(src + TILE, n, h, s);
  };

  f32x16 XA, DA, XB, DB;
  float nlv[16];  // -lse log2(e) of the rows of the tile being exponentiated
  float ndl[16];  // -delta of the rows of the tile whose dP is formed next: its start

  // Step j.  Phase 1: X, dP of tile j+1 under dS of tile j and the packs of
  // P and dS.  Phase 2: dV^T += dO^T P and dK^T += Q^T dS of tile j under
  // the mask (partial tiles) and exponentials of tile j+1.  Ring use and
  // the DMA's place after the dP MFMA as in the dq kernel, with the rows'
  // terms in the same stage.
  auto step = [&](auto st, int j, int t_end, f32x16& P, f32x16& DP, f32x16& Xn, f32x16& DPn) {
    constexpr int ST = decltype(st)::value;
    using NX = IC<(ST + 1) % STAGES>;
    using N2 = IC<(ST + 2) % STAGES>;
    using AH = IC<(ST + AHEAD) % STAGES>;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      keep_in_acc(accV[c]);
      keep_in_acc(accK[c]);
    }
    const uint16_t* nx = stage(NX{});
    const uint16_t* cur = stage(st);
    u32x4 PK[2], DSK[2];
    u32x4 doT[NG], qT[NG];
    auto ds_pair = [&](int jj) {  // DP holds dP - delta
      DSK[jj >> 3][(jj & 7) >> 1] = pack_bf16(P[jj] * DP[jj], P[jj + 1] * DP[jj + 1]);
      PK[jj >> 3][(jj & 7) >> 1] = pack_bf16(P[jj], P[jj + 1]);
      pin(DSK[jj >> 3][(jj & 7) >> 1]);
      pin(PK[jj >> 3][(jj & 7) >> 1]);
    };
    auto trread = [&](int gidx) {
      doT[gidx] = TG::tr_frag(cur + TILE, lane, gidx);
      qT[gidx] = TG::tr_frag(cur, lane, gidx);
    };
    // range-list plans: this step's DMA tile and the next tile's entry,
    // prefetched by the previous step
    int dma_tile = 0, next_e = 0;
    if constexpr (TABLE) {
      dma_tile = __builtin_amdgcn_readfirstlane(pf_dma) & 0xffffff;
      next_e = __builtin_amdgcn_readfirstlane(pf_next);
    }
    auto dma = [&](int s) {
#pragma unroll
      for (int q = s * LPT / KS; q < (s + 1) * LPT / KS; ++q)
        issue_part(stage(AH{}), rstage(AH{}), j + AHEAD, q, t_end, dma_tile);
    };

    constexpr int PAIRS = 8 / KS;  // dS element pairs per k-step
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (s == 0) mfma_v_first_ba(Xn, qf[s], kf[s]);
      else mfma_v_acc_ba(Xn, qf[s], kf[s]);
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0) prefetch_entries(j + 1);
      if (s + 2 < KS) qdread(nx, s + 2);
#pragma unroll
      for (int u = 0; u < PAIRS; ++u) ds_pair(2 * (s * PAIRS + u));
      __builtin_amdgcn_sched_barrier(0);
      if (s == 0) mfma_v_init_ba(DPn, dof[s], vf[s], *(const f32x16*)ndl);
      else mfma_v_acc_ba(DPn, dof[s], vf[s]);
      __builtin_amdgcn_sched_barrier(0);
      dma(s);
      if (s == 1) hold(*(const f32x16*)ndl);  // two MFMAs past its read as the start of dP
#pragma unroll
      for (int gq = s * NG / KS; gq < (s + 1) * NG / KS; ++gq) trread(gq);
      // -lse log2(e) of tile j+1's rows for phase 2's exponentials: read here,
      // where the stage is resident and the reads have a phase to land
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        if (s == KS - 4 + q4) rows_read(rstage(NX{}), 1, q4, nlv);
      __builtin_amdgcn_sched_barrier(0);
    }

    // phase 2: 2 NG slots; the last score product is two MFMAs back at the
    // first one.  The transposed reads were all issued in phase 1 (under
    // the exponentials here they left too few issue slots).  The barrier
    // slot is 2 NG - 6; the first reads of tile j+2 follow it, in the next
    // two slots.
    constexpr int UB = 2 * (NG - 3);  // slot of the barrier
#pragma unroll
    for (int gidx = 0; gidx < NG; ++gidx) {
      const int c2 = gidx / DC, c = gidx % DC;
#pragma unroll
      for (int sl = 0; sl < 2; ++sl) {
        if (sl == 0) accV[c] = mfma_bf16(doT[gidx], PK[c2], accV[c]);
        else accK[c] = mfma_bf16(qT[gidx], DSK[c2], accK[c]);
        __builtin_amdgcn_sched_barrier(0);
        const int u = 2 * gidx + sl;
        if constexpr (TABLE) {
          if (u == 0 && !((next_e >> (24 + wave)) & 1)) mask_tile(Xn, (next_e & 0xffffff) * BQ);  // rare
        } else {
          if (u == 0 && !tile_whole(j + 1)) mask_tile(Xn, span_tile(sp, j + 1) * BQ);  // rare
        }
        if (u == UB && ST % BAR == 0) {
          wait_lgkmcnt<0>();
          wait_vmcnt<(AHEAD - BAR - 1) * LPT>();
          barrier_nofence();
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          if (k * 2 * NG / 16 == u) {
            Xn[k] = __builtin_amdgcn_exp2f(fmaf(Xn[k], sl2, nlv[k]));
            pin(Xn[k]);
          }
        }
        if (u == UB + 1) {
          qdread(stage(N2{}), 0);
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) rows_read(rstage(N2{}), 0, q4, ndl);  // for the next step's dP
        }
        if (u == UB + 2) qdread(stage(N2{}), 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  auto first_tile = [&](int t_begin, int t_end) {
    unrolled_while<0, AHEAD>([&](auto st) {
      issue(st, t_begin + decltype(st)::value, t_end);
      return true;
    });
    wait_vmcnt<(AHEAD - 2) * LPT>();  // first two tiles
    barrier_nofence();
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      rows_read(rstage(IC<0>{}), 1, q4, nlv);
      rows_read(rstage(IC<0>{}), 0, q4, ndl);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qdread(ring[0], s);
      if (s == 0) {
        mfma_v_first_ba(XA, qf[s], kf[s]);
        mfma_v_init_ba(DA, dof[s], vf[s], *(const f32x16*)ndl);
      } else {
        mfma_v_acc_ba(XA, qf[s], kf[s]);
        mfma_v_acc_ba(DA, dof[s], vf[s]);
      }
      if (s == 1) hold(*(const f32x16*)ndl);
    }
    __builtin_amdgcn_sched_barrier(0);
    acc_hazard_wait();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (TABLE) {
      const int e = entry(t_begin);
      if (!((e >> (24 + wave)) & 1)) mask_tile(XA, (e & 0xffffff) * BQ);
    } else {
      if (!tile_whole(t_begin)) mask_tile(XA, span_tile(sp, t_begin) * BQ);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) XA[i] = __builtin_amdgcn_exp2f(fmaf(XA[i], sl2, nlv[i]));
    qdread(ring[1], 0);
    qdread(ring[1], 1);
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) rows_read(rstage(IC<1>{}), 0, q4, ndl);
  };

  if (ntiles > 0) {
    first_tile(0, ntiles);
    prefetch_entries(0);
    for (int j = 0; j < ntiles; j += STAGES) {
      const bool more = unrolled_while<0, STAGES>([&](auto st) {
        constexpr int S = decltype(st)::value;
        if constexpr (S % 2 == 0) step(st, j + S, ntiles, XA, DA, XB, DB);
        else step(st, j + S, ntiles, XB, DB, XA, DA);
        return j + S + 1 < ntiles;
      });
      if (!more) break;
    }
    wait_vmcnt<0>();
    wait_lgkmcnt<0>();
    barrier_nofence();
  }

  // ---- epilogue: dv = acc_v, dk = scale acc_k
  acc_hazard_wait();
  if (key_ok) {
    const float scale = p.scale;
    uint16_t* Kg = (uint16_t*)p.dk + base + (size_t)key * D;
    uint16_t* Vg = (uint16_t*)p.dv + base + (size_t)key * D;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = 32 * c + 8 * g4 + 4 * h;
        float xk[4], xv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xk[e] = acc_read(accK[c][4 * g4 + e]) * scale;
          xv[e] = acc_read(accV[c][4 * g4 + e]);
        }
        *(u32x2*)(Kg + d0) = u32x2{pack_bf16(xk[0], xk[1]), pack_bf16(xk[2], xk[3])};
        *(u32x2*)(Vg + d0) = u32x2{pack_bf16(xv[0], xv[1]), pack_bf16(xv[2], xv[3])};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernels: 32 rows (keys) per workgroup, 8 lanes per row (key), each
// lane owning D/8 consecutive columns; pairs are taken one at a time from
// the same schedules with the exact mask, in fp32 throughout.
__device__ __forceinline__ float sum8(float x) {
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) x += __shfl_xor(x, o, 8);
  return x;
}

// TABLE: range-list plans; each row (key) walks its own intervals from the
// table in ascending order.
template <int D, bool TABLE>
__global__ void __launch_bounds__(256) bwd_dq_fp32_kernel(BwdParams p) {
  constexpr int BR = 32, BC = 32, E = D / 8;
  const MaskGeom g = p.g;
  const int N = g.seq_len;
  const int slice = threadIdx.x & 7, lr = threadIdx.x >> 3;
  const int bh = blockIdx.x / p.n_qblocks;
  int r0, r1, ntiles = 0;
  TileSpans sp{0, 0, 0, 0};
  if constexpr (TABLE) {
    r0 = p.tb_order[blockIdx.x - bh * p.n_qblocks] * BR;
    r1 = r0 + BR < N ? r0 + BR : N;
  } else {
    const int qb = heavy_first_qblock(g, BR, blockIdx.x - bh * p.n_qblocks);
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
  const int qrow = row_ok ? row : r0;
  const size_t roff = base + (size_t)qrow * D + slice * E;
  float q[E], dob[E], acc[E];
  float part = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = ((const float*)p.q)[roff + e];
    dob[e] = ((const float*)p.dout)[roff + e];
    part = fmaf(dob[e], ((const float*)p.o)[roff + e], part);
    acc[e] = 0.f;
  }
  const float delta = sum8(part);
  const float lse = p.lse[(size_t)bh * N + qrow];
  // (range-list plans: the most negative finite float for a row in no group,
  // which has no key; as in the bf16 kernel)
  const float nl = TABLE && lse == -INFINITY ? -FLT_MAX : -lse * kLog2e;
  if (row_ok && slice < 2) p.ws[(size_t)bh * 2 * N + (size_t)slice * N + row] = slice ? nl : -delta;
  const float sl2 = p.score_log2;
  auto key_step = [&](int j) {
    const float* kj = K + (size_t)j * D;
    const float* vj = V + (size_t)j * D;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      s = fmaf(q[e], kj[e], s);
      dp = fmaf(dob[e], vj[e], dp);
    }
    s = sum8(s);
    dp = sum8(dp);
    const float pj = exp2f(fmaf(s, sl2, nl));
    const float ds = pj * (dp - delta);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = fmaf(ds, kj[e], acc[e]);
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
  float* dQ = (float*)p.dq + base + (size_t)row * D + slice * E;
#pragma unroll
  for (int e = 0; e < E; ++e) dQ[e] = acc[e] * p.scale;
}

template <int D, bool TABLE>
__global__ void __launch_bounds__(256) bwd_dkdv_fp32_kernel(BwdParams p) {
  constexpr int BK = 32, BQ = 32, E = D / 8;
  const MaskGeom g = p.g;
  const int N = g.seq_len;
  const int slice = threadIdx.x & 7, lk = threadIdx.x >> 3;
  const int bh = blockIdx.x / p.n_kblocks;
  int k0, k1, ntiles = 0;
  TileSpans sp{0, 0, 0, 0};
  if constexpr (TABLE) {
    k0 = p.cb_order[blockIdx.x - bh * p.n_kblocks] * BK;
    k1 = k0 + BK < N ? k0 + BK : N;
  } else {
    qblock_rows(g, BK, blockIdx.x - bh * p.n_kblocks, &k0, &k1);
    sp = block_tiles(block_col_ranges(g, k0, k1), BQ);
    ntiles = span_count(sp);
  }
  const int key = k0 + lk;
  const bool key_ok = key < k1;
  const Ranges cr = TABLE ? Ranges{0, 0, 0, 0} : (key_ok ? col_ranges(g, key) : Ranges{0, 0, 0, 0});
  const size_t base = (size_t)bh * (size_t)N * D;
  const float* __restrict__ Q = (const float*)p.q + base + slice * E;
  const float* __restrict__ dO = (const float*)p.dout + base + slice * E;
  const float* __restrict__ ndl = p.ws + (size_t)bh * 2 * N;  // -delta
  const float* __restrict__ nlr = ndl + N;
  const int krow = key_ok ? key : k0;
  float kk[E], vv[E], ak[E], av[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kk[e] = ((const float*)p.k)[base + (size_t)krow * D + slice * E + e];
    vv[e] = ((const float*)p.v)[base + (size_t)krow * D + slice * E + e];
    ak[e] = 0.f;
    av[e] = 0.f;
  }
  const float sl2 = p.score_log2;
  auto row_step = [&](int i) {
    const float* qi = Q + (size_t)i * D;
    const float* doi = dO + (size_t)i * D;
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      s = fmaf(qi[e], kk[e], s);
      dp = fmaf(doi[e], vv[e], dp);
    }
    s = sum8(s);
    dp = sum8(dp);
    const float pij = exp2f(fmaf(s, sl2, nlr[i]));
    const float ds = pij * (dp + ndl[i]);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      av[e] = fmaf(pij, doi[e], av[e]);
      ak[e] = fmaf(ds, qi[e], ak[e]);
    }
  };
  if constexpr (TABLE) {
    if (key_ok) {  // uniform across the key's 8 lanes
      const int info = p.cb_cols[key];
      const int n_iv = info & 255, iv_off = info >> 8;
      for (int k = 0; k < n_iv; ++k)
        for (int i = p.cb_iv[2 * (iv_off + k)], i1 = p.cb_iv[2 * (iv_off + k) + 1]; i < i1; ++i) row_step(i);
    }
  } else {
    for (int it = 0; it < ntiles; ++it) {
      const int q0 = span_tile(sp, it) * BQ;
      const int q1 = q0 + BQ < N ? q0 + BQ : N;
      for (int i = q0; i < q1; ++i) {
        if (!in_ranges(cr, i)) continue;  // uniform across the key's 8 lanes
        row_step(i);
      }
    }
  }
  if (!key_ok) return;
  float* dK = (float*)p.dk + base + (size_t)key * D + slice * E;
  float* dV = (float*)p.dv + base + (size_t)key * D + slice * E;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    dK[e] = ak[e] * p.scale;
    dV[e] = av[e];
  }
}

// ---------------------------------------------------------------------------
void bwd_block_sizes(int dtype, int head_dim, int* block_q, int* block_kv) {
  (void)head_dim;
  if (dtype == kBf16) {
    *block_q = kBf16Waves * 32;
    *block_kv = kBf16Waves * 32;
  } else {
    *block_q = 32;
    *block_kv = 32;
  }
}

namespace {

template <int D, bool TABLE>
void launch_bwd_kernels(int dtype, int bh, const BwdParams& p, hipStream_t stream) {
  const dim3 gq((unsigned)bh * (unsigned)p.n_qblocks), gk((unsigned)bh * (unsigned)p.n_kblocks);
  if (dtype == kBf16) {
    // both kernels take their tasks from the call's work queues, one after the other
    const dim3 block(kBf16Waves * 64);
    if constexpr (TABLE)
      hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, kBf16Waves>), dim3((unsigned)queue_grid((int)gq.x)), block, 0,
                         stream, p);
    else
      hipLaunchKernelGGL((bwd_dq2_bf16_kernel<D, kBf16Waves>), dim3((unsigned)queue_grid((int)gq.x)), block, 0,
                         stream, p);
    hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, kBf16Waves, TABLE>), dim3((unsigned)queue_grid((int)gk.x)), block, 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((bwd_dq_fp32_kernel<D, TABLE>), gq, dim3(256), 0, stream, p);
    hipLaunchKernelGGL((bwd_dkdv_fp32_kernel<D, TABLE>), gk, dim3(256), 0, stream, p);
  }
}

}  // namespace

hipError_t launch_bwd(int dtype, int head_dim, int bh, const BwdParams& p, hipStream_t stream) {
  const bool table = p.cb_ent != nullptr;
  if (head_dim == 128) {
    if (table) launch_bwd_kernels<128, true>(dtype, bh, p, stream);
    else launch_bwd_kernels<128, false>(dtype, bh, p, stream);
  } else {
    if (table) launch_bwd_kernels<64, true>(dtype, bh, p, stream);
    else launch_bwd_kernels<64, false>(dtype, bh, p, stream);
  }
  return hipGetLastError();
}

}  // namespace attn_jvp
