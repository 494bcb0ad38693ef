// attn_jvp_launch.h -- internal interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mask_index.h"

namespace attn_jvp {

constexpr int kBf16 = 0;
constexpr int kFp32 = 1;
constexpr int kBf16Waves = 4;   // waves per bf16 workgroup; 32 query rows per wave
constexpr int kBf16BlockK = 32;  // keys per bf16 tile

// Range-list plans: the bf16 kernel stages a query block's tile entries in
// LDS next to the 128 KB ring, so a block may stream at most this many tiles.
constexpr int kMaxTableEntries = 7680;
// The primal-only instance (K and V in a 64 KB ring) fits two workgroups per
// CU with at most this many entries staged (64 KB + 15.5 KB + the queue word
// each); range-list plans whose blocks stream more take the one-workgroup
// instance.
constexpr int kPoMaxTableEntries = 3968;
constexpr int32_t kTableMagic = 0x314a5441;  // "ATJ1"

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* tq;
  const void* tk;
  const void* tv;
  void* o;
  void* to;
  float* lse;
  MaskGeom g;
  int32_t n_qblocks;  // query blocks per (b, h); the grid is (b, h) x blocks
  float score_log2;   // scale * log2(e)
  float scale;
  int32_t ctz;        // clean-tangent-zero plan (teacher forcing only)
  int32_t primal;     // with ctz: every block forms o and lse only (no tangents; to may be null)
  int32_t side;       // teacher forcing: -1 every query block, 0 the clean side's only, 1 the noisy side's
  // range-list plans (all null otherwise): sections of the device table
  const int32_t* tb_blk;    // [n_qblocks + 1] first entry of each query block
  const int32_t* tb_order;  // [n_qblocks] launch order
  const int32_t* tb_ent;    // tile | (whole bit of wave w) << (24 + w)
  const int32_t* tb_rows;   // [N] (first interval << 8) | interval count
  const int32_t* tb_iv;     // (lo, hi) pairs
  int32_t tb_max_entries;   // the most entries any query block streams
  // bf16 kernels: the work queues of this call (kQueueWords words, take_task)
  // and the number of tasks, (b, h) slices x n_qblocks
  int32_t* queues;
  int32_t n_tasks;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* ws;          // per (b, h): [2][N] floats, -delta then -lse * log2(e)
  MaskGeom g;
  int32_t n_qblocks;  // dq kernel: query blocks per (b, h)
  int32_t n_kblocks;  // dk/dv kernel: key blocks per (b, h)
  float score_log2;   // scale * log2(e)
  float scale;
  // range-list plans (all null otherwise): sections of the device table.
  // Query side, as in FwdParams (the dq kernel walks the forward's schedule):
  const int32_t* tb_blk;
  const int32_t* tb_order;
  const int32_t* tb_ent;
  const int32_t* tb_rows;
  const int32_t* tb_iv;
  // columns (the dk/dv kernel): per key block its 32-row query tiles, per key
  // its row intervals
  const int32_t* cb_blk;    // [n_kblocks + 1] first entry of each key block
  const int32_t* cb_order;  // [n_kblocks] launch order
  const int32_t* cb_ent;    // query tile | (whole bit of wave w) << (24 + w)
  const int32_t* cb_cols;   // [N] (first interval << 8) | interval count
  const int32_t* cb_iv;     // (lo, hi) row intervals
  // bf16 kernels: the work queues of this call (kQueueWords words, take_task),
  // used by the dq kernel and then, zeroed again, by the dk/dv kernel; the
  // number of (b, h) slices (tasks: n_slices x n_qblocks, n_slices x n_kblocks)
  int32_t* queues;
  int32_t n_slices;
};

// int32 words per call of the bf16 kernels' work queues (take_task uses 9).
constexpr int kQueueWords = 16;

// Workgroups of a grid that takes n tasks from work queues (take_task): half
// as many again (rounded to whole XCD rounds), which lets a faster XCD take up
// to that many of the other XCDs' tasks (the last tasks are light, so it may
// need many: with an eighth more, the fast XCDs ran out of workgroups before
// the end of the dk/dv launch); the spare workgroups of the slower ones find
// the queues empty and exit within microseconds.
inline int queue_grid(int n) { return n + 8 * ((n + 15) / 16); }

// Query rows per block and keys per tile of the kernel chosen for dtype/head_dim.
void block_sizes(int dtype, int head_dim, int* block_q, int* block_k);

// Launch one forward + JVP over `grid` workgroups; returns hipGetLastError().
hipError_t launch_fwd(int dtype, int head_dim, int grid, const FwdParams& p, hipStream_t stream);

// Rows per dq-kernel block and keys per dk/dv-kernel block of the backward.
void bwd_block_sizes(int dtype, int head_dim, int* block_q, int* block_kv);

// Key blocks per XCD group of the dk/dv kernel's launch order (launch_task).
constexpr int kDkdvXcdGroup = 32;
// Query blocks per XCD group of the forward + JVP's launch order.
constexpr int kFwdXcdGroup = 128;
// The same for the noisy-side launch of clean-tangent-zero plans.
constexpr int kCtzNoisyXcdGroup = 64;

// Launch the backward (dq kernel, then dk/dv kernel) for bh = B * H slices.
hipError_t launch_bwd(int dtype, int head_dim, int bh, const BwdParams& p, hipStream_t stream);

}  // namespace attn_jvp
