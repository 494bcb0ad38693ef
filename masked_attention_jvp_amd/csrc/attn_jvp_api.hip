// attn_jvp_api.hip -- the C ABI declared in include/attn_jvp.h: plan
// creation and validation, schedule introspection and the launch entry point.
// Planning is pure host arithmetic on the four mask integers; the kernels
// derive their key ranges and tiles from the same functions (mask_index.h),
// so the exported ranges and tile map are exactly what the device walks.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "attn_jvp.h"
#include "attn_jvp_launch.h"
#include "mask_index.h"

using namespace attn_jvp;

// Schedule of a range-list plan (query groups x key intervals), serialised
// into one int32 table that the caller places in device memory:
//   [0..7]     header: magic, n_qblocks, n_entries, n_intervals, max entries per
//              query block, n_kblocks, n_col_entries, n_col_intervals
//   blk        [n_qblocks + 1]  first entry of each query block
//   order      [n_qblocks]      launch order (workgroup t -> query block)
//   entries    one per streamed key tile: tile | (whole bit of wave w) << (24 + w)
//   rows       [N]              per query row: (first interval << 8) | interval count
//   intervals  [2 n_intervals]  key intervals (lo, hi), merged and sorted per group
// and the same for the columns of the mask, which the backward's dk/dv kernel
// walks (key blocks of 32 x waves keys, 32-row query tiles; per key the
// merged row intervals that see it):
//   cblk [n_kblocks + 1], corder [n_kblocks], centries, cols [N], cintervals.
// The column sections are empty (n_kblocks = 0) when the backward cannot take
// the plan (bwd_error says why).
struct RangeSchedule {
  std::vector<int32_t> table;
  int64_t off_blk = 0, off_order = 0, off_ent = 0, off_rows = 0, off_iv = 0;
  int64_t off_cblk = 0, off_corder = 0, off_cent = 0, off_cols = 0, off_civ = 0;
  int32_t n_entries = 0, max_entries = 0;
  int32_t n_kblocks = 0, n_col_entries = 0;
  std::vector<uint8_t> ent_class;  // per entry: 1 every row of the block sees the whole tile, 2 otherwise
  bool rows_over_two = false;      // some row has more than two key intervals
  bool cols_over_two = false;      // some key is seen by more than two row intervals
  std::string bwd_error;           // non-empty: the backward refuses this plan
};

struct attn_jvp_plan {
  RangeSchedule* rs = nullptr;  // range-list plans only
  MaskGeom g;
  int32_t batch, heads, head_dim, dtype;
  float scale;
  uint32_t flags;
  int32_t block_q, block_k;
  int32_t n_qblocks, n_ktiles;
  int64_t allowed_pairs;
  int64_t visited_tiles;
  int64_t useful_flops;
  // backward: rows per dq block, keys per dk/dv block, blocks per (b, h)
  int32_t bwd_block_q, bwd_block_kv;
  int32_t bwd_n_qblocks, bwd_n_kblocks;
  int64_t bwd_useful_flops;
};

namespace {

thread_local std::string g_detail;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_detail = buf;
  return code;
}

int ok() {
  g_detail.clear();
  return ATTN_JVP_OK;
}

// Allowed pairs per (b, h): sum over chunks of rows * keys.
int64_t count_pairs(const MaskGeom& g) {
  int64_t total = 0;
  const int32_t nch = g.side_len / g.chunk_len;
  for (int32_t side = 0; side < (g.tf ? 2 : 1); ++side)
    for (int32_t c = 0; c < nch; ++c) {
      const Ranges r = row_ranges(g, side * g.side_len + c * g.chunk_len);
      const int64_t keys = (int64_t)(r.hi1 - r.lo1) + (r.hi2 > r.lo2 ? r.hi2 - r.lo2 : 0);
      total += keys * g.chunk_len;
    }
  return total;
}

// Useful FLOPs per (b, h): 12 d per allowed pair; with clean-tangent-zero,
// 4 d per clean-row pair, 8 d per noisy-row / clean-key pair, 12 d per
// noisy-row / noisy-key pair.  Rows of one chunk share their key ranges.
int64_t count_flops(const MaskGeom& g, int32_t head_dim, bool ctz) {
  int64_t total = 0;
  const int32_t nch = g.side_len / g.chunk_len;
  for (int32_t side = 0; side < (g.tf ? 2 : 1); ++side)
    for (int32_t c = 0; c < nch; ++c) {
      const Ranges r = row_ranges(g, side * g.side_len + c * g.chunk_len);
      const int64_t k1 = r.hi1 - r.lo1, k2 = r.hi2 > r.lo2 ? r.hi2 - r.lo2 : 0;  // clean, noisy keys
      int64_t per_row;
      if (!ctz) per_row = 12 * (k1 + k2);
      else if (side == 0) per_row = 4 * k1;
      else per_row = 8 * k1 + 12 * k2;
      total += per_row * g.chunk_len;
    }
  return total * head_dim;
}

// Class of key tile [k0, k1) for rows [r0, r1): 0 none allowed, 1 all, 2 some.
int tile_class(const MaskGeom& g, int32_t r0, int32_t r1, int32_t k0, int32_t k1) {
  bool any = false, all = true;
  int32_t i = r0;
  while (i < r1) {
    const Ranges r = row_ranges(g, i);
    const int32_t pos = is_noisy(g, i) ? i - g.side_len : i;
    const int32_t chunk_end = (pos / g.chunk_len + 1) * g.chunk_len + (is_noisy(g, i) ? g.side_len : 0);
    any = any || meets(r, k0, k1);
    all = all && covers(r, k0, k1);
    i = chunk_end < r1 ? chunk_end : r1;
  }
  return !any ? 0 : (all ? 1 : 2);
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Per-device architecture check, cached: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch[64];

int check_device(int* dev_out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_JVP_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  *dev_out = dev;
  if (dev < 0 || dev >= 64) return fail(ATTN_JVP_E_UNSUPPORTED_DEVICE, "device index %d out of range", dev);
  int st = g_arch[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(ATTN_JVP_E_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(st, std::memory_order_relaxed);
    if (st == 2) return fail(ATTN_JVP_E_UNSUPPORTED_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  }
  if (st == 2) return fail(ATTN_JVP_E_UNSUPPORTED_DEVICE, "device %d is not gfx950", dev);
  return ATTN_JVP_OK;
}

// One axis of a range-list schedule.  Items (query rows; keys for the
// columns) are cut into blocks of bq from 0, the other axis into tiles of bt.
// grp[i] is the group of item i (-1: none); group g's intervals on the other
// axis are (iv[2k], iv[2k+1]) for g_iv[g] <= k < g_iv[g+1], sorted, disjoint
// and not touching.  Per block: the tiles that meet the intervals of its
// items' groups, ascending, each with a whole bit per wave of 32 items (every
// item of the wave sees the whole tile; waves without items never mask) and
// its class (1: every item of the block sees the whole tile, 2: not); the
// blocks' heavy-first order (more tiles first, stable).
struct SideSchedule {
  std::vector<int32_t> blk, order, ent;
  std::vector<uint8_t> cls;
  int32_t max_entries = 0;
};

void build_side(int32_t n, const std::vector<int32_t>& grp, const std::vector<int32_t>& g_iv,
                const std::vector<int32_t>& iv, int32_t bq, int32_t bt, SideSchedule* s) {
  const int32_t nb = cdiv(n, bq), nw = bq / 32;
  // does group g (or "no group", g < 0) see all of [t0, t1)?
  auto covers_g = [&](int32_t g, int32_t t0, int32_t t1) {
    if (g < 0) return false;
    for (int32_t k = g_iv[g]; k < g_iv[g + 1]; ++k)
      if (iv[2 * k] <= t0 && t1 <= iv[2 * k + 1]) return true;
    return false;
  };
  s->blk.assign(nb + 1, 0);
  s->ent.clear();
  s->cls.clear();
  s->max_entries = 0;
  std::vector<std::pair<int32_t, int32_t>> runs;
  std::vector<int32_t> bgroups;
  for (int32_t b = 0; b < nb; ++b) {
    const int32_t r0 = b * bq, r1 = std::min(r0 + bq, n);
    bgroups.clear();  // distinct groups of the block's items (-1: items in no group)
    for (int32_t r = r0; r < r1; ++r)
      if (bgroups.empty() || bgroups.back() != grp[r]) bgroups.push_back(grp[r]);
    runs.clear();
    for (int32_t g : bgroups) {
      if (g < 0) continue;
      for (int32_t k = g_iv[g]; k < g_iv[g + 1]; ++k) runs.emplace_back(iv[2 * k] / bt, cdiv(iv[2 * k + 1], bt));
    }
    std::sort(runs.begin(), runs.end());
    int32_t at = -1;
    for (const auto& run : runs) {
      for (int32_t t = std::max(run.first, at); t < run.second; ++t) {
        const int32_t t0 = t * bt, t1c = std::min(t0 + bt, n);
        int32_t e = t;
        for (int32_t w = 0; w < nw; ++w) {
          const int32_t wa = r0 + 32 * w, wb = std::min(wa + 32, r1);
          bool whole = true;
          // every item of the wave sees the whole tile (past n: zeros, not whole)
          for (int32_t r = wa; r < wb && whole; ++r) {
            if (r > wa && grp[r] == grp[r - 1]) continue;
            whole = t0 + bt <= n && covers_g(grp[r], t0, t0 + bt);
          }
          if (whole) e |= 1 << (24 + w);
        }
        bool all = true;
        for (int32_t g : bgroups) all = all && covers_g(g, t0, t1c);
        s->ent.push_back(e);
        s->cls.push_back(all ? 1 : 2);
      }
      at = std::max(at, run.second);
    }
    s->blk[b + 1] = (int32_t)s->ent.size();
    s->max_entries = std::max(s->max_entries, s->blk[b + 1] - s->blk[b]);
  }
  s->order.resize(nb);
  for (int32_t b = 0; b < nb; ++b) s->order[b] = b;
  std::stable_sort(s->order.begin(), s->order.end(), [&](int32_t a, int32_t b2) {
    return s->blk[a + 1] - s->blk[a] > s->blk[b2 + 1] - s->blk[b2];
  });
}

// The columns of a range-list mask: key j is seen by the rows of every group
// one of whose intervals holds j.  Sweeping the interval ends from left to
// right, the set of such groups is constant between consecutive ends; each
// stretch gets the merged row intervals of its groups (touching ones joined),
// and consecutive stretches with equal lists share one column group.
// Returns false if the column intervals would exceed 2^23.
bool build_columns(int32_t n, const std::vector<int32_t>& g_lo, const std::vector<int32_t>& g_hi,
                   const std::vector<int32_t>& g_iv, const std::vector<int32_t>& ivs,
                   std::vector<int32_t>* col_grp, std::vector<int32_t>* c_iv, std::vector<int32_t>* civs,
                   int32_t* max_count) {
  struct Ev { int32_t x, add, a, b; };
  std::vector<Ev> ev;
  for (size_t g = 0; g < g_lo.size(); ++g)
    for (int32_t k = g_iv[g]; k < g_iv[g + 1]; ++k) {
      ev.push_back({ivs[2 * k], 1, g_lo[g], g_hi[g]});
      ev.push_back({ivs[2 * k + 1], 0, g_lo[g], g_hi[g]});
    }
  // at equal x, ends (add = 0) before starts
  std::sort(ev.begin(), ev.end(), [](const Ev& u, const Ev& v) { return u.x != v.x ? u.x < v.x : u.add < v.add; });
  col_grp->assign(n, -1);
  c_iv->assign(1, 0);
  civs->clear();
  *max_count = 0;
  std::map<int32_t, int32_t> active;  // row_lo -> row_hi of the groups that see the current keys
  std::vector<int32_t> cur, prev;
  int32_t prev_id = -1, prev_end = -1;
  size_t e = 0;
  while (e < ev.size()) {
    const int32_t x = ev[e].x;
    for (; e < ev.size() && ev[e].x == x; ++e) {
      if (ev[e].add) active[ev[e].a] = ev[e].b;
      else active.erase(ev[e].a);
    }
    const int32_t y = e < ev.size() ? ev[e].x : n;
    if (y <= x || active.empty()) continue;
    cur.clear();
    for (const auto& r : active) {
      if (!cur.empty() && r.first == cur.back()) cur.back() = r.second;
      else {
        cur.push_back(r.first);
        cur.push_back(r.second);
      }
    }
    int32_t id;
    if (prev_id >= 0 && prev_end == x && cur == prev) {
      id = prev_id;
    } else {
      civs->insert(civs->end(), cur.begin(), cur.end());
      if (civs->size() / 2 >= (size_t(1) << 23)) return false;
      id = (int32_t)c_iv->size() - 1;
      c_iv->push_back((int32_t)(civs->size() / 2));
      *max_count = std::max(*max_count, (int32_t)(cur.size() / 2));
      prev = cur;
    }
    for (int32_t j = x; j < y; ++j) (*col_grp)[j] = id;
    prev_id = id;
    prev_end = y;
  }
  return true;
}

}  // namespace

// Workspace of attn_jvp_bwd_noalloc: a file-scope device array, so that
// that entry point allocates nothing.  Each GPU the library runs on holds its
// own copy until the process ends.  Host code never uses the array's name as
// an address (on the host it is a stand-in, not device memory): the device
// address of each GPU's copy comes from hipGetSymbolAddress, once per device,
// and is kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(32) << 20;  // 8 bytes per row: B H N <= 4,194,304
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

// Device address of this device's scratch array (dev is current).
int scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(ATTN_JVP_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}

// Work queues of the bf16 kernels (take_task): a ring of kQueueSlots slots
// of kQueueWords int32 in a file-scope device array, zero when the library
// loads and zero again after every launch that used a slot, so no call
// allocates for them (attn_jvp_bwd_noalloc included).  Calls on a device take
// the slots in turn; a slot is used again kQueueSlots calls later, so calls
// of this library that run at the same time on one GPU (on several streams)
// must number at most kQueueSlots.  Host code takes each GPU's address of the
// array from hipGetSymbolAddress, once per device.
constexpr int kQueueSlots = 256;
static __device__ __align__(256) int32_t task_queues[kQueueSlots * kQueueWords];
std::mutex g_queue_mu;
int32_t* g_queue_ptr[64];
std::atomic<uint32_t> g_queue_next[64];

// The next slot of this device's ring (dev is current).
int queue_slot(int dev, int32_t** out) {
  {
    std::lock_guard<std::mutex> lock(g_queue_mu);
    if (g_queue_ptr[dev] == nullptr) {
      void* ptr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(task_queues));
      if (e != hipSuccess || ptr == nullptr)
        return fail(ATTN_JVP_E_HIP, "hipGetSymbolAddress(task_queues) on device %d: %s", dev, hipGetErrorString(e));
      g_queue_ptr[dev] = (int32_t*)ptr;
    }
  }
  const uint32_t slot = g_queue_next[dev].fetch_add(1, std::memory_order_relaxed) % kQueueSlots;
  *out = g_queue_ptr[dev] + (size_t)slot * kQueueWords;
  return ok();
}

// Measurement: workgroup w (of kClockSampleGroups, one per XCD when
// workgroups go to the 8 XCDs round robin) stores its XCD number, the shader
// clock counter (s_memtime, counting at the XCD's shader clock) and the
// constant 100 MHz real-time counter (s_memrealtime).
constexpr int kClockSampleGroups = 8;
__global__ void clock_sample_kernel(uint64_t* out) {
  if (threadIdx.x == 0) {
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t rt = __builtin_amdgcn_s_memrealtime();
    out[4 * blockIdx.x + 0] = xcc & 0xf;
    out[4 * blockIdx.x + 1] = t;
    out[4 * blockIdx.x + 2] = rt;
    out[4 * blockIdx.x + 3] = 0;
  }
}

extern "C" {

int attn_jvp_create(attn_jvp_plan** out, const attn_jvp_mask_desc* mask, int32_t batch, int32_t heads,
                    int32_t head_dim, int32_t dtype, float softmax_scale) {
  return attn_jvp_create_ex(out, mask, batch, heads, head_dim, dtype, softmax_scale, 0u);
}

int attn_jvp_create_ex(attn_jvp_plan** out, const attn_jvp_mask_desc* mask, int32_t batch, int32_t heads,
                       int32_t head_dim, int32_t dtype, float softmax_scale, uint32_t flags) {
  if (out == nullptr || mask == nullptr) return fail(ATTN_JVP_E_NULL, "out and mask must be non-NULL");
  *out = nullptr;
  const attn_jvp_mask_desc& m = *mask;
  if (m.tokens_per_frame < 1 || m.n_frames < 1 || m.frames_per_chunk < 1)
    return fail(ATTN_JVP_E_INVALID, "tokens_per_frame, n_frames and frames_per_chunk must be >= 1 (got %d, %d, %d)",
                m.tokens_per_frame, m.n_frames, m.frames_per_chunk);
  if (m.tf_layout != 0 && m.tf_layout != 1)
    return fail(ATTN_JVP_E_INVALID, "tf_layout must be 0 or 1 (got %d)", m.tf_layout);
  if (m.n_frames % m.frames_per_chunk != 0)
    return fail(ATTN_JVP_E_INVALID, "n_frames (%d) must be a multiple of frames_per_chunk (%d)", m.n_frames,
                m.frames_per_chunk);
  if (batch < 1 || heads < 1) return fail(ATTN_JVP_E_INVALID, "batch and heads must be >= 1 (got %d, %d)", batch, heads);
  if (head_dim != 64 && head_dim != 128) return fail(ATTN_JVP_E_INVALID, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_FP32) return fail(ATTN_JVP_E_INVALID, "unknown dtype %d", dtype);
  if (!std::isfinite(softmax_scale)) return fail(ATTN_JVP_E_INVALID, "softmax_scale must be finite");
  if (flags & ~ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO) return fail(ATTN_JVP_E_INVALID, "unknown flag bits 0x%x", flags);
  if ((flags & ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO) && m.tf_layout != 1)
    return fail(ATTN_JVP_E_INVALID, "ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO needs tf_layout = 1");

  const int64_t side = (int64_t)m.tokens_per_frame * m.n_frames;
  const int64_t n = side * (m.tf_layout ? 2 : 1);
  // The bf16 kernel forms per-head byte offsets in 32 bits (buffer offsets);
  // the fp32 kernel indexes elements with 64-bit offsets.
  const int64_t per_head = n * head_dim * (dtype == ATTN_JVP_BF16 ? 2 : 1);
  if (n >= (int64_t(1) << 31) || per_head >= (int64_t(1) << 31))
    return fail(ATTN_JVP_E_OVERFLOW, "sequence of %lld tokens x d=%d exceeds the per-head limit (2^31 %s)",
                (long long)n, head_dim, dtype == ATTN_JVP_BF16 ? "bytes" : "elements");

  attn_jvp_plan* p = new (std::nothrow) attn_jvp_plan;
  if (p == nullptr) return fail(ATTN_JVP_E_NOMEM, "plan allocation failed");
  p->g = MaskGeom{(int32_t)side, m.tokens_per_frame * m.frames_per_chunk, m.tf_layout, (int32_t)n};
  p->batch = batch;
  p->heads = heads;
  p->head_dim = head_dim;
  p->dtype = dtype;
  p->flags = flags;
  p->scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  block_sizes(dtype, head_dim, &p->block_q, &p->block_k);
  p->n_qblocks = n_query_blocks(p->g, p->block_q);
  p->n_ktiles = n_key_tiles(p->g, p->block_k);
  const int64_t grid = (int64_t)batch * heads * p->n_qblocks;
  if (grid >= (int64_t(1) << 31)) {
    delete p;
    return fail(ATTN_JVP_E_OVERFLOW, "grid of %lld workgroups does not fit", (long long)grid);
  }
  p->allowed_pairs = count_pairs(p->g);
  int64_t visited = 0;
  for (int32_t qb = 0; qb < p->n_qblocks; ++qb) {
    int32_t r0, r1;
    qblock_rows(p->g, p->block_q, qb, &r0, &r1);
    visited += span_count(block_tiles(block_ranges(p->g, r0, r1), p->block_k));
  }
  p->visited_tiles = visited;
  p->useful_flops = count_flops(p->g, head_dim, (flags & ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO) != 0) * batch * heads;
  bwd_block_sizes(dtype, head_dim, &p->bwd_block_q, &p->bwd_block_kv);
  p->bwd_n_qblocks = n_query_blocks(p->g, p->bwd_block_q);
  p->bwd_n_kblocks = n_query_blocks(p->g, p->bwd_block_kv);  // key blocks are cut per side too
  p->bwd_useful_flops = 10 * p->allowed_pairs * head_dim * batch * heads;
  if ((int64_t)batch * heads * (p->bwd_n_qblocks > p->bwd_n_kblocks ? p->bwd_n_qblocks : p->bwd_n_kblocks) >=
      (int64_t(1) << 31)) {
    delete p;
    return fail(ATTN_JVP_E_OVERFLOW, "backward grid does not fit");
  }
  *out = p;
  return ok();
}

int attn_jvp_create_ranges(attn_jvp_plan** out, int32_t n_tokens, int32_t n_groups,
                           const attn_jvp_query_group* groups, int32_t n_intervals, const int32_t* intervals,
                           int32_t batch, int32_t heads, int32_t head_dim, int32_t dtype, float softmax_scale) {
  if (out == nullptr) return fail(ATTN_JVP_E_NULL, "out must be non-NULL");
  *out = nullptr;
  if (n_groups > 0 && groups == nullptr) return fail(ATTN_JVP_E_NULL, "groups is NULL");
  if (n_intervals > 0 && intervals == nullptr) return fail(ATTN_JVP_E_NULL, "intervals is NULL");
  if (n_tokens < 1) return fail(ATTN_JVP_E_INVALID, "n_tokens must be >= 1 (got %d)", n_tokens);
  if (n_groups < 0 || n_intervals < 0) return fail(ATTN_JVP_E_INVALID, "n_groups and n_intervals must be >= 0");
  if (batch < 1 || heads < 1) return fail(ATTN_JVP_E_INVALID, "batch and heads must be >= 1 (got %d, %d)", batch, heads);
  if (head_dim != 64 && head_dim != 128) return fail(ATTN_JVP_E_INVALID, "head_dim must be 64 or 128 (got %d)", head_dim);
  if (dtype != ATTN_JVP_BF16 && dtype != ATTN_JVP_FP32) return fail(ATTN_JVP_E_INVALID, "unknown dtype %d", dtype);
  if (!std::isfinite(softmax_scale)) return fail(ATTN_JVP_E_INVALID, "softmax_scale must be finite");
  const int64_t n = n_tokens;
  const int64_t per_head = n * head_dim * (dtype == ATTN_JVP_BF16 ? 2 : 1);
  if (per_head >= (int64_t(1) << 31))
    return fail(ATTN_JVP_E_OVERFLOW, "sequence of %lld tokens x d=%d exceeds the per-head limit (2^31 %s)",
                (long long)n, head_dim, dtype == ATTN_JVP_BF16 ? "bytes" : "elements");

  // Validate and normalise the groups: sorted, disjoint query intervals;
  // each group's key intervals sorted and merged (empty ones dropped).
  std::vector<int32_t> g_lo(n_groups), g_hi(n_groups), g_iv(n_groups + 1, 0), ivs;
  for (int32_t g = 0; g < n_groups; ++g) {
    const attn_jvp_query_group& q = groups[g];
    if (q.row_lo < 0 || q.row_lo >= q.row_hi || q.row_hi > n_tokens)
      return fail(ATTN_JVP_E_INVALID, "group %d: rows [%d, %d) not a non-empty part of [0, %d)", g, q.row_lo,
                  q.row_hi, n_tokens);
    if (g > 0 && q.row_lo < g_hi[g - 1])
      return fail(ATTN_JVP_E_INVALID, "group %d: rows start at %d, before the end of group %d (%d); groups must be "
                  "sorted and disjoint", g, q.row_lo, g - 1, g_hi[g - 1]);
    if (q.key_begin < 0 || q.key_begin > q.key_end || q.key_end > n_intervals)
      return fail(ATTN_JVP_E_INVALID, "group %d: intervals [%d, %d) outside [0, %d)", g, q.key_begin, q.key_end,
                  n_intervals);
    std::vector<std::pair<int32_t, int32_t>> kv;
    for (int32_t k = q.key_begin; k < q.key_end; ++k) {
      const int32_t lo = intervals[2 * k], hi = intervals[2 * k + 1];
      if (lo < 0 || hi < lo || hi > n_tokens)
        return fail(ATTN_JVP_E_INVALID, "group %d: key interval [%d, %d) not inside [0, %d)", g, lo, hi, n_tokens);
      if (lo < hi) kv.emplace_back(lo, hi);
    }
    std::sort(kv.begin(), kv.end());
    std::vector<std::pair<int32_t, int32_t>> merged;
    for (const auto& iv : kv) {
      if (!merged.empty() && iv.first <= merged.back().second) merged.back().second = std::max(merged.back().second, iv.second);
      else merged.push_back(iv);
    }
    if (merged.size() > 255)
      return fail(ATTN_JVP_E_INVALID, "group %d has %zu key intervals after merging; at most 255", g, merged.size());
    g_lo[g] = q.row_lo;
    g_hi[g] = q.row_hi;
    for (const auto& iv : merged) {
      ivs.push_back(iv.first);
      ivs.push_back(iv.second);
    }
    g_iv[g + 1] = (int32_t)(ivs.size() / 2);
    if (g_iv[g + 1] >= (1 << 23)) return fail(ATTN_JVP_E_OVERFLOW, "more than 2^23 key intervals");
  }

  attn_jvp_plan* p = new (std::nothrow) attn_jvp_plan;
  RangeSchedule* rs = p ? new (std::nothrow) RangeSchedule : nullptr;
  if (rs == nullptr) {
    delete p;
    return fail(ATTN_JVP_E_NOMEM, "plan allocation failed");
  }
  p->rs = rs;
  p->g = MaskGeom{n_tokens, n_tokens, 0, n_tokens};  // only seq_len is used by range plans
  p->batch = batch;
  p->heads = heads;
  p->head_dim = head_dim;
  p->dtype = dtype;
  p->flags = 0;
  p->scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)head_dim);
  block_sizes(dtype, head_dim, &p->block_q, &p->block_k);
  const int32_t bq = p->block_q, bk = p->block_k;
  p->n_qblocks = cdiv(n_tokens, bq);
  p->n_ktiles = cdiv(n_tokens, bk);
  if ((int64_t)batch * heads * p->n_qblocks >= (int64_t(1) << 31)) {
    delete rs;
    delete p;
    return fail(ATTN_JVP_E_OVERFLOW, "grid does not fit");
  }

  try {
    std::vector<int32_t> row_group(n_tokens, -1);
    int64_t pairs = 0;
    for (int32_t g = 0; g < n_groups; ++g) {
      int64_t keys = 0;
      for (int32_t k = g_iv[g]; k < g_iv[g + 1]; ++k) keys += ivs[2 * k + 1] - ivs[2 * k];
      pairs += keys * (g_hi[g] - g_lo[g]);
      for (int32_t r = g_lo[g]; r < g_hi[g]; ++r) row_group[r] = g;
    }
    SideSchedule qs;
    build_side(n_tokens, row_group, g_iv, ivs, bq, bk, &qs);
    rs->max_entries = qs.max_entries;
    if (dtype == ATTN_JVP_BF16 && rs->max_entries > kMaxTableEntries) {
      const int32_t me = rs->max_entries;
      delete rs;
      delete p;
      return fail(ATTN_JVP_E_OVERFLOW, "a query block streams %d key tiles; range-list plans allow at most %d", me,
                  kMaxTableEntries);
    }
    rs->n_entries = (int32_t)qs.ent.size();
    const int32_t n_iv = (int32_t)(ivs.size() / 2);

    // the columns, for the backward's dk/dv kernel
    bwd_block_sizes(dtype, head_dim, &p->bwd_block_q, &p->bwd_block_kv);
    std::vector<int32_t> col_grp, c_iv, civs;
    int32_t max_col = 0;
    SideSchedule ks;
    if (!build_columns(n_tokens, g_lo, g_hi, g_iv, ivs, &col_grp, &c_iv, &civs, &max_col)) {
      rs->bwd_error = "the columns of the mask need more than 2^23 row intervals";
    } else if (max_col > 255) {
      rs->bwd_error = "some key is seen by " + std::to_string(max_col) + " separate row intervals; at most 255";
    } else {
      build_side(n_tokens, col_grp, c_iv, civs, p->bwd_block_kv, 32, &ks);
      if (dtype == ATTN_JVP_BF16 && ks.max_entries > kMaxTableEntries)
        rs->bwd_error = "a key block streams " + std::to_string(ks.max_entries) +
                        " query tiles; the backward allows at most " + std::to_string(kMaxTableEntries);
    }
    if (!rs->bwd_error.empty()) {
      ks = SideSchedule{};
      ks.blk.assign(1, 0);
      civs.clear();
      col_grp.assign(n_tokens, -1);
    }
    rs->n_kblocks = (int32_t)ks.order.size();
    rs->n_col_entries = (int32_t)ks.ent.size();

    std::vector<int32_t>& tb = rs->table;
    tb.assign(8, 0);
    tb[0] = kTableMagic;
    tb[1] = p->n_qblocks;
    tb[2] = rs->n_entries;
    tb[3] = n_iv;
    tb[4] = rs->max_entries;
    tb[5] = rs->n_kblocks;
    tb[6] = rs->n_col_entries;
    tb[7] = (int32_t)(civs.size() / 2);
    auto put = [&](int64_t* off, const std::vector<int32_t>& v) {
      *off = (int64_t)tb.size();
      tb.insert(tb.end(), v.begin(), v.end());
    };
    put(&rs->off_blk, qs.blk);
    put(&rs->off_order, qs.order);
    put(&rs->off_ent, qs.ent);
    rs->off_rows = (int64_t)tb.size();
    for (int32_t r = 0; r < n_tokens; ++r) {
      const int32_t g = row_group[r];
      const int32_t cnt = g < 0 ? 0 : g_iv[g + 1] - g_iv[g];
      tb.push_back(g < 0 ? 0 : (g_iv[g] << 8) | cnt);
      rs->rows_over_two = rs->rows_over_two || cnt > 2;
    }
    put(&rs->off_iv, ivs);
    put(&rs->off_cblk, ks.blk);
    put(&rs->off_corder, ks.order);
    put(&rs->off_cent, ks.ent);
    rs->off_cols = (int64_t)tb.size();
    for (int32_t j = 0; j < n_tokens; ++j) {
      const int32_t c = col_grp[j];
      const int32_t cnt = c < 0 ? 0 : c_iv[c + 1] - c_iv[c];
      tb.push_back(c < 0 ? 0 : (c_iv[c] << 8) | cnt);
      rs->cols_over_two = rs->cols_over_two || cnt > 2;
    }
    put(&rs->off_civ, civs);
    rs->ent_class = std::move(qs.cls);
    p->allowed_pairs = pairs;
    p->visited_tiles = rs->n_entries;
    p->useful_flops = 12 * pairs * head_dim * batch * heads;
    p->bwd_n_qblocks = p->n_qblocks;  // the dq kernel walks the forward's blocks and tiles
    p->bwd_n_kblocks = cdiv(n_tokens, p->bwd_block_kv);
    p->bwd_useful_flops = 10 * pairs * head_dim * batch * heads;
    if ((int64_t)batch * heads * p->bwd_n_kblocks >= (int64_t(1) << 31)) {
      delete rs;
      delete p;
      return fail(ATTN_JVP_E_OVERFLOW, "backward grid does not fit");
    }
  } catch (const std::bad_alloc&) {
    delete rs;
    delete p;
    return fail(ATTN_JVP_E_NOMEM, "plan tables do not fit in host memory");
  }
  *out = p;
  return ok();
}

int attn_jvp_plan_table_size(const attn_jvp_plan* p, size_t* bytes) {
  if (p == nullptr || bytes == nullptr) return fail(ATTN_JVP_E_NULL, "plan and bytes must be non-NULL");
  *bytes = p->rs ? p->rs->table.size() * sizeof(int32_t) : 0;
  return ok();
}

int attn_jvp_plan_table(const attn_jvp_plan* p, void* host_out, size_t bytes) {
  if (p == nullptr || host_out == nullptr) return fail(ATTN_JVP_E_NULL, "plan and host_out must be non-NULL");
  if (p->rs == nullptr) return fail(ATTN_JVP_E_INVALID, "descriptor plans have no table");
  const size_t need = p->rs->table.size() * sizeof(int32_t);
  if (bytes < need) return fail(ATTN_JVP_E_INVALID, "host_out holds %zu bytes, need %zu", bytes, need);
  std::memcpy(host_out, p->rs->table.data(), need);
  return ok();
}

int attn_jvp_destroy(attn_jvp_plan* p) {
  if (p) delete p->rs;
  delete p;
  return ok();
}

namespace {

// primal: o and lse only; tq, tk, tv and t_o are absent (NULL) and never touched.
int fwd_common(const attn_jvp_plan* p, const void* table, const void* q, const void* k, const void* v,
               const void* tq, const void* tk, const void* tv, void* o, void* t_o, float* lse, void* hip_stream,
               bool primal = false) {
  const void* ins[6] = {q, k, v, tq, tk, tv};
  static const char* names[8] = {"q", "k", "v", "tq", "tk", "tv", "o", "t_o"};
  void* outs[2] = {o, t_o};
  const int n_in = primal ? 3 : 6, n_out = primal ? 1 : 2;
  for (int i = 0; i < n_in; ++i)
    if (ins[i] == nullptr) return fail(ATTN_JVP_E_NULL, "%s is NULL", names[i]);
  for (int i = 0; i < n_out; ++i)
    if (outs[i] == nullptr) return fail(ATTN_JVP_E_NULL, "%s is NULL", names[6 + i]);
  for (int i = 0; i < n_in; ++i)
    if ((uintptr_t)ins[i] % 16) return fail(ATTN_JVP_E_ALIGN, "%s is not 16-byte aligned", names[i]);
  for (int i = 0; i < n_out; ++i)
    if ((uintptr_t)outs[i] % 16) return fail(ATTN_JVP_E_ALIGN, "%s is not 16-byte aligned", names[6 + i]);
  if ((uintptr_t)lse % 4) return fail(ATTN_JVP_E_ALIGN, "lse is not 4-byte aligned");

  const size_t elt = p->dtype == ATTN_JVP_BF16 ? 2 : 4;
  const size_t rows = (size_t)p->batch * p->heads * (size_t)p->g.seq_len;
  const size_t bytes = rows * p->head_dim * elt;
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlaps(outs[i], bytes, ins[j], bytes))
        return fail(ATTN_JVP_E_INVALID, "%s overlaps input %s", names[6 + i], names[j]);
    if (lse && overlaps(lse, rows * 4, outs[i], bytes)) return fail(ATTN_JVP_E_INVALID, "lse overlaps %s", names[6 + i]);
  }
  if (!primal && overlaps(o, bytes, t_o, bytes)) return fail(ATTN_JVP_E_INVALID, "o overlaps t_o");
  if (lse)
    for (int j = 0; j < n_in; ++j)
      if (overlaps(lse, rows * 4, ins[j], bytes)) return fail(ATTN_JVP_E_INVALID, "lse overlaps input %s", names[j]);
  if (table) {
    const size_t tbytes = p->rs->table.size() * sizeof(int32_t);
    for (int i = 0; i < n_out; ++i)
      if (overlaps(outs[i], bytes, table, tbytes)) return fail(ATTN_JVP_E_INVALID, "%s overlaps the table", names[6 + i]);
    if (lse && overlaps(lse, rows * 4, table, tbytes)) return fail(ATTN_JVP_E_INVALID, "lse overlaps the table");
  }

  int dev;
  int st = check_device(&dev);
  if (st != ATTN_JVP_OK) return st;

  FwdParams fp;
  fp.q = q;
  fp.k = k;
  fp.v = v;
  fp.tq = tq;
  fp.tk = tk;
  fp.tv = tv;
  fp.o = o;
  fp.to = t_o;
  fp.lse = lse;
  fp.g = p->g;
  fp.n_qblocks = p->n_qblocks;
  fp.scale = p->scale;
  fp.score_log2 = p->scale * 1.4426950408889634f;
  fp.ctz = (p->flags & ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO) ? 1 : 0;
  fp.primal = 0;
  fp.side = -1;
  if (primal) {  // the clean-tangent-zero kernel with every block in its primal mode
    fp.tq = fp.tk = fp.tv = q;  // never read
    fp.to = nullptr;
    fp.ctz = 1;
    fp.primal = 1;
  }
  fp.tb_blk = fp.tb_order = fp.tb_ent = fp.tb_rows = fp.tb_iv = nullptr;
  fp.tb_max_entries = table ? p->rs->max_entries : 0;
  if (table) {
    const int32_t* t = (const int32_t*)table;
    fp.tb_blk = t + p->rs->off_blk;
    fp.tb_order = t + p->rs->off_order;
    fp.tb_ent = t + p->rs->off_ent;
    fp.tb_rows = t + p->rs->off_rows;
    fp.tb_iv = t + p->rs->off_iv;
  }
  st = queue_slot(dev, &fp.queues);
  if (st != ATTN_JVP_OK) return st;
  const int grid = p->batch * p->heads * fp.n_qblocks;
  hipError_t e = launch_fwd(p->dtype, p->head_dim, grid, fp, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(ATTN_JVP_E_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

int attn_jvp_fwd(const attn_jvp_plan* p, const void* q, const void* k, const void* v, const void* tq,
                 const void* tk, const void* tv, void* o, void* t_o, float* lse, void* hip_stream) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
  if (p->rs) return fail(ATTN_JVP_E_INVALID, "range-list plans run through attn_jvp_fwd_table");
  return fwd_common(p, nullptr, q, k, v, tq, tk, tv, o, t_o, lse, hip_stream);
}

int attn_jvp_fwd_primal(const attn_jvp_plan* p, const void* q, const void* k, const void* v, void* o, float* lse,
                        void* hip_stream) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
  if (p->rs) return fail(ATTN_JVP_E_INVALID, "range-list plans run the primal forward through attn_jvp_fwd_primal_table");
  return fwd_common(p, nullptr, q, k, v, nullptr, nullptr, nullptr, o, nullptr, lse, hip_stream, true);
}

int attn_jvp_fwd_primal_table(const attn_jvp_plan* p, const void* device_table, const void* q, const void* k,
                              const void* v, void* o, float* lse, void* hip_stream) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
  if (p->rs == nullptr) return fail(ATTN_JVP_E_INVALID, "descriptor plans have no table: use attn_jvp_fwd_primal");
  if (device_table == nullptr) return fail(ATTN_JVP_E_NULL, "device_table is NULL");
  if ((uintptr_t)device_table % 4) return fail(ATTN_JVP_E_ALIGN, "device_table is not 4-byte aligned");
  return fwd_common(p, device_table, q, k, v, nullptr, nullptr, nullptr, o, nullptr, lse, hip_stream, true);
}

int attn_jvp_fwd_table(const attn_jvp_plan* p, const void* device_table, const void* q, const void* k,
                       const void* v, const void* tq, const void* tk, const void* tv, void* o, void* t_o,
                       float* lse, void* hip_stream) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
  if (p->rs == nullptr) return fail(ATTN_JVP_E_INVALID, "descriptor plans have no table: use attn_jvp_fwd");
  if (device_table == nullptr) return fail(ATTN_JVP_E_NULL, "device_table is NULL");
  if ((uintptr_t)device_table % 4) return fail(ATTN_JVP_E_ALIGN, "device_table is not 4-byte aligned");
  return fwd_common(p, device_table, q, k, v, tq, tk, tv, o, t_o, lse, hip_stream);
}

int attn_jvp_bwd_workspace_size(const attn_jvp_plan* p, size_t* bytes) {
  if (p == nullptr || bytes == nullptr) return fail(ATTN_JVP_E_NULL, "plan and bytes must be non-NULL");
  *bytes = (size_t)p->batch * p->heads * (size_t)p->g.seq_len * 2 * sizeof(float);
  return ok();
}

namespace {

int bwd_common(const attn_jvp_plan* p, const void* table, const void* q, const void* k, const void* v,
               const void* o, const float* lse, const void* d_o, void* dq, void* dk, void* dv, float* workspace,
               void* hip_stream) {
  static const char* names[10] = {"q", "k", "v", "o", "d_o", "lse", "dq", "dk", "dv", "workspace"};
  const void* ins[6] = {q, k, v, o, d_o, lse};
  void* outs[4] = {dq, dk, dv, workspace};
  for (int i = 0; i < 6; ++i)
    if (ins[i] == nullptr) return fail(ATTN_JVP_E_NULL, "%s is NULL", names[i]);
  for (int i = 0; i < 4; ++i)
    if (outs[i] == nullptr) return fail(ATTN_JVP_E_NULL, "%s is NULL", names[6 + i]);
  const size_t elt = p->dtype == ATTN_JVP_BF16 ? 2 : 4;
  const size_t rows = (size_t)p->batch * p->heads * (size_t)p->g.seq_len;
  const size_t tbytes = rows * p->head_dim * elt;
  const size_t in_bytes[6] = {tbytes, tbytes, tbytes, tbytes, tbytes, rows * 4};
  const size_t out_bytes[4] = {tbytes, tbytes, tbytes, rows * 8};
  for (int i = 0; i < 10; ++i) {
    const uintptr_t a = (uintptr_t)(i < 6 ? ins[i] : outs[i - 6]);
    const int need = (i == 5 || i == 9) ? 4 : 16;  // lse and workspace: fp32 rows
    if (a % need) return fail(ATTN_JVP_E_ALIGN, "%s is not %d-byte aligned", names[i], need);
  }
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j]))
        return fail(ATTN_JVP_E_INVALID, "%s overlaps input %s", names[6 + i], names[j]);
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j]))
        return fail(ATTN_JVP_E_INVALID, "%s overlaps %s", names[6 + i], names[6 + j]);
    if (table && overlaps(outs[i], out_bytes[i], table, p->rs->table.size() * sizeof(int32_t)))
      return fail(ATTN_JVP_E_INVALID, "%s overlaps the table", names[6 + i]);
  }

  int dev;
  int st = check_device(&dev);
  if (st != ATTN_JVP_OK) return st;

  BwdParams bp;
  bp.q = q;
  bp.k = k;
  bp.v = v;
  bp.o = o;
  bp.dout = d_o;
  bp.lse = lse;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.ws = workspace;
  bp.g = p->g;
  bp.n_qblocks = p->bwd_n_qblocks;
  bp.n_kblocks = p->bwd_n_kblocks;
  bp.scale = p->scale;
  bp.score_log2 = p->scale * 1.4426950408889634f;
  bp.tb_blk = bp.tb_order = bp.tb_ent = bp.tb_rows = bp.tb_iv = nullptr;
  bp.cb_blk = bp.cb_order = bp.cb_ent = bp.cb_cols = bp.cb_iv = nullptr;
  if (table) {
    const int32_t* t = (const int32_t*)table;
    const RangeSchedule& rs = *p->rs;
    bp.tb_blk = t + rs.off_blk;
    bp.tb_order = t + rs.off_order;
    bp.tb_ent = t + rs.off_ent;
    bp.tb_rows = t + rs.off_rows;
    bp.tb_iv = t + rs.off_iv;
    bp.cb_blk = t + rs.off_cblk;
    bp.cb_order = t + rs.off_corder;
    bp.cb_ent = t + rs.off_cent;
    bp.cb_cols = t + rs.off_cols;
    bp.cb_iv = t + rs.off_civ;
  }
  bp.n_slices = p->batch * p->heads;
  st = queue_slot(dev, &bp.queues);
  if (st != ATTN_JVP_OK) return st;
  hipError_t e = launch_bwd(p->dtype, p->head_dim, p->batch * p->heads, bp, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(ATTN_JVP_E_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

int attn_jvp_bwd(const attn_jvp_plan* p, const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* d_o, void* dq, void* dk, void* dv, float* workspace,
                 void* hip_stream) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
  if (p->rs) return fail(ATTN_JVP_E_INVALID, "range-list plans run the backward through attn_jvp_bwd_table");
  return bwd_common(p, nullptr, q, k, v, o, lse, d_o, dq, dk, dv, workspace, hip_stream);
}

int attn_jvp_bwd_noalloc(const attn_jvp_plan* p, const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* d_o, void* dq, void* dk, void* dv, void* hip_stream) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
  if (p->rs) return fail(ATTN_JVP_E_INVALID, "range-list plans run the backward through attn_jvp_bwd_table");
  static const char* names[9] = {"q", "k", "v", "o", "lse", "d_o", "dq", "dk", "dv"};
  const void* args[9] = {q, k, v, o, lse, d_o, dq, dk, dv};
  for (int i = 0; i < 9; ++i)
    if (args[i] == nullptr) return fail(ATTN_JVP_E_NULL, "%s is NULL", names[i]);
  const size_t need = (size_t)p->batch * p->heads * (size_t)p->g.seq_len * 2 * sizeof(float);
  if (need > kScratchBytes)
    return fail(ATTN_JVP_E_OVERFLOW, "attn_jvp_bwd_noalloc needs %zu workspace bytes (8 B H N), above its fixed %zu "
                "(B H N <= %zu); use attn_jvp_bwd with a caller workspace", need, kScratchBytes,
                kScratchBytes / 8);
  int dev;
  int st = check_device(&dev);
  if (st != ATTN_JVP_OK) return st;
  void* ws = nullptr;
  st = scratch_address(dev, &ws);
  if (st != ATTN_JVP_OK) return st;
  return bwd_common(p, nullptr, q, k, v, o, lse, d_o, dq, dk, dv, (float*)ws, hip_stream);
}

int attn_jvp_bwd_table(const attn_jvp_plan* p, const void* device_table, const void* q, const void* k,
                       const void* v, const void* o, const float* lse, const void* d_o, void* dq, void* dk,
                       void* dv, float* workspace, void* hip_stream) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
  if (p->rs == nullptr) return fail(ATTN_JVP_E_INVALID, "descriptor plans have no table: use attn_jvp_bwd");
  if (!p->rs->bwd_error.empty()) return fail(ATTN_JVP_E_INVALID, "no backward for this plan: %s", p->rs->bwd_error.c_str());
  if (device_table == nullptr) return fail(ATTN_JVP_E_NULL, "device_table is NULL");
  if ((uintptr_t)device_table % 4) return fail(ATTN_JVP_E_ALIGN, "device_table is not 4-byte aligned");
  return bwd_common(p, device_table, q, k, v, o, lse, d_o, dq, dk, dv, workspace, hip_stream);
}

int attn_jvp_plan_bwd_info(const attn_jvp_plan* p, int32_t* block_q, int32_t* block_kv, int32_t* n_query_blocks,
                           int32_t* n_key_blocks) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
  if (block_q) *block_q = p->bwd_block_q;
  if (block_kv) *block_kv = p->bwd_block_kv;
  if (n_query_blocks) *n_query_blocks = p->bwd_n_qblocks;
  if (n_key_blocks) *n_key_blocks = p->bwd_n_kblocks;
  return ok();
}

int attn_jvp_plan_bwd_flops(const attn_jvp_plan* p, int64_t* useful_flops) {
  if (p == nullptr || useful_flops == nullptr) return fail(ATTN_JVP_E_NULL, "plan and useful_flops must be non-NULL");
  *useful_flops = p->bwd_useful_flops;
  return ok();
}

int attn_jvp_key_ranges(const attn_jvp_plan* p, int32_t* out, size_t n) {
  if (p == nullptr || out == nullptr) return fail(ATTN_JVP_E_NULL, "plan and host_out must be non-NULL");
  if (n < (size_t)p->g.seq_len * 4)
    return fail(ATTN_JVP_E_INVALID, "host_out holds %zu int32, need %zu", n, (size_t)p->g.seq_len * 4);
  if (p->rs) {
    if (!p->rs->bwd_error.empty()) return fail(ATTN_JVP_E_INVALID, "no backward for this plan: %s", p->rs->bwd_error.c_str());
    if (p->rs->cols_over_two) return fail(ATTN_JVP_E_INVALID, "some key is seen by more than two row intervals");
    const int32_t* cols = p->rs->table.data() + p->rs->off_cols;
    const int32_t* iv = p->rs->table.data() + p->rs->off_civ;
    for (int32_t j = 0; j < p->g.seq_len; ++j) {
      const int32_t off = cols[j] >> 8, cnt = cols[j] & 255;
      out[4 * j + 0] = cnt >= 1 ? iv[2 * off] : 0;
      out[4 * j + 1] = cnt >= 1 ? iv[2 * off + 1] : 0;
      out[4 * j + 2] = cnt >= 2 ? iv[2 * off + 2] : 0;
      out[4 * j + 3] = cnt >= 2 ? iv[2 * off + 3] : 0;
    }
    return ok();
  }
  for (int32_t j = 0; j < p->g.seq_len; ++j) {
    const Ranges r = col_ranges(p->g, j);
    out[4 * j + 0] = r.lo1;
    out[4 * j + 1] = r.hi1;
    out[4 * j + 2] = r.lo2;
    out[4 * j + 3] = r.hi2;
  }
  return ok();
}

const char* attn_jvp_error_string(int code) {
  switch (code) {
    case ATTN_JVP_OK: return "ok";
    case ATTN_JVP_E_INVALID: return "invalid argument";
    case ATTN_JVP_E_NULL: return "null pointer";
    case ATTN_JVP_E_ALIGN: return "misaligned pointer";
    case ATTN_JVP_E_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
    case ATTN_JVP_E_HIP: return "HIP runtime error";
    case ATTN_JVP_E_NOMEM: return "out of host memory";
    case ATTN_JVP_E_OVERFLOW: return "size overflow";
    default: return "unknown error code";
  }
}

const char* attn_jvp_last_error_detail(void) { return g_detail.c_str(); }

int attn_jvp_plan_info(const attn_jvp_plan* p, int64_t* seq_len, int32_t* block_q, int32_t* block_k,
                       int32_t* n_qblocks, int32_t* n_ktiles, int64_t* allowed_pairs, int64_t* visited_tiles) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
  if (seq_len) *seq_len = p->g.seq_len;
  if (block_q) *block_q = p->block_q;
  if (block_k) *block_k = p->block_k;
  if (n_qblocks) *n_qblocks = p->n_qblocks;
  if (n_ktiles) *n_ktiles = p->n_ktiles;
  if (allowed_pairs) *allowed_pairs = p->allowed_pairs;
  if (visited_tiles) *visited_tiles = p->visited_tiles;
  return ok();
}

int attn_jvp_plan_flops(const attn_jvp_plan* p, int64_t* useful_flops) {
  if (p == nullptr || useful_flops == nullptr) return fail(ATTN_JVP_E_NULL, "plan and useful_flops must be non-NULL");
  *useful_flops = p->useful_flops;
  return ok();
}

int attn_jvp_launch_order(const attn_jvp_plan* p, int32_t* out, size_t n) {
  if (p == nullptr || out == nullptr) return fail(ATTN_JVP_E_NULL, "plan and host_out must be non-NULL");
  if (n < (size_t)p->n_qblocks)
    return fail(ATTN_JVP_E_INVALID, "host_out holds %zu int32, need %d", n, p->n_qblocks);
  if (p->rs) {
    std::memcpy(out, p->rs->table.data() + p->rs->off_order, sizeof(int32_t) * p->n_qblocks);
    return ok();
  }
  if ((p->flags & ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO) && p->dtype == ATTN_JVP_BF16) {
    // two launches: the clean side's blocks, then the noisy side's, each heavy first
    const int32_t nbs = p->n_qblocks / 2;
    for (int32_t t = 0; t < p->n_qblocks; ++t) out[t] = (t < nbs ? 0 : nbs) + nbs - 1 - (t < nbs ? t : t - nbs);
    return ok();
  }
  const bool balanced = (p->flags & ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO) != 0;
  for (int32_t t = 0; t < p->n_qblocks; ++t) out[t] = heavy_first_qblock(p->g, p->block_q, t, balanced);
  return ok();
}

int attn_jvp_bwd_launch_order(const attn_jvp_plan* p, int32_t* out, size_t n) {
  if (p == nullptr || out == nullptr) return fail(ATTN_JVP_E_NULL, "plan and host_out must be non-NULL");
  if (p->rs && !p->rs->bwd_error.empty())
    return fail(ATTN_JVP_E_INVALID, "no backward for this plan: %s", p->rs->bwd_error.c_str());
  const int64_t total = (int64_t)p->batch * p->heads * p->bwd_n_kblocks;
  if (n < (size_t)total) return fail(ATTN_JVP_E_INVALID, "host_out holds %zu int32, need %lld", n, (long long)total);
  const int32_t nkb = p->bwd_n_kblocks;
  for (int32_t b = 0; b < (int32_t)total; ++b) {
    const int32_t task = launch_task(b, (int32_t)total, nkb, kDkdvXcdGroup);
    if (p->rs) {  // range-list plans: the table's heavy-first key-block order within each (b, h)
      const int32_t bh = task / nkb;
      out[b] = bh * nkb + p->rs->table[p->rs->off_corder + (task - bh * nkb)];
    } else {
      out[b] = task;
    }
  }
  return ok();
}

int attn_jvp_row_ranges(const attn_jvp_plan* p, int32_t* out, size_t n) {
  if (p == nullptr || out == nullptr) return fail(ATTN_JVP_E_NULL, "plan and host_out must be non-NULL");
  if (n < (size_t)p->g.seq_len * 4)
    return fail(ATTN_JVP_E_INVALID, "host_out holds %zu int32, need %zu", n, (size_t)p->g.seq_len * 4);
  if (p->rs) {
    if (p->rs->rows_over_two) return fail(ATTN_JVP_E_INVALID, "some row has more than two key intervals");
    const int32_t* rows = p->rs->table.data() + p->rs->off_rows;
    const int32_t* iv = p->rs->table.data() + p->rs->off_iv;
    for (int32_t i = 0; i < p->g.seq_len; ++i) {
      const int32_t off = rows[i] >> 8, cnt = rows[i] & 255;
      out[4 * i + 0] = cnt >= 1 ? iv[2 * off] : 0;
      out[4 * i + 1] = cnt >= 1 ? iv[2 * off + 1] : 0;
      out[4 * i + 2] = cnt >= 2 ? iv[2 * off + 2] : 0;
      out[4 * i + 3] = cnt >= 2 ? iv[2 * off + 3] : 0;
    }
    return ok();
  }
  for (int32_t i = 0; i < p->g.seq_len; ++i) {
    const Ranges r = row_ranges(p->g, i);
    out[4 * i + 0] = r.lo1;
    out[4 * i + 1] = r.hi1;
    out[4 * i + 2] = r.lo2;
    out[4 * i + 3] = r.hi2;
  }
  return ok();
}

int attn_jvp_tile_map(const attn_jvp_plan* p, uint8_t* out, size_t n) {
  if (p == nullptr || out == nullptr) return fail(ATTN_JVP_E_NULL, "plan and host_out must be non-NULL");
  const size_t need = (size_t)p->n_qblocks * p->n_ktiles;
  if (n < need) return fail(ATTN_JVP_E_INVALID, "host_out holds %zu bytes, need %zu", n, need);
  std::memset(out, 0, need);
  if (p->rs) {
    const int32_t* blk = p->rs->table.data() + p->rs->off_blk;
    const int32_t* ent = p->rs->table.data() + p->rs->off_ent;
    for (int32_t qb = 0; qb < p->n_qblocks; ++qb)
      for (int32_t e = blk[qb]; e < blk[qb + 1]; ++e) out[(size_t)qb * p->n_ktiles + (ent[e] & 0xffffff)] = p->rs->ent_class[e];
    return ok();
  }
  for (int32_t qb = 0; qb < p->n_qblocks; ++qb) {
    int32_t r0, r1;
    qblock_rows(p->g, p->block_q, qb, &r0, &r1);
    const TileSpans sp = block_tiles(block_ranges(p->g, r0, r1), p->block_k);
    uint8_t* row = out + (size_t)qb * p->n_ktiles;
    for (int32_t it = 0, nt = span_count(sp); it < nt; ++it) row[span_tile(sp, it)] = 1;
    for (int32_t kt = 0; kt < p->n_ktiles; ++kt) {
      const int32_t k0 = kt * p->block_k;
      const int32_t k1 = k0 + p->block_k < p->g.seq_len ? k0 + p->block_k : p->g.seq_len;
      const int cls = tile_class(p->g, r0, r1, k0, k1);
      if (row[kt]) row[kt] = cls == 0 ? 3 : (uint8_t)cls;
      else row[kt] = cls == 0 ? 0 : 4;
    }
  }
  return ok();
}

int attn_jvp_clock_sample(void* device_out, void* stream) {
  if (device_out == nullptr) return fail(ATTN_JVP_E_NULL, "device_out must be non-NULL");
  if ((uintptr_t)device_out % 8 != 0) return fail(ATTN_JVP_E_ALIGN, "device_out must be 8-byte aligned");
  int dev = -1;
  const int st = check_device(&dev);
  if (st != ATTN_JVP_OK) return st;
  hipLaunchKernelGGL(clock_sample_kernel, dim3(kClockSampleGroups), dim3(64), 0, (hipStream_t)stream,
                     (uint64_t*)device_out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ATTN_JVP_E_HIP, "clock sample launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
