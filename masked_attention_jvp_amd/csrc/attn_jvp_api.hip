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
#include <new>
#include <string>

#include "attn_jvp.h"
#include "attn_jvp_launch.h"
#include "mask_index.h"

using namespace attn_jvp;

struct attn_jvp_plan {
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

}  // namespace

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

int attn_jvp_destroy(attn_jvp_plan* p) {
  delete p;
  return ok();
}

int attn_jvp_fwd(const attn_jvp_plan* p, const void* q, const void* k, const void* v, const void* tq,
                 const void* tk, const void* tv, void* o, void* t_o, float* lse, void* hip_stream) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
  const void* ins[6] = {q, k, v, tq, tk, tv};
  static const char* names[8] = {"q", "k", "v", "tq", "tk", "tv", "o", "t_o"};
  void* outs[2] = {o, t_o};
  for (int i = 0; i < 6; ++i)
    if (ins[i] == nullptr) return fail(ATTN_JVP_E_NULL, "%s is NULL", names[i]);
  for (int i = 0; i < 2; ++i)
    if (outs[i] == nullptr) return fail(ATTN_JVP_E_NULL, "%s is NULL", names[6 + i]);
  for (int i = 0; i < 6; ++i)
    if ((uintptr_t)ins[i] % 16) return fail(ATTN_JVP_E_ALIGN, "%s is not 16-byte aligned", names[i]);
  for (int i = 0; i < 2; ++i)
    if ((uintptr_t)outs[i] % 16) return fail(ATTN_JVP_E_ALIGN, "%s is not 16-byte aligned", names[6 + i]);
  if ((uintptr_t)lse % 4) return fail(ATTN_JVP_E_ALIGN, "lse is not 4-byte aligned");

  const size_t elt = p->dtype == ATTN_JVP_BF16 ? 2 : 4;
  const size_t rows = (size_t)p->batch * p->heads * (size_t)p->g.seq_len;
  const size_t bytes = rows * p->head_dim * elt;
  for (int i = 0; i < 2; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], bytes, ins[j], bytes))
        return fail(ATTN_JVP_E_INVALID, "%s overlaps input %s", names[6 + i], names[j]);
    if (lse && overlaps(lse, rows * 4, outs[i], bytes)) return fail(ATTN_JVP_E_INVALID, "lse overlaps %s", names[6 + i]);
  }
  if (overlaps(o, bytes, t_o, bytes)) return fail(ATTN_JVP_E_INVALID, "o overlaps t_o");
  if (lse)
    for (int j = 0; j < 6; ++j)
      if (overlaps(lse, rows * 4, ins[j], bytes)) return fail(ATTN_JVP_E_INVALID, "lse overlaps input %s", names[j]);

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
  const int grid = p->batch * p->heads * p->n_qblocks;
  hipError_t e = launch_fwd(p->dtype, p->head_dim, grid, fp, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(ATTN_JVP_E_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int attn_jvp_bwd_workspace_size(const attn_jvp_plan* p, size_t* bytes) {
  if (p == nullptr || bytes == nullptr) return fail(ATTN_JVP_E_NULL, "plan and bytes must be non-NULL");
  *bytes = (size_t)p->batch * p->heads * (size_t)p->g.seq_len * 2 * sizeof(float);
  return ok();
}

int attn_jvp_bwd(const attn_jvp_plan* p, const void* q, const void* k, const void* v, const void* o,
                 const float* lse, const void* d_o, void* dq, void* dk, void* dv, float* workspace,
                 void* hip_stream) {
  if (p == nullptr) return fail(ATTN_JVP_E_NULL, "plan is NULL");
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
  hipError_t e = launch_bwd(p->dtype, p->head_dim, p->batch * p->heads, bp, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(ATTN_JVP_E_HIP, "kernel launch: %s", hipGetErrorString(e));
  return ok();
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
  const bool balanced = (p->flags & ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO) != 0;
  for (int32_t t = 0; t < p->n_qblocks; ++t) out[t] = heavy_first_qblock(p->g, p->block_q, t, balanced);
  return ok();
}

int attn_jvp_bwd_launch_order(const attn_jvp_plan* p, int32_t* out, size_t n) {
  if (p == nullptr || out == nullptr) return fail(ATTN_JVP_E_NULL, "plan and host_out must be non-NULL");
  const int64_t total = (int64_t)p->batch * p->heads * p->bwd_n_kblocks;
  if (n < (size_t)total) return fail(ATTN_JVP_E_INVALID, "host_out holds %zu int32, need %lld", n, (long long)total);
  for (int32_t b = 0; b < (int32_t)total; ++b) out[b] = xcd_grouped(b, (int32_t)total, kDkdvXcdGroup);
  return ok();
}

int attn_jvp_row_ranges(const attn_jvp_plan* p, int32_t* out, size_t n) {
  if (p == nullptr || out == nullptr) return fail(ATTN_JVP_E_NULL, "plan and host_out must be non-NULL");
  if (n < (size_t)p->g.seq_len * 4)
    return fail(ATTN_JVP_E_INVALID, "host_out holds %zu int32, need %zu", n, (size_t)p->g.seq_len * 4);
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

}  // extern "C"
