/*
 * attn_jvp.h -- C ABI of the fused block-causal / teacher-forcing masked
 * attention forward + forward-mode JVP for AMD Instinct MI355X (gfx950).
 *
 * The operation (Causal-rCM, arXiv 2606.25473, Appendix B, eqs. 42-45):
 * for every batch b, head h and query row i,
 *
 *   s_ij  = scale * q_i . k_j,          ts_ij = scale * (tq_i . k_j + q_i . tk_j)
 *   p_ij  = softmax over the keys j that the mask allows (0 for masked keys)
 *   o_i   = sum_j p_ij v_j
 *   to_i  = sum_j p_ij (ts_ij - sum_k p_ik ts_ik) v_j + sum_j p_ij tv_j
 *   lse_i = log sum_j exp(s_ij)          (natural log, over allowed keys)
 *
 * i.e. o and its directional derivative along (tq, tk, tv) with the mask
 * held fixed (Appendix B: the mask is a discrete routing object without a
 * tangent).  The mask comes from four integers (section 2.3, section 3.1.1
 * eq. 8, section 4 chunking):
 *
 *   T_f = tokens_per_frame, F = n_frames, c = frames_per_chunk,
 *   T = T_f * c tokens per chunk, N_h = T_f * F tokens per side.
 *   tf_layout = 0: plain block-causal sequence of N = N_h tokens; token i
 *                  sees every token of its own chunk and of earlier chunks.
 *   tf_layout = 1: teacher-forcing packed sequence [clean | noisy] of
 *                  N = 2 N_h tokens.  Clean tokens are block-causal among
 *                  themselves and never see noisy tokens; a noisy token of
 *                  chunk k sees the clean tokens of chunks < k and the noisy
 *                  tokens of chunk k.
 *
 * Layout: q, k, v, tq, tk, tv, o, to are contiguous [B, H, N, d] arrays
 * (d innermost) in one element type: bf16 (ATTN_JVP_BF16, bf16 matrix-core
 * products with fp32 accumulation, outputs rounded to nearest even) or fp32
 * (ATTN_JVP_FP32, fp32 arithmetic throughout).  lse is [B, H, N] fp32.
 * All device pointers must be 16-byte aligned (lse: 4-byte).
 *
 * Ownership: the caller owns every buffer.  A plan owns host memory only; the
 * library never allocates device memory and never synchronises.  It holds two
 * fixed arrays per GPU for the process's lifetime: the workspace of
 * attn_jvp_bwd_noalloc and the bf16 kernels' work queues, a ring of 256
 * slots of 64 bytes that the calls on a GPU take in turn (each call's
 * workgroups take their tasks from its slot, which is zero again when the
 * call's kernels have run).  So at most 256 calls of this library may run at
 * the same time on one GPU (on several streams); calls ordered on one stream
 * are never limited.  attn_jvp_fwd only enqueues work on the given stream;
 * buffers must stay valid until the stream reaches that point.  Outputs must
 * not overlap inputs.  A plan is immutable after creation and may be used
 * from several threads and streams.
 *
 * Errors: every function returns ATTN_JVP_OK or an error code and never
 * throws.  Argument errors are detected before any device work is enqueued.
 * Faults inside the kernel surface at the caller's next synchronisation.
 * attn_jvp_last_error_detail() returns a thread-local description of the
 * last error raised on the calling thread.
 */
#ifndef ATTN_JVP_H
#define ATTN_JVP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct attn_jvp_plan attn_jvp_plan;

/* Mask descriptor (see above).  Every field >= 1 except tf_layout in {0, 1};
 * n_frames must be a multiple of frames_per_chunk (all chunks equal). */
typedef struct {
  int32_t tokens_per_frame;
  int32_t n_frames;
  int32_t frames_per_chunk;
  int32_t tf_layout;
} attn_jvp_mask_desc;

enum { ATTN_JVP_BF16 = 0, ATTN_JVP_FP32 = 1 };

enum {
  ATTN_JVP_OK = 0,
  ATTN_JVP_E_INVALID = 1,            /* bad descriptor, size, dtype, head_dim or scale; aliasing */
  ATTN_JVP_E_NULL = 2,               /* a required pointer is NULL */
  ATTN_JVP_E_ALIGN = 3,              /* a pointer is not aligned as required */
  ATTN_JVP_E_UNSUPPORTED_DEVICE = 4, /* the current HIP device is not gfx950 */
  ATTN_JVP_E_HIP = 5,                /* a HIP runtime call failed (detail has the HIP error text) */
  ATTN_JVP_E_NOMEM = 6,              /* host allocation failed */
  ATTN_JVP_E_OVERFLOW = 7            /* N >= 2^31, N*d >= 2^30 (bf16) or 2^31 (fp32), or the grid does not fit */
};

/* Plan flags (attn_jvp_create_ex).
 *
 * ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO (tf_layout = 1 only): the clean half of
 * the sequence carries no tangent, as in teacher-forcing sCM, where the JVP
 * runs through the same packed teacher-forcing mask and the clean context's
 * tangent is zero while only the noisy tokens move (Causal-rCM, section
 * 3.1.2, the text after eq. 17).  The result equals the general operation
 * with tq, tk, tv set to 0 on tokens 0 .. N_h-1, and:
 *   - the clean halves of tq, tk and tv are never read (any contents,
 *     including NaN, are allowed there);
 *   - t_o is exactly 0 on clean rows, which form only o and lse;
 *   - noisy rows against clean keys form ts = scale * tq . k and no p tv
 *     term; noisy rows against noisy keys do the general work.
 * About half the general work on the 21-frame teacher-forcing sequences. */
#define ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO 1u

/* Build a plan for one mask, shape and element type.
 *   out           receives the plan (set to NULL on error)
 *   mask          mask descriptor (read, not kept)
 *   batch, heads  B and H (>= 1)
 *   head_dim      d: 64 or 128
 *   dtype         ATTN_JVP_BF16 or ATTN_JVP_FP32
 *   softmax_scale scale applied to scores and score tangents;
 *                 <= 0 selects 1/sqrt(d); must be finite
 * Pure host work: touches no device. */
int attn_jvp_create(attn_jvp_plan** out, const attn_jvp_mask_desc* mask, int32_t batch,
                    int32_t heads, int32_t head_dim, int32_t dtype, float softmax_scale);

/* attn_jvp_create with plan flags (a bitwise OR of ATTN_JVP_FLAG_* values;
 * 0 gives the same plan as attn_jvp_create).  Unknown bits, or
 * ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO with tf_layout = 0, give
 * ATTN_JVP_E_INVALID. */
int attn_jvp_create_ex(attn_jvp_plan** out, const attn_jvp_mask_desc* mask, int32_t batch,
                       int32_t heads, int32_t head_dim, int32_t dtype, float softmax_scale,
                       uint32_t flags);

/* Range-list masks (Causal-rCM, Appendix B, "sparse custom mask
 * representation"): the mask is a set of query groups, each a contiguous
 * interval of query rows with a list of allowed key intervals; a row in no
 * group sees no key (its o and t_o are 0 and its lse is -inf).  This covers
 * dense attention (one group, one key interval), block-causal and
 * teacher-forcing masks with chunks of any size (e.g. an initial chunk of
 * another size, the cA-B patterns of section 4) and understanding /
 * generation layouts (section 4.2.2, Figure 9).
 *
 * Groups are given sorted by row_lo and disjoint; every interval lies in
 * [0, n_tokens).  A group's intervals may come in any order and may overlap
 * or touch: the plan sorts and merges them (at most 255 after merging).
 * Query blocks are cut from row 0 over the whole sequence; each block
 * streams the key tiles that meet the intervals of its rows' groups. */
typedef struct {
  int32_t row_lo, row_hi;      /* query rows [row_lo, row_hi) */
  int32_t key_begin, key_end;  /* the group's key intervals: intervals[2k], intervals[2k+1] (half-open) for
                                  key_begin <= k < key_end */
} attn_jvp_query_group;

/* Build a plan from a range list of n_tokens tokens (arguments as in
 * attn_jvp_create otherwise; no plan flags).  Pure host work: the plan
 * holds, besides its host copy, a schedule table (attn_jvp_plan_table) that
 * the caller places in device memory and passes to attn_jvp_fwd_table.
 * ATTN_JVP_E_OVERFLOW if, in a bf16 plan, one query block streams more than
 * 7680 key tiles (the kernel stages a block's tile list in LDS). */
int attn_jvp_create_ranges(attn_jvp_plan** out, int32_t n_tokens, int32_t n_groups,
                           const attn_jvp_query_group* groups, int32_t n_intervals,
                           const int32_t* intervals, int32_t batch, int32_t heads, int32_t head_dim,
                           int32_t dtype, float softmax_scale);

/* Bytes of a range-list plan's schedule table (0 for descriptor plans). */
int attn_jvp_plan_table_size(const attn_jvp_plan* plan, size_t* bytes);

/* Copy a range-list plan's schedule table (int32 words, independent of the
 * device) to host memory of at least attn_jvp_plan_table_size() bytes.  The
 * caller copies it to device memory it owns, 4-byte aligned, and keeps it
 * there while kernels that use it may run. */
int attn_jvp_plan_table(const attn_jvp_plan* plan, void* host_out, size_t bytes);

/* attn_jvp_fwd for range-list plans: the same operation and arguments, with
 * the plan's schedule table in device memory (bytes from attn_jvp_plan_table
 * of this plan; its contents are not checked).  attn_jvp_fwd refuses range-
 * list plans and this call refuses descriptor plans (ATTN_JVP_E_INVALID).
 * Range-list plans have no clean-tangent-zero option; their forward without
 * tangents is attn_jvp_fwd_primal_table and their backward
 * attn_jvp_bwd_table. */
int attn_jvp_fwd_table(const attn_jvp_plan* plan, const void* device_table, const void* q,
                       const void* k, const void* v, const void* tq, const void* tk, const void* tv,
                       void* o, void* t_o, float* lse, void* hip_stream);

/* Enqueue o, to (and lse when non-NULL) for the plan's shape on `hip_stream`
 * (a hipStream_t; NULL is the null stream), on the current HIP device.
 * Checks pointers, alignment, overlap and the device architecture first. */
int attn_jvp_fwd(const attn_jvp_plan* plan, const void* q, const void* k, const void* v,
                 const void* tq, const void* tk, const void* tv, void* o, void* t_o,
                 float* lse, void* hip_stream);

/* The masked attention alone, without tangents: o (and lse when non-NULL)
 * of the plan's mask, as attn_jvp_fwd computes them (bit-identical), at
 * 4 d useful flops per allowed pair instead of 12 d.  This is the forward
 * that the backward (attn_jvp_bwd) pairs with: together they replace the
 * plain FlashAttention-2 of a student's training step (Causal-rCM, section
 * 3.2.1 and the TF-dCM comparison of section 6).  Descriptor plans; the
 * plan's flags do not matter.  In bf16 it runs a primal-only instance of the
 * forward kernel (K and V tiles only, two workgroups per CU); the per-row
 * arithmetic is the forward's.  Same checks and error codes as attn_jvp_fwd. */
int attn_jvp_fwd_primal(const attn_jvp_plan* plan, const void* q, const void* k, const void* v,
                        void* o, float* lse, void* hip_stream);

/* attn_jvp_fwd_primal for range-list plans, with the plan's schedule table
 * in device memory (as for attn_jvp_fwd_table): o and lse bit-identical to
 * attn_jvp_fwd_table's, at 4 d useful flops per allowed pair.  Refuses
 * descriptor plans, and attn_jvp_fwd_primal refuses range-list plans
 * (ATTN_JVP_E_INVALID).  Same checks and error codes as attn_jvp_fwd_table. */
int attn_jvp_fwd_primal_table(const attn_jvp_plan* plan, const void* device_table, const void* q,
                              const void* k, const void* v, void* o, float* lse, void* hip_stream);

/* Backward of the masked attention (without tangents) on the same plan:
 * the gradients of a loss L with respect to q, k and v given dO = dL/do
 * (Causal-rCM, section 3.2.1: the student's FlashAttention-2 based masked
 * attention trains through it; the mask is held fixed as in the forward).
 * With P the masked softmax of the scaled scores and lse from attn_jvp_fwd:
 *
 *   P_ij    = exp(scale q_i . k_j - lse_i)  on allowed pairs, 0 otherwise
 *   delta_i = sum_d dO_id o_id
 *   dS_ij   = P_ij (dO_i . v_j - delta_i)
 *   dq_i    = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,  dv_j = sum_i P_ij dO_i
 *
 *   q, k, v, o, d_o   [B, H, N, d] inputs in the plan's element type; o and
 *                     lse are the outputs of attn_jvp_fwd for q, k, v (any
 *                     tangents: they do not enter o and lse)
 *   lse               [B, H, N] fp32 (natural log), 4-byte aligned
 *   dq, dk, dv        [B, H, N, d] outputs in the plan's element type
 *                     (bf16: fp32 accumulation, rounded to nearest even)
 *   workspace         attn_jvp_bwd_workspace_size() bytes of device memory,
 *                     4-byte aligned, owned by the caller; its contents on
 *                     entry are ignored.  On completion it holds, per (b, h),
 *                     N floats -delta_i followed by N floats -lse_i log2(e),
 *                     i.e. workspace[(b H + h) 2N + i] = -delta_i.
 * Enqueues two kernels on `hip_stream` (the dq kernel, which also fills the
 * workspace, then the dk/dv kernel).  Their workgroups take tasks through
 * integer atomics on the call's queue slot, but no result is accumulated by
 * atomics and a task's arithmetic does not depend on the workgroup that runs
 * it, so results do not depend on scheduling.  No output may overlap an input or another output.  The plan's
 * flags do not matter here.  Same checks and error codes as attn_jvp_fwd. */
int attn_jvp_bwd(const attn_jvp_plan* plan, const void* q, const void* k, const void* v,
                 const void* o, const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                 float* workspace, void* hip_stream);

/* attn_jvp_bwd for range-list plans: the same operation, arguments and
 * workspace contents, with the plan's schedule table in device memory (the
 * table of attn_jvp_fwd_table, whose column sections this call uses).  o and
 * lse come from attn_jvp_fwd_table; a row in no group (lse = -inf) gets
 * dq = 0, delta = 0 and contributes nothing to dk and dv, and its second
 * workspace entry is the most negative finite float instead of +inf.
 * Refuses descriptor plans, and range-list plans whose mask columns do not fit
 * the kernels (ATTN_JVP_E_INVALID, detail says why: a key seen by more than
 * 255 separate row intervals, or, in bf16, a key block that streams more than
 * 7680 query tiles); attn_jvp_bwd refuses range-list plans. */
int attn_jvp_bwd_table(const attn_jvp_plan* plan, const void* device_table, const void* q,
                       const void* k, const void* v, const void* o, const float* lse, const void* d_o,
                       void* dq, void* dk, void* dv, float* workspace, void* hip_stream);

/* attn_jvp_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results (bit for
 * bit), with the workspace in a fixed device array of the library, 32 MiB per
 * GPU, which each GPU the library runs on holds until the process ends.  The
 * call allocates nothing.  Plans with 8 B H N > 32 MiB (B H N > 4,194,304
 * rows) get ATTN_JVP_E_OVERFLOW; range-list plans get ATTN_JVP_E_INVALID.
 * All calls on one GPU share that array, which keeps the last call's
 * contents (no call needs it cleared: the dq kernel writes every entry the
 * dk/dv kernel reads), so calls whose work overlaps in time on one GPU (two
 * streams, or two threads) race and give wrong results: order them on one
 * stream, or use attn_jvp_bwd with separate workspaces.  The first call on a
 * device looks up that device's array (hipGetSymbolAddress, with the device
 * current); ATTN_JVP_E_HIP if that fails.  Other arguments and errors as for
 * attn_jvp_bwd. */
int attn_jvp_bwd_noalloc(const attn_jvp_plan* plan, const void* q, const void* k, const void* v,
                         const void* o, const float* lse, const void* d_o, void* dq, void* dk, void* dv,
                         void* hip_stream);

/* Workspace bytes attn_jvp_bwd needs for the plan: 8 B H N. */
int attn_jvp_bwd_workspace_size(const attn_jvp_plan* plan, size_t* bytes);

/* Geometry of the backward: rows per dq-kernel block and query blocks per
 * (b, h) (the dq kernel walks the forward's key tiles for each), keys per
 * dk/dv-kernel block and key blocks per (b, h).  Key blocks are cut per side
 * like query blocks (clean side from key 0, noisy side from key N_h; range-
 * list plans: from key 0 over the whole sequence); a key block streams the
 * 32-row query tiles of the rows that attend to any of its keys
 * (attn_jvp_key_ranges).  Any output pointer may be NULL. */
int attn_jvp_plan_bwd_info(const attn_jvp_plan* plan, int32_t* block_q, int32_t* block_kv,
                           int32_t* n_query_blocks, int32_t* n_key_blocks);

/* Launch order of the dk/dv kernel: position b (0 <= b < B H n_key_blocks)
 * is task host_out[b], i.e. (b, h) slice task / n_key_blocks and key block
 * task mod n_key_blocks, and is meant for XCD b mod 8 (workgroups go to the
 * 8 XCDs round robin).  Ranks within a slice are heavy first (the earliest
 * keys of a side are seen by the most rows; range-list plans: the key blocks
 * that stream more query tiles first, in the table's order).  Orders of at
 * least 2048 tasks and 2 rounds of 256: each round gives each XCD a group of
 * 32 consecutive positions of a rank-major sequence (32 neighbouring key
 * blocks of one slice, which stream nearly the same query tiles through that
 * XCD's L2: the rank group 0 of every slice, then rank group 1, ...; where 32
 * does not divide n_key_blocks, the task order itself), the group-to-XCD
 * direction alternating from round to round; only an even number of rounds
 * is grouped, the rest follows the sequence.  Smaller orders: rank b / (B H)
 * of slice b mod (B H), heavy first across all slices.  The kernel's
 * workgroups take these positions from 8 queues, one per XCD (queue x:
 * positions x, x + 8, ...), and a workgroup whose XCD's queue is empty takes
 * the next position of another's.  n is the capacity of host_out in int32
 * elements. */
int attn_jvp_bwd_launch_order(const attn_jvp_plan* plan, int32_t* host_out, size_t n);

/* Useful floating-point operations of one attn_jvp_bwd call (all B * H
 * heads): 10 d per allowed (query, key) pair, i.e. 2 per multiply-add of the
 * five products q.k, dO.v, dS k, dS q and P dO (the dq kernel recomputes the
 * scores and dO.v, which is not counted). */
int attn_jvp_plan_bwd_flops(const attn_jvp_plan* plan, int64_t* useful_flops);

/* Free a plan.  NULL is accepted. */
int attn_jvp_destroy(attn_jvp_plan* plan);

/* Static text for an error code. */
const char* attn_jvp_error_string(int code);

/* Thread-local detail of the last error on this thread ("" if none). */
const char* attn_jvp_last_error_detail(void);

/* Geometry of the plan's schedule (Appendix B, "sparse custom mask
 * representation": one task per query block; each task streams only the key
 * tiles that meet its allowed key ranges).  Query blocks are cut per side
 * (clean side from token 0, noisy side from token N_h); key tiles are cut
 * from key 0 over the whole sequence.  Any output pointer may be NULL.
 *   seq_len                N
 *   block_q, block_k       query rows per block, keys per tile
 *   n_query_blocks         query blocks per (b, h)
 *   n_key_tiles            key tiles per (b, h)
 *   allowed_pairs_per_head allowed (query, key) pairs per (b, h)
 *   visited_tiles_per_head key tiles the kernel streams, summed over blocks */
int attn_jvp_plan_info(const attn_jvp_plan* plan, int64_t* seq_len, int32_t* block_q,
                       int32_t* block_k, int32_t* n_query_blocks, int32_t* n_key_tiles,
                       int64_t* allowed_pairs_per_head, int64_t* visited_tiles_per_head);

/* Useful floating-point operations of one attn_jvp_fwd call of the plan
 * (all B * H heads): 2 per multiply-add of the products the operation needs
 * over allowed (query, key) pairs, i.e. 12 d per pair for q.k, tq.k, q.tk,
 * p.v, p.tv and (p ts).v.  With ATTN_JVP_FLAG_CLEAN_TANGENT_ZERO: 4 d per
 * clean-row pair (q.k, p.v), 8 d per noisy-row / clean-key pair (q.k, tq.k,
 * p.v, (p ts).v) and 12 d per noisy-row / noisy-key pair.  Masked pairs
 * inside partially allowed tiles and the exponentials are not counted. */
int attn_jvp_plan_flops(const attn_jvp_plan* plan, int64_t* useful_flops);

/* Per-row allowed key ranges, as the kernel uses them: host_out[4*i + 0..3]
 * = lo1, hi1, lo2, hi2 (half-open, empty when lo >= hi) for rows
 * i = 0..N-1.  n is the capacity of host_out in int32 elements (>= 4N).
 * Range-list plans: the first two intervals of the row's group (zeros for
 * rows in no group); ATTN_JVP_E_INVALID if some group has more than two. */
int attn_jvp_row_ranges(const attn_jvp_plan* plan, int32_t* host_out, size_t n);

/* Per-key allowed query ranges (the columns of the mask), as the backward's
 * dk/dv kernel uses them: host_out[4*j + 0..3] = lo1, hi1, lo2, hi2 for keys
 * j = 0..N-1: row i attends to key j iff lo1 <= i < hi1 or lo2 <= i < hi2.
 * Range-list plans: the first two row intervals of the key (zeros for a key
 * no row sees); ATTN_JVP_E_INVALID if some key is seen by more than two, or
 * if the plan has no backward.  n is the capacity of host_out in int32
 * elements (>= 4N). */
int attn_jvp_key_ranges(const attn_jvp_plan* plan, int32_t* host_out, size_t n);

/* Launch order: workgroup t (0 <= t < n_query_blocks) of every (b, h)
 * handles query block host_out[t] (index order of attn_jvp_tile_map).
 * This is the order of attn_jvp_fwd.  Heaviest (latest) blocks first.  With
 * tf_layout = 1 the sides alternate block by block; bf16 clean-tangent-zero
 * plans make two launches, so their first n_query_blocks / 2 entries are the
 * clean side's blocks and the rest the noisy side's, each heaviest first.
 * Range-list plans: host_out holds the heavy-first order of the query blocks
 * (more streamed tiles first).  "Workgroup t" is the logical task t: over
 * the whole B H grid (of each launch), the tasks are ordered in XCD groups
 * of 128 (64 in the noisy-side launch of a clean-tangent-zero plan) under the
 * rule of attn_jvp_bwd_launch_order (there with groups of 32) and taken from
 * its per-XCD queues, except on the smaller grids: there
 * clean-tangent-zero plans keep the index order, and general teacher-forcing
 * plans go heavy first across the slices in groups of 32 consecutive tasks
 * of one slice.  (attn_jvp_fwd_primal of descriptor plans, whatever the
 * plan's flags, takes the clean and noisy blocks of the same chunks in
 * groups of 8 and 8, so that the round-robin hand-out of workgroups to the 8
 * XCDs gives each XCD both sides, in the index order on small grids.)  n is
 * the capacity of host_out in int32 elements. */
int attn_jvp_launch_order(const attn_jvp_plan* plan, int32_t* host_out, size_t n);

/* Tile map, row-major [n_query_blocks][n_key_tiles], query blocks in index
 * order (clean side first): 0 = not streamed, 1 = streamed, every pair
 * allowed (no masking), 2 = streamed, some pairs masked.  Two further codes
 * flag schedule defects and never occur in a correct plan: 3 = streamed but
 * no pair allowed, 4 = not streamed although a pair is allowed.
 * n is the capacity of host_out in bytes. */
int attn_jvp_tile_map(const attn_jvp_plan* plan, uint8_t* host_out, size_t n);

/* Measurement helper (not part of the operation): enqueues on `stream` a
 * small kernel of 8 workgroups, one per XCD of an MI355X, and workgroup w
 * stores into device_out[4w .. 4w+3] (uint64): its XCD number, the XCD's
 * shader clock counter (s_memtime, which counts at the shader clock), the
 * constant 100 MHz real-time counter (s_memrealtime), and 0.  Two samples
 * taken on one stream around a run of launches give each XCD's average
 * shader clock over that run: 100 MHz * (change of the shader counter) /
 * (change of the real-time counter), pairing entries by XCD number.
 * device_out: at least 32 uint64 of device memory, 8-byte aligned, owned by
 * the caller.  Errors: ATTN_JVP_E_NULL, ATTN_JVP_E_ALIGN, a device that is
 * not gfx950, or ATTN_JVP_E_HIP if the launch fails. */
int attn_jvp_clock_sample(void* device_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_JVP_H */
