// kernel_common.h -- gfx950 device building blocks shared by the forward/JVP
// and the backward kernels: bf16 matrix-core products (register and
// vector-register forms), lane-pair reductions, bf16 packing, buffer
// resources and HBM -> LDS DMA, transposing LDS reads, the LDS row swizzle,
// accumulation-register access, explicit waits and barriers, and the
// workgroups' per-XCD work queues.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn_jvp {

// Work queues.  A grid of more workgroups than tasks (queue_grid) takes the n
// positions of a static order (launch_task) from 8 queues, queue y holding
// positions y, y + 8, y + 16, .. in that order: the ones the static grid would
// give XCD y, since workgroups go to the XCDs round robin.  A workgroup takes
// the next position of its own XCD's queue, else of the next queue that has any
// left, and gets -1 when all are empty; so every position is taken exactly
// once, an XCD keeps its share (and its L2 locality) while it lasts, and one
// that runs faster (the XCDs' clocks under the power cap differ) takes the ends
// of the others'.  Which workgroup runs a task does not change its results.  q:
// 9 int32, the 8 queue counters and the number of workgroups that have taken
// (kQueueWords per call); zero before the launch.  The last workgroup to take
// sets them back to zero (every taking is complete by then: each workgroup
// counts itself only after its own atomics have returned), so launches that use
// q one after another, on one stream or joined by events, find it zeroed;
// launches that use it at the same time would race.  Called by one lane.
__device__ __forceinline__ int take_task(int32_t* q, int n) {
  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  int pos = -1;
  for (int k = 0; k < 8 && pos < 0; ++k) {
    const int y = (int)((xcc + k) & 7);
    const int ny = (n - y + 7) >> 3;  // positions y, y + 8, .. below n
    if (__hip_atomic_load(&q[y], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= ny) continue;
    const int i = __hip_atomic_fetch_add(&q[y], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (i < ny) pos = 8 * i + y;
  }
  const int taken = __hip_atomic_fetch_add(&q[8], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (taken == (int)(gridDim.x * gridDim.y * gridDim.z) - 1) {
    for (int i = 0; i < 9; ++i) __hip_atomic_store(&q[i], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return pos;
}
// The workgroup's position (take_task by its first lane), the same in every
// lane; -1: none is left and the workgroup has no task.  Once per kernel.
__device__ __forceinline__ int workgroup_task(int32_t* q, int n) {
  __shared__ int pos_shared;
  if (threadIdx.x == 0) pos_shared = take_task(q, n);
  __syncthreads();
  return pos_shared;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Combine a value with the one held by lane l^32 (symmetric ops only: the
// swap returns own and partner values, one in each result).
__device__ __forceinline__ float pair_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Raw buffer resource over [base, base + bytes): out-of-range loads return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
// Buffer descriptor as four dwords (base, stride 0, byte size, the same
// config word as make_rsrc): for the DMA below.  Loads at or past `bytes`
// (vector + scalar offset, checked on the device) return zeros.
// The empty asm keeps the four words together in one scalar register quad, as
// the DMA instruction takes them (the compiler would otherwise share the
// words two descriptors have in common and rebuild a quad before each DMA).
__device__ __forceinline__ i32x4_t make_desc(const void* base, int bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4_t d{(int32_t)(uint32_t)a, (int32_t)(uint32_t)((a >> 32) & 0xffff), bytes, 0x00020000};
  asm volatile("" : "+s"(d));
  return d;
}
// LDS byte address of a pointer into LDS: the low 32 bits of its generic
// address (a generic LDS address is the LDS aperture base plus the LDS
// offset), with no null-pointer handling as in a cast to the LDS space.
__device__ __forceinline__ int lds_addr(const void* p) { return (int)(uint32_t)(uintptr_t)p; }
// 16 bytes per lane from global (byte offset voff + soff, soff wave-uniform)
// straight into LDS at lds + 16 * lane, written out rather than through the
// compiler builtin.  Where the compiler tracks its own LDS DMA against later
// LDS reads, it may wait for every DMA in flight (vmcnt(0))
// before a read of another ring stage, which exposes the whole DMA latency
// once per tile.  A kernel using this DMA orders its ring itself (explicit vmcnt waits and
// barriers before a stage is read or refilled), so the DMA is hidden from the
// compiler; the memory clobber keeps LDS accesses from moving across.
// Vector-memory loads complete in order, so the compiler's own waits for its
// loads stay correct (they only cover more).  M0 (the LDS base of the DMA) is
// an input operand, so the compiler sets it and knows its value afterwards;
// the s_nop gives the one wait state an M0 write needs before the DMA.
__device__ __forceinline__ void load16_lds_asm(i32x4_t r, uint16_t* lds, int voff, int soff) {
  // soff and the LDS address are wave-uniform; readfirstlane puts them in
  // scalar registers where the compiler computed them in vector ones
  const int m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  const int so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(r), "s"(so), "{m0}"(m0) : "memory");
}
// The same with the LDS byte address given as a wave-uniform integer.
__device__ __forceinline__ void load16_lds_at(i32x4_t r, int lds_byte, int voff, int soff) {
  const int m0 = __builtin_amdgcn_readfirstlane(lds_byte);
  const int so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(r), "s"(so), "{m0}"(m0) : "memory");
}
// 4 bytes per lane into LDS at lds + 4 * lane (same scheme as above).
__device__ __forceinline__ void load4_lds_asm(i32x4_t r, float* lds, int voff, int soff) {
  const int m0 = __builtin_amdgcn_readfirstlane(lds_addr(lds));
  const int so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(r), "s"(so), "{m0}"(m0) : "memory");
}
// The two bf16 halves of a packed word as floats (exact).
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ u32x2 read_tr16(const uint16_t* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)p));
}

// 16-byte group swizzle of a tile row: group g of row `key` is stored at
// g ^ row_swz<D>(key).  gfx950 LDS has 64 banks (256 bytes per cycle).
// * 16-byte fragment reads serve 16 lanes, i.e. 16 consecutive rows at one
//   logical group: the swizzle maps them to 16 distinct bank groups.
// * A transposing read serves a 16-lane group with 4 rows 4k..4k+3 and 16
//   or 32 consecutive columns: the swizzle puts each of the 4 rows into its
//   own aligned 64-byte bank group.
// d = 128 rows are 256 bytes (all 64 banks); d = 64 rows are 128 bytes, so
// rows of opposite parity already sit in opposite bank halves.
template <int D>
__device__ __forceinline__ int row_swz(int key) {
  if constexpr (D == 128) return ((key & 3) << 2) | ((key >> 2) & 3);
  else return (((key >> 1) & 1) << 2) | ((key >> 2) & 3);
}

// Vector access to accumulation registers, written out so that the compiler
// sees no vector-ALU reader of the loop-carried accumulators (it would
// otherwise keep a second copy of all of them in vector registers and refresh
// it on every tile).  Callers run acc_hazard_wait() first: an MFMA result may
// be read by a vector instruction only after enough wait states (24 here,
// above the requirement of the 32x32 bf16 MFMA).
__device__ __forceinline__ void acc_hazard_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}
__device__ __forceinline__ float acc_write(float v) {
  float a;
  asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(a) : "v"(v));
  return a;
}

// Score products in vector-register form: the scores go straight from the
// matrix cores to the vector ALUs, with no accumulator-to-vector copies (on
// gfx950 such a copy next to running MFMAs costs several times a plain vector
// op).  Written out because the compiler gives all MFMAs of a kernel one
// register form, and the output accumulators need the accumulation registers.
// The compiler inserts the waits for the operands (LDS reads, loads) but does
// not see the result hazard: vector instructions read these results only
// after at least two further MFMAs have been issued, or after
// acc_hazard_wait() fenced by sched_barrier on both sides (plain vector code
// may otherwise be scheduled across the asm).
__device__ __forceinline__ void mfma_v_first(f32x16& d, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v_acc(f32x16& d, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

// Keep a loop-carried accumulator tile in accumulation registers: an empty
// asm that takes and returns it there, so that the register allocator gives
// the loop's phi the accumulation class instead of carrying a vector-register
// copy around the loop.  Emits no instruction.
__device__ __forceinline__ void keep_in_acc(f32x16& a) { asm volatile("" : "+a"(a)); }
// The same for a resident MFMA operand: defined in accumulation registers,
// it stays there for its "a"-constrained uses.
__device__ __forceinline__ void keep_in_acc(u32x4& a) { asm volatile("" : "+a"(a)); }

// The same with the B operand in accumulation registers (operands that stay
// resident for a whole task, where vector registers are short).
__device__ __forceinline__ void mfma_v_first_ba(f32x16& d, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_v_acc_ba(f32x16& d, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// First product of a chain started from c instead of 0 (d = a b + c; c kept).
__device__ __forceinline__ void mfma_v_init_ba(f32x16& d, u32x4 a, u32x4 b, const f32x16& c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
}

// Hide a tile's value from the compiler (emits no instruction): a tile of
// equal values otherwise becomes one register plus copies, which the register
// allocator shuffles around a loop that rewrites the tile.
__device__ __forceinline__ void opaque(f32x16& a) { asm volatile("" : "+v"(a)); }

// Pin a value to this point of the instruction stream: it must be computed
// before the (volatile, hence ordered) empty asm, so the compiler cannot sink
// it into a later block.  Emits no instruction.
__device__ __forceinline__ void pin(float x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void pin(uint32_t x) { asm volatile("" ::"v"(x)); }
// Keep the start value c of an MFMA chain (mfma_v_init_ba) allocated until
// this point: the compiler does not know that the matrix core reads it over
// several passes after issue, and would reuse its registers at once.  Place
// it after two further MFMAs.
__device__ __forceinline__ void hold(const f32x16& c) { asm volatile("" ::"v"(c)); }

// Workgroup barrier without a memory fence: the fence of __syncthreads()
// would wait for every LDS DMA in flight.  Visibility of the tile about to be
// read comes from the explicit vmcnt wait before it; the memory clobber keeps
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// Explicit waits, as the s_waitcnt builtin rather than inline asm: the
// compiler then sees them and knows which of its own loads (and LDS DMAs) have
// completed, so it adds no waits of its own for them later (an inline-asm wait
// is opaque to it).  gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8; a field at its maximum does not wait.  The builtin
// itself does not order memory accesses, so empty memory-clobbering asm on
// both sides keeps loads and stores from moving across the wait.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (N << 8));
  asm volatile("" ::: "memory");
}

}  // namespace attn_jvp
