// attn_jvp_kernels.hip -- gfx950 kernels for block-causal / teacher-forcing
// masked attention forward + forward-mode JVP.
//
// What is computed (Causal-rCM, arXiv 2606.25473, Appendix B, eqs. 42-45 and
// Algorithm 1): one online-softmax pass per query block that keeps, beside
// the FlashAttention-2 accumulators (row max m, row sum l, sum p~ v), the JVP
// accumulators sum p~ tv, sum p~ ts v and the row term r = sum p~ ts, all
// rescaled by the same online factor; the epilogue forms
//   o = acc_o / l,   to = (acc_tv + acc_tsv) / l - (r / l) o
// with the normalised o.  Here acc_tv and acc_tsv share one register tile:
// both take the same rescale and the same 1/l, so their sum is carried
// directly.
//
// bf16 kernel layout (one workgroup = one query block of 32*NW rows, one
// wave = 32 query rows, 64-wide wavefronts on v_mfma_f32_32x32x16_bf16):
// * scores are formed transposed, S^T = K Q^T, so lane l owns query l%32 and
//   16 of the 32 keys of a subtile; row max and row sums are in-lane plus one
//   permlane32 swap with the partner lane l^32;
// * inside each 32-key subtile, MFMA row m stands for key perm32(m) (bits 2
//   and 3 swapped).  With that order the S^T accumulator, converted to bf16,
//   is already the B operand of O^T += V^T P^T, so no shuffle is needed;
// * K and tK sit in LDS row-major, V and tV transposed ([d][key]), each with
//   an XOR swizzle on 16-byte groups so the 16-byte fragment reads of a wave
//   hit distinct banks;
// * rescaling is lazy: the stored row max only moves when a tile's max
//   exceeds it by more than 2^8 (in exp2 units), which keeps every p~ <= 256
//   and is exact in real arithmetic because l, r and the accumulators all
//   share the stored max;
// * whole key tiles outside the block's key ranges are never visited; the
//   element mask is applied only when some row of the wave does not cover
//   the whole tile.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "attn_jvp_launch.h"
#include "mask_index.h"

namespace attn_jvp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLazyRescaleLog2 = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

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

// Key order inside a 32-key subtile: MFMA row m holds key perm32(m).
__device__ __forceinline__ int perm32(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

// 16-byte group swizzles of the K rows and of the transposed V rows.
__device__ __forceinline__ int k_swz(int key) { return (key & 3) | ((key >> 1) & 4); }
template <int BC>
__device__ __forceinline__ int v_swz(int d) { return ((d & 7) ^ ((d >> 3) & 7)) & (BC / 8 - 1); }

template <int D, int BC, int NW>
__global__ void __launch_bounds__(NW * 64, 1) fwd_bf16_kernel(FwdParams p) {
  static_assert(BC == 64, "the swizzles and subtile order assume 64-key tiles");
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int DCH = D / 8;                 // 16-byte chunks per row
  constexpr int KS = D / 16;                 // k-steps of the score products
  constexpr int DC = D / 32;                 // 32-wide column blocks of the outputs
  constexpr int NSUB = BC / 32;              // 32-key subtiles per tile
  constexpr int KCH = BC * DCH / NT;         // K chunks staged per thread
  constexpr int VIT = (BC / 2) * DCH / NT;   // V items (2 keys x 8 d) per thread
  static_assert(KCH * NT == BC * DCH && VIT * NT == (BC / 2) * DCH, "staging split");

  __shared__ __attribute__((aligned(16))) uint16_t sK[BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t stK[BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * BC];
  __shared__ __attribute__((aligned(16))) uint16_t stV[D * BC];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;

  const MaskGeom g = p.g;
  const int N = g.seq_len;
  const int bh = blockIdx.x / p.n_qblocks;
  const int qb = heavy_first_qblock(g, BR, blockIdx.x - bh * p.n_qblocks);
  int r0, r1;
  qblock_rows(g, BR, qb, &r0, &r1);
  const TileSpans sp = block_tiles(block_ranges(g, r0, r1), BC);
  const int ntiles = span_count(sp);

  const size_t base = (size_t)bh * (size_t)N * D;
  const uint16_t* __restrict__ Qg = (const uint16_t*)p.q + base;
  const uint16_t* __restrict__ Kg = (const uint16_t*)p.k + base;
  const uint16_t* __restrict__ Vg = (const uint16_t*)p.v + base;
  const uint16_t* __restrict__ tQg = (const uint16_t*)p.tq + base;
  const uint16_t* __restrict__ tKg = (const uint16_t*)p.tk + base;
  const uint16_t* __restrict__ tVg = (const uint16_t*)p.tv + base;

  const int row = r0 + wave * 32 + n;
  const bool row_ok = row < r1;
  const Ranges rr = row_ok ? row_ranges(g, row) : Ranges{0, 0, 0, 0};

  const u32x4 zero4 = {0u, 0u, 0u, 0u};
  u32x4 qf[KS], tqf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const size_t off = (size_t)row * D + 16 * s + 8 * h;
    qf[s] = row_ok ? *(const u32x4*)(Qg + off) : zero4;
    tqf[s] = row_ok ? *(const u32x4*)(tQg + off) : zero4;
  }

  // ---- global -> register prefetch of one tile -------------------------------
  // Buffer loads: reads past the end of the (b, h) slice return zeros.
  const int slice_bytes = N * D * 2;
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(Kg, slice_bytes);
  const __amdgpu_buffer_rsrc_t rtK = make_rsrc(tKg, slice_bytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(Vg, slice_bytes);
  const __amdgpu_buffer_rsrc_t rtV = make_rsrc(tVg, slice_bytes);
  u32x4 kr[KCH], tkr[KCH], vr[VIT][2], tvr[VIT][2];
  auto gload = [&](int kt) {
    const int k0 = kt * BC;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * NT;
      const int off = ((k0 + c / DCH) * D + (c % DCH) * 8) * 2;
      kr[i] = load16(rK, off);
      tkr[i] = load16(rtK, off);
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int it = tid + i * NT;
      const int off = ((k0 + 2 * (it / DCH)) * D + (it % DCH) * 8) * 2;
      vr[i][0] = load16(rV, off);
      tvr[i][0] = load16(rtV, off);
      vr[i][1] = load16(rV, off + 2 * D);
      tvr[i][1] = load16(rtV, off + 2 * D);
    }
  };
  // ---- register -> LDS, K row-major, V transposed ----------------------------
  auto lstore = [&]() {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * NT;
      const int key = c / DCH, ch = c % DCH;
      const int off = key * D + ((ch ^ k_swz(key)) << 3);
      *(u32x4*)(sK + off) = kr[i];
      *(u32x4*)(stK + off) = tkr[i];
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int it = tid + i * NT;
      const int dc = it % DCH, kp = it / DCH;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int d = 8 * dc + j;
        const int off = d * BC + (((kp >> 2) ^ v_swz<BC>(d)) << 3) + 2 * (kp & 3);
        const uint32_t a0 = vr[i][0][j >> 1], a1 = vr[i][1][j >> 1];
        const uint32_t b0 = tvr[i][0][j >> 1], b1 = tvr[i][1][j >> 1];
        const uint32_t wv = (j & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
        const uint32_t wt = (j & 1) ? ((b0 >> 16) | (b1 & 0xffff0000u)) : ((b0 & 0xffffu) | (b1 << 16));
        *(uint32_t*)(sV + off) = wv;
        *(uint32_t*)(stV + off) = wt;
      }
    }
  };

  f32x16 accO[DC], accT[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      accO[c][i] = 0.f;
      accT[c][i] = 0.f;
    }
  }
  float m = -INFINITY, l = 0.f, r = 0.f;
  const float sl2 = p.score_log2;
  const float scale = p.scale;

  if (ntiles > 0) gload(span_tile(sp, 0));
  for (int it = 0; it < ntiles; ++it) {
    const int k0 = span_tile(sp, it) * BC;
    __syncthreads();
    lstore();
    __syncthreads();
    if (it + 1 < ntiles) gload(span_tile(sp, it + 1));

    const bool masked = !__all(covers(rr, k0, k0 + BC));
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      // S^T and tS^T of one 32-key subtile
      f32x16 S, TS;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        S[i] = 0.f;
        TS[i] = 0.f;
      }
      const int skey = sub * 32 + perm32(n);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int off = skey * D + (((2 * s + h) ^ k_swz(skey)) << 3);
        const u32x4 kf = *(const u32x4*)(sK + off);
        const u32x4 tkf = *(const u32x4*)(stK + off);
        S = mfma_bf16(kf, qf[s], S);
        TS = mfma_bf16(kf, tqf[s], TS);
        TS = mfma_bf16(tkf, qf[s], TS);
      }

      // element mask where some row of the wave does not cover the whole tile
      if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + sub * 32 + perm32(8 * (i >> 2) + 4 * h + (i & 3));
          if (!in_ranges(rr, key)) {
            S[i] = -INFINITY;
            TS[i] = 0.f;
          }
        }
      }

      // online softmax with lazy rescaling (exp2 units)
      float tmax = S[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, S[i]);
      const float tmax_x = pair_max(tmax) * sl2;
      if (__any(tmax_x > m + kLazyRescaleLog2)) {
        const float mn = fmaxf(m, tmax_x);
        const float alpha = (mn == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m - mn);
        m = mn;
        l *= alpha;
        r *= alpha;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          accO[c] *= alpha;
          accT[c] *= alpha;
        }
      }
      const float mu = (m == -INFINITY) ? 0.f : m;

      u32x4 P[2], W[2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int i = 8 * c2 + j;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(S[i], sl2, -mu));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(S[i + 1], sl2, -mu));
          const float w0 = p0 * (TS[i] * scale);
          const float w1 = p1 * (TS[i + 1] * scale);
          l += p0 + p1;
          r += w0 + w1;
          P[c2][j >> 1] = pack_bf16(p0, p1);
          W[c2][j >> 1] = pack_bf16(w0, w1);
        }
      }

      // O^T += V^T P^T ;  T^T += tV^T P^T + V^T W^T
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int gk = 4 * sub + 2 * c2 + h;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
          const int d = 32 * c + n;
          const int off = d * BC + ((gk ^ v_swz<BC>(d)) << 3);
          const u32x4 vf = *(const u32x4*)(sV + off);
          const u32x4 tvf = *(const u32x4*)(stV + off);
          accO[c] = mfma_bf16(vf, P[c2], accO[c]);
          accT[c] = mfma_bf16(tvf, P[c2], accT[c]);
          accT[c] = mfma_bf16(vf, W[c2], accT[c]);
        }
      }
    }
  }

  // ---- epilogue: o = acc_o / l ; to = acc_t / l - (r / l) o ------------------
  const float lt = pair_sum(l);
  const float rt = pair_sum(r);
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
          o4[e] = accO[c][4 * g4 + e] * inv;
          t4[e] = accT[c][4 * g4 + e] * inv - rb * o4[e];
        }
        u32x2 ov = {pack_bf16(o4[0], o4[1]), pack_bf16(o4[2], o4[3])};
        u32x2 tv = {pack_bf16(t4[0], t4[1]), pack_bf16(t4[2], t4[3])};
        *(u32x2*)(Og + d0) = ov;
        *(u32x2*)(tOg + d0) = tv;
      }
    }
    if (h == 0 && p.lse != nullptr)
      p.lse[(size_t)bh * N + row] = lt > 0.f ? m * kLn2 + logf(lt) : -INFINITY;
  }
}

// fp32 kernel: 32 query rows per workgroup, 8 lanes per row, each lane owning
// D/8 consecutive columns.  Keys are taken one at a time from the same tile
// schedule as the bf16 kernel, with the exact per-row mask; the online
// softmax is the plain FlashAttention-2 recurrence in fp32 (no lazy scaling).
template <int D>
__global__ void __launch_bounds__(256) fwd_fp32_kernel(FwdParams p) {
  constexpr int BR = 32, BC = 32, E = D / 8;
  const MaskGeom g = p.g;
  const int N = g.seq_len;
  const int slice = threadIdx.x & 7, lr = threadIdx.x >> 3;
  const int bh = blockIdx.x / p.n_qblocks;
  const int qb = heavy_first_qblock(g, BR, blockIdx.x - bh * p.n_qblocks);
  int r0, r1;
  qblock_rows(g, BR, qb, &r0, &r1);
  const TileSpans sp = block_tiles(block_ranges(g, r0, r1), BC);
  const int ntiles = span_count(sp);
  const int row = r0 + lr;
  const bool row_ok = row < r1;
  const Ranges rr = row_ok ? row_ranges(g, row) : Ranges{0, 0, 0, 0};

  const size_t base = (size_t)bh * (size_t)N * D;
  const float* __restrict__ K = (const float*)p.k + base + slice * E;
  const float* __restrict__ V = (const float*)p.v + base + slice * E;
  const float* __restrict__ tK = (const float*)p.tk + base + slice * E;
  const float* __restrict__ tV = (const float*)p.tv + base + slice * E;
  float q[E], tq[E], ao[E], at[E];
  const int qrow = row_ok ? row : r0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    q[e] = ((const float*)p.q)[base + (size_t)qrow * D + slice * E + e];
    tq[e] = ((const float*)p.tq)[base + (size_t)qrow * D + slice * E + e];
    ao[e] = 0.f;
    at[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f, r = 0.f;
  for (int it = 0; it < ntiles; ++it) {
    const int k0 = span_tile(sp, it) * BC;
    const int k1 = k0 + BC < N ? k0 + BC : N;
    for (int j = k0; j < k1; ++j) {
      if (!in_ranges(rr, j)) continue;  // uniform across the row's 8 lanes
      const float* kj = K + (size_t)j * D;
      const float* tkj = tK + (size_t)j * D;
      float s = 0.f, ts = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        s = fmaf(q[e], kj[e], s);
        ts = fmaf(tq[e], kj[e], fmaf(q[e], tkj[e], ts));
      }
#pragma unroll
      for (int o = 1; o < 8; o <<= 1) {
        s += __shfl_xor(s, o, 8);
        ts += __shfl_xor(ts, o, 8);
      }
      s *= p.scale;
      ts *= p.scale;
      const float mn = fmaxf(m, s);
      const float alpha = expf(m - mn);
      const float pj = expf(s - mn);
      l = l * alpha + pj;
      r = r * alpha + pj * ts;
      const float* vj = V + (size_t)j * D;
      const float* tvj = tV + (size_t)j * D;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        ao[e] = ao[e] * alpha + pj * vj[e];
        at[e] = at[e] * alpha + pj * tvj[e] + (pj * ts) * vj[e];
      }
      m = mn;
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
    tO[e] = at[e] * inv - rb * o;
  }
  if (slice == 0 && p.lse != nullptr) p.lse[(size_t)bh * N + row] = l > 0.f ? m + logf(l) : -INFINITY;
}

// ---------------------------------------------------------------------------
void block_sizes(int dtype, int head_dim, int* block_q, int* block_k) {
  (void)head_dim;
  if (dtype == kBf16) {
    *block_q = kBf16Waves * 32;
    *block_k = 64;
  } else {
    *block_q = 32;
    *block_k = 32;
  }
}

hipError_t launch_fwd(int dtype, int head_dim, int grid, const FwdParams& p, hipStream_t stream) {
  if (dtype == kBf16) {
    if (head_dim == 128)
      hipLaunchKernelGGL((fwd_bf16_kernel<128, 64, kBf16Waves>), dim3(grid), dim3(kBf16Waves * 64), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<64, 64, kBf16Waves>), dim3(grid), dim3(kBf16Waves * 64), 0, stream, p);
  } else {
    if (head_dim == 128)
      hipLaunchKernelGGL((fwd_fp32_kernel<128>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_fp32_kernel<64>), dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace attn_jvp
