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
};

// Query rows per block and keys per tile of the kernel chosen for dtype/head_dim.
void block_sizes(int dtype, int head_dim, int* block_q, int* block_k);

// Launch one forward + JVP over `grid` workgroups; returns hipGetLastError().
hipError_t launch_fwd(int dtype, int head_dim, int grid, const FwdParams& p, hipStream_t stream);

}  // namespace attn_jvp
