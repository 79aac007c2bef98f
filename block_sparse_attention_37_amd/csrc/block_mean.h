// Mean of one block of `block` consecutive indexer keys, computed by a whole 256-lane
// workgroup in a fixed order, so every kernel that compresses a block gets bit-identical
// values.
//
// Qwen4-Exp model page, Qwen4ExpTextConfig / indexer_compress_ratio: that many consecutive
// token keys are averaged into one index block.
#pragma once

#include "qsa_device.h"

namespace qsa {

// Each lane loads 16 contiguous bytes of a key row per step (whole rows, coalesced); the
// partial column sums of the RG row groups meet in LDS and are added in row-group order,
// then scaled by 1/block.  `rows` points at the block's first key row (DI elements per row);
// `part` is LDS scratch of SCRATCH floats.  The lanes tid < DI return the mean of column tid;
// the others return 0.  Contains one __syncthreads(), so every thread of the workgroup calls
// it; only the first 256 threads load and add.
template <typename T, int DI>
struct BlockMean {
  static constexpr int CPT = 16 / sizeof(T);  // columns per lane (one 16-byte load)
  static constexpr int TPR = DI / CPT;        // lanes per key row
  static constexpr int RG = 256 / TPR;        // row groups per workgroup
  static constexpr int SCRATCH = RG * (DI + 1);

  static __device__ __forceinline__ void add(float* acc, const u32x4& v) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] += bf16_to_f32(v[w] & 0xffffu);
        acc[2 * w + 1] += bf16_to_f32(v[w] >> 16);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[w] += __uint_as_float(v[w]);
    }
  }

  static __device__ __forceinline__ float run(const T* __restrict__ rows, int block, float* part,
                                              int tid) {
    if (tid < 256) {
      const int rg = tid / TPR;
      const int c0 = (tid % TPR) * CPT;
      float acc[CPT];
#pragma unroll
      for (int i = 0; i < CPT; ++i) acc[i] = 0.f;
      const T* base = rows + c0;
      int r = rg;
      // four independent 16-byte loads in flight per lane per step
      for (; r + 3 * RG < block; r += 4 * RG) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          v[u] = *reinterpret_cast<const u32x4*>(base + (size_t)(r + u * RG) * DI);
#pragma unroll
        for (int u = 0; u < 4; ++u) add(acc, v[u]);
      }
      for (; r < block; r += RG) add(acc, *reinterpret_cast<const u32x4*>(base + (size_t)r * DI));
#pragma unroll
      for (int i = 0; i < CPT; ++i) part[rg * (DI + 1) + c0 + i] = acc[i];
    }
    __syncthreads();
    float s = 0.f;
    if (tid < DI) {
      const int groups = block < RG ? block : RG;
      for (int g = 0; g < groups; ++g) s += part[g * (DI + 1) + tid];
      s = s / (float)block;
    }
    return s;
  }
};

}  // namespace qsa
