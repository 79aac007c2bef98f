// Key-block compression: mean of every complete block of `block` indexer keys.
//
// Qwen4-Exp model page, Qwen4ExpTextConfig / indexer_compress_ratio (consecutive token
// keys averaged into one index block); overview (the incomplete trailing block is not
// compressed).
//
// HBM-bound stream.  One workgroup (256 lanes) per (sequence, block): each lane loads
// 16 contiguous bytes of a key row per step, so a wave covers whole rows with fully
// coalesced loads; partial column sums of the row groups meet in LDS and are added in
// row-group order (deterministic), then scaled by 1/block.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

template <typename T, int DI>
__global__ __launch_bounds__(256) void compress_keys_kernel(
    const T* __restrict__ ik, const int32_t* __restrict__ kv_lens, float* __restrict__ cmp,
    int max_len, int block, int max_blocks) {
  constexpr int CPT = 16 / sizeof(T);        // columns per lane (one 16-byte load)
  constexpr int TPR = DI / CPT;              // lanes per key row
  constexpr int RG = 256 / TPR;              // row groups per workgroup
  __shared__ float part[RG][DI + 1];

  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int len = kv_lens ? kv_lens[b] : max_len;
  if (j >= len / block) return;              // incomplete or absent block: untouched

  const int tid = threadIdx.x;
  const int rg = tid / TPR;
  const int c0 = (tid % TPR) * CPT;
  float acc[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) acc[i] = 0.f;

  const T* base = ik + ((size_t)b * max_len + (size_t)j * block) * DI + c0;
  int r = rg;
  // four independent 16-byte loads in flight per lane per step
  for (; r + 3 * RG < block; r += 4 * RG) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      v[u] = *reinterpret_cast<const u32x4*>(base + (size_t)(r + u * RG) * DI);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc[2 * w] += bf16_to_f32(v[u][w] & 0xffffu);
          acc[2 * w + 1] += bf16_to_f32(v[u][w] >> 16);
        }
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[w] += __uint_as_float(v[u][w]);
      }
    }
  }
  for (; r < block; r += RG) {
    u32x4 v = *reinterpret_cast<const u32x4*>(base + (size_t)r * DI);
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
#pragma unroll
  for (int i = 0; i < CPT; ++i) part[rg][c0 + i] = acc[i];
  __syncthreads();
  if (tid < DI) {
    float s = 0.f;
    const int groups = block < RG ? block : RG;
    for (int g = 0; g < groups; ++g) s += part[g][tid];
    cmp[((size_t)b * max_blocks + j) * DI + tid] = s / (float)block;
  }
}

template <typename T, int DI>
static hipError_t launch_compress_t(const void* ik, const int32_t* kv_lens, float* cmp, int batch,
                                    int max_len, int block, hipStream_t stream) {
  const int max_blocks = max_len / block;
  if (max_blocks == 0 || batch == 0) return hipSuccess;
  dim3 grid(max_blocks, batch);
  hipLaunchKernelGGL((compress_keys_kernel<T, DI>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(ik), kv_lens, cmp, max_len, block, max_blocks);
  return hipGetLastError();
}

hipError_t launch_compress(const void* ik, const int32_t* kv_lens, float* cmp, int batch,
                           int max_len, int d_idx, int block, bool bf16, hipStream_t stream) {
  if (bf16) {
    switch (d_idx) {
      case 32: return launch_compress_t<uint16_t, 32>(ik, kv_lens, cmp, batch, max_len, block, stream);
      case 64: return launch_compress_t<uint16_t, 64>(ik, kv_lens, cmp, batch, max_len, block, stream);
      case 128: return launch_compress_t<uint16_t, 128>(ik, kv_lens, cmp, batch, max_len, block, stream);
    }
  } else {
    switch (d_idx) {
      case 32: return launch_compress_t<float, 32>(ik, kv_lens, cmp, batch, max_len, block, stream);
      case 64: return launch_compress_t<float, 64>(ik, kv_lens, cmp, batch, max_len, block, stream);
      case 128: return launch_compress_t<float, 128>(ik, kv_lens, cmp, batch, max_len, block, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace qsa
