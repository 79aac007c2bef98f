// Key-block compression: mean of every complete block of `block` indexer keys.
//
// Qwen4-Exp model page, Qwen4ExpTextConfig / indexer_compress_ratio (consecutive token
// keys averaged into one index block); overview (the incomplete trailing block is not
// compressed).
//
// HBM-bound stream.  One workgroup (256 lanes) per (sequence, block) runs BlockMean
// (block_mean.h): whole key rows with coalesced 16-byte loads, partial column sums added in
// a fixed order (deterministic, and bit-identical to every other user of BlockMean).
#include "block_mean.h"
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

template <typename T, int DI>
__global__ __launch_bounds__(256) void compress_keys_kernel(
    const T* __restrict__ ik, const int32_t* __restrict__ kv_lens, float* __restrict__ cmp,
    int max_len, int block, int max_blocks) {
  __shared__ float part[BlockMean<T, DI>::SCRATCH];
  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int len = kv_lens ? kv_lens[b] : max_len;
  if (j >= len / block) return;              // incomplete or absent block: untouched
  const float m = BlockMean<T, DI>::run(ik + ((size_t)b * max_len + (size_t)j * block) * DI, block,
                                        part, threadIdx.x);
  if (threadIdx.x < DI) cmp[((size_t)b * max_blocks + j) * DI + threadIdx.x] = m;
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
