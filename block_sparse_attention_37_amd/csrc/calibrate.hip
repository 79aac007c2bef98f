// Calibration kernels: what the chip sustains on the two resources that bound the QSA
// kernels, measured on the same device and in the same run as the kernels themselves.
//   * qsa_calib_stream_read: every byte of a large device buffer read once with 16-byte
//     loads, many in flight per lane (the HBM read rate the decode kernels are held to).
//   * qsa_calib_mfma_bf16: back-to-back v_mfma_f32_32x32x16_bf16 on register operands, four
//     independent accumulators per wave, two waves per SIMD on every CU (the dense bf16
//     matrix rate the prefill attention kernels are held to).
// Neither takes part in the QSA path; bench.py reports the QSA kernels against these rates
// next to the vendor peaks.
#include "qsa_calibrate.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;  // 16-byte loads in flight per lane

// Grid-stride read of n16 16-byte units; the XOR of everything read goes to sink[block] so
// the loads cannot be dropped.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                   size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  u32x4 acc{0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * stride < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= src[i];
  uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int o = 32; o >= 1; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t part[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kReadThreads / 64; ++w) r ^= part[w];
    sink[blockIdx.x] = r;
  }
}

constexpr int kMfmaThreads = 512;  // 8 waves: two per SIMD
constexpr int kMfmaChains = 4;     // independent accumulators per wave

// iters x kMfmaChains MFMAs per wave on operands derived from the seed (never zero-folded);
// the accumulators' sum goes to sink[wave] so nothing is dropped.
__global__ __launch_bounds__(kMfmaThreads, 1) void mfma_bf16_kernel(int iters, float seed,
                                                                   float* __restrict__ sink) {
  const float s = seed + 1e-3f * (threadIdx.x & 63);
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(s + 0.125f * i);
    b[i] = (__bf16)(s - 0.0625f * i);
  }
  f32x16 c[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[k][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k)
      c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) t += c[k][r];
  sink[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = t;
}

}  // namespace

extern "C" {

int qsa_calib_stream_read(const void* src, size_t bytes, uint32_t* sink, int blocks,
                          hipStream_t stream) {
  if (src == nullptr || sink == nullptr || blocks < 1 || (bytes & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0)
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kReadThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int qsa_calib_mfma_bf16(int iters, int blocks, float* sink, double* flops, hipStream_t stream) {
  if (sink == nullptr || flops == nullptr || iters < 1 || blocks < 1) return 1;
  *flops = (double)blocks * (kMfmaThreads / 64) * kMfmaChains * (double)iters * 32.0 * 32.0 *
           16.0 * 2.0;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(kMfmaThreads), 0, stream, iters,
                     0.5f, sink);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

int qsa_calib_mfma_sink_floats(int blocks) { return blocks * kMfmaThreads; }

}  // extern "C"
