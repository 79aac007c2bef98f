// float32 block-sparse attention (prefill and decode) on the vector ALUs.
//
// Qwen4-Exp model page, overview: a query attends its selected contiguous blocks plus its
// own incomplete trailing block; usage tips: softmax attention over the selected tokens,
// grouped-query heads.
//
// Serves float32 inputs, whose tolerance rules out bf16 matrix cores.  One wave per
// (sequence, query, head): 64 tokens of T(p) at a time get their logits (one token per
// lane), the wave keeps an online softmax, and the weighted values accumulate per lane
// over the head dimension.  Deterministic: fixed-order wave reductions, no atomics.
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ kv_lens, float* __restrict__ out,
    float* __restrict__ lse, int n_q, int kv_stride_len, int seq_fixed, int h_q, int h_kv,
    int block, int top_k, float scale) {
  constexpr int DPL = (D + 63) / 64;  // head dims per lane
  __shared__ float qs[D];
  __shared__ float ps[64];
  __shared__ int ts[64];

  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int g = h / (h_q / h_kv);
  int len = kv_lens ? kv_lens[b] : seq_fixed;
  len = len < 0 ? 0 : (len > kv_stride_len ? kv_stride_len : len);
  const int p = len - n_q + i;
  const size_t qo = (((size_t)b * n_q + i) * h_q + h) * D;
  for (int d = lane; d < D; d += 64) qs[d] = q[qo + d];
  __syncthreads();

  const int n = p >= 0 ? (p + 1) / block : 0;
  const int trail0 = n * block;
  const int ntrail = p >= 0 ? p + 1 - trail0 : 0;
  const int total = top_k * block + ntrail;
  const int32_t* srow = sel + ((size_t)b * n_q + i) * top_k;

  float m_run = -__builtin_inff(), l_run = 0.f;
  float acc[DPL];
#pragma unroll
  for (int u = 0; u < DPL; ++u) acc[u] = 0.f;

  for (int base = 0; base < total; base += 64) {
    const int idx = base + lane;
    int s = -1;
    if (idx < top_k * block) {
      const int j = srow[idx / block];
      if (j >= 0 && j < n) s = j * block + idx % block;
    } else if (idx < total) {
      s = trail0 + (idx - top_k * block);
    }
    float x = -__builtin_inff();
    if (s >= 0) {
      const float* kr = k + (((size_t)b * kv_stride_len + s) * h_kv + g) * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = __builtin_fmaf(qs[d], kr[d], dot);
      x = dot * scale;
    }
    const float mx = wave_max(x);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
    const float alpha = expf(m_run - m_use);
    const float e = (s >= 0) ? expf(x - m_use) : 0.f;
    l_run = l_run * alpha + wave_sum(e);
    m_run = m_new;
    ps[lane] = e;
    ts[lane] = s;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      const int d = u * 64 + lane;
      float a = acc[u] * alpha;
      if (d < D) {
        for (int t = 0; t < 64; ++t) {
          const int st = ts[t];
          if (st >= 0) a = __builtin_fmaf(ps[t], v[(((size_t)b * kv_stride_len + st) * h_kv + g) * D + d], a);
        }
      }
      acc[u] = a;
    }
    __syncthreads();
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int u = 0; u < DPL; ++u) {
    const int d = u * 64 + lane;
    if (d < D) out[qo + d] = acc[u] * inv;
  }
  if (lse && lane == 0)
    lse[((size_t)b * n_q + i) * h_q + h] = l_run > 0.f ? m_run + logf(l_run) : -__builtin_inff();
}

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, const int32_t* sel,
                           const int32_t* kv_lens, float* out, float* lse, int batch, int n_q,
                           int kv_stride_len, int seq_fixed, int h_q, int h_kv, int d, int block,
                           int top_k, float sm_scale, hipStream_t stream) {
  if (batch == 0 || n_q == 0) return hipSuccess;
  dim3 grid(n_q, h_q, batch);
#define QSA_F32(DD)                                                                              \
  hipLaunchKernelGGL((attn_f32_kernel<DD>), grid, dim3(64), 0, stream, q, k, v, sel, kv_lens, out, \
                     lse, n_q, kv_stride_len, seq_fixed, h_q, h_kv, block, top_k, sm_scale);       \
  return hipGetLastError()
  if (d == 64) { QSA_F32(64); }
  if (d == 128) { QSA_F32(128); }
  if (d == 256) { QSA_F32(256); }
#undef QSA_F32
  return hipErrorInvalidValue;
}

}  // namespace qsa
