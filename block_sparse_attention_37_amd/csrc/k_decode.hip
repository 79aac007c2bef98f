// Block-sparse decode attention (one new query token per sequence) on bf16 matrix cores.
//
// Qwen4-Exp model page, overview: the query attends its selected contiguous blocks and
// its own incomplete trailing block; usage tips: cached generation keeps the QSA indexer
// state on device, the attention key/value cache is a per-sequence store.
//
// HBM-bound: every selected key/value byte is read once.  The token list of a sequence
// (selected blocks in ascending order, then the trailing tokens) is cut into 64-key
// chunks; a workgroup handles one (sequence, KV head, split) = a contiguous run of those
// chunks and streams them through LDS, double-buffered, with fully coalesced 16-byte loads
// of whole key/value rows.  The G query heads sharing the KV head form the 16 MFMA rows
// (rows >= G are zero).  Each of the 4 waves takes 16 keys of a chunk:
//   S^T = K . Q^T on 16x16x32 MFMAs, O^T += V^T . P^T on 16x16x16 MFMAs,
// with per-wave online softmax; the waves' partial states meet in LDS at the end.  With
// more than one split, each split writes a normalised partial output and its
// log-sum-exp to the caller's workspace and a small merge kernel combines them.
#include "qsa_device.h"
#include "qsa_internal.h"

#include <climits>

namespace qsa {

namespace {
constexpr int KC = 64;
constexpr int kTargetWorkgroups = 1024;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x16_bf16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<s16x4>(a), bitcast<s16x4>(b), c, 0, 0, 0);
}
}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void decode_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ sel, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int max_len, int h_q, int h_kv,
    int G, int block, int top_k, float scale_log2, int nsplit) {
  constexpr int NC16 = D / 8;
  constexpr int KIT = KC * NC16 / 256;
  constexpr int VQ = KC / 4 * NC16;
  constexpr int NQT = D / 32;  // k-steps of S^T (32 dims each)
  constexpr int NDT = D / 16;  // 16-row d tiles of O^T

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KC * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * KC];
  __shared__ int32_t list[kMaxTopK];
  __shared__ int32_t list_n;
  __shared__ float wm[4][16];
  __shared__ float wl[4][16];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int len = kv_lens[b];
  len = len < 0 ? 0 : (len > max_len ? max_len : len);
  const int n = len / block;
  const int ntrail = len - n * block;

  // compact the valid selected blocks (0 <= j < n), keeping their order
  if (wave == 0) {
    int base = 0;
    for (int e0 = 0; e0 < top_k; e0 += 64) {
      const int e = e0 + lane;
      int j = -1;
      if (e < top_k) j = sel[(size_t)b * top_k + e];
      const bool ok = (e < top_k) && j >= 0 && j < n;
      const uint64_t m = __ballot(ok);
      if (ok) list[base + __popcll(m & lanemask_lt())] = j;
      base += __popcll(m);
    }
    if (lane == 0) list_n = base;
  }
  __syncthreads();
  const int mv = list_n;
  const int nsub = (block + KC - 1) / KC;
  const int tunits = (ntrail + KC - 1) / KC;
  const int nchunks = mv * nsub + tunits;
  const int c_begin = (int)((long long)nchunks * split / nsplit);
  const int c_end = (int)((long long)nchunks * (split + 1) / nsplit);

  const size_t kv_row = (size_t)h_kv * D;
  const uint16_t* kbase = kc + ((size_t)b * max_len * h_kv + g) * D;
  const uint16_t* vbase = vc + ((size_t)b * max_len * h_kv + g) * D;

  auto chunk_keys = [&](int u, int& key0, int& ck) {
    if (u < mv * nsub) {
      const int j = list[u / nsub], sub = u % nsub;
      key0 = j * block + sub * KC;
      ck = min(KC, block - sub * KC);
    } else {
      const int tu = u - mv * nsub;
      key0 = n * block + tu * KC;
      ck = min(KC, ntrail - tu * KC);
    }
  };

  u32x4 kreg[KIT];
  u32x4 vreg[4];
  auto load_chunk = [&](int u) {
    int key0, ck;
    chunk_keys(u, key0, ck);
#pragma unroll
    for (int i = 0; i < KIT; ++i) {
      const int e = i * 256 + tid;
      const int r = e / NC16, c = e % NC16;
      kreg[i] = (r < ck) ? *reinterpret_cast<const u32x4*>(kbase + (size_t)(key0 + r) * kv_row + c * 8)
                         : u32x4{0u, 0u, 0u, 0u};
    }
    if (tid < VQ) {
      const int c = tid % NC16, quad = tid / NC16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = quad * 4 + i;
        vreg[i] = (r < ck) ? *reinterpret_cast<const u32x4*>(vbase + (size_t)(key0 + r) * kv_row + c * 8)
                           : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KIT; ++i) {
      const int e = i * 256 + tid;
      const int r = e / NC16, c = e % NC16;
      *reinterpret_cast<u32x4*>(&Ks[buf][r * D + ((c ^ (r & (NC16 - 1))) * 8)]) = kreg[i];
    }
    if (tid < VQ) {
      const int c = tid % NC16, quad = tid / NC16;
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int d = c * 8 + dd;
        const int w = dd >> 1;
        uint32_t lo, hi;
        if (dd & 1) {
          lo = (vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u);
          hi = (vreg[2][w] >> 16) | (vreg[3][w] & 0xffff0000u);
        } else {
          lo = (vreg[0][w] & 0xffffu) | (vreg[1][w] << 16);
          hi = (vreg[2][w] & 0xffffu) | (vreg[3][w] << 16);
        }
        const int unit = quad ^ ((d >> 1) & 15);
        *reinterpret_cast<u32x2*>(&Vt[buf][d * KC + unit * 4]) = u32x2{lo, hi};
      }
    }
  };

  // query rows: lane holds row nr = lane & 15 (query head g*G + nr when nr < G)
  const int nr = lane & 15;
  const int quarter = lane >> 4;
  bf16x8 qreg[NQT];
  {
    const bool ok = nr < G;
    const uint16_t* qp = q + ((size_t)b * h_q + g * G + (ok ? nr : 0)) * D + quarter * 8;
#pragma unroll
    for (int t = 0; t < NQT; ++t) {
      u32x4 w = ok ? *reinterpret_cast<const u32x4*>(qp + t * 32) : u32x4{0u, 0u, 0u, 0u};
      qreg[t] = bitcast<bf16x8>(w);
    }
  }

  float m_run = -__builtin_inff();
  float l_run = 0.f;
  f32x4 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (c_begin < c_end) {
    load_chunk(c_begin);
    store_chunk(0);
  }
  __syncthreads();
  int buf = 0;
  for (int u = c_begin; u < c_end; ++u) {
    const bool have_next = u + 1 < c_end;
    if (have_next) load_chunk(u + 1);
    int key0, ck;
    chunk_keys(u, key0, ck);
    const int kw = wave * 16;  // this wave's keys inside the chunk
    if (kw < ck) {
      f32x4 s{0.f, 0.f, 0.f, 0.f};
      const int kr = kw + nr;
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        const int c = 4 * t + quarter;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[buf][kr * D + ((c ^ (kr & (NC16 - 1))) * 8)]);
        s = mfma16x16x32(a, qreg[t], s);
      }
      float mx = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kw + 4 * quarter + r;
        const float x = key < ck ? s[r] * scale_log2 : -__builtin_inff();
        s[r] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -__builtin_inff()) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      const float e0 = __builtin_amdgcn_exp2f(s[0] - m_use);
      const float e1 = __builtin_amdgcn_exp2f(s[1] - m_use);
      const float e2 = __builtin_amdgcn_exp2f(s[2] - m_use);
      const float e3 = __builtin_amdgcn_exp2f(s[3] - m_use);
      l_run = l_run * alpha + ((e0 + e1) + (e2 + e3));
      m_run = m_new;
      const u32x2 pb{pack_bf16x2(e0, e1), pack_bf16x2(e2, e3)};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        O[dt] *= alpha;
        const int d = dt * 16 + nr;
        const int unit = (4 * wave + quarter) ^ ((d >> 1) & 15);
        const u32x2 a = *reinterpret_cast<const u32x2*>(&Vt[buf][d * KC + unit * 4]);
        O[dt] = mfma16x16x16_bf16(a, pb, O[dt]);
      }
    }
    if (have_next) store_chunk(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // ---- combine the 4 waves (rows nr, d = dt*16 + 4*quarter + r) ----
  float lsum = l_run + __shfl_xor(l_run, 16);
  lsum += __shfl_xor(lsum, 32);
  if (quarter == 0) {
    wm[wave][nr] = m_run;
    wl[wave][nr] = lsum;
  }
  float* wo = reinterpret_cast<float*>(&Ks[0][0]);  // [4][D][16] floats, fits in Ks
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 4; ++r) wo[(wave * D + dt * 16 + 4 * quarter + r) * 16 + nr] = O[dt][r];
  __syncthreads();

  for (int e = tid; e < G * D; e += 256) {
    const int row = e / D, d = e % D;
    float M = -__builtin_inff();
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][row]);
    const float Mu = (M == -__builtin_inff()) ? 0.f : M;
    float L = 0.f, acc = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = __builtin_amdgcn_exp2f(wm[w][row] - Mu);
      L += wl[w][row] * f;
      acc += wo[(w * D + d) * 16 + row] * f;
    }
    const float o = L > 0.f ? acc / L : 0.f;
    const float lse2 = L > 0.f ? (M + __log2f(L)) : -__builtin_inff();  // log2 domain
    const int h = g * G + row;
    if (nsplit == 1) {
      const uint32_t bits = f32_to_bf16(o);
      out[((size_t)b * h_q + h) * D + d] = (uint16_t)bits;
      if (lse && d == 0) lse[(size_t)b * h_q + h] = lse2 * kLn2;
    } else {
      ws_o[(((size_t)b * h_q + h) * nsplit + split) * D + d] = o;
      if (d == 0) ws_lse[((size_t)b * h_q + h) * nsplit + split] = lse2;
    }
  }
}

// One workgroup per (sequence, query head): combine the splits' partial results.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(const float* __restrict__ ws_o,
                                                       const float* __restrict__ ws_lse,
                                                       uint16_t* __restrict__ out,
                                                       float* __restrict__ lse, int nsplit) {
  const size_t bh = blockIdx.x;
  const int d = threadIdx.x;
  const float* ls = ws_lse + bh * nsplit;
  float M = -__builtin_inff();
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ls[s]);
  const float Mu = (M == -__builtin_inff()) ? 0.f : M;
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < nsplit; ++s) {
    const float f = __builtin_amdgcn_exp2f(ls[s] - Mu);
    L += f;
    acc += f * ws_o[(bh * nsplit + s) * D + d];
  }
  out[bh * D + d] = (uint16_t)f32_to_bf16(L > 0.f ? acc / L : 0.f);
  if (lse && d == 0) lse[bh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

bool decode_bf16_supported(int group, int d, int block, int top_k) {
  if (d != 64 && d != 128) return false;
  if (group < 1 || group > 16) return false;
  return block >= 1 && block <= 1024 && top_k >= 1 && top_k <= kMaxTopK;
}

int decode_num_splits(int batch, int h_kv, int block, int top_k) {
  const long long units = (long long)batch * h_kv;
  if (units <= 0) return 1;
  long long want = (kTargetWorkgroups + units - 1) / units;
  const long long chunks = (long long)top_k * ((block + KC - 1) / KC) + (block + KC - 2) / KC;
  if (want > chunks) want = chunks;
  if (want > 32) want = 32;
  if (want < 1) want = 1;
  return (int)want;
}

size_t decode_workspace_bytes(int batch, int h_q, int d, int nsplit) {
  if (nsplit <= 1) return 0;
  return (size_t)batch * h_q * nsplit * (d + 1) * sizeof(float);
}

template <int D>
static hipError_t launch_decode_t(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* kv_lens, const int32_t* sel, void* out,
                                  float* lse, int batch, int max_len, int h_q, int h_kv,
                                  int block, int top_k, float sm_scale, void* workspace,
                                  int nsplit, hipStream_t stream) {
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o ? ws_o + (size_t)batch * h_q * nsplit * D : nullptr;
  dim3 grid(nsplit, h_kv, batch);
  hipLaunchKernelGGL((decode_bf16_kernel<D>), grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache),
                     static_cast<const uint16_t*>(v_cache), kv_lens, sel,
                     static_cast<uint16_t*>(out), lse, ws_o, ws_lse, max_len, h_q, h_kv,
                     h_q / h_kv, block, top_k, sm_scale * kLog2e, nsplit);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nsplit == 1) return err;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(batch * h_q), dim3(D), 0, stream, ws_o,
                     ws_lse, static_cast<uint16_t*>(out), lse, nsplit);
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* kv_lens, const int32_t* sel, void* out, float* lse,
                              int batch, int max_len, int h_q, int h_kv, int d, int block,
                              int top_k, float sm_scale, void* workspace, int nsplit,
                              hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (d == 128)
    return launch_decode_t<128>(q, k_cache, v_cache, kv_lens, sel, out, lse, batch, max_len, h_q,
                                h_kv, block, top_k, sm_scale, workspace, nsplit, stream);
  if (d == 64)
    return launch_decode_t<64>(q, k_cache, v_cache, kv_lens, sel, out, lse, batch, max_len, h_q,
                               h_kv, block, top_k, sm_scale, workspace, nsplit, stream);
  return hipErrorInvalidValue;
}

}  // namespace qsa
