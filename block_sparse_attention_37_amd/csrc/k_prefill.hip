// Block-sparse prefill attention on bf16 matrix cores (gfx950 MFMA), online softmax.
//
// Qwen4-Exp model page, overview: each query attends to its selected contiguous token
// blocks plus its own incomplete trailing block, uncompressed; usage tips: the selected
// tokens feed ordinary softmax attention; num_attention_heads / num_key_value_heads give
// grouped-query attention.
//
// Work decomposition
//   * A workgroup (4 waves) owns MQ = 4 * (32 / G) consecutive query positions of one
//     KV head g; a wave owns 32 MFMA rows = (32 / G) positions x the G query heads that
//     read KV head g.  All G heads of a position share its selection, so the rows of a
//     wave differ in selection only per position.
//   * The workgroup walks the UNION of the blocks its positions need (selected blocks
//     plus the own blocks of positions whose trailing part is non-empty), kept as a
//     bitmap in LDS and visited in ascending order.  Each block is streamed through LDS in
//     chunks of 64 keys (K row-major, V transposed), double-buffered: the global loads of
//     chunk u+1 are in flight while chunk u is multiplied.
//   * Per row visibility of a block: the lane walks its position's ascending selection
//     list in step with the union (one compare per block), or the block is the
//     position's own block with a non-empty trailing part; keys after p are masked
//     (causal part of the trailing block).  A wave with no visible row skips the block.
//   * Transposed products keep one query row per lane:  S^T = K . Q^T  (A = K from LDS,
//     B = Q^T held in registers) and  O^T = V^T . P^T  (A = V^T from LDS, B = P^T taken
//     straight from the S^T accumulators, the key order inside an MFMA step permuted
//     identically on both operands).  Row max/sum need one exchange with lane ^ 32.
#include "qsa_device.h"
#include "qsa_internal.h"

#include <climits>

namespace qsa {

namespace {

constexpr int KC = 64;  // keys per LDS chunk

struct ChunkIter {
  int wi;         // bitmap word index
  uint32_t bits;  // remaining bits of that word
  int j;          // current block
  int sub;        // 64-key sub-chunk inside the block
};

__device__ __forceinline__ bool next_block(const uint32_t* bm, int words, ChunkIter& it) {
  while (it.bits == 0u) {
    if (++it.wi >= words) return false;
    it.bits = bm[it.wi];
  }
  const int t = __builtin_ctz(it.bits);
  it.bits &= it.bits - 1u;
  it.j = it.wi * 32 + t;
  it.sub = 0;
  return true;
}

__device__ __forceinline__ bool advance(const uint32_t* bm, int words, int nsub, ChunkIter& it) {
  if (it.sub + 1 < nsub) {
    ++it.sub;
    return true;
  }
  return next_block(bm, words, it);
}

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ sel, uint16_t* __restrict__ out,
    float* __restrict__ lse, int seq, int h_q, int h_kv, int block, int top_k, float scale_log2,
    int ntiles, int total_wg) {
  constexpr int PW = 32 / G;       // positions per wave
  constexpr int MQ = 4 * PW;       // positions per workgroup
  constexpr int NC16 = D / 8;      // 16-byte chunks per key row
  constexpr int KIT = KC * NC16 / 256;  // K 16-byte items per lane per chunk
  constexpr int VQ = KC / 4 * NC16;     // V items (4 keys x 16 bytes)
  constexpr int NDT = D / 32;      // 32-wide d tiles of O^T
  constexpr int NKS = D / 16;      // k-steps of S^T = K . Q^T

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KC * D];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * KC];
  extern __shared__ __attribute__((aligned(16))) int32_t dyn[];
  int32_t* sel_s = dyn;                                         // [MQ][top_k]
  uint32_t* bm = reinterpret_cast<uint32_t*>(dyn + MQ * top_k);  // union bitmap

  // ---- which tile: consecutive tiles of one head land on the same XCD (L2) ----
  const int wg = blockIdx.x;
  const int per = total_wg / 8;
  const int logical = (wg < per * 8) ? (wg % 8) * per + wg / 8 : wg;
  const int tile = logical % ntiles;
  const int g = (logical / ntiles) % h_kv;
  const int b = logical / (ntiles * h_kv);
  const int p0 = tile * MQ;
  const int p_hi = min(p0 + MQ, seq) - 1;
  const int words = (p_hi / block) / 32 + 1;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- selection rows of the tile -> LDS; union bitmap ----
  for (int e = tid; e < MQ * top_k; e += 256) {
    const int pos = e / top_k;
    const int p = p0 + pos;
    int j = INT_MAX;
    if (p < seq) {
      const int jj = sel[((size_t)b * seq + p) * top_k + (e - pos * top_k)];
      if (jj >= 0 && jj < (p + 1) / block) j = jj;
    }
    sel_s[e] = j;
  }
  for (int w = tid; w < words; w += 256) bm[w] = 0u;
  __syncthreads();
  for (int e = tid; e < MQ * top_k; e += 256) {
    const int j = sel_s[e];
    if (j != INT_MAX) atomicOr(&bm[j >> 5], 1u << (j & 31));
  }
  if (tid < MQ) {
    const int p = p0 + tid;
    if (p < seq && (p + 1) % block != 0) {
      const int j = p / block;
      atomicOr(&bm[j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();

  // ---- this lane's query row ----
  const int row = lane & 31;
  const int half = lane >> 5;
  const int pos = wave * PW + row / G;
  const int hh = g * G + row % G;
  const int p = p0 + pos;
  const bool valid_row = p < seq;
  const int own_block = (valid_row && (p + 1) % block != 0) ? p / block : -1;

  bf16x8 qreg[NKS];
  {
    const uint16_t* qp = q + (((size_t)b * seq + (valid_row ? p : 0)) * h_q + hh) * D + half * 8;
#pragma unroll
    for (int t = 0; t < NKS; ++t) qreg[t] = bitcast<bf16x8>(*reinterpret_cast<const u32x4*>(qp + t * 16));
  }

  int ptr = 0;
  int cur_sel = valid_row ? sel_s[pos * top_k] : INT_MAX;
  bool vis = false;

  float m_run = -__builtin_inff();
  float l_run = 0.f;
  f32x16 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;

  const int nsub = (block + KC - 1) / KC;
  const uint32_t kv_row = (uint32_t)h_kv * D;  // elements between consecutive tokens
  const uint16_t* kbase = k + ((size_t)b * seq * h_kv + g) * D;
  const uint16_t* vbase = v + ((size_t)b * seq * h_kv + g) * D;

  // K goes global -> LDS directly (no registers): wave-instruction i fills rows
  // i*(256/NC16) + wave*RPI .. +RPI-1, lane -> (row lane/NC16, physical chunk lane%NC16),
  // so the lane fetches the logical chunk that the XOR swizzle maps to that slot.
  constexpr int RPI = 64 / NC16;
  const int wave_u = wave_uniform(wave);
  const int k_lrow = lane / NC16;
  const int k_pc = lane % NC16;
  // V rows vq*4+i (chunk vc) are staged in registers and written transposed.
  const int vc = tid % NC16, vq = tid / NC16;
  u32x4 vreg[4];

  auto chunk_keys = [&](const ChunkIter& it, int& key0, int& ck) {
    key0 = it.j * block + it.sub * KC;
    ck = min(KC, block - it.sub * KC);
    ck = min(ck, seq - key0);
  };

  // Rows past the chunk are clamped into the tensor; their keys are masked.
  auto load_chunk = [&](const ChunkIter& it, int buf) {
    const int key0 = it.j * block + it.sub * KC;
#pragma unroll
    for (int i = 0; i < KIT; ++i) {
      const int r = i * (256 / NC16) + wave_u * RPI + k_lrow;
      const int c = k_pc ^ (r & (NC16 - 1));
      const uint32_t row = (uint32_t)min(key0 + r, seq - 1);
      global_to_lds16(kbase + row * kv_row + c * 8, &Ks[buf][(i * (256 / NC16) + wave_u * RPI) * D]);
    }
    if (tid < VQ) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t row = (uint32_t)min(key0 + vq * 4 + i, seq - 1);
        vreg[i] = *reinterpret_cast<const u32x4*>(vbase + row * kv_row + vc * 8);
      }
    }
  };

  auto store_chunk = [&](int buf) {
    if (tid < VQ) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // element pairs (2w, 2w+1) of the 4 rows -> V^T rows d = vc*8 + 2w, +1
        const uint32_t e0lo = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
        const uint32_t e0hi = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x05040100u);
        const uint32_t e1lo = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
        const uint32_t e1hi = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x07060302u);
        const int d0 = vc * 8 + 2 * w, d1 = d0 + 1;
        *reinterpret_cast<u32x2*>(&Vt[buf][d0 * KC + ((vq ^ ((d0 >> 1) & 15)) * 4)]) = u32x2{e0lo, e0hi};
        *reinterpret_cast<u32x2*>(&Vt[buf][d1 * KC + ((vq ^ ((d1 >> 1) & 15)) * 4)]) = u32x2{e1lo, e1hi};
      }
    }
  };

  ChunkIter cur{0, bm[0], -1, 0};
  bool have = next_block(bm, words, cur);
  if (have) {
    load_chunk(cur, 0);
    store_chunk(0);
  }
  wait_all_memory();  // LDS-direct loads are counted by vmcnt
  __syncthreads();
  int buf = 0;
  const float ninf = -__builtin_inff();

  while (have) {
    ChunkIter nxt = cur;
    const bool have_next = advance(bm, words, nsub, nxt);
    if (have_next) load_chunk(nxt, buf ^ 1);

    if (cur.sub == 0) {
      const bool hit = (cur_sel == cur.j);
      if (hit) {
        ++ptr;
        cur_sel = (ptr < top_k) ? sel_s[pos * top_k + ptr] : INT_MAX;
      }
      vis = valid_row && (hit || cur.j == own_block);
    }

    if (__ballot(vis) != 0ull) {
      int key0, ck;
      chunk_keys(cur, key0, ck);
      const bool emask = ck < KC || key0 + KC - 1 > p0;  // keys past the chunk or after p
      // one 32-key tile at a time: S^T tile -> online softmax -> P^T -> O^T update
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (kt == 1 && ck <= 32) break;
        f32x16 S;
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = 0.f;
        {
          const int kr = kt * 32 + row;
#pragma unroll
          for (int t = 0; t < NKS; ++t) {
            const int c = t * 2 + half;
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Ks[buf][kr * D + ((c ^ (kr & (NC16 - 1))) * 8)]);
            S = mfma32x32x16(a, qreg[t], S);
          }
        }
        if (emask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr = kt * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
            if (kr >= ck || key0 + kr > p) S[r] = ninf;
          }
        }
        float mx = ninf;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // the running max moves only when it grows by more than 8 (log2 units): rare
        // rescales, and every exponent below stays <= 8
        const float m_cand = vis ? fmaxf(m_run, mx * scale_log2) : m_run;
        const bool need = m_cand > m_run + 8.0f;
        if (__ballot(need) != 0ull) {
          const float m_new = need ? m_cand : m_run;
          // lanes that keep their max (possibly still -inf) keep their state exactly
          const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
        }
        const float nb = (vis && m_run != ninf) ? -m_run : ninf;
        float psum = 0.f;
        bf16x8 P[2];
#pragma unroll
        for (int uu = 0; uu < 2; ++uu) {
          u32x4 w;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * uu + 2 * jj], scale_log2, nb));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[8 * uu + 2 * jj + 1], scale_log2, nb));
            psum += e0 + e1;
            w[jj] = pack_bf16x2(e0, e1);
          }
          P[uu] = bitcast<bf16x8>(w);
        }
        l_run += psum;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int d = dt * 32 + row;
          const int sw = (d >> 1) & 15;
#pragma unroll
          for (int uu = 0; uu < 2; ++uu) {
            const int u = 2 * kt + uu;
            const u32x2 lo = *reinterpret_cast<const u32x2*>(&Vt[buf][d * KC + (((4 * u + half) ^ sw) * 4)]);
            const u32x2 hi = *reinterpret_cast<const u32x2*>(&Vt[buf][d * KC + (((4 * u + 2 + half) ^ sw) * 4)]);
            const bf16x8 a = bitcast<bf16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
            O[dt] = mfma32x32x16(a, P[uu], O[dt]);
          }
        }
      }
    }

    if (have_next) store_chunk(buf ^ 1);
    wait_all_memory();
    __syncthreads();
    buf ^= 1;
    cur = nxt;
    have = have_next;
  }

  // ---- epilogue ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (valid_row) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = out + (((size_t)b * seq + p) * h_q + hh) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = dt * 32 + 8 * rg + 4 * half;
        u32x2 w{pack_bf16x2(O[dt][4 * rg] * inv, O[dt][4 * rg + 1] * inv),
                pack_bf16x2(O[dt][4 * rg + 2] * inv, O[dt][4 * rg + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + d0) = w;
      }
    }
    if (lse && half == 0)
      lse[((size_t)b * seq + p) * h_q + hh] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
  }
}

template <int D, int G>
static size_t prefill_dyn_lds(int seq, int block, int top_k) {
  constexpr int MQ = 4 * (32 / G);
  const int words = ((seq - 1) / block) / 32 + 1;
  return (size_t)(MQ * top_k + words) * 4;
}

bool prefill_bf16_supported(int group, int d, int block, int top_k, int seq) {
  if (d != 64 && d != 128) return false;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16 && group != 32) return false;
  if (block < 1 || block > 1024 || top_k < 1 || top_k > kMaxTopK) return false;
  const int mq = 4 * (32 / group);
  const size_t dyn = (size_t)(mq * top_k + ((seq - 1) / block) / 32 + 1) * 4;
  const size_t stat = (size_t)2 * 2 * KC * d * 2;
  if ((long long)seq * 32 * d >= (1ll << 31)) return false;  // 32-bit offsets within a sequence
  return stat + dyn <= 96 * 1024;
}

template <int D, int G>
static hipError_t launch_prefill_t(const void* q, const void* k, const void* v, const int32_t* sel,
                                   void* out, float* lse, int batch, int seq, int h_q, int h_kv,
                                   int block, int top_k, float sm_scale, hipStream_t stream) {
  constexpr int MQ = 4 * (32 / G);
  const int ntiles = (seq + MQ - 1) / MQ;
  const long long total = (long long)ntiles * h_kv * batch;
  if (total > INT_MAX) return hipErrorInvalidValue;
  const size_t dyn = prefill_dyn_lds<D, G>(seq, block, top_k);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G>), dim3((unsigned)total), dim3(256), dyn, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), sel, static_cast<uint16_t*>(out), lse, seq,
                     h_q, h_kv, block, top_k, sm_scale * kLog2e, ntiles, (int)total);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(int group, const void* q, const void* k, const void* v,
                                   const int32_t* sel, void* out, float* lse, int batch, int seq,
                                   int h_q, int h_kv, int block, int top_k, float sm_scale,
                                   hipStream_t stream) {
  switch (group) {
    case 1: return launch_prefill_t<D, 1>(q, k, v, sel, out, lse, batch, seq, h_q, h_kv, block, top_k, sm_scale, stream);
    case 2: return launch_prefill_t<D, 2>(q, k, v, sel, out, lse, batch, seq, h_q, h_kv, block, top_k, sm_scale, stream);
    case 4: return launch_prefill_t<D, 4>(q, k, v, sel, out, lse, batch, seq, h_q, h_kv, block, top_k, sm_scale, stream);
    case 8: return launch_prefill_t<D, 8>(q, k, v, sel, out, lse, batch, seq, h_q, h_kv, block, top_k, sm_scale, stream);
    case 16: return launch_prefill_t<D, 16>(q, k, v, sel, out, lse, batch, seq, h_q, h_kv, block, top_k, sm_scale, stream);
    case 32: return launch_prefill_t<D, 32>(q, k, v, sel, out, lse, batch, seq, h_q, h_kv, block, top_k, sm_scale, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, const int32_t* sel,
                               void* out, float* lse, int batch, int seq, int h_q, int h_kv,
                               int d, int block, int top_k, float sm_scale, hipStream_t stream) {
  if (batch == 0 || seq == 0) return hipSuccess;
  const int group = h_q / h_kv;
  if (d == 128)
    return launch_prefill_d<128>(group, q, k, v, sel, out, lse, batch, seq, h_q, h_kv, block, top_k, sm_scale, stream);
  if (d == 64)
    return launch_prefill_d<64>(group, q, k, v, sel, out, lse, batch, seq, h_q, h_kv, block, top_k, sm_scale, stream);
  return hipErrorInvalidValue;
}

}  // namespace qsa
