// Block-sparse prefill attention on bf16 matrix cores (gfx950 MFMA), online softmax.
//
// Qwen4-Exp model page, overview: each query attends to its selected contiguous token
// blocks plus its own incomplete trailing block, uncompressed; usage tips: the selected
// tokens feed ordinary softmax attention; num_attention_heads / num_key_value_heads give
// grouped-query attention.
//
// Work decomposition
//   * A workgroup of NW waves owns MQ = NW * (32 / G) consecutive query positions of one
//     KV head g; a wave owns 32 MFMA rows = (32 / G) positions x the G query heads that
//     read KV head g.  All G heads of a position share its selection, so the rows of a
//     wave differ in selection only per position.
//   * The workgroup walks the UNION of the blocks its positions need (selected blocks
//     plus the own blocks of positions whose trailing part is non-empty), kept as a
//     bitmap in LDS and visited in ascending order.  Each block is streamed through LDS in
//     chunks of 64 keys.  K and V rows go global -> LDS directly (no registers) through
//     NS stages: while chunk u is multiplied, chunks u+1 .. u+NS-1 are in flight.  Every
//     chunk is shared by the NW waves (256 MFMA rows), which sets the flops per byte of L2
//     traffic.
//   * Per row visibility of a block: the lane walks its position's ascending selection
//     list in step with the union (one compare per block), or the block is the
//     position's own block with a non-empty trailing part; keys after p are masked
//     (causal part of the trailing block).  A wave with no visible row skips the block.
//   * Transposed products keep one query row per lane:  S^T = K . Q^T  (A = K rows from
//     LDS, B = Q^T held in registers) and  O^T = V^T . P^T  (A = V^T gathered from the
//     row-major V tile by the LDS transpose read ds_read_b64_tr_b16, B = P^T taken straight
//     from the S^T accumulators; the key order inside an MFMA step is permuted identically
//     on both operands).  Row max and sum need one exchange with lane ^ 32.
//   * Online softmax in base 2 with the scale folded into one FMA per score; the running
//     max is raised only when it grows by more than 8 (log2 units), so rescaling the
//     accumulators is rare and every exponent stays <= 8.
#include "qsa_device.h"
#include "qsa_internal.h"

#include <climits>

namespace qsa {

namespace {

constexpr int KC = 64;   // keys per LDS chunk
constexpr int NW = 8;    // waves per workgroup
constexpr int NS = 4;    // LDS stages (chunks in flight + the one being used)

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int N>
struct Int {
  static constexpr int value = N;
};

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

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
#endif
}

// Workgroup barrier without the memory fence __syncthreads() implies: that fence would
// drain every outstanding LDS-direct load.  The loop waits for exactly the chunk it needs
// (wait_vmcnt) before the barrier; the LDS it reads was filled only by those loads, and
// the clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_no_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_barrier" ::: "memory");
#endif
}

__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return bitcast<u32x2>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
#else
  (void)p;
  return u32x2{0u, 0u};
#endif
}

// XOR swizzles of 16-byte chunks inside a row of the LDS tiles.
//  K: row r, chunk c -> c ^ (r mod NC16): the 32 rows an MFMA operand read touches at one
//     chunk spread over all banks.
//  V: the transpose read touches 8 consecutive rows x 64 bytes; rows r..r+3 must use
//     disjoint 64-byte column groups.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(NW * 64, 1) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ sel, uint16_t* __restrict__ out,
    float* __restrict__ lse, int seq, int h_q, int h_kv, int block, int top_k, float scale_log2,
    int ntiles, int total_wg) {
  constexpr int NT = NW * 64;
  constexpr int PW = 32 / G;       // positions per wave
  constexpr int MQ = NW * PW;      // positions per workgroup
  constexpr int NC16 = D / 8;      // 16-byte chunks per key row
  constexpr int RPI = 64 / NC16;   // rows one wave fills per LDS-direct instruction
  constexpr int RPP = NW * RPI;    // rows all waves fill per instruction
  constexpr int DPT = KC / RPP;    // instructions per wave per tile (K or V)
  constexpr int DPC = 2 * DPT;     // per chunk (K and V)
  constexpr int NDT = D / 32;      // 32-wide d tiles of O^T
  constexpr int NKS = D / 16;      // k-steps of S^T = K . Q^T
  static_assert(KC % RPP == 0, "tile rows");

  // One array per stage (K rows, then V rows): every access below names its array
  // statically, and all LDS the loop reads is statically allocated, so the compiler can
  // tell the in-flight LDS-direct loads of other stages from the reads of this one and
  // does not drain the load queue before each LDS read.
  __shared__ __attribute__((aligned(16))) uint16_t KV0[2 * KC * D], KV1[2 * KC * D],
      KV2[2 * KC * D], KV3[2 * KC * D];
  static_assert(NS == 4, "one named array per stage");
  __shared__ int32_t sel_s[kPrefillSelCap];    // [MQ][top_k]
  __shared__ uint32_t bm[kPrefillMaxBlocks / 32];  // union bitmap

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
  const int wave = wave_uniform(tid >> 6);

  // ---- selection rows of the tile -> LDS; union bitmap ----
  for (int e = tid; e < MQ * top_k; e += NT) {
    const int pos = e / top_k;
    const int p = p0 + pos;
    int j = INT_MAX;
    if (p < seq) {
      const int jj = sel[((size_t)b * seq + p) * top_k + (e - pos * top_k)];
      if (jj >= 0 && jj < (p + 1) / block) j = jj;
    }
    sel_s[e] = j;
  }
  for (int w = tid; w < words; w += NT) bm[w] = 0u;
  __syncthreads();
  for (int e = tid; e < MQ * top_k; e += NT) {
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
    for (int t = 0; t < NKS; ++t) {
      u32x4 w = *reinterpret_cast<const u32x4*>(qp + t * 16);
      // opaque to the optimizer: keeps Q in registers instead of re-loading it per chunk
      // (a re-load would also wait on the untracked K/V loads in flight)
      keep_in_register(w);
      qreg[t] = bitcast<bf16x8>(w);
    }
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

  // LDS-direct loads: wave instruction i fills rows i*RPP + wave*RPI .. +RPI-1; lane ->
  // (row lane / NC16, physical chunk lane % NC16) and fetches the logical chunk that the
  // swizzle maps to that slot.  Rows past the chunk are clamped into the tensor (masked).
  const int d_row = lane / NC16;
  const int d_pc = lane % NC16;
  auto issue = [&](const ChunkIter& it, auto stage_tag) __attribute__((always_inline)) {
    constexpr int SI = decltype(stage_tag)::value;
    const uint32_t kd = lds_addr(SI == 0 ? KV0 : SI == 1 ? KV1 : SI == 2 ? KV2 : KV3);
    const uint32_t vd = kd + KC * D * 2;
    const int key0 = it.j * block + it.sub * KC;
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
      const int r0 = i * RPP + wave * RPI;
      const int r = r0 + d_row;
      const uint32_t grow = (uint32_t)min(key0 + r, seq - 1);
      global_to_lds16_untracked(kbase + grow * kv_row + (d_pc ^ swz_k<D>(r)) * 8, kd + r0 * D * 2);
      global_to_lds16_untracked(vbase + grow * kv_row + (d_pc ^ swz_v<D>(r)) * 8, vd + r0 * D * 2);
    }
  };

  // transpose-read lane geometry (see the O^T product below)
  const int tr_g = lane >> 4, tr_m = lane & 15;
  const int tr_row = 4 * (tr_g >> 1) + (tr_m >> 2);      // + 16u (+8 for the upper 4 keys)
  const int tr_d = 16 * (tr_g & 1) + 4 * (tr_m & 3);     // + 32*dt

  ChunkIter it_issue{0, bm[0], -1, 0};
  bool more_issue = next_block(bm, words, it_issue);
  ChunkIter it = it_issue;
  bool more = more_issue;
  int issued = 0;
  auto issue_next = [&](auto stage_tag) __attribute__((always_inline)) {
    if (more_issue) {
      issue(it_issue, stage_tag);
      ++issued;
      more_issue = advance(bm, words, nsub, it_issue);
    }
  };
  issue_next(Int<0>{});
  issue_next(Int<1>{});
  issue_next(Int<2>{});

  const float ninf = -__builtin_inff();
  int u = 0;

  // One 32-key tile of the chunk in stage Kst: S^T tile -> online softmax -> P^T -> O^T.
  auto do_tile = [&](const uint16_t* Kst, const uint16_t* Vst, int kt, int key0, int ck,
                     bool emask) __attribute__((always_inline)) {
    f32x16 S;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = 0.f;
    {
      const int kr = kt * 32 + row;
#pragma unroll
      for (int t = 0; t < NKS; ++t) {
        const int c = t * 2 + half;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&Kst[kr * D + ((c ^ swz_k<D>(kr)) * 8)]);
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
    // A operand of step u: V at d = 32*dt + (lane % 32), keys 16u + 4*(lane/32) + {0..3}
    // and 16u + 8 + 4*(lane/32) + {0..3}; each half is one transpose read in which the
    // lane supplies row 16u + tr_row (+8), columns 32*dt + tr_d .. +3.
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int r_lo = 16 * (2 * kt + uu) + tr_row;
      const int r_hi = r_lo + 8;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int dcol = 32 * dt + tr_d;
        const u32x2 lo = lds_read_tr16(&Vst[r_lo * D + (((dcol >> 3) ^ swz_v<D>(r_lo)) * 8) + (dcol & 7)]);
        const u32x2 hi = lds_read_tr16(&Vst[r_hi * D + (((dcol >> 3) ^ swz_v<D>(r_hi)) * 8) + (dcol & 7)]);
        const bf16x8 a = bitcast<bf16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
        O[dt] = mfma32x32x16(a, P[uu], O[dt]);
      }
    }
  };

  // One chunk per call, stage S fixed at compile time.
  auto step = [&](auto stage_tag) __attribute__((always_inline)) -> bool {
    constexpr int S = decltype(stage_tag)::value;
    const uint16_t* Kst = S == 0 ? KV0 : S == 1 ? KV1 : S == 2 ? KV2 : KV3;
    const uint16_t* Vst = Kst + KC * D;
    if (!more) return false;
    // chunk u must have landed; the (at most NS-2) chunks after it may stay in flight
    const int after = issued - u - 1;
    if (after >= 2) wait_vmcnt<2 * DPC>();
    else if (after == 1) wait_vmcnt<DPC>();
    else wait_vmcnt<0>();
    barrier_no_fence();
    issue_next(Int<(S + NS - 1) % NS>{});  // refills the stage chunk u-1 used

    if (it.sub == 0) {
      const bool hit = (cur_sel == it.j);
      if (hit) {
        ++ptr;
        cur_sel = (ptr < top_k) ? sel_s[pos * top_k + ptr] : INT_MAX;
      }
      vis = valid_row && (hit || it.j == own_block);
    }
    if (__ballot(vis) != 0ull) {
      const int key0 = it.j * block + it.sub * KC;
      const int ck = min(min(KC, block - it.sub * KC), seq - key0);
      const bool emask = ck < KC || key0 + KC - 1 > p0;  // keys past the chunk or after p
      do_tile(Kst, Vst, 0, key0, ck, emask);
      if (ck > 32) do_tile(Kst, Vst, 1, key0, ck, emask);
    }

    more = advance(bm, words, nsub, it);
    ++u;
    return more;
  };
  while (step(Int<0>{}) && step(Int<1>{}) && step(Int<2>{}) && step(Int<3>{})) {
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

bool prefill_bf16_supported(int group, int d, int block, int top_k, int seq) {
  if (d != 64 && d != 128) return false;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16 && group != 32) return false;
  if (block < 1 || block > 1024 || top_k < 1 || top_k > kMaxTopK) return false;
  if ((long long)seq * 32 * d >= (1ll << 31)) return false;  // 32-bit offsets within a sequence
  if ((long long)NW * (32 / group) * top_k > kPrefillSelCap) return false;
  return (seq + block - 1) / block <= kPrefillMaxBlocks;
}

template <int D, int G>
static hipError_t launch_prefill_t(const void* q, const void* k, const void* v, const int32_t* sel,
                                   void* out, float* lse, int batch, int seq, int h_q, int h_kv,
                                   int block, int top_k, float sm_scale, hipStream_t stream) {
  constexpr int MQ = NW * (32 / G);
  const int ntiles = (seq + MQ - 1) / MQ;
  const long long total = (long long)ntiles * h_kv * batch;
  if (total > INT_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G>), dim3((unsigned)total), dim3(NW * 64), 0, stream,
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
