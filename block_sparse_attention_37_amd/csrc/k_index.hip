// Indexer scores + per-query top-k block selection, fused; scores never reach HBM.
//
// Qwen4-Exp model page, overview: several indexer query heads score the compressed key
// blocks and each query keeps its most relevant contiguous blocks; Qwen4ExpTextConfig:
// indexer_n_heads (query heads), indexer_kv_heads (one key head), indexer_head_dim,
// indexer_budget (tokens kept from complete blocks, here top_k blocks).
//
// Score of block j for a query = sum over heads of <iq_h, cmp_j> = <sum_h iq_h, cmp_j>;
// the head sum is formed once per query in float32.  Candidates are the complete blocks
// j < n(p) = floor((p+1)/block).  Ranking is by (score desc, block index asc).
//
// Several queries per sequence (prefill): one workgroup handles QT consecutive queries:
//   1. head-summed queries -> LDS ([dim][query], read back as broadcasts),
//   2. every lane scores some blocks for all QT queries (compressed keys come from L2,
//      each row read once per workgroup) -> scores in LDS,
//   3. one wave per query selects (select_topk_wave: a bitwise search for the m-th largest
//      score with wave ballots, ties to the lowest block ids, ids written in ascending
//      order).  No sorting network, no atomics: the result is deterministic.
// One query per sequence (decode steps, single-token chunks): index_topk_one_kernel spends
// a 1024-lane workgroup on each sequence, reading the compressed keys coalesced.
#include "block_mean.h"
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

namespace {

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
}
template <typename F>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t x, F op) {
  x = op(x, dpp_u32<0xb1>(x));   // quad_perm [1,0,3,2]
  x = op(x, dpp_u32<0x4e>(x));   // quad_perm [2,3,0,1]
  x = op(x, dpp_u32<0x141>(x));  // row_half_mirror
  x = op(x, dpp_u32<0x140>(x));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = op(a[0], a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (uint32_t)wave_uniform((int)op(c[0], c[1]));
}

// Keeps the top m = min(top_k, n) of the n scores sc[0..n) (LDS), ranked by (score desc,
// block id asc), on one wave: the candidates sit in NR registers per lane (block
// j = r*64 + lane); a bitwise search on the order-preserving integer image of the scores
// finds the m-th largest value with wave ballots, starting below the bits that every
// valid key shares (from the wave max and min) and stopping once exactly m keys reach the
// threshold (the kept set is then fixed); ties at the threshold go to the lowest ids; the
// kept ids are written in ascending order (ballot prefix counts) to out[0..m), then -1 up
// to top_k; out_scores (optional) gets their scores, -inf after.
template <int NR>
__device__ __forceinline__ void select_topk_wave(const float* sc, int n, int top_k, int lane,
                                                 int32_t* __restrict__ out,
                                                 float* __restrict__ out_scores) {
  const uint64_t lt = lanemask_lt();
  const int m = min(top_k, n);
  uint32_t key[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int j = r * 64 + lane;
    key[r] = (j < n) ? orderable(sc[j]) : 0u;  // valid keys are >= 1
  }
  // threshold: the largest value t built bit by bit with at least m keys >= t (the m-th
  // largest key, or a value below it with exactly m keys above); 0 keeps every candidate
  uint32_t thr = 0;
  if (m < n) {
    uint32_t hi = 0u, lo = 0xffffffffu;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      hi = max(hi, key[r]);
      lo = key[r] != 0u ? min(lo, key[r]) : lo;
    }
    hi = wave_reduce_u32(hi, [](uint32_t a, uint32_t b) { return max(a, b); });
    lo = wave_reduce_u32(lo, [](uint32_t a, uint32_t b) { return min(a, b); });
    if (hi == lo) {
      thr = hi;  // every valid key is equal
    } else {
      int bit = 31 - __builtin_clz(hi ^ lo);
      thr = hi & ~((2u << bit) - 1u);  // the bits above `bit`, shared by every valid key
      for (; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int r = 0; r < NR; ++r) cnt += __popcll(__ballot(key[r] >= cand));
        if (cnt >= m) {
          thr = cand;
          if (cnt == m) break;
        }
      }
    }
  }
  int cnt_gt = 0;
#pragma unroll
  for (int r = 0; r < NR; ++r) cnt_gt += __popcll(__ballot(key[r] > thr));
  const int need = m - cnt_gt;  // ties at thr to take, lowest ids first

  int base = 0, eq_seen = 0;
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const bool eq = (key[r] == thr) && (key[r] != 0u);
    const uint64_t eqm = __ballot(eq);
    const bool take = (key[r] > thr) || (eq && (eq_seen + __popcll(eqm & lt)) < need);
    eq_seen += __popcll(eqm);
    const uint64_t tm = __ballot(take);
    if (take) {
      const int pos = base + __popcll(tm & lt);
      const int j = r * 64 + lane;
      out[pos] = j;
      if (out_scores) out_scores[pos] = sc[j];
    }
    base += __popcll(tm);
  }
  for (int pos = m + lane; pos < top_k; pos += 64) {
    out[pos] = -1;
    if (out_scores) out_scores[pos] = -__builtin_inff();
  }
}

// acc[k] += element k of a 16-byte load of T values (8 bf16 or 4 float).
template <typename T>
__device__ __forceinline__ void add_row16(float* acc, const u32x4& v) {
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

}  // namespace

template <typename T, int NR, int QT>
__global__ __launch_bounds__(256) void index_topk_kernel(
    const T* __restrict__ iq, const float* __restrict__ cmp, const int32_t* __restrict__ kv_lens,
    int32_t* __restrict__ sel, float* __restrict__ sel_scores, int n_q, int h_idx, int d_idx,
    int max_blocks, int block, int top_k) {
  constexpr int NC = NR * 64;
  __shared__ float qs[128][QT];  // d_idx <= 128
  __shared__ float sc[QT][NC];

  const int b = blockIdx.y;
  const int i0 = blockIdx.x * QT;
  const int tid = threadIdx.x;
  const int len = kv_lens ? kv_lens[b] : n_q;
  const int nq_here = min(QT, n_q - i0);
  const int cap = min(max_blocks, NC);
  // query qi sits at position p0 + qi; positions < 0 are padding (a sequence shorter than
  // n_q): no candidates, so their rows are all -1
  const int p0 = len - n_q + i0;
  if (p0 + nq_here - 1 < 0) {  // padding only: no loads, no barrier
    for (int e = tid; e < nq_here * top_k; e += 256) {
      const size_t o = ((size_t)b * n_q + i0) * top_k + e;
      sel[o] = -1;
      if (sel_scores) sel_scores[o] = -__builtin_inff();
    }
    return;
  }

  // 1. head-summed indexer queries (zero for padding rows, which score nothing).  The QT
  // queries' indexer rows are one contiguous [QT][h_idx][d_idx] slab; a lane owns CPT
  // consecutive dims of one query and adds its heads in order from 16-byte loads, eight
  // heads in flight at a time.
  {
    constexpr int CPT = 16 / sizeof(T);
    const int lanes_per_q = d_idx / CPT;
    if (tid < QT * lanes_per_q) {
      const int qi = tid / lanes_per_q, c0 = (tid % lanes_per_q) * CPT;
      float acc[CPT];
#pragma unroll
      for (int k = 0; k < CPT; ++k) acc[k] = 0.f;
      if (qi < nq_here && p0 + qi >= 0) {
        const T* src = iq + ((size_t)b * n_q + i0 + qi) * h_idx * d_idx + c0;
        int h = 0;
        for (; h + 8 <= h_idx; h += 8) {
          u32x4 v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const u32x4*>(src + (size_t)(h + u) * d_idx);
#pragma unroll
          for (int u = 0; u < 8; ++u) add_row16<T>(acc, v[u]);
        }
        for (; h < h_idx; ++h) add_row16<T>(acc, *reinterpret_cast<const u32x4*>(src + (size_t)h * d_idx));
      }
#pragma unroll
      for (int k = 0; k < CPT; ++k) qs[c0 + k][qi] = acc[k];
    }
  }
  __syncthreads();

  // 2. scores of candidate blocks (the last query of the tile sees the most)
  const int p_last = p0 + nq_here - 1;
  const int n_last = max(0, min((p_last + 1) / block, cap));
  // One row per lane and pass, 16 dims (four 16-byte loads) at a time.
  for (int j = tid; j < n_last; j += 256) {
    const float* row = cmp + ((size_t)b * max_blocks + j) * d_idx;
    float acc[QT];
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) acc[qi] = 0.f;
    for (int c0 = 0; c0 < d_idx; c0 += 16) {
      f32x4 kv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) kv[t] = *reinterpret_cast<const f32x4*>(row + c0 + 4 * t);
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc)
#pragma unroll
          for (int qi = 0; qi < QT; ++qi)
            acc[qi] = __builtin_fmaf(qs[c0 + 4 * t + cc][qi], kv[t][cc], acc[qi]);
    }
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) sc[qi][j] = acc[qi];
  }
  __syncthreads();

  // 3. selection, one wave per query
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int qi = wave; qi < nq_here; qi += 4) {
    const int p = p0 + qi;
    const int n = max(0, min((p + 1) / block, cap));
    const size_t orow = ((size_t)b * n_q + i0 + qi) * top_k;
    select_topk_wave<NR>(sc[qi], n, top_k, lane, sel + orow, sel_scores ? sel_scores + orow : nullptr);
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum of x over aligned groups of L lanes (L = 8, 16 or 32); every lane of a group gets it.
// Within a 16-lane row the partners come from DPP (quad swaps, then half-row and row
// mirrors); across the two rows of a 32-lane half, from v_permlane16_swap.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(L == 8 || L == 16 || L == 32, "group size");
  x += dpp_f32<0xb1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4e>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  if constexpr (L >= 16) x += dpp_f32<0x140>(x);  // row_mirror
  if constexpr (L >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

// Four consecutive elements of a T row, as float.
template <typename T>
__device__ __forceinline__ f32x4 load4(const T* p);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
template <>
__device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t* p) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p);
  return f32x4{bf16_to_f32(w[0] & 0xffffu), bf16_to_f32(w[0] >> 16), bf16_to_f32(w[1] & 0xffffu),
               bf16_to_f32(w[1] >> 16)};
}

// One query per sequence: the query sits at position kv_lens[b] - 1 (1 - 1 = 0 without
// kv_lens).  One 1024-lane workgroup per sequence:
//   1. every lane forms the head-summed query (float32, heads in order) for the four dims
//      it scores, 4 * (lane % (DI / 4)) ..; no LDS, no barrier;
//   2. the compressed-key rows are read whole, DI / 4 lanes per row, one 16-byte load each,
//      U rounds of loads in flight; a row's dot product is finished by group_sum -> LDS;
//   3. wave 0 selects (select_topk_wave).
// UPD (decode step with the indexer-state update): before scoring, a sequence whose length
// L is a positive multiple of `block` gets the block its newest token completes,
// j = L / block - 1, compressed from the indexer-key cache `ik` (BlockMean, bit-identical
// to the compression kernel) and written to cmp; that block is scored from the LDS copy.
template <typename T, int DI, int NR, bool UPD>
__global__ __launch_bounds__(1024) void index_topk_one_kernel(
    const T* __restrict__ iq, float* cmp, const int32_t* __restrict__ kv_lens,
    int32_t* __restrict__ sel, float* __restrict__ sel_scores, int h_idx, int max_blocks,
    int block, int top_k, const T* __restrict__ ik, int ik_max_len) {
  constexpr int NC = NR * 64;
  constexpr int LPR = DI / 4;     // lanes per compressed-key row
  constexpr int RPW = 64 / LPR;   // rows per wave and round
  constexpr int RPR = 16 * RPW;   // rows per round (16 waves)
  constexpr int U = 4;            // rounds whose loads are in flight together
  __shared__ float sc[NC];
  __shared__ float part[UPD ? BlockMean<T, DI>::SCRATCH : 1];
  __shared__ float newrow[UPD ? DI : 1];

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int len = kv_lens ? kv_lens[b] : 1;
  const int n = max(0, min(len / block, min(max_blocks, NC)));

  int j_new = -1;
  if constexpr (UPD) {
    if (len > 0 && len <= ik_max_len && len % block == 0 && len / block <= max_blocks) {
      j_new = len / block - 1;
      const float m = BlockMean<T, DI>::run(
          ik + ((size_t)b * ik_max_len + (size_t)j_new * block) * DI, block, part, tid);
      if (tid < DI) {
        newrow[tid] = m;
        cmp[((size_t)b * max_blocks + j_new) * DI + tid] = m;
      }
      __syncthreads();
    }
  }

  const int sub = lane % LPR;
  const int c0 = 4 * sub;
  f32x4 qv = {0.f, 0.f, 0.f, 0.f};
  {
    const T* src = iq + (size_t)b * h_idx * DI + c0;
    for (int h = 0; h < h_idx; ++h) qv += load4<T>(src + (size_t)h * DI);
  }

  const int rw = wave * RPW + lane / LPR;  // this lane's row within a round
  const float* crow = cmp + (size_t)b * max_blocks * DI + c0;
  for (int r0 = 0; r0 < n; r0 += U * RPR) {
    f32x4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = r0 + u * RPR + rw;
      kv[u] = j < n ? *reinterpret_cast<const f32x4*>(crow + (size_t)j * DI) : f32x4{0.f, 0.f, 0.f, 0.f};
      if (UPD && j == j_new) kv[u] = *reinterpret_cast<const f32x4*>(newrow + c0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float acc = qv[0] * kv[u][0];
      acc = __builtin_fmaf(qv[1], kv[u][1], acc);
      acc = __builtin_fmaf(qv[2], kv[u][2], acc);
      acc = __builtin_fmaf(qv[3], kv[u][3], acc);
      acc = group_sum<LPR>(acc);
      const int j = r0 + u * RPR + rw;
      if (sub == 0 && j < n) sc[j] = acc;
    }
  }
  __syncthreads();

  if (wave == 0)
    select_topk_wave<NR>(sc, n, top_k, lane, sel + (size_t)b * top_k,
                         sel_scores ? sel_scores + (size_t)b * top_k : nullptr);
}

template <typename T, int NR, int QT>
static hipError_t launch_index_t(const void* iq, const float* cmp, const int32_t* kv_lens,
                                 int32_t* sel, float* sel_scores, int batch, int n_q, int h_idx,
                                 int d_idx, int max_blocks, int block, int top_k,
                                 hipStream_t stream) {
  dim3 grid((n_q + QT - 1) / QT, batch);
  hipLaunchKernelGGL((index_topk_kernel<T, NR, QT>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(iq), cmp, kv_lens, sel, sel_scores, n_q, h_idx, d_idx,
                     max_blocks, block, top_k);
  return hipGetLastError();
}

template <typename T, int NR, bool UPD>
static hipError_t launch_index_one(const void* iq, float* cmp, const int32_t* kv_lens,
                                   int32_t* sel, float* sel_scores, int batch, int h_idx,
                                   int d_idx, int max_blocks, int block, int top_k,
                                   const void* ik, int ik_max_len, hipStream_t stream) {
#define QSA_ONE(DI)                                                                           \
  hipLaunchKernelGGL((index_topk_one_kernel<T, DI, NR, UPD>), dim3(batch), dim3(1024), 0, stream, \
                     static_cast<const T*>(iq), cmp, kv_lens, sel, sel_scores, h_idx,           \
                     max_blocks, block, top_k, static_cast<const T*>(ik), ik_max_len);          \
  return hipGetLastError()
  if (d_idx == 32) { QSA_ONE(32); }
  if (d_idx == 64) { QSA_ONE(64); }
  if (d_idx == 128) { QSA_ONE(128); }
#undef QSA_ONE
  return hipErrorInvalidValue;
}

template <typename T, int NR>
static hipError_t launch_index_nr(const void* iq, const float* cmp, const int32_t* kv_lens,
                                  int32_t* sel, float* sel_scores, int batch, int n_q, int h_idx,
                                  int d_idx, int max_blocks, int block, int top_k,
                                  const void* ik, int ik_max_len, float* cmp_out,
                                  hipStream_t stream) {
  if (cmp_out != nullptr)  // decode step with the indexer-state update (cmp_out == cmp)
    return launch_index_one<T, NR, true>(iq, cmp_out, kv_lens, sel, sel_scores, batch, h_idx,
                                         d_idx, max_blocks, block, top_k, ik, ik_max_len, stream);
  if (n_q == 1)
    return launch_index_one<T, NR, false>(iq, const_cast<float*>(cmp), kv_lens, sel, sel_scores,
                                          batch, h_idx, d_idx, max_blocks, block, top_k, nullptr,
                                          0, stream);
  // Queries per workgroup.  Scoring runs on as many lanes as there are candidates and
  // selection on one wave per query, so a workgroup's time grows with its queries; small
  // tiles keep many workgroups resident (LDS for scores: QT * NR * 256 bytes) and were
  // measured fastest (4 up to 256 candidates, 8 beyond).
  constexpr int QTM = NR <= 4 ? 4 : NR <= 32 ? 8 : 4;
  return launch_index_t<T, NR, QTM>(iq, cmp, kv_lens, sel, sel_scores, batch, n_q, h_idx, d_idx,
                                    max_blocks, block, top_k, stream);
}

template <typename T>
static hipError_t launch_index_dt(const void* iq, const float* cmp, const int32_t* kv_lens,
                                  int32_t* sel, float* sel_scores, int batch, int n_q, int h_idx,
                                  int d_idx, int max_blocks, int block, int top_k,
                                  const void* ik, int ik_max_len, float* cmp_out,
                                  hipStream_t stream) {
#define QSA_NR(nr)                                                                           \
  return launch_index_nr<T, nr>(iq, cmp, kv_lens, sel, sel_scores, batch, n_q, h_idx, d_idx, \
                                max_blocks, block, top_k, ik, ik_max_len, cmp_out, stream)
  const int need = max_blocks;
  if (need <= 128) QSA_NR(2);
  if (need <= 256) QSA_NR(4);
  if (need <= 512) QSA_NR(8);
  if (need <= 1024) QSA_NR(16);
  if (need <= 2048) QSA_NR(32);
  QSA_NR(64);
#undef QSA_NR
}

hipError_t launch_index_topk(const void* iq, const float* cmp, const int32_t* kv_lens,
                             int32_t* sel, float* sel_scores, int batch, int n_q, int h_idx,
                             int d_idx, int max_blocks, int block, int top_k, bool bf16,
                             hipStream_t stream) {
  if (batch == 0 || n_q == 0) return hipSuccess;
  if (bf16)
    return launch_index_dt<uint16_t>(iq, cmp, kv_lens, sel, sel_scores, batch, n_q, h_idx, d_idx,
                                     max_blocks, block, top_k, nullptr, 0, nullptr, stream);
  return launch_index_dt<float>(iq, cmp, kv_lens, sel, sel_scores, batch, n_q, h_idx, d_idx,
                                max_blocks, block, top_k, nullptr, 0, nullptr, stream);
}

hipError_t launch_index_topk_decode(const void* iq, const void* ik, float* cmp,
                                    const int32_t* kv_lens, int32_t* sel, float* sel_scores,
                                    int batch, int max_len, int h_idx, int d_idx, int max_blocks,
                                    int block, int top_k, bool bf16, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (bf16)
    return launch_index_dt<uint16_t>(iq, cmp, kv_lens, sel, sel_scores, batch, 1, h_idx, d_idx,
                                     max_blocks, block, top_k, ik, max_len, cmp, stream);
  return launch_index_dt<float>(iq, cmp, kv_lens, sel, sel_scores, batch, 1, h_idx, d_idx,
                                max_blocks, block, top_k, ik, max_len, cmp, stream);
}

}  // namespace qsa
