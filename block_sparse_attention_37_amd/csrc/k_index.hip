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
// One workgroup handles QT consecutive queries of one sequence:
//   1. head-summed queries -> LDS ([dim][query], read back as broadcasts),
//   2. every lane scores some blocks for all QT queries (compressed keys come from L2,
//      each row read once per workgroup) -> scores in LDS,
//   3. one wave per query: the candidates sit in NR registers per lane (block
//      j = r*64 + lane); a 32-step bitwise search on the order-preserving integer image of
//      the scores finds the m-th largest value with wave ballots; ties at that value go
//      to the lowest block ids; the kept ids come out in ascending order via ballot
//      prefix counts.  No sorting network, no atomics: the result is deterministic.
#include "block_mean.h"
#include "qsa_device.h"
#include "qsa_internal.h"

namespace qsa {

// UPD_DI > 0 (decode, QT == 1, d_idx == UPD_DI): before scoring, a sequence whose length L
// is a positive multiple of `block` gets the block its newest token completes,
// j = L / block - 1, compressed from the indexer-key cache `ik` (BlockMean, bit-identical to
// the compression kernel) and written to cmp; that block is scored from the LDS copy.
template <typename T, int NR, int QT, int UPD_DI>
__global__ __launch_bounds__(256) void index_topk_kernel(
    const T* __restrict__ iq, const float* cmp_in, const int32_t* __restrict__ kv_lens,
    int32_t* __restrict__ sel, float* __restrict__ sel_scores, int n_q, int h_idx, int d_idx,
    int max_blocks, int block, int top_k, const T* __restrict__ ik, int ik_max_len,
    float* cmp_out) {
  constexpr int NC = NR * 64;
  __shared__ float qs[128][QT];  // d_idx <= 128
  __shared__ float sc[QT][NC];
  __shared__ float part[UPD_DI > 0 ? BlockMean<T, (UPD_DI > 0 ? UPD_DI : 32)>::SCRATCH : 1];
  __shared__ float newrow[UPD_DI > 0 ? UPD_DI : 1];
  const float* cmp = cmp_in;

  const int b = blockIdx.y;
  const int i0 = blockIdx.x * QT;
  const int tid = threadIdx.x;
  const int len = kv_lens ? kv_lens[b] : n_q;
  const int nq_here = min(QT, n_q - i0);
  const int cap = min(max_blocks, NC);

  int j_new = -1;  // block compressed here (decode state update), scored from newrow
  if constexpr (UPD_DI > 0) {
    static_assert(QT == 1, "the state update is a decode step");
    if (len > 0 && len <= ik_max_len && len % block == 0 && len / block <= max_blocks) {
      j_new = len / block - 1;
      const float m = BlockMean<T, UPD_DI>::run(
          ik + ((size_t)b * ik_max_len + (size_t)j_new * block) * UPD_DI, block, part, tid);
      if (tid < UPD_DI) {
        newrow[tid] = m;
        cmp_out[((size_t)b * max_blocks + j_new) * UPD_DI + tid] = m;
      }
    }
  }

  // 1. head-summed indexer queries
  for (int e = tid; e < QT * d_idx; e += 256) {
    const int qi = e / d_idx, c = e % d_idx;
    float s = 0.f;
    if (qi < nq_here) {
      const T* src = iq + ((size_t)b * n_q + i0 + qi) * h_idx * d_idx + c;
      for (int h = 0; h < h_idx; ++h) s += Elem<T>::load(src, (size_t)h * d_idx);
    }
    qs[c][qi] = s;
  }
  __syncthreads();

  // 2. scores of candidate blocks (the last query of the tile sees the most)
  const int p_last = len - n_q + i0 + nq_here - 1;
  const int n_last = max(0, min((p_last + 1) / block, cap));
  for (int j = tid; j < n_last; j += 256) {
    const float* row = (UPD_DI > 0 && j == j_new) ? newrow : cmp + ((size_t)b * max_blocks + j) * d_idx;
    float acc[QT];
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) acc[qi] = 0.f;
    for (int c = 0; c < d_idx; c += 4) {
      const f32x4 kv = *reinterpret_cast<const f32x4*>(row + c);
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
        for (int qi = 0; qi < QT; ++qi) acc[qi] = __builtin_fmaf(qs[c + cc][qi], kv[cc], acc[qi]);
      }
    }
#pragma unroll
    for (int qi = 0; qi < QT; ++qi) sc[qi][j] = acc[qi];
  }
  __syncthreads();

  // 3. selection, one wave per query
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint64_t lt = lanemask_lt();
  for (int qi = wave; qi < nq_here; qi += 4) {
    const int p = len - n_q + i0 + qi;
    const int n = max(0, min((p + 1) / block, cap));
    const int m = min(top_k, n);
    uint32_t key[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int j = r * 64 + lane;
      key[r] = (j < n) ? orderable(sc[qi][j]) : 0u;  // valid keys are >= 1
    }
    uint32_t thr = 0;  // m-th largest key; 0 keeps every valid candidate
    if (m < n) {
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = thr | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int r = 0; r < NR; ++r) cnt += __popcll(__ballot(key[r] >= cand));
        if (cnt >= m) thr = cand;
      }
    }
    int cnt_gt = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) cnt_gt += __popcll(__ballot(key[r] > thr));
    const int need = m - cnt_gt;  // ties at thr to take, lowest ids first

    const size_t orow = ((size_t)b * n_q + i0 + qi) * top_k;
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
        sel[orow + pos] = j;
        if (sel_scores) sel_scores[orow + pos] = sc[qi][j];
      }
      base += __popcll(tm);
    }
    for (int pos = m + lane; pos < top_k; pos += 64) {
      sel[orow + pos] = -1;
      if (sel_scores) sel_scores[orow + pos] = -__builtin_inff();
    }
  }
}

template <typename T, int NR, int QT, int UPD_DI>
static hipError_t launch_index_t(const void* iq, const float* cmp, const int32_t* kv_lens,
                                 int32_t* sel, float* sel_scores, int batch, int n_q, int h_idx,
                                 int d_idx, int max_blocks, int block, int top_k,
                                 const void* ik, int ik_max_len, float* cmp_out,
                                 hipStream_t stream) {
  dim3 grid((n_q + QT - 1) / QT, batch);
  hipLaunchKernelGGL((index_topk_kernel<T, NR, QT, UPD_DI>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(iq), cmp, kv_lens, sel, sel_scores, n_q, h_idx, d_idx,
                     max_blocks, block, top_k, static_cast<const T*>(ik), ik_max_len, cmp_out);
  return hipGetLastError();
}

template <typename T, int NR>
static hipError_t launch_index_nr(const void* iq, const float* cmp, const int32_t* kv_lens,
                                  int32_t* sel, float* sel_scores, int batch, int n_q, int h_idx,
                                  int d_idx, int max_blocks, int block, int top_k,
                                  const void* ik, int ik_max_len, float* cmp_out,
                                  hipStream_t stream) {
  // Queries per workgroup.  Scoring runs on as many lanes as there are candidates and
  // selection on one wave per query, so a workgroup's time grows with its queries; small
  // tiles keep many workgroups resident (LDS for scores: QT * NR * 256 bytes) and were
  // measured fastest (4 up to 256 candidates, 8 beyond).
  constexpr int QTM = NR <= 4 ? 4 : NR <= 32 ? 8 : 4;
#define QSA_IDX(qt, upd)                                                                   \
  return launch_index_t<T, NR, qt, upd>(iq, cmp, kv_lens, sel, sel_scores, batch, n_q, h_idx, \
                                        d_idx, max_blocks, block, top_k, ik, ik_max_len,      \
                                        cmp_out, stream)
  if (cmp_out != nullptr) {  // decode step with the indexer-state update
    if (d_idx == 32) QSA_IDX(1, 32);
    if (d_idx == 64) QSA_IDX(1, 64);
    QSA_IDX(1, 128);
  }
  if (n_q == 1) QSA_IDX(1, 0);
  QSA_IDX(QTM, 0);
#undef QSA_IDX
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
