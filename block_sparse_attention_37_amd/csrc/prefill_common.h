// Pieces shared by the two block-sparse prefill kernels (32-row waves for head dims 64
// and 128, 16-row tiles for 256): the walk over the union bitmap of visited blocks,
// scheduling hints, wave priority and cross-lane reductions of one query row.
#pragma once

#include "qsa_device.h"

namespace qsa {
namespace {

struct ChunkIter {
  int wi;         // bitmap word index
  uint32_t bits;  // remaining bits of that word
  int j;          // current block
  int sub;        // sub-chunk of the block (chunk = the kernel's keys per LDS stage)
};

// The bitmap is the same for every lane: its words are made wave-uniform so the walk runs
// on the scalar unit.
__device__ __forceinline__ bool next_block(const uint32_t* bm, int words, ChunkIter& it) {
  while (it.bits == 0u) {
    if (++it.wi >= words) return false;
    it.bits = (uint32_t)wave_uniform((int)bm[it.wi]);
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

// Dispatch order of the prefill tiles.  Workgroup ids go to the 8 XCDs round-robin
// (wg % 8); this gives each XCD runs of kTileRun consecutive logical tiles, then moves on
// to the next XCD, so neighbouring tiles (which select many of the same blocks) share an
// L2 while every XCD gets an even share of every sequence and KV head.  A run of 32 tiles
// fills the 32 CUs of an XCD with neighbours: at 128k the L2 misses of the attention
// kernel (FETCH_SIZE) measured 20.5 GB per launch with runs of 4, 15.5 GB with 16,
// 11.8 GB with 32, 15.4 GB with 64 and 18.4 GB with 128, at 23.5, 23.55, 23.7, 24.5 and
// 25.65 ms; at 4k, 72, 78 and 72 us for runs of 4, 16 and 32.  (Giving each XCD one
// contiguous eighth of the grid instead put whole sequences of a varlen batch, or whole
// ranges of positions, on one XCD: measured 1.45 ms vs 0.88 ms on 8 prompts of mixed
// length, 27.3 ms vs 23.8 ms at 128k.)  A permutation of [0, total).
constexpr int kTileRun = 32;
__device__ __forceinline__ int tile_order(int wg, int total) {
  const int full = total / (8 * kTileRun) * (8 * kTileRun);
  if (wg >= full) return wg;
  const int xcd = wg % 8, k = wg / 8;
  return (k / kTileRun) * 8 * kTileRun + xcd * kTileRun + k % kTileRun;
}

// A tile whose rows are all padding (p < 0 for every row: its sequence is shorter than n_q)
// writes zeros to its output rows and -inf to their log-sum-exp, the values the full path
// gives such rows, and the workgroup leaves without loading anything.  Rows q0 .. q0+rows-1
// of sequence b, query heads g*G .. g*G+G-1 (contiguous in a row: G*D bf16, 16-byte units;
// the entry points require 16-byte aligned tensors).  No barrier: a workgroup-uniform
// early exit.
template <int D, int G>
__device__ __forceinline__ void write_padding_tile(uint16_t* __restrict__ out,
                                                   float* __restrict__ lse, int b, int n_q,
                                                   int h_q, int g, int q0, int rows, int tid,
                                                   int nthreads) {
  constexpr int UPR = G * D / 8;  // 16-byte units per query position
  uint16_t* base = out + (((size_t)b * n_q + q0) * h_q + g * G) * D;
  for (int e = tid; e < rows * UPR; e += nthreads) {
    const int r = e / UPR;
    *reinterpret_cast<u32x4*>(base + (size_t)r * h_q * D + (e - r * UPR) * 8) = u32x4{0u, 0u, 0u, 0u};
  }
  if (lse) {
    for (int e = tid; e < rows * G; e += nthreads) {
      const int r = e / G;
      lse[((size_t)b * n_q + q0 + r) * h_q + g * G + (e - r * G)] = -__builtin_inff();
    }
  }
}

// The softmax scale as the prefill kernels apply it.  They take the row maximum of the raw
// scores and fold the scale into one FMA per score afterwards, which needs a positive scale:
// a negative scale would turn the maximum into the minimum, and a zero scale would multiply
// the -inf of masked keys by 0.  The sign goes into Q instead, exactly: S = K.(-Q)^T is -S
// bit for bit (every product changes sign, the sums round symmetrically), so a negative
// scale flips the sign bit of every bf16 element of Q and uses |scale|.  A zero scale gives
// every visible key the same weight: Q is zeroed (every score is exactly 0) and the scale
// is 1, so masked keys keep -inf.
struct PrefillScale {
  float scale_log2;  // positive scale in log2 units
  uint32_t q_and;    // applied to each 32-bit pair of bf16 Q elements: (x & q_and) ^ q_xor
  uint32_t q_xor;
};
inline PrefillScale prefill_scale(float sm_scale, float log2e) {
  if (sm_scale == 0.0f) return {1.0f, 0u, 0u};
  if (sm_scale < 0.0f) return {-sm_scale * log2e, 0xFFFFFFFFu, 0x80008000u};
  return {sm_scale * log2e, 0xFFFFFFFFu, 0u};
}

// Instruction-order hints for the scheduler (no effect on results): mask selects the
// instruction class (0x8 MFMA, 0x100 LDS read), n how many of them come next.
template <int MASK, int N>
__device__ __forceinline__ void sched_group() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
#endif
}
constexpr int kSchedMfma = 0x8;
constexpr int kSchedDsRead = 0x100;
constexpr int kReadAhead = 4;  // LDS operand reads issued ahead of their MFMA (measured best
                               // for the 32-row kernel)

// Issue priority of this wave among the waves of its SIMD (s_setprio).
template <int P>
__device__ __forceinline__ void set_wave_priority() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_setprio(P);
#endif
}

// max / sum of x over the lane pair (l, l ^ 32): v_permlane32_swap leaves each lane with
// its own value and its partner's, in some order, which max and sum do not care about.
__device__ __forceinline__ float pair_max(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
#else
  return x;
#endif
}
__device__ __forceinline__ float pair_sum(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
#else
  return x;
#endif
}

// max / sum of x over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 4-key groups of
// one query row in a 16x16 MFMA tile): v_permlane16_swap pairs l with l ^ 16 the way
// v_permlane32_swap pairs l with l ^ 32.
__device__ __forceinline__ float quad_max(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_max(fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])));
#else
  return x;
#endif
}
__device__ __forceinline__ float quad_sum(float x) {
#if defined(__HIP_DEVICE_COMPILE__)
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return pair_sum(__uint_as_float(a[0]) + __uint_as_float(a[1]));
#else
  return x;
#endif
}

}  // namespace
}  // namespace qsa
