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
//     NS = 4 stages: while chunk u is multiplied (and the V of chunk u-1 still read),
//     chunks u+1 and u+2 are in flight.  Every chunk is shared by the NW waves (256 MFMA
//     rows), which sets the flops per byte of L2 traffic.
//   * Per row visibility of a block: one bit per position per union block (visibility
//     words, built in the prologue from the selection rows: a selected id inside [0, n(p)),
//     in any order, or the position's own block when its trailing part is non-empty); keys
//     after p are masked (causal part of the trailing block).  A wave with no visible row
//     skips the block.
//   * Transposed products keep one query row per lane:  S^T = K . Q^T  (A = K rows from
//     LDS, B = Q^T held in registers) and  O^T = V^T . P^T  (A = V^T gathered from the
//     row-major V tile by the LDS transpose read ds_read_b64_tr_b16, B = P^T taken straight
//     from the S^T accumulators; the key order inside an MFMA step is permuted identically
//     on both operands).  Row max and sum need one exchange with lane ^ 32.
//   * Online softmax in base 2 with the scale folded into one FMA per score.  A chunk's
//     probabilities are computed with the running max as it stands; the chunk's row max is
//     taken only for a row's first visible chunk or when the probabilities sum past 2^10,
//     and the running max is raised only when it grows by more than 8 (log2 units), so
//     rescaling the accumulators is rare and every probability stays <= 2^10.
#include "prefill_common.h"
#include "qsa_device.h"
#include "qsa_internal.h"

#include <climits>

namespace qsa {

namespace {

constexpr int KC = 64;   // keys per LDS chunk
constexpr int NW = 8;    // waves per workgroup
constexpr int NS = 4;    // LDS stages (chunks in flight + the one being used); a power of 2
// Visibility words kept in LDS next to the 128 KB ring (one bit per position per union
// block): every union block of a tile fits unless a tile holds more than 64 positions and a
// very large union, which then goes through in windows of kVisWords / words-per-block blocks.
constexpr int kVisWords = 7680;

// LDS layout of one stage (byte offsets), chosen so that every operand read of a lane is
// one base register plus an immediate and no read has a bank conflict (both checked with
// the SQ_LDS_BANK_CONFLICT counter on gfx950 for exactly these lane patterns):
//  K: D/16 slabs of 16 columns (one per k-step t of S^T = K . Q^T), slab t at t * 2048;
//     row r at r * 32, its two 16-byte units swapped when bit 3 of r is set (with bit 2,
//     or no swap, the ds_read_b128 of 32 rows takes two passes).
//  V: D/32 slabs of 32 columns (one per 32-wide d tile of O^T), after the K slabs, slab dt at
//     dt * 4096; row r at r * 64, its two 32-byte halves swapped when bit 1 of r is set.
__device__ __forceinline__ int k_unit_swap(int r) { return (r >> 3) & 1; }
__device__ __forceinline__ int v_half_swap(int r) { return (r >> 1) & 1; }

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(NW * 64, 1) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ sel, uint16_t* __restrict__ out,
    float* __restrict__ lse, int n_q, int kv_len_all, int h_q, int h_kv, int block, int top_k,
    float scale_log2, uint32_t q_and, uint32_t q_xor, int ntiles, int total_wg,
    const int32_t* __restrict__ kv_lens, int kv_stride) {
  constexpr int NT = NW * 64;
  constexpr int PW = 32 / G;       // positions per wave
  constexpr int MQ = NW * PW;      // positions per workgroup
  constexpr int VW = (MQ + 31) / 32;       // visibility words per union block
  constexpr int UW = kVisWords / VW;       // union blocks per visibility window
  constexpr int KP = D / 8;        // 1 KB pieces of a K chunk (= of a V chunk)
  constexpr int KI = KP / NW;      // K pieces per wave per chunk
  constexpr int DPC = 2 * KI;      // LDS-direct instructions per wave per chunk (K + V)
  static_assert(KI * NW == KP && KI >= 1, "load split");
  static_assert(2 * DPC < 64, "vmcnt range");
  static_assert(KC == 64, "slab layout assumes 64-key chunks");
  static_assert(32 % PW == 0, "a wave's positions share one visibility word");
  constexpr int NDT = D / 32;      // 32-wide d tiles of O^T
  constexpr int NKS = D / 16;      // k-steps of S^T = K . Q^T

  // NS stages of (K chunk, V chunk).  The LDS-direct loads are issued outside the
  // compiler's view (global_to_lds16_untracked), so a stage may be picked at run time
  // without the compiler draining the load queue before LDS reads.
  constexpr int TILE = KC * D;     // elements of one K (or V) chunk
  __shared__ __attribute__((aligned(16))) uint16_t ring[NS * 2 * TILE];
  __shared__ uint32_t bm[kPrefillMaxBlocks / 32];     // union bitmap
  __shared__ uint32_t wpre[kPrefillMaxBlocks / 32];   // union blocks below each bitmap word
  __shared__ uint32_t vis_w[kVisWords];               // [union block of the window][VW]

  // ---- which tile: runs of consecutive tiles of one head share an XCD (L2), and every
  // XCD gets a share of every sequence (tile_order); tiles are dispatched from the end of
  // the sequence (most candidate blocks) backwards, so the last workgroups to start are
  // the cheap ones near the beginning ----
  const int wg = blockIdx.x;
  const int logical = tile_order(wg, total_wg);
  const int tile = ntiles - 1 - logical % ntiles;
  const int g = (logical / ntiles) % h_kv;
  const int b = logical / (ntiles * h_kv);
  // keys of this sequence: kv_lens[b] (clamped to the kv_stride rows of its K/V slab), or
  // the common length
  const int kv_len = kv_lens ? min(max(kv_lens[b], 0), kv_stride) : kv_len_all;
  // query rows q0 .. q0+MQ-1 sit at positions p = p_off + row (bottom-right causal); rows
  // with p < 0 are padding (a sequence shorter than n_q)
  const int p_off = kv_len - n_q;
  const int q0 = tile * MQ;
  const int p0 = p_off + q0;
  const int p_hi = p_off + min(q0 + MQ, n_q) - 1;
  const int words = p_hi >= 0 ? (p_hi / block) / 32 + 1 : 0;

  const int tid = threadIdx.x;
  if (p_hi < 0) {  // padding rows only
    write_padding_tile<D, G>(out, lse, b, n_q, h_q, g, q0, min(MQ, n_q - q0), tid, NT);
    return;
  }
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);

  // ---- this lane's query row; its Q loads are issued first, so that their latency
  // overlaps the selection rows' loads and the visibility build ----
  const int row = lane & 31;
  const int half = lane >> 5;
  const int pos = wave * PW + row / G;
  const int hh = g * G + row % G;
  const int p = p0 + pos;
  const bool valid_row = p >= 0 && p < kv_len;
  const bool pad_row = p < 0 && q0 + pos < n_q;  // a padding row: zero output
  u32x4 qraw[NKS];
  {
    const uint16_t* qp = q + (((size_t)b * n_q + (valid_row ? p - p_off : 0)) * h_q + hh) * D + half * 8;
#pragma unroll
    for (int t = 0; t < NKS; ++t) qraw[t] = *reinterpret_cast<const u32x4*>(qp + t * 16);
  }

  // ---- the blocks the tile needs (union bitmap) and, per union block, which positions see
  // it (visibility words).  A position sees block j iff j is one of its selection entries
  // inside [0, n(p)) (any order; repeats and entries outside that range change nothing) or
  // j is its own block with a non-empty trailing part.  The selection rows are read from
  // global memory twice (L2): once for the bitmap, once for the words. ----
  for (int w = tid; w < max(words, 1); w += NT) bm[w] = 0u;
  __syncthreads();
  auto entry = [&](int e) __attribute__((always_inline)) {  // block of entry e, or -1
    const int r = e / top_k;
    const int pr = p0 + r;
    if (pr < 0 || pr >= kv_len) return -1;
    const int jj = sel[((size_t)b * n_q + q0 + r) * top_k + (e - r * top_k)];
    return (jj >= 0 && jj < (pr + 1) / block) ? jj : -1;
  };
  auto own = [&](int r) __attribute__((always_inline)) {  // own block of position r, or -1
    const int pr = p0 + r;
    return (pr >= 0 && pr < kv_len && (pr + 1) % block != 0) ? pr / block : -1;
  };
  for (int e = tid; e < MQ * top_k + MQ; e += NT) {
    const int j = e < MQ * top_k ? entry(e) : own(e - MQ * top_k);
    if (j >= 0) atomicOr(&bm[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  if (wave == 0) {  // exclusive prefix counts of the bitmap words (two words per lane)
    const int w0 = 2 * lane;
    const uint32_t c0 = w0 < words ? __builtin_popcount(bm[w0]) : 0u;
    const uint32_t c1 = w0 + 1 < words ? __builtin_popcount(bm[w0 + 1]) : 0u;
    uint32_t incl = c0 + c1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    const uint32_t excl = incl - c0 - c1;
    if (w0 < words) wpre[w0] = excl;
    if (w0 + 1 < words) wpre[w0 + 1] = excl + c0;
  }
  // union index of block j (j in the bitmap)
  auto uidx = [&](int j) __attribute__((always_inline)) {
    return (int)(wpre[j >> 5] + __builtin_popcount(bm[j >> 5] & ((1u << (j & 31)) - 1u)));
  };
  // visibility words of union blocks [win * UW, (win + 1) * UW)
  auto build_vis = [&](int win) __attribute__((always_inline)) {
    for (int i = tid; i < kVisWords; i += NT) vis_w[i] = 0u;
    __syncthreads();
    const int lo = win * UW;
    for (int e = tid; e < MQ * top_k + MQ; e += NT) {
      const int r = e < MQ * top_k ? e / top_k : e - MQ * top_k;
      const int j = e < MQ * top_k ? entry(e) : own(r);
      if (j >= 0) {
        const int u = uidx(j) - lo;
        if (u >= 0 && u < UW) atomicOr(&vis_w[u * VW + (r >> 5)], 1u << (r & 31));
      }
    }
    __syncthreads();
  };
  build_vis(0);

  bf16x8 qreg[NKS];
#pragma unroll
  for (int t = 0; t < NKS; ++t) {
    // opaque to the optimizer: keeps Q in registers instead of re-loading it per chunk
    // (a re-load would also wait on the untracked K/V loads in flight)
    qraw[t] = (qraw[t] & q_and) ^ q_xor;  // sign of the scale (PrefillScale)
    keep_in_register(qraw[t]);
    qreg[t] = bitcast<bf16x8>(qraw[t]);
  }

  float m_run = -__builtin_inff();
  float l_run = 0.f;
  f32x16 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;

  const int nsub = (block + KC - 1) / KC;
  const uint32_t kv_row = (uint32_t)h_kv * D;  // elements between consecutive tokens
  // K / V of this sequence and KV head, as scalar addresses
  const uint64_t kbase = uniform_ptr(k + ((size_t)b * kv_stride * h_kv + g) * D);
  const uint64_t vbase = uniform_ptr(v + ((size_t)b * kv_stride * h_kv + g) * D);

  // number of chunks the workgroup walks
  int nblk = 0;
  for (int w = 0; w < words; ++w) nblk += __builtin_popcount((uint32_t)wave_uniform((int)bm[w]));
  const int n = wave_uniform(nblk * nsub);

  // LDS-direct loads: each instruction fills 1 KB of a stage (64 lanes x 16 bytes).
  //  K: 2 per slab; piece part of slab t holds rows 32*part .. +31, lane -> (row lane / 2,
  //     physical unit lane % 2) and fetches the logical unit the swap maps there.
  //  V: 4 per slab; piece part of slab dt holds rows 16*part .. +15, lane -> (row lane / 4,
  //     physical unit lane % 4).
  // Every wave issues its own KI K pieces and KI V pieces of each chunk at the start of its
  // vector phase (both groups), from scalar base addresses, two instructions per save and
  // restore of M0.  Rows past the sequence are clamped to its last key (their keys are
  // masked).
  const uint32_t ring_lds = lds_addr(ring);
  ChunkIter it_load{0, (uint32_t)wave_uniform((int)bm[0]), -1, 0};
  next_block(bm, words, it_load);
  int issued = 0;
  int ld_key0 = 0;
  uint32_t ld_st0 = 0;
  const uint32_t kv_row_bytes = kv_row * 2u;
  uint64_t ld_kb = 0, ld_vb = 0;  // byte addresses of the base K / V row of the chunk
  int ld_base = 0;                // that row: the chunk's first key, clamped to the last one
  bool ld_full = true;            // every row of the chunk lies inside the sequence
  auto begin_chunk_load = [&]() __attribute__((always_inline)) {
    ld_key0 = it_load.j * block + it_load.sub * KC;
    ld_st0 = ring_lds + ((uint32_t)issued & (NS - 1)) * (2 * TILE * 2);
    // a chunk may start past the last key (the tail of a block longer than a chunk): it then
    // reads the last key into every row (all of its scores are masked)
    ld_base = min(ld_key0, kv_len - 1);
    const uint64_t row0 = (uint64_t)(uint32_t)ld_base * kv_row_bytes;
    ld_kb = kbase + row0;
    ld_vb = vbase + row0;
    ld_full = ld_key0 + KC <= kv_len;
  };
  // Piece i of this wave: row r_of(i) of the chunk and a byte offset lane_off[i] from the
  // chunk's first row (K pieces first, then V pieces).  A chunk that lies inside the
  // sequence is loaded from a scalar base (its first row) plus these fixed offsets, with no
  // vector address arithmetic; the last chunk of a sequence clamps rows past its end to the
  // last key (their scores are masked).
  auto r_of = [&](int i) __attribute__((always_inline)) {
    return i < KI ? 32 * ((wave * KI + i) & 1) + (lane >> 1)
                  : 16 * ((wave * KI + i - KI) & 3) + (lane >> 2);
  };
  auto col_of = [&](int i) __attribute__((always_inline)) {
    const int r = r_of(i);
    return i < KI ? 16 * ((wave * KI + i) >> 1) + 8 * ((lane & 1) ^ k_unit_swap(r))
                  : 32 * ((wave * KI + i - KI) >> 2) + 8 * ((lane & 3) ^ (2 * v_half_swap(r)));
  };
  auto lds_of = [&](int i) __attribute__((always_inline)) {  // byte offset inside a stage
    return i < KI ? (uint32_t)(((wave * KI + i) >> 1) * 2048 + ((wave * KI + i) & 1) * 1024)
                  : (uint32_t)(TILE * 2 + ((wave * KI + i - KI) >> 2) * 4096 +
                               ((wave * KI + i - KI) & 3) * 1024);
  };
  uint32_t lane_off[DPC];
#pragma unroll
  for (int i = 0; i < DPC; ++i) lane_off[i] = (uint32_t)(r_of(i) * (int)kv_row + col_of(i)) * 2u;
  // byte offset of piece i from the base row (rows past the sequence clamped to its last
  // key; never below the base row, so the unsigned offset cannot wrap)
  auto piece_off = [&](int i) __attribute__((always_inline)) {
    if (ld_full) return lane_off[i];
    const int r = min(ld_key0 + r_of(i), kv_len - 1) - ld_base;
    return (uint32_t)(r * (int)kv_row + col_of(i)) * 2u;
  };
  // pieces i (K) and KI + i (V): one instruction pair
  auto load_pair = [&](int i) __attribute__((always_inline)) {
    global_to_lds16x2_saddr_untracked(ld_kb, piece_off(i), ld_st0 + lds_of(i), ld_vb,
                                      piece_off(KI + i), ld_st0 + lds_of(KI + i));
  };
  auto end_chunk_load = [&]() __attribute__((always_inline)) {
    ++issued;
    if (issued < n) advance(bm, words, nsub, it_load);
  };
  auto issue_whole = [&]() __attribute__((always_inline)) {
    if (issued < n) {
      begin_chunk_load();
      if (ld_full) {
#pragma unroll
        for (int i = 0; i < KI; ++i)
          global_to_lds16x2_saddr_untracked(ld_kb, lane_off[i], ld_st0 + lds_of(i), ld_vb,
                                            lane_off[KI + i], ld_st0 + lds_of(KI + i));
      } else {
#pragma unroll
        for (int i = 0; i < KI; ++i) load_pair(i);
      }
      end_chunk_load();
    }
  };

  // transpose-read lane geometry (see the O^T product below)
  const int tr_g = lane >> 4, tr_m = lane & 15;
  const int tr_row = 4 * (tr_g >> 1) + (tr_m >> 2);      // + 16u (+8 for the upper 4 keys)
  const int tr_d = 16 * (tr_g & 1) + 4 * (tr_m & 3);     // + 32*dt
  // per-lane byte offsets of the operand reads inside a stage
  const int k_lane = row * 32 + 16 * (half ^ k_unit_swap(row));
  const int v_lane = TILE * 2 + tr_row * 64 + ((tr_d * 2) ^ (32 * v_half_swap(tr_row)));

  const float ninf = -__builtin_inff();

  // Ping-pong: waves 0 .. NW/2-1 (group A) and NW/2 .. NW-1 (group B) hold one wave per
  // SIMD each and run the same sequence of phases half a step apart:
  //   MFMA phase of chunk c:  S(c) = K(c) . Q^T  and  O += V(c-1)^T . P(c-1)
  //   VALU phase of chunk c:  mask, row max, lazy rescale, P(c) = exp2(...), row sums, and
  //                           this wave's loads of chunk c + 2 (A) or c + 3 (B)
  // Between two workgroup barriers one group runs an MFMA phase while the other runs a
  // VALU phase, so each SIMD has matrix work from one wave and vector work from the other.
  // S and P are single buffers: each phase consumes what the previous one of the same
  // wave produced.
  f32x16 S[2];
  bf16x8 P[4];

  auto mfma_phase = [&](int c, bool do_s, bool do_pv) __attribute__((always_inline)) {
    // the wave in its matrix phase goes first when both waves of a SIMD can issue
    set_wave_priority<2>();
    const char* Ks = reinterpret_cast<const char*>(ring + ((uint32_t)c & (NS - 1)) * (2 * TILE));
    const char* Vp =
        reinterpret_cast<const char*>(ring + ((uint32_t)(c + NS - 1) & (NS - 1)) * (2 * TILE));
    if (do_s) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) S[kt][r] = 0.f;
#pragma unroll
        for (int t = 0; t < NKS; ++t) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + k_lane + t * 2048 + kt * 1024);
          S[kt] = mfma32x32x16(a, qreg[t], S[kt]);
        }
      }
      // operand reads run kReadAhead MFMAs ahead
      sched_group<kSchedDsRead, kReadAhead>();
#pragma unroll
      for (int i = 0; i < 2 * NKS - kReadAhead; ++i) {
        sched_group<kSchedMfma, 1>();
        sched_group<kSchedDsRead, 1>();
      }
      sched_group<kSchedMfma, kReadAhead>();
    }
    if (do_pv) {
      // A operand of 16-key step st: V at d = 32*dt + (lane % 32), keys 16st + 4*half +
      // {0..3} and 16st + 8 + 4*half + {0..3}; each half is one transpose read in which the
      // lane supplies row 16st + tr_row (+8), columns 32*dt + tr_d .. +3.
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const char* vb = Vp + v_lane + dt * 4096 + st * 1024;
          const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(vb));
          const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(vb + 512));
          const bf16x8 a = bitcast<bf16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
          O[dt] = mfma32x32x16(a, P[st], O[dt]);
        }
      }
      // two transpose reads per MFMA, running kReadAhead MFMAs ahead
      sched_group<kSchedDsRead, 2 * kReadAhead>();
#pragma unroll
      for (int i = 0; i < 4 * NDT - kReadAhead; ++i) {
        sched_group<kSchedMfma, 1>();
        sched_group<kSchedDsRead, 2>();
      }
      sched_group<kSchedMfma, kReadAhead>();
    }
    set_wave_priority<0>();
  };

  // S holds the scores of a whole 64-key chunk; keys past the chunk (clamped rows, finite)
  // and keys after the row's position are masked.  Key 32*kt + 8*(r/4) + 4*half + r%4.
  auto valu_phase = [&](bool vis, int key0, int ck) __attribute__((always_inline)) {
    // this wave's share of the chunk it fetches next (the address unit accepts them
    // without stalling the wave)
    issue_whole();
    if (ck < KC || key0 + KC - 1 > p0) {
      const int lim = min(ck - 1, p - key0) - 4 * half;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kt * 32 + 8 * (r >> 2) + (r & 3) > lim) S[kt][r] = ninf;
    }
    // P = exp2(scale * S - m_run) with the running max m_run as it stands, row sum into lsum.
    // All exponent arguments first, then the exponentials, so that independent instructions
    // separate each producer from its consumer.
    float lsum = 0.f;
    auto probabilities = [&]() __attribute__((always_inline)) {
      const float nb = (vis && m_run != ninf) ? -m_run : ninf;
      float e[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) e[i] = __builtin_fmaf(S[i >> 4][i & 15], scale_log2, nb);
#pragma unroll
      for (int i = 0; i < 32; ++i) e[i] = __builtin_amdgcn_exp2f(e[i]);
      // B operand of 16-key step st: S registers 8*(st & 1) .. +7 of key tile st / 2
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const int i0 = 16 * (st >> 1) + 8 * (st & 1);
        P[st] = bitcast<bf16x8>(u32x4{pack_bf16x2(e[i0], e[i0 + 1]), pack_bf16x2(e[i0 + 2], e[i0 + 3]),
                                      pack_bf16x2(e[i0 + 4], e[i0 + 5]), pack_bf16x2(e[i0 + 6], e[i0 + 7])});
      }
#pragma unroll
      for (int w = 16; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) e[i] += e[i + w];
      lsum = pair_sum(e[0]);
    };
    // The row max is taken only when needed: at a row's first visible chunk, or when the
    // probabilities computed with the current m_run sum to more than 2^10 (then some score
    // may exceed m_run by more than 10 in log2 units).  Otherwise every probability is at
    // most 2^10 and the chunk keeps m_run.
    const bool first = vis && m_run == ninf;
    bool redo = __ballot(first) != 0ull;
    if (!redo) {
      probabilities();
      redo = __ballot(vis && lsum > 1024.0f) != 0ull;
    }
    if (redo) {
      // row max: a tree over the lane's 32 scores (short dependency chains), then the other
      // half of the row on lane ^ 32; four chains of three-input maxima (v_max3)
      float c[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int k0 = g >> 1, r0 = 8 * (g & 1);
        float x = fmaxf(fmaxf(S[k0][r0], S[k0][r0 + 1]), S[k0][r0 + 2]);
        x = fmaxf(fmaxf(x, S[k0][r0 + 3]), S[k0][r0 + 4]);
        x = fmaxf(fmaxf(x, S[k0][r0 + 5]), S[k0][r0 + 6]);
        c[g] = fmaxf(x, S[k0][r0 + 7]);
      }
      const float mx = pair_max(fmaxf(fmaxf(fmaxf(c[0], c[1]), c[2]), c[3]));
      // the running max moves only when it grows by more than 8 (log2 units): rare
      // rescales, and every exponent stays <= 8
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
      probabilities();
    }
    // each half of the row holds the full sum (pair_sum); count it once per lane pair
    l_run += half ? 0.f : lsum;
  };

  // ---- visibility of each chunk for this lane's row: one word per union block ----
  ChunkIter it_vis{0, (uint32_t)wave_uniform((int)bm[0]), -1, 0};
  int ub = -1;   // union index of the current block
  int win = 0;   // visibility window held in vis_w
  bool vis = false;
  const int vword = pos >> 5, vbit = pos & 31;
  auto visit = [&](bool first) __attribute__((always_inline)) {
    if (first) next_block(bm, words, it_vis);
    else advance(bm, words, nsub, it_vis);
    if (it_vis.sub == 0) {
      ++ub;
      if constexpr (UW < kPrefillMaxBlocks) {
        if (ub >= (win + 1) * UW) {  // next window (only for very large unions): every
          __syncthreads();           // wave has read the words of this one
          ++win;
          build_vis(win);
        }
      }
      vis = valid_row && ((vis_w[(ub - win * UW) * VW + vword] >> vbit) & 1u);
    }
  };

  // Chunk u: both groups meet barrier 1 (after chunk u has landed) and barrier 2.
  //   group A:  barrier 1, MFMA phase u, barrier 2, VALU phase u (+ its loads of chunk u+2)
  //   group B:  barrier 1, VALU phase u-1 (+ its loads of chunk u+2), barrier 2, MFMA phase u
  // followed by the O product of chunk n-1.  Chunk u+2 takes the stage of chunk u-2,
  // whose last readers (the O products of chunk u-2, in the MFMA phases u-1 of both
  // groups) ended before barrier 1 of chunk u.  Each wave loads its own share of every
  // chunk inside its vector phase, where a load instruction that waits for the address
  // unit holds up only vector work of one wave while the other wave of its SIMD runs
  // matrix work.  Each group computes the visibility of chunk u+1 at the end of its
  // iteration u, where the LDS read completes while it waits at the next barrier.  The
  // groups run separate loops with the same barriers, so each loop is straight-line code
  // for the register allocator; each branch ends with its own tail and epilogue, so O
  // needs no copies where the branches would meet.
  bool vis_prev = false, any_prev = false;
  int key0_prev = 0, ck_prev = 0;
  auto chunk_sync = [&](int u) __attribute__((always_inline)) {
    // chunk u must have landed (every wave waits for its own share); this wave's share of
    // chunk u+1 may stay in flight
    if (issued > u + 1) wait_vmcnt<DPC>();
    else wait_vmcnt<0>();
    barrier_no_fence();
  };
  auto chunk_visit = [&](int u, bool& vis_u, bool& any_u, int& key0_u, int& ck_u)
      __attribute__((always_inline)) {
    visit(u == 0);
    vis_u = vis;
    key0_u = it_vis.j * block + it_vis.sub * KC;
    ck_u = min(min(KC, block - it_vis.sub * KC), kv_len - key0_u);
    any_u = __ballot(vis) != 0ull;
  };
  // chunks 0 and 1: every wave issues its share
  issue_whole();
  issue_whole();
  auto epilogue = [&]() __attribute__((always_inline)) {
    const float l_tot = pair_sum(l_run);  // the row's sum sits in its half-0 lane
    if (valid_row || pad_row) {
      const float inv = (valid_row && l_tot > 0.f) ? 1.f / l_tot : 0.f;
      const size_t orow = ((size_t)b * n_q + (q0 + pos)) * h_q + hh;
      uint16_t* op = out + orow * D;
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
        lse[orow] = (valid_row && l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : -__builtin_inff();
    }
  };
  // visibility of chunk u is computed at the end of iteration u-1, where its LDS read
  // completes during the barrier wait
  bool vis_c = false, any_c = false;
  int key0_c = 0, ck_c = 0;
  if (n > 0) chunk_visit(0, vis_c, any_c, key0_c, ck_c);
  if (wave < NW / 2) {
    for (int u = 0; u < n; ++u) {
      chunk_sync(u);
      mfma_phase(u, any_c, any_prev);
      barrier_no_fence();
      if (any_c) valu_phase(vis_c, key0_c, ck_c);
      else issue_whole();
      any_prev = any_c;
      if (u + 1 < n) chunk_visit(u + 1, vis_c, any_c, key0_c, ck_c);
    }
    if (any_prev) mfma_phase(n, false, true);
    epilogue();
  } else {
    for (int u = 0; u < n; ++u) {
      chunk_sync(u);
      if (any_prev) valu_phase(vis_prev, key0_prev, ck_prev);
      else issue_whole();
      barrier_no_fence();
      mfma_phase(u, any_c, any_prev);
      vis_prev = vis_c;
      any_prev = any_c;
      key0_prev = key0_c;
      ck_prev = ck_c;
      if (u + 1 < n) chunk_visit(u + 1, vis_c, any_c, key0_c, ck_c);
    }
    if (any_prev) valu_phase(vis_prev, key0_prev, ck_prev);
    if (any_prev) mfma_phase(n, false, true);
    epilogue();
  }
}

bool prefill_bf16_supported(int group, int d, int block, int top_k, int kv_len, int h_kv) {
  if (d == 256) return prefill_bf16_rt_supported(group, d, block, top_k, kv_len, h_kv);
  if (d != 64 && d != 128) return false;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16 && group != 32) return false;
  if (block < 1 || block > 1024 || top_k < 1 || top_k > kMaxTopK) return false;
  // element offsets of K / V rows within one sequence are 32-bit
  if ((long long)kv_len * h_kv * d >= (1ll << 32)) return false;
  return (kv_len + block - 1) / block <= kPrefillMaxBlocks;
}

template <int D, int G>
static hipError_t launch_prefill_t(const void* q, const void* k, const void* v, const int32_t* sel,
                                   void* out, float* lse, int batch, int n_q, int kv_len,
                                   const int32_t* kv_lens, int kv_stride, int h_q, int h_kv,
                                   int block, int top_k, float sm_scale, hipStream_t stream) {
  constexpr int MQ = NW * (32 / G);
  const int ntiles = (n_q + MQ - 1) / MQ;
  const long long total = (long long)ntiles * h_kv * batch;
  if (total > INT_MAX) return hipErrorInvalidValue;
  const PrefillScale sc = prefill_scale(sm_scale, kLog2e);
  hipLaunchKernelGGL((prefill_bf16_kernel<D, G>), dim3((unsigned)total), dim3(NW * 64), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), sel, static_cast<uint16_t*>(out), lse, n_q,
                     kv_len, h_q, h_kv, block, top_k, sc.scale_log2, sc.q_and, sc.q_xor, ntiles,
                     (int)total, kv_lens, kv_stride);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_prefill_d(int group, const void* q, const void* k, const void* v,
                                   const int32_t* sel, void* out, float* lse, int batch, int n_q,
                                   int kv_len, const int32_t* kv_lens, int kv_stride, int h_q,
                                   int h_kv, int block, int top_k, float sm_scale,
                                   hipStream_t stream) {
#define QSA_G(g)                                                                             \
  return launch_prefill_t<D, g>(q, k, v, sel, out, lse, batch, n_q, kv_len, kv_lens, kv_stride, \
                                h_q, h_kv, block, top_k, sm_scale, stream)
  switch (group) {
    case 1: QSA_G(1);
    case 2: QSA_G(2);
    case 4: QSA_G(4);
    case 8: QSA_G(8);
    case 16: QSA_G(16);
    case 32: QSA_G(32);
  }
#undef QSA_G
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_bf16(const void* q, const void* k, const void* v, const int32_t* sel,
                               void* out, float* lse, int batch, int n_q, int kv_len,
                               const int32_t* kv_lens, int kv_stride, int h_q, int h_kv, int d,
                               int block, int top_k, float sm_scale, hipStream_t stream) {
  if (batch == 0 || n_q == 0) return hipSuccess;
  const int group = h_q / h_kv;
  if (d == 256)
    return launch_prefill_bf16_rt(q, k, v, sel, out, lse, batch, n_q, kv_len, kv_lens, kv_stride,
                                  h_q, h_kv, d, block, top_k, sm_scale, stream);
  if (d == 128)
    return launch_prefill_d<128>(group, q, k, v, sel, out, lse, batch, n_q, kv_len, kv_lens,
                                 kv_stride, h_q, h_kv, block, top_k, sm_scale, stream);
  if (d == 64)
    return launch_prefill_d<64>(group, q, k, v, sel, out, lse, batch, n_q, kv_len, kv_lens,
                                kv_stride, h_q, h_kv, block, top_k, sm_scale, stream);
  return hipErrorInvalidValue;
}

}  // namespace qsa
