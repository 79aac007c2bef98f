// Block-sparse prefill attention for head dim 256 on bf16 matrix cores (gfx950 MFMA).
//
// Qwen4-Exp model page, overview: each query attends to its selected contiguous token
// blocks plus its own incomplete trailing block, uncompressed; model configuration: the
// default attention shape is 16 query heads over 2 key/value heads of dimension 256.
//
// Same method and work decomposition as the 32-row kernel for head dims 64 and 128 (one
// workgroup of NW waves per run of consecutive positions of one KV head, walking the union
// of the blocks they need through an LDS ring fed by LDS-direct loads, two wave groups in
// ping-pong between MFMA and VALU phases).  What changes with D = 256 is the budget:
//   * A wave holds RT tiles of 16 query rows on 16x16x32 MFMAs: RT = 1 (2 when G = 32, one
//     position of 32 heads).  Per lane that is O^T 16 x f32x4 and Q^T 8 x bf16x8 per tile.
//   * Chunks are 32 keys (a stage is 16 KB of K and 16 KB of V), so four stages fit 128 KB
//     of LDS next to the union bitmap and the visibility words.
//   * S^T = K . Q^T (A = K rows from LDS, B = Q^T in registers): lane l holds keys
//     16*kt + 4*(l/16) + {0..3} of query row l % 16.  O^T = V^T . P^T (A = V^T through the
//     transpose read, B = P^T straight from the S^T accumulators, keys permuted identically
//     on both operands).  A row's keys sit in four lanes (l, l^16, l^32, l^48).
#include "prefill_common.h"
#include "qsa_device.h"
#include "qsa_internal.h"

#include <climits>

namespace qsa {

namespace {

constexpr int RT_KC = 32;  // keys per LDS chunk
constexpr int RT_NW = 8;   // waves per workgroup
constexpr int RT_NS = 4;   // LDS stages
// Visibility words kept in LDS next to the 128 KB ring (one bit per position per union
// block): every union block of a tile fits when a tile holds at most 32 positions; larger
// tiles (G = 1, 2) with very large unions go through in windows of kRtVisWords /
// words-per-block blocks.
constexpr int kRtVisWords = 7680;

// 16-row MFMA tiles per wave.
template <int G>
struct RtTiles {
  static constexpr int value = (G == 32) ? 2 : 1;
};

// LDS layout of one stage (byte offsets):
//  K: D/32 slabs of 32 columns (one per k-step t), slab t at t * KC * 64; row r at r * 64,
//     its four 16-byte units permuted by XOR with (r >> 1) & 3.  A read takes one unit of
//     16 consecutive rows; with this permutation it has no bank conflict (measured with
//     SQ_LDS_BANK_CONFLICT on gfx950 for rows 0..15 and 16..31).
//  V: D/16 slabs of 16 columns (one per 16-wide d tile), after the K slabs, slab dt at
//     dt * KC * 32; row r at r * 32.  The 16 lanes of a transpose-read group read 4 whole
//     rows = 128 contiguous bytes (no conflict, measured).
__device__ __forceinline__ int rt_k_swz(int r) { return (r >> 1) & 3; }

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(RT_NW * 64, 1) void prefill_bf16_rt_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ sel, uint16_t* __restrict__ out,
    float* __restrict__ lse, int n_q, int kv_len_all, int h_q, int h_kv, int block, int top_k,
    float scale_log2, uint32_t q_and, uint32_t q_xor, int ntiles, int total_wg,
    const int32_t* __restrict__ kv_lens, int kv_stride) {
  constexpr int NW = RT_NW, NS = RT_NS, KC = RT_KC;
  constexpr int NT = NW * 64;
  constexpr int RT = RtTiles<G>::value;
  constexpr int PW = 16 * RT / G;  // positions per wave
  constexpr int MQ = NW * PW;      // positions per workgroup
  static_assert(PW * G == 16 * RT, "a wave holds whole positions");
  constexpr int NKT = D / 32;      // 32-wide k-steps of S^T
  constexpr int NDT = D / 16;      // 16-wide d tiles of O^T
  constexpr int NKB = KC / 16;     // 16-key tiles of S^T per chunk
  constexpr int NPS = KC / 32;     // 32-key steps of O^T per chunk
  constexpr int KSLAB = KC * 64;   // bytes of one K slab
  constexpr int VSLAB = KC * 32;   // bytes of one V slab
  constexpr int KPARTS = KC / 16;  // 1 KB pieces per K slab (16 rows x 64 bytes)
  constexpr int VPARTS = KC / 32;  // 1 KB pieces per V slab (32 rows x 32 bytes)
  constexpr int KP = KPARTS * NKT;
  constexpr int VP = VPARTS * NDT;
  constexpr int KI = KP / (NW / 2);  // pieces per group-A wave (group B issues none)
  constexpr int VI = VP / (NW / 2);
  constexpr int DPC = KI + VI;       // LDS-direct instructions per group-A wave per chunk
  static_assert(KI * (NW / 2) == KP && VI * (NW / 2) == VP, "load split");
  static_assert(2 * DPC < 64, "vmcnt range");

  constexpr int VW = (MQ + 31) / 32;      // visibility words per union block
  constexpr int UW = kRtVisWords / VW;    // union blocks per visibility window

  constexpr int TILE = KC * D;  // elements of one K (or V) chunk
  __shared__ __attribute__((aligned(16))) uint16_t ring[NS * 2 * TILE];
  __shared__ uint32_t bm[kPrefillMaxBlocks / 32];    // union bitmap
  __shared__ uint32_t wpre[kPrefillMaxBlocks / 32];  // union blocks below each bitmap word
  __shared__ uint32_t vis_w[kRtVisWords];            // [union block of the window][VW]

  // ---- tile order as in the 32-row kernel (tile_order: runs of consecutive tiles per
  // XCD), heaviest (last) tiles first ----
  const int wg = blockIdx.x;
  const int logical = tile_order(wg, total_wg);
  const int tile = ntiles - 1 - logical % ntiles;
  const int g = (logical / ntiles) % h_kv;
  const int b = logical / (ntiles * h_kv);
  // keys of this sequence (kv_lens[b] clamped to the K/V slab's kv_stride rows, or the
  // common length); query rows with p < 0 are padding
  const int kv_len = kv_lens ? min(max(kv_lens[b], 0), kv_stride) : kv_len_all;
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

  // ---- this lane's query rows: column `col` of each row tile; `quad` picks 4 keys of a
  // 16-key tile (S^T, O^T rows) or 8 elements of an operand.  Their Q loads are issued
  // first, so that their latency overlaps the selection rows' loads and the bitmap ----
  const int col = lane & 15;
  const int quad = lane >> 4;
  // position of row tile rt (16 * rt + col < 32 when G = 32)
  auto pos_of = [&](int rt) __attribute__((always_inline)) {
    return wave * PW + (16 * rt + col) / G;
  };
  auto p_of = [&](int rt) __attribute__((always_inline)) { return p0 + pos_of(rt); };
  auto valid_of = [&](int rt) __attribute__((always_inline)) {
    return p_of(rt) >= 0 && p_of(rt) < kv_len;
  };

  u32x4 qraw[RT][NKT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int hh = g * G + (16 * rt + col) % G;
    const int qi = valid_of(rt) ? p_of(rt) - p_off : 0;
    const uint16_t* qp = q + (((size_t)b * n_q + qi) * h_q + hh) * D + quad * 8;
#pragma unroll
    for (int t = 0; t < NKT; ++t) qraw[rt][t] = *reinterpret_cast<const u32x4*>(qp + t * 32);
  }

  // ---- the blocks the tile needs (union bitmap) and, per union block, which positions see
  // it (visibility words).  A position sees block j iff j is one of its selection entries
  // inside [0, n(p)) (any order; entries outside that range change nothing) or j is its
  // own block with a non-empty trailing part.  The selection rows are read from global
  // memory twice (L2): once for the bitmap, once for the words. ----
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
    for (int i = tid; i < kRtVisWords; i += NT) vis_w[i] = 0u;
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

  bf16x8 qreg[RT][NKT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      qraw[rt][t] = (qraw[rt][t] & q_and) ^ q_xor;  // sign of the scale (PrefillScale)
      keep_in_register(qraw[rt][t]);  // Q stays in registers (no re-load behind the untracked loads)
      qreg[rt][t] = bitcast<bf16x8>(qraw[rt][t]);
    }

  float m_run[RT], l_run[RT];
  f32x4 O[NDT][RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -__builtin_inff();
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) O[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int nsub = (block + KC - 1) / KC;
  const uint32_t kv_row = (uint32_t)h_kv * D;  // elements between consecutive tokens
  const uint16_t* kbase = k + ((size_t)b * kv_stride * h_kv + g) * D;
  const uint16_t* vbase = v + ((size_t)b * kv_stride * h_kv + g) * D;

  int nblk = 0;
  for (int w = 0; w < words; ++w) nblk += __builtin_popcount((uint32_t)wave_uniform((int)bm[w]));
  const int n = wave_uniform(nblk * nsub);

  // LDS-direct loads (1 KB each), issued by group A only:
  //  K piece (t, part): rows 16*part + lane / 4, physical unit lane % 4 of slab t;
  //  V piece (dt, part): rows 32*part + lane / 2, columns 16*dt + 8*(lane % 2).
  // Group-A wave w issues K pieces w*KI .. +KI-1 and V pieces w*VI .. +VI-1.  Rows past the
  // chunk are clamped into the tensor (their keys are masked).
  const uint32_t ring_lds = lds_addr(ring);
  ChunkIter it_load{0, (uint32_t)wave_uniform((int)bm[0]), -1, 0};
  next_block(bm, words, it_load);
  int issued = 0;
  auto issue_next = [&]() __attribute__((always_inline)) {
    if (issued < n) {
      const int key0 = it_load.j * block + it_load.sub * KC;
      const uint32_t st0 = ring_lds + (uint32_t)(issued % NS) * (2 * TILE * 2);
#pragma unroll
      for (int i = 0; i < KI; ++i) {
        const int id = wave * KI + i, t = id / KPARTS, part = id % KPARTS;
        const int r = 16 * part + (lane >> 2);
        const int c = 32 * t + 8 * ((lane & 3) ^ rt_k_swz(r));
        const uint32_t grow = (uint32_t)min(key0 + r, kv_len - 1);
        global_to_lds16_untracked(kbase + grow * kv_row + c, st0 + t * KSLAB + part * 1024);
      }
#pragma unroll
      for (int i = 0; i < VI; ++i) {
        const int id = wave * VI + i, dt = id / VPARTS, part = id % VPARTS;
        const int r = 32 * part + (lane >> 1);
        const int c = 16 * dt + 8 * (lane & 1);
        const uint32_t grow = (uint32_t)min(key0 + r, kv_len - 1);
        global_to_lds16_untracked(vbase + grow * kv_row + c,
                                  st0 + TILE * 2 + dt * VSLAB + part * 1024);
      }
      ++issued;
      if (issued < n) advance(bm, words, nsub, it_load);
    }
  };

  // per-lane byte offsets of the operand reads inside a stage
  //  K: key 16*kt + col, columns 32*t + 8*quad .. +7
  //  V (transpose read): group quad reads rows 4*quad + col / 4 (+16 for the upper half),
  //  columns 16*dt + 4*(col % 4) .. +3, i.e. 8 bytes at 8 * lane
  const int k_lane = col * 64 + 16 * (quad ^ rt_k_swz(col));
  const int v_lane = TILE * 2 + 8 * lane;
  const float ninf = -__builtin_inff();

  // S[kt][rt]: keys 16*kt + 4*quad + {0..3}; P[ps][rt]: B operand of 32-key step ps, element
  // i = key 32*ps + 16*(i / 4) + 4*quad + i % 4.  Both get a value on every path (zeros
  // where a phase is skipped), so no stale copy is kept in registers across phases.
  f32x4 S[NKB][RT];
  bf16x8 P[NPS][RT];
  auto clear_p = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int ps = 0; ps < NPS; ++ps)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) P[ps][rt] = bitcast<bf16x8>(u32x4{0u, 0u, 0u, 0u});
  };

  // MFMA phase of chunk c: O += V(c-1)^T . P(c-1) first (P then dies), then S(c) = K(c).Q^T
  auto mfma_phase = [&](int c, bool do_s, bool do_pv) __attribute__((always_inline)) {
    set_wave_priority<2>();
    const char* Ks = reinterpret_cast<const char*>(ring + (c % NS) * (2 * TILE));
    const char* Vp = reinterpret_cast<const char*>(ring + ((c + NS - 1) % NS) * (2 * TILE));
    if (do_pv) {
#pragma unroll
      for (int ps = 0; ps < NPS; ++ps) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const char* vb = Vp + v_lane + dt * VSLAB + ps * 1024;
          const u32x2 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(vb));
          const u32x2 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(vb + 512));
          const bf16x8 a = bitcast<bf16x8>(u32x4{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) O[dt][rt] = mfma16x16x32(a, P[ps][rt], O[dt][rt]);
        }
      }
      sched_group<kSchedDsRead, 2 * kReadAhead>();
#pragma unroll
      for (int i = 0; i < NPS * NDT - kReadAhead; ++i) {
        sched_group<kSchedMfma, RT>();
        sched_group<kSchedDsRead, 2>();
      }
      sched_group<kSchedMfma, RT * kReadAhead>();
    }
    if (do_s) {
#pragma unroll
      for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) S[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
#pragma unroll
        for (int kt = 0; kt < NKB; ++kt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + k_lane + t * KSLAB + kt * 1024);
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) S[kt][rt] = mfma16x16x32(a, qreg[rt][t], S[kt][rt]);
        }
      }
      sched_group<kSchedDsRead, kReadAhead>();
#pragma unroll
      for (int i = 0; i < NKB * NKT - kReadAhead; ++i) {
        sched_group<kSchedMfma, RT>();
        sched_group<kSchedDsRead, 1>();
      }
      sched_group<kSchedMfma, RT * kReadAhead>();
    } else {
#pragma unroll
      for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) S[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    set_wave_priority<0>();
  };

  // P = exp2(score * scale - running max) for this lane's 4-key groups of the chunk, with the
  // running max as it stands; this lane's share of each row's sum into lpart.
  auto probabilities = [&](const bool* vis, float* lpart) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float nb = (vis[rt] && m_run[rt] != ninf) ? -m_run[rt] : ninf;
      f32x4 e[NKB];
#pragma unroll
      for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) e[kt][r] = __builtin_fmaf(S[kt][rt][r], scale_log2, nb);
#pragma unroll
      for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) e[kt][r] = __builtin_amdgcn_exp2f(e[kt][r]);
      f32x4 sum = e[0];
#pragma unroll
      for (int kt = 1; kt < NKB; ++kt) sum += e[kt];
      lpart[rt] = (sum[0] + sum[1]) + (sum[2] + sum[3]);
#pragma unroll
      for (int ps = 0; ps < NPS; ++ps) {
        const f32x4 a = e[2 * ps], c = e[2 * ps + 1];
        P[ps][rt] = bitcast<bf16x8>(u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                          pack_bf16x2(c[0], c[1]), pack_bf16x2(c[2], c[3])});
      }
    }
  };
  // VALU phase of the chunk at key0 with ck valid keys: mask (keys past the chunk or after
  // the row's position), then the probabilities with the running max as it stands.  The
  // row max over the row's four lanes is taken only when needed: at a row's first visible
  // chunk, or when some lane's share of a row's probabilities exceeds 2^8 (so the row's
  // sum may exceed 2^10 and a score the running max by more than 10 in log2 units); the
  // chunk is then done again after a lazy rescale (the running max moves only when it grows
  // by more than 8), so every probability stays <= 2^10.
  auto valu_phase = [&](const bool* vis, int key0, int ck) __attribute__((always_inline)) {
    if (ck < KC || key0 + KC - 1 > p0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int lim = min(ck - 1, p_of(rt) - key0) - 4 * quad;
#pragma unroll
        for (int kt = 0; kt < NKB; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kt + r > lim) S[kt][rt][r] = ninf;
      }
    }
    float lpart[RT];
    bool first = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) first |= vis[rt] && m_run[rt] == ninf;
    bool redo = __ballot(first) != 0ull;
    if (!redo) {
      probabilities(vis, lpart);
      bool big = false;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) big |= vis[rt] && lpart[rt] > 256.0f;
      redo = __ballot(big) != 0ull;
    }
    if (redo) {
      bool need[RT];
      float m_new[RT];
      bool any_need = false;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float mx = ninf;
#pragma unroll
        for (int kt = 0; kt < NKB; ++kt)
          mx = fmaxf(fmaxf(mx, fmaxf(S[kt][rt][0], S[kt][rt][1])), fmaxf(S[kt][rt][2], S[kt][rt][3]));
        mx = quad_max(mx);
        const float m_cand = vis[rt] ? fmaxf(m_run[rt], mx * scale_log2) : m_run[rt];
        need[rt] = m_cand > m_run[rt] + 8.0f;
        m_new[rt] = need[rt] ? m_cand : m_run[rt];
        any_need |= need[rt];
      }
      if (__ballot(any_need) != 0ull) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          // lanes that keep their max (possibly still -inf) keep their state exactly
          const float alpha = need[rt] ? __builtin_amdgcn_exp2f(m_run[rt] - m_new[rt]) : 1.0f;
          l_run[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) O[dt][rt] *= alpha;
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) m_run[rt] = m_new[rt];
      probabilities(vis, lpart);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) l_run[rt] += lpart[rt];
  };

  // ---- visibility of each chunk for this lane's rows: one word per union block ----
  ChunkIter it_vis{0, (uint32_t)wave_uniform((int)bm[0]), -1, 0};
  int ub = -1;   // union index of the current block
  int win = 0;   // visibility window held in vis_w
  bool vis[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) vis[rt] = false;
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
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int ps = pos_of(rt);
        vis[rt] = valid_of(rt) && ((vis_w[(ub - win * UW) * VW + (ps >> 5)] >> (ps & 31)) & 1u);
      }
    }
  };
  auto chunk_visit = [&](int u, bool* vis_u, bool& any_u, int& key0_u, int& ck_u)
      __attribute__((always_inline)) {
    visit(u == 0);
    bool a = false;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      vis_u[rt] = vis[rt];
      a |= vis[rt];
    }
    key0_u = it_vis.j * block + it_vis.sub * KC;
    ck_u = min(min(KC, block - it_vis.sub * KC), kv_len - key0_u);
    any_u = __ballot(a) != 0ull;
  };
  auto chunk_sync = [&](int u) __attribute__((always_inline)) {
    // chunk u must have landed (group A waits for its own loads; group B has none); chunk
    // u+1 may stay in flight
    if (issued > u + 1) wait_vmcnt<DPC>();
    else wait_vmcnt<0>();
    barrier_no_fence();
  };

  auto epilogue = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float l_tot = quad_sum(l_run[rt]);
      const int p = p_of(rt);
      const bool valid = p >= 0 && p < kv_len;
      // rows past n_q do not exist; padding rows (p < 0) get zeros and lse = -inf
      if (valid || (p < 0 && p - p_off < n_q)) {
        const int hh = g * G + (16 * rt + col) % G;
        const size_t orow = ((size_t)b * n_q + (p - p_off)) * h_q + hh;
        const float inv = (valid && l_tot > 0.f) ? 1.f / l_tot : 0.f;
        uint16_t* op = out + orow * D + 4 * quad;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const f32x4 o = O[dt][rt];
          *reinterpret_cast<u32x2*>(op + 16 * dt) =
              u32x2{pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv)};
        }
        if (lse && quad == 0)
          lse[orow] = (valid && l_tot > 0.f) ? (m_run[rt] + __log2f(l_tot)) * kLn2
                                             : -__builtin_inff();
      }
    }
  };

  // Chunk u (as in the 32-row kernel):
  //   group A:  barrier 1, MFMA phase u, loads of chunk u+2, barrier 2, VALU phase u
  //   group B:  barrier 1, VALU phase u-1, barrier 2, MFMA phase u
  // then the O product of chunk n-1.  Chunk u+2 takes the stage of chunk u-2, last read by
  // group B's O product in its MFMA phase u-1, before barrier 1 of chunk u.  The
  // visibility of chunk u+1 is computed at the end of iteration u, in both groups (any
  // rebuild of the visibility window, a workgroup barrier, comes at the same point).
  bool vis_c[RT], vis_prev[RT];
  bool any_c = false, any_prev = false;
  int key0_c = 0, ck_c = 0, key0_prev = 0, ck_prev = 0;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) vis_c[rt] = vis_prev[rt] = false;
  if (n > 0) chunk_visit(0, vis_c, any_c, key0_c, ck_c);
  if (wave < NW / 2) {
    issue_next();
    issue_next();
    for (int u = 0; u < n; ++u) {
      chunk_sync(u);
      mfma_phase(u, any_c, any_prev);
      issue_next();
      barrier_no_fence();
      if (any_c) valu_phase(vis_c, key0_c, ck_c);
      else clear_p();
      any_prev = any_c;
      if (u + 1 < n) chunk_visit(u + 1, vis_c, any_c, key0_c, ck_c);
    }
    if (any_prev) mfma_phase(n, false, true);
    epilogue();
  } else {
    for (int u = 0; u < n; ++u) {
      chunk_sync(u);
      if (any_prev) valu_phase(vis_prev, key0_prev, ck_prev);
      else clear_p();
      barrier_no_fence();
      mfma_phase(u, any_c, any_prev);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) vis_prev[rt] = vis_c[rt];
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

bool prefill_bf16_rt_supported(int group, int d, int block, int top_k, int kv_len, int h_kv) {
  if (d != 256) return false;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16 && group != 32) return false;
  if (block < 1 || block > 1024 || top_k < 1 || top_k > kMaxTopK) return false;
  if ((long long)kv_len * h_kv * d >= (1ll << 32)) return false;  // 32-bit element offsets
  return (kv_len + block - 1) / block <= kPrefillMaxBlocks;
}

template <int D, int G>
static hipError_t launch_prefill_rt_t(const void* q, const void* k, const void* v,
                                      const int32_t* sel, void* out, float* lse, int batch,
                                      int n_q, int kv_len, const int32_t* kv_lens, int kv_stride,
                                      int h_q, int h_kv, int block, int top_k, float sm_scale,
                                      hipStream_t stream) {
  constexpr int MQ = RT_NW * (16 * RtTiles<G>::value / G);
  const int ntiles = (n_q + MQ - 1) / MQ;
  const long long total = (long long)ntiles * h_kv * batch;
  if (total > INT_MAX) return hipErrorInvalidValue;
  const PrefillScale sc = prefill_scale(sm_scale, kLog2e);
  hipLaunchKernelGGL((prefill_bf16_rt_kernel<D, G>), dim3((unsigned)total), dim3(RT_NW * 64), 0,
                     stream, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), sel, static_cast<uint16_t*>(out), lse, n_q,
                     kv_len, h_q, h_kv, block, top_k, sc.scale_log2, sc.q_and, sc.q_xor, ntiles,
                     (int)total, kv_lens, kv_stride);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16_rt(const void* q, const void* k, const void* v, const int32_t* sel,
                                  void* out, float* lse, int batch, int n_q, int kv_len,
                                  const int32_t* kv_lens, int kv_stride, int h_q, int h_kv, int d,
                                  int block, int top_k, float sm_scale, hipStream_t stream) {
  if (batch == 0 || n_q == 0) return hipSuccess;
  if (d != 256) return hipErrorInvalidValue;
#define QSA_G(gg)                                                                          \
  return launch_prefill_rt_t<256, gg>(q, k, v, sel, out, lse, batch, n_q, kv_len, kv_lens,    \
                                      kv_stride, h_q, h_kv, block, top_k, sm_scale, stream)
  switch (h_q / h_kv) {
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

}  // namespace qsa
