// Block-sparse decode attention (one new query token per sequence) on bf16 matrix cores.
//
// Qwen4-Exp model page, overview: the query attends its selected contiguous blocks and
// its own incomplete trailing block; usage tips: cached generation keeps the QSA indexer
// state on device, the attention key/value cache is a per-sequence store.
//
// HBM-bound: every selected key/value byte is read once.  The token list of a sequence
// (selected blocks in ascending order, then the trailing tokens) is cut into 64-key
// chunks; a workgroup handles one (sequence, KV head, split) = a contiguous run of those
// chunks.  Key and value rows go global -> LDS directly (global_load_lds_dwordx4, no
// registers) through a ring of NS stages, so NS-1 chunks are always in flight while one
// is used; the loads are issued outside the compiler's view and waited for by count.  The
// G query heads sharing the KV head form the 16 MFMA rows (rows >= G are zero).  Each of
// the 4 waves takes 16 keys of a chunk:
//   S^T = K . Q^T on 16x16x32 MFMAs (A = K rows from LDS),
//   O^T += V^T . P^T on 16x16x16 MFMAs (A = V^T through the LDS transpose read),
// with per-wave online softmax; the waves' partial states meet in LDS at the end.  With
// more than one split, each split writes a normalised partial output and its
// log-sum-exp to the caller's workspace and a small merge kernel combines them.
//
// LDS layout of a stage: K rows, then V rows, each row D*2 bytes with its 16-byte units
// permuted by XOR (K: with r & (D/8 - 1); V: with 2 * (r & (D/16 - 1))).  Every LDS-direct
// load instruction then fetches whole rows (full cache lines), and the operand reads of a
// wave (16 rows x one unit for K, 16 rows x 32 bytes for the V transpose read) spread over
// all banks.
#include "qsa_device.h"
#include "qsa_internal.h"

#include <climits>
#include <mutex>

namespace qsa {

namespace {
constexpr int KC = 64;  // keys per chunk

// LDS stages: four at D <= 128 (128 KB); two at D = 256, where a stage alone is 64 KB.
template <int D>
struct DecodeStages {
  static constexpr int value = D >= 256 ? 2 : 4;
};

__device__ __forceinline__ f32x4 mfma16x16x16_bf16(u32x2 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<s16x4>(a), bitcast<s16x4>(b), c, 0, 0, 0);
}
template <int D>
__device__ __forceinline__ int k_swz(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int v_swz(int r) { return 2 * (r & (D / 16 - 1)); }
}  // namespace

template <int D>
__global__ __launch_bounds__(256, 1) void decode_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc,
    const uint16_t* __restrict__ vc, const int32_t* __restrict__ kv_lens,
    const int32_t* __restrict__ sel, uint16_t* __restrict__ out, float* __restrict__ lse,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int max_len, int h_q, int h_kv,
    int G, int block, int top_k, float scale_log2, int nsplit) {
  constexpr int NQT = D / 32;   // k-steps of S^T = K slabs
  constexpr int NDT = D / 16;   // 16-row d tiles of O^T = V slabs
  constexpr int TILE = KC * D;  // elements of one K (or V) chunk
  constexpr int NU = D / 8;       // 16-byte units per row
  constexpr int RPI = 64 / NU;    // rows per LDS-direct instruction (1 KB)
  constexpr int KI = KC / 4 / RPI;  // instructions per wave per K (or V) chunk: 16 rows each
  constexpr int DPC = 2 * KI;     // LDS-direct instructions per wave per chunk
  constexpr int NS = DecodeStages<D>::value;
  static_assert(2 * DPC < 64, "vmcnt range");
  static_assert(4 * D * 16 * 4 <= NS * 2 * KC * D * 2, "the wave merge reuses the ring");

  __shared__ __attribute__((aligned(16))) uint16_t ring[NS * 2 * TILE];
  __shared__ int32_t list[kMaxTopK];
  __shared__ int32_t list_n;
  __shared__ float wm[4][16];
  __shared__ float wl[4][16];

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_uniform(tid >> 6);

  int len = kv_lens[b];
  len = len < 0 ? 0 : (len > max_len ? max_len : len);
  const int n = len / block;
  const int ntrail = len - n * block;

  // query rows: lane holds row nr = lane & 15 (query head g*G + nr when nr < G).  The Q
  // loads are issued before the selection is read, so the two latencies overlap.
  const int nr = lane & 15;
  const int quarter = lane >> 4;
  u32x4 qraw[NQT];
  {
    const bool ok = nr < G;
    const uint16_t* qp = q + ((size_t)b * h_q + g * G + (ok ? nr : 0)) * D + quarter * 8;
#pragma unroll
    for (int t = 0; t < NQT; ++t)
      qraw[t] = ok ? *reinterpret_cast<const u32x4*>(qp + t * 32) : u32x4{0u, 0u, 0u, 0u};
  }

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
  bf16x8 qreg[NQT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) {
    // opaque to the optimizer: Q stays in registers (a re-load inside the loop would also
    // wait for the key/value loads in flight); its wait comes before those loads are issued
    keep_in_register(qraw[t]);
    qreg[t] = bitcast<bf16x8>(qraw[t]);
  }
  const int mv = list_n;
  const int nsub = (block + KC - 1) / KC;
  const int tunits = (ntrail + KC - 1) / KC;
  const int nchunks = mv * nsub + tunits;
  const int c_begin = (int)((long long)nchunks * split / nsplit);
  const int c_end = (int)((long long)nchunks * (split + 1) / nsplit);
  const int nch = c_end - c_begin;

  const uint32_t kv_row = (uint32_t)h_kv * D;  // elements between consecutive tokens
  const uint16_t* kbase = kc + ((size_t)b * max_len * h_kv + g) * D;
  const uint16_t* vbase = vc + ((size_t)b * max_len * h_kv + g) * D;

  auto chunk_keys = [&](int u, int& key0, int& ck) __attribute__((always_inline)) {
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

  // LDS-direct loads of chunk u into stage u % NS: each instruction fills 1 KB = RPI whole
  // rows; wave w fills rows 16w .. 16w+15 of K and of V; lane -> (row lane / NU, physical
  // unit lane % NU) and fetches the logical unit the swizzle maps there.  Rows past the
  // chunk re-read its last key (their scores are masked).
  const uint32_t ring_lds = lds_addr(ring);
  const int l_row = lane / NU, l_unit = lane % NU;
  auto issue = [&](int u) __attribute__((always_inline)) {
    int key0, ck;
    chunk_keys(u, key0, ck);
    const uint32_t st = ring_lds + (uint32_t)(u % NS) * (2 * TILE * 2);
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int r0 = 16 * wave + RPI * i;
      const int r = r0 + l_row;
      const uint32_t grow = (uint32_t)(key0 + min(r, ck - 1));
      global_to_lds16_untracked(kbase + grow * kv_row + 8 * (l_unit ^ k_swz<D>(r)), st + r0 * D * 2);
      global_to_lds16_untracked(vbase + grow * kv_row + 8 * (l_unit ^ v_swz<D>(r)),
                                st + TILE * 2 + r0 * D * 2);
    }
  };

  int issued = 0;
  for (; issued < NS - 1 && issued < nch; ++issued) issue(c_begin + issued);

  float m_run = -__builtin_inff();
  float l_run = 0.f;
  f32x4 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane byte offsets of the operand reads inside a stage (this wave's 16 keys):
  //   K: row kw + nr, logical unit 4t + quarter;
  //   V (transpose read): row kw + 4*quarter + nr / 4, columns 16*dt + 4*(nr % 4) .. +3.
  const int kw = wave * 16;
  int k_off[NQT], v_off[NDT];
#pragma unroll
  for (int t = 0; t < NQT; ++t) k_off[t] = (kw + nr) * D * 2 + 16 * ((4 * t + quarter) ^ k_swz<D>(kw + nr));
  {
    const int vr = kw + 4 * quarter + (nr >> 2);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      v_off[dt] = TILE * 2 + vr * D * 2 + 16 * ((2 * dt + ((nr & 3) >> 1)) ^ v_swz<D>(vr)) + 8 * (nr & 1);
  }

  for (int i = 0; i < nch; ++i) {
    // chunk i must have landed; the (at most NS-2) chunks after it may stay in flight
    const int after = issued - i - 1;
    if (after >= 2) wait_vmcnt<2 * DPC>();
    else if (after == 1) wait_vmcnt<DPC>();
    else wait_vmcnt<0>();
    barrier_no_fence();
    // every wave is past chunk i-1: its stage takes chunk i+NS-1
    if (issued < nch) {
      issue(c_begin + issued);
      ++issued;
    }
    const int u = c_begin + i;
    int key0, ck;
    chunk_keys(u, key0, ck);
    const char* st = reinterpret_cast<const char*>(ring + (u % NS) * (2 * TILE));
    if (kw < ck) {
      f32x4 s{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < NQT; ++t) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + k_off[t]);
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
      // B operand: P^T at keys 4*quarter + {0..3}, column nr (the S^T accumulator layout)
      const u32x2 pb{pack_bf16x2(e0, e1), pack_bf16x2(e2, e3)};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        O[dt] *= alpha;
        // A operand: V^T rows d = 16*dt + nr, keys 4*quarter + {0..3} of this wave
        const u32x2 a = lds_read_tr16(reinterpret_cast<const uint16_t*>(st + v_off[dt]));
        O[dt] = mfma16x16x16_bf16(a, pb, O[dt]);
      }
    }
  }
  __syncthreads();  // every wave is done with the ring before it holds the partial outputs

  // ---- combine the 4 waves (rows nr, d = dt*16 + 4*quarter + r) ----
  float lsum = l_run + __shfl_xor(l_run, 16);
  lsum += __shfl_xor(lsum, 32);
  if (quarter == 0) {
    wm[wave][nr] = m_run;
    wl[wave][nr] = lsum;
  }
  float* wo = reinterpret_cast<float*>(ring);  // [4][D][16] floats, fits in the ring
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

// The same combination with one wave per (sequence, query head) for NSP = 2 .. 4 splits: each
// lane takes D / 64 consecutive elements, and every load of the partial results is issued
// before any of them is used, so the kernel waits for memory once.  Per element the
// arithmetic is that of decode_merge_kernel.
template <int D, int NSP>
__global__ __launch_bounds__(64) void decode_merge_few_kernel(const float* __restrict__ ws_o,
                                                             const float* __restrict__ ws_lse,
                                                             uint16_t* __restrict__ out,
                                                             float* __restrict__ lse) {
  constexpr int E = D / 64;
  static_assert(E == 1 || E == 2 || E == 4, "elements per lane");
  const size_t bh = blockIdx.x;
  const int lane = threadIdx.x;
  float ls[NSP];
  float o[NSP][E];
#pragma unroll
  for (int s = 0; s < NSP; ++s) ls[s] = ws_lse[bh * NSP + s];
#pragma unroll
  for (int s = 0; s < NSP; ++s) {
    const float* src = ws_o + (bh * NSP + s) * D + lane * E;
    if constexpr (E == 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[s][e] = x[e];
    } else if constexpr (E == 2) {
      const f32x2_t x = *reinterpret_cast<const f32x2_t*>(src);
      o[s][0] = x[0];
      o[s][1] = x[1];
    } else {
      o[s][0] = *src;
    }
  }
  float M = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < NSP; ++s) M = fmaxf(M, ls[s]);
  const float Mu = (M == -__builtin_inff()) ? 0.f : M;
  float L = 0.f, acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s = 0; s < NSP; ++s) {
    const float f = __builtin_amdgcn_exp2f(ls[s] - Mu);
    L += f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += f * o[s][e];
  }
  uint32_t bits[E];
#pragma unroll
  for (int e = 0; e < E; ++e) bits[e] = f32_to_bf16(L > 0.f ? acc[e] / L : 0.f);
  uint16_t* dst = out + bh * D + lane * E;
  if constexpr (E == 4) {
    *reinterpret_cast<u32x2*>(dst) = u32x2{bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16)};
  } else if constexpr (E == 2) {
    *reinterpret_cast<uint32_t*>(dst) = bits[0] | (bits[1] << 16);
  } else {
    *dst = (uint16_t)bits[0];
  }
  if (lse && lane == 0) lse[bh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

bool decode_bf16_supported(int group, int d, int block, int top_k, int max_len, int h_kv) {
  if (d != 64 && d != 128 && d != 256) return false;
  if (group < 1 || group > 16) return false;
  // element offsets of K / V rows within one sequence's cache are 32-bit
  if ((long long)max_len * h_kv * d >= (1ll << 32)) return false;
  return block >= 1 && block <= 1024 && top_k >= 1 && top_k <= kMaxTopK;
}

// Workgroups that run at once: one per CU (the LDS ring takes 128 KB at D = 128).  The count
// is read from the device current at the first call; the initialisation of a function-local
// static is thread-safe, so concurrent first calls from several host threads agree.
static int decode_slots() {
  static const int slots = [] {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    return cus;
  }();
  return slots;
}

// Splits of each (sequence, KV head): the smallest count whose workgroups fill at least 90%
// of whole rounds of the workgroups that run at once, with at least ~4 chunks per split.
int decode_num_splits(int batch, int h_kv, int block, int top_k) {
  const long long units = (long long)batch * h_kv;
  if (units <= 0) return 1;
  const long long slots = decode_slots();
  const long long chunks = (long long)top_k * ((block + KC - 1) / KC) + (block + KC - 2) / KC;
  long long max_split = chunks / 4;
  if (max_split > 32) max_split = 32;
  if (max_split < 1) max_split = 1;
  for (long long s = 1; s <= max_split; ++s) {
    const long long wgs = units * s;
    const long long rounds = (wgs + slots - 1) / slots;
    if (wgs * 10 >= rounds * slots * 9) return (int)s;
  }
  return (int)max_split;
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
  uint16_t* o16 = static_cast<uint16_t*>(out);
  const dim3 rows(batch * h_q);
  switch (nsplit) {
    case 2: hipLaunchKernelGGL((decode_merge_few_kernel<D, 2>), rows, dim3(64), 0, stream, ws_o, ws_lse, o16, lse); break;
    case 3: hipLaunchKernelGGL((decode_merge_few_kernel<D, 3>), rows, dim3(64), 0, stream, ws_o, ws_lse, o16, lse); break;
    case 4: hipLaunchKernelGGL((decode_merge_few_kernel<D, 4>), rows, dim3(64), 0, stream, ws_o, ws_lse, o16, lse); break;
    default:
      hipLaunchKernelGGL((decode_merge_kernel<D>), rows, dim3(D), 0, stream, ws_o, ws_lse, o16, lse, nsplit);
  }
  return hipGetLastError();
}

hipError_t launch_decode_bf16(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* kv_lens, const int32_t* sel, void* out, float* lse,
                              int batch, int max_len, int h_q, int h_kv, int d, int block,
                              int top_k, float sm_scale, void* workspace, int nsplit,
                              hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  if (d == 256)
    return launch_decode_t<256>(q, k_cache, v_cache, kv_lens, sel, out, lse, batch, max_len, h_q,
                                h_kv, block, top_k, sm_scale, workspace, nsplit, stream);
  if (d == 128)
    return launch_decode_t<128>(q, k_cache, v_cache, kv_lens, sel, out, lse, batch, max_len, h_q,
                                h_kv, block, top_k, sm_scale, workspace, nsplit, stream);
  if (d == 64)
    return launch_decode_t<64>(q, k_cache, v_cache, kv_lens, sel, out, lse, batch, max_len, h_q,
                               h_kv, block, top_k, sm_scale, workspace, nsplit, stream);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Decode without a caller workspace, for callers that cannot allocate device memory.  The
// split-K partial results go to `scratch`, a file-scope device array of
// kDecodeScratchBytes that every device holds from the library's load until the process
// ends.  In host code `scratch` only names the symbol; its device address (one per device)
// comes from hipGetSymbolAddress, looked up once per device with that device current and
// kept in g_scratch_ptr.  Calls on one device share the array, so two calls in flight on
// that device at once race; a split writes every partial it later reads, so nothing needs
// clearing between calls.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  *ptr = g_scratch_ptr[dev];
  return g_scratch_err[dev];
}

}  // namespace qsa
