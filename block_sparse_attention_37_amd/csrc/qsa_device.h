// Device-side helpers shared by the QSA kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 is carried as raw 16-bit patterns in memory.
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float -> bf16 bit pattern, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even; one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Element loads that turn either storage type into float.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
};

__device__ __forceinline__ uint64_t lanemask_lt() {
  return (uint64_t(1) << __lane_id()) - 1;
}

// Monotone map of a float score to uint32 (bigger float -> bigger integer), -0 == +0.
__device__ __forceinline__ uint32_t orderable(float x) {
  x = (x == 0.0f) ? 0.0f : x;
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// gfx950-only builtins, kept out of the host pass of the single-source compile (the host
// pass never runs device code, but it must still see kernel templates it can stub).
__device__ __forceinline__ void global_to_lds16(const void* gptr, void* lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  // each lane's 16 bytes land at lds_base + 16 * lane (lds_base is wave-uniform)
  __builtin_amdgcn_global_load_lds(gptr, lds_base, 16, 0, 0);
#endif
}

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Same 16-byte global -> LDS load, issued so that the compiler does not track it.  The
// compiler cannot tell LDS-direct loads into one buffer from LDS reads of another and
// would drain every such load before each LDS read; kernels using this form count the
// loads themselves and wait for them (s_waitcnt vmcnt) before the barrier that publishes
// the buffer.  No register is written by the instruction, and M0 / the address are read
// when it issues (M0 gets its previous value back right after).
__device__ __forceinline__ void global_to_lds16_untracked(const void* gptr, uint32_t lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t saved;  // M0 is reserved by the compiler: restore it after use
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(gptr));
#else
  (void)gptr;
  (void)lds_base;
#endif
}
// Two 16-byte global -> LDS loads from scalar bases (as global_to_lds16_saddr_untracked),
// sharing one save and restore of M0.
__device__ __forceinline__ void global_to_lds16x2_saddr_untracked(uint64_t sbase0, uint32_t voff0,
                                                                  uint32_t lds0, uint64_t sbase1,
                                                                  uint32_t voff1, uint32_t lds1) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t saved;  // M0 is reserved by the compiler: restore it after use
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %3, %5\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %4, %6\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds0)), "s"(__builtin_amdgcn_readfirstlane(lds1)),
        "v"(voff0), "v"(voff1), "s"(sbase0), "s"(sbase1));
#else
  (void)sbase0; (void)voff0; (void)lds0; (void)sbase1; (void)voff1; (void)lds1;
#endif
}

// A pointer every lane holds the same value of, moved to scalar registers.
__device__ __forceinline__ uint64_t uniform_ptr(const void* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return ((uint64_t)hi << 32) | lo;
#else
  return reinterpret_cast<uint64_t>(p);
#endif
}

// The same load with a scalar base: the lane reads sbase + voff (bytes; voff a 32-bit
// per-lane offset), so a loop that moves the base per iteration spends no vector
// instructions on addresses.
__device__ __forceinline__ void global_to_lds16_saddr_untracked(const void* sbase, uint32_t voff,
                                                                uint32_t lds_base) {
#if defined(__HIP_DEVICE_COMPILE__)
  uint32_t saved;  // M0 is reserved by the compiler: restore it after use
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(uniform_ptr(sbase)));
#else
  (void)sbase;
  (void)voff;
  (void)lds_base;
#endif
}

__device__ __forceinline__ void wait_all_memory() {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_s_waitcnt(0);
#endif
}
__device__ __forceinline__ int wave_uniform(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_readfirstlane(x);
#else
  return x;
#endif
}

// Makes a value opaque to the optimizer (no rematerialization, no sinking of its load).
__device__ __forceinline__ void keep_in_register(u32x4& w) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(w));
#endif
}

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size");
  return __builtin_bit_cast(To, f);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
#endif
}

// Workgroup barrier without the memory fence __syncthreads() implies: that fence would
// drain every outstanding LDS-direct load.  Callers wait for exactly the loads they need
// (wait_vmcnt) before the barrier; the clobber keeps the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void barrier_no_fence() {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_barrier" ::: "memory");
#endif
}

// LDS transpose read (ds_read_b64_tr_b16): inside each group of 16 lanes, lane i receives
// element i % 4 of the four 16-bit elements that lanes 4j + i / 4 (j = 0..3) point at.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return bitcast<u32x2>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
#else
  (void)p;
  return u32x2{0u, 0u};
#endif
}

}  // namespace qsa
