// common.h -- device helpers shared by the gfx950 kernels of libpa.so.
//
// Wave64 cross-lane primitives (DPP within a 16-lane row, swaps across rows),
// bf16 / E4M3 element handling; the kernels' parameter blocks are in params.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "params.h"

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x32_t __attribute__((ext_vector_type(32)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---- scalar conversions ------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (round to nearest even), lo in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return (uint16_t)(pack_bf16x2(x, 0.f) & 0xffffu);
}

// Two E4M3 codes (bytes 0,1 or 2,3 of w) -> packed bf16 pair; exact.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}

// bf16x2 dot product accumulated in fp32: a.lo*b.lo + a.hi*b.hi + c.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// 16-byte non-temporal global load (streamed data, read once).
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- cross-lane --------------------------------------------------------------

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_MIRROR = 0x140;

// All-reduce over each 16-lane row.
__device__ __forceinline__ float row_max16(float x) {
  x = fmaxf(x, dpp<DPP_XOR1>(x));
  x = fmaxf(x, dpp<DPP_XOR2>(x));
  x = fmaxf(x, dpp<DPP_ROW_HALF_MIRROR>(x));
  x = fmaxf(x, dpp<DPP_ROW_MIRROR>(x));
  return x;
}
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<DPP_XOR1>(x);
  x += dpp<DPP_XOR2>(x);
  x += dpp<DPP_ROW_HALF_MIRROR>(x);
  x += dpp<DPP_ROW_MIRROR>(x);
  return x;
}

// Swap-adds across lane rows (v_permlane32_swap / v_permlane16_swap, VALU).
// swap_add32(a, b): lanes 0..31 get a(l) + a(l+32), lanes 32..63 get
//   b(l-32) + b(l)  -- the two halves keep different values, fully summed.
// swap_add16(a, b): rows 0 and 2 (lanes 0-15, 32-47) get a(l) + a(l+16),
//   rows 1 and 3 get b(l-16) + b(l).
// With a == b both give the plain sum over the lane pair.
__device__ __forceinline__ float swap_add32(float a, float b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_add16(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return uniform((int)(threadIdx.x >> 6)); }

// Flags and counters in LDS shared by the waves of a workgroup: relaxed LDS
// atomics with fences restricted to LDS.  A plain acquire / release at
// workgroup scope would also wait for every outstanding global load of the
// wave (s_waitcnt vmcnt(0)), draining the K/V tiles it has in flight.
__device__ __forceinline__ int lds_load_acquire(const int32_t* p) {
  const int v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return v;
}
__device__ __forceinline__ void lds_store_release(int32_t* p, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int lds_add_release(int32_t* p, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int lds_exchange_acq_rel(int32_t* p, int v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  const int r = __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return r;
}

// Orders the calling wave's LDS writes before its following LDS reads, so
// its lanes read what other lanes of the same wave wrote.
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Workgroup barrier ordering LDS only: the calling waves' outstanding global
// loads stay in flight across it (a full __syncthreads would drain them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace pa
