// Device helpers shared by the HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace cpa {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// v_exp_f32 / v_log_f32: base-2 exponential and logarithm in hardware;
// exp2(-inf) = 0 and log2(0) = -inf.
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// bf16 <-> fp32. The narrowing conversion rounds to nearest even
// (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Workgroup barrier for LDS hand-offs only. __syncthreads() also waits for
// every outstanding global load of the wave (its release fence is a full
// s_waitcnt), which would expose the latency of tiles prefetched for later
// steps; here only LDS operations (lgkmcnt) must complete before s_barrier.
// The signal fences keep the compiler from moving memory accesses across it;
// a load's own consumer still gets its vmcnt wait from the compiler.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xc07f);  // vmcnt and expcnt unconstrained, lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Global position of local slot l on `rank` under round-robin placement with
// groups of `il` positions dealt to the cp ranks in turn.
__device__ __forceinline__ int rr_global_pos(int l, int cp, int rank, int il) {
  const int grp = l / il;
  return (grp * cp + rank) * il + (l - grp * il);
}

// Number of positions in [0, n) stored on `rank` (same placement).
__device__ __forceinline__ int rr_count_below(int n, int cp, int rank, int il) {
  if (n <= 0) return 0;
  const int cyc = il * cp;
  const int full = n / cyc;
  int rest = n - full * cyc - rank * il;
  rest = rest < 0 ? 0 : (rest > il ? il : rest);
  return full * il + rest;
}

}  // namespace cpa
