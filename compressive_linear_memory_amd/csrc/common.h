// Device helpers shared by the libinfini kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace infini {

typedef uint16_t bf16_t;   // bfloat16 storage bits

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even.  NaN stays NaN (quiet bit forced).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct io;
template <> struct io<float> {
  __device__ __forceinline__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct io<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(bf16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Tokens of sequence b of the call: all N, or, in a variable-length batch,
// lens[b] clamped to [0, N] (so no length can move an access outside the
// padded [N] rows of its slot).
__device__ __forceinline__ int seq_len_of(const int* lens, int b, int N) {
  return lens ? min(max(lens[b], 0), N) : N;
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads also waits
// for every outstanding global load and store of the wave; after this one,
// global loads issued before it stay in flight (their registers are waited
// for where they are used) and global stores drain in the background.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// max / sum over the four lanes l, l^16, l^32, l^48 (the four 16-lane rows
// of a wave): v_permlane16_swap exchanges rows 0<->1 and 2<->3,
// v_permlane32_swap the two wave halves, and each returns the lane's own
// value and its partner's; no LDS round trip.
__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ELU(x) + 1 with alpha = 1.
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }
// Its derivative: 1 for x > 0, exp(x) otherwise.
__device__ __forceinline__ float elu1_grad(float x) { return x > 0.f ? 1.f : __expf(x); }
// sigmoid with exact 0 / 1 at -inf / +inf.
__device__ __forceinline__ float sigmoid(float b) { return 1.f / (1.f + __expf(-b)); }

}  // namespace infini
