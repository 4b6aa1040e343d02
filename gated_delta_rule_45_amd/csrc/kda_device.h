// kda_device.h -- device helpers shared by the KDA HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): raw (stride 0) addressing with
// the gfx9-family data-format word. Accesses outside the range read zero and
// drop writes, so a tile's loads and stores cannot leave the tile.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// A value the caller knows to be the same in every lane (for example one
// loaded from a wave-uniform address), moved to a scalar register so that
// buffer resources and LDS bases built from it need no per-lane handling.
__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform(int64_t x) {
  const uint64_t u = static_cast<uint64_t>(x);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(u)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(u >> 32)));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Cache policy for streamed data touched once per call (the nt bit).
constexpr int kStreamPolicy = 2;

template <int kPolicy>
__device__ __forceinline__ f32x4 buffer_load_f32x4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kPolicy));
}

template <int kPolicy>
__device__ __forceinline__ void buffer_store_f32x4(f32x4 v, __amdgpu_buffer_rsrc_t r, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, kPolicy);
}

// bf16 is the upper half of an fp32: widening is a shift.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (gfx950's v_cvt_pk_bf16_f32;
// NaN stays a NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Loads N consecutive bf16 (N in {2,4,8,16,32}) with the widest aligned
// vector loads and widens them. The address must be aligned to min(2N, 16)
// bytes.
template <int N>
__device__ __forceinline__ void load_bf16(const uint16_t* p, float* out) {
  if constexpr (N >= 8) {
    static_assert(N % 8 == 0, "N must be a multiple of 8");
#pragma unroll
    for (int c = 0; c < N / 8; ++c) {
      uint4 w = reinterpret_cast<const uint4*>(p)[c];
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[c * 8 + 2 * i] = __uint_as_float(ws[i] << 16);
        out[c * 8 + 2 * i + 1] = __uint_as_float(ws[i] & 0xffff0000u);
      }
    }
  } else if constexpr (N == 4) {
    uint2 w = *reinterpret_cast<const uint2*>(p);
    out[0] = __uint_as_float(w.x << 16);
    out[1] = __uint_as_float(w.x & 0xffff0000u);
    out[2] = __uint_as_float(w.y << 16);
    out[3] = __uint_as_float(w.y & 0xffff0000u);
  } else {
    static_assert(N == 2, "unsupported N");
    uint32_t w = *reinterpret_cast<const uint32_t*>(p);
    out[0] = __uint_as_float(w << 16);
    out[1] = __uint_as_float(w & 0xffff0000u);
  }
}

// 1 / (1 + e^-z) with the hardware exponential and reciprocal (about 1 ulp
// each; the result is within a few ulp of the correctly rounded value).
__device__ __forceinline__ float sigmoid_f32(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// softplus(x) = max(x, 0) + ln(1 + e^-|x|). The log argument lies in
// (1, 2], where the hardware log2 (about 1 ulp) needs no range reduction.
__device__ __forceinline__ float softplus_f32(float x) {
  return fmaxf(x, 0.0f) + 0.693147180559945f * __builtin_amdgcn_logf(1.0f + __expf(-fabsf(x)));
}

// Per-channel log-decay from the raw gate input (same reading as the header):
//   x = raw_g + dt_bias, a = exp(A_log[h]);
//   g = -a * softplus(x)  or  g = lower_bound * sigmoid(a * x).
// softplus is evaluated as max(x, 0) + log(1 + exp(-|x|)), which cannot
// overflow; for large |x| the log term is below fp32 resolution of the sum.
__device__ __forceinline__ float gate_log_decay(float raw_g, float dt_bias, float a,
                                                bool has_lb, float lb) {
  const float x = raw_g + dt_bias;
  if (has_lb) return lb * sigmoid_f32(a * x);
  return -a * softplus_f32(x);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations (lgkmcnt = 0) and meets the other waves, but leaves global loads
// and stores in flight (unlike __syncthreads, whose fence drains them).
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt = 63, expcnt = 7, lgkmcnt = 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace kda
