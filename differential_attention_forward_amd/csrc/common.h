// Shared device-side types and helpers for the differential-attention HIP
// library (gfx950 / CDNA4).  Nothing here is visible through the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace diffattn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(bf16))));
typedef bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(bf16))));
typedef bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(bf16))));
typedef float floatx16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float floatx4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

// log2(e): scores are carried in base-2 units so that exp() is one v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// Number of XCDs on MI355X; consecutive workgroup ids are dispatched
// round-robin over them, each XCD with its own L2.
constexpr int kNumXcd = 8;

// Maps a hardware workgroup id to a logical work index such that the
// workgroups an XCD runs back to back get consecutive work indices (so they
// share K/V in that XCD's L2).  Bijective on [0, n).
__device__ inline int xcd_remap(int bid, int n) {
  const int x = bid % kNumXcd;
  const int j = bid / kNumXcd;
  const int base = n / kNumXcd;
  const int rem = n % kNumXcd;
  return x * base + (x < rem ? x : rem) + j;
}

__device__ inline float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ inline float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// lambda of head h from its four re-parameterisation vectors ([H, Dl] each):
// exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init (aifetchly "Differential
// Transformer: Canceling LLM Attention Noise", section 3).  Called by a whole
// wave; strided fp32 products, a fixed-order wave reduction and two expf, so
// every caller (the lambda kernel, the fused prefill) gets the same bits.
// The result is returned in every lane.
__device__ inline float reparam_lambda(const float* __restrict__ lq1, const float* __restrict__ lk1,
                                       const float* __restrict__ lq2, const float* __restrict__ lk2,
                                       int h, int Dl, float lambda_init) {
  const int lane = threadIdx.x & 63;
  const size_t base = (size_t)h * Dl;
  float d1 = 0.0f, d2 = 0.0f;
  for (int i = lane; i < Dl; i += 64) {
    d1 = fmaf(lq1[base + i], lk1[base + i], d1);
    d2 = fmaf(lq2[base + i], lk2[base + i], d2);
  }
  d1 = wave_sum(d1);
  d2 = wave_sum(d2);
  const float e1 = expf(d1);
  const float e2 = expf(d2);
  return (e1 - e2) + lambda_init;
}

// bf16 <-> fp32 on raw 16-bit patterns (bf16 is the top half of an fp32).
__device__ inline float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace diffattn
