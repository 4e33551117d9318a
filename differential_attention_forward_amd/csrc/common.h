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

// Causal work order.  Each XCD takes a contiguous range of the logical
// workgroup ids (xcd_remap); when that range holds whole heads, its query
// tiles go heaviest first across all of those heads (every head's last tile,
// then every head's second to last, ...), so that the XCD's compute units
// start the long causal rows first and finish together.  Otherwise each
// head's tiles go heaviest first, head after head.
__device__ inline void causal_order(int w, int n, int nqt, int& bh, int& qi) {
  const int per = n / kNumXcd;
  if (n % kNumXcd == 0 && per % nqt == 0) {
    const int hpx = per / nqt;
    const int x = w / per, j = w % per;
    bh = x * hpx + j % hpx;
    qi = j / hpx;
  } else {
    bh = w / nqt;
    qi = w % nqt;
  }
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

// Debug builds (-DDIFFATTN_LDS_POISON) fill every LDS array a kernel declares
// with all-ones words (NaN as fp32 and as bf16) at entry, before anything else
// touches LDS, so that reading LDS the kernel never wrote (a missing wait or
// barrier, a stray index) changes the result instead of reusing a stale value
// that happens to be right.  No-ops otherwise.  Every thread of the workgroup
// calls both, poison first for each array, then done once.
__device__ inline void lds_poison(void* p, size_t bytes) {
#ifdef DIFFATTN_LDS_POISON
  uint32_t* w = (uint32_t*)p;
  for (size_t i = threadIdx.x; i < bytes / 4; i += blockDim.x) w[i] = 0xffffffffu;
#else
  (void)p;
  (void)bytes;
#endif
}
__device__ inline void lds_poison_done() {
#ifdef DIFFATTN_LDS_POISON
  __syncthreads();
#endif
}

// bf16 <-> fp32 on raw 16-bit patterns (bf16 is the top half of an fp32).
__device__ inline float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// One 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4): lane i
// reads base + off_i (base uniform, kept in SGPRs; off_i an unsigned 32-bit
// byte offset) and its 16 bytes land at lds + 16 i.  Issued through asm so that
// the compiler's wait-count bookkeeping does not make every later LDS read wait
// for all tile loads in flight; their completion is awaited explicitly
// (vmcnt) before the tile barrier.
__device__ inline void dma16(const void* base, uint32_t off, const void* lds) {
  const uint32_t m = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds;
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m) : "memory", "m0");
}

// A pointer that is the same in every lane, moved to scalar registers (64-bit
// address arithmetic runs on the VALU, which would keep it in VGPRs).
template <typename Tp>
__device__ inline const Tp* scalar_ptr(const Tp* p) {
  // readfirstlane returns int: widen through uint32_t, not by sign extension
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (const Tp*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
}

// s_waitcnt vmcnt(N) lgkmcnt(0), then a workgroup barrier; the empty asm
// statements keep the compiler from moving memory accesses across it.
template <int N>
__device__ inline void wait_vm_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (((N >> 4) & 3) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte column swizzles.  gfx950's LDS has 64 banks of 4 bytes (256 bytes
// per clock): a ds_read_b128 serves 16 lanes per cycle and a
// ds_read_b64_tr_b16 32 lanes, so those lanes must cover 256 distinct bytes
// modulo 256.
//  K (row pitch 2D bytes): lanes 0..15 read rows r..r+15 at one logical
//  chunk; the swizzle makes (row mod (256 / pitch), physical chunk) distinct
//  over those 16 rows.
//  V (row pitch 2 DV bytes): the 32 lanes of a transposing read cover four
//  rows (keys) and one 64-byte group of four chunks per row; the swizzle
//  moves each of the four rows to its own 64-byte quarter of the banks.
template <int D>
__device__ inline int swz_k(int row) {
  return D == 32 ? ((row >> 2) & 3) : D == 64 ? ((row >> 1) & 7) : (row & 15);
}
template <int DV>
__device__ inline int swz_v(int row) {
  return DV >= 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
}

__device__ inline floatx16 splat16(float x) {
  floatx16 v;
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = x;
  return v;
}

// Probabilities 2^s of one 32x32 score block as a lane holds it (16 keys of
// one query), rounded to bf16 into the B-operand layout of the P.V MFMA, and
// the lane's fp32 sum of the unrounded values (a pairwise tree).  The sum is
// formed with plain fp32 adds: v_dot2c_f32_bf16 over the rounded values would
// take one instruction per pair but shares the matrix pipe, and stalls for
// the length of the other wave's MFMA stream on the same SIMD.
__device__ inline float expo16(const floatx16& s, bf16x8 (&pk)[2]) {
  float a[4];  // four running partial sums, so few values stay live
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float pa = __builtin_amdgcn_exp2f(s[2 * j]);
    const float pb = __builtin_amdgcn_exp2f(s[2 * j + 1]);
    const bf16x2 pw = {(bf16)pa, (bf16)pb};
    pk[j >> 2][2 * (j & 3)] = pw[0];
    pk[j >> 2][2 * (j & 3) + 1] = pw[1];
    if (j < 2) {
      a[2 * j] = pa;
      a[2 * j + 1] = pb;
    } else {
      a[(2 * j) & 3] += pa;
      a[(2 * j + 1) & 3] += pb;
    }
  }
  return (a[0] + a[1]) + (a[2] + a[3]);
}

__device__ inline float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace diffattn
