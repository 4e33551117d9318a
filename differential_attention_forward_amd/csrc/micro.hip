// Microbenchmarks of the gfx950 units the differential-attention kernels are
// bound by: the matrix cores (bf16 MFMA issue rate and the clock they run
// at), HBM (streaming read, copy, and the global -> LDS DMA path the prefill
// stages tiles with), LDS reads (the row reads and transposing reads that
// feed the MFMA operands), and the VALU next to an MFMA stream (fp32 adds,
// v_dot2c and v_exp on the wave that shares a SIMD with an MFMA wave).
// These are the measured ceilings the kernels' roofline fractions are read
// against; nothing here is on the attention path.
//
// Clock records: every timed wave stores, from lane 0, four 64-bit values at
// clk[4 * wave]: s_memtime (the shader clock counter) and s_memrealtime (a
// constant 100 MHz counter) at its start and at its end.  Their ratio is the
// clock the wave ran at.
#include "../../include/diffattn_micro.h"
#include "common.h"

namespace {

using namespace diffattn;

constexpr int kThreads = 512;  // 8 waves: waves w and w + 4 share a SIMD

__device__ inline void clock_mark(uint64_t& c, uint64_t& r) {
  c = __builtin_amdgcn_s_memtime();
  r = __builtin_amdgcn_s_memrealtime();
}

__device__ inline void clock_store(unsigned long long* clk, uint64_t c0, uint64_t c1, uint64_t r0, uint64_t r1) {
  if ((threadIdx.x & 63) == 0) {
    const size_t w = (size_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    clk[4 * w + 0] = c0;
    clk[4 * w + 1] = c1;
    clk[4 * w + 2] = r0;
    clk[4 * w + 3] = r1;
  }
}

__device__ inline void mfma_operands(bf16x8& a, bf16x8& b) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)((lane + e) * (1.0f / 512.0f));
    b[e] = (bf16)((e - lane) * (1.0f / 1024.0f));
  }
}

// `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16 per wave (32768
// flops each); 8 accumulators keep the matrix pipe busy without waiting on
// a result.
__device__ inline float mfma_stream(int iters) {
  bf16x8 a, b;
  mfma_operands(a, b);
  floatx16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = splat16(0.0f);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  return s;
}

__global__ __launch_bounds__(kThreads) void mfma_kernel(int iters, float* sink, unsigned long long* clk) {
  uint64_t c0, r0, c1, r1;
  clock_mark(c0, r0);
  const float s = mfma_stream(iters);
  clock_mark(c1, r1);
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
  clock_store(clk, c0, c1, r0, r1);
}

// Streaming read of n16 16-byte words, grid-stride, four loads in flight per
// lane; the words are folded together so that no load is dead.
__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ src, size_t n16, float* sink) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= (a ^ b) ^ (c ^ d);
  }
  for (; i < n16; i += stride) acc ^= src[i];
  sink[(size_t)blockIdx.x * 256 + threadIdx.x] = __uint_as_float((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) & 0x3fffffffu);
}

__global__ __launch_bounds__(256) void hbm_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

// Global -> LDS DMA stream (global_load_lds_dwordx4, the prefill's tile
// staging path).  Block b streams bytes [b * per_block, (b + 1) * per_block)
// of src; each wave copies 1 KiB per instruction into its own ring of 8
// 1 KiB LDS slots, with up to 6 copies in flight.  per_block is a multiple of
// 8 KiB (8 waves x 1 KiB).
constexpr int kDmaSlots = 8;
__global__ __launch_bounds__(kThreads) void lds_dma_kernel(const char* __restrict__ src, size_t per_block, float* sink) {
  __shared__ __attribute__((aligned(1024))) char ring[kThreads / 64][kDmaSlots][1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: LDS address in m0
  const size_t n = per_block / (kThreads / 64 * 1024);  // copies per wave
  const char* base = src + (size_t)blockIdx.x * per_block + (size_t)wave * 1024;
  for (size_t k = 0; k < n; ++k) {
    dma16(scalar_ptr(base + k * (kThreads / 64) * 1024), (uint32_t)lane * 16u, &ring[wave][k & (kDmaSlots - 1)][0]);
    // at most 6 copies outstanding, so a slot is never rewritten while its
    // previous copy is in flight
    __builtin_amdgcn_s_waitcnt((5 & 15) | (0 << 14) | (7 << 4) | (15 << 8));
  }
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = (float)ring[wave][lane & 7][lane * 16];
}

// LDS read rate: 8 waves per block, one block per CU (the 96 KiB of LDS it
// declares leave no room for a second), each wave reading its own 4 KiB
// region with conflict-free addresses: ds_read_b128 (16 lanes cover 256
// contiguous bytes) or ds_read_b64_tr_b16 (32 lanes cover 256 contiguous
// bytes).  8 reads per round.
template <bool TR>
__global__ __launch_bounds__(kThreads) void lds_read_kernel(int iters, float* sink, unsigned long long* clk) {
  __shared__ __attribute__((aligned(1024))) char lds[96 * 1024];
  for (int i = threadIdx.x; i < 96 * 1024 / 16; i += kThreads) {
    const uint32_t v = (uint32_t)i * 2654435761u;
    *(u32x4*)(lds + 16 * i) = u32x4{v, v ^ 1u, v ^ 2u, v ^ 3u};
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const char* region = lds + (threadIdx.x >> 6) * 4096;
  uint32_t off = TR ? lane * 8 : lane * 16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  uint64_t c0, r0, c1, r1;
  clock_mark(c0, r0);
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(off));  // the addresses are opaque: every round reads again
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if constexpr (TR) {
        const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(region + ((off + k * 512) & 4095)));
        const u32x2 w = __builtin_bit_cast(u32x2, v);
        acc[k & 3] ^= w[0] ^ w[1];
      } else {
        acc ^= *(const u32x4*)(region + ((off + k * 1024) & 4095));
      }
    }
  }
  clock_mark(c1, r1);
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = __uint_as_float((acc[0] ^ acc[1] ^ acc[2] ^ acc[3]) & 0x3fffffffu);
  clock_store(clk, c0, c1, r0, r1);
}

// VALU next to an MFMA stream.  Waves 4..7 run `iters` rounds of 32
// independent VALU operations (KIND 0: fp32 add, 1: v_dot2c_f32_bf16, 2:
// v_exp_f32, 3: v_exp_f32 alternating with fp32 adds, 4: v_exp_f32
// alternating with v_cvt_pk_bf16_f32: whether the transcendental unit lets
// ordinary VALU work issue beside it); waves 0..3, each on the SIMD of one of them, stream MFMAs for
// mfma_iters rounds when mfma_iters > 0 and exit at once otherwise.  One
// block per CU (96 KiB of LDS declared).  The clock records of waves 4..7
// give the VALU op's issue interval with and without the MFMA neighbour.
template <int KIND>
__global__ __launch_bounds__(kThreads) void valu_kernel(int iters, int mfma_iters, float* sink, unsigned long long* clk) {
  __shared__ char hold[96 * 1024];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float s = 0.0f;
  uint64_t c0 = 0, r0 = 0, c1 = 0, r1 = 0;
  if (wave < 4) {
    if (mfma_iters > 0) s = mfma_stream(mfma_iters);
  } else {
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = (lane + i) * -1e-3f;
    const float y = lane * 1e-6f;
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    clock_mark(c0, r0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if constexpr (KIND == 0) {
          x[i] = x[i] + y;
        } else if constexpr (KIND == 1) {
          x[i] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x[(i + 7) & 31]), ones, x[i], false);
        } else if constexpr (KIND == 2) {
          x[i] = __builtin_amdgcn_exp2f(x[i]);
        } else if constexpr (KIND == 3) {
          // v_exp_f32 and an independent fp32 add, alternating in issue order
          if (i % 2 == 0)
            asm volatile("v_exp_f32 %0, %0\n\tv_add_f32 %1, %1, %2" : "+v"(x[i]), "+v"(x[i + 1]) : "v"(y));
        } else {
          // v_exp_f32 and an independent bf16 pair conversion, alternating
          if (i % 2 == 0)
            asm volatile("v_exp_f32 %0, %0\n\tv_cvt_pk_bf16_f32 %1, %1, %2" : "+v"(x[i]), "+v"(x[i + 1]) : "v"(y));
        }
      }
      asm volatile("" : "+v"(x[0]), "+v"(x[8]), "+v"(x[16]), "+v"(x[24]));
    }
    clock_mark(c1, r1);
#pragma unroll
    for (int i = 0; i < 32; ++i) s += x[i];
  }
  hold[threadIdx.x] = (char)lane;
  __syncthreads();
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s + (float)hold[(threadIdx.x + 1) & 511];
  clock_store(clk, c0, c1, r0, r1);
}

int check_out(const void* sink, size_t sink_elems, int blocks, int threads, const void* clk, size_t clk_elems) {
  if (!sink || blocks < 1) return (int)hipErrorInvalidValue;
  if (sink_elems < (size_t)blocks * threads) return (int)hipErrorInvalidValue;
  if (clk && clk_elems < (size_t)blocks * (threads / 64) * 4) return (int)hipErrorInvalidValue;
  return 0;
}

int launched() { return (int)hipGetLastError(); }

}  // namespace

extern "C" {

int diffattn_micro_mfma(int blocks, int iters, float* sink, size_t sink_elems, unsigned long long* clk,
                        size_t clk_elems, hipStream_t stream) {
  if (!clk || iters < 1) return (int)hipErrorInvalidValue;
  if (int e = check_out(sink, sink_elems, blocks, kThreads, clk, clk_elems)) return e;
  mfma_kernel<<<blocks, kThreads, 0, stream>>>(iters, sink, clk);
  return launched();
}

int diffattn_micro_hbm_read(const void* src, size_t bytes, int blocks, float* sink, size_t sink_elems,
                            hipStream_t stream) {
  if (!src || bytes < 16 || bytes % 16 || (uintptr_t)src % 16) return (int)hipErrorInvalidValue;
  if (int e = check_out(sink, sink_elems, blocks, 256, nullptr, 0)) return e;
  hbm_read_kernel<<<blocks, 256, 0, stream>>>((const u32x4*)src, bytes / 16, sink);
  return launched();
}

int diffattn_micro_hbm_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream) {
  if (!src || !dst || blocks < 1 || bytes < 16 || bytes % 16 || (uintptr_t)src % 16 || (uintptr_t)dst % 16)
    return (int)hipErrorInvalidValue;
  const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
  if (s < d + bytes && d < s + bytes) return (int)hipErrorInvalidValue;
  hbm_copy_kernel<<<blocks, 256, 0, stream>>>((const u32x4*)src, (u32x4*)dst, bytes / 16);
  return launched();
}

int diffattn_micro_lds_dma(const void* src, size_t bytes, int blocks, float* sink, size_t sink_elems,
                           hipStream_t stream) {
  if (!src || (uintptr_t)src % 16) return (int)hipErrorInvalidValue;
  if (int e = check_out(sink, sink_elems, blocks, kThreads, nullptr, 0)) return e;
  const size_t unit = (size_t)(kThreads / 64) * 1024;
  if (bytes % ((size_t)blocks * unit) || bytes == 0) return (int)hipErrorInvalidValue;
  lds_dma_kernel<<<blocks, kThreads, 0, stream>>>((const char*)src, bytes / blocks, sink);
  return launched();
}

int diffattn_micro_lds_read(int transposing, int blocks, int iters, float* sink, size_t sink_elems,
                            unsigned long long* clk, size_t clk_elems, hipStream_t stream) {
  if (!clk || iters < 1) return (int)hipErrorInvalidValue;
  if (int e = check_out(sink, sink_elems, blocks, kThreads, clk, clk_elems)) return e;
  if (transposing)
    lds_read_kernel<true><<<blocks, kThreads, 0, stream>>>(iters, sink, clk);
  else
    lds_read_kernel<false><<<blocks, kThreads, 0, stream>>>(iters, sink, clk);
  return launched();
}

int diffattn_micro_valu(int kind, int mfma_iters, int blocks, int iters, float* sink, size_t sink_elems,
                        unsigned long long* clk, size_t clk_elems, hipStream_t stream) {
  if (!clk || iters < 1 || mfma_iters < 0 || kind < 0 || kind > 4) return (int)hipErrorInvalidValue;
  if (int e = check_out(sink, sink_elems, blocks, kThreads, clk, clk_elems)) return e;
  if (kind == 0) valu_kernel<0><<<blocks, kThreads, 0, stream>>>(iters, mfma_iters, sink, clk);
  if (kind == 1) valu_kernel<1><<<blocks, kThreads, 0, stream>>>(iters, mfma_iters, sink, clk);
  if (kind == 2) valu_kernel<2><<<blocks, kThreads, 0, stream>>>(iters, mfma_iters, sink, clk);
  if (kind == 3) valu_kernel<3><<<blocks, kThreads, 0, stream>>>(iters, mfma_iters, sink, clk);
  if (kind == 4) valu_kernel<4><<<blocks, kThreads, 0, stream>>>(iters, mfma_iters, sink, clk);
  return launched();
}

}  // extern "C"
