/*
 * diffattn_micro.h -- C ABI of libdiffattn_micro.so, the microbenchmarks that
 * measure the gfx950 ceilings the differential-attention kernels are read
 * against: bf16 MFMA issue rate and the clock it runs at, HBM streaming read
 * and copy, the global -> LDS DMA stream, LDS row and transposing reads, and
 * VALU issue next to an MFMA stream.  Measurement only: nothing here is on
 * the attention path, and the attention library does not depend on it.
 *
 * Conventions: pointers are caller-owned DEVICE pointers, 16-byte aligned;
 * each call enqueues one kernel on `stream` and returns a hipError_t value
 * (0 = launched; hipErrorInvalidValue for a null pointer, a size that does
 * not fit the kernel's partition, or a sink / clock buffer too small, checked
 * before the launch).  Calls are timed by the caller (events on `stream`).
 *
 * Sinks: `sink` receives one float per thread (blocks x threads), a fold of
 * what the thread read or computed, so that no timed work is dead code.
 * Clock records: `clk` receives, per timed wave w (blocks x 8 waves, 512
 * threads a block), clk[4w .. 4w+3] = shader clock counter (s_memtime) at
 * start and end, 100 MHz real-time counter (s_memrealtime) at start and end;
 * a wave that is not timed leaves zeros.
 */
#ifndef DIFFATTN_MICRO_H
#define DIFFATTN_MICRO_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bf16 MFMA issue: every wave of `blocks` x 512 threads runs `iters` rounds
 * of 8 independent v_mfma_f32_32x32x16_bf16 (32768 flops each).
 * sink >= blocks*512 floats, clk >= blocks*32 records. */
int diffattn_micro_mfma(int blocks, int iters, float* sink, size_t sink_elems, unsigned long long* clk,
                        size_t clk_elems, hipStream_t stream);

/* Streaming read of `bytes` (a multiple of 16) from src by blocks x 256
 * threads, 16-byte non-temporal loads.  sink >= blocks*256 floats. */
int diffattn_micro_hbm_read(const void* src, size_t bytes, int blocks, float* sink, size_t sink_elems,
                            hipStream_t stream);

/* Copy of `bytes` (a multiple of 16) from src to dst (not overlapping) by
 * blocks x 256 threads. */
int diffattn_micro_hbm_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream);

/* global_load_lds_dwordx4 stream of `bytes` from src into LDS rings, by
 * blocks x 512 threads; bytes must be a multiple of blocks * 8192.
 * sink >= blocks*512 floats. */
int diffattn_micro_lds_dma(const void* src, size_t bytes, int blocks, float* sink, size_t sink_elems,
                           hipStream_t stream);

/* LDS reads, one block of 512 threads per CU: `iters` rounds of 8
 * conflict-free ds_read_b128 (transposing = 0, 1 KiB a wave-instruction) or
 * ds_read_b64_tr_b16 (transposing = 1, 512 B) per wave.
 * sink >= blocks*512 floats, clk >= blocks*32 records. */
int diffattn_micro_lds_read(int transposing, int blocks, int iters, float* sink, size_t sink_elems,
                            unsigned long long* clk, size_t clk_elems, hipStream_t stream);

/* VALU issue next to an MFMA stream, one block of 512 threads per CU: waves
 * 4..7 run `iters` rounds of 32 independent operations of kind 0 (fp32 add),
 * 1 (v_dot2c_f32_bf16), 2 (v_exp_f32), 3 (v_exp_f32 alternating with fp32
 * adds) or 4 (v_exp_f32 alternating with v_cvt_pk_bf16_f32); kind outside
 * 0..4 is hipErrorInvalidValue; waves 0..3, each sharing a SIMD with
 * one of them, run the MFMA stream above for mfma_iters rounds (0: they exit
 * at once).  Only waves 4..7 are timed.
 * sink >= blocks*512 floats, clk >= blocks*32 records. */
int diffattn_micro_valu(int kind, int mfma_iters, int blocks, int iters, float* sink, size_t sink_elems,
                        unsigned long long* clk, size_t clk_elems, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DIFFATTN_MICRO_H */
