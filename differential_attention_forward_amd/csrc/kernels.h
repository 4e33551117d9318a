// Internal launch interface between the C ABI (abi.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace diffattn {

// What one dispatch can express: at most 2^31 - 1 workgroups along x, and a
// grid of at most 2^32 - 1 work-items (the dispatch packet holds the grid
// size in work-items as a 32-bit value).  Every launcher checks its shape.
inline bool grid_fits(long long blocks, long long threads) {
  return blocks >= 1 && blocks <= 0x7fffffffLL && blocks * threads <= 0xffffffffLL;
}

// Threads of a decode split-K workgroup (decode_partial_kernel and
// decode_v2_mma_kernel): the decode grid is B x H (x Hkv for V2) x S of them.
constexpr int kDecodeThreads = 256;

// Every prefill, training-forward and backward launch runs at most 4
// work-items per query (or key) row of its padded row range, and pads each
// head's T rows by at most 255, so 4 B H (T + 255) bounds their grids; the
// entry points refuse larger shapes before any launch.  (Such shapes need
// more than 2^30 rows, i.e. inputs far beyond one GPU's memory.)
inline bool row_grid_fits(long long B, long long H, long long T) {
  return 4 * B * H * (T + 255) <= 0xffffffffLL;
}

struct FwdArgs {
  const void* q1;
  const void* k1;
  const void* q2;
  const void* k2;
  const void* v;
  const float* lam;   // [H], or null when lvec[0] is set
  // fused lambda: the four re-parameterisation vectors [H, Dl] (lvec[0] null
  // = use lam), lambda_init added to it, and an optional [H] copy of lambda
  const float* lvec[4];
  int Dl;
  float lam_init;
  float* lam_out;
  void* out;
  // training forward (bf16 kernel only; null = inference): each map's
  // normalised output t1 = A1 V, t2 = A2 V as fp32 [B,H,T,2D], and the
  // log2-domain log-sum-exp of each map's scaled scores, fp32 [B,H,2,T]
  float* save_o1;
  float* save_o2;
  float* save_lse;
  int B, H, T;
  int Hkv;            // V2 only: KV heads; head h reads KV head h / (H / Hkv)
  int window;         // causal sliding window W (bf16 kernel): keys i - W < j <= i; 0 = none
  float score_scale;  // log2(e) / sqrt(D)
  float out_scale;    // 1 - lambda_init (head norm only)
  float eps;
  // bf16 kernel: element strides of q1, k1, q2, k2, v, out (in that order)
  // between batches, heads and rows; each row is contiguous.  K and V index
  // KV heads.  Dense layouts get them from dense_strides().
  long long sb[6], sh[6];
  int sr[6];
};

// Strides of densely packed [B, H, T, D] queries, [B, Hkv, T, D] keys,
// [B, Hkv, T, DV] values and a [B, H, T, DV] output.
inline void dense_strides(FwdArgs& a, int H, int Hkv, int T, int D, int DV) {
  const long long w[6] = {D, D, D, D, DV, DV};
  const long long heads[6] = {H, Hkv, H, Hkv, Hkv, H};
  for (int i = 0; i < 6; ++i) {
    a.sr[i] = (int)w[i];
    a.sh[i] = (long long)T * w[i];
    a.sb[i] = heads[i] * T * w[i];
  }
}

struct DecodeArgs {
  const void* q1;     // [B,H,D]
  const void* k1;     // [B,H,L,D]
  const void* q2;
  const void* k2;
  const void* v;      // [B,H,L,2D]
  const float* lam;   // [H]
  float* ws;          // [B,H,S, 2*(2D+2)] fp32 partial states
  void* out;          // [B,H,2D]
  const int* lens;    // [B] filled cache rows per sequence, or null (all L)
  int B, H, L, S;
  int Hkv;            // V2 only: KV heads; head h reads KV head h / (H / Hkv)
  float score_scale;
  float out_scale;
  float eps;
};

// Backward pass (bf16).  Inputs as in the forward; o1, o2, lse are what the
// training forward saved.  Workspace: dopre [B,H,T,2D] bf16, stats
// [B,H,4,Tp] fp32 (lse1, lse2, D1, D2; Tp = T rounded up to 64) and
// dlam_part [B,H,nchunk] fp32 (nchunk = Tp / 64).
struct BwdArgs {
  const void* q1;
  const void* k1;
  const void* q2;
  const void* k2;
  const void* v;
  const void* dout;    // [B,H,T,2D]
  const float* o1;     // [B,H,T,2D]
  const float* o2;
  const float* lse;    // [B,H,2,T]
  const float* lam;    // [H]
  void* dopre;
  float* stats;
  float* dlam_part;
  void* dq1;
  void* dk1;
  void* dq2;
  void* dk2;
  void* dv;
  float* dlam;         // [H]
  const float* lvec[4];  // optional [H, Dl] re-parameterisation vectors
  float* dlvec[4];       // their gradients (set iff lvec[0] is)
  int Dl;
  int B, H, T, Tp, nchunk;
  float score_scale;   // log2(e) / sqrt(D)
  float grad_scale;    // 1 / sqrt(D)
  float out_scale;     // 1 - lambda_init (head norm only)
  float eps;
};

// dtype: 0 = fp32, 1 = bf16 (same codes as the public enum)
hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, bool causal, bool headnorm,
                      hipStream_t stream);
// Device address of the library-held decode scratch of the current device
// (DIFFATTN_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned), looked up on the
// first call per device.
hipError_t decode_scratch(void** ptr);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int D, bool headnorm,
                         hipStream_t stream);
// DIFF V2 decode, bf16: q1/q2 [B,H,D], k/v caches [B,Hkv,L,D], out [B,H,D];
// group size H / Hkv in {1, 2, 4}, D = 64 or 128
hipError_t launch_decode_v2(const DecodeArgs& a, int D, hipStream_t stream);
// standard softmax attention, bf16, Q/K/V/O [B,H,T,D] (D = 64 or 128)
hipError_t launch_attention(const FwdArgs& a, int D, bool causal, hipStream_t stream);
// DIFF V2, bf16: Q1/Q2/O [B,H,T,D], K/V [B,Hkv,T,D] (D = 64 or 128)
hipError_t launch_v2(const FwdArgs& a, int D, bool causal, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int D, bool causal, bool headnorm, hipStream_t stream);
hipError_t launch_lambda(const float* lq1, const float* lk1, const float* lq2,
                         const float* lk2, int H, int Dl, float lambda_init, float* out,
                         hipStream_t stream);

}  // namespace diffattn
