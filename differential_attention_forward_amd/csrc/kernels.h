// Internal launch interface between the C ABI (abi.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace diffattn {

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
  int B, H, T;
  float score_scale;  // log2(e) / sqrt(D)
  float out_scale;    // 1 - lambda_init (head norm only)
  float eps;
};

struct DecodeArgs {
  const void* q1;     // [B,H,D]
  const void* k1;     // [B,H,L,D]
  const void* q2;
  const void* k2;
  const void* v;      // [B,H,L,2D]
  const float* lam;   // [H]
  float* ws;          // [B,H,S, 2*(2D+2)] fp32 partial states
  void* out;          // [B,H,2D]
  int B, H, L, S;
  float score_scale;
  float out_scale;
  float eps;
};

// dtype: 0 = fp32, 1 = bf16 (same codes as the public enum)
hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, bool causal, bool headnorm,
                      hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int dtype, int D, bool headnorm,
                         hipStream_t stream);
// standard softmax attention, bf16, Q/K/V/O [B,H,T,D] (D = 64 or 128)
hipError_t launch_attention(const FwdArgs& a, int D, bool causal, hipStream_t stream);
hipError_t launch_lambda(const float* lq1, const float* lk1, const float* lq2,
                         const float* lk2, int H, int Dl, float lambda_init, float* out,
                         hipStream_t stream);

}  // namespace diffattn
