// lambda_h = exp(lq1_h . lk1_h) - exp(lq2_h . lk2_h) + lambda_init
// (aifetchly "Differential Transformer: Canceling LLM Attention Noise",
// section 3; paperleet "Differential Transformer Attention", the scalar
// parameterisation).  One wave per head (reparam_lambda, shared with the
// prefill kernels' fused path).  The result stays on the device so the
// forward call can consume it without a host round trip.
#include "common.h"
#include "kernels.h"

namespace diffattn {
namespace {

__global__ __launch_bounds__(64) void lambda_kernel(const float* __restrict__ lq1,
                                                    const float* __restrict__ lk1,
                                                    const float* __restrict__ lq2,
                                                    const float* __restrict__ lk2, int Dl,
                                                    float lambda_init, float* __restrict__ out) {
  const int h = blockIdx.x;
  const float lam = reparam_lambda(lq1, lk1, lq2, lk2, h, Dl, lambda_init);
  if (threadIdx.x == 0) out[h] = lam;
}

}  // namespace

hipError_t launch_lambda(const float* lq1, const float* lk1, const float* lq2, const float* lk2,
                         int H, int Dl, float lambda_init, float* out, hipStream_t stream) {
  if (!grid_fits(H, 64)) return hipErrorInvalidConfiguration;
  lambda_kernel<<<dim3(H), dim3(64), 0, stream>>>(lq1, lk1, lq2, lk2, Dl, lambda_init, out);
  return hipGetLastError();
}

}  // namespace diffattn
