// C ABI of the differential-attention library: argument validation on the
// host (before any HIP call) and dispatch to the kernels.  Declarations and
// the contract of every entry point are in include/diffattn.h.
#include <math.h>
#include <stdint.h>

#include "../../include/diffattn.h"
#include "kernels.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

size_t elem_bytes(int dtype) { return dtype == DIFFATTN_BF16 ? 2 : 4; }

bool supported_d(int D) { return D == 32 || D == 64 || D == 128; }

diffattn_status from_hip(hipError_t e) { return e == hipSuccess ? DIFFATTN_OK : DIFFATTN_ERR_HIP; }

}  // namespace

extern "C" {

const char* diffattn_status_string(int status) {
  switch (status) {
    case DIFFATTN_OK: return "ok";
    case DIFFATTN_ERR_INVALID: return "invalid argument";
    case DIFFATTN_ERR_UNSUPPORTED: return "unsupported dtype, head width, alignment or size";
    case DIFFATTN_ERR_WORKSPACE: return "decode workspace missing or too small";
    case DIFFATTN_ERR_HIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

float diffattn_lambda_init(int layer) {
  if (layer < 1) return NAN;
  return (float)(0.8 - 0.6 * exp(-0.3 * (double)(layer - 1)));
}

diffattn_status diffattn_lambda(const float* lq1, const float* lk1, const float* lq2,
                                const float* lk2, int H, int Dl, float lambda_init,
                                float* lambda_out, hipStream_t stream) {
  if (!lq1 || !lk1 || !lq2 || !lk2 || !lambda_out || H < 1 || Dl < 1) return DIFFATTN_ERR_INVALID;
  const void* ins[4] = {lq1, lk1, lq2, lk2};
  for (const void* p : ins)
    if (!aligned(p, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(lambda_out, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  const size_t nin = (size_t)H * Dl * sizeof(float), nout = (size_t)H * sizeof(float);
  for (const void* p : ins)
    if (overlaps(lambda_out, nout, p, nin)) return DIFFATTN_ERR_INVALID;
  return from_hip(diffattn::launch_lambda(lq1, lk1, lq2, lk2, H, Dl, lambda_init, lambda_out,
                                          stream));
}

namespace {

// Checks shared by the two prefill entry points; fills the tensor part of a.
diffattn_status check_fwd(int dtype, int B, int H, int T, int D, const void* q1, const void* k1,
                          const void* q2, const void* k2, const void* v, int headnorm, float eps,
                          void* out, diffattn::FwdArgs& a, size_t& out_bytes) {
  if (!q1 || !k1 || !q2 || !k2 || !v || !out) return DIFFATTN_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1) return DIFFATTN_ERR_INVALID;
  if (headnorm && !(eps > 0.0f)) return DIFFATTN_ERR_INVALID;
  if (dtype != DIFFATTN_F32 && dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
  if (!supported_d(D)) return DIFFATTN_ERR_UNSUPPORTED;
  const void* ins[5] = {q1, k1, q2, k2, v};
  for (const void* p : ins)
    if (!aligned(p, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(out, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  // every (b, h) slice and every work index must fit the 32-bit index math
  if ((long long)B * H > 0x7fffffffLL || (long long)T * 2 * D > 0x7fffffffLL)
    return DIFFATTN_ERR_UNSUPPORTED;
  const size_t es = elem_bytes(dtype);
  const size_t nqk = (size_t)B * H * T * D * es;
  const size_t nv = 2 * nqk;
  const size_t sizes[5] = {nqk, nqk, nqk, nqk, nv};
  for (int i = 0; i < 5; ++i)
    if (overlaps(out, nv, ins[i], sizes[i])) return DIFFATTN_ERR_INVALID;
  a.q1 = q1;
  a.k1 = k1;
  a.q2 = q2;
  a.k2 = k2;
  a.v = v;
  a.lam = nullptr;
  for (int i = 0; i < 4; ++i) a.lvec[i] = nullptr;
  a.Dl = 0;
  a.lam_init = 0.0f;
  a.lam_out = nullptr;
  a.out = out;
  a.B = B;
  a.H = H;
  a.T = T;
  a.score_scale = (float)(1.4426950408889634 / sqrt((double)D));
  out_bytes = nv;
  return DIFFATTN_OK;
}

}  // namespace

diffattn_status diffattn_fwd(int dtype, int B, int H, int T, int D, const void* q1,
                             const void* k1, const void* q2, const void* k2, const void* v,
                             const float* lambda, int causal, int headnorm, float lambda_init,
                             float eps, void* out, hipStream_t stream) {
  diffattn::FwdArgs a;
  size_t nout = 0;
  const diffattn_status st = check_fwd(dtype, B, H, T, D, q1, k1, q2, k2, v, headnorm, eps, out, a, nout);
  if (st != DIFFATTN_OK) return st;
  if (!lambda) return DIFFATTN_ERR_INVALID;
  if (!aligned(lambda, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  if (overlaps(out, nout, lambda, (size_t)H * sizeof(float))) return DIFFATTN_ERR_INVALID;
  a.lam = lambda;
  a.out_scale = 1.0f - lambda_init;
  a.eps = eps;
  return from_hip(diffattn::launch_fwd(a, dtype, D, causal != 0, headnorm != 0, stream));
}

diffattn_status diffattn_fwd_reparam(int dtype, int B, int H, int T, int D, const void* q1,
                                     const void* k1, const void* q2, const void* k2,
                                     const void* v, const float* lq1, const float* lk1,
                                     const float* lq2, const float* lk2, int Dl, int causal,
                                     int headnorm, float lambda_init, float eps,
                                     float* lambda_out, void* out, hipStream_t stream) {
  diffattn::FwdArgs a;
  size_t nout = 0;
  const diffattn_status st = check_fwd(dtype, B, H, T, D, q1, k1, q2, k2, v, headnorm, eps, out, a, nout);
  if (st != DIFFATTN_OK) return st;
  if (!lq1 || !lk1 || !lq2 || !lk2 || Dl < 1) return DIFFATTN_ERR_INVALID;
  const float* vecs[4] = {lq1, lk1, lq2, lk2};
  for (const float* p : vecs)
    if (!aligned(p, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  if (lambda_out && !aligned(lambda_out, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  const size_t nvec = (size_t)H * Dl * sizeof(float), nlam = (size_t)H * sizeof(float);
  for (const float* p : vecs) {
    if (overlaps(out, nout, p, nvec)) return DIFFATTN_ERR_INVALID;
    if (lambda_out && overlaps(lambda_out, nlam, p, nvec)) return DIFFATTN_ERR_INVALID;
  }
  if (lambda_out) {
    if (overlaps(lambda_out, nlam, out, nout)) return DIFFATTN_ERR_INVALID;
    const void* ins[5] = {q1, k1, q2, k2, v};
    const size_t nqk = nout / 2;
    const size_t sizes[5] = {nqk, nqk, nqk, nqk, nout};
    for (int i = 0; i < 5; ++i)
      if (overlaps(lambda_out, nlam, ins[i], sizes[i])) return DIFFATTN_ERR_INVALID;
  }
  for (int i = 0; i < 4; ++i) a.lvec[i] = vecs[i];
  a.Dl = Dl;
  a.lam_init = lambda_init;
  a.lam_out = lambda_out;
  a.out_scale = 1.0f - lambda_init;
  a.eps = eps;
  return from_hip(diffattn::launch_fwd(a, dtype, D, causal != 0, headnorm != 0, stream));
}

diffattn_status diffattn_attention_fwd(int dtype, int B, int H, int T, int D, const void* q,
                                       const void* k, const void* v, int causal, void* out,
                                       hipStream_t stream) {
  if (!q || !k || !v || !out) return DIFFATTN_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1) return DIFFATTN_ERR_INVALID;
  if (dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return DIFFATTN_ERR_UNSUPPORTED;
  const void* ins[3] = {q, k, v};
  for (const void* p : ins)
    if (!aligned(p, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(out, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  if ((long long)B * H > 0x7fffffffLL || (long long)T * D > 0x7fffffffLL) return DIFFATTN_ERR_UNSUPPORTED;
  const size_t n = (size_t)B * H * T * D * elem_bytes(dtype);
  for (const void* p : ins)
    if (overlaps(out, n, p, n)) return DIFFATTN_ERR_INVALID;
  diffattn::FwdArgs a;
  a.q1 = q;
  a.k1 = k;
  a.q2 = nullptr;
  a.k2 = nullptr;
  a.v = v;
  a.lam = nullptr;
  for (int i = 0; i < 4; ++i) a.lvec[i] = nullptr;
  a.Dl = 0;
  a.lam_init = 0.0f;
  a.lam_out = nullptr;
  a.out = out;
  a.B = B;
  a.H = H;
  a.T = T;
  a.score_scale = (float)(1.4426950408889634 / sqrt((double)D));
  a.out_scale = 1.0f;
  a.eps = 1.0f;
  return from_hip(diffattn::launch_attention(a, D, causal != 0, stream));
}

int diffattn_decode_default_splits(int B, int H, int L) {
  if (B < 1 || H < 1 || L < 1) return 0;
  // aim for ~4096 workgroups in flight, chunks of at least 256 keys
  const long long bh = (long long)B * H;
  long long s = (4096 + bh - 1) / bh;
  const long long smax = L / 256 > 1 ? L / 256 : 1;
  if (s > smax) s = smax;
  if (s < 1) s = 1;
  return (int)s;
}

size_t diffattn_decode_workspace_bytes(int B, int H, int L, int D, int num_splits) {
  if (B < 1 || H < 1 || L < 1 || D < 1 || num_splits < 0 || num_splits > L) return 0;
  const int s = num_splits ? num_splits : diffattn_decode_default_splits(B, H, L);
  return (size_t)B * H * s * 2 * (2 * (size_t)D + 2) * sizeof(float);
}

diffattn_status diffattn_decode(int dtype, int B, int H, int L, int D, const void* q1,
                                const void* k1, const void* q2, const void* k2, const void* v,
                                const float* lambda, int headnorm, float lambda_init, float eps,
                                int num_splits, void* workspace, size_t workspace_bytes,
                                void* out, hipStream_t stream) {
  if (!q1 || !k1 || !q2 || !k2 || !v || !lambda || !out) return DIFFATTN_ERR_INVALID;
  if (B < 1 || H < 1 || L < 1) return DIFFATTN_ERR_INVALID;
  if (headnorm && !(eps > 0.0f)) return DIFFATTN_ERR_INVALID;
  if (num_splits < 0 || num_splits > L) return DIFFATTN_ERR_INVALID;
  if (dtype != DIFFATTN_F32 && dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
  if (!supported_d(D)) return DIFFATTN_ERR_UNSUPPORTED;
  const void* ins[5] = {q1, k1, q2, k2, v};
  for (const void* p : ins)
    if (!aligned(p, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(out, 16) || !aligned(lambda, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  const int S = num_splits ? num_splits : diffattn_decode_default_splits(B, H, L);
  if ((long long)B * H * S > 0x7fffffffLL || (long long)L * 2 * D > 0x7fffffffLL)
    return DIFFATTN_ERR_UNSUPPORTED;
  const size_t need = diffattn_decode_workspace_bytes(B, H, L, D, S);
  if (!workspace || workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  const size_t es = elem_bytes(dtype);
  const size_t nq = (size_t)B * H * D * es;
  const size_t nk = (size_t)B * H * L * D * es;
  const size_t sizes[5] = {nq, nk, nq, nk, 2 * nk};
  const size_t nout = 2 * nq;
  for (int i = 0; i < 5; ++i) {
    if (overlaps(out, nout, ins[i], sizes[i])) return DIFFATTN_ERR_INVALID;
    if (overlaps(workspace, need, ins[i], sizes[i])) return DIFFATTN_ERR_INVALID;
  }
  if (overlaps(out, nout, workspace, need) || overlaps(out, nout, lambda, (size_t)H * 4) ||
      overlaps(workspace, need, lambda, (size_t)H * 4))
    return DIFFATTN_ERR_INVALID;

  diffattn::DecodeArgs a;
  a.q1 = q1;
  a.k1 = k1;
  a.q2 = q2;
  a.k2 = k2;
  a.v = v;
  a.lam = lambda;
  a.ws = (float*)workspace;
  a.out = out;
  a.B = B;
  a.H = H;
  a.L = L;
  a.S = S;
  a.score_scale = (float)(1.4426950408889634 / sqrt((double)D));
  a.out_scale = 1.0f - lambda_init;
  a.eps = eps;
  return from_hip(diffattn::launch_decode(a, dtype, D, headnorm != 0, stream));
}

}  // extern "C"
