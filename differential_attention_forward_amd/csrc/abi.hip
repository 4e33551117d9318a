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

struct Span {
  const void* p;
  size_t n;
};

// every span in outs must be disjoint from every span in ins and from the
// other outs (null entries are skipped)
bool disjoint(const Span* ins, int nin, const Span* outs, int nout) {
  for (int i = 0; i < nout; ++i) {
    if (!outs[i].p) continue;
    for (int j = 0; j < nin; ++j)
      if (ins[j].p && overlaps(outs[i].p, outs[i].n, ins[j].p, ins[j].n)) return false;
    for (int j = i + 1; j < nout; ++j)
      if (outs[j].p && overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return false;
  }
  return true;
}

}  // namespace

extern "C" {

const char* diffattn_status_string(int status) {
  switch (status) {
    case DIFFATTN_OK: return "ok";
    case DIFFATTN_ERR_INVALID: return "invalid argument";
    case DIFFATTN_ERR_UNSUPPORTED: return "unsupported dtype, head width, alignment or size";
    case DIFFATTN_ERR_WORKSPACE: return "workspace or saved-state buffer missing or too small";
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
  if (!diffattn::grid_fits(H, 64)) return DIFFATTN_ERR_UNSUPPORTED;  // one 64-thread workgroup per head
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
  // every (b, h) slice and every work index must fit the 32-bit index math,
  // and the launch grid what one dispatch can express
  if ((long long)B * H > 0x7fffffffLL || (long long)T * 2 * D > 0x7fffffffLL ||
      !diffattn::row_grid_fits(B, H, T))
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
  a.save_o1 = nullptr;
  a.save_o2 = nullptr;
  a.save_lse = nullptr;
  a.B = B;
  a.H = H;
  a.Hkv = H;
  a.window = 0;
  a.T = T;
  a.score_scale = (float)(1.4426950408889634 / sqrt((double)D));
  diffattn::dense_strides(a, H, H, T, D, 2 * D);
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

diffattn_status diffattn_fwd_window(int dtype, int B, int H, int T, int D, const void* q1,
                                    const void* k1, const void* q2, const void* k2, const void* v,
                                    const float* lambda, int window, int headnorm, float lambda_init,
                                    float eps, void* out, hipStream_t stream) {
  diffattn::FwdArgs a;
  size_t nout = 0;
  const diffattn_status st = check_fwd(dtype, B, H, T, D, q1, k1, q2, k2, v, headnorm, eps, out, a, nout);
  if (st != DIFFATTN_OK) return st;
  if (!lambda || window < 1) return DIFFATTN_ERR_INVALID;
  if (dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(lambda, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  if (overlaps(out, nout, lambda, (size_t)H * sizeof(float))) return DIFFATTN_ERR_INVALID;
  a.lam = lambda;
  a.window = window < T ? window : 0;  // a window covering every key is the causal mask
  a.out_scale = 1.0f - lambda_init;
  a.eps = eps;
  return from_hip(diffattn::launch_fwd(a, dtype, D, true, headnorm != 0, stream));
}

namespace {

// Byte span [lo, hi) touched by a [B, H, T, width] tensor with element
// strides sb, sh, sr (all >= 0) and 2-byte elements.
Span strided_span(const void* p, int B, int H, int T, const long long* st, int width) {
  const long long last = (long long)(B - 1) * st[0] + (long long)(H - 1) * st[1] + (long long)(T - 1) * st[2];
  return {p, (size_t)(last + width) * 2};
}

// Whether distinct (b, h, t) rows of a [B, H, T, width] tensor with strides
// st = (sb, sh, sr) never share an element: ordered by stride, every extent
// must fit inside the next stride.
bool rows_disjoint(int B, int H, int T, const long long* st, int width) {
  long long s[3] = {st[0], st[1], st[2]};
  long long n[3] = {B, H, T};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (s[j] < s[i] || (s[j] == s[i] && n[j] < n[i])) {
        long long t = s[i]; s[i] = s[j]; s[j] = t;
        t = n[i]; n[i] = n[j]; n[j] = t;
      }
  long long extent = width;  // elements covered by one row
  for (int i = 0; i < 3; ++i) {
    if (n[i] == 1) continue;
    if (s[i] < extent) return false;
    extent = s[i] * (n[i] - 1) + extent;
  }
  return true;
}

}  // namespace

diffattn_status diffattn_fwd_strided(int dtype, int B, int H, int T, int D, const void* q1,
                                     const void* k1, const void* q2, const void* k2, const void* v,
                                     const long long* strides, const float* lambda, int causal,
                                     int headnorm, float lambda_init, float eps, void* out,
                                     hipStream_t stream) {
  if (!q1 || !k1 || !q2 || !k2 || !v || !out || !strides || !lambda) return DIFFATTN_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1) return DIFFATTN_ERR_INVALID;
  if (headnorm && !(eps > 0.0f)) return DIFFATTN_ERR_INVALID;
  for (int i = 0; i < 18; ++i)
    if (strides[i] < 0) return DIFFATTN_ERR_INVALID;
  if (dtype != DIFFATTN_BF16 || !supported_d(D)) return DIFFATTN_ERR_UNSUPPORTED;
  const void* ptr[6] = {q1, k1, q2, k2, v, out};
  const int width[6] = {D, D, D, D, 2 * D, 2 * D};
  for (int i = 0; i < 6; ++i) {
    if (!aligned(ptr[i], 16)) return DIFFATTN_ERR_UNSUPPORTED;
    // 128-bit row accesses: every stride a multiple of 8 bf16 elements
    for (int j = 0; j < 3; ++j)
      if (strides[3 * i + j] % 8) return DIFFATTN_ERR_UNSUPPORTED;
  }
  if (!aligned(lambda, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  if ((long long)B * H > 0x7fffffffLL || (long long)T * 2 * D > 0x7fffffffLL || !diffattn::row_grid_fits(B, H, T))
    return DIFFATTN_ERR_UNSUPPORTED;
  // K and V rows are fetched at 32-bit byte offsets from their (b, h) slice;
  // query and output row strides are ints
  for (int i = 0; i < 6; ++i) {
    const long long rs = strides[3 * i + 2];
    if (rs > 0x7fffffffLL) return DIFFATTN_ERR_UNSUPPORTED;
    if ((i == 1 || i == 3 || i == 4) && ((long long)(T - 1) * rs + width[i]) * 2 > 0x7fffffffLL)
      return DIFFATTN_ERR_UNSUPPORTED;
  }
  if (!rows_disjoint(B, H, T, strides + 15, 2 * D)) return DIFFATTN_ERR_INVALID;
  Span ins[6];
  for (int i = 0; i < 5; ++i) ins[i] = strided_span(ptr[i], B, H, T, strides + 3 * i, width[i]);
  ins[5] = {lambda, (size_t)H * sizeof(float)};
  const Span outs[1] = {strided_span(out, B, H, T, strides + 15, 2 * D)};
  if (!disjoint(ins, 6, outs, 1)) return DIFFATTN_ERR_INVALID;

  diffattn::FwdArgs a;
  a.q1 = q1;
  a.k1 = k1;
  a.q2 = q2;
  a.k2 = k2;
  a.v = v;
  a.lam = lambda;
  for (int i = 0; i < 4; ++i) a.lvec[i] = nullptr;
  a.Dl = 0;
  a.lam_init = 0.0f;
  a.lam_out = nullptr;
  a.out = out;
  a.save_o1 = nullptr;
  a.save_o2 = nullptr;
  a.save_lse = nullptr;
  a.B = B;
  a.H = H;
  a.Hkv = H;
  a.window = 0;
  a.T = T;
  a.score_scale = (float)(1.4426950408889634 / sqrt((double)D));
  a.out_scale = 1.0f - lambda_init;
  a.eps = eps;
  for (int i = 0; i < 6; ++i) {
    a.sb[i] = strides[3 * i];
    a.sh[i] = strides[3 * i + 1];
    a.sr[i] = (int)strides[3 * i + 2];
  }
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
  if ((long long)B * H > 0x7fffffffLL || (long long)T * D > 0x7fffffffLL || !diffattn::row_grid_fits(B, H, T))
    return DIFFATTN_ERR_UNSUPPORTED;
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
  a.save_o1 = nullptr;
  a.save_o2 = nullptr;
  a.save_lse = nullptr;
  a.B = B;
  a.H = H;
  a.Hkv = H;
  a.window = 0;
  a.T = T;
  a.score_scale = (float)(1.4426950408889634 / sqrt((double)D));
  a.out_scale = 1.0f;
  a.eps = 1.0f;
  diffattn::dense_strides(a, H, H, T, D, D);
  return from_hip(diffattn::launch_attention(a, D, causal != 0, stream));
}

// ---- training: forward that saves what the backward needs, and the backward --

namespace {

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool train_sizes_ok(int B, int H, int T, int D) {
  if (B < 1 || H < 1 || T < 1 || (D != 32 && D != 64 && D != 128)) return false;
  return (long long)B * H <= 0x7fffffffLL && (long long)T * 2 * D <= 0x7fffffffLL &&
         diffattn::row_grid_fits(B, H, T);
}

}  // namespace

size_t diffattn_train_saved_bytes(int B, int H, int T, int D) {
  if (!train_sizes_ok(B, H, T, D)) return 0;
  const size_t bht = (size_t)B * H * T;
  return 2 * bht * 2 * D * sizeof(float) + 2 * bht * sizeof(float);
}

diffattn_status diffattn_fwd_train(int dtype, int B, int H, int T, int D, const void* q1,
                                   const void* k1, const void* q2, const void* k2, const void* v,
                                   const float* lambda, int causal, int headnorm, float lambda_init,
                                   float eps, void* out, void* saved, size_t saved_bytes,
                                   hipStream_t stream) {
  diffattn::FwdArgs a;
  size_t nout = 0;
  const diffattn_status st = check_fwd(dtype, B, H, T, D, q1, k1, q2, k2, v, headnorm, eps, out, a, nout);
  if (st != DIFFATTN_OK) return st;
  if (!lambda || !saved) return DIFFATTN_ERR_INVALID;
  if (dtype != DIFFATTN_BF16 || !train_sizes_ok(B, H, T, D)) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(lambda, 4) || !aligned(saved, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  const size_t need = diffattn_train_saved_bytes(B, H, T, D);
  if (saved_bytes < need) return DIFFATTN_ERR_WORKSPACE;
  const size_t nqk = nout / 2;
  const Span ins[6] = {{q1, nqk}, {k1, nqk}, {q2, nqk}, {k2, nqk}, {v, nout}, {lambda, (size_t)H * 4}};
  const Span outs[2] = {{out, nout}, {saved, need}};
  if (!disjoint(ins, 6, outs, 2)) return DIFFATTN_ERR_INVALID;
  const size_t bht = (size_t)B * H * T;
  a.lam = lambda;
  a.out_scale = 1.0f - lambda_init;
  a.eps = eps;
  a.save_o1 = (float*)saved;
  a.save_o2 = (float*)saved + bht * 2 * D;
  a.save_lse = (float*)saved + 2 * bht * 2 * D;
  return from_hip(diffattn::launch_fwd(a, dtype, D, causal != 0, headnorm != 0, stream));
}

size_t diffattn_bwd_workspace_bytes(int B, int H, int T, int D) {
  if (!train_sizes_ok(B, H, T, D)) return 0;
  const size_t bh = (size_t)B * H;
  const size_t tp = round_up((size_t)T, 64);
  return round_up(bh * T * 2 * D * 2, 256) + round_up(bh * 4 * tp * 4, 256) + bh * (tp / 64) * 4;
}

diffattn_status diffattn_bwd(int dtype, int B, int H, int T, int D, const void* q1, const void* k1,
                             const void* q2, const void* k2, const void* v, const float* lambda,
                             const void* dout, const void* saved, size_t saved_bytes, int causal,
                             int headnorm, float lambda_init, float eps, void* dq1, void* dk1,
                             void* dq2, void* dk2, void* dv, float* dlambda, const float* lq1,
                             const float* lk1, const float* lq2, const float* lk2, int Dl,
                             float* dlq1, float* dlk1, float* dlq2, float* dlk2, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (!q1 || !k1 || !q2 || !k2 || !v || !lambda || !dout || !saved) return DIFFATTN_ERR_INVALID;
  if (!dq1 || !dk1 || !dq2 || !dk2 || !dv || !dlambda) return DIFFATTN_ERR_INVALID;
  if (B < 1 || H < 1 || T < 1) return DIFFATTN_ERR_INVALID;
  if (headnorm && !(eps > 0.0f)) return DIFFATTN_ERR_INVALID;
  const bool vec = lq1 != nullptr;
  const void* vp[8] = {lq1, lk1, lq2, lk2, dlq1, dlk1, dlq2, dlk2};
  for (const void* p : vp)
    if ((p != nullptr) != vec) return DIFFATTN_ERR_INVALID;
  if (vec && Dl < 1) return DIFFATTN_ERR_INVALID;
  if (dtype != DIFFATTN_BF16 || !train_sizes_ok(B, H, T, D)) return DIFFATTN_ERR_UNSUPPORTED;
  const void* t16[13] = {q1, k1, q2, k2, v, dout, saved, dq1, dk1, dq2, dk2, dv, workspace};
  for (const void* p : t16)
    if (p && !aligned(p, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(lambda, 4) || !aligned(dlambda, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  for (const void* p : vp)
    if (p && !aligned(p, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  const size_t need_saved = diffattn_train_saved_bytes(B, H, T, D);
  const size_t need_ws = diffattn_bwd_workspace_bytes(B, H, T, D);
  if (saved_bytes < need_saved || !workspace || workspace_bytes < need_ws) return DIFFATTN_ERR_WORKSPACE;
  const size_t nqk = (size_t)B * H * T * D * 2, nv = 2 * nqk, nl = (size_t)H * 4;
  const size_t nvec = vec ? (size_t)H * Dl * 4 : 0;
  const Span ins[11] = {{q1, nqk}, {k1, nqk}, {q2, nqk}, {k2, nqk}, {v, nv}, {dout, nv},
                        {saved, need_saved}, {lambda, nl}, {lq1, nvec}, {lk1, nvec}, {lq2, nvec}};
  const Span ins2[1] = {{lk2, nvec}};
  const Span outs[11] = {{dq1, nqk}, {dk1, nqk}, {dq2, nqk}, {dk2, nqk}, {dv, nv}, {dlambda, nl},
                         {dlq1, nvec}, {dlk1, nvec}, {dlq2, nvec}, {dlk2, nvec}, {workspace, need_ws}};
  if (!disjoint(ins, 11, outs, 11) || !disjoint(ins2, 1, outs, 11)) return DIFFATTN_ERR_INVALID;

  diffattn::BwdArgs a;
  const size_t bh = (size_t)B * H, bht = bh * T;
  const int Tp = (int)round_up((size_t)T, 64);
  a.q1 = q1;
  a.k1 = k1;
  a.q2 = q2;
  a.k2 = k2;
  a.v = v;
  a.dout = dout;
  a.o1 = (const float*)saved;
  a.o2 = (const float*)saved + bht * 2 * D;
  a.lse = (const float*)saved + 2 * bht * 2 * D;
  a.lam = lambda;
  char* ws = (char*)workspace;
  a.dopre = ws;
  a.stats = (float*)(ws + round_up(bht * 2 * D * 2, 256));
  a.dlam_part = (float*)(ws + round_up(bht * 2 * D * 2, 256) + round_up(bh * 4 * Tp * 4, 256));
  a.dq1 = dq1;
  a.dk1 = dk1;
  a.dq2 = dq2;
  a.dk2 = dk2;
  a.dv = dv;
  a.dlam = dlambda;
  const float* lv[4] = {lq1, lk1, lq2, lk2};
  float* dlv[4] = {dlq1, dlk1, dlq2, dlk2};
  for (int i = 0; i < 4; ++i) {
    a.lvec[i] = lv[i];
    a.dlvec[i] = dlv[i];
  }
  a.Dl = vec ? Dl : 0;
  a.B = B;
  a.H = H;
  a.T = T;
  a.Tp = Tp;
  a.nchunk = Tp / 64;
  a.score_scale = (float)(1.4426950408889634 / sqrt((double)D));
  a.grad_scale = (float)(1.0 / sqrt((double)D));
  a.out_scale = 1.0f - lambda_init;
  a.eps = eps;
  return from_hip(diffattn::launch_bwd(a, D, causal != 0, headnorm != 0, stream));
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

namespace {

diffattn_status decode_impl(int dtype, int B, int H, int L, int D, const void* q1, const void* k1,
                            const void* q2, const void* k2, const void* v, const float* lambda,
                            const int* lengths, int headnorm, float lambda_init, float eps,
                            int num_splits, void* workspace, size_t workspace_bytes, void* out,
                            hipStream_t stream, bool lib_scratch = false) {
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
  // split-K grid of B H S workgroups, reduce grid of B H
  if (!diffattn::grid_fits((long long)B * H * S, diffattn::kDecodeThreads) ||
      !diffattn::grid_fits((long long)B * H, 256) || (long long)L * 2 * D > 0x7fffffffLL)
    return DIFFATTN_ERR_UNSUPPORTED;
  const size_t need = diffattn_decode_workspace_bytes(B, H, L, D, S);
  if (lib_scratch) {
    // the library's own array of the current device instead of a caller's
    if (need > DIFFATTN_NOALLOC_SCRATCH_BYTES) return DIFFATTN_ERR_WORKSPACE;
    if (diffattn::decode_scratch(&workspace) != hipSuccess) return DIFFATTN_ERR_HIP;
    workspace_bytes = DIFFATTN_NOALLOC_SCRATCH_BYTES;
  }
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
  if (lengths) {
    if (!aligned(lengths, 4)) return DIFFATTN_ERR_UNSUPPORTED;
    const size_t nl = (size_t)B * sizeof(int);
    if (overlaps(out, nout, lengths, nl) || overlaps(workspace, need, lengths, nl))
      return DIFFATTN_ERR_INVALID;
  }

  diffattn::DecodeArgs a;
  a.lens = lengths;
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
  a.Hkv = H;
  a.score_scale = (float)(1.4426950408889634 / sqrt((double)D));
  a.out_scale = 1.0f - lambda_init;
  a.eps = eps;
  return from_hip(diffattn::launch_decode(a, dtype, D, headnorm != 0, stream));
}

}  // namespace

diffattn_status diffattn_decode(int dtype, int B, int H, int L, int D, const void* q1,
                                const void* k1, const void* q2, const void* k2, const void* v,
                                const float* lambda, int headnorm, float lambda_init, float eps,
                                int num_splits, void* workspace, size_t workspace_bytes,
                                void* out, hipStream_t stream) {
  return decode_impl(dtype, B, H, L, D, q1, k1, q2, k2, v, lambda, nullptr, headnorm, lambda_init,
                     eps, num_splits, workspace, workspace_bytes, out, stream);
}

diffattn_status diffattn_decode_ragged(int dtype, int B, int H, int L, int D, const void* q1,
                                       const void* k1, const void* q2, const void* k2,
                                       const void* v, const float* lambda, const int* lengths,
                                       int headnorm, float lambda_init, float eps, int num_splits,
                                       void* workspace, size_t workspace_bytes, void* out,
                                       hipStream_t stream) {
  if (!lengths) return DIFFATTN_ERR_INVALID;
  return decode_impl(dtype, B, H, L, D, q1, k1, q2, k2, v, lambda, lengths, headnorm, lambda_init,
                     eps, num_splits, workspace, workspace_bytes, out, stream);
}

diffattn_status diffattn_decode_noalloc(int dtype, int B, int H, int L, int D, const void* q1,
                                        const void* k1, const void* q2, const void* k2,
                                        const void* v, const float* lambda, int headnorm,
                                        float lambda_init, float eps, int num_splits, void* out,
                                        hipStream_t stream) {
  return decode_impl(dtype, B, H, L, D, q1, k1, q2, k2, v, lambda, nullptr, headnorm, lambda_init,
                     eps, num_splits, nullptr, 0, out, stream, true);
}

// ---- DIFF V2: two query heads per differential head, K/V shared per group ----

diffattn_status diffattn_v2_fwd(int dtype, int B, int H, int Hkv, int T, int D, const void* q1,
                                const void* q2, const void* k, const void* v, const float* lambda,
                                int causal, void* out, hipStream_t stream) {
  if (!q1 || !q2 || !k || !v || !lambda || !out) return DIFFATTN_ERR_INVALID;
  if (B < 1 || H < 1 || Hkv < 1 || T < 1 || H % Hkv) return DIFFATTN_ERR_INVALID;
  if (dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return DIFFATTN_ERR_UNSUPPORTED;
  const void* ins[4] = {q1, q2, k, v};
  for (const void* p : ins)
    if (!aligned(p, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(out, 16) || !aligned(lambda, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  if ((long long)B * H > 0x7fffffffLL || (long long)T * D > 0x7fffffffLL || !diffattn::row_grid_fits(B, H, T))
    return DIFFATTN_ERR_UNSUPPORTED;
  const size_t nq = (size_t)B * H * T * D * 2, nkv = (size_t)B * Hkv * T * D * 2;
  const size_t sizes[4] = {nq, nq, nkv, nkv};
  for (int i = 0; i < 4; ++i)
    if (overlaps(out, nq, ins[i], sizes[i])) return DIFFATTN_ERR_INVALID;
  if (overlaps(out, nq, lambda, (size_t)H * 4)) return DIFFATTN_ERR_INVALID;
  diffattn::FwdArgs a;
  a.q1 = q1;
  a.k1 = k;
  a.q2 = q2;
  a.k2 = k;
  a.v = v;
  a.lam = lambda;
  for (int i = 0; i < 4; ++i) a.lvec[i] = nullptr;
  a.Dl = 0;
  a.lam_init = 0.0f;
  a.lam_out = nullptr;
  a.out = out;
  a.save_o1 = nullptr;
  a.save_o2 = nullptr;
  a.save_lse = nullptr;
  a.B = B;
  a.H = H;
  a.T = T;
  a.Hkv = Hkv;
  a.window = 0;
  a.score_scale = (float)(1.4426950408889634 / sqrt((double)D));
  a.out_scale = 1.0f;
  a.eps = 1.0f;
  diffattn::dense_strides(a, H, Hkv, T, D, D);
  return from_hip(diffattn::launch_v2(a, D, causal != 0, stream));
}

size_t diffattn_v2_decode_workspace_bytes(int B, int H, int Hkv, int L, int D, int num_splits) {
  if (B < 1 || H < 1 || Hkv < 1 || L < 1 || D < 1 || num_splits < 0 || num_splits > L) return 0;
  const int s = num_splits ? num_splits : diffattn_decode_default_splits(B, Hkv, L);
  return (size_t)B * H * s * 2 * ((size_t)D + 2) * sizeof(float);
}

diffattn_status diffattn_v2_decode(int dtype, int B, int H, int Hkv, int L, int D, const void* q1,
                                   const void* q2, const void* k, const void* v, const float* lambda,
                                   int num_splits, void* workspace, size_t workspace_bytes, void* out,
                                   hipStream_t stream) {
  if (!q1 || !q2 || !k || !v || !lambda || !out) return DIFFATTN_ERR_INVALID;
  if (B < 1 || H < 1 || Hkv < 1 || L < 1 || H % Hkv) return DIFFATTN_ERR_INVALID;
  if (num_splits < 0 || num_splits > L) return DIFFATTN_ERR_INVALID;
  if (dtype != DIFFATTN_BF16) return DIFFATTN_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return DIFFATTN_ERR_UNSUPPORTED;
  const int grp = H / Hkv;
  if (grp != 1 && grp != 2 && grp != 4) return DIFFATTN_ERR_UNSUPPORTED;
  const void* ins[4] = {q1, q2, k, v};
  for (const void* p : ins)
    if (!aligned(p, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  if (!aligned(out, 16) || !aligned(lambda, 4)) return DIFFATTN_ERR_UNSUPPORTED;
  const int S = num_splits ? num_splits : diffattn_decode_default_splits(B, Hkv, L);
  if (!diffattn::grid_fits((long long)B * Hkv * S, diffattn::kDecodeThreads) ||
      !diffattn::grid_fits((long long)B * H, 256) || (long long)B * H * S > 0x7fffffffLL ||
      (long long)L * D > 0x7fffffffLL)
    return DIFFATTN_ERR_UNSUPPORTED;
  const size_t need = diffattn_v2_decode_workspace_bytes(B, H, Hkv, L, D, S);
  if (!workspace || workspace_bytes < need) return DIFFATTN_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return DIFFATTN_ERR_UNSUPPORTED;
  const size_t nq = (size_t)B * H * D * 2, nkv = (size_t)B * Hkv * L * D * 2;
  const size_t sizes[4] = {nq, nq, nkv, nkv};
  for (int i = 0; i < 4; ++i) {
    if (overlaps(out, nq, ins[i], sizes[i])) return DIFFATTN_ERR_INVALID;
    if (overlaps(workspace, need, ins[i], sizes[i])) return DIFFATTN_ERR_INVALID;
  }
  if (overlaps(out, nq, workspace, need) || overlaps(out, nq, lambda, (size_t)H * 4) ||
      overlaps(workspace, need, lambda, (size_t)H * 4))
    return DIFFATTN_ERR_INVALID;
  diffattn::DecodeArgs a;
  a.lens = nullptr;
  a.q1 = q1;
  a.k1 = k;
  a.q2 = q2;
  a.k2 = k;
  a.v = v;
  a.lam = lambda;
  a.ws = (float*)workspace;
  a.out = out;
  a.B = B;
  a.H = H;
  a.L = L;
  a.S = S;
  a.Hkv = Hkv;
  a.score_scale = (float)(1.4426950408889634 / sqrt((double)D));
  a.out_scale = 1.0f;
  a.eps = 1.0f;
  return from_hip(diffattn::launch_decode_v2(a, D, stream));
}

}  // extern "C"
