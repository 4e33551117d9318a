// Differential-attention prefill forward for gfx950 (CDNA4).
//
// Computes, per (batch, head),
//   O = (softmax(Q1 K1^T / sqrt(D) + M) - lam_h softmax(Q2 K2^T / sqrt(D) + M)) V
// (paperleet "Differential Transformer Attention", equation for A1, A2, O; the
// causal mask M is -inf on future keys in both branches), optionally followed
// by an RMS norm over the 2D output channels of each token and a constant
// x (1 - lambda_init) (aifetchly "Differential Transformer: Canceling LLM
// Attention Noise", section 4).
//
// Design (one pass over K/V, both maps at once):
//  * One workgroup = NW waves = BR query rows of one (b, h); each wave owns
//    32*NQB queries.  Q1/Q2 fragments stay in VGPRs for the whole kernel.
//  * K1, K2 and V tiles of BC keys are staged global -> VGPR -> LDS, double
//    buffered: the global loads of tile t+1 are in flight while tile t is
//    computed, one barrier per tile.  V is written to LDS transposed
//    ([channel][key]) so that it can be the A operand of the P.V MFMA.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: lane l then holds 16 keys of query l%32, so the
//    row max is an in-lane reduction plus one exchange with lane l^32, and
//    the probabilities P^T land in exactly the register layout the P.V MFMA
//    wants as its B operand (no data movement).
//  * Two independent online-softmax states per query row (one per map) with
//    lazy rescaling: the running max only moves (and the accumulators are
//    only rescaled) when a block max exceeds it by more than kTau (log2
//    units), so steady-state blocks do no rescale work.
//  * The row sums are taken over the bf16-rounded probabilities actually fed
//    to the MFMA (v_dot2_f32_bf16 against 1.0), so a value offset shared by
//    all keys passes through with weights that sum exactly to one.
//  * Both P1.V and P2.V are fed from one V tile in LDS: each V fragment read
//    serves both branches (V is read from memory once, not once per map).
//  * Causal: key blocks above a wave's last query are skipped; only blocks
//    that straddle the diagonal evaluate the mask.  Query tiles are issued
//    heaviest first and workgroups are remapped so that each XCD works
//    through consecutive tiles of the same heads (K/V reuse in its L2).
//  * fp32 inputs use the same structure with v_mfma_f32_32x32x2_f32 and
//    fp32 probabilities (V kept row-major in LDS).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace diffattn {
namespace {

constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units): p <= 2^8

template <int D, int NQB, int NW, int BC, bool F32, bool SPLIT>
struct Cfg {
  static constexpr int DV = 2 * D;
  static constexpr int QPW = 32 * NQB;
  static constexpr int NBR = SPLIT ? 1 : 2;         // maps handled by one wave
  static constexpr int NWQ = SPLIT ? NW / 2 : NW;   // waves per map
  static constexpr int BR = NWQ * QPW;              // query rows per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int ES = F32 ? 4 : 2;
  static constexpr int EPC = 16 / ES;               // elements per 16-byte chunk
  static constexpr int KP = F32 ? D + 4 : D + 8;    // K row pitch (elements)
  // V in LDS: fp32 row-major [BC][DV]; bf16 transposed [DV][BC]
  static constexpr int VP = F32 ? DV + 4 : BC + 8;
  static constexpr int KTILE = BC * KP;
  static constexpr int VTILE = F32 ? BC * VP : DV * VP;
  static constexpr int STAGE = 2 * KTILE + VTILE;   // elements per LDS stage
  static constexpr int NKC = BC * D / EPC;          // 16-B chunks per K tile
  static constexpr int NKPT = (NKC + NT - 1) / NT;
  // V staging units: fp32 plain 16-B chunks; bf16 blocks of 4 keys x 8 channels
  static constexpr int NVU = F32 ? BC * DV / EPC : (BC / 4) * (DV / 8);
  static constexpr int NVPT = (NVU + NT - 1) / NT;
  static constexpr int VREG = F32 ? 1 : 4;
  static constexpr int NKB = BC / 32;               // 32-key blocks per tile
  static constexpr int CB = DV / 32;                // 32-channel output blocks
  static constexpr int KSTEPS = F32 ? D / 2 : D / 16;
  // split mode: map-2 waves hand acc2/l2 to their map-1 partners through LDS
  static constexpr int XP = DV + 4;                 // exchange row pitch (floats)
  static constexpr int XBYTES = SPLIT ? NWQ * QPW * XP * 4 : 0;
  static constexpr int RBYTES = 2 * STAGE * ES;
  static constexpr int SMEM = RBYTES > XBYTES ? RBYTES : XBYTES;
  static_assert(BC % 32 == 0, "key tile must hold whole 32-key blocks");
  static_assert(!SPLIT || NW % 2 == 0, "split mode pairs waves");
  static_assert(SMEM <= 160 * 1024, "LDS budget exceeded");
};

// Position of key quad kq inside the transposed V row: within every group of
// 4 quads (16 keys) the middle two are swapped, which is the key order in
// which one lane's 8 probabilities reach the MFMA (keys 0-3 and 8-11 in the
// lower lane half, 4-7 and 12-15 in the upper half).
__device__ inline int vt_quad_pos(int kq) { return kq ^ ((((kq >> 1) ^ kq) & 1) * 3); }

template <bool F32>
using QFrag = typename std::conditional<F32, float, bf16x8>::type;
template <bool F32>
using Elem = typename std::conditional<F32, float, bf16>::type;

template <int D, int NQB, int NW, int BC, bool F32, bool SPLIT, bool CAUSAL, bool HEADNORM>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW >= 8 ? 2 : 1, NW >= 8 ? 2 : 1))) void fwd_kernel(FwdArgs a) {
  using C = Cfg<D, NQB, NW, BC, F32, SPLIT>;
  using E = Elem<F32>;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::SMEM];
  E* const smem = (E*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int T = a.T;

  const int nqt = (T + C::BR - 1) / C::BR;
  const int w = xcd_remap(blockIdx.x, a.B * a.H * nqt);
  const int bh = w / nqt;
  const int qi = w % nqt;
  const int qt = CAUSAL ? (nqt - 1 - qi) : qi;  // heaviest causal tiles first
  const int h = bh % a.H;

  const size_t qk_off = (size_t)bh * T * D;
  const size_t v_off = (size_t)bh * T * C::DV;
  const E* __restrict__ Q1 = (const E*)a.q1 + qk_off;
  const E* __restrict__ Q2 = (const E*)a.q2 + qk_off;
  const E* __restrict__ K1 = (const E*)a.k1 + qk_off;
  const E* __restrict__ K2 = (const E*)a.k2 + qk_off;
  const E* __restrict__ V = (const E*)a.v + v_off;

  // split mode: waves [0, NWQ) run map 1 and [NWQ, 2 NWQ) map 2 on the same rows
  const int wbr = SPLIT ? wave / C::NWQ : 0;
  const int wq = SPLIT ? wave % C::NWQ : wave;
  const int q_tile0 = qt * C::BR;
  const int q0 = q_tile0 + wq * C::QPW;
  const int q_last = min(q0 + C::QPW, T) - 1;
  const bool wave_active = q0 < T;
  const int k_end = CAUSAL ? min(T, q_tile0 + C::BR) : T;
  const int ntiles = (k_end + BC - 1) / BC;
  const float sc = a.score_scale;
  const float lamv = a.lam[h];

  // ---- Q fragments (B operand of S^T = K Q^T) -------------------------------
  QFrag<F32> qf[C::NBR][NQB][C::KSTEPS];
#pragma unroll
  for (int br = 0; br < C::NBR; ++br) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // rows past the end read row T-1 (always in bounds) and are zeroed
      const int query = q0 + qb * 32 + l32;
      const bool ok = query < T;
      const E* src = ((br + wbr) ? Q2 : Q1) + (size_t)min(query, T - 1) * D;
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        if constexpr (F32) {
          const float x = src[2 * ks + hi];
          qf[br][qb][ks] = ok ? x : 0.0f;
        } else {
          u32x4 raw = *(const u32x4*)(src + ks * 16 + hi * 8);
          raw = ok ? raw : u32x4{0u, 0u, 0u, 0u};
          qf[br][qb][ks] = __builtin_bit_cast(bf16x8, raw);
        }
      }
    }
  }

  floatx16 acc[C::NBR][NQB][C::CB];
  float mu[C::NBR][NQB];
  float lsum[C::NBR][NQB];
#pragma unroll
  for (int br = 0; br < C::NBR; ++br)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      mu[br][qb] = kNegInf;
      lsum[br][qb] = 0.0f;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[br][qb][cb][r] = 0.0f;
    }

  // ---- staging registers ------------------------------------------------------
  u32x4 rk[2][C::NKPT];
  u32x4 rv[C::NVPT][C::VREG];
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  // Global -> register staging of one key tile.  Keys past the end load row
  // T-1 (always in bounds) and are replaced by zeros, so there is no branch.
  auto load_tile = [&](int kt) {
    const int kbase = kt * BC;
#pragma unroll
    for (int i = 0; i < C::NKPT; ++i) {
      const int c = (C::NKC % C::NT == 0) ? tid + i * C::NT : min(tid + i * C::NT, C::NKC - 1);
      const int row = c / (D / C::EPC);
      const int col = c % (D / C::EPC);
      const int key = kbase + row;
      const size_t off = (size_t)min(key, T - 1) * D + col * C::EPC;
      const u32x4 x1 = *(const u32x4*)(K1 + off);
      const u32x4 x2 = *(const u32x4*)(K2 + off);
      rk[0][i] = key < T ? x1 : zero4;
      rk[1][i] = key < T ? x2 : zero4;
    }
#pragma unroll
    for (int i = 0; i < C::NVPT; ++i) {
      const int u = (C::NVU % C::NT == 0) ? tid + i * C::NT : min(tid + i * C::NT, C::NVU - 1);
      if constexpr (F32) {
        const int row = u / (C::DV / 4);
        const int col = u % (C::DV / 4);
        const int key = kbase + row;
        const u32x4 x = *(const u32x4*)(V + (size_t)min(key, T - 1) * C::DV + col * 4);
        rv[i][0] = key < T ? x : zero4;
      } else {
        const int kq = u % (BC / 4);
        const int cc = u / (BC / 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kbase + kq * 4 + r;
          const u32x4 x = *(const u32x4*)(V + (size_t)min(key, T - 1) * C::DV + cc * 8);
          rv[i][r] = key < T ? x : zero4;
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    E* Ks1 = smem + buf * C::STAGE;
    E* Ks2 = Ks1 + C::KTILE;
    E* Vs = Ks2 + C::KTILE;
#pragma unroll
    for (int i = 0; i < C::NKPT; ++i) {
      const int c = tid + i * C::NT;
      if (C::NKC % C::NT == 0 || c < C::NKC) {
        const int row = c / (D / C::EPC);
        const int col = c % (D / C::EPC);
        *(u32x4*)(Ks1 + row * C::KP + col * C::EPC) = rk[0][i];
        *(u32x4*)(Ks2 + row * C::KP + col * C::EPC) = rk[1][i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::NVPT; ++i) {
      const int u = tid + i * C::NT;
      if (C::NVU % C::NT == 0 || u < C::NVU) {
        if constexpr (F32) {
          const int row = u / (C::DV / 4);
          const int col = u % (C::DV / 4);
          *(u32x4*)(Vs + row * C::VP + col * 4) = rv[i][0];
        } else {
          // 4 keys x 8 channels -> 8 channel rows of 4 keys each
          const int kq = u % (BC / 4);
          const int cc = u / (BC / 4);
          const int pos = vt_quad_pos(kq) * 4;
#pragma unroll
          for (int wd = 0; wd < 4; ++wd) {
            const uint32_t a0 = rv[i][0][wd], a1 = rv[i][1][wd];
            const uint32_t a2 = rv[i][2][wd], a3 = rv[i][3][wd];
            const u32x2 even = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
            const u32x2 odd = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
            *(u32x2*)(Vs + (cc * 8 + 2 * wd) * C::VP + pos) = even;
            *(u32x2*)(Vs + (cc * 8 + 2 * wd + 1) * C::VP + pos) = odd;
          }
        }
      }
    }
  };

  auto compute_tile = [&](int kt, int buf) {
    const E* Ks1 = smem + buf * C::STAGE;
    const E* Ks2 = Ks1 + C::KTILE;
    const E* Vs = Ks2 + C::KTILE;
    const E* Kmap[2] = {SPLIT && wbr ? Ks2 : Ks1, Ks2};  // K tile of each map this wave runs
#pragma unroll
    for (int kb = 0; kb < C::NKB; ++kb) {
      const int key0 = kt * BC + kb * 32;
      if (key0 >= T) break;
      if (CAUSAL && key0 > q_last) break;

      // S^T = K Q^T for the maps this wave runs
      floatx16 s[C::NBR][NQB];
#pragma unroll
      for (int br = 0; br < C::NBR; ++br)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[br][qb][r] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
        for (int br = 0; br < C::NBR; ++br) {
          if constexpr (F32) {
            const float av = Kmap[br][(kb * 32 + l32) * C::KP + 2 * ks + hi];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
              s[br][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, qf[br][qb][ks], s[br][qb], 0, 0, 0);
          } else {
            const bf16x8 av = *(const bf16x8*)(Kmap[br] + (kb * 32 + l32) * C::KP + ks * 16 + hi * 8);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
              s[br][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[br][qb][ks], s[br][qb], 0, 0, 0);
          }
        }
      }

      // mask: causal blocks that reach past the wave's first query, or the
      // ragged end of the key axis for full attention
      const bool need_mask = CAUSAL ? (key0 + 31 > q0) : (key0 + 32 > T);
      if (need_mask) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const int query = q0 + qb * 32 + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool masked = CAUSAL ? (key > query) : (key >= T);
            if (masked) {
#pragma unroll
              for (int br = 0; br < C::NBR; ++br) s[br][qb][r] = kNegInf;
            }
          }
        }
      }

      // online softmax: one independent state per map and query row
      float mx[C::NBR][NQB];
      bool need = false;
#pragma unroll
      for (int br = 0; br < C::NBR; ++br)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          float m = s[br][qb][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) m = fmaxf(m, s[br][qb][r]);
          m = fmaxf(m, __shfl_xor(m, 32));
          m *= sc;
          mx[br][qb] = m;
          need |= m > mu[br][qb] + kTau;
        }
      if (__any(need)) {
#pragma unroll
        for (int br = 0; br < C::NBR; ++br)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const float mn = fmaxf(mu[br][qb], mx[br][qb]);
            const float alpha = (mn == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f(mu[br][qb] - mn);
            mu[br][qb] = mn;
            lsum[br][qb] *= alpha;
#pragma unroll
            for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
              for (int r = 0; r < 16; ++r) acc[br][qb][cb][r] *= alpha;
          }
      }

      if constexpr (F32) {
        float p[C::NBR][NQB][16];
#pragma unroll
        for (int br = 0; br < C::NBR; ++br)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const float msub = mu[br][qb] == kNegInf ? 0.0f : mu[br][qb];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              p[br][qb][r] = __builtin_amdgcn_exp2f(fmaf(s[br][qb][r], sc, -msub));
              lsum[br][qb] += p[br][qb][r];
            }
          }
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int krow = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const float av = Vs[krow * C::VP + cb * 32 + l32];
#pragma unroll
            for (int br = 0; br < C::NBR; ++br)
#pragma unroll
              for (int qb = 0; qb < NQB; ++qb)
                acc[br][qb][cb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, p[br][qb][r], acc[br][qb][cb], 0, 0, 0);
          }
      } else {
        bf16x8 pk[C::NBR][NQB][2];
        const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
        for (int br = 0; br < C::NBR; ++br)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) {
            const float msub = mu[br][qb] == kNegInf ? 0.0f : mu[br][qb];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float pa = __builtin_amdgcn_exp2f(fmaf(s[br][qb][8 * ks + 2 * j], sc, -msub));
                const float pb = __builtin_amdgcn_exp2f(fmaf(s[br][qb][8 * ks + 2 * j + 1], sc, -msub));
                const bf16x2 pw = {(bf16)pa, (bf16)pb};
                lsum[br][qb] = __builtin_amdgcn_fdot2_f32_bf16(pw, ones, lsum[br][qb], false);
                pk[br][qb][ks][2 * j] = pw[0];
                pk[br][qb][ks][2 * j + 1] = pw[1];
              }
            }
          }
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 av = *(const bf16x8*)(Vs + (cb * 32 + l32) * C::VP + kb * 32 + ks * 16 + hi * 8);
#pragma unroll
            for (int br = 0; br < C::NBR; ++br)
#pragma unroll
              for (int qb = 0; qb < NQB; ++qb)
                acc[br][qb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pk[br][qb][ks], acc[br][qb][cb], 0, 0, 0);
          }
      }
    }
  };

  // ---- main loop over key tiles ----------------------------------------------
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const bool more = kt + 1 < ntiles;
    if (more) load_tile(kt + 1);
    if (wave_active) compute_tile(kt, kt & 1);
    if (more) store_tile((kt + 1) & 1);
    __syncthreads();
  }

  // ---- split mode: map-2 waves hand t2 = acc2 / l2 to their map-1 partners ----
  float* const xch = (float*)smem_raw;
  if constexpr (SPLIT) {
    if (wbr == 1 && wave_active) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float l2 = lsum[0][qb] + __shfl_xor(lsum[0][qb], 32);
        const float inv2 = 1.0f / l2;
        float* row = xch + (wq * C::QPW + qb * 32 + l32) * C::XP;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const floatx4 t = {acc[0][qb][cb][4 * g] * inv2, acc[0][qb][cb][4 * g + 1] * inv2,
                               acc[0][qb][cb][4 * g + 2] * inv2, acc[0][qb][cb][4 * g + 3] * inv2};
            *(floatx4*)(row + cb * 32 + 8 * g + 4 * hi) = t;
          }
      }
    }
    __syncthreads();
    if (wbr == 1) return;
  }
  if (!wave_active) return;

  // ---- epilogue: combine the maps, optional head norm, store -----------------
  E* __restrict__ O = (E*)a.out + v_off;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int query = q0 + qb * 32 + l32;
    const float l1 = lsum[0][qb] + __shfl_xor(lsum[0][qb], 32);
    const float inv1 = 1.0f / l1;
    float inv2 = 0.0f;
    if constexpr (!SPLIT) {
      const float l2 = lsum[1][qb] + __shfl_xor(lsum[1][qb], 32);
      inv2 = 1.0f / l2;
    }
    const float* xrow = xch + (wq * C::QPW + qb * 32 + l32) * C::XP;
    float o[C::CB][16];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // t1 - lam * t2 with both maps rounded identically (no contraction)
        const float t1 = acc[0][qb][cb][r] * inv1;
        float t2;
        if constexpr (SPLIT) t2 = xrow[cb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3)];
        else t2 = acc[C::NBR - 1][qb][cb][r] * inv2;
        const float lt2 = lamv * t2;
        o[cb][r] = t1 - lt2;
      }
    if constexpr (HEADNORM) {
      float ss = 0.0f;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss = fmaf(o[cb][r], o[cb][r], ss);
      ss += __shfl_xor(ss, 32);
      const float f = rsqrtf(ss * (1.0f / C::DV) + a.eps) * a.out_scale;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= f;
    }
    if (query < T) {
      E* dst = O + (size_t)query * C::DV;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ch = cb * 32 + 8 * g + 4 * hi;
          if constexpr (F32) {
            const floatx4 v4 = {o[cb][4 * g], o[cb][4 * g + 1], o[cb][4 * g + 2], o[cb][4 * g + 3]};
            *(floatx4*)(dst + ch) = v4;
          } else {
            const bf16x4 v4 = {(bf16)o[cb][4 * g], (bf16)o[cb][4 * g + 1], (bf16)o[cb][4 * g + 2],
                               (bf16)o[cb][4 * g + 3]};
            *(bf16x4*)(dst + ch) = v4;
          }
        }
    }
  }
}

// ============================================================================
// bf16 path: asynchronous global -> LDS staging
// ============================================================================
//
// K1, K2 and V tiles of 64 keys go straight from global memory into LDS with
// global_load_lds_dwordx4 (each wave instruction fills one contiguous KiB), so
// no VGPRs are spent on staging and NSTAGE - 1 tiles are in flight while one
// is computed.  Rows are XOR-swizzled at 16-byte granularity instead of
// padded: K rows so that the 32 lanes reading one 16-byte column of 32 rows
// (the S^T A operand) hit distinct banks, V rows so that the transposing
// reads below are conflict free.  V stays key-major in LDS; the A operand of
// O^T = V^T P^T is assembled by two ds_read_b64_tr_b16 per MFMA.  Within a
// group of 16 lanes that instruction hands lane j element (j mod 4) of the
// 8-byte chunks addressed by lanes 4k + j/4 (k = 0..3); addressing row
// (key) 4*hi + k and column 4*(j/4) of each 16-column group gives every lane
// four consecutive keys of its own channel, in the key order in which the
// lane's probabilities reach the MFMA.

template <int D, int NQB, int NW, int NSTAGE, bool SPLIT>
struct CfgB {
  static constexpr int BC = 64;
  static constexpr int DV = 2 * D;
  static constexpr int QPW = 32 * NQB;
  static constexpr int NBR = SPLIT ? 1 : 2;
  static constexpr int NWQ = SPLIT ? NW / 2 : NW;
  static constexpr int BR = NWQ * QPW;
  static constexpr int NT = NW * 64;
  static constexpr int KBYTES = BC * D * 2;
  static constexpr int VBYTES = BC * DV * 2;
  static constexpr int STAGE = 2 * KBYTES + VBYTES;
  static constexpr int KSEG = KBYTES / 1024;   // 1-KiB segments per K tile
  static constexpr int NSEG = STAGE / 1024;    // per stage
  static constexpr int SEGW = (NSEG + NW - 1) / NW;  // most loads one wave issues per tile
  static constexpr int SEGW_MIN = NSEG / NW;          // fewest (waits use this: safe)
  static constexpr int CB = DV / 32;
  static constexpr int KSTEPS = D / 16;
  static constexpr int XP = DV + 4;
  static constexpr int XBYTES = SPLIT ? NWQ * QPW * XP * 4 : 0;
  static constexpr int RBYTES = NSTAGE * STAGE;
  static constexpr int SMEM = RBYTES > XBYTES ? RBYTES : XBYTES;
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "two to four stages");
  static_assert(SMEM <= 160 * 1024, "LDS budget exceeded");
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4_t;

// 16-byte column swizzles (see above)
template <int D>
__device__ inline int swz_k(int row) { return D == 32 ? ((row >> 1) & 3) : (row & 7); }
__device__ inline int swz_v(int row) { return (row & 3) << 1; }

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

__device__ inline float swap_halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float swap_halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int NQB, int NW, int NSTAGE, bool SPLIT, bool CAUSAL, bool HEADNORM>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void fwd_bf16_kernel(FwdArgs a) {
  using C = CfgB<D, NQB, NW, NSTAGE, SPLIT>;
  constexpr int BC = C::BC;
  constexpr int PD = NSTAGE - 1;  // prefetch distance in tiles
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int T = a.T;

  const int nqt = (T + C::BR - 1) / C::BR;
  const int w = xcd_remap(blockIdx.x, a.B * a.H * nqt);
  const int bh = w / nqt;
  const int qi = w % nqt;
  const int qt = CAUSAL ? (nqt - 1 - qi) : qi;  // heaviest causal tiles first
  const int h = bh % a.H;

  const size_t qk_off = (size_t)bh * T * D;
  const size_t v_off = (size_t)bh * T * C::DV;
  const bf16* __restrict__ Q1 = (const bf16*)a.q1 + qk_off;
  const bf16* __restrict__ Q2 = (const bf16*)a.q2 + qk_off;
  const bf16* __restrict__ K1 = scalar_ptr((const bf16*)a.k1 + qk_off);
  const bf16* __restrict__ K2 = scalar_ptr((const bf16*)a.k2 + qk_off);
  const bf16* __restrict__ V = scalar_ptr((const bf16*)a.v + v_off);

  const int wbr = SPLIT ? wave / C::NWQ : 0;
  const int wq = SPLIT ? wave % C::NWQ : wave;
  const int q_tile0 = qt * C::BR;
  const int q0 = q_tile0 + wq * C::QPW;
  const int q_last = min(q0 + C::QPW, T) - 1;
  const bool wave_active = q0 < T;
  const int k_end = CAUSAL ? min(T, q_tile0 + C::BR) : T;
  const int ntiles = (k_end + BC - 1) / BC;
  const float sc = a.score_scale;
  const float lamv = a.lam[h];

  // ---- asynchronous tile loads ------------------------------------------------
  // Segment g of a K tile (1 KiB) holds rows RK g .. RK g + RK - 1; lane l
  // copies row RK g + l / CK, 16-byte column (l % CK) ^ swz_k(row).  The
  // swizzle depends on g only through its parity (D = 128), so a lane's
  // column offset takes one of two values; likewise for V.  Keys past the end
  // load row T-1 (in bounds); their scores are masked.
  constexpr int CK = D / 8, RK = 64 / CK, CV = C::DV / 8, RV = 64 / CV;
  const int rl_k = lane / CK, rl_v = lane / CV;
  auto issue_rt = [&](int kt, char* sb) __attribute__((always_inline)) {
    const int key0 = kt * BC;
#pragma unroll
    for (int i = 0; i < C::SEGW; ++i) {
      const int seg = wave + i * NW;
      if (seg >= C::NSEG) break;
      if (seg < 2 * C::KSEG) {
        const int which = seg / C::KSEG;
        const int g = seg % C::KSEG;
        const int r = g * RK + rl_k;
        const int c = (lane % CK) ^ swz_k<D>((g & 1) * RK + rl_k);
        const uint32_t row = (uint32_t)min(key0 + r, T - 1);
        dma16(which ? K2 : K1, row * (D * 2) + c * 16, sb + which * C::KBYTES + g * 1024);
      } else {
        const int g = seg - 2 * C::KSEG;
        const int r = g * RV + rl_v;
        const int c = (lane % CV) ^ swz_v((g & 1) * RV + rl_v);
        const uint32_t row = (uint32_t)min(key0 + r, T - 1);
        dma16(V, row * (C::DV * 2) + c * 16, sb + 2 * C::KBYTES + g * 1024);
      }
    }
  };
  auto issue = [&](int kt, auto st) __attribute__((always_inline)) {
    issue_rt(kt, smem + decltype(st)::value * C::STAGE);
  };

  // ---- Q fragments (B operand of S^T = K Q^T) -------------------------------
  bf16x8 qf[C::NBR][NQB][C::KSTEPS];
#pragma unroll
  for (int br = 0; br < C::NBR; ++br) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int query = q0 + qb * 32 + l32;
      const bool ok = query < T;
      const bf16* src = ((br + wbr) ? Q2 : Q1) + (size_t)min(query, T - 1) * D;
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        u32x4 raw = *(const u32x4*)(src + ks * 16 + hi * 8);
        raw = ok ? raw : u32x4{0u, 0u, 0u, 0u};
        qf[br][qb][ks] = __builtin_bit_cast(bf16x8, raw);
      }
    }
  }

  // Q is in registers before any tile load is issued, so the compiler's wait
  // for it does not also wait for the asynchronous tile loads
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0)
  // prologue: tiles 0 .. PD-1 into stages 0 .. PD-1
  issue(0, std::integral_constant<int, 0>{});
  if constexpr (PD > 1)
    if (1 < ntiles) issue(1, std::integral_constant<int, 1>{});
  if constexpr (PD > 2)
    if (2 < ntiles) issue(2, std::integral_constant<int, 2>{});

  floatx16 acc[C::NBR][NQB][C::CB];
  float mu[C::NBR][NQB];
  float lsum[C::NBR][NQB];
#pragma unroll
  for (int br = 0; br < C::NBR; ++br)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      mu[br][qb] = kNegInf;
      lsum[br][qb] = 0.0f;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[br][qb][cb][r] = 0.0f;
    }

  // per-lane LDS offsets (bytes) that do not depend on the block
  const int k_rd = l32 * (2 * D);                 // + kb*32 rows, + chunk ^ swizzle
  const int swk = swz_k<D>(l32);
  const int vq = lane & 3;
  const int vkq = (lane >> 2) & 3;
  const int v_row = 4 * hi + vkq;                 // + kb*32 + 16*ks + 8*t
  const int v_chunk = 2 * ((lane >> 4) & 1) + (vq >> 1);  // + 4*cb
  const int v_sw = swz_v(vkq);
  const int v_byte = (vq & 1) * 8;
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};

  // A 32-key block kb of tile kt takes part only if it holds a key this wave
  // may attend to.
  auto kb_live = [&](int kt, int kb) __attribute__((always_inline)) {
    const int key0 = kt * BC + kb * 32;
    return key0 < T && (!CAUSAL || key0 <= q_last);
  };

  // S^T of block kb for both maps (raw dot products, scale applied later)
  auto qk = [&](int kb, const char* sb, floatx16 (&s)[C::NBR][NQB]) __attribute__((always_inline)) {
    const char* Kb[2] = {sb + (SPLIT && wbr ? C::KBYTES : 0), sb + C::KBYTES};
#pragma unroll
    for (int br = 0; br < C::NBR; ++br)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[br][qb][r] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
#pragma unroll
      for (int br = 0; br < C::NBR; ++br) {
        const bf16x8 av = *(const bf16x8*)(Kb[br] + kb * 32 * (2 * D) + k_rd + (((2 * ks + hi) ^ swk) << 4));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          s[br][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[br][qb][ks], s[br][qb], 0, 0, 0);
      }
    }
  };

  // mask, running maxima (lazy rescale of acc and lsum), probabilities P^T as
  // the bf16 B operand of the P.V product, row sums of those bf16 values
  auto softmax = [&](int kt, int kb, floatx16 (&s)[C::NBR][NQB], bf16x8 (&pk)[C::NBR][NQB][2])
      __attribute__((always_inline)) {
    const int key0 = kt * BC + kb * 32;
    const bool need_mask = CAUSAL ? (key0 + 31 > q0) : (key0 + 32 > T);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int query = q0 + qb * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool masked = CAUSAL ? (key > query) : (key >= T);
          if (masked) {
#pragma unroll
            for (int br = 0; br < C::NBR; ++br) s[br][qb][r] = kNegInf;
          }
        }
      }
    }

    float mx[C::NBR][NQB];
    bool need = false;
#pragma unroll
    for (int br = 0; br < C::NBR; ++br)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        float m = s[br][qb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) m = fmaxf(m, s[br][qb][r]);
        m = swap_halves_max(m) * sc;
        mx[br][qb] = m;
        need |= m > mu[br][qb] + kTau;
      }
    if (__any(need)) {
#pragma unroll
      for (int br = 0; br < C::NBR; ++br)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          const float mn = fmaxf(mu[br][qb], mx[br][qb]);
          const float alpha = (mn == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f(mu[br][qb] - mn);
          mu[br][qb] = mn;
          lsum[br][qb] *= alpha;
#pragma unroll
          for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[br][qb][cb][r] *= alpha;
        }
    }

#pragma unroll
    for (int br = 0; br < C::NBR; ++br)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float msub = mu[br][qb] == kNegInf ? 0.0f : mu[br][qb];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float pa = __builtin_amdgcn_exp2f(fmaf(s[br][qb][8 * ks + 2 * j], sc, -msub));
            const float pb = __builtin_amdgcn_exp2f(fmaf(s[br][qb][8 * ks + 2 * j + 1], sc, -msub));
            const bf16x2 pw = {(bf16)pa, (bf16)pb};
            lsum[br][qb] = __builtin_amdgcn_fdot2_f32_bf16(pw, ones, lsum[br][qb], false);
            pk[br][qb][ks][2 * j] = pw[0];
            pk[br][qb][ks][2 * j + 1] = pw[1];
          }
        }
      }
  };

  // acc += P^T-weighted V rows of block kb; each V fragment serves both maps
  auto pv = [&](int kb, const char* sb, const bf16x8 (&pk)[C::NBR][NQB][2]) __attribute__((always_inline)) {
    const char* Vb = sb + 2 * C::KBYTES;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* base = Vb + (kb * 32 + 16 * ks + v_row) * (2 * C::DV) + (((4 * cb + v_chunk) ^ v_sw) << 4) + v_byte;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)base);
        const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(base + 8 * (2 * C::DV)));
        const bf16x8 av = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
#pragma unroll
        for (int br = 0; br < C::NBR; ++br)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            acc[br][qb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pk[br][qb][ks], acc[br][qb][cb], 0, 0, 0);
      }
  };

  if (PD < ntiles) wait_vm_barrier<C::SEGW_MIN * (PD - 1)>();
  else wait_vm_barrier<0>();
  // ---- main loop: tile kt computed while tiles kt+1 .. kt+PD load ------------
  auto compute_tile = [&](int kt, const char* sb) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      if (!kb_live(kt, kb)) break;
      floatx16 s[C::NBR][NQB];
      bf16x8 pk[C::NBR][NQB][2];
      qk(kb, sb, s);
      softmax(kt, kb, s, pk);
      pv(kb, sb, pk);
    }
  };
  // unrolled by NSTAGE so that every stage offset is a compile-time constant
  auto step = [&](int kt, auto st) __attribute__((always_inline)) {
    constexpr int S = decltype(st)::value;
    if (kt + PD < ntiles) issue(kt + PD, std::integral_constant<int, (S + PD) % NSTAGE>{});
    if (wave_active) compute_tile(kt, smem + S * C::STAGE);
    if (kt + PD < ntiles) wait_vm_barrier<C::SEGW_MIN * (PD - 1)>();
    else wait_vm_barrier<0>();
  };
  for (int kt = 0; kt < ntiles; kt += NSTAGE) {
    step(kt, std::integral_constant<int, 0>{});
    if (kt + 1 < ntiles) step(kt + 1, std::integral_constant<int, 1>{});
    if constexpr (NSTAGE > 2)
      if (kt + 2 < ntiles) step(kt + 2, std::integral_constant<int, 2>{});
    if constexpr (NSTAGE > 3)
      if (kt + 3 < ntiles) step(kt + 3, std::integral_constant<int, 3>{});
  }

  // ---- split mode: map-2 waves hand t2 = acc2 / l2 to their map-1 partners ----
  float* const xch = (float*)smem;
  if constexpr (SPLIT) {
    if (wbr == 1 && wave_active) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float inv2 = 1.0f / swap_halves_sum(lsum[0][qb]);
        float* row = xch + (wq * C::QPW + qb * 32 + l32) * C::XP;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const floatx4 t = {acc[0][qb][cb][4 * g] * inv2, acc[0][qb][cb][4 * g + 1] * inv2,
                               acc[0][qb][cb][4 * g + 2] * inv2, acc[0][qb][cb][4 * g + 3] * inv2};
            *(floatx4*)(row + cb * 32 + 8 * g + 4 * hi) = t;
          }
      }
    }
    __syncthreads();
    if (wbr == 1) return;
  }
  if (!wave_active) return;

  // ---- epilogue: combine the maps, optional head norm, store -----------------
  bf16* __restrict__ O = (bf16*)a.out + v_off;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int query = q0 + qb * 32 + l32;
    const float inv1 = 1.0f / swap_halves_sum(lsum[0][qb]);
    float inv2 = 0.0f;
    if constexpr (!SPLIT) inv2 = 1.0f / swap_halves_sum(lsum[1][qb]);
    const float* xrow = xch + (wq * C::QPW + qb * 32 + l32) * C::XP;
    float o[C::CB][16];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // t1 - lam * t2 with both maps rounded identically (no contraction)
        const float t1 = acc[0][qb][cb][r] * inv1;
        float t2;
        if constexpr (SPLIT) t2 = xrow[cb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3)];
        else t2 = acc[C::NBR - 1][qb][cb][r] * inv2;
        const float lt2 = lamv * t2;
        o[cb][r] = t1 - lt2;
      }
    if constexpr (HEADNORM) {
      float ss = 0.0f;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) ss = fmaf(o[cb][r], o[cb][r], ss);
      ss = swap_halves_sum(ss);
      const float f = rsqrtf(ss * (1.0f / C::DV) + a.eps) * a.out_scale;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[cb][r] *= f;
    }
    if (query < T) {
      bf16* dst = O + (size_t)query * C::DV;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const bf16x4 v4 = {(bf16)o[cb][4 * g], (bf16)o[cb][4 * g + 1], (bf16)o[cb][4 * g + 2],
                             (bf16)o[cb][4 * g + 3]};
          *(bf16x4*)(dst + cb * 32 + 8 * g + 4 * hi) = v4;
        }
    }
  }
}

template <int D, int NQB, int NW, int NSTAGE, bool SPLIT>
hipError_t launch_bf16(const FwdArgs& a, bool causal, bool headnorm, hipStream_t stream) {
  using C = CfgB<D, NQB, NW, NSTAGE, SPLIT>;
  const long nqt = (a.T + C::BR - 1) / C::BR;
  const long grid = (long)a.B * a.H * nqt;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), b(C::NT);
  if (causal) {
    if (headnorm) fwd_bf16_kernel<D, NQB, NW, NSTAGE, SPLIT, true, true><<<g, b, 0, stream>>>(a);
    else fwd_bf16_kernel<D, NQB, NW, NSTAGE, SPLIT, true, false><<<g, b, 0, stream>>>(a);
  } else {
    if (headnorm) fwd_bf16_kernel<D, NQB, NW, NSTAGE, SPLIT, false, true><<<g, b, 0, stream>>>(a);
    else fwd_bf16_kernel<D, NQB, NW, NSTAGE, SPLIT, false, false><<<g, b, 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <int D, int NQB, int NW, int BC, bool F32, bool SPLIT>
hipError_t launch_cfg(const FwdArgs& a, bool causal, bool headnorm, hipStream_t stream) {
  using C = Cfg<D, NQB, NW, BC, F32, SPLIT>;
  const long nqt = (a.T + C::BR - 1) / C::BR;
  const long grid = (long)a.B * a.H * nqt;
  if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), b(C::NT);
  if (causal) {
    if (headnorm) fwd_kernel<D, NQB, NW, BC, F32, SPLIT, true, true><<<g, b, 0, stream>>>(a);
    else fwd_kernel<D, NQB, NW, BC, F32, SPLIT, true, false><<<g, b, 0, stream>>>(a);
  } else {
    if (headnorm) fwd_kernel<D, NQB, NW, BC, F32, SPLIT, false, true><<<g, b, 0, stream>>>(a);
    else fwd_kernel<D, NQB, NW, BC, F32, SPLIT, false, false><<<g, b, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, bool causal, bool headnorm,
                      hipStream_t stream) {
  if (dtype == 1) {  // bf16
    switch (D) {
      case 32: return launch_bf16<32, 1, 8, 3, false>(a, causal, headnorm, stream);
      case 64:
        // short causal rows: one map per wave, three waves per SIMD (more
        // latency hiding); long causal rows: both maps per wave (less LDS
        // traffic per MFMA); full attention: one map and 64 rows per wave
        if (causal && a.T <= 4096) return launch_bf16<64, 1, 12, 3, true>(a, causal, headnorm, stream);
        if (causal) return launch_bf16<64, 1, 8, 3, false>(a, causal, headnorm, stream);
        return launch_bf16<64, 2, 8, 3, true>(a, causal, headnorm, stream);
      case 128: return launch_bf16<128, 1, 8, 2, true>(a, causal, headnorm, stream);
    }
  } else {  // fp32
    switch (D) {
      case 32: return launch_cfg<32, 1, 4, 32, true, false>(a, causal, headnorm, stream);
      case 64: return launch_cfg<64, 1, 4, 32, true, false>(a, causal, headnorm, stream);
      case 128: return launch_cfg<128, 1, 4, 32, true, true>(a, causal, headnorm, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace diffattn
