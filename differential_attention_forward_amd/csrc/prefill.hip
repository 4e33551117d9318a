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
// Design shared by both kernels (one pass over K/V, both maps at once):
//  * One workgroup = NW waves = BR query rows of one (b, h); each wave owns
//    32*NQB queries.  Q1/Q2 fragments stay in VGPRs for the whole kernel.
//    Either every wave runs both maps, or (split mode) waves pair up, one per
//    map, on the same rows and the map-2 wave hands t2 = acc2 / l2 to its
//    partner through LDS at the end.
//  * Scores are computed transposed, S^T = K Q^T: lane l then holds 16 keys
//    of query l%32, so the row max is an in-lane reduction plus one exchange
//    with lane l^32, and the probabilities P^T land in exactly the register
//    layout the P.V MFMA wants as its B operand (no data movement).
//  * Two independent online-softmax states per query row (one per map) with
//    lazy rescaling: the running max only moves (and the accumulators are
//    only rescaled) when a block max exceeds it by more than kTau (log2
//    units), so steady-state blocks do no rescale work.
//  * Both P1.V and P2.V are fed from one V tile in LDS: each V fragment read
//    serves both branches (V is read from memory once, not once per map).
//  * Causal: key blocks above a wave's last query are skipped; only blocks
//    that straddle the diagonal evaluate the mask.  Query tiles are issued
//    heaviest first and workgroups are remapped so that each XCD works
//    through consecutive tiles of the same heads (K/V reuse in its L2).
//
// bf16 (fwd_bf16_kernel): K1, K2, V tiles of 64 keys go global -> LDS
// directly (asynchronous DMA, NSTAGE-deep ring), v_mfma_f32_32x32x16_bf16,
// probabilities rounded to bf16 for the P.V product.
// fp32 (fwd_f32_kernel): tiles of 32 to 128 keys staged global -> VGPR ->
// LDS, double buffered, v_mfma_f32_32x32x2_f32, fp32 probabilities.
#include "common.h"
#include "kernels.h"

namespace diffattn {
namespace {

constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units): p <= 2^8
constexpr float kRescaleSum = 256.0f;  // 2^kTau: a partial row sum above it may hold a p > 2^kTau

// lambda of head h: read from the [H] array, or (fused path) formed here by
// every wave from the four vectors, with the same bits as the lambda kernel;
// the first query tile of batch 0 stores it to lam_out when asked.
__device__ inline float head_lambda(const FwdArgs& a, int h, int qt, int bh) {
  if (a.lvec[0] == nullptr) return a.lam[h];
  const float lam = reparam_lambda(a.lvec[0], a.lvec[1], a.lvec[2], a.lvec[3], h, a.Dl, a.lam_init);
  if (a.lam_out != nullptr && qt == 0 && bh == h && threadIdx.x == 0) a.lam_out[h] = lam;
  return lam;
}

template <int D, int NQB, int NW, int BC, bool SPLIT>
struct Cfg {
  static constexpr int DV = 2 * D;
  static constexpr int QPW = 32 * NQB;
  static constexpr int NBR = SPLIT ? 1 : 2;         // maps handled by one wave
  static constexpr int NWQ = SPLIT ? NW / 2 : NW;   // waves per map
  static constexpr int BR = NWQ * QPW;              // query rows per workgroup
  static constexpr int NT = NW * 64;
  static constexpr int ES = 4;
  static constexpr int EPC = 16 / ES;               // elements per 16-byte chunk
  static constexpr int KP = D + 4;                 // K row pitch (floats)
  static constexpr int VP = DV + 4;                 // V row pitch (floats), row-major [BC][DV]
  static constexpr int KTILE = BC * KP;
  static constexpr int VTILE = BC * VP;
  static constexpr int STAGE = 2 * KTILE + VTILE;   // elements per LDS stage
  static constexpr int NKC = BC * D / EPC;          // 16-B chunks per K tile
  static constexpr int NKPT = (NKC + NT - 1) / NT;
  static constexpr int NVU = BC * DV / EPC;         // 16-B chunks per V tile
  static constexpr int NVPT = (NVU + NT - 1) / NT;
  static constexpr int NKB = BC / 32;               // 32-key blocks per tile
  static constexpr int CB = DV / 32;                // 32-channel output blocks
  static constexpr int KSTEPS = D / 2;
  // split mode: map-2 waves hand acc2/l2 to their map-1 partners through LDS
  static constexpr int XP = DV + 4;                 // exchange row pitch (floats)
  static constexpr int XBYTES = SPLIT ? NWQ * QPW * XP * 4 : 0;
  static constexpr int RBYTES = 2 * STAGE * ES;
  static constexpr int SMEM = RBYTES > XBYTES ? RBYTES : XBYTES;
  static_assert(BC % 32 == 0, "key tile must hold whole 32-key blocks");
  static_assert(!SPLIT || NW % 2 == 0, "split mode pairs waves");
  static_assert(SMEM <= 160 * 1024, "LDS budget exceeded");
};

template <int D, int NQB, int NW, int BC, bool SPLIT, bool CAUSAL, bool HEADNORM>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW >= 8 ? 2 : 1, NW >= 8 ? 2 : 1))) void fwd_f32_kernel(FwdArgs a) {
  using C = Cfg<D, NQB, NW, BC, SPLIT>;
  __shared__ __attribute__((aligned(16))) char smem_raw[C::SMEM];
  float* const smem = (float*)smem_raw;
  lds_poison(smem_raw, sizeof(smem_raw));
  lds_poison_done();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int T = a.T;

  const int nqt = (T + C::BR - 1) / C::BR;
  const int w = xcd_remap(blockIdx.x, a.B * a.H * nqt);
  int bh, qi;
  if (CAUSAL) causal_order(w, a.B * a.H * nqt, nqt, bh, qi);
  else bh = w / nqt, qi = w % nqt;
  const int qt = CAUSAL ? (nqt - 1 - qi) : qi;  // heaviest causal tiles first
  const int h = bh % a.H;

  const size_t qk_off = (size_t)bh * T * D;
  const size_t v_off = (size_t)bh * T * C::DV;
  const float* __restrict__ Q1 = (const float*)a.q1 + qk_off;
  const float* __restrict__ Q2 = (const float*)a.q2 + qk_off;
  const float* __restrict__ K1 = (const float*)a.k1 + qk_off;
  const float* __restrict__ K2 = (const float*)a.k2 + qk_off;
  const float* __restrict__ V = (const float*)a.v + v_off;

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
  const float lamv = head_lambda(a, h, qt, bh);

  // ---- Q fragments (B operand of S^T = K Q^T) -------------------------------
  float qf[C::NBR][NQB][C::KSTEPS];
#pragma unroll
  for (int br = 0; br < C::NBR; ++br) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      // rows past the end read row T-1 (always in bounds) and are zeroed
      const int query = q0 + qb * 32 + l32;
      const bool ok = query < T;
      const float* src = ((br + wbr) ? Q2 : Q1) + (size_t)min(query, T - 1) * D;
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        const float x = src[2 * ks + hi];
        qf[br][qb][ks] = ok ? x : 0.0f;
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
  u32x4 rv[C::NVPT];
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
      const int row = u / (C::DV / 4);
      const int col = u % (C::DV / 4);
      const int key = kbase + row;
      const u32x4 x = *(const u32x4*)(V + (size_t)min(key, T - 1) * C::DV + col * 4);
      rv[i] = key < T ? x : zero4;
    }
  };

  auto store_tile = [&](int buf) {
    float* Ks1 = smem + buf * C::STAGE;
    float* Ks2 = Ks1 + C::KTILE;
    float* Vs = Ks2 + C::KTILE;
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
        const int row = u / (C::DV / 4);
        const int col = u % (C::DV / 4);
        *(u32x4*)(Vs + row * C::VP + col * 4) = rv[i];
      }
    }
  };

  auto compute_tile = [&](int kt, int buf) {
    const float* Ks1 = smem + buf * C::STAGE;
    const float* Ks2 = Ks1 + C::KTILE;
    const float* Vs = Ks2 + C::KTILE;
    const float* Kmap[2] = {SPLIT && wbr ? Ks2 : Ks1, Ks2};  // K tile of each map this wave runs
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
          const float av = Kmap[br][(kb * 32 + l32) * C::KP + 2 * ks + hi];
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            s[br][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, qf[br][qb][ks], s[br][qb], 0, 0, 0);
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
  float* __restrict__ O = (float*)a.out + v_off;
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
    // the output is formed in place in map 1's accumulators: a separate array
    // of the same size would double the live registers (D = 128 spilled)
    floatx16 (&o)[C::CB] = acc[0][qb];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        // t1 - lam * t2 with both maps rounded identically (no contraction)
        const float t1 = o[cb][r] * inv1;
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
      float* dst = O + (size_t)query * C::DV;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ch = cb * 32 + 8 * g + 4 * hi;
          const floatx4 v4 = {o[cb][4 * g], o[cb][4 * g + 1], o[cb][4 * g + 2], o[cb][4 * g + 3]};
          *(floatx4*)(dst + ch) = v4;
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

// MAPS = 2: differential attention (Q1, K1, Q2, K2 of width D, V of width
// 2D); with SHKV, the V2 form instead: both maps read one K tile and one V
// tile of width D, shared by a group of heads.  MAPS = 1: standard softmax
// attention (Q, K, V of width D), the
// comparison kernel of the same size as a differential head of width D/2.
template <int D, int NQB, int NW, int NSTAGE, bool SPLIT, int MAPS = 2, bool SHKV = false>
struct CfgB {
  static constexpr int BC = 64;
  static constexpr int DV = MAPS == 2 && !SHKV ? 2 * D : D;
  static constexpr int KT = SHKV ? 1 : MAPS;        // K tiles per stage
  static constexpr int QPW = 32 * NQB;
  static constexpr int NBR = SPLIT || MAPS == 1 ? 1 : 2;
  static constexpr int NWQ = SPLIT ? NW / 2 : NW;
  static constexpr int BR = NWQ * QPW;
  static constexpr int NT = NW * 64;
  static constexpr int KBYTES = BC * D * 2;
  static constexpr int VBYTES = BC * DV * 2;
  static constexpr int STAGE = KT * KBYTES + VBYTES;
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
  // -mu as a register tuple held across blocks (16 VGPRs per map and query
  // block), or rebuilt from mu before every block where registers are short
  static constexpr bool NEGMU_REGS = NBR * NQB == 1 && D <= 64;
  static_assert(NSTAGE >= 2 && NSTAGE <= 4, "two to four stages");
  static_assert(MAPS == 2 || !SPLIT, "one map: nothing to split");
  static_assert(MAPS == 2 || !SHKV, "shared K/V is the two-map V2 form");
  static_assert(SMEM <= 160 * 1024, "LDS budget exceeded");
};

template <int D, int NQB, int NW, int NSTAGE, bool SPLIT, bool CAUSAL, bool HEADNORM, int MAPS = 2,
          bool SHKV = false, bool WIN = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW < 8 ? 2 : NW / 4, NW < 8 ? 2 : NW / 4))) void fwd_bf16_kernel(FwdArgs a) {
  using C = CfgB<D, NQB, NW, NSTAGE, SPLIT, MAPS, SHKV>;
  constexpr int BC = C::BC;
  constexpr int PD = NSTAGE - 1;  // prefetch distance in tiles
  // One-map waves at D <= 64 in eight-wave workgroups (two waves per SIMD,
  // 256 registers each, about 170 used) read a block's LDS fragments ahead
  // of their MFMAs: every K fragment before the first score MFMA, every V
  // fragment right after the score MFMAs, in flight during the softmax.  Left
  // to itself the compiler issues each read just before its MFMA and waits on
  // it at once, about six LDS round trips per block and wave; the early
  // reads take 204 registers and 3-5% off the T = 4096 causal prefill
  // (bit-identical).  Other shapes have no registers to spare.
  constexpr bool PREF = C::NBR * NQB == 1 && D <= 64 && !SHKV && NW == 8;
  // One-map waves at D = 128 have no registers for that in the split shape
  // (250-255 used): there each fragment read is issued one MFMA ahead
  // instead (PIPE), into a second 4-register buffer.  Left to itself the
  // compiler waits on every read at once (lgkmcnt(0) before each of the 24
  // MFMAs of a block); one read in flight behind each MFMA takes 2.7% off
  // the D = 128 full prefill and 1.2% off the D = 128 V2 prefill
  // (bit-identical).  The V2 form has the registers for all of a block's K
  // reads up front (176 used) but gains nothing more from them.
  constexpr bool PIPE = C::NBR * NQB == 1 && D == 128;
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  lds_poison(smem, sizeof(smem));
  lds_poison_done();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int T = a.T;

  const int nqt = (T + C::BR - 1) / C::BR;
  // the division by nqt runs on the VALU: say that the results are uniform so
  // that every loop bound and branch derived from them stays scalar
  const int w = xcd_remap(blockIdx.x, a.B * a.H * nqt);
  int bh_, qi_;
  if (CAUSAL) causal_order(w, a.B * a.H * nqt, nqt, bh_, qi_);
  else bh_ = w / nqt, qi_ = w % nqt;
  const int bh = __builtin_amdgcn_readfirstlane(bh_);
  const int qi = __builtin_amdgcn_readfirstlane(qi_);
  const int qt = CAUSAL ? (nqt - 1 - qi) : qi;  // heaviest causal tiles first
  const int h = bh % a.H;

  // V2: head h of batch b reads KV head h / (H / Hkv) of that batch.  Each
  // tensor is addressed through its own batch, head and row strides.
  const int bb = bh / a.H;
  const int kvh = SHKV ? h / (a.H / a.Hkv) : h;
  const size_t o_off = (size_t)bh * T * C::DV;  // the saved training maps are dense
  const bf16* __restrict__ Q1 = (const bf16*)a.q1 + (bb * a.sb[0] + h * a.sh[0]);
  const bf16* __restrict__ Q2 = (const bf16*)a.q2 + (bb * a.sb[2] + h * a.sh[2]);
  const bf16* __restrict__ K1 = scalar_ptr((const bf16*)a.k1 + (bb * a.sb[1] + kvh * a.sh[1]));
  const bf16* __restrict__ K2 =
      SHKV ? K1 : scalar_ptr((const bf16*)a.k2 + (bb * a.sb[3] + kvh * a.sh[3]));
  const bf16* __restrict__ V = scalar_ptr((const bf16*)a.v + (bb * a.sb[4] + kvh * a.sh[4]));
  // row strides: queries and output in elements, K and V rows in bytes
  const int rq[2] = {a.sr[0], a.sr[2]};
  const uint32_t rk_b[2] = {2u * (uint32_t)a.sr[1], 2u * (uint32_t)a.sr[3]};
  const uint32_t rv_b = 2u * (uint32_t)a.sr[4];

  const int wbr = SPLIT ? wave / C::NWQ : 0;
  const int wq = SPLIT ? wave % C::NWQ : wave;
  const int q_tile0 = qt * C::BR;
  const int q0 = q_tile0 + wq * C::QPW;
  const int q_last = min(q0 + C::QPW, T) - 1;
  const bool wave_active = q0 < T;
  const int k_end = CAUSAL ? min(T, q_tile0 + C::BR) : T;
  // sliding window (causal only): row i sees keys i - W < j <= i.  Key tiles
  // below the workgroup's first row's window are never loaded: the
  // workgroup's tiles are kt0 .. kt0 + ntiles - 1, and the loop's step kt
  // names one of them through ptile.
  const int W = CAUSAL && WIN ? a.window : 0;
  const int kt0 = W > 0 ? max(0, q_tile0 - W + 1) / BC : 0;
  const int ntiles = (k_end + BC - 1) / BC - kt0;
  // With a window, step kt visits tile kt0 + ((kt - kt0) mod ntiles): the
  // workgroups of consecutive query tiles, which run side by side on one XCD,
  // then read the same key tile at the same step (their windows overlap in
  // all but a few tiles), so each tile is fetched into that XCD's L2 about
  // once rather than once per workgroup (T = 32768, W = 4096: 1.50 -> 0.51 GB
  // fetched per launch, 2% less time).  The online softmax takes the tiles
  // in any order.  Without a window kt0 = 0 and the order is the natural one.
  const int krot = W > 0 ? (ntiles - kt0 % ntiles) % ntiles : 0;
  auto ptile = [&](int kt) __attribute__((always_inline)) {
    const int r = kt + krot;
    return kt0 + (r >= ntiles ? r - ntiles : r);
  };
  const float sc = a.score_scale;
  float lamv = 0.0f;
  if constexpr (MAPS == 2) {
    lamv = head_lambda(a, h, qt, bh);
    // formed here, before the tile loads start (not sunk into the loop)
    asm volatile("" ::"v"(lamv));
  }

  // ---- asynchronous tile loads ------------------------------------------------
  // Segment g of a K tile (1 KiB) holds rows RK g .. RK g + RK - 1; lane l
  // copies row RK g + l / CK, 16-byte column (l % CK) ^ swz_k(row); likewise
  // for V.  Keys past the end load row T-1 (in bounds); their scores are
  // masked.
  constexpr int CK = D / 8, RK = 64 / CK, CV = C::DV / 8, RV = 64 / CV;
  const int rl_k = lane / CK, rl_v = lane / CV;
  auto issue_rt = [&](int kt, char* sb) __attribute__((always_inline)) {
    const int key0 = ptile(kt) * BC;
#pragma unroll
    for (int i = 0; i < C::SEGW; ++i) {
      const int seg = wave + i * NW;
      if (seg >= C::NSEG) break;
      if (seg < C::KT * C::KSEG) {
        const int which = seg / C::KSEG;
        const int g = seg % C::KSEG;
        const int r = g * RK + rl_k;
        const int c = (lane % CK) ^ swz_k<D>(r);
        const uint32_t row = (uint32_t)min(key0 + r, T - 1);
        dma16(which ? K2 : K1, row * rk_b[which] + c * 16, sb + which * C::KBYTES + g * 1024);
      } else {
        const int g = seg - C::KT * C::KSEG;
        const int r = g * RV + rl_v;
        const int c = (lane % CV) ^ swz_v<C::DV>(r);
        const uint32_t row = (uint32_t)min(key0 + r, T - 1);
        dma16(V, row * rv_b + c * 16, sb + C::KT * C::KBYTES + g * 1024);
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
      const bf16* src = ((br + wbr) ? Q2 : Q1) + (size_t)min(query, T - 1) * rq[br + wbr];
#pragma unroll
      for (int ks = 0; ks < C::KSTEPS; ++ks) {
        u32x4 raw = *(const u32x4*)(src + ks * 16 + hi * 8);
        raw = ok ? raw : u32x4{0u, 0u, 0u, 0u};
        // scores come out of the MFMA already in base-2 units: q * log2(e) / sqrt(D)
        // rounded once to bf16 (relative error <= 2^-8 per element)
        const bf16x8 q = __builtin_bit_cast(bf16x8, raw);
        bf16x8 qs;
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[e] = (bf16)((float)q[e] * sc);
        qf[br][qb][ks] = qs;
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

  // Softmax state per map and query row: the reference mu (base-2 units),
  // the row sum lsum of 2^(s - mu) and the accumulators.  negmu holds -mu
  // in all 16 elements and is the accumulator input of the first score MFMA,
  // so the scores arrive with the reference already subtracted.  mu starts
  // at 0 and is set to the exact row max by the first block in which the row
  // sees a key.
  floatx16 acc[C::NBR][NQB][C::CB];
  floatx16 negmu[C::NEGMU_REGS ? C::NBR : 1][C::NEGMU_REGS ? NQB : 1];
  float mu[C::NBR][NQB];
  float lsum[C::NBR][NQB];
  bool seen[C::NBR][NQB];
#pragma unroll
  for (int br = 0; br < C::NBR; ++br)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      mu[br][qb] = 0.0f;
      lsum[br][qb] = 0.0f;
      seen[br][qb] = false;
      if constexpr (C::NEGMU_REGS) negmu[br][qb] = splat16(0.0f);
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
  const int v_sw = swz_v<C::DV>(vkq);  // rows 16 ks + 4 hi + vkq (+ 8): same swizzle
  const int v_byte = (vq & 1) * 8;

  // A 32-key block kb of tile kt takes part only if it holds a key this wave
  // may attend to.
  auto kb_live = [&](int kt, int kb) __attribute__((always_inline)) {
    const int key0 = ptile(kt) * BC + kb * 32;
    return key0 < T && (!CAUSAL || key0 <= q_last) && (W == 0 || key0 + 31 > q0 - W);
  };

  // S^T of block kb for both maps: scaled scores minus the row reference
  // (base-2 units), the reference entering as the first MFMA's accumulator
  auto qk = [&](int kb, const char* sb, floatx16 (&s)[C::NBR][NQB]) __attribute__((always_inline)) {
    // (V2: one K tile serves both maps, and each fragment is read once)
    const char* Kb[2] = {sb + (SPLIT && wbr && !SHKV ? C::KBYTES : 0), sb + (SHKV ? 0 : C::KBYTES)};
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      bf16x8 av;
#pragma unroll
      for (int br = 0; br < C::NBR; ++br) {
        if (br == 0 || !SHKV)
          av = *(const bf16x8*)(Kb[br] + kb * 32 * (2 * D) + k_rd + (((2 * ks + hi) ^ swk) << 4));
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          s[br][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[br][qb][ks], ks > 0 ? s[br][qb]
                                                               : C::NEGMU_REGS ? negmu[br][qb]
                                                               : splat16(-mu[br][qb]), 0, 0, 0);
      }
    }
  };

  // The same products with the reads issued ahead (PREF): all K fragments of
  // block kb, then the score MFMAs, the order pinned by a scheduling barrier.
  auto qk_early = [&](int kb, const char* sb, floatx16 (&s)[C::NBR][NQB]) __attribute__((always_inline)) {
    const char* Kb = sb + (SPLIT && wbr ? C::KBYTES : 0) + kb * 32 * (2 * D) + k_rd;
    bf16x8 kfr[C::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) kfr[ks] = *(const bf16x8*)(Kb + (((2 * ks + hi) ^ swk) << 4));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks)
      s[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[ks], qf[0][0][ks], ks > 0 ? s[0][0]
                                                        : C::NEGMU_REGS ? negmu[0][0]
                                                        : splat16(-mu[0][0]), 0, 0, 0);
  };

  // (PIPE) the score product with each K fragment read one MFMA ahead
  auto qk_pipe = [&](int kb, const char* sb, floatx16 (&s)[C::NBR][NQB]) __attribute__((always_inline)) {
    const char* Kb = sb + (SPLIT && wbr && !SHKV ? C::KBYTES : 0) + kb * 32 * (2 * D) + k_rd;
    bf16x8 cur = *(const bf16x8*)(Kb + ((hi ^ swk) << 4));
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      bf16x8 nxt;
      if (ks + 1 < C::KSTEPS) nxt = *(const bf16x8*)(Kb + (((2 * (ks + 1) + hi) ^ swk) << 4));
      __builtin_amdgcn_sched_barrier(0);
      s[0][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[0][0][ks], ks > 0 ? s[0][0]
                                                        : C::NEGMU_REGS ? negmu[0][0]
                                                        : splat16(-mu[0][0]), 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (ks + 1 < C::KSTEPS) cur = nxt;
    }
  };

  // -inf on the keys of block kb that a row may not see (causal: key > query;
  // full attention: keys past the ragged end), both maps
  auto mask_block = [&](int kt, int kb, floatx16 (&s)[C::NBR][NQB]) __attribute__((always_inline)) {
    const int key0 = ptile(kt) * BC + kb * 32;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int query = q0 + qb * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        const bool masked = CAUSAL ? (key > query || (W > 0 && query - key >= W)) : (key >= T);
#pragma unroll
        for (int br = 0; br < C::NBR; ++br) s[br][qb][r] = masked ? kNegInf : s[br][qb][r];
      }
    }
  };

  // probabilities 2^(s - mu) rounded to bf16 (the B operand of the P.V
  // product) and each lane's sum over its 16 keys.  One-map waves sum the
  // fp32 values with adds (expo16); two-map waves, whose registers are
  // short, sum the rounded pairs with v_dot2 as they are produced.
  auto expo_one = [&](const floatx16& s, bf16x8 (&pk)[2], float& bsum) __attribute__((always_inline)) {
    if constexpr (C::NBR * NQB == 1) {
      bsum = expo16(s, pk);
    } else {
      const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
      float b = 0.0f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float pa = __builtin_amdgcn_exp2f(s[8 * ks + 2 * j]);
          const float pb = __builtin_amdgcn_exp2f(s[8 * ks + 2 * j + 1]);
          const bf16x2 pw = {(bf16)pa, (bf16)pb};
          b = __builtin_amdgcn_fdot2_f32_bf16(pw, ones, b, false);
          pk[ks][2 * j] = pw[0];
          pk[ks][2 * j + 1] = pw[1];
        }
      bsum = b;
    }
  };
  auto expo = [&](floatx16 (&s)[C::NBR][NQB], bf16x8 (&pk)[C::NBR][NQB][2], float (&bsum)[C::NBR][NQB])
      __attribute__((always_inline)) {
#pragma unroll
    for (int br = 0; br < C::NBR; ++br)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) expo_one(s[br][qb], pk[br][qb], bsum[br][qb]);
  };

  // Lazy rescale, after expo: the reference only moves when some probability
  // of the block would exceed 2^kTau (then the lane's partial sum does), or
  // while a row has not yet seen a key (seen[] false): the first block in
  // which it sees one sets mu to the exact row max.  Otherwise mu stays at or
  // below the running row max and within kTau of it from below, so every
  // p <= 2^kTau and the final row sum is >= 1.  The rare path rescales acc and
  // lsum and recomputes the block's probabilities.
  auto settle = [&](bool first, floatx16 (&s)[C::NBR][NQB], bf16x8 (&pk)[C::NBR][NQB][2],
                    float (&bsum)[C::NBR][NQB]) __attribute__((always_inline)) {
    bool need = false;
#pragma unroll
    for (int br = 0; br < C::NBR; ++br)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) need |= bsum[br][qb] > kRescaleSum;
    // without a window every row sees key 0, in the wave's first block
    if constexpr (WIN) {
#pragma unroll
      for (int br = 0; br < C::NBR; ++br)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) need |= !seen[br][qb];
    } else {
      need |= first;
    }
    if (__any(need)) {
#pragma unroll
      for (int br = 0; br < C::NBR; ++br)
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          float m = s[br][qb][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) m = fmaxf(m, s[br][qb][r]);
          m = swap_halves_max(m);  // block max of s - mu over the row's 32 keys
          // a row's first visible key sets the reference; afterwards it only
          // ever rises
          const bool had = WIN ? seen[br][qb] : !first;
          if constexpr (WIN) seen[br][qb] = had || m != kNegInf;
          const float delta = had ? fmaxf(m, 0.0f) : (m == kNegInf ? 0.0f : m);
          // before the row's first visible key its state is empty (nothing to
          // scale): 2^-delta could overflow there (delta = the block max, which
          // may lie far below zero) and 0 x inf would be NaN; afterwards
          // delta >= 0 and the factor is at most 1
          const float alpha = had ? __builtin_amdgcn_exp2f(-delta) : 1.0f;
          mu[br][qb] += delta;
          lsum[br][qb] *= alpha;
#pragma unroll
          for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[br][qb][cb][r] *= alpha;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if constexpr (C::NEGMU_REGS) negmu[br][qb][r] = -mu[br][qb];
            s[br][qb][r] -= delta;
          }
          expo_one(s[br][qb], pk[br][qb], bsum[br][qb]);
        }
    }
#pragma unroll
    for (int br = 0; br < C::NBR; ++br)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) lsum[br][qb] += bsum[br][qb];
  };

  // One V fragment of block kb (A operand of the P.V product): keys
  // 16 ks .. 16 ks + 15 of output columns 32 cb .. 32 cb + 31, read with two
  // transposing LDS reads from the row-major V tile
  auto vread = [&](int kb, const char* sb, int cb, int ks) __attribute__((always_inline)) {
    const char* base = sb + C::KT * C::KBYTES + (kb * 32 + 16 * ks + v_row) * (2 * C::DV) +
                       (((4 * cb + v_chunk) ^ v_sw) << 4) + v_byte;
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)base);
    const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(base + 8 * (2 * C::DV)));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
  };
  // acc += P^T-weighted V rows of block kb; each V fragment serves both maps
  auto pv = [&](int kb, const char* sb, const bf16x8 (&pk)[C::NBR][NQB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 av = vread(kb, sb, cb, ks);
#pragma unroll
        for (int br = 0; br < C::NBR; ++br)
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
            acc[br][qb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pk[br][qb][ks], acc[br][qb][cb], 0, 0, 0);
      }
  };

  // (PREF) the V fragments of block kb, read before the softmax, and the P.V
  // MFMAs that use them after it
  auto load_v = [&](int kb, const char* sb, bf16x8 (&vfr)[C::CB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) vfr[cb][ks] = vread(kb, sb, cb, ks);
  };
  // (PIPE) the P.V product with each V fragment read one MFMA ahead
  auto pv_pipe = [&](int kb, const char* sb, const bf16x8 (&pk)[C::NBR][NQB][2]) __attribute__((always_inline)) {
    bf16x8 cur = vread(kb, sb, 0, 0);
#pragma unroll
    for (int i = 0; i < 2 * C::CB; ++i) {
      bf16x8 nxt;
      if (i + 1 < 2 * C::CB) nxt = vread(kb, sb, (i + 1) / 2, (i + 1) % 2);
      __builtin_amdgcn_sched_barrier(0);
      acc[0][0][i / 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pk[0][0][i % 2], acc[0][0][i / 2], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < 2 * C::CB) cur = nxt;
    }
  };
  auto pv_early = [&](const bf16x8 (&vfr)[C::CB][2], const bf16x8 (&pk)[C::NBR][NQB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        acc[0][0][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[cb][ks], pk[0][0][ks], acc[0][0][cb], 0, 0, 0);
  };

  if (PD < ntiles) wait_vm_barrier<C::SEGW_MIN * (PD - 1)>();
  else wait_vm_barrier<0>();
  // ---- main loop: tile kt computed while tiles kt+1 .. kt+PD load ------------
  auto compute_tile = [&](int kt, const char* sb) __attribute__((always_inline)) {
    // whether any block of this tile crosses the causal diagonal (or the
    // ragged end) for this wave's rows
    const int tk0 = ptile(kt) * BC;
    const bool masked = CAUSAL ? (tk0 + BC - 1 > q0 || (W > 0 && tk0 <= q_last - W)) : (tk0 + BC > T);
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb) {
      // (with a window the live blocks need not be a prefix of the tile)
      if (!kb_live(kt, kb)) {
        if constexpr (WIN) continue;
        else break;
      }
      floatx16 s[C::NBR][NQB];
      bf16x8 pk[C::NBR][NQB][2];
      float bs[C::NBR][NQB];
      if constexpr (PREF) {
        bf16x8 vfr[C::CB][2];
        qk_early(kb, sb, s);
        load_v(kb, sb, vfr);
        __builtin_amdgcn_sched_barrier(0);
        if (masked) mask_block(kt, kb, s);
        expo(s, pk, bs);
        settle(kt == 0 && kb == 0, s, pk, bs);
        pv_early(vfr, pk);
      } else if constexpr (PIPE) {
        qk_pipe(kb, sb, s);
        if (masked) mask_block(kt, kb, s);
        expo(s, pk, bs);
        settle(kt == 0 && kb == 0, s, pk, bs);
        pv_pipe(kb, sb, pk);
      } else {
        qk(kb, sb, s);
        if (masked) mask_block(kt, kb, s);
        expo(s, pk, bs);
        settle(kt == 0 && kb == 0, s, pk, bs);
        pv(kb, sb, pk);
      }
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

  // The accumulators are normalised in place (acc * (1 / l), the same
  // product every consumer used before): the saved map, the exchanged map and
  // the output then read one set of registers.  Forming acc * inv separately
  // for each consumer made the compiler keep a second full copy live across
  // the training-forward branch (spills at D = 128).
  auto normalise = [&](floatx16 (&ac)[C::CB], float inv) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) ac[cb][r] = ac[cb][r] * inv;
  };
  // training forward: map br's normalised output and its log-sum-exp
  auto save_map = [&](int br, int query, float m, float l, const floatx16 (&ac)[C::CB])
      __attribute__((always_inline)) {
    if (a.save_o1 == nullptr || query >= T) return;
    float* dst = (br ? a.save_o2 : a.save_o1) + o_off + (size_t)query * C::DV;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 t = {ac[cb][4 * g], ac[cb][4 * g + 1], ac[cb][4 * g + 2], ac[cb][4 * g + 3]};
        *(floatx4*)(dst + cb * 32 + 8 * g + 4 * hi) = t;
      }
    if (hi == 0) a.save_lse[((size_t)bh * 2 + br) * T + query] = m + __log2f(l);
  };

  // ---- split mode: map-2 waves hand t2 = acc2 / l2 to their map-1 partners ----
  float* const xch = (float*)smem;
  if constexpr (SPLIT) {
    if (wbr == 1 && wave_active) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const float l2 = swap_halves_sum(lsum[0][qb]);
        normalise(acc[0][qb], 1.0f / l2);
        save_map(1, q0 + qb * 32 + l32, mu[0][qb], l2, acc[0][qb]);
        float* row = xch + (wq * C::QPW + qb * 32 + l32) * C::XP;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const floatx4 t = {acc[0][qb][cb][4 * g], acc[0][qb][cb][4 * g + 1], acc[0][qb][cb][4 * g + 2],
                               acc[0][qb][cb][4 * g + 3]};
            *(floatx4*)(row + cb * 32 + 8 * g + 4 * hi) = t;
          }
      }
    }
    __syncthreads();
    if (wbr == 1) return;
  }
  if (!wave_active) return;

  // ---- epilogue: combine the maps, optional head norm, store -----------------
  bf16* __restrict__ O = (bf16*)a.out + (bb * a.sb[5] + h * a.sh[5]);
  // rows staged through LDS for whole-row stores: split waves use their own
  // exchange rows (already read by then), other shapes a slice of the free
  // tile ring per wave, where that fits
  constexpr int NCH = C::DV / 8;  // 16-byte columns per output row
  constexpr bool STAGE_OUT = SPLIT ? (2 * C::DV <= 4 * C::XP) : (NW * NQB * 32 * 2 * C::DV <= C::SMEM);
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int query = q0 + qb * 32 + l32;
    const float l1 = swap_halves_sum(lsum[0][qb]);
    normalise(acc[0][qb], 1.0f / l1);
    if constexpr (MAPS == 2) save_map(0, query, mu[0][qb], l1, acc[0][qb]);
    if constexpr (!SPLIT && MAPS == 2) {
      const float l2 = swap_halves_sum(lsum[1][qb]);
      normalise(acc[1][qb], 1.0f / l2);
      save_map(1, query, mu[1][qb], l2, acc[1][qb]);
    }
    const float* xrow = xch + (wq * C::QPW + qb * 32 + l32) * C::XP;
    // the output is formed in place in map 1's accumulators
    floatx16 (&o)[C::CB] = acc[0][qb];
    if constexpr (MAPS == 2) {
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // t1 - lam * t2 with both maps rounded identically (no contraction)
          float t2;
          if constexpr (SPLIT) t2 = xrow[cb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3)];
          else t2 = acc[C::NBR - 1][qb][cb][r];
          const float lt2 = lamv * t2;
          o[cb][r] = o[cb][r] - lt2;
        }
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
    if constexpr (STAGE_OUT) {
      // The lane layout holds 8 bytes of a row per 16-byte column, so direct
      // stores touch 32 rows per instruction.  Instead the wave writes its
      // 32 rows to its own LDS rows (16-byte columns XOR-swizzled by the row,
      // conflict-free both ways), then stores whole rows: 16-byte lanes,
      // NCH lanes per row.
      char* stg = SPLIT ? (char*)(xch + (wq * C::QPW + qb * 32) * C::XP)
                        : smem + (wave * NQB + qb) * 32 * (2 * C::DV);
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const bf16x4 v4 = {(bf16)o[cb][4 * g], (bf16)o[cb][4 * g + 1], (bf16)o[cb][4 * g + 2],
                             (bf16)o[cb][4 * g + 3]};
          const int col = (4 * cb + g) ^ (l32 & (NCH - 1));
          *(bf16x4*)(stg + l32 * (2 * C::DV) + col * 16 + hi * 8) = v4;
        }
      constexpr int RPI = 64 / NCH;  // rows per store instruction
#pragma unroll
      for (int i = 0; i < 32 / RPI; ++i) {
        const int r = i * RPI + lane / NCH;
        const int c = lane % NCH;
        const u32x4 w4 = *(const u32x4*)(stg + r * (2 * C::DV) + ((c ^ (r & (NCH - 1))) << 4));
        const int row = q0 + qb * 32 + r;
        if (row < T) *(u32x4*)(O + (size_t)row * a.sr[5] + c * 8) = w4;
      }
    } else if (query < T) {
      bf16* dst = O + (size_t)query * a.sr[5];
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

// ============================================================================
// bf16 two-map prefill with the two waves of each SIMD in opposite phases
// ============================================================================
//
// Per 32-key block a wave has a matrix phase (the P.V products of the previous
// block, then the score products of this block: 24 MFMAs at D = 64) and a
// vector phase (mask, exponentials, bf16 rounding, row sums, the rare
// rescale, then the V fragments of this block read ahead for the next matrix
// phase).  Eight waves share a compute unit, two per SIMD.  If both waves of a
// SIMD reach their vector phase together, the matrix core idles meanwhile;
// here the second wave of each SIMD starts one phase late (one extra barrier
// before its first phase, the first wave one extra after its last) and a
// workgroup barrier separates consecutive phases, so while one wave issues
// MFMAs the other runs its exponentials.  The matrix-phase wave runs at raised
// issue priority.
//
// Tiles of 64 keys (K1, K2, V) go global -> LDS by DMA into a four-stage ring.
// Block b reads its K tile in its matrix phase and its V tile at the end of
// its vector phase, so tile t is read in the wave's phases 4t .. 4t+3, i.e.
// between barriers 4t and 4t+5 counting both wave groups.  A wave's share of
// tile u is issued in two halves at the start of the vector phases of blocks
// 2u-5 and 2u-4 (phases 4u-9 and 4u-7) into stage u % 4, after every read of
// tile u-4; the vector phase has slack, the matrix phase none, and spreading
// the issue keeps four waves from queueing all their loads at one moment.
// Each wave waits for its own loads of tile u at the end of the matrix phase
// of block 2u-1 (phase 4u-2), before the barrier that publishes it for phase
// 4u.
template <int D, bool CAUSAL, bool HEADNORM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_pp_kernel(FwdArgs a) {
  constexpr int NW = 8, NSTAGE = 4;
  using C = CfgB<D, 1, NW, NSTAGE, false>;
  constexpr int BC = C::BC;
  constexpr int SEGW = C::NSEG / NW;
  static_assert(C::NSEG % NW == 0 && SEGW % 2 == 0 && SEGW <= 4, "every wave issues the same even number of tile loads");
  static_assert(2 * SEGW <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[C::SMEM];
  __shared__ int simd_of[NW];
  lds_poison(smem, sizeof(smem));
  lds_poison(simd_of, sizeof(simd_of));
  lds_poison_done();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int T = a.T;

  const int nqt = (T + C::BR - 1) / C::BR;
  const int w = xcd_remap(blockIdx.x, a.B * a.H * nqt);
  int bh_, qi_;
  if (CAUSAL) causal_order(w, a.B * a.H * nqt, nqt, bh_, qi_);
  else bh_ = w / nqt, qi_ = w % nqt;
  const int bh = __builtin_amdgcn_readfirstlane(bh_);
  const int qi = __builtin_amdgcn_readfirstlane(qi_);
  const int qt = CAUSAL ? (nqt - 1 - qi) : qi;  // heaviest causal tiles first
  const int h = bh % a.H;
  const int bb = bh / a.H;
  const size_t o_off = (size_t)bh * T * C::DV;
  const bf16* __restrict__ Q1 = (const bf16*)a.q1 + (bb * a.sb[0] + h * a.sh[0]);
  const bf16* __restrict__ Q2 = (const bf16*)a.q2 + (bb * a.sb[2] + h * a.sh[2]);
  const bf16* __restrict__ K1 = scalar_ptr((const bf16*)a.k1 + (bb * a.sb[1] + h * a.sh[1]));
  const bf16* __restrict__ K2 = scalar_ptr((const bf16*)a.k2 + (bb * a.sb[3] + h * a.sh[3]));
  const bf16* __restrict__ V = scalar_ptr((const bf16*)a.v + (bb * a.sb[4] + h * a.sh[4]));
  const int rq[2] = {a.sr[0], a.sr[2]};
  const uint32_t rk_b[2] = {2u * (uint32_t)a.sr[1], 2u * (uint32_t)a.sr[3]};
  const uint32_t rv_b = 2u * (uint32_t)a.sr[4];

  const int q_tile0 = qt * C::BR;
  const int q0 = q_tile0 + wave * 32;
  const int q_last = min(q0 + 32, T) - 1;
  const int k_end = CAUSAL ? min(T, q_tile0 + C::BR) : T;
  const int ntiles = (k_end + BC - 1) / BC;
  const int nblk = (k_end + 31) / 32;
  const float sc = a.score_scale;
  const float lamv = head_lambda(a, h, qt, bh);
  asm volatile("" ::"v"(lamv));

  // ---- tile loads (as in fwd_bf16_kernel) -------------------------------------
  constexpr int CK = D / 8, RK = 64 / CK, CV = C::DV / 8, RV = 64 / CV;
  const int rl_k = lane / CK, rl_v = lane / CV;
  // this wave's load slot i of tile kt: segment wave + i NW of the stage,
  // K1 and K2 segments first, then V.  When every wave's slot i is of the
  // same kind (the K segment count a multiple of NW), the kind is known at
  // compile time and the issue has no branches.
  auto issue_slot = [&](int kt, auto slot) __attribute__((always_inline)) {
    constexpr int i = decltype(slot)::value;
    char* sb = smem + (kt & (NSTAGE - 1)) * C::STAGE;
    const int key0 = kt * BC;
    const int seg = wave + i * NW;
    constexpr bool uniform_kind = C::KSEG % NW == 0;
    const bool isk = uniform_kind ? (i * NW < 2 * C::KSEG) : (seg < 2 * C::KSEG);
    if (isk) {
      const int which = uniform_kind ? (i * NW) / C::KSEG : seg / C::KSEG;
      const int g = seg % C::KSEG;
      const int r = g * RK + rl_k;
      const int c = (lane % CK) ^ swz_k<D>(r);
      const uint32_t row = (uint32_t)min(key0 + r, T - 1);
      dma16(which ? K2 : K1, row * rk_b[which] + c * 16, sb + which * C::KBYTES + g * 1024);
    } else {
      const int g = seg - 2 * C::KSEG;
      const int r = g * RV + rl_v;
      const int c = (lane % CV) ^ swz_v<C::DV>(r);
      const uint32_t row = (uint32_t)min(key0 + r, T - 1);
      dma16(V, row * rv_b + c * 16, sb + 2 * C::KBYTES + g * 1024);
    }
  };
  auto issue = [&](int kt) __attribute__((always_inline)) {
    issue_slot(kt, std::integral_constant<int, 0>{});
    if constexpr (SEGW > 1) issue_slot(kt, std::integral_constant<int, 1>{});
    if constexpr (SEGW > 2) issue_slot(kt, std::integral_constant<int, 2>{});
    if constexpr (SEGW > 3) issue_slot(kt, std::integral_constant<int, 3>{});
  };
  // wait until at most n (0, 1 or 2) tiles of this wave's loads are in flight
  auto wait_tiles = [&](int n) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    if (n >= 2) __builtin_amdgcn_s_waitcnt(((2 * SEGW) & 15) | ((((2 * SEGW) >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
    else if (n == 1) __builtin_amdgcn_s_waitcnt((SEGW & 15) | (((SEGW >> 4) & 3) << 14) | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
  };
  auto phase_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- Q fragments (B operand of S^T = K Q^T), pre-scaled by log2(e)/sqrt(D) --
  bf16x8 qf[2][C::KSTEPS];
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    const int query = q0 + l32;
    const bool ok = query < T;
    const bf16* src = (br ? Q2 : Q1) + (size_t)min(query, T - 1) * rq[br];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
      u32x4 raw = *(const u32x4*)(src + ks * 16 + hi * 8);
      raw = ok ? raw : u32x4{0u, 0u, 0u, 0u};
      const bf16x8 q = __builtin_bit_cast(bf16x8, raw);
      bf16x8 qs;
#pragma unroll
      for (int e = 0; e < 8; ++e) qs[e] = (bf16)((float)q[e] * sc);
      qf[br][ks] = qs;
    }
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): Q in registers

  // prologue: tiles 0, 1, 2; tile 0 is published by the barrier below, which
  // also publishes each wave's SIMD number
  issue(0);
  if (1 < ntiles) issue(1);
  if (2 < ntiles) issue(2);
  if (lane == 0) simd_of[wave] = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4) & 3;  // HW_ID.SIMD_ID
  wait_tiles(min(ntiles, 3) - 1);
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));  // lgkmcnt(0) only: the SIMD number is in LDS
  phase_barrier();
  // the later of the two waves on this SIMD (by wave number) runs one phase late
  int late = 0;
  {
    const int mine = simd_of[wave];
#pragma unroll
    for (int j = 0; j < NW; ++j) late += (j < wave && simd_of[j] == mine) ? 1 : 0;
    late = __builtin_amdgcn_readfirstlane(late & 1);
  }

  floatx16 acc[2][C::CB];
  float mu[2], lsum[2];
#pragma unroll
  for (int br = 0; br < 2; ++br) {
    mu[br] = 0.0f;
    lsum[br] = 0.0f;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[br][cb][r] = 0.0f;
  }

  const int k_rd = l32 * (2 * D);
  const int swk = swz_k<D>(l32);
  const int vq = lane & 3;
  const int vkq = (lane >> 2) & 3;
  const int v_row = 4 * hi + vkq;
  const int v_chunk = 2 * ((lane >> 4) & 1) + (vq >> 1);
  const int v_sw = swz_v<C::DV>(vkq);
  const int v_byte = (vq & 1) * 8;

  auto stage_of = [&](int b) __attribute__((always_inline)) -> const char* {
    return smem + ((b >> 1) & (NSTAGE - 1)) * C::STAGE + (b & 1) * 32 * (2 * D);
  };
  auto vstage_of = [&](int b) __attribute__((always_inline)) -> const char* {
    return smem + ((b >> 1) & (NSTAGE - 1)) * C::STAGE + 2 * C::KBYTES + (b & 1) * 32 * (2 * C::DV);
  };

  auto mask_block = [&](int b, floatx16 (&s)[2]) __attribute__((always_inline)) {
    const int key0 = b * 32;
    const int query = q0 + l32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      const bool masked = CAUSAL ? (key > query) : (key >= T);
#pragma unroll
      for (int br = 0; br < 2; ++br) s[br][r] = masked ? kNegInf : s[br][r];
    }
  };
  auto expo_one = [&](const floatx16& s, bf16x8 (&pk)[2], float& bsum) __attribute__((always_inline)) {
    bsum = expo16(s, pk);
  };
  // lazy rescale (as in fwd_bf16_kernel): the reference moves only when a
  // probability of the block could exceed 2^kTau, or on the first block
  auto settle = [&](bool first, floatx16 (&s)[2], bf16x8 (&pk)[2][2], float (&bsum)[2]) __attribute__((always_inline)) {
    bool need = first;
#pragma unroll
    for (int br = 0; br < 2; ++br) need |= bsum[br] > kRescaleSum;
    if (__any(need)) {
#pragma unroll
      for (int br = 0; br < 2; ++br) {
        float m = s[br][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) m = fmaxf(m, s[br][r]);
        m = swap_halves_max(m);
        const float delta = first ? (m == kNegInf ? 0.0f : m) : fmaxf(m, 0.0f);
        // the first block finds the state empty: no scaling (2^-delta could
        // overflow for a block max far below zero, and 0 x inf is NaN)
        const float alpha = first ? 1.0f : __builtin_amdgcn_exp2f(-delta);
        mu[br] += delta;
        lsum[br] *= alpha;
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[br][cb][r] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[br][r] -= delta;
        expo_one(s[br], pk[br], bsum[br]);
      }
    }
#pragma unroll
    for (int br = 0; br < 2; ++br) lsum[br] += bsum[br];
  };
  auto load_vf = [&](int b, bf16x8 (&vf)[C::CB][2]) __attribute__((always_inline)) {
    const char* vb = vstage_of(b) + v_row * (2 * C::DV) + v_byte;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* base = vb + 16 * ks * (2 * C::DV) + (((4 * cb + v_chunk) ^ v_sw) << 4);
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)base);
        const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(base + 8 * (2 * C::DV)));
        vf[cb][ks] = bf16x8{lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
      }
  };
  auto pv = [&](int cb0, int ncb, const bf16x8 (&vf)[C::CB][2], const bf16x8 (&pk)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = cb0; cb < cb0 + ncb; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int br = 0; br < 2; ++br)
          acc[br][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[cb][ks], pk[br][ks], acc[br][cb], 0, 0, 0);
  };
  // matrix phase: the P.V product of the previous block in two halves, the
  // first half's freed registers taking the K fragments of the first half of
  // the score product, then the score products, the second half's K
  // fragments read into the first half's registers.  The order is pinned so
  // that the reads fly behind independent MFMAs and no more than 48
  // registers of fragments, probabilities and scores are live at once (the
  // budget of two waves per SIMD).
  bf16x8 kf[C::KSTEPS / 2][2];
  constexpr int KH = C::KSTEPS / 2, CH = C::CB / 2;
  auto qk_half = [&](int b, int ks0, floatx16 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < KH; ++k)
#pragma unroll
      for (int br = 0; br < 2; ++br) {
        const int ks = ks0 + k;
        s[br] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k][br], qf[br][ks], ks > 0 ? s[br] : splat16(-mu[br]), 0, 0, 0);
      }
  };
  auto load_kf_half = [&](int b, int ks0) __attribute__((always_inline)) {
    const char* kb = stage_of(b) + k_rd;
#pragma unroll
    for (int k = 0; k < KH; ++k)
#pragma unroll
      for (int br = 0; br < 2; ++br)
        kf[k][br] = *(const bf16x8*)(kb + br * C::KBYTES + (((2 * (ks0 + k) + hi) ^ swk) << 4));
  };
  auto matrix_phase = [&](int b, bool do_pv, bool do_qk, const bf16x8 (&vf)[C::CB][2],
                          const bf16x8 (&pk)[2][2], floatx16 (&s)[2]) __attribute__((always_inline)) {
    if (do_pv) pv(0, CH, vf, pk);
    __builtin_amdgcn_sched_barrier(0);
    if (do_qk) load_kf_half(b, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (do_pv) pv(CH, C::CB - CH, vf, pk);
    __builtin_amdgcn_sched_barrier(0);
    if (do_qk) {
      qk_half(b, 0, s);
      __builtin_amdgcn_sched_barrier(0);
      load_kf_half(b, KH);
      __builtin_amdgcn_sched_barrier(0);
      qk_half(b, KH, s);
    }
  };

  // ---- main loop: phase 2b = matrix phase of block b, 2b+1 = its vector phase
  // Every wave of the workgroup runs the phases of all nblk blocks; a wave's
  // live blocks (keys it may see) are a prefix [0, n_live), after which it
  // only issues its share of the tile loads and joins the barriers.
  const int n_live = q0 < T ? (CAUSAL ? q_last / 32 + 1 : nblk) : 0;
  // vector phase of block b: half of this wave's share of tile (b+5)/2
  auto dma_issue = [&](int b) __attribute__((always_inline)) {
    const int u = (b + 5) >> 1;
    if (u >= 3 && u < ntiles) {
      if (b & 1) {
        issue_slot(u, std::integral_constant<int, 0>{});
        if constexpr (SEGW == 4) issue_slot(u, std::integral_constant<int, 1>{});
      } else {
        issue_slot(u, std::integral_constant<int, SEGW / 2>{});
        if constexpr (SEGW == 4) issue_slot(u, std::integral_constant<int, 3>{});
      }
    }
  };
  // end of the matrix phase of block b (odd): tile (b+1)/2 complete for this
  // wave; tile (b+3)/2, issued since, stays in flight
  auto dma_wait = [&](int b) __attribute__((always_inline)) {
    if (b & 1) {
      const int u = (b + 1) >> 1;
      if (u < ntiles) wait_tiles(u + 1 < ntiles ? 1 : 0);
    }
  };
  bf16x8 pk[2][2];
  bf16x8 vf[C::CB][2];
  floatx16 s[2];
  auto vector_phase = [&](int b, bool first) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(0);
    dma_issue(b);
    const int key0 = b * 32;
    if (CAUSAL ? (key0 + 31 > q0) : (key0 + 32 > T)) mask_block(b, s);
    float bs[2];
    expo_one(s[0], pk[0], bs[0]);
    expo_one(s[1], pk[1], bs[1]);
    settle(first, s, pk, bs);
    __builtin_amdgcn_sched_barrier(0);
    load_vf(b, vf);
  };
  if (late) phase_barrier();
  int b = 0;
  if (n_live > 0) {
    __builtin_amdgcn_s_setprio(1);
    matrix_phase(0, false, true, vf, pk, s);
    phase_barrier();
    vector_phase(0, true);
    phase_barrier();
    for (b = 1; b < n_live; ++b) {
      __builtin_amdgcn_s_setprio(1);
      matrix_phase(b, true, true, vf, pk, s);
      dma_wait(b);
      phase_barrier();
      vector_phase(b, false);
      phase_barrier();
    }
    // matrix phase n_live: the last block's P.V product only
    __builtin_amdgcn_s_setprio(1);
    matrix_phase(b, true, false, vf, pk, s);
    dma_wait(b);
  }
  __builtin_amdgcn_s_setprio(0);
  // the rest of the workgroup's phases: tile loads and barriers only
  for (int c = b; c < nblk; ++c) {
    phase_barrier();  // end of matrix phase c
    dma_issue(c);     // vector phase c
    phase_barrier();
    dma_wait(c + 1);  // matrix phase c+1
  }
  if (!late) phase_barrier();
  if (q0 >= T) return;

  // ---- epilogue: combine the maps, optional head norm, store -----------------
  // maps normalised in place (one product per element, read by the saved
  // map and the output alike), as in fwd_bf16_kernel
  auto save_map = [&](int br, int query, float m, float l, const floatx16 (&ac)[C::CB])
      __attribute__((always_inline)) {
    if (a.save_o1 == nullptr || query >= T) return;
    float* dst = (br ? a.save_o2 : a.save_o1) + o_off + (size_t)query * C::DV;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const floatx4 t = {ac[cb][4 * g], ac[cb][4 * g + 1], ac[cb][4 * g + 2], ac[cb][4 * g + 3]};
        *(floatx4*)(dst + cb * 32 + 8 * g + 4 * hi) = t;
      }
    if (hi == 0) a.save_lse[((size_t)bh * 2 + br) * T + query] = m + __log2f(l);
  };
  bf16* __restrict__ O = (bf16*)a.out + (bb * a.sb[5] + h * a.sh[5]);
  const int query = q0 + l32;
  const float l1 = swap_halves_sum(lsum[0]);
  const float l2 = swap_halves_sum(lsum[1]);
  const float inv1 = 1.0f / l1;
  const float inv2 = 1.0f / l2;
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc[0][cb][r] = acc[0][cb][r] * inv1;
      acc[1][cb][r] = acc[1][cb][r] * inv2;
    }
  save_map(0, query, mu[0], l1, acc[0]);
  save_map(1, query, mu[1], l2, acc[1]);
  floatx16 (&o)[C::CB] = acc[0];
#pragma unroll
  for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // t1 - lam * t2 with both maps rounded identically (no contraction)
      const float lt2 = lamv * acc[1][cb][r];
      o[cb][r] = o[cb][r] - lt2;
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
    bf16* dst = O + (size_t)query * a.sr[5];
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

template <int D>
hipError_t launch_pp(const FwdArgs& a, bool causal, bool headnorm, hipStream_t stream) {
  using C = CfgB<D, 1, 8, 4, false>;
  const long nqt = (a.T + C::BR - 1) / C::BR;
  const long grid = (long)a.B * a.H * nqt;
  if (!grid_fits(grid, C::NT)) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), b(C::NT);
  if (causal) {
    if (headnorm) fwd_pp_kernel<D, true, true><<<g, b, 0, stream>>>(a);
    else fwd_pp_kernel<D, true, false><<<g, b, 0, stream>>>(a);
  } else {
    if (headnorm) fwd_pp_kernel<D, false, true><<<g, b, 0, stream>>>(a);
    else fwd_pp_kernel<D, false, false><<<g, b, 0, stream>>>(a);
  }
  return hipGetLastError();
}

template <int D, int NQB, int NW, int NSTAGE, bool SPLIT>
hipError_t launch_bf16(const FwdArgs& a, bool causal, bool headnorm, hipStream_t stream) {
  using C = CfgB<D, NQB, NW, NSTAGE, SPLIT>;
  const long nqt = (a.T + C::BR - 1) / C::BR;
  const long grid = (long)a.B * a.H * nqt;
  if (!grid_fits(grid, C::NT)) return hipErrorInvalidConfiguration;
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

template <int D, int NQB, int NW, int NSTAGE, bool SPLIT>
hipError_t launch_window(const FwdArgs& a, bool headnorm, hipStream_t stream) {
  using C = CfgB<D, NQB, NW, NSTAGE, SPLIT>;
  const long nqt = (a.T + C::BR - 1) / C::BR;
  const long grid = (long)a.B * a.H * nqt;
  if (!grid_fits(grid, C::NT)) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), b(C::NT);
  if (headnorm) fwd_bf16_kernel<D, NQB, NW, NSTAGE, SPLIT, true, true, 2, false, true><<<g, b, 0, stream>>>(a);
  else fwd_bf16_kernel<D, NQB, NW, NSTAGE, SPLIT, true, false, 2, false, true><<<g, b, 0, stream>>>(a);
  return hipGetLastError();
}

template <int D, int NQB, int NW, int NSTAGE, bool SPLIT>
hipError_t launch_v2_d(const FwdArgs& a, bool causal, hipStream_t stream) {
  using C = CfgB<D, NQB, NW, NSTAGE, SPLIT, 2, true>;
  const long nqt = (a.T + C::BR - 1) / C::BR;
  const long grid = (long)a.B * a.H * nqt;
  if (!grid_fits(grid, C::NT)) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), b(C::NT);
  if (causal) fwd_bf16_kernel<D, NQB, NW, NSTAGE, SPLIT, true, false, 2, true><<<g, b, 0, stream>>>(a);
  else fwd_bf16_kernel<D, NQB, NW, NSTAGE, SPLIT, false, false, 2, true><<<g, b, 0, stream>>>(a);
  return hipGetLastError();
}

template <int D, int NQB, int NW, int NSTAGE>
hipError_t launch_std(const FwdArgs& a, bool causal, hipStream_t stream) {
  using C = CfgB<D, NQB, NW, NSTAGE, false, 1>;
  const long nqt = (a.T + C::BR - 1) / C::BR;
  const long grid = (long)a.B * a.H * nqt;
  if (!grid_fits(grid, C::NT)) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), b(C::NT);
  if (causal) fwd_bf16_kernel<D, NQB, NW, NSTAGE, false, true, false, 1><<<g, b, 0, stream>>>(a);
  else fwd_bf16_kernel<D, NQB, NW, NSTAGE, false, false, false, 1><<<g, b, 0, stream>>>(a);
  return hipGetLastError();
}

template <int D, int NQB, int NW, int BC, bool SPLIT>
hipError_t launch_f32(const FwdArgs& a, bool causal, bool headnorm, hipStream_t stream) {
  using C = Cfg<D, NQB, NW, BC, SPLIT>;
  const long nqt = (a.T + C::BR - 1) / C::BR;
  const long grid = (long)a.B * a.H * nqt;
  if (!grid_fits(grid, C::NT)) return hipErrorInvalidConfiguration;
  const dim3 g((unsigned)grid), b(C::NT);
  if (causal) {
    if (headnorm) fwd_f32_kernel<D, NQB, NW, BC, SPLIT, true, true><<<g, b, 0, stream>>>(a);
    else fwd_f32_kernel<D, NQB, NW, BC, SPLIT, true, false><<<g, b, 0, stream>>>(a);
  } else {
    if (headnorm) fwd_f32_kernel<D, NQB, NW, BC, SPLIT, false, true><<<g, b, 0, stream>>>(a);
    else fwd_f32_kernel<D, NQB, NW, BC, SPLIT, false, false><<<g, b, 0, stream>>>(a);
  }
  return hipGetLastError();
}

// Compute units of the current device (256 on MI355X); used only to pick a
// launch shape, so a failed query falls back to that value.
long compute_units() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 256;
  return cus;
}

}  // namespace

hipError_t launch_v2(const FwdArgs& a, int D, bool causal, hipStream_t stream) {
  switch (D) {
    case 64:
      // Short causal rows: one map per wave, in 128- or 192-row workgroups
      // by the rule launch_fwd applies to D = 64 causal rows (B2 H16 T4096:
      // 0.223 -> 0.164 ms; B4 H32 T1024: 0.076 -> 0.068 ms).  Otherwise both
      // maps per wave: K and V fragments each serve two MFMAs.
      if (causal && a.T <= 4096) {
        const long wg128 = (long)a.B * a.H * ((a.T + 127) / 128);
        const long cus = compute_units();
        if (wg128 <= cus || (a.T > 2048 && wg128 <= 4 * cus)) return launch_v2_d<64, 1, 8, 3, true>(a, causal, stream);
        return launch_v2_d<64, 1, 12, 3, true>(a, causal, stream);
      }
      return launch_v2_d<64, 1, 8, 3, false>(a, causal, stream);
    // one map per wave (registers: the accumulators alone take 64 VGPRs per map)
    case 128: return launch_v2_d<128, 1, 8, 3, true>(a, causal, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attention(const FwdArgs& a, int D, bool causal, hipStream_t stream) {
  switch (D) {
    case 64: return launch_std<64, 1, 8, 3>(a, causal, stream);
    case 128:
      // Short causal rows: 128-row workgroups of four waves, two LDS stages
      // (two workgroups per CU) even out the causal triangle (B2 H16 T4096:
      // 0.189 -> 0.170 ms); longer causal rows: 384-row workgroups at three
      // waves per SIMD (168 registers, 16 bytes of spills; B1 H16 T32768:
      // 3.92 -> 3.79 ms); full attention: 256 rows, two waves per SIMD.
      if (causal && a.T <= 4096) return launch_std<128, 1, 4, 2>(a, causal, stream);
      if (causal) return launch_std<128, 1, 12, 3>(a, causal, stream);
      return launch_std<128, 1, 8, 3>(a, causal, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int D, bool causal, bool headnorm,
                      hipStream_t stream) {
  if (dtype == 1 && a.window > 0) {  // causal sliding window (bf16)
    switch (D) {
      case 32: {
        // With at least four 192-row workgroups per compute unit, one map per
        // wave at three waves per SIMD hides more latency (T = 32768, W =
        // 4096, 16 heads: 1.065 -> 0.961 ms; T = 8192, W = 1024, 32 heads:
        // 0.186 -> 0.180 ms); with fewer, both maps per wave.
        const long wg192 = (long)a.B * a.H * ((a.T + 191) / 192);
        if (wg192 >= 4 * compute_units()) return launch_window<32, 1, 12, 3, true>(a, headnorm, stream);
        return launch_window<32, 1, 8, 3, false>(a, headnorm, stream);
      }
      case 64: {
        // One map per wave.  With at least two 192-row workgroups per compute
        // unit, three waves per SIMD hide more latency than two (T = 32768,
        // W = 4096, 16 heads: 1.57 -> 1.50 ms, also 4.9% ahead of both maps
        // per wave in 256-row workgroups there; T = 8192, W = 1024, 32 heads:
        // 4.8%); with fewer, the 128-row workgroups with early reads.
        const long wg192 = (long)a.B * a.H * ((a.T + 191) / 192);
        if (wg192 >= 2 * compute_units()) return launch_window<64, 1, 12, 3, true>(a, headnorm, stream);
        return launch_window<64, 1, 8, 3, true>(a, headnorm, stream);
      }
      case 128: return launch_window<128, 1, 8, 2, true>(a, headnorm, stream);
    }
    return hipErrorInvalidValue;
  }
  if (dtype == 1) {  // bf16
    switch (D) {
      case 32:
        // Causal rows beyond 2048 keys: one map per wave in 128- or 192-row
        // workgroups (the rule of D = 64 below), which even out the causal
        // triangle that 256-row two-map workgroups leave uneven (B2 H16
        // T4096: 0.204 -> 0.140 ms).  Shorter causal rows and full attention
        // keep both maps per wave, where each fragment read feeds two MFMAs.
        if (causal && a.T > 2048) {
          const long wg128 = (long)a.B * a.H * ((a.T + 127) / 128);
          if (wg128 <= 4 * compute_units()) return launch_bf16<32, 1, 8, 3, true>(a, causal, headnorm, stream);
          return launch_bf16<32, 1, 12, 3, true>(a, causal, headnorm, stream);
        }
        return launch_bf16<32, 1, 8, 3, false>(a, causal, headnorm, stream);
      case 64:
        // Short causal rows run one map per wave.  With few workgroups per
        // compute unit the finer 128-row workgroups (two waves per SIMD)
        // balance the causal triangle better; otherwise 192-row workgroups
        // with three waves per SIMD hide more latency (measured on MI355X
        // over T = 2048 / 4096 and 8 .. 64 heads).  Long causal rows run both
        // maps per wave with the two waves of each SIMD in opposite phases
        // (fwd_pp_kernel); full attention runs both maps per wave (0.6-4.4%
        // ahead of one map over 64 rows per wave, bit-identical).
        if (causal && a.T <= 4096) {
          const long wg128 = (long)a.B * a.H * ((a.T + 127) / 128);
          const long cus = compute_units();
          if (wg128 <= cus || (a.T > 2048 && wg128 <= 4 * cus))
            return launch_bf16<64, 1, 8, 3, true>(a, causal, headnorm, stream);
          return launch_bf16<64, 1, 12, 3, true>(a, causal, headnorm, stream);
        }
        if (causal) return launch_pp<64>(a, causal, headnorm, stream);
        return launch_bf16<64, 1, 8, 3, false>(a, causal, headnorm, stream);
      case 128: return launch_bf16<128, 1, 8, 2, true>(a, causal, headnorm, stream);
    }
  } else {  // fp32
    // Eight waves (two per SIMD) wherever their registers fit in 256: with
    // one wave per SIMD nothing hides a wave's LDS reads and softmax behind
    // another wave's MFMAs.  One map per wave except for D = 32 full
    // attention, whose 256-row two-map workgroups carry equal work and read
    // each K/V tile once for both maps; D = 128 needs one wave per SIMD
    // (its accumulators and Q fragments alone take 192 registers).
    switch (D) {
      case 32:
        if (causal) return launch_f32<32, 1, 8, 128, true>(a, causal, headnorm, stream);
        return launch_f32<32, 1, 8, 64, false>(a, causal, headnorm, stream);
      case 64: return launch_f32<64, 1, 8, 64, true>(a, causal, headnorm, stream);
      case 128: return launch_f32<128, 1, 4, 32, true>(a, causal, headnorm, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace diffattn
