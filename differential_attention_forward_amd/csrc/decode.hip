// Differential-attention decode for gfx950: one new query per (batch, head)
// against a KV cache of L rows, no mask.
//
// It computes the same O = (softmax(q1 K1^T / sqrt(D)) - lam softmax(q2 K2^T /
// sqrt(D))) V as the prefill path for a single query row (paperleet
// "Differential Transformer Attention", equation for A1, A2, O), with the
// optional RMS head norm and x (1 - lambda_init) (aifetchly "Differential
// Transformer: Canceling LLM Attention Noise", section 4).  The French lesson
// page ("Le problème", "V1 contre V2") names the decode cost of the first
// version: the value cache was loaded twice per step.  Here each cache byte is
// read once: K1 and K2 once for the two score vectors, V once for both
// weighted sums.
//
// Split-K: the cache is cut into S chunks; decode_partial_kernel turns each
// (b, h, chunk) into two partial softmax states (running max m, sum l and the
// 2D-wide weighted sum of V rows, one state per map), written to an fp32
// workspace; decode_reduce_kernel then merges the S states of each (b, h) in
// a fixed order (deterministic), combines the two maps, applies the optional
// norm and stores the output row.  Stream order between the two launches is
// the cross-workgroup barrier.
//
// Inside a chunk a workgroup walks sub-chunks of kSub keys: first all scores
// of the sub-chunk (8-lane groups each own one key row, 16-byte coalesced
// loads, dot products reduced across the group), then one block-wide max per
// map, the exponentials, and finally the V pass (each lane owns 8 channels of
// a V row).  Partial state is rescaled only when a sub-chunk raises the max.
// Cache rows are read exactly once, with nontemporal 16-byte loads (no reuse
// to keep in L2), eight in flight per lane.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace diffattn {
namespace {

constexpr int kThreads = kDecodeThreads;
constexpr int kWaves = kThreads / 64;
constexpr int kSub = 512;  // keys per sub-chunk (scores kept in LDS)
constexpr int kUnroll = 8;
constexpr int kMaxSplitsLds = 1024;  // per-split maxima staged in LDS by the reduce

template <bool F32>
using Elem = typename std::conditional<F32, float, bf16>::type;

// 16-byte chunk -> fp32 values
template <bool F32>
__device__ inline void unpack16(const u32x4& w, float* f) {
  if constexpr (F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16lo(w[i]);
      f[2 * i + 1] = bf16hi(w[i]);
    }
  }
}

__device__ inline float block_reduce_max(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, red[i]);
  return r;
}

template <int D, bool F32>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(DecodeArgs a) {
  using E = Elem<F32>;
  constexpr int DV = 2 * D;
  constexpr int EPC = F32 ? 4 : 8;    // elements per 16-byte chunk
  constexpr int LPK = D / EPC;        // lanes per K row
  constexpr int KPR = kThreads / LPK; // key rows per pass (score phase)
  constexpr int LPV = DV / EPC;       // lanes per V row
  constexpr int VPR = kThreads / LPV; // V rows per pass
  constexpr int RS = 2 * (DV + 2);    // floats per (b, h, split) record
  static_assert(LPK <= 64 && LPV <= 64, "row must fit in one wave");

  __shared__ float2 sp[kSub];         // per key: (s1, s2) then (p1, p2)
  __shared__ float red[kWaves];
  __shared__ float accred[kWaves][2][DV];
  __shared__ float lred[kWaves][2];
  lds_poison(sp, sizeof(sp));
  lds_poison(red, sizeof(red));
  lds_poison(accred, sizeof(accred));
  lds_poison(lred, sizeof(lred));
  lds_poison_done();

  const int tid = threadIdx.x;
  const int S = a.S;
  const int split = blockIdx.x % S;
  const int bh = blockIdx.x / S;
  const int L = a.L;
  // ragged caches: sequence b uses its first lens[b] rows (clamped to [0, L])
  const int Lb = a.lens ? min(max(a.lens[bh / a.H], 0), L) : L;
  const int chunk = (Lb + S - 1) / S;
  const int kb = min(Lb, split * chunk);
  const int ke = min(Lb, kb + chunk);

  const E* __restrict__ K1 = (const E*)a.k1 + (size_t)bh * L * D;
  const E* __restrict__ K2 = (const E*)a.k2 + (size_t)bh * L * D;
  const E* __restrict__ V = (const E*)a.v + (size_t)bh * L * DV;
  const float sc = a.score_scale;

  // this lane's slice of q1 and q2 (score phase layout)
  const int ksub = tid % LPK;
  float q1f[EPC], q2f[EPC];
  {
    const E* q1p = (const E*)a.q1 + (size_t)bh * D + ksub * EPC;
    const E* q2p = (const E*)a.q2 + (size_t)bh * D + ksub * EPC;
    unpack16<F32>(*(const u32x4*)q1p, q1f);
    unpack16<F32>(*(const u32x4*)q2p, q2f);
  }
  const int vsub = tid % LPV;

  float m1 = kNegInf, m2 = kNegInf;  // running maxima (log2 units)
  float l1 = 0.0f, l2 = 0.0f;        // this thread's share of the sums
  float acc1[EPC], acc2[EPC];        // this thread's channels vsub*EPC ..
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc1[e] = acc2[e] = 0.0f;

  for (int base = kb; base < ke; base += kSub) {
    const int n = min(kSub, ke - base);

    // ---- scores: s = q . k * log2(e)/sqrt(D) -----------------------------------
    for (int k0 = tid / LPK; k0 < n; k0 += KPR * kUnroll) {
      u32x4 w1[kUnroll], w2[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int kk = min(k0 + u * KPR, n - 1);  // clamped: always in bounds
        const size_t off = (size_t)(base + kk) * D + ksub * EPC;
        w1[u] = __builtin_nontemporal_load((const u32x4*)(K1 + off));
        w2[u] = __builtin_nontemporal_load((const u32x4*)(K2 + off));
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        float k1f[EPC], k2f[EPC];
        unpack16<F32>(w1[u], k1f);
        unpack16<F32>(w2[u], k2f);
        float d1 = 0.0f, d2 = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          d1 = fmaf(q1f[e], k1f[e], d1);
          d2 = fmaf(q2f[e], k2f[e], d2);
        }
#pragma unroll
        for (int o = 1; o < LPK; o <<= 1) {
          d1 += __shfl_xor(d1, o);
          d2 += __shfl_xor(d2, o);
        }
        const int kk = k0 + u * KPR;
        if (ksub == 0 && kk < n) sp[kk] = make_float2(d1 * sc, d2 * sc);
      }
    }
    __syncthreads();

    // ---- block max per map, rescale the running state --------------------------
    float bm1 = kNegInf, bm2 = kNegInf;
    for (int kk = tid; kk < n; kk += kThreads) {
      bm1 = fmaxf(bm1, sp[kk].x);
      bm2 = fmaxf(bm2, sp[kk].y);
    }
    bm1 = block_reduce_max(bm1, red);
    bm2 = block_reduce_max(bm2, red);
    const float n1 = fmaxf(m1, bm1), n2 = fmaxf(m2, bm2);
    const float al1 = __builtin_amdgcn_exp2f(m1 - n1);  // m = -inf -> 0
    const float al2 = __builtin_amdgcn_exp2f(m2 - n2);
    m1 = n1;
    m2 = n2;
    l1 *= al1;
    l2 *= al2;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      acc1[e] *= al1;
      acc2[e] *= al2;
    }
    for (int kk = tid; kk < n; kk += kThreads) {
      const float2 s = sp[kk];
      const float p1 = __builtin_amdgcn_exp2f(s.x - m1);
      const float p2 = __builtin_amdgcn_exp2f(s.y - m2);
      l1 += p1;
      l2 += p2;
      sp[kk] = make_float2(p1, p2);
    }
    __syncthreads();

    // ---- V pass: both weighted sums from one read of each V row ----------------
    for (int k0 = tid / LPV; k0 < n; k0 += VPR * kUnroll) {
      u32x4 wv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int kk = min(k0 + u * VPR, n - 1);
        wv[u] = __builtin_nontemporal_load((const u32x4*)(V + (size_t)(base + kk) * DV + vsub * EPC));
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int kk = k0 + u * VPR;
        if (kk < n) {
          const float2 p = sp[kk];
          float vf[EPC];
          unpack16<F32>(wv[u], vf);
#pragma unroll
          for (int e = 0; e < EPC; ++e) {
            acc1[e] = fmaf(p.x, vf[e], acc1[e]);
            acc2[e] = fmaf(p.y, vf[e], acc2[e]);
          }
        }
      }
    }
    __syncthreads();  // sp is rewritten by the next sub-chunk
  }

  // ---- reduce the per-thread shares and write the partial record ---------------
  l1 = wave_sum(l1);
  l2 = wave_sum(l2);
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
#pragma unroll
    for (int o = LPV; o < 64; o <<= 1) {
      acc1[e] += __shfl_xor(acc1[e], o);
      acc2[e] += __shfl_xor(acc2[e], o);
    }
  }
  if (lane < LPV) {
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      accred[wave][0][vsub * EPC + e] = acc1[e];
      accred[wave][1][vsub * EPC + e] = acc2[e];
    }
  }
  if (lane == 0) {
    lred[wave][0] = l1;
    lred[wave][1] = l2;
  }
  __syncthreads();
  float* rec = a.ws + ((size_t)bh * S + split) * RS;
  for (int i = tid; i < 2 * DV; i += kThreads) {
    const int br = i / DV, c = i % DV;
    float t = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) t += accred[wv][br][c];
    rec[br * (DV + 2) + 2 + c] = t;
  }
  if (tid < 2) {
    float t = 0.0f;
#pragma unroll
    for (int wv = 0; wv < kWaves; ++wv) t += lred[wv][tid];
    rec[tid * (DV + 2)] = tid == 0 ? m1 : m2;
    rec[tid * (DV + 2) + 1] = t;
  }
}

template <int DV, bool F32, bool HEADNORM>
__global__ __launch_bounds__(256) void decode_reduce_kernel(DecodeArgs a) {
  // One workgroup per (b, h): 256 threads = DV channels x (256 / DV) split
  // groups (DV = 2D for the first version, D for V2).  The per-split maxima
  // are staged in LDS first; each thread then merges a fixed, contiguous
  // range of splits for its channel (independent loads, unrolled), and the
  // split groups are combined in a fixed order, so the result does not depend
  // on timing.
  using E = Elem<F32>;
  constexpr int RS = 2 * (DV + 2);
  constexpr int NG = 256 / DV;  // split groups
  __shared__ float sm[2][kMaxSplitsLds];
  __shared__ float part[NG][4][DV];
  __shared__ float red[4];
  __shared__ float mred[4][2];
  lds_poison(sm, sizeof(sm));
  lds_poison(part, sizeof(part));
  lds_poison(red, sizeof(red));
  lds_poison(mred, sizeof(mred));
  lds_poison_done();

  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int c = tid % DV;
  const int grp = tid / DV;
  const int S = a.S;
  const float* __restrict__ rec = a.ws + (size_t)bh * S * RS;

  float M1 = kNegInf, M2 = kNegInf;
  for (int s = tid; s < S; s += 256) {
    const float m1 = rec[(size_t)s * RS], m2 = rec[(size_t)s * RS + DV + 2];
    if (s < kMaxSplitsLds) {
      sm[0][s] = m1;
      sm[1][s] = m2;
    }
    M1 = fmaxf(M1, m1);
    M2 = fmaxf(M2, m2);
  }
  M1 = wave_max(M1);
  M2 = wave_max(M2);
  if ((tid & 63) == 0) {
    mred[tid >> 6][0] = M1;
    mred[tid >> 6][1] = M2;
  }
  __syncthreads();
  M1 = fmaxf(fmaxf(mred[0][0], mred[1][0]), fmaxf(mred[2][0], mred[3][0]));
  M2 = fmaxf(fmaxf(mred[0][1], mred[1][1]), fmaxf(mred[2][1], mred[3][1]));

  const int per = (S + NG - 1) / NG;
  const int s0 = grp * per;
  const int s1 = min(S, s0 + per);
  float L1 = 0.0f, L2 = 0.0f, A1 = 0.0f, A2 = 0.0f;
#pragma unroll 8
  for (int s = s0; s < s1; ++s) {
    const float* r = rec + (size_t)s * RS;
    const float m1 = s < kMaxSplitsLds ? sm[0][s] : r[0];
    const float m2 = s < kMaxSplitsLds ? sm[1][s] : r[DV + 2];
    // empty chunk: m = -inf -> 0; no key at all (M = -inf): nothing to add
    const float f1 = M1 == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m1 - M1);
    const float f2 = M2 == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(m2 - M2);
    L1 = fmaf(f1, r[1], L1);
    A1 = fmaf(f1, r[2 + c], A1);
    L2 = fmaf(f2, r[DV + 3], L2);
    A2 = fmaf(f2, r[DV + 4 + c], A2);
  }
  part[grp][0][c] = L1;
  part[grp][1][c] = A1;
  part[grp][2][c] = L2;
  part[grp][3][c] = A2;
  __syncthreads();
  // every thread stays for the barriers below; split group 0 finishes the row
  float o = 0.0f;
  if (grp == 0) {
    L1 = A1 = L2 = A2 = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      L1 += part[g][0][c];
      A1 += part[g][1][c];
      L2 += part[g][2][c];
      A2 += part[g][3][c];
    }
    // a sequence with no cached row (length 0) gives a zero row
    const float t1 = L1 > 0.0f ? A1 * (1.0f / L1) : 0.0f;
    const float t2 = L2 > 0.0f ? A2 * (1.0f / L2) : 0.0f;
    const float lt2 = a.lam[bh % a.H] * t2;
    o = t1 - lt2;
  }
  if constexpr (HEADNORM) {
    const float ss = wave_sum(o * o);  // threads outside group 0 contribute 0
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    o *= rsqrtf((red[0] + red[1] + red[2] + red[3]) * (1.0f / DV) + a.eps) * a.out_scale;
  }
  if (grp != 0) return;
  ((E*)a.out)[(size_t)bh * DV + c] = (E)o;
}

template <int D, bool F32>
hipError_t launch_d(const DecodeArgs& a, bool headnorm, hipStream_t stream) {
  const long nblk = (long)a.B * a.H * a.S;
  if (!grid_fits(nblk, kThreads) || !grid_fits((long long)a.B * a.H, 256)) return hipErrorInvalidConfiguration;
  decode_partial_kernel<D, F32><<<dim3((unsigned)nblk), dim3(kThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g((unsigned)(a.B * a.H)), b(256);
  if (headnorm) decode_reduce_kernel<2 * D, F32, true><<<g, b, 0, stream>>>(a);
  else decode_reduce_kernel<2 * D, F32, false><<<g, b, 0, stream>>>(a);
  return hipGetLastError();
}

// DIFF V2 decode partial (the French lesson page, "V1 contre V2": the two
// queries of a differential head read one shared K/V cache, so the cache is
// read once per step and the arithmetic per cache byte rises).  One workgroup
// per (b, KV head g, split) serves all G differential heads of the group; the
// records it writes have the first version's layout with value width D, one
// per (b, head, split), so decode_reduce_kernel<D> finishes them.  With NR =
// 2G query rows per cache row a VALU form needs more VALU time per key than
// HBM takes to deliver it at D = 128, so this runs on the matrix cores.
// Here the scores of all NR rows come from one MFMA chain S^T = K Q^T (keys x
// query columns: column c < G is map 1 of head c, G <= c < 2G map 2 of head
// c - G; the other columns hold zero queries and are dropped), and the
// weighted sums from O^T = V^T P^T, exactly the prefill's formulation
// (scores in base-2 units with the reference as the accumulator input, lazy
// rescale).  Each wave streams its own 32-key blocks (blocks w, w + 4, ...):
// nontemporal 16-byte register loads run kPf blocks ahead, and each block is
// written to a private LDS slot just before its fragments are read (the V
// fragments need the transposing LDS read).  No workgroup barrier in the
// loop; the four waves' states are merged at the end into one record per
// (head, map).
template <int D, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_v2_mma_kernel(DecodeArgs a) {
  constexpr int NR = 2 * G;
  constexpr int KSTEPS = D / 16;
  constexpr int CB = D / 32;
  constexpr int KB = 32 * D * 2;      // bytes of one 32-key block of K (or V)
  constexpr int CK = D / 8;           // 16-byte chunks per row
  constexpr int RK = 64 / CK;         // rows per 1-KiB load segment
  constexpr int NSEG = KB / 1024;     // segments per block, per tensor
  constexpr int RS = 2 * (D + 2);
  constexpr float kTauSum = 256.0f;   // rescale trigger (p <= 2^8)
  constexpr int kPf = 2;              // blocks in flight per wave, in registers
  static_assert(NR <= 32, "query columns");
  __shared__ __attribute__((aligned(1024))) char smem[kWaves][2 * KB];
  lds_poison(smem, sizeof(smem));
  lds_poison_done();

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = a.S;
  const int split = blockIdx.x % S;
  const int bg = blockIdx.x / S;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int head0 = b * a.H + g * G;
  const int L = a.L;
  const int chunk = (L + S - 1) / S;
  const int kb = min(L, split * chunk);
  const int ke = min(L, kb + chunk);
  // (uniform: every loop bound and branch below stays scalar)
  const int nblk = __builtin_amdgcn_readfirstlane((ke - kb + 31) / 32);
  const bf16* __restrict__ K = scalar_ptr((const bf16*)a.k1 + (size_t)bg * L * D);
  const bf16* __restrict__ V = scalar_ptr((const bf16*)a.v + (size_t)bg * L * D);

  // query fragments (B operand), scaled to base-2 units and rounded once
  const float sc = a.score_scale;
  bf16x8 qf[KSTEPS];
  {
    const bool ok = l32 < NR;
    const bf16* src = (const bf16*)(l32 < G ? a.q1 : a.q2) + (size_t)(head0 + (ok ? l32 % G : 0)) * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      u32x4 raw = *(const u32x4*)(src + ks * 16 + hi * 8);
      raw = ok ? raw : u32x4{0u, 0u, 0u, 0u};
      const bf16x8 q = __builtin_bit_cast(bf16x8, raw);
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = (bf16)((float)q[e] * sc);
    }
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): q before the cache loads start

  // Block j (keys kb + 32 j ..) is read with coalesced 16-byte loads: load
  // sg of a lane takes row sg RK + lane / CK, 16-byte chunk
  // (lane % CK) ^ swizzle(row), and stage() stores it at byte 16 lane of
  // segment sg of the wave's slot, so the slot holds each row with its chunks
  // permuted by the same swizzle the fragment reads undo.  Rows past the
  // chunk end load row ke - 1 (in bounds) and are masked.
  // (global address space: loads that the compiler counts on vmcnt alone)
  typedef __attribute__((address_space(1))) const u32x4 gu32x4;
  u32x4 kr[kPf][NSEG], vr[kPf][NSEG];
  auto load = [&](int j, u32x4 (&kk)[NSEG], u32x4 (&vv)[NSEG]) __attribute__((always_inline)) {
    const int key0 = kb + 32 * j;
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
      const int r = sg * RK + lane / CK;
      const uint32_t row = (uint32_t)min(key0 + r, ke - 1);
      kk[sg] = __builtin_nontemporal_load((gu32x4*)(K + row * D + (((lane % CK) ^ swz_k<D>(r)) << 3)));
      vv[sg] = __builtin_nontemporal_load((gu32x4*)(V + row * D + (((lane % CK) ^ swz_v<D>(r)) << 3)));
    }
  };
  char* const sk = smem[wave];
  const char* const sv = sk + KB;
  auto stage = [&](const u32x4 (&kk)[NSEG], const u32x4 (&vv)[NSEG]) __attribute__((always_inline)) {
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) {
      *(u32x4*)(sk + sg * 1024 + lane * 16) = kk[sg];
      *(u32x4*)(sk + KB + sg * 1024 + lane * 16) = vv[sg];
    }
  };

  floatx16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = splat16(0.0f);
  floatx16 negmu = splat16(0.0f);
  float mu = 0.0f, lsum = 0.0f;
  bool started = false;
  const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
  const int k_rd = l32 * (2 * D);
  const int swk = swz_k<D>(l32);
  const int vq = lane & 3, vkq = (lane >> 2) & 3;
  const int v_row = 4 * hi + vkq;
  const int v_chunk = 2 * ((lane >> 4) & 1) + (vq >> 1);
  const int v_sw = swz_v<D>(vkq);
  const int v_byte = (vq & 1) * 8;

  // One block of the loop below: stage it, refill its registers kPf blocks
  // ahead, compute.  Loads are issued whether or not their block exists (one
  // past the chunk reads row ke - 1 again, from cache) so that every path
  // issues them in the same order and each wait counts only the loads
  // issued after the block's own.
  auto block = [&](int j, u32x4 (&kk)[NSEG], u32x4 (&vv)[NSEG]) __attribute__((always_inline)) {
    // the previous block's fragment reads are issued before these writes (a
    // wave's LDS operations run in order), and these writes before the reads
    // below
    asm volatile("" ::: "memory");
    stage(kk, vv);
    asm volatile("" ::: "memory");
    load(j + kWaves * kPf, kk, vv);
    if (j >= nblk) return;
    floatx16 s;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const bf16x8 kf = *(const bf16x8*)(sk + k_rd + (((2 * ks + hi) ^ swk) << 4));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], ks == 0 ? negmu : s, 0, 0, 0);
    }
    const int key0 = kb + 32 * j;
    if (key0 + 32 > ke) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[r] = key >= ke ? kNegInf : s[r];
      }
    }
    bf16x8 pk[2];
    float bs = 0.0f;
    auto expo = [&]() __attribute__((always_inline)) {
      bs = 0.0f;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pa = __builtin_amdgcn_exp2f(s[8 * kh + 2 * e]);
          const float pb = __builtin_amdgcn_exp2f(s[8 * kh + 2 * e + 1]);
          const bf16x2 pw = {(bf16)pa, (bf16)pb};
          bs = __builtin_amdgcn_fdot2_f32_bf16(pw, ones, bs, false);
          pk[kh][2 * e] = pw[0];
          pk[kh][2 * e + 1] = pw[1];
        }
    };
    expo();
    // lazy rescale as in the prefill: the wave's first block sets the
    // reference to the exact column max; later only a partial sum above 2^8
    if (__any(!started || bs > kTauSum)) {
      float m = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fmaxf(m, s[r]);
      m = swap_halves_max(m);
      const float delta = started ? fmaxf(m, 0.0f) : m;  // the first block always has a visible key
      // the first block finds the state empty: no scaling (2^-delta could
      // overflow for a block max far below zero, and 0 x inf is NaN)
      const float alpha = started ? __builtin_amdgcn_exp2f(-delta) : 1.0f;
      mu += delta;
      lsum *= alpha;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[cb][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] -= delta;
      negmu = splat16(-mu);
      expo();
    }
    started = true;
    lsum += bs;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* base = sv + (16 * ks + v_row) * (2 * D) + (((4 * cb + v_chunk) ^ v_sw) << 4) + v_byte;
        const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)base);
        const bf16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(base + 8 * (2 * D)));
        const bf16x8 vf = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk[ks], acc[cb], 0, 0, 0);
      }
  };

#pragma unroll
  for (int p = 0; p < kPf; ++p) load(wave + kWaves * p, kr[p], vr[p]);
  for (int j = wave; j < nblk; j += kWaves * kPf) {
#pragma unroll
    for (int p = 0; p < kPf; ++p) block(j + kWaves * p, kr[p], vr[p]);
  }

  // ---- merge the four waves' states; one record per (head, map) -------------
  const float ltot = swap_halves_sum(lsum);
  if (!started) mu = kNegInf;  // a wave with no block contributes nothing
  __syncthreads();              // every wave is done with its LDS slot
  float* mw = (float*)&smem[0][0];  // [wave][column][D + 2]
  if (l32 < NR) {
    float* row = mw + (wave * NR + l32) * (D + 2);
    if (hi == 0) {
      row[0] = mu;
      row[1] = ltot;
    }
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) row[2 + cb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3)] = acc[cb][r];
  }
  __syncthreads();
  for (int i = tid; i < NR * D; i += kThreads) {
    const int c = i / D, ch = i % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[(w * NR + c) * (D + 2)]);
    float Lsum = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float* row = mw + (w * NR + c) * (D + 2);
      const float f = M == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(row[0] - M);
      Lsum = fmaf(f, row[1], Lsum);
      A = fmaf(f, row[2 + ch], A);
    }
    float* rec = a.ws + ((size_t)(head0 + c % G) * S + split) * RS + (c / G) * (D + 2);
    rec[2 + ch] = A;
    if (ch == 0) {
      rec[0] = M;
      rec[1] = Lsum;
    }
  }
}

template <int D, int G>
hipError_t launch_v2_d(const DecodeArgs& a, hipStream_t stream) {
  const long nblk = (long)a.B * a.Hkv * a.S;
  if (!grid_fits(nblk, kThreads) || !grid_fits((long long)a.B * a.H, 256)) return hipErrorInvalidConfiguration;
  decode_v2_mma_kernel<D, G><<<dim3((unsigned)nblk), dim3(kThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_reduce_kernel<D, false, false><<<dim3((unsigned)(a.B * a.H)), dim3(256), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_v2(const DecodeArgs& a, int D, hipStream_t stream) {
  const int grp = a.H / a.Hkv;
  if (D == 64) {
    if (grp == 1) return launch_v2_d<64, 1>(a, stream);
    if (grp == 2) return launch_v2_d<64, 2>(a, stream);
    if (grp == 4) return launch_v2_d<64, 4>(a, stream);
  } else if (D == 128) {
    if (grp == 1) return launch_v2_d<128, 1>(a, stream);
    if (grp == 2) return launch_v2_d<128, 2>(a, stream);
    if (grp == 4) return launch_v2_d<128, 4>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, int dtype, int D, bool headnorm, hipStream_t stream) {
  if (dtype == 1) {
    switch (D) {
      case 32: return launch_d<32, false>(a, headnorm, stream);
      case 64: return launch_d<64, false>(a, headnorm, stream);
      case 128: return launch_d<128, false>(a, headnorm, stream);
    }
  } else {
    switch (D) {
      case 32: return launch_d<32, true>(a, headnorm, stream);
      case 64: return launch_d<64, true>(a, headnorm, stream);
      case 128: return launch_d<128, true>(a, headnorm, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace diffattn
