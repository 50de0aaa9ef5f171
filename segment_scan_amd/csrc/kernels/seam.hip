// seam.hip -- the seam-window step at reuse, fused with the ordered
// composition of the cached body pairs (delta-rule families).
//
// [youleyou, full-attention paragraph] the first w tokens of each reused
// segment (w = 8 by default) are kept out of its cache entry and recomputed
// under the full prefix; to make that possible the linear layers compute the
// window's own T and S on the fly, advance the running state through the
// window and forward every seam token's output to the full-attention layer
// above.  [youleyou, linear-layer paragraph] the body of the segment is then
// applied from its cached pair, S <- T_B S + S_B.
//
// One workgroup per chain; wave w keeps state columns 32w .. 32w+31 in
// registers for the whole request.  Per segment:
//  1. the window, in sub-chunks of up to 16 tokens, in the UT form with start
//     state S0, prefix G of the log gates and Gamma_ts = exp(G_t - G_s):
//        Abar = (I + strict_lower(diag(b) (Gamma o K K^T)))^-1 diag(b)
//        Z    = Abar (V - diag(exp(G)) K S0)
//        o_t  = exp(G_t) q_t^T S0 + sum_{s<=t} Gamma_ts (q_t . k_s) z_s
//        S    = exp(G_n) S0 + K^T diag(exp(G_n - G)) Z
//     [K;Q] S0 is one 32 x 32 MFMA tile per wave (B operand straight from the
//     state registers), the 16 x 16 solve is fp32 on the VALU, and the rank-16
//     state update is one MFMA k-step;
//  2. the body pair: S <- exp(g) U S + S_B with U staged in LDS and the
//     product in three-term split-bf16 MFMA (fp32-class), the next segment's
//     U in flight meanwhile.
#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

constexpr int SUB = 16;  // window tokens per sub-chunk

template <int D, bool IN_F32>
struct SeamCfg {
  static constexpr int NW = D / 32;
  static constexpr int NTH = NW * 64;
  static constexpr int NTI = IN_F32 ? 3 : 1;
  static constexpr int NTS = IN_F32 ? 3 : 2;   // terms of the state in window products
  static constexpr int NTC = 3;                // terms in the body product (fp32 pairs)
  static constexpr int P = D + 4;              // fp32 pitch of the staged U
  static constexpr int KTP = 24;               // bf16 pitch of K^T [d][16]
  static constexpr int U_BYTES = D * P * 4;
  static constexpr int KQ_BYTES = NTI * 32 * D * 2;   // [K;Q] rows, swizzled
  static constexpr int KT_BYTES = NTI * D * KTP * 2;  // K^T
  static constexpr int V_BYTES = SUB * D * 4;         // V fp32
  static constexpr int W_BYTES = NW * 2 * SUB * 33 * 4;  // per wave: R/Z and QS
  static constexpr int SM_BYTES = (2 * SUB * 17 + 6 * SUB) * 4;  // Abar, Omega, small
  static constexpr int OFF_U = 0;
  static constexpr int OFF_KQ = OFF_U + U_BYTES;
  static constexpr int OFF_KT = OFF_KQ + KQ_BYTES;
  static constexpr int OFF_V = OFF_KT + KT_BYTES;
  static constexpr int OFF_W = OFF_V + V_BYTES;
  static constexpr int OFF_SM = OFF_W + W_BYTES;
  static constexpr int LDS = OFF_SM + SM_BYTES;
};

template <int W>
__device__ __forceinline__ int swz(int row, int col) {
  return row * W + ((((col >> 3) ^ (row & 7)) << 3) | (col & 7));
}

template <int D, bool IN_F32, bool BODY>
__global__ __launch_bounds__(D * 2) void seam_delta_kernel(const SeamArgs a) {
  using Cfg = SeamCfg<D, IN_F32>;
  constexpr int NRT = D / 32, NTH = Cfg::NTH, NTI = Cfg::NTI, NTS = Cfg::NTS, NTC = Cfg::NTC;
  constexpr int P = Cfg::P, KTP = Cfg::KTP;
  constexpr int KQS = 32 * D;     // term stride of [K;Q]
  constexpr int KTS = D * KTP;    // term stride of K^T
  constexpr int LD_PER_T = D * D / 4 / NTH;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* sU = reinterpret_cast<float*>(smem + Cfg::OFF_U);
  bf16_t* sKQ = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_KQ);
  bf16_t* sKt = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_KT);
  float* sV = reinterpret_cast<float*>(smem + Cfg::OFF_V);
  float* sW = reinterpret_cast<float*>(smem + Cfg::OFF_W);
  float* sAb = reinterpret_cast<float*>(smem + Cfg::OFF_SM);  // [16][17]
  float* sOm = sAb + SUB * 17;                                 // [16][17]
  float* sBeta = sOm + SUB * 17;
  float* sLg = sBeta + SUB;
  float* sG = sLg + SUB;
  float* sEG = sG + SUB;
  float* sEW = sEG + SUB;
  float* sMisc = sEW + SUB;

  const int chain = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int h = lane >> 5;
  const int n_chain = a.n_chain;
  const int col = 32 * wave + (lane & 31);
  const size_t chain_off = (size_t)chain * D * D;
  const size_t seg_stride = (size_t)n_chain * D * D;
  float* sR = sW + wave * 2 * SUB * 33;  // this wave's R, then Z   [16][33]
  float* sQS = sR + SUB * 33;            // this wave's Q S0        [16][33]

  f32x16 Sb[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) Sb[rt][r] = a.S_run[chain_off + (size_t)(32 * rt + acc_row(r, lane)) * D + col];

  f32x4 ureg[LD_PER_T];
  auto load_U = [&](int s) {
    const f32x4* src = reinterpret_cast<const f32x4*>(a.bU + (size_t)s * seg_stride + chain_off);
#pragma unroll
    for (int i = 0; i < LD_PER_T; ++i) ureg[i] = src[i * NTH + tid];
  };
  if constexpr (BODY) load_U(0);

  for (int seg = 0; seg < a.n_seg; ++seg) {
    f32x16 Sbody[NRT];
    float gB = 0.f;
    if constexpr (BODY) {
      // U of this segment -> LDS (the previous segment's readers are done)
#pragma unroll
      for (int i = 0; i < LD_PER_T; ++i) {
        const int e = (i * NTH + tid) * 4;
        *reinterpret_cast<f32x4*>(sU + (e / D) * P + (e % D)) = ureg[i];
      }
      if (seg + 1 < a.n_seg) load_U(seg + 1);
      const float* Sg = a.bS + (size_t)seg * seg_stride + chain_off;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) Sbody[rt][r] = Sg[(size_t)(32 * rt + acc_row(r, lane)) * D + col];
      gB = a.bg[(size_t)seg * n_chain + chain];
    }

    // ---------------- window tokens, sub-chunks of <= 16 ----------------------
    for (int j0 = 0; j0 < a.w; j0 += SUB) {
      const int n = min(SUB, a.w - j0);
      const size_t tok0 = (size_t)seg * a.w + j0;
      // stage [K;Q] (rows 0-15 keys, 16-31 queries), K^T, V, beta, log gate
      for (int e = tid; e < 32 * (D / 8); e += NTH) {
        const int row = e / (D / 8), cb = (e % (D / 8)) * 8;
        const int t = row & 15;
        float x[8];
        if (t < n) {
          load8<IN_F32>(row < 16 ? a.k : a.q, ((tok0 + t) * n_chain + chain) * D + cb, x);
        } else {
#pragma unroll
          for (int c = 0; c < 8; ++c) x[c] = 0.f;
        }
        const Frag<NTI> f = split8<NTI>(x);
#pragma unroll
        for (int i = 0; i < NTI; ++i) {
          *reinterpret_cast<bf16x8*>(sKQ + i * KQS + swz<D>(row, cb)) = f.t[i];
          if (row < 16) {
#pragma unroll
            for (int c = 0; c < 8; ++c) sKt[i * KTS + (cb + c) * KTP + t] = f.t[i][c];
          }
        }
      }
      for (int e = tid; e < SUB * (D / 4); e += NTH) {
        const int t = e / (D / 4), cb = (e % (D / 4)) * 4;
        f32x4 vv = {0.f, 0.f, 0.f, 0.f};
        if (t < n) {
          float x[8];
          if constexpr (IN_F32) {
            vv = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.v) + ((tok0 + t) * n_chain + chain) * D + cb);
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] = load1<false>(a.v, ((tok0 + t) * n_chain + chain) * D + cb + c);
            vv = f32x4{x[0], x[1], x[2], x[3]};
          }
        }
        *reinterpret_cast<f32x4*>(sV + t * D + cb) = vv;
      }
      if (tid < SUB) {
        float b = 0.f, lg = 0.f;
        if (tid < n) {
          const size_t idx = (tok0 + tid) * n_chain + chain;
          b = load1<IN_F32>(a.beta, idx);
          if (a.lg) lg = load1<IN_F32>(a.lg, idx);
        }
        sBeta[tid] = b;
        sLg[tid] = lg;
      }
      __syncthreads();

      if (wave == 0) {
        // gate prefix (lanes 0-15)
        float G = wave_incl_scan(lane < SUB ? sLg[lane] : 0.f);
        const float GC = __shfl(G, SUB - 1, 64);
        if (lane < SUB) {
          sG[lane] = G;
          sEG[lane] = expf(G);
          sEW[lane] = expf(GC - G);
        }
        if (lane == 0) sMisc[0] = expf(GC);
        // [K;Q] K^T : rows 0-15 K K^T, rows 16-31 Q K^T (columns 0-15 used)
        f32x16 P2 = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          Frag<NTI> fa, fb;
#pragma unroll
          for (int i = 0; i < NTI; ++i) {
            fa.t[i] = *reinterpret_cast<const bf16x8*>(sKQ + i * KQS + swz<D>(lane & 31, 16 * ks + 8 * h));
            fb.t[i] = *reinterpret_cast<const bf16x8*>(sKQ + i * KQS + swz<D>((lane & 15), 16 * ks + 8 * h));
          }
          mma<NTI, NTI>(P2, fa, fb);
        }
        const int cc = lane & 31;
        if (cc < SUB) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = acc_row(r, lane);
            if (rr < SUB) {  // K K^T: M = strict_lower(diag(b) (Gamma o K K^T))
              const float gm = (rr > cc) ? expf(sG[rr] - sG[cc]) : 0.f;
              sAb[rr * 17 + cc] = sBeta[rr] * gm * P2[r];
            } else {         // Q K^T: Omega = tril_incl(Gamma o Q K^T)
              const int tq = rr - SUB;
              sOm[tq * 17 + cc] = (tq >= cc) ? expf(sG[tq] - sG[cc]) * P2[r] : 0.f;
            }
          }
        }
      }
      __syncthreads();
      if (wave == 0 && lane < SUB) {
        // column `lane` of (I + M)^-1, then Abar = (I + M)^-1 diag(b)
        const int c = lane;
        float x[SUB];
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
          float acc = 0.f;
#pragma unroll
          for (int k = 0; k < r; ++k)
            if (k >= c) acc = fmaf(sAb[r * 17 + k], x[k], acc);
          x[r] = (r < c) ? 0.f : ((r == c) ? 1.f : -acc);
        }
        const float bc = sBeta[c];
#pragma unroll
        for (int r = 0; r < SUB; ++r) sAb[r * 17 + c] = x[r] * bc;
      }

      // Y = [K;Q] S0 for this wave's 32 columns
      f32x16 Y = zero16();
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const Frag<NTS> fb = acc_as_b<NTS>(Sb[rt], m);
          Frag<NTI> fa;
          const int kb = 32 * rt + 16 * m + 4 * h;
#pragma unroll
          for (int i = 0; i < NTI; ++i) {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(sKQ + i * KQS + swz<D>(lane & 31, kb));
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(sKQ + i * KQS + swz<D>(lane & 31, kb + 8));
            fa.t[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
          mma<NTI, NTS>(Y, fa, fb);
        }
      // rows 0-15: R = V - exp(G) K S0 ; rows 16-31: Q S0
      const int cl = lane & 31;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = acc_row(r, lane);
        if (rr < SUB)
          sR[rr * 33 + cl] = sV[rr * D + col] - sEG[rr] * Y[r];
        else
          sQS[(rr - SUB) * 33 + cl] = Y[r];
      }
      __syncthreads();  // Abar ready, R and QS of every wave in LDS
      // Z = Abar R: lane (cl, h) computes rows 8h .. 8h+7
      float z[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = 8 * h + i;
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < SUB; ++s)
          if (s <= t) acc = fmaf(sAb[t * 17 + s], sR[s * 33 + cl], acc);
        z[i] = acc;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i) sR[(8 * h + i) * 33 + cl] = z[i];  // sR now holds Z
      __syncthreads();
      // outputs o_t = exp(G_t) (Q S0)_t + sum_{s<=t} Omega_ts Z_s
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int t = 8 * h + i;
        if (t < n) {
          float acc = sEG[t] * sQS[t * 33 + cl];
#pragma unroll
          for (int s = 0; s < SUB; ++s)
            if (s <= t) acc = fmaf(sOm[t * 17 + s], sR[s * 33 + cl], acc);
          a.o[((tok0 + t) * n_chain + chain) * D + col] = acc;
        }
      }
      // S = exp(G_n) S0 + K^T diag(exp(G_n - G)) Z   (one MFMA k-step of 16 tokens)
      {
        const float eGC = sMisc[0];
        float zz[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) zz[j] = sR[(8 * h + j) * 33 + cl] * sEW[8 * h + j];
        const Frag<NTS> fb = split8<NTS>(zz);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
          for (int r = 0; r < 16; ++r) Sb[rt][r] *= eGC;
          Frag<NTI> fa;
#pragma unroll
          for (int i = 0; i < NTI; ++i)
            fa.t[i] = *reinterpret_cast<const bf16x8*>(sKt + i * KTS + (32 * rt + (lane & 31)) * KTP + 8 * h);
          mma<NTI, NTS>(Sb[rt], fa, fb);
        }
      }
      __syncthreads();  // window scratch is reused by the next sub-chunk
    }

    // ---------------- body pair: S <- exp(g) U S + S_B ----------------------------
    if constexpr (BODY) {
      f32x16 T[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) T[rt] = zero16();
#pragma unroll
      for (int kt = 0; kt < NRT; ++kt)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const Frag<NTC> fb = acc_as_b<NTC>(Sb[kt], m);
          const int kcol = 32 * kt + 16 * m + 4 * h;
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const float* urow = sU + (32 * rt + (lane & 31)) * P;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(urow + kcol);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(urow + kcol + 8);
            float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const Frag<NTC> fa = split8<NTC>(x);
            mma<NTC, NTC>(T[rt], fa, fb);
          }
        }
      const float e = expf(gB);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) Sb[rt][r] = fmaf(e, T[rt][r], Sbody[rt][r]);
      __syncthreads();  // sU is overwritten by the next segment
    }
  }

#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) a.S_run[chain_off + (size_t)(32 * rt + acc_row(r, lane)) * D + col] = Sb[rt][r];
}

template <int D, bool F32, bool BODY>
hipError_t launch_t(const SeamArgs& a, hipStream_t stream) {
  constexpr int lds = SeamCfg<D, F32>::LDS;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&seam_delta_kernel<D, F32, BODY>), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((seam_delta_kernel<D, F32, BODY>), dim3(a.n_chain), dim3(D * 2), lds, stream, a);
  return hipGetLastError();
}

template <int D, bool F32>
hipError_t launch_d(const SeamArgs& a, hipStream_t stream) {
  return a.bS ? launch_t<D, F32, true>(a, stream) : launch_t<D, F32, false>(a, stream);
}

}  // namespace

bool seam_supported(int fam, int d, bool window_pairs) {
  return fam == 3 && (d == 64 || d == 128) && !window_pairs;
}

hipError_t launch_seam(int fam, int d, bool in_f32, const SeamArgs& a, hipStream_t stream) {
  if (!seam_supported(fam, d, a.wS != nullptr)) return hipErrorInvalidValue;
  if (d == 128) return in_f32 ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
  return in_f32 ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
}

}  // namespace hypic
