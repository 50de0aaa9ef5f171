// build_delta.hip -- segment build for the delta-rule families (DeltaNet, GDN):
// emits the factored transition T_C = exp(g) U and S(C|0) of every
// (segment, chain).
//
// [youleyou, linear-layer paragraph] T_C is the product of the segment's
// per-token transitions A_t = a_t (I - beta_t k_t k_t^T), here a dense
// "Householder-like" d x d matrix, and S(C|0) the final state from a zero
// start.  The scalar gate commutes with the Householder-like factors, so T_C
// is kept as exp(g) U with g = sum log a_t and U = prod (I - beta_t k_t k_t^T),
// which cannot underflow.
//
// Within a segment the kernel runs 64-token chunks joined by the composition
// law of the same paragraph (one segment split into pieces joined by operator
// composition, as in [hwlabs, section 병렬 콜드 프리필]).  A chunk's product
// of 64 rank-1 factors is applied in the compact WY/UT form: with keys K,
// values V, weights b, log gates a (prefix G within the chunk, Gamma_ts =
// exp(G_t - G_s)),
//   M0   = strict_lower(diag(b) K K^T),  N = (I + M0)^-1,  A0 = N diag(b)
//   Abar = Gamma o A0
//   U   <- U - K^T (A0 (K U))
//   S   <- exp(G_C) S + K^T diag(exp(G_C - G)) (Abar (V - diag(exp(G)) K S))
// which equals running the 64 tokens one by one (the tests check this algebra
// against the token-by-token oracle).
//
// Mapping (one workgroup of 4 waves per unit): the state [U | S] (d x 2d fp32)
// lives in registers, each wave owning d/2 columns (waves 0-1: U, waves 2-3:
// S) as MFMA accumulator tiles for the whole segment.  Columns evolve
// independently, so the waves only share the per-chunk operands in LDS:
// K (row-major and transposed), and A0 / Abar split into bf16 terms.  Every
// product K Z, A Y, K^T X takes its B operand directly from the accumulator
// registers of the previous step (no LDS round trip), so per chunk the state
// never leaves the register file.  The Gram matrix runs on MFMA, the 64 x 64
// unit-triangular inverse in fp32 on the VALU (16 x 16 diagonal blocks by
// forward substitution, then block rows).
#include <type_traits>

#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

constexpr int C = 64;  // tokens per chunk

template <int D, bool IN_F32>
struct DeltaCfg {
  static constexpr int NTI = IN_F32 ? 3 : 1;  // bf16 terms of input operands (K)
  static constexpr int NTD = IN_F32 ? 3 : 2;  // bf16 terms of derived operands
  static constexpr int NRT = D / 32;          // row tiles of the state
  static constexpr int CT = D / 64;           // 32-column tiles per wave (d/2 columns)
  static constexpr int CPW = D / 2;           // state columns per wave
  static constexpr int KP = D + 4;            // bf16 pitch of K [t][d]
  static constexpr int TP = C + 4;            // bf16 pitch of K^T [d][t] and of A [t][t']
  static constexpr int NP = 65;               // fp32 pitch of the inverse work array
  // LDS layout (bytes)
  static constexpr int K_BYTES = NTI * C * KP * 2;
  static constexpr int KT_BYTES = NTI * D * TP * 2;
  static constexpr int A_BYTES_BF = 2 * NTD * C * TP * 2;  // A0 and Abar, terms
  static constexpr int N_BYTES = C * NP * 4;                // fp32 inverse (aliases A region)
  static constexpr int A_BYTES = A_BYTES_BF > N_BYTES ? A_BYTES_BF : N_BYTES;
  static constexpr int T_BYTES = 3 * 16 * 17 * 4;           // block-row scratch
  static constexpr int OFF_K = 0;
  static constexpr int OFF_KT = OFF_K + K_BYTES;
  static constexpr int OFF_A = OFF_KT + KT_BYTES;
  static constexpr int OFF_T = OFF_A + A_BYTES;
  static constexpr int OFF_SMALL = OFF_T + T_BYTES;
  static constexpr int SMALL_BYTES = 6 * C * 4;  // beta, lg, G, eG, eW, misc
  static constexpr int LDS = OFF_SMALL + SMALL_BYTES;
  static constexpr int MIN_WAVES = IN_F32 ? 1 : 2;  // waves per SIMD (LDS allows 2 WGs for bf16)
};

template <int D, bool IN_F32>
__global__ __launch_bounds__(256, (IN_F32 ? 1 : 2)) void build_delta_kernel(const BuildArgs a) {
  using Cfg = DeltaCfg<D, IN_F32>;
  constexpr int NTI = Cfg::NTI, NTD = Cfg::NTD, NRT = Cfg::NRT, CT = Cfg::CT, CPW = Cfg::CPW;
  constexpr int NP = Cfg::NP, KP = Cfg::KP, TP = Cfg::TP;
  constexpr int KTS = C * KP;  // term stride (elements) of K
  constexpr int TTS = D * TP;  // term stride of K^T
  constexpr int ATS = C * TP;  // term stride of the A tiles

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_K);
  bf16_t* sKt = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_KT);
  bf16_t* sA0 = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_A);  // NTD terms
  bf16_t* sAb = sA0 + NTD * ATS;                                 // NTD terms
  float* sN = reinterpret_cast<float*>(smem + Cfg::OFF_A);       // aliases sA0/sAb
  float* sT = reinterpret_cast<float*>(smem + Cfg::OFF_T);
  float* sBeta = reinterpret_cast<float*>(smem + Cfg::OFF_SMALL);
  float* sLg = sBeta + C;
  float* sG = sLg + C;
  float* sEG = sG + C;     // exp(G_t)
  float* sEW = sEG + C;    // exp(G_C - G_t)
  float* sMisc = sEW + C;  // [0] = exp(G_C)

  const int lane0 = lane_id();
  const int wave = wave_id();
  const int n_chain = a.n_chain;
  const int slot = blockIdx.x / n_chain;  // longest segments first
  const int chain = blockIdx.x % n_chain;
  const int t_begin = a.seg.beg[slot];
  const int t_end = a.seg.end[slot];
  const size_t unit = (size_t)a.seg.out[slot] * n_chain + chain;
  const bool s_wave = wave >= 2;
  const int col0 = (wave & 1) * CPW;  // first state column of this wave (within U or S)

  // ---- running state: U = I (waves 0-1), S = 0 (waves 2-3) -------------------
  f32x16 Z[NRT][CT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rt + acc_row(r, lane0);
        const int col = col0 + 32 * ct + (lane0 & 31);
        Z[rt][ct][r] = (!s_wave && row == col) ? 1.f : 0.f;
      }
  double g_acc = 0.0;

  for (int c0 = t_begin; c0 < t_end; c0 += C) {
    const int nv = min(C, t_end - c0);
    // per-lane values are re-derived each chunk (see opaque() in common.h)
    const int tid = opaque(threadIdx.x);
    const int lane = tid & 63;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const bf16_t* pK = sK + l32 * KP + 4 * h;
    const bf16_t* pKg = sK + l32 * KP + 8 * h;
    const bf16_t* pKt = sKt + l32 * TP + 4 * h;
    const bf16_t* pA = (s_wave ? sAb : sA0) + l32 * TP + 4 * h;

    // ---- stage K (row-major + transposed), beta, log gate ----------------------
    if (tid < D) {
      const int tb = tid & 7, db = tid >> 3;
      if constexpr (!IN_F32) {
        bf16x8 rows[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int t = tb * 8 + r;
          if (t < nv) {
            rows[r] = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16_t*>(a.k) +
                                                       ((size_t)(c0 + t) * n_chain + chain) * D + db * 8);
          } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) rows[r][c] = (bf16_t)0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) st8(sK + (tb * 8 + r) * KP + db * 8, rows[r]);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          bf16x8 col;
#pragma unroll
          for (int r = 0; r < 8; ++r) col[r] = rows[r][c];
          st8(sKt + (db * 8 + c) * TP + tb * 8, col);
        }
      } else {
        float x[8][8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int t = tb * 8 + r;
          if (t < nv) {
            load8<true>(a.k, ((size_t)(c0 + t) * n_chain + chain) * D + db * 8, x[r]);
          } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) x[r][c] = 0.f;
          }
        }
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const Frag<NTI> f = split8<NTI>(x[r]);
#pragma unroll
          for (int i = 0; i < NTI; ++i) st8(sK + i * KTS + (tb * 8 + r) * KP + db * 8, f.t[i]);
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float col[8];
#pragma unroll
          for (int r = 0; r < 8; ++r) col[r] = x[r][c];
          const Frag<NTI> f = split8<NTI>(col);
#pragma unroll
          for (int i = 0; i < NTI; ++i) st8(sKt + i * TTS + (db * 8 + c) * TP + tb * 8, f.t[i]);
        }
      }
    } else if (tid >= 128 && tid < 128 + C) {
      const int t = tid - 128;
      float b = 0.f, lg = 0.f;
      if (t < nv) {
        const size_t idx = (size_t)(c0 + t) * n_chain + chain;
        b = load1<IN_F32>(a.beta, idx);
        if (a.lg) lg = load1<IN_F32>(a.lg, idx);
      }
      sBeta[t] = b;
      sLg[t] = lg;
    }
    __syncthreads();

    // ---- gate prefix (wave 3) and Gram tiles (waves 0-2) ----------------------
    if (wave == 3) {
      const float G = wave_incl_scan(sLg[lane]);
      const float GC = __shfl(G, 63, 64);
      sG[lane] = G;
      sEG[lane] = expf(G);
      sEW[lane] = expf(GC - G);
      if (lane == 0) sMisc[0] = expf(GC);
      g_acc += (double)GC;  // every lane of wave 3 keeps the same sum
    } else {
      // tiles (0,0), (1,0), (1,1) of K K^T; only t > t' is needed
      const int tt = (wave == 0) ? 0 : 1;
      const int tp = (wave == 2) ? 1 : 0;
      f32x16 acc = zero16();
      const bf16_t* pa = pKg + 32 * tt * KP;
      const bf16_t* pb = pKg + 32 * tp * KP;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const Frag<NTI> fa = lds_frag<NTI>(pa, KTS, 16 * ks);
        const Frag<NTI> fb = lds_frag<NTI>(pb, KTS, 16 * ks);
        mma<NTI, NTI>(acc, fa, fb);
      }
      const int cc = 32 * tp + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = 32 * tt + acc_row(r, lane);
        sN[rr * NP + cc] = (rr > cc) ? sBeta[rr] * acc[r] : 0.f;
      }
      if (wave == 0) {
        // the strictly-upper tile (0,1) is zero
#pragma unroll
        for (int r = 0; r < 16; ++r) sN[acc_row(r, lane) * NP + 32 + l32] = 0.f;
      }
    }
    __syncthreads();

    // ---- N = (I + M0)^-1: 16 x 16 diagonal blocks (wave 0) -------------------
    if (wave == 0) {
      const int b = lane >> 4, c = lane & 15;
      const float* Mb = sN + (16 * b) * NP + 16 * b;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < r; ++k)
          if (k >= c) acc = fmaf(Mb[r * NP + k], x[k], acc);
        x[r] = (r < c) ? 0.f : ((r == c) ? 1.f : -acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sN[(16 * b + r) * NP + 16 * b + c] = x[r];
    }
    // ---- block rows i = 1..3: N_ij = -N_ii sum_{k=j}^{i-1} M_ik N_kj ----------
    {
      const int r = tid >> 4, c = tid & 15;
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        __syncthreads();
#pragma unroll
        for (int j = 0; j < i; ++j) {
          float acc = 0.f;
          const float* Mrow = sN + (16 * i + r) * NP;
          for (int k = j; k < i; ++k)
#pragma unroll 4
            for (int m = 0; m < 16; ++m) acc = fmaf(Mrow[16 * k + m], sN[(16 * k + m) * NP + 16 * j + c], acc);
          sT[(j * 16 + r) * 17 + c] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < i; ++j) {
          float acc = 0.f;
          const float* Nrow = sN + (16 * i + r) * NP + 16 * i;
#pragma unroll
          for (int m = 0; m < 16; ++m) acc = fmaf(Nrow[m], sT[(j * 16 + m) * 17 + c], acc);
          sN[(16 * i + r) * NP + 16 * j + c] = -acc;
        }
      }
    }
    __syncthreads();

    // ---- A0 = N diag(beta), Abar = Gamma o A0, split to bf16 terms -----------
    {
      const int t = tid >> 2;
      const int cb = (tid & 3) * 16;
      float nv16[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int tp = cb + j;
        nv16[j] = (tp <= t) ? sN[t * NP + tp] : 0.f;
      }
      __syncthreads();  // sN is overwritten below
      const float Gt = sG[t];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float a0[8], ab[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int tp = cb + 8 * half + j;
          a0[j] = nv16[8 * half + j] * sBeta[tp];
          ab[j] = (tp <= t) ? a0[j] * expf(Gt - sG[tp]) : 0.f;
        }
        const Frag<NTD> f0 = split8<NTD>(a0);
        const Frag<NTD> fb = split8<NTD>(ab);
#pragma unroll
        for (int i = 0; i < NTD; ++i) {
          st8(sA0 + i * ATS + t * TP + cb + 8 * half, f0.t[i]);
          st8(sAb + i * ATS + t * TP + cb + 8 * half, fb.t[i]);
        }
      }
    }
    __syncthreads();

    // ---- per wave: Y = K Z, X = A Y, Z += K^T X (per 32-column tile) ---------
    const float eGC = sMisc[0];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int gcol = col0 + 32 * ct + l32;
      // values of this tile's rows, kept in the input dtype until used
      using VT = typename std::conditional<IN_F32, float, bf16_t>::type;
      VT vv[2][16];
      if (s_wave) {
        const VT* vsrc = reinterpret_cast<const VT*>(a.v) + ((size_t)c0 * n_chain + chain) * D + gcol;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int t = 32 * tt + acc_row(r, lane);
            vv[tt][r] = (t < nv) ? vsrc[(size_t)t * n_chain * D] : (VT)0.f;
          }
      }
      // product 1: Y[tt] = K[tt rows] * Z[:, ct]
      f32x16 Y[2] = {zero16(), zero16()};
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const Frag<NTD> fb = acc_as_b<NTD>(Z[rt][ct], m);
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const Frag<NTI> fa = lds_a_perm<NTI>(pK, KTS, 32 * tt * KP + 32 * rt + 16 * m);
            mma<NTI, NTD>(Y[tt], fa, fb);
          }
        }
      // S waves: R = V - diag(exp(G)) Y
      if (s_wave) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int r = 0; r < 16; ++r) Y[tt][r] = (float)vv[tt][r] - sEG[32 * tt + acc_row(r, lane)] * Y[tt][r];
      }
      // product 2: X[tt] = sum_{tp <= tt} A[tt, tp] * Y[tp]  (A lower triangular)
      f32x16 X[2] = {zero16(), zero16()};
#pragma unroll
      for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const Frag<NTD> fb = acc_as_b<NTD>(Y[tp], m);
#pragma unroll
          for (int tt = tp; tt < 2; ++tt) {
            const Frag<NTD> fa = lds_a_perm<NTD>(pA, ATS, 32 * tt * TP + 32 * tp + 16 * m);
            mma<NTD, NTD>(X[tt], fa, fb);
          }
        }
      // U waves: Z -= K^T X.  S waves: Z = exp(G_C) Z + K^T diag(exp(G_C - G)) X
      if (s_wave) {
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int r = 0; r < 16; ++r) Z[rt][ct][r] *= eGC;
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int r = 0; r < 16; ++r) X[tt][r] *= s_wave ? sEW[32 * tt + acc_row(r, lane)] : -1.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const Frag<NTD> fb = acc_as_b<NTD>(X[tt], m);
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            const Frag<NTI> fa = lds_a_perm<NTI>(pKt, TTS, 32 * rt * TP + 32 * tt + 16 * m);
            mma<NTI, NTD>(Z[rt][ct], fa, fb);
          }
        }
    }
    __syncthreads();
  }

  // ---- write U (waves 0-1) or S (waves 2-3), and g -----------------------------
  float* dst = (s_wave ? a.S : a.U) + unit * D * D;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        dst[(size_t)(32 * rt + acc_row(r, lane0)) * D + col0 + 32 * ct + (lane0 & 31)] = Z[rt][ct][r];
  if (wave == 3 && lane0 == 0) a.g[unit] = (float)g_acc;
}

template <int D, bool F32>
hipError_t launch_t(const BuildArgs& a, int n_blocks, hipStream_t stream) {
  constexpr int lds = DeltaCfg<D, F32>::LDS;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&build_delta_kernel<D, F32>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((build_delta_kernel<D, F32>), dim3(n_blocks), dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

namespace {
bool use_delta2(int d, bool in_f32, const SegTable& seg) {
  if (d != 128 || in_f32) return false;
  for (int s = 0; s < seg.n_seg; ++s)
    if (seg_len(seg, s) > kDelta2MaxSegLen) return false;
  return true;
}
}  // namespace

size_t build_delta_workspace(int d, bool in_f32, const SegTable& seg, int n_chain) {
  return use_delta2(d, in_f32, seg) ? delta2_workspace_bytes(seg, n_chain) : 0;
}

hipError_t launch_build_delta_single(int d, bool in_f32, const BuildArgs& a, int n_blocks, hipStream_t stream) {
  if (d == 128) return in_f32 ? launch_t<128, true>(a, n_blocks, stream) : launch_t<128, false>(a, n_blocks, stream);
  if (d == 64) return in_f32 ? launch_t<64, true>(a, n_blocks, stream) : launch_t<64, false>(a, n_blocks, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_build_delta(int d, bool in_f32, const BuildArgs& a, int n_blocks, void* ws,
                              hipStream_t stream) {
  if (use_delta2(d, in_f32, a.seg)) return launch_build_delta2(a, ws, stream);
  return launch_build_delta_single(d, in_f32, a, n_blocks, stream);
}

}  // namespace hypic
