// seam_kda.hip -- the seam-window step for the KDA family (the delta rule with
// one gate per key channel), fused with the composition of the body pairs.
//
// [youleyou, full-attention paragraph] at reuse the first w tokens of each
// segment are run on the running state, each emitting o_t = S_t^T q_t, before
// the segment's cached body pair is applied [youleyou, linear-layer paragraph]:
// S <- T_B S + S_B with the dense T_B = exp(g) U.
//
// One workgroup of 4 waves per chain; the running state S (d x d fp32) stays in
// MFMA accumulators for the whole request, wave w owning columns 32w .. 32w+31
// (at d = 64 waves 2-3 only stage data).  In that layout a lane holds half the
// rows of one column, so a window token
//   S <- diag(alpha) S,  u = S^T k,  S <- S + beta k (v - u)^T,  o = S^T q
// is per-lane work plus one cross-half add for each of u and o; the token's
// k, q, alpha are read from LDS as broadcasts.  The body product U S runs on
// bf16 MFMA with U split into two bf16 terms (three for fp32 tokens) and staged
// in LDS in two halves of rows, the state used as the B operand straight from
// the accumulators.
#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

constexpr int GRP = 8;  // window tokens staged at once

template <int D, bool IN_F32>
struct SeamKdaCfg {
  static constexpr int NT = IN_F32 ? 3 : 2;  // bf16 terms of U and of the state as B operand
  static constexpr int NRT = D / 32;         // row tiles of the state
  static constexpr int NCT = D / 32;         // column tiles (one per wave; waves >= NCT idle)
  static constexpr int UP = D + 8;           // bf16 pitch of a staged U row
  static constexpr int HR = D / 2;           // U rows staged at once
  static constexpr int U_BYTES = NT * HR * UP * 2;
  static constexpr int W_BYTES = 4 * GRP * D * 4;  // k, q, alpha, v of a group
  static constexpr int OFF_U = 0;
  static constexpr int OFF_W = OFF_U + U_BYTES;
  static constexpr int OFF_B = OFF_W + W_BYTES;    // beta of a group
  static constexpr int LDS = OFF_B + GRP * 4;
};

template <int D, bool IN_F32>
__global__ __launch_bounds__(256) void seam_kda_kernel(const SeamArgs a) {
  using Cfg = SeamKdaCfg<D, IN_F32>;
  constexpr int NT = Cfg::NT, NRT = Cfg::NRT, NCT = Cfg::NCT, UP = Cfg::UP, HR = Cfg::HR;
  constexpr int UTS = HR * UP;  // term stride of the staged U half
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  bf16_t* sU = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_U);
  float* sK = reinterpret_cast<float*>(smem + Cfg::OFF_W);
  float* sQ = sK + GRP * D;
  float* sA = sQ + GRP * D;
  float* sV = sA + GRP * D;
  float* sB = reinterpret_cast<float*>(smem + Cfg::OFF_B);

  const int chain = blockIdx.x;
  const int n_chain = a.n_chain;
  const int tid = threadIdx.x;
  const int lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wave = tid >> 6;
  const bool owner = wave < NCT;  // this wave holds state columns
  const int col = 32 * wave + l32;
  const size_t chain_off = (size_t)chain * D * D;

  f32x16 Z[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      Z[rt][r] = owner ? a.S_run[chain_off + (size_t)(32 * rt + acc_row(r, lane)) * D + col] : 0.f;

  for (int seg = 0; seg < a.n_seg; ++seg) {
    // ---- window tokens, GRP at a time ---------------------------------------
    for (int t0 = 0; t0 < a.w; t0 += GRP) {
      const int n = min(GRP, a.w - t0);
      const size_t tok0 = (size_t)seg * a.w + t0;
      __syncthreads();  // the previous group's (or body's) readers are done
      for (int e = tid; e < GRP * D; e += 256) {
        const int t = e / D, c = e % D;
        const size_t row = ((tok0 + t) * n_chain + chain) * D + c;
        const bool in = t < n;
        sK[e] = in ? load1<IN_F32>(a.k, row) : 0.f;
        sQ[e] = in ? load1<IN_F32>(a.q, row) : 0.f;
        sV[e] = in ? load1<IN_F32>(a.v, row) : 0.f;
        sA[e] = in ? __expf(load1<IN_F32>(a.lg, row)) : 1.f;
      }
      if (tid < GRP) sB[tid] = tid < n ? load1<IN_F32>(a.beta, (tok0 + tid) * n_chain + chain) : 0.f;
      __syncthreads();
      if (owner) {
        for (int t = 0; t < n; ++t) {
          const float* kt = sK + t * D;
          const float* qt = sQ + t * D;
          const float* at = sA + t * D;
          float up = 0.f;
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int row0 = 32 * rt + 8 * r4 + 4 * h;  // rows row0 .. row0+3 are elements 4*r4 .. 4*r4+3
              const f32x4 a4 = *reinterpret_cast<const f32x4*>(at + row0);
              const f32x4 k4 = *reinterpret_cast<const f32x4*>(kt + row0);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float s = Z[rt][4 * r4 + j] * a4[j];
                Z[rt][4 * r4 + j] = s;
                up = fmaf(s, k4[j], up);
              }
            }
          const float u = up + __shfl_xor(up, 32, 64);
          const float bw = sB[t] * (sV[t * D + col] - u);
          float op = 0.f;
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int row0 = 32 * rt + 8 * r4 + 4 * h;
              const f32x4 k4 = *reinterpret_cast<const f32x4*>(kt + row0);
              const f32x4 q4 = *reinterpret_cast<const f32x4*>(qt + row0);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float s = fmaf(k4[j], bw, Z[rt][4 * r4 + j]);
                Z[rt][4 * r4 + j] = s;
                op = fmaf(s, q4[j], op);
              }
            }
          const float o = op + __shfl_xor(op, 32, 64);
          if (h == 0) a.o[((tok0 + t) * n_chain + chain) * D + col] = o;
        }
      }
    }
    if (!a.bS) continue;

    // ---- body pair: S <- exp(g) U S + S_B ---------------------------------------
    const size_t unit = (size_t)seg * n_chain + chain;
    const float eg = __expf(a.bg[unit]);
    const float* Ug = a.bU + unit * D * D;
    const float* Sg = a.bS + unit * D * D;
    f32x16 W[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) W[rt] = zero16();
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {  // unrolled: W is indexed by hf
      __syncthreads();  // the window's (or the previous half's) readers are done
      // stage U rows hf*HR .. hf*HR+HR-1 split into NT bf16 terms
      for (int e = tid; e < HR * (D / 8); e += 256) {
        const int r = e / (D / 8), c8 = e % (D / 8);
        float x[8];
        load8<true>(Ug, (size_t)(hf * HR + r) * D + 8 * c8, x);
        const Frag<NT> f = split8<NT>(x);
#pragma unroll
        for (int i = 0; i < NT; ++i) st8(sU + i * UTS + r * UP + 8 * c8, f.t[i]);
      }
      __syncthreads();
      if (owner) {
        const bf16_t* pU = sU + l32 * UP + 4 * h;
#pragma unroll
        for (int rti = 0; rti < NRT; ++rti)
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            const Frag<NT> fb = acc_as_b<NT>(Z[rti], m);
#pragma unroll
            for (int ro = 0; ro < NRT / 2; ++ro) {
              const Frag<NT> fa = lds_a_perm<NT>(pU, UTS, 32 * ro * UP + 32 * rti + 16 * m);
              mma<NT, NT>(W[hf * (NRT / 2) + ro], fa, fb);
            }
          }
      }
    }
    if (owner) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          Z[rt][r] = fmaf(eg, W[rt][r], Sg[(size_t)(32 * rt + acc_row(r, lane)) * D + col]);
    }
  }
  if (owner) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) a.S_run[chain_off + (size_t)(32 * rt + acc_row(r, lane)) * D + col] = Z[rt][r];
  }
}

template <int D, bool F32>
hipError_t launch_t(const SeamArgs& a, hipStream_t stream) {
  constexpr int lds = SeamKdaCfg<D, F32>::LDS;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&seam_kda_kernel<D, F32>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((seam_kda_kernel<D, F32>), dim3(a.n_chain), dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_seam_kda(int d, bool in_f32, const SeamArgs& a, hipStream_t stream) {
  if (d == 128) return in_f32 ? launch_t<128, true>(a, stream) : launch_t<128, false>(a, stream);
  if (d == 64) return in_f32 ? launch_t<64, true>(a, stream) : launch_t<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace hypic
