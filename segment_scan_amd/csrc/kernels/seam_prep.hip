// seam_prep.hip -- the part of the delta-rule seam-window step that does not
// depend on the running state, for every window at once.
//
// [youleyou, full-attention paragraph] each reused segment's first w tokens
// are run through the linear layer on the running state.  In the chunk form of
// the delta rule (sub-chunks of up to 8 tokens; G the gate prefix within the
// sub-chunk, Gamma_ts = exp(G_t - G_s), n tokens) the state enters only
// through R = V - diag(exp(G)) K S:
//   S' = exp(G_n) S + (C K)^T R,             C = Abar^T diag(exp(G_n - G))
//   O  = diag(exp(G)) Q S + W2 R,            W2 = (tril(Q K^T) o Gamma) Abar
//   Abar = (I + strict_lower(diag(b) (Gamma o K K^T)))^-1 diag(b).
// C, W2 and the gate factors depend on the window's tokens alone, so this
// kernel forms them for all (segment, sub-chunk, chain) windows in parallel --
// one wave each, fp32 -- and the serial chain kernel only applies them.
#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

constexpr int SUB = 8;

template <int D, bool IN_F32>
__global__ __launch_bounds__(64) void seam_prep_kernel(const SeamArgs a, float* ws, int n_sub) {
  __shared__ __attribute__((aligned(16))) float sK[SUB][D];
  __shared__ __attribute__((aligned(16))) float sQ[SUB][D];
  __shared__ float sKK[SUB * SUB], sQK[SUB * SUB];
  __shared__ float sB[SUB], sG[SUB];

  const int n_chain = a.n_chain;
  const int chain = blockIdx.x % n_chain;
  const int rest = blockIdx.x / n_chain;
  const int sub = rest % n_sub, seg = rest / n_sub;
  const int t0 = sub * SUB;
  const int n = min(SUB, a.w - t0);
  const size_t tok0 = (size_t)seg * a.w + t0;
  const int lane = threadIdx.x;

  // ---- bf16 tokens: [K; Q] K^T on 16x16x32 bf16 MFMA (exact products), operands
  // straight from memory: lane (row l16, group g) holds k = 32 ks + 8 g .. of K
  // row l16 (Q row l16 - 8) as A and of key l16 as B; output row 4 g + j, column l16
  if constexpr (!IN_F32) {
    const int l16 = lane & 15, g = lane >> 4, t = l16 & (SUB - 1);
    const uint16_t* arow = reinterpret_cast<const uint16_t*>(l16 < SUB ? a.k : a.q) +
                           ((tok0 + t) * n_chain + chain) * D + 8 * g;
    const uint16_t* brow = reinterpret_cast<const uint16_t*>(a.k) + ((tok0 + t) * n_chain + chain) * D + 8 * g;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      bf16x8 fa{}, fb{};
      if (t < n) fa = *reinterpret_cast<const bf16x8*>(arow + 32 * ks);
      if (l16 < SUB && t < n) fb = *reinterpret_cast<const bf16x8*>(brow + 32 * ks);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
    }
    if (l16 < SUB) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * g + j;
        (r < SUB ? sKK : sQK)[(r & (SUB - 1)) * SUB + l16] = acc[j];
      }
    }
  }
  // ---- fp32 tokens: the sub-chunk's keys and queries (fp32), zero past n ----------
  if constexpr (IN_F32)
  for (int i = lane; i < 2 * SUB * (D / 8); i += 64) {
    const int which = i / (SUB * (D / 8)), j = i % (SUB * (D / 8));
    const int t = j / (D / 8), d8 = j % (D / 8);
    float x[8];
    if (t < n) {
      load8<IN_F32>(which ? a.q : a.k, ((tok0 + t) * n_chain + chain) * D + 8 * d8, x);
    } else {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) x[jj] = 0.f;
    }
    float* dst = (which ? &sQ[t][0] : &sK[t][0]) + 8 * d8;
    *reinterpret_cast<f32x4*>(dst) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
  }
  float lg = 0.f;
  if (lane < SUB) {
    const size_t idx = (tok0 + lane) * n_chain + chain;
    sB[lane] = lane < n ? load1<IN_F32>(a.beta, idx) : 0.f;
    lg = (lane < n && a.lg) ? load1<IN_F32>(a.lg, idx) : 0.f;
  }
  const float G = wave_incl_scan(lg);  // lanes >= SUB add zeros
  if (lane < SUB) sG[lane] = G;
  __syncthreads();

  // ---- lane p: one of the 28 products k_t.k_s (s < t) or 36 products q_t.k_s (s <= t)
  if constexpr (IN_F32) {
    int t, s;
    bool kk;
    if (lane < SUB * (SUB - 1) / 2) {
      t = 1;
      int r = lane;
      while (r >= t) { r -= t; ++t; }
      s = r;
      kk = true;
    } else {
      t = 0;
      int r = lane - SUB * (SUB - 1) / 2;
      while (r > t) { r -= t + 1; ++t; }
      s = r;
      kk = false;
    }
    const float* x = kk ? &sK[t][0] : &sQ[t][0];
    float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; d += 2) {
      acc0 = fmaf(x[d], sK[s][d], acc0);
      acc1 = fmaf(x[d + 1], sK[s][d + 1], acc1);
    }
    (kk ? sKK : sQK)[t * SUB + s] = acc0 + acc1;
  }
  __syncthreads();

  // ---- lane s < 8: column s of (I + M)^-1 (M_ts = b_t Gamma_ts k_t.k_s), then C, W2
  float* rec = ws + (size_t)blockIdx.x * SEAM_REC_FLOATS;
  if (lane < SUB) {
    const int s = lane;
    const float Gn = sG[SUB - 1];  // padded tokens carry zero gates
    float x[SUB];
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < t; ++u) acc = fmaf(sB[t] * __expf(sG[t] - sG[u]) * sKK[t * SUB + u], x[u], acc);
      x[t] = (t < s) ? 0.f : ((t == s) ? 1.f : -acc);
    }
    const float bs = sB[s];
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      rec[t * SUB + s] = x[t] * bs * __expf(Gn - sG[t]);  // C^T[t][s] = Abar[t][s] exp(G_n - G_t)
      float w2 = 0.f;
#pragma unroll
      for (int u = 0; u <= t; ++u) w2 = fmaf(__expf(sG[t] - sG[u]) * sQK[t * SUB + u], x[u] * bs, w2);
      rec[SUB * SUB + t * SUB + s] = w2;  // W2[t][s]
    }
    rec[2 * SUB * SUB + s] = __expf(sG[s]);
    if (s == 0) rec[2 * SUB * SUB + SUB] = __expf(Gn);
  }
  constexpr int USED = 2 * SUB * SUB + SUB + 1;  // the rest of the record is padding
  if (lane >= SUB && lane < SUB + SEAM_REC_FLOATS - USED) rec[USED + lane - SUB] = 0.f;
}

}  // namespace

size_t seam_workspace_bytes(int n_seg, int w, int n_chain) {
  const int n_sub = (w + SUB - 1) / SUB;
  return (size_t)n_seg * n_sub * n_chain * SEAM_REC_FLOATS * 4;
}

hipError_t launch_seam_prep(int d, bool in_f32, const SeamArgs& a, float* ws, hipStream_t stream) {
  const int n_sub = (a.w + SUB - 1) / SUB;
  const dim3 grid(a.n_seg * n_sub * a.n_chain);
  if (d == 128) {
    if (in_f32) hipLaunchKernelGGL((seam_prep_kernel<128, true>), grid, dim3(64), 0, stream, a, ws, n_sub);
    else hipLaunchKernelGGL((seam_prep_kernel<128, false>), grid, dim3(64), 0, stream, a, ws, n_sub);
  } else if (d == 64) {
    if (in_f32) hipLaunchKernelGGL((seam_prep_kernel<64, true>), grid, dim3(64), 0, stream, a, ws, n_sub);
    else hipLaunchKernelGGL((seam_prep_kernel<64, false>), grid, dim3(64), 0, stream, a, ws, n_sub);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace hypic
