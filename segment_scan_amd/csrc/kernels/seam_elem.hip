// seam_elem.hip -- the seam-window step for the naive, scalar-decay and
// diagonal-gate families, fused with the composition of the body pairs.
//
// [youleyou, full-attention paragraph] at reuse the first w tokens of each
// segment are run on the running state, each emitting o_t = S_t^T q_t, before
// the segment's cached body pair is applied [youleyou, linear-layer paragraph]:
// S <- T_B S + S_B, here with T_B = I, exp(g) I or diag(exp(g)).
//
// For these families every state column evolves on its own and every update
// is elementwise in the column (S[:, c] <- a_t o S[:, c] + k_t v_t[c]), so one
// thread owns one column of one chain for the whole request and keeps it in
// registers: a window token costs 2d fused multiply-adds per thread (update and
// output dot product) and the body pair is a coalesced stream over rows.  The
// window tokens are staged in LDS in groups of 8; each group's body-pair column
// is already in flight while the window runs.
#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

constexpr int GRP = 8;  // window tokens staged at once

template <int FAM, int D, bool IN_F32>
__global__ __launch_bounds__(D) void seam_elem_kernel(const SeamArgs a) {
  __shared__ __attribute__((aligned(16))) float sK[GRP][D];
  __shared__ __attribute__((aligned(16))) float sQ[GRP][D];
  __shared__ __attribute__((aligned(16))) float sA[GRP][D];  // diag: per-channel gates
  __shared__ float sAs[GRP];                                   // scalar: per-token gates
  __shared__ __attribute__((aligned(16))) float sE[D];         // body gates exp(g)

  const int chain = blockIdx.x;
  const int c = threadIdx.x;  // the thread's state column
  const int n_chain = a.n_chain;
  const size_t chain_off = (size_t)chain * D * D;
  const size_t seg_stride = (size_t)n_chain * D * D;

  float S[D];
#pragma unroll
  for (int d = 0; d < D; ++d) S[d] = a.S_run[chain_off + (size_t)d * D + c];

  float a_chain = 1.f;  // scalar family with one gate per chain (fp32 log gate)
  if (FAM == 1 && a.gate_per_chain) a_chain = __expf(reinterpret_cast<const float*>(a.lg)[chain]);

  for (int seg = 0; seg < a.n_seg; ++seg) {
    // body pair column of this segment: in flight while the window runs
    float B[D];
    if (a.bS) {
      const float* src = a.bS + (size_t)seg * seg_stride + chain_off + c;
#pragma unroll
      for (int d = 0; d < D; ++d) B[d] = src[(size_t)d * D];
    }
    for (int t0 = 0; t0 < a.w; t0 += GRP) {
      const int n = min(GRP, a.w - t0);
      const size_t tok0 = (size_t)seg * a.w + t0;
      __syncthreads();  // the previous group's readers are done
      float vt[GRP];
#pragma unroll
      for (int t = 0; t < GRP; ++t) {
        const size_t row = ((tok0 + t) * n_chain + chain) * D + c;
        sK[t][c] = t < n ? load1<IN_F32>(a.k, row) : 0.f;
        sQ[t][c] = t < n ? load1<IN_F32>(a.q, row) : 0.f;
        vt[t] = t < n ? load1<IN_F32>(a.v, row) : 0.f;
        if constexpr (FAM == 2) sA[t][c] = t < n ? __expf(load1<IN_F32>(a.lg, row)) : 1.f;
      }
      if constexpr (FAM == 1) {
        if (!a.gate_per_chain && c < GRP)
          sAs[c] = c < n ? __expf(load1<IN_F32>(a.lg, (tok0 + c) * n_chain + chain)) : 1.f;
      }
      __syncthreads();
      for (int t = 0; t < n; ++t) {
        const float at = FAM == 1 ? (a.gate_per_chain ? a_chain : sAs[t]) : 1.f;
        float o0 = 0.f, o1 = 0.f;
#pragma unroll
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const f32x4 k4 = *reinterpret_cast<const f32x4*>(&sK[t][4 * d4]);
          const f32x4 q4 = *reinterpret_cast<const f32x4*>(&sQ[t][4 * d4]);
          f32x4 a4 = {at, at, at, at};
          if constexpr (FAM == 2) a4 = *reinterpret_cast<const f32x4*>(&sA[t][4 * d4]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float& s = S[4 * d4 + j];
            s = (FAM == 0) ? fmaf(k4[j], vt[t], s) : fmaf(a4[j], s, k4[j] * vt[t]);
            if (j & 1) o1 = fmaf(s, q4[j], o1); else o0 = fmaf(s, q4[j], o0);
          }
        }
        a.o[((tok0 + t) * n_chain + chain) * D + c] = o0 + o1;
      }
    }
    if (a.bS) {
      if constexpr (FAM == 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) S[d] += B[d];
      } else if constexpr (FAM == 1) {
        const float e = __expf(a.bg[(size_t)seg * n_chain + chain]);
#pragma unroll
        for (int d = 0; d < D; ++d) S[d] = fmaf(e, S[d], B[d]);
      } else {
        __syncthreads();
        sE[c] = __expf(a.bg[((size_t)seg * n_chain + chain) * D + c]);
        __syncthreads();
#pragma unroll
        for (int d = 0; d < D; ++d) S[d] = fmaf(sE[d], S[d], B[d]);
      }
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) a.S_run[chain_off + (size_t)d * D + c] = S[d];
}

template <int FAM, int D>
hipError_t launch_fam_d(bool in_f32, const SeamArgs& a, hipStream_t stream) {
  if (in_f32)
    hipLaunchKernelGGL((seam_elem_kernel<FAM, D, true>), dim3(a.n_chain), dim3(D), 0, stream, a);
  else
    hipLaunchKernelGGL((seam_elem_kernel<FAM, D, false>), dim3(a.n_chain), dim3(D), 0, stream, a);
  return hipGetLastError();
}

template <int FAM>
hipError_t launch_fam(int d, bool in_f32, const SeamArgs& a, hipStream_t stream) {
  if (d == 128) return launch_fam_d<FAM, 128>(in_f32, a, stream);
  if (d == 64) return launch_fam_d<FAM, 64>(in_f32, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_seam_elem(int fam, int d, bool in_f32, const SeamArgs& a, hipStream_t stream) {
  switch (fam) {
    case 0: return launch_fam<0>(d, in_f32, a, stream);
    case 1: return launch_fam<1>(d, in_f32, a, stream);
    case 2: return launch_fam<2>(d, in_f32, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hypic
