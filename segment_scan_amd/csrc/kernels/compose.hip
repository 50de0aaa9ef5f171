// compose.hip -- ordered composition of cached pairs along each chain.
//
// [youleyou, linear-layer paragraph] S(C1.C2) = T(C2) S(C1) + S(C2): each
// cached pair is applied by left-multiplying the running state by T_C and
// adding S(C|0).  [hwlabs, section 세그먼트 누적 전이 연산자] the same law gives
// T_ABC = T_C T_B T_A for the transition of the concatenation.
//
// Naive, scalar and diagonal families: T is I, exp(g) I or diag(exp(g)), so
// the chain is elementwise, S <- a_s * S + S_s per element; a pure HBM stream,
// one thread per 4 consecutive state elements, looping over the segments with
// the next eight segments' loads in flight.  (The dense delta-family chain is in
// chain.hip.)
#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

// ---------------------------------------------------------------- elementwise

template <int FAM, int D>
__global__ __launch_bounds__(256) void compose_elem_kernel(const ComposeArgs a) {
  constexpr int V4_PER_CHAIN = D * D / 4;
  constexpr int BLOCKS_PER_CHAIN = V4_PER_CHAIN / 256;
  const int h = blockIdx.x / BLOCKS_PER_CHAIN;  // output (chain, or group of pairs of a chain)
  const int v4 = (blockIdx.x % BLOCKS_PER_CHAIN) * 256 + threadIdx.x;  // float4 index in the state
  const int row = (v4 * 4) / D;
  const int n_chain = a.n_chain;
  const size_t chain_off = (size_t)h * D * D;  // outputs and start state
  // the output's first pair: group h / n_chain of chain h % n_chain
  const size_t pair0 = (size_t)(h / n_chain) * a.n_seg * n_chain + h % n_chain;
  const size_t seg_stride = (size_t)n_chain * D * D;
  constexpr int GL = (FAM == 2) ? D : 1;

  f32x4 cur;
  if (a.S_init) {
    cur = reinterpret_cast<const f32x4*>(a.S_init + chain_off)[v4];
  } else {
    cur = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float* Sp = a.S + pair0 * D * D + 4 * (size_t)v4;
  // PF segments' loads in flight per thread (a register ring refilled group by
  // group), so that few threads per chain still keep the memory system busy
  constexpr int PF = 8;
  f32x4 buf[PF];
  float gb[PF];
  auto issue = [&](int s0) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int s = min(s0 + j, a.n_seg - 1);  // past the end: a reread, never used
      buf[j] = *reinterpret_cast<const f32x4*>(Sp + (size_t)s * seg_stride);
      if constexpr (FAM != 0) gb[j] = a.g[(pair0 + (size_t)s * n_chain) * GL + (FAM == 2 ? row : 0)];
    }
  };
  issue(0);
  for (int s0 = 0; s0 < a.n_seg; s0 += PF) {
    f32x4 cb[PF];
    float cg[PF];
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      cb[j] = buf[j];
      cg[j] = FAM != 0 ? gb[j] : 0.f;
    }
    if (s0 + PF < a.n_seg) issue(s0 + PF);
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int s = s0 + j;
      if (s >= a.n_seg) break;
      if (a.prefix) reinterpret_cast<f32x4*>(a.prefix + (size_t)s * seg_stride + chain_off)[v4] = cur;
      if constexpr (FAM == 0) {
        cur = cur + cb[j];
      } else {
        const float e = expf(cg[j]);
#pragma unroll
        for (int k = 0; k < 4; ++k) cur[k] = fmaf(e, cur[k], cb[j][k]);
      }
    }
  }
  reinterpret_cast<f32x4*>(a.S_out + chain_off)[v4] = cur;

  // g_total: summed in fp64 by the chain's first block
  if (a.g_tot && (blockIdx.x % BLOCKS_PER_CHAIN) == 0 && threadIdx.x < GL) {
    double acc = 0.0;
    if constexpr (FAM != 0) {
      for (int s = 0; s < a.n_seg; ++s) acc += (double)a.g[(pair0 + (size_t)s * n_chain) * GL + threadIdx.x];
    }
    a.g_tot[(size_t)h * GL + threadIdx.x] = (float)acc;
  }
}

template <int FAM, int D>
hipError_t launch_elem_t(const ComposeArgs& a, hipStream_t stream) {
  const int blocks = a.n_out * (D * D / 4 / 256);
  hipLaunchKernelGGL((compose_elem_kernel<FAM, D>), dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compose_elem(int fam, int d, const ComposeArgs& a, hipStream_t stream) {
  if (d == 128) {
    switch (fam) {
      case 0: return launch_elem_t<0, 128>(a, stream);
      case 1: return launch_elem_t<1, 128>(a, stream);
      case 2: return launch_elem_t<2, 128>(a, stream);
    }
  } else if (d == 64) {
    switch (fam) {
      case 0: return launch_elem_t<0, 64>(a, stream);
      case 1: return launch_elem_t<1, 64>(a, stream);
      case 2: return launch_elem_t<2, 64>(a, stream);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace hypic
