// compose.hip -- ordered composition of cached pairs along each chain.
//
// [youleyou, linear-layer paragraph] S(C1.C2) = T(C2) S(C1) + S(C2): each
// cached pair is applied by left-multiplying the running state by T_C and
// adding S(C|0).  [hwlabs, section 세그먼트 누적 전이 연산자] the same law gives
// T_ABC = T_C T_B T_A for the transition of the concatenation.
//
// Two kernels:
//  - compose_elem (naive, scalar, diagonal): T is I, exp(g) I or diag(exp(g)),
//    so the chain is elementwise, S <- a_s * S + S_s per element; a pure HBM
//    stream, one thread per 4 consecutive state elements, looping over the
//    segments with the next segment's loads in flight.
//  - compose_dense (delta family): S <- exp(g_s) U_s S + S_s with a dense
//    d x d U_s.  One workgroup per chain, one wave per 32 state columns; the
//    state block stays in registers for the whole chain (it is the B operand
//    of the next product, read straight from the accumulator layout), U_s is
//    double-buffered through LDS, and the product runs on MFMA in three-term
//    split-bf16, which keeps fp32 accuracy on fp32 pairs.
#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

// ---------------------------------------------------------------- elementwise

template <int FAM, int D>
__global__ __launch_bounds__(256) void compose_elem_kernel(const ComposeArgs a) {
  constexpr int V4_PER_CHAIN = D * D / 4;
  constexpr int BLOCKS_PER_CHAIN = V4_PER_CHAIN / 256;
  const int h = blockIdx.x / BLOCKS_PER_CHAIN;
  const int v4 = (blockIdx.x % BLOCKS_PER_CHAIN) * 256 + threadIdx.x;  // float4 index in the chain
  const int row = (v4 * 4) / D;
  const int n_chain = a.n_chain;
  const size_t chain_off = (size_t)h * D * D;
  const size_t seg_stride = (size_t)n_chain * D * D;
  constexpr int GL = (FAM == 2) ? D : 1;

  f32x4 cur;
  if (a.S_init) {
    cur = reinterpret_cast<const f32x4*>(a.S_init + chain_off)[v4];
  } else {
    cur = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const f32x4* Sp = reinterpret_cast<const f32x4*>(a.S + chain_off) + v4;
  f32x4 nxt = Sp[0];
  float gn = 0.f;
  if constexpr (FAM != 0) gn = a.g[(size_t)h * GL + (FAM == 2 ? row : 0)];
  for (int s = 0; s < a.n_seg; ++s) {
    const f32x4 Si = nxt;
    const float gi = gn;
    if (s + 1 < a.n_seg) {
      nxt = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(Sp) + (size_t)(s + 1) * seg_stride);
      if constexpr (FAM != 0) gn = a.g[((size_t)(s + 1) * n_chain + h) * GL + (FAM == 2 ? row : 0)];
    }
    if (a.prefix) {
      reinterpret_cast<f32x4*>(a.prefix + (size_t)s * seg_stride + chain_off)[v4] = cur;
    }
    if constexpr (FAM == 0) {
      cur = cur + Si;
    } else {
      const float e = expf(gi);
#pragma unroll
      for (int j = 0; j < 4; ++j) cur[j] = fmaf(e, cur[j], Si[j]);
    }
  }
  reinterpret_cast<f32x4*>(a.S_out + chain_off)[v4] = cur;

  // g_total: summed in fp64 by the chain's first block
  if (a.g_tot && (blockIdx.x % BLOCKS_PER_CHAIN) == 0 && threadIdx.x < GL) {
    double acc = 0.0;
    if constexpr (FAM != 0) {
      for (int s = 0; s < a.n_seg; ++s) acc += (double)a.g[((size_t)s * n_chain + h) * GL + threadIdx.x];
    }
    a.g_tot[(size_t)h * GL + threadIdx.x] = (float)acc;
  }
}

// ---------------------------------------------------------------- dense (delta)

constexpr int NT_C = 3;  // split terms for fp32-class products

// One wave: T = U * Sblk for the wave's 32 columns, U read from LDS (fp32,
// row pitch P floats), Sblk from the accumulator tiles.
template <int D, int P>
__device__ __forceinline__ void dense_product(const float* __restrict__ sU, const f32x16 (&Sb)[D / 32],
                                              f32x16 (&T)[D / 32], int lane) {
  constexpr int NRT = D / 32;
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) T[rt] = zero16();
  const int h = lane >> 5;
#pragma unroll
  for (int kt = 0; kt < NRT; ++kt) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const Frag<NT_C> fb = acc_as_b<NT_C>(Sb[kt], m);
      const int kcol = 32 * kt + 16 * m + 4 * h;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const float* urow = sU + (32 * rt + (lane & 31)) * P;
        const f32x4 lo = *reinterpret_cast<const f32x4*>(urow + kcol);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(urow + kcol + 8);
        float x[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const Frag<NT_C> fa = split8<NT_C>(x);
        mma<NT_C, NT_C>(T[rt], fa, fb);
      }
    }
  }
}

template <int D, bool WANT_UT>
__global__ __launch_bounds__(D * 2) void compose_dense_kernel(const ComposeArgs a) {
  constexpr int NW = D / 32;         // waves: one per 32 state columns
  constexpr int NTH = NW * 64;
  constexpr int NRT = D / 32;
  constexpr int P = D + 4;           // LDS row pitch (floats)
  constexpr int V4_U = D * D / 4;    // float4 per U matrix
  constexpr int LD_PER_T = V4_U / NTH;

  extern __shared__ __attribute__((aligned(16))) float smem[];
  float* sU0 = smem;
  float* sU1 = smem + D * P;

  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int n_chain = a.n_chain;
  const int col = 32 * wave + (lane & 31);
  const size_t chain_off = (size_t)h * D * D;
  const size_t seg_stride = (size_t)n_chain * D * D;

  // running state block (rows 0..D-1, this wave's 32 columns), accumulator layout
  f32x16 Sb[NRT];
  f32x16 Ut[NRT];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * rt + acc_row(r, lane);
      Sb[rt][r] = a.S_init ? a.S_init[chain_off + (size_t)row * D + col] : 0.f;
      if constexpr (WANT_UT) Ut[rt][r] = (row == col) ? 1.f : 0.f;
    }
  }

  // stage U_0
  f32x4 ureg[LD_PER_T];
  auto load_U = [&](int s) {
    const f32x4* src = reinterpret_cast<const f32x4*>(a.U + (size_t)s * seg_stride + chain_off);
#pragma unroll
    for (int i = 0; i < LD_PER_T; ++i) ureg[i] = src[i * NTH + tid];
  };
  auto store_U = [&](float* dst) {
#pragma unroll
    for (int i = 0; i < LD_PER_T; ++i) {
      const int e = (i * NTH + tid) * 4;
      *reinterpret_cast<f32x4*>(dst + (e / D) * P + (e % D)) = ureg[i];
    }
  };
  load_U(0);
  store_U(sU0);
  __syncthreads();

  double gsum = 0.0;
  for (int s = 0; s < a.n_seg; ++s) {
    float* cur_U = (s & 1) ? sU1 : sU0;
    float* nxt_U = (s & 1) ? sU0 : sU1;
    if (s + 1 < a.n_seg) load_U(s + 1);

    // S_s for this wave's block, accumulator layout
    f32x16 Si[NRT];
    const float* Sg = a.S + (size_t)s * seg_stride + chain_off;
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) Si[rt][r] = Sg[(size_t)(32 * rt + acc_row(r, lane)) * D + col];
    const float gs = a.g[(size_t)s * n_chain + h];
    gsum += (double)gs;

    if (a.prefix) {
      float* pp = a.prefix + (size_t)s * seg_stride + chain_off;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) pp[(size_t)(32 * rt + acc_row(r, lane)) * D + col] = Sb[rt][r];
    }

    f32x16 T[NRT];
    dense_product<D, P>(cur_U, Sb, T, lane);
    const float e = expf(gs);
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) Sb[rt][r] = fmaf(e, T[rt][r], Si[rt][r]);

    if constexpr (WANT_UT) {
      f32x16 T2[NRT];
      dense_product<D, P>(cur_U, Ut, T2, lane);
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) Ut[rt] = T2[rt];
    }

    if (s + 1 < a.n_seg) store_U(nxt_U);
    __syncthreads();
  }

#pragma unroll
  for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const size_t idx = chain_off + (size_t)(32 * rt + acc_row(r, lane)) * D + col;
      a.S_out[idx] = Sb[rt][r];
      if constexpr (WANT_UT) a.U_tot[idx] = Ut[rt][r];
    }
  if (a.g_tot && tid == 0) a.g_tot[h] = (float)gsum;
}

template <int D, bool UT>
hipError_t launch_dense_t(const ComposeArgs& a, hipStream_t stream) {
  const size_t lds = 2 * (size_t)D * (D + 4) * sizeof(float);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&compose_dense_kernel<D, UT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((compose_dense_kernel<D, UT>), dim3(a.n_chain), dim3(D * 2), lds, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dense_d(const ComposeArgs& a, hipStream_t stream) {
  return a.U_tot ? launch_dense_t<D, true>(a, stream) : launch_dense_t<D, false>(a, stream);
}

template <int FAM, int D>
hipError_t launch_elem_t(const ComposeArgs& a, hipStream_t stream) {
  const int blocks = a.n_chain * (D * D / 4 / 256);
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

hipError_t launch_compose_dense(int d, const ComposeArgs& a, hipStream_t stream) {
  if (d == 128) return launch_dense_d<128>(a, stream);
  if (d == 64) return launch_dense_d<64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace hypic
