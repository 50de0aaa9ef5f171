// rerotate.hip -- rotary re-rotation of cached pairs, in place.
//
// [youleyou, linear-layer paragraph] a cached segment of a linear layer whose
// keys carry a rotary encoding is aligned exactly at a new position by
// re-rotating its state.  With keys rotated by R(t) (the pairs (2i, 2i+1) of
// the d_k axis turned by t * theta_i, theta_i = base^(-2i/d_k)), moving the
// segment by p turns every key into R(p) k, every per-token transition into
// R(p) A_t R(p)^T and every write into R(p) k v^T, so the pair becomes
// (R(p) U R(p)^T, R(p) S) with g unchanged.
//
// A pure HBM stream: one workgroup per d x d matrix (S of a unit, or U of a
// unit for the delta family); each thread holds the same float4 column block
// of a row pair (2i, 2i+1), so the row rotation is local, and for U the column
// rotation is local too (a float4 holds two column pairs).  Loads are issued
// before the segment's cos/sin table is formed, so the table's fp64 sincos
// overlaps the memory latency.  Every byte is touched once, so loads and
// stores are non-temporal (measured: 5.26 -> 5.51 TB/s on the warm request's
// 24.7 GB pass; an in-place elementwise torch op over the same buffers runs at
// 5.94 TB/s).
#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

template <int D>
__global__ __launch_bounds__(256) void rerotate_kernel(float* __restrict__ S, float* __restrict__ U,
                                                       const int32_t* __restrict__ pos, int n_chain,
                                                       int units, double base) {
  constexpr int C4 = D / 4;              // float4 per row
  constexpr int PER = D * D / 8 / 256;   // row-pair float4 items per thread
  static_assert(PER >= 1 && D * D / 8 == PER * 256, "one matrix per workgroup");
  __shared__ float2 cs[D / 2];
  const bool two_sided = (int)blockIdx.x >= units;  // U matrices follow the S matrices
  const int u = two_sided ? (int)blockIdx.x - units : (int)blockIdx.x;
  float* M = (two_sided ? U : S) + (size_t)u * D * D;

  f32x4 r0[PER], r1[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int item = threadIdx.x + 256 * k;
    const int rp = item / C4, c4 = item % C4;
    r0[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(M + (size_t)(2 * rp) * D + 4 * c4));
    r1[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(M + (size_t)(2 * rp + 1) * D + 4 * c4));
  }
  if (threadIdx.x < D / 2) {
    const double p = (double)pos[u / n_chain];
    const double theta = pow(base, -2.0 * (double)threadIdx.x / (double)D);
    double sn, c;
    sincos(p * theta, &sn, &c);
    cs[threadIdx.x] = make_float2((float)c, (float)sn);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int item = threadIdx.x + 256 * k;
    const int rp = item / C4, c4 = item % C4;
    const float2 t = cs[rp];
    f32x4 a, b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // rows: (a, b) <- (c a - s b, s a + c b)
      a[j] = fmaf(t.x, r0[k][j], -(t.y * r1[k][j]));
      b[j] = fmaf(t.y, r0[k][j], t.x * r1[k][j]);
    }
    if (two_sided) {  // columns (4c4, 4c4+1) and (4c4+2, 4c4+3): x R^T
      const float2 t0 = cs[2 * c4], t1 = cs[2 * c4 + 1];
      f32x4 a2, b2;
      a2[0] = fmaf(t0.x, a[0], -(t0.y * a[1]));
      a2[1] = fmaf(t0.y, a[0], t0.x * a[1]);
      a2[2] = fmaf(t1.x, a[2], -(t1.y * a[3]));
      a2[3] = fmaf(t1.y, a[2], t1.x * a[3]);
      b2[0] = fmaf(t0.x, b[0], -(t0.y * b[1]));
      b2[1] = fmaf(t0.y, b[0], t0.x * b[1]);
      b2[2] = fmaf(t1.x, b[2], -(t1.y * b[3]));
      b2[3] = fmaf(t1.y, b[2], t1.x * b[3]);
      a = a2;
      b = b2;
    }
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(M + (size_t)(2 * rp) * D + 4 * c4));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(M + (size_t)(2 * rp + 1) * D + 4 * c4));
  }
}

}  // namespace

hipError_t launch_rerotate(int d, float* S, float* U, const int32_t* pos, int n_seg, int n_chain, double base,
                           hipStream_t stream) {
  const int units = n_seg * n_chain;
  const int blocks = units * (U ? 2 : 1);
  if (d == 128)
    hipLaunchKernelGGL(rerotate_kernel<128>, dim3(blocks), dim3(256), 0, stream, S, U, pos, n_chain, units, base);
  else
    hipLaunchKernelGGL(rerotate_kernel<64>, dim3(blocks), dim3(256), 0, stream, S, U, pos, n_chain, units, base);
  return hipGetLastError();
}

}  // namespace hypic
