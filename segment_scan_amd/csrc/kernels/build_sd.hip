// build_sd.hip -- segment build for the naive, scalar-decay and diagonal-gate
// families: emits S(C|0) and the log-transition g of every (segment, chain).
//
// [youleyou, linear-layer paragraph] T_C is the product of the segment's
// per-token transitions and S(C|0) its final state from a zero start.  For
// these families the transition is (a diagonal of) exponentials of summed log
// gates, and the zero-start state has the closed form
//     S(C|0) = sum_t diag(exp(g - G_t)) k_t v_t^T,   g = G_L,
// where G_t is the inclusive prefix sum of the log gates.  The kernel streams
// 64-token chunks and joins them with the composition law of the same
// paragraph: S <- diag(exp(G_chunk)) S + Ktil_c^T V_c, Ktil weighted to the
// chunk end.  The chunk product is a d x 64 x d contraction over tokens, run on
// MFMA with the decay-weighted keys split into bf16 terms (values are exact
// bf16 inputs).
//
// Grid: one workgroup per (segment, chain) unit, 4d threads (8 waves at d =
// 128, two 32 x 32 state tiles each).  Per chunk: the 64 x d key and value
// tiles are loaded with 16-byte loads (4 tokens x 8 channels per thread; half
// the threads keys and gates, half values), transposed in registers and written
// to LDS as [channel][token] tiles, so each MFMA operand is one 16-byte LDS read.
#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

constexpr int C = 64;  // tokens per chunk

// Raw (unconverted) 8 consecutive input elements: 16 bytes of bf16 or 32 of fp32.
template <bool IN_F32>
struct Raw8 {
  uint4 w[IN_F32 ? 2 : 1];
};

// 8 consecutive elements at byte offset voff + soff of a buffer (zeros past its end).
template <bool IN_F32>
__device__ __forceinline__ Raw8<IN_F32> ldraw8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  Raw8<IN_F32> x;
  x.w[0] = buffer_load16(r, voff, soff);
  if constexpr (IN_F32) x.w[1] = buffer_load16(r, voff + 16, soff);
  return x;
}

template <bool IN_F32>
__device__ __forceinline__ void cvt8(const Raw8<IN_F32>& r, float (&x)[8]) {
  if constexpr (IN_F32) {
    const uint32_t u[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w, r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = __uint_as_float(u[j]);
  } else {
    const uint32_t u[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(u[j] << 16);
      x[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
  }
}

// ORDERED: workgroup rows read their segment from the launch's slot table
// (ragged launches); a contiguous launch of equal lengths computes it, which
// keeps the table lookup (and the registers it costs this register-bound
// kernel) out of their code.
// TOK: tokens per staging thread; the workgroup has 2 (C / TOK) (D / 8)
// threads (half stage keys and gates, half values).
#ifndef HYPIC_SD_WPE
#define HYPIC_SD_WPE 2
#endif
#ifndef HYPIC_SD_SUB
#define HYPIC_SD_SUB 4
#endif
template <int FAM, int D, bool IN_F32, bool ORDERED, int TOK>
__global__ __launch_bounds__(2 * (C / TOK) * (D / 8)) __attribute__((amdgpu_waves_per_eu(HYPIC_SD_WPE)))
void build_sd_kernel(const BuildArgs a) {
  constexpr int NTK = IN_F32 ? 3 : 2;  // bf16 terms of decay-weighted keys
  constexpr int NTV = IN_F32 ? 3 : 1;  // bf16 terms of values (bf16 inputs are exact)
  constexpr int NRT = D / 32;          // 32-row tiles along d
  constexpr int NTHR = 2 * (C / TOK) * (D / 8);
  constexpr int NWAVE = NTHR / 64;     // waves of the workgroup
  constexpr int TPW = NRT * NRT / NWAVE;  // accumulator tiles per wave
  constexpr int NTB = C / TOK;         // token blocks of a chunk
  static_assert(TPW >= 1 && NRT * NRT == TPW * NWAVE, "tiles per wave");
  constexpr bool DIAG = (FAM == 2);
  constexpr bool GATED = (FAM == 1 || FAM == 2);

  __shared__ __attribute__((aligned(16))) bf16_t sK[NTK][D * C];
  __shared__ __attribute__((aligned(16))) bf16_t sV[NTV][D * C];
  __shared__ float sW[C];        // scalar: weight exp(G_C - G_t)
  __shared__ __attribute__((aligned(16))) float sTot[NTB][D];  // diag: per-token-block sums of log gates
  __shared__ float sGC[D];       // chunk log-transition (scalar: entry 0)
  __shared__ float sEGC[D];      // exp of it

  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = wave_id();
  const int n_chain = a.n_chain;
  const int u_local = blockIdx.x;
  const int slot = u_local / n_chain;
  const int h = u_local % n_chain;
  const int len0 = a.seg.end[0] - a.seg.beg[0];
  const int t_begin = ORDERED ? a.seg.beg[slot] : a.seg.beg[0] + slot * len0;
  const int t_end = ORDERED ? a.seg.end[slot] : t_begin + len0;
  const size_t unit = (size_t)(ORDERED ? a.seg.out[slot] : a.seg.out[0] + slot) * n_chain + h;

  f32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; ++i) acc[i] = zero16();

  double g_acc = 0.0;  // scalar: lane 0 of wave 0; diag: thread tid < D for channel tid

  // staging role: the first half of the waves stage keys (and diagonal gates),
  // the second values (a wave-uniform choice, so the source is a scalar base)
  const bool is_k = wave_id_uniform() < NWAVE / 2;
  const bool is_v = !is_k;
  const int sid = is_k ? tid : tid - NTHR / 2;
  const int tb = sid % NTB;  // block of TOK tokens
  const int db = sid / NTB;  // 8-channel block
  const void* src = is_k ? a.k : a.v;
  constexpr uint32_t ESZ = IN_F32 ? 4 : 2;
  const uint32_t row_bytes = (uint32_t)n_chain * D * ESZ;  // one token of all chains
  const uint32_t voff = (uint32_t)(tb * TOK) * row_bytes + db * 8 * ESZ;

  // raw inputs of the chunk being staged; the next chunk's are loaded while the
  // matrix cores work on this one.  Buffer loads over the chunk's valid rows:
  // tokens past the segment's end read as zeros.
  Raw8<IN_F32> rx[TOK];
  Raw8<IN_F32> rg[TOK];
  float lg_scalar = 0.f;
  auto issue_loads = [&](int c0) {
    const int nv = min(C, t_end - c0);
    const size_t row0 = ((size_t)c0 * n_chain + h) * D * ESZ;  // byte offset of token c0, chain h
    const uint32_t bytes = (uint32_t)(nv - 1) * row_bytes + D * ESZ;
    {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(reinterpret_cast<const char*>(src) + row0, bytes);
#pragma unroll
      for (int r = 0; r < TOK; ++r) rx[r] = ldraw8<IN_F32>(rs, voff, r * row_bytes);
    }
    if constexpr (DIAG) {
      if (is_k) {
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(reinterpret_cast<const char*>(a.lg) + row0, bytes);
#pragma unroll
        for (int r = 0; r < TOK; ++r) rg[r] = ldraw8<IN_F32>(rs, voff, r * row_bytes);
      }
    }
    if constexpr (FAM == 1) {
      if (wave == 0) {
        lg_scalar = 0.f;
        if (lane < nv)
          lg_scalar = a.gate_per_chain ? reinterpret_cast<const float*>(a.lg)[h]
                                       : load1<IN_F32>(a.lg, (size_t)(c0 + lane) * n_chain + h);
      }
    }
  };
  issue_loads(t_begin);

  for (int c0 = t_begin; c0 < t_end; c0 += C) {
    // ---- gates: scalar prefix over the chunk (wave 0) -------------------------
    if constexpr (FAM == 1) {
      if (wave == 0) {
        const float G = wave_incl_scan(lg_scalar);
        const float GC = __shfl(G, 63, 64);
        sW[lane] = expf(GC - G);
        if (lane == 0) {
          sGC[0] = GC;
          sEGC[0] = expf(GC);
          g_acc += (double)GC;
        }
      }
      __syncthreads();
    }

    // ---- gates: diagonal prefix per channel (key-staging threads) ---------------
    float pre[8], tot[8];
    if constexpr (DIAG) {
      if (is_k) {
        float run[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) run[c] = 0.f;
#pragma unroll
        for (int r = 0; r < TOK; ++r) {
          float x[8];
          cvt8<IN_F32>(rg[r], x);
#pragma unroll
          for (int c = 0; c < 8; ++c) run[c] += x[c];
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) sTot[tb][db * 8 + c] = run[c];
      }
      __syncthreads();
      if (is_k) {
#pragma unroll
        for (int c = 0; c < 8; ++c) pre[c] = tot[c] = 0.f;
        // block by block (two 16-byte reads each), so few reads are in flight
#pragma unroll 2
        for (int b = 0; b < NTB; ++b) {
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(&sTot[b][db * 8]);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(&sTot[b][db * 8 + 4]);
          const float w = b < tb ? 1.f : 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            tot[c] += x0[c];
            tot[4 + c] += x1[c];
            pre[c] = fmaf(w, x0[c], pre[c]);
            pre[4 + c] = fmaf(w, x1[c], pre[4 + c]);
          }
        }
        if (tb == 0) {
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            sGC[db * 8 + c] = tot[c];
            sEGC[db * 8 + c] = expf(tot[c]);
          }
        }
      }
    }

    // ---- stage keys (decay-weighted, split) and values, transposed -------------
    // in sub-blocks of SUB tokens (fewer live registers than the whole block)
    {
      constexpr int SUB = TOK < HYPIC_SD_SUB ? TOK : HYPIC_SD_SUB;
      float run[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) run[c] = 0.f;
#pragma unroll
      for (int r0 = 0; r0 < TOK; r0 += SUB) {
        float x[SUB][8];  // [token r][channel c]
#pragma unroll
        for (int r = 0; r < SUB; ++r) {
          cvt8<IN_F32>(rx[r0 + r], x[r]);
          if (is_k && GATED) {
            if constexpr (DIAG) {
              float lgr[8];
              cvt8<IN_F32>(rg[r0 + r], lgr);
#pragma unroll
              for (int c = 0; c < 8; ++c) {
                run[c] += lgr[c];
                x[r][c] *= __expf(tot[c] - (pre[c] + run[c]));
              }
            } else {
#pragma unroll
              for (int c = 0; c < 8; ++c) x[r][c] *= sW[tb * TOK + r0 + r];
            }
          }
        }
        // column c of the sub-block = SUB tokens of channel db*8+c: part of one
        // 16-byte LDS row chunk (chunk (tb TOK + r0) / 8 of the row)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          float col[SUB];
#pragma unroll
          for (int r = 0; r < SUB; ++r) col[r] = x[r][c];
          const int row = db * 8 + c;
          const int t0 = tb * TOK + r0;
          const int off = swz64(row, t0 / 8) + t0 % 8;
          using SubV = __attribute__((__vector_size__(SUB * sizeof(__bf16)))) __bf16;
          if (is_k) {
#pragma unroll
            for (int i = 0; i < NTK; ++i) {
              SubV tv;
#pragma unroll
              for (int r = 0; r < SUB; ++r) {
                tv[r] = (bf16_t)col[r];
                if (i + 1 < NTK) col[r] -= (float)tv[r];
              }
              *reinterpret_cast<SubV*>(&sK[i][off]) = tv;
            }
          } else {
#pragma unroll
            for (int i = 0; i < NTV; ++i) {
              SubV tv;
#pragma unroll
              for (int r = 0; r < SUB; ++r) {
                tv[r] = (bf16_t)col[r];
                if (i + 1 < NTV) col[r] -= (float)tv[r];
              }
              *reinterpret_cast<SubV*>(&sV[i][off]) = tv;
            }
          }
        }
      }
    }
    if (c0 + C < t_end) issue_loads(c0 + C);
    __syncthreads();

    if constexpr (DIAG) {
      if (tid < D) g_acc += (double)sGC[tid];
    }

    // ---- decay the running state to the chunk end, then add Ktil^T V ----------
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int tt = wave * TPW + i;
      const int rt = tt / NRT;
      if constexpr (FAM == 1) {
        const float e = sEGC[0];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= e;
      } else if constexpr (DIAG) {
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= sEGC[32 * rt + acc_row(r, lane)];
      }
    }
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      const int chunk = 2 * ks + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const int tt = wave * TPW + i;
        const int rt = tt / NRT, ct = tt % NRT;
        Frag<NTK> fa;
        Frag<NTV> fb;
#pragma unroll
        for (int j = 0; j < NTK; ++j)
          fa.t[j] = *reinterpret_cast<const bf16x8*>(&sK[j][swz64(32 * rt + (lane & 31), chunk)]);
#pragma unroll
        for (int j = 0; j < NTV; ++j)
          fb.t[j] = *reinterpret_cast<const bf16x8*>(&sV[j][swz64(32 * ct + (lane & 31), chunk)]);
        mma<NTK, NTV>(acc[i], fa, fb);
      }
    }
    __syncthreads();
  }

  // ---- write S(C|0) and g ------------------------------------------------------
  float* S = a.S + unit * D * D;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int tt = wave * TPW + i;
    const int rt = tt / NRT, ct = tt % NRT;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[(size_t)(32 * rt + acc_row(r, lane)) * D + 32 * ct + (lane & 31)] = acc[i][r];
  }
  if constexpr (DIAG) {
    if (tid < D) a.g[unit * D + tid] = (float)g_acc;
  } else {
    if (tid == 0) a.g[unit] = (float)g_acc;  // naive: 0
  }
}

#ifndef HYPIC_SD_TOK
#define HYPIC_SD_TOK 8
#endif
template <int FAM, int D, bool F32>
hipError_t launch_t(const BuildArgs& a, int n_blocks, hipStream_t stream) {
  constexpr int TOK = HYPIC_SD_TOK;
  constexpr int NTHR = 2 * (C / TOK) * (D / 8);
  if (seg_uniform(a.seg))
    hipLaunchKernelGGL((build_sd_kernel<FAM, D, F32, false, TOK>), dim3(n_blocks), dim3(NTHR), 0, stream, a);
  else
    hipLaunchKernelGGL((build_sd_kernel<FAM, D, F32, true, TOK>), dim3(n_blocks), dim3(NTHR), 0, stream, a);
  return hipGetLastError();
}

template <int FAM>
hipError_t launch_fam(int d, bool f32, const BuildArgs& a, int n_blocks, hipStream_t stream) {
  if (d == 128) return f32 ? launch_t<FAM, 128, true>(a, n_blocks, stream) : launch_t<FAM, 128, false>(a, n_blocks, stream);
  if (d == 64) return f32 ? launch_t<FAM, 64, true>(a, n_blocks, stream) : launch_t<FAM, 64, false>(a, n_blocks, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_build_sd(int fam, int d, bool in_f32, const BuildArgs& a, int n_blocks,
                           hipStream_t stream) {
  switch (fam) {
    case 0: return launch_fam<0>(d, in_f32, a, n_blocks, stream);
    case 1: return launch_fam<1>(d, in_f32, a, n_blocks, stream);
    case 2: return launch_fam<2>(d, in_f32, a, n_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace hypic
