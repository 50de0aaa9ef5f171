// build_sd.hip -- segment build for the naive, scalar-decay and diagonal-gate
// families: emits S(C|0) and the log-transition g of every (segment, chain).
//
// [youleyou, linear-layer paragraph] T_C is the product of the segment's
// per-token transitions and S(C|0) its final state from a zero start.  For
// these families the transition is (a diagonal of) exponentials of summed log
// gates, and the zero-start state has the closed form
//     S(C|0) = sum_t diag(exp(g - G_t)) k_t v_t^T,   g = G_L,
// where G_t is the inclusive prefix sum of the log gates.  The kernel streams
// 64-token chunks from the segment's end to its start: the weight of token t
// is exp of the sum of the log gates after it, which is the sum over the chunks
// already streamed (R) plus the sum after t inside its own chunk, so every
// chunk adds Ktil_c^T V_c to the state with no rescaling of the state between
// chunks (the same sum the composition law of the same paragraph gives,
// S <- diag(exp(G_chunk)) S + Ktil_c^T V_c, folded into the key weights).  The
// chunk product is a d x 64 x d contraction over tokens, run on MFMA with the
// decay-weighted keys split into bf16 terms (values are exact bf16 inputs).
//
// Grid: one workgroup per (segment, chain) unit, 2d threads (4 waves at d =
// 128; wave w owns the state's 32-row tile w, all its column tiles).  Per
// chunk: the 64 x d key, gate and value tiles are loaded with 16-byte loads (4
// tokens x 8 channels of each per thread), transposed in registers and written
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

// element j of 8 raw input elements
template <bool IN_F32>
__device__ __forceinline__ float elem8(const Raw8<IN_F32>& r, int j) {
  const uint4& u = r.w[IN_F32 ? j / 4 : 0];
  const int k = IN_F32 ? j % 4 : j / 2;
  const uint32_t w = k == 0 ? u.x : k == 1 ? u.y : k == 2 ? u.z : u.w;
  if constexpr (IN_F32) return __uint_as_float(w);
  return __uint_as_float((j & 1) ? (w & 0xffff0000u) : (w << 16));
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
//
// Staging: each thread stages 4 tokens (token block tb) x 8 channels (channel
// block db) of the keys (with their gates) and of the values, so the key work
// (decay weights, splits) is spread evenly over all waves.  A wave covers 8
// token blocks x 8 channel blocks: every load instruction reads 8 token rows of
// 128 contiguous bytes, and its transposed LDS writes spread evenly over the
// banks.  Wave w owns accumulator row tile w.
#ifndef HYPIC_SD_WPE
#define HYPIC_SD_WPE 2
#endif
constexpr int TB = 4;        // tokens per staging thread
constexpr int NTB = C / TB;  // token blocks of a chunk

__device__ __forceinline__ uint32_t word_at(const uint4& u, int j) {
  return j == 0 ? u.x : j == 1 ? u.y : j == 2 ? u.z : u.w;
}

template <int FAM, int D, bool IN_F32, bool ORDERED>
__global__ __launch_bounds__(NTB * (D / 8)) __attribute__((amdgpu_waves_per_eu(HYPIC_SD_WPE)))
void build_sd_kernel(const BuildArgs a) {
  constexpr int NTK = IN_F32 ? 3 : 2;  // bf16 terms of decay-weighted keys
  constexpr int NTV = IN_F32 ? 3 : 1;  // bf16 terms of values (bf16 inputs are exact)
  constexpr int NRT = D / 32;          // 32-row tiles along d
  constexpr int NTHR = NTB * (D / 8);
  static_assert(NTHR / 64 == NRT, "one accumulator row tile per wave");
  constexpr bool DIAG = (FAM == 2);
  constexpr uint32_t ESZ = IN_F32 ? 4 : 2;

  __shared__ __attribute__((aligned(16))) bf16_t sK[NTK][D * C];
  __shared__ __attribute__((aligned(16))) bf16_t sV[NTV][D * C];
  __shared__ __attribute__((aligned(16))) float sW[C];  // scalar: weight exp(R + G_C - G_t)
  // diag: per channel, the sums of the log gates of token blocks 0..7 and 8..15
  __shared__ __attribute__((aligned(16))) float sHalf[2][DIAG ? D : 4];

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

  f32x16 acc[NRT];  // tile (row tile wave, column tile i)
#pragma unroll
  for (int i = 0; i < NRT; ++i) acc[i] = zero16();

  // sum of the log gates streamed so far (the chunks after the current one):
  // scalar: every lane of wave 0 (double); diag: R[c] for the thread's channels
  // db * 8 + c (float, for the key weights), and in double for channel
  // db * 8 + (lane & 7) by the threads of token blocks 0..7 (the output g)
  double g_acc = 0.0;
  float R[DIAG ? 8 : 1] = {};

  const int tb = 8 * (wave & 1) + (lane & 7);  // 16 token blocks: two waves' worth
  const int db = 8 * (wave >> 1) + (lane >> 3);
  const uint32_t row_bytes = (uint32_t)n_chain * D * ESZ;  // one token of all chains
  const uint32_t voff = (uint32_t)(tb * TB) * row_bytes + db * 8 * ESZ;

  // raw inputs of the chunk being staged; the next chunk's (the one before it
  // in the segment) are loaded while the matrix cores work on this one.  Buffer
  // loads over the chunk's valid rows: tokens outside the segment read as
  // zeros.  (Loads two chunks ahead, or a third workgroup per CU, measured
  // slower: more requests in flight do not raise the throughput of this
  // access pattern.)
  Raw8<IN_F32> rk[TB], rv[TB], rg[DIAG ? TB : 1];
  float lg_scalar = 0.f;
  // Issued unconditionally, also before the segment's first chunk (an empty
  // range: zeros, no memory touched), so the loop carries one set of load registers.
  // Issued unconditionally, also past the segment's last chunk (an empty range:
  // zeros, no memory touched), so the loop carries one set of load registers.
  auto issue_loads = [&](int c0) {
    const int nv = c0 >= t_begin ? min(C, t_end - c0) : 0;
    c0 = max(c0, t_begin);
    const size_t row0 = ((size_t)c0 * n_chain + h) * D * ESZ;  // byte offset of token c0, chain h
    const uint32_t bytes = nv > 0 ? (uint32_t)(nv - 1) * row_bytes + D * ESZ : 0u;
    const __amdgpu_buffer_rsrc_t rsk = buffer_rsrc(reinterpret_cast<const char*>(a.k) + row0, bytes);
    const __amdgpu_buffer_rsrc_t rsv = buffer_rsrc(reinterpret_cast<const char*>(a.v) + row0, bytes);
#pragma unroll
    for (int r = 0; r < TB; ++r) {
      rk[r] = ldraw8<IN_F32>(rsk, voff, r * row_bytes);
      rv[r] = ldraw8<IN_F32>(rsv, voff, r * row_bytes);
    }
    if constexpr (DIAG) {
      const __amdgpu_buffer_rsrc_t rsg = buffer_rsrc(reinterpret_cast<const char*>(a.lg) + row0, bytes);
#pragma unroll
      for (int r = 0; r < TB; ++r) rg[r] = ldraw8<IN_F32>(rsg, voff, r * row_bytes);
    }
    if constexpr (FAM == 1) {
      // token c0 + lane's gate (zero past the end): a per-chain fp32 constant, or
      // per token (the buffer then covers the chunk's valid tokens of chain h)
      const bool per_tok = !a.gate_per_chain;
      const uint32_t gbytes = per_tok && nv > 0 ? ((uint32_t)(nv - 1) * n_chain + 1) * ESZ : 0u;
      const __amdgpu_buffer_rsrc_t rs =
          buffer_rsrc(reinterpret_cast<const char*>(a.lg) + ((size_t)c0 * n_chain + h) * ESZ, gbytes);
      const uint32_t go = (uint32_t)lane * n_chain * ESZ;
      const float tok = IN_F32 ? __uint_as_float(buffer_load4(rs, go, 0))
                               : __uint_as_float((uint32_t)buffer_load2(rs, go, 0) << 16);
      const float chn = per_tok ? 0.f : reinterpret_cast<const float*>(a.lg)[h];
      lg_scalar = tok + (lane < nv ? chn : 0.f);
    }
  };
  // LDS element offsets, as XOR patterns on a few base registers (the swizzle
  // swz64 written out: offsets that differ only in the XORed bits and an added
  // constant need no register of their own).  Staging: channel db * 8 + c,
  // tokens t0 .. t0 + 3 of the chunk = swz64(db * 8 + c, t0 / 8) + t0 % 8.
  const int stage_base = db * 512 + (((tb >> 1) ^ (db & 7)) << 3) + 4 * (tb & 1);
  // k step ks of A (keys, row 32 wave + lane % 32) and of B (values, row 32 i + lane % 32)
  const int l32 = lane & 31;
  const int kbase = 2048 * wave + 64 * l32 + (((lane >> 5) ^ (l32 & 7) ^ ((4 * wave + (l32 >> 3)) & 7)) << 3);
  const int vbase = 64 * l32 + (((lane >> 5) ^ (l32 & 7) ^ (l32 >> 3)) << 3);
  const int n_chunks = (t_end - t_begin + C - 1) / C;
  issue_loads(t_begin + (n_chunks - 1) * C);

  for (int c0 = t_begin + (n_chunks - 1) * C; c0 >= t_begin; c0 -= C) {
    // (the bases pass through opaque() so that the offsets are formed where they
    // are used rather than kept in registers across the loop)
    const int sb = opaque(stage_base);
    auto stage_off = [&](int c) { return (sb ^ (c << 3)) + 64 * c; };
    // ---- stage values, transposed (first: their registers are then free) ------
    {
      const int t0 = tb * TB;
      if constexpr (IN_F32) {
        bf16x4 vt[NTV][8];
#pragma unroll
        for (int r = 0; r < TB; ++r) {
          float x[8];
          cvt8<IN_F32>(rv[r], x);
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            float y = x[c];
#pragma unroll
            for (int i = 0; i < NTV; ++i) {
              const bf16_t hb = (bf16_t)y;
              vt[i][c][r] = hb;
              if (i + 1 < NTV) y -= (float)hb;
            }
          }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int off = stage_off(c);
#pragma unroll
          for (int i = 0; i < NTV; ++i) *reinterpret_cast<bf16x4*>(&sV[i][off]) = vt[i][c];
        }
      } else {
        // bf16 values are exact: a 16-bit transpose (byte permutes), no conversion
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          const uint32_t w01 = __builtin_amdgcn_perm(word_at(rv[1].w[0], c / 2), word_at(rv[0].w[0], c / 2), sel);
          const uint32_t w23 = __builtin_amdgcn_perm(word_at(rv[3].w[0], c / 2), word_at(rv[2].w[0], c / 2), sel);
          const int off = stage_off(c);
          *reinterpret_cast<uint2*>(&sV[0][off]) = make_uint2(w01, w23);
        }
      }
    }

    // ---- gates: scalar prefix over the chunk (wave 0) -------------------------
    if constexpr (FAM == 1) {
      if (wave == 0) {
        const float G = wave_incl_scan(lg_scalar);
        const float GC = __shfl(G, 63, 64);
        sW[lane] = expf((float)g_acc + (GC - G));
        g_acc += (double)GC;
      }
      __syncthreads();
    }

    // ---- gates: per channel, the sum over the tokens after this thread's block
    float sfx[8];
    if constexpr (DIAG) {
      // Token block tb = 8 (wave & 1) + (lane & 7): the 8 blocks of a half are 8
      // consecutive lanes, so the sums over the later blocks of the half are a
      // suffix scan across those lanes (row shifts, masked at the 8-lane
      // boundary); the other half's total comes through LDS.
      const int tl = lane & 7;
      const int half = wave & 1;
      float tot[8], suf[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) tot[c] = 0.f;
#pragma unroll
      for (int r = 0; r < TB; ++r) {
        float x[8];
        cvt8<IN_F32>(rg[r], x);
#pragma unroll
        for (int c = 0; c < 8; ++c) tot[c] += x[c];
      }
      // (the lanes past the boundary are masked with an AND, not a select, so
      // that every lane takes part in each row shift: a lane left out of one
      // would read as zero to its neighbour)
      const int m1 = -(int)(tl + 1 < 8), m2 = -(int)(tl + 2 < 8), m4 = -(int)(tl + 4 < 8);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float v = tot[c];
        v += __int_as_float(__float_as_int(dpp_row_shl<1>(v)) & m1);
        v += __int_as_float(__float_as_int(dpp_row_shl<2>(v)) & m2);
        v += __int_as_float(__float_as_int(dpp_row_shl<4>(v)) & m4);
        suf[c] = v;  // blocks tl .. 7 of the half
      }
      if (tl == 0) {
        *reinterpret_cast<f32x4*>(&sHalf[half][db * 8]) = f32x4{suf[0], suf[1], suf[2], suf[3]};
        *reinterpret_cast<f32x4*>(&sHalf[half][db * 8 + 4]) = f32x4{suf[4], suf[5], suf[6], suf[7]};
      }
      __syncthreads();
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(&sHalf[0][db * 8]);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(&sHalf[0][db * 8 + 4]);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(&sHalf[1][db * 8]);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(&sHalf[1][db * 8 + 4]);
      const float h0[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      const float h1[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        sfx[c] = R[c] + ((suf[c] - tot[c]) + (half == 0 ? h1[c] : 0.f));
        R[c] += h0[c] + h1[c];
      }
      if (half == 0) g_acc += (double)sHalf[0][db * 8 + tl] + (double)sHalf[1][db * 8 + tl];
    }

    // ---- stage keys (decay-weighted, split) and values, transposed -------------
    // the 4 tokens of channel db*8+c are one 8-byte piece of LDS row db*8+c
    {
      const int t0 = tb * TB;
      f32x4 w4;
      if constexpr (FAM == 1) w4 = *reinterpret_cast<const f32x4*>(&sW[t0]);
      // channel by channel (its 4 tokens' terms written as soon as they are formed)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        bf16x4 kt[NTK];   // [term], token r in element r
        float run = 0.f;  // diag: log gates of this block's tokens after token r
#pragma unroll
        for (int r = TB - 1; r >= 0; --r) {
          float x = elem8<IN_F32>(rk[r], c);
          if constexpr (DIAG) {
            x *= __expf(sfx[c] + run);
            run += elem8<IN_F32>(rg[r], c);
          } else if constexpr (FAM == 1) {
            x *= w4[r];
          }
#pragma unroll
          for (int i = 0; i < NTK; ++i) {
            const bf16_t hb = (bf16_t)x;
            kt[i][r] = hb;
            if (i + 1 < NTK) x -= (float)hb;
          }
        }
        const int off = stage_off(c);
#pragma unroll
        for (int i = 0; i < NTK; ++i) *reinterpret_cast<bf16x4*>(&sK[i][off]) = kt[i];
        sched_fence();
      }
    }
    issue_loads(c0 - C);
    __syncthreads();

    // ---- add Ktil^T V (keys weighted to the segment end) -------------------------
    const int bk = opaque(kbase), bv = opaque(vbase);
#pragma unroll
    for (int ks = 0; ks < C / 16; ++ks) {
      Frag<NTK> fa;
#pragma unroll
      for (int j = 0; j < NTK; ++j)
        fa.t[j] = *reinterpret_cast<const bf16x8*>(&sK[j][bk ^ (ks << 4)]);
#pragma unroll
      for (int i = 0; i < NRT; ++i) {
        Frag<NTV> fb;
#pragma unroll
        for (int j = 0; j < NTV; ++j)
          fb.t[j] = *reinterpret_cast<const bf16x8*>(&sV[j][(bv ^ (ks << 4) ^ ((i & 1) << 5)) + 2048 * i]);
        mma<NTK, NTV>(acc[i], fa, fb);
      }
      sched_fence();  // bounds how far ahead the fragments are read (registers)
    }
    __syncthreads();
  }

  // ---- write S(C|0) and g ------------------------------------------------------
  float* S = a.S + unit * D * D;
#pragma unroll
  for (int i = 0; i < NRT; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) S[(size_t)(32 * wave + acc_row(r, lane)) * D + 32 * i + (lane & 31)] = acc[i][r];
  }
  if constexpr (DIAG) {
    if ((wave & 1) == 0) a.g[unit * D + db * 8 + (lane & 7)] = (float)g_acc;
  } else {
    if (tid == 0) a.g[unit] = (float)g_acc;  // naive: 0 (scalar: lane 0 of wave 0)
  }
}

template <int FAM, int D, bool F32>
hipError_t launch_t(const BuildArgs& a, int n_blocks, hipStream_t stream) {
  constexpr int NTHR = NTB * (D / 8);
  if (seg_uniform(a.seg))
    hipLaunchKernelGGL((build_sd_kernel<FAM, D, F32, false>), dim3(n_blocks), dim3(NTHR), 0, stream, a);
  else
    hipLaunchKernelGGL((build_sd_kernel<FAM, D, F32, true>), dim3(n_blocks), dim3(NTHR), 0, stream, a);
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
