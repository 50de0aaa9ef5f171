// chain.hip -- the ordered chain of dense (delta-rule) pairs along each chain
// (layer x head): composition of cached pairs, and the seam-window step fused
// with it.
//
// [youleyou, linear-layer paragraph] S(C1.C2) = T(C2) S(C1) + S(C2): a cached
// pair is applied by left-multiplying the running state by T_C = exp(g) U and
// adding S(C|0); [hwlabs, section 세그먼트 누적 전이 연산자] T_ABC = T_C T_B T_A.
// [youleyou, full-attention paragraph] at reuse the first w tokens of each
// segment are not in its cache entry: the linear layer runs them on the
// running state, emits each one's output o_t = S_t^T q_t, and then the body
// pair of the segment is applied.
//
// Work split.  Columns of the state are independent under both operations
// (T acts on the d_k axis, a window token writes k_t v_t^T column by column),
// so a workgroup owns one chain and a group of 32-column blocks (all of them
// when there are enough chains to fill the GPU, one when there are few, so
// that few chains still spread over many CUs; the workgroups of one chain are
// placed on one XCD and share its L2 copy of U).  Wave (rb, cb) owns the
// 32 x 32 output tile at rows 32 rb, columns 32 cb of the group.
//
// Per cached pair: U (fp32 in HBM) is split once per workgroup into fp16
// hi + lo terms, each row scaled by a power of two, and staged in LDS; the
// running state lives in LDS as fp32 (column-major, so a B fragment is 32
// contiguous bytes) and is split into hi + lo with a per-column power-of-two
// scale taken from the column maxima its writers leave behind.  The product
// keeps hi*hi + hi*lo + lo*hi on 32x32x16 fp16 MFMA: ~2^-22 relative per
// operand, fp32 class, in three products where three-term bf16 needs six.  The
// next pair's U and S tile are in flight during the current product.
//
// Per seam window (sub-chunks of up to 8 tokens, fp32 on the VALU; the chunk
// form of the delta rule with start state S, gate prefix G within the
// sub-chunk, Gamma_ts = exp(G_t - G_s) and n tokens):
//   Abar = (I + strict_lower(diag(b) (Gamma o K K^T)))^-1 diag(b)
//   R    = V - diag(exp(G)) K S
//   S'   = exp(G_n) S + (Abar^T diag(exp(G_n - G)) K)^T R
//   O    = diag(exp(G)) Q S + ((tril(Q K^T) o Gamma) Abar) R
// so that both the new state and the outputs are one pass over R.
#include <algorithm>

#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

constexpr int SUB = 8;  // window tokens per sub-chunk

template <int D, int NCB, bool SEAM>
struct ChainCfg {
  static constexpr int NRB = D / 32;         // row blocks (waves per column block)
  static constexpr int NW = NRB * NCB;       // waves
  static constexpr int NTH = 64 * NW;
  static constexpr int COLS = 32 * NCB;      // state columns of the workgroup
  static constexpr int NCG = (D / 32) / NCB; // column groups per chain
  static constexpr int UP = D + 8;           // fp16 pitch of the split U
  static constexpr int SP = D + 4;           // fp32 pitch of the state (column-major)
  static constexpr int NSLOT = D / 16;       // partial column maxima (16-row slices)
  static constexpr int LDU = D * D / 4 / NTH;  // float4 of U per thread
  static constexpr int OFF_UH = 0;
  static constexpr int OFF_UL = OFF_UH + D * UP * 2;
  static constexpr int OFF_S = OFF_UL + D * UP * 2;
  static constexpr int OFF_CM = OFF_S + COLS * SP * 4;
  static constexpr int OFF_RF = OFF_CM + NSLOT * COLS * 4;
  static constexpr int OFF_W = OFF_RF + D * 4;
  // window buffers (fp32): K, Q, Kz [SUB][D]; V, R [SUB][COLS]; small arrays
  static constexpr int OFF_WK = OFF_W;
  static constexpr int OFF_WQ = OFF_WK + SUB * D * 4;
  static constexpr int OFF_WKZ = OFF_WQ + SUB * D * 4;
  static constexpr int OFF_WV = OFF_WKZ + SUB * D * 4;
  static constexpr int OFF_WR = OFF_WV + SUB * COLS * 4;
  static constexpr int OFF_WSM = OFF_WR + SUB * COLS * 4;
  static constexpr int WSM_FLOATS = SEAM_REC_FLOATS;
  static constexpr int LDS = SEAM ? OFF_WSM + WSM_FLOATS * 4 : OFF_W;
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(D * D / 4 % NTH == 0, "U staging");
};

struct ChainArgs {
  const float* g;     // pairs [n_seg, n_chain]; U, S [n_seg, n_chain, D, D]
  const float* U;
  const float* S;     // nullptr: no pairs (seam windows only)
  const float* S_in;  // [n_chain, D, D] or nullptr (zero)
  float* S_out;       // may equal S_in
  float* prefix;      // compose: state before each segment, or nullptr
  float* g_tot;
  float* U_tot;
  const void* q;      // seam tokens [n_seg * w, n_chain, D]
  const void* k;
  const void* v;
  const void* beta;
  const void* lg;     // nullptr: no gate
  const float* wrec;  // per-window records of seam_prep
  float* o;
  int n_seg;
  int n_chain;
  int w;
  // Blocked composition: when blk_len > 0 the grid holds n_units =
  // ceil(n_seg / blk_len) * n_chain units; unit u composes segments
  // [b * blk_len, min((b + 1) * blk_len, n_seg)) of chain c (b = u / n_chain,
  // c = u % n_chain) from a zero state, and its outputs (S_out, U_tot, g_tot)
  // are indexed by u -- a pairs array of the blocks.  blk_len = 0: one unit
  // per chain over all segments.
  int blk_len;
  int n_units;
};

// power-of-two exponent that maps a block maximum m into [2^14, 2^15)
__device__ __forceinline__ int split_exp(float m) {
  if (!(m > 0.f)) return 0;
  int e;
  frexpf(m, &e);
  return e - 15;
}

// 8 floats -> fp16 hi and lo fragments, both rounded to nearest: |x - hi| <=
// 2^-11 |x| and |x - hi - lo| <= 2^-22 |x| (within fp16's normal range)
__device__ __forceinline__ void split_pair8(const float (&x)[8], f16x8& hi, f16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    hi[j] = (f16_t)x[j];
    lo[j] = (f16_t)(x[j] - (float)hi[j]);
  }
}

template <int D, int NCB, bool SEAM, bool IN_F32>
__global__ __launch_bounds__(64 * (D / 32) * NCB) void chain_kernel(const ChainArgs a) {
  using Cfg = ChainCfg<D, NCB, SEAM>;
  constexpr int NRB = Cfg::NRB, NTH = Cfg::NTH, COLS = Cfg::COLS, NCG = Cfg::NCG;
  constexpr int UP = Cfg::UP, SP = Cfg::SP, NSLOT = Cfg::NSLOT, LDU = Cfg::LDU;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  f16_t* sUh = reinterpret_cast<f16_t*>(smem + Cfg::OFF_UH);
  f16_t* sUl = reinterpret_cast<f16_t*>(smem + Cfg::OFF_UL);
  float* sS = reinterpret_cast<float*>(smem + Cfg::OFF_S);    // [col][row]
  float* sCM = reinterpret_cast<float*>(smem + Cfg::OFF_CM);  // [slot][col]
  float* sRF = reinterpret_cast<float*>(smem + Cfg::OFF_RF);  // 2^e of each U row

  // ---- which chain, which columns ------------------------------------------------
  // The NCG workgroups of one chain take block ids that are equal modulo 8, so
  // the round-robin dispatch puts them on one XCD.
  int chain, cgrp;
  if constexpr (NCG == 1) {
    chain = blockIdx.x;
    cgrp = 0;
  } else {
    const int blk = blockIdx.x / (8 * NCG), rem = blockIdx.x % (8 * NCG);
    cgrp = rem / 8;
    chain = blk * 8 + (rem % 8);
    if (chain >= a.n_units) return;  // padding of the unit count to a multiple of 8
  }
  const bool ut = blockIdx.y == 1;  // this workgroup composes U_total instead of S
  const int n_chain = a.n_chain;
  const int col0 = cgrp * COLS;     // first state column of the workgroup
  // pairs of this unit: index pidx + s * n_chain for its segments s < nseg
  const int blk = a.blk_len > 0 ? chain / n_chain : 0;
  const int pidx = a.blk_len > 0 ? blk * a.blk_len * n_chain + chain % n_chain : chain;
  const int nseg = a.blk_len > 0 ? min(a.blk_len, a.n_seg - blk * a.blk_len) : a.n_seg;
  const size_t chain_off = (size_t)chain * D * D;  // outputs, start state, tokens: by unit
  const size_t pair_off = (size_t)pidx * D * D;
  const size_t seg_stride = (size_t)n_chain * D * D;
  const bool pairs = a.S != nullptr;

  // Lane-derived indices.  refresh() re-derives them from an opaque copy of the
  // thread id at the top of each phase, so that addresses built from them are
  // recomputed where used instead of being kept live through the whole loop.
  int tid, lane, rb, cb, l32, h, tcol;
  auto refresh = [&]() {
    tid = opaque((int)threadIdx.x);
    lane = tid & 63;
    rb = (tid >> 6) % NRB;
    cb = (tid >> 6) / NRB;
    l32 = lane & 31;
    h = lane >> 5;
    tcol = 32 * cb + l32;  // this lane's tile column within the group
  };
  refresh();

  // ---- helpers ---------------------------------------------------------------------
  f32x4 ureg[LDU];
  auto issue_U = [&](int s) {
    const f32x4* src = reinterpret_cast<const f32x4*>(a.U + (size_t)s * seg_stride + pair_off);
#pragma unroll
    for (int i = 0; i < LDU; ++i) ureg[i] = src[i * NTH + tid];
  };
  // split the staged U into sUh / sUl, each row scaled by 2^-e (sRF = 2^e)
  auto store_U = [&]() {
#pragma unroll
    for (int i = 0; i < LDU; ++i) {
      const int f = i * NTH + tid;
      const int row = f / (D / 4), c4 = f % (D / 4);
      float m = fmaxf(fmaxf(fabsf(ureg[i][0]), fabsf(ureg[i][1])), fmaxf(fabsf(ureg[i][2]), fabsf(ureg[i][3])));
#pragma unroll
      for (int o = 1; o < D / 4; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      const int e = split_exp(m);
      const float s = ldexpf(1.f, -e);
      f16x4 hv, lv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float xs = ureg[i][j] * s;
        hv[j] = (f16_t)xs;
        lv[j] = (f16_t)(xs - (float)hv[j]);
      }
      *reinterpret_cast<f16x4*>(sUh + row * UP + 4 * c4) = hv;
      *reinterpret_cast<f16x4*>(sUl + row * UP + 4 * c4) = lv;
      if (c4 == 0) sRF[row] = ldexpf(1.f, e);
    }
  };
  // the lane's 16 tile elements of a [D][D] matrix (accumulator layout)
  auto tile_idx = [&](int r) { return (size_t)(32 * rb + acc_row(r, lane)) * D + col0 + tcol; };
  // a tile of a [D][D] matrix at p: rows 8q + 4h + j (q, j < 4) of the lane's
  // block; the lane offset is taken through opaque() so that its 16 addresses
  // are formed at each use instead of being kept live across the segment loop
  auto tile_ptr = [&](const float* base) {
    return base + (size_t)opaque(32 * rb + 4 * h) * D + col0 + tcol;
  };
  f32x16 Si;  // S tile of the next pair
  auto issue_Si = [&](int s) {
    const float* p = tile_ptr(a.S + (size_t)s * seg_stride + pair_off);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) Si[4 * q + j] = p[(8 * q + j) * D];
  };
  auto store_tile = [&](float* base, const f32x16& t) {
    float* p = const_cast<float*>(tile_ptr(base));
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 4; ++j) p[(8 * q + j) * D] = t[4 * q + j];
  };
  // write a tile into the LDS state and its partial column maxima
  auto put_tile = [&](const f32x16& t) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(sS + tcol * SP + 32 * rb + 8 * q + 4 * h) =
          f32x4{t[4 * q], t[4 * q + 1], t[4 * q + 2], t[4 * q + 3]};
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(t[r]));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    sCM[(2 * rb + h) * COLS + tcol] = m;  // rows 32 rb + 16 h .. + 15 share the tile's maximum
  };

  // ---- start state -----------------------------------------------------------------
  f32x16 St;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (ut) {
      St[r] = (32 * rb + acc_row(r, lane) == col0 + tcol) ? 1.f : 0.f;
    } else {
      St[r] = a.S_in ? a.S_in[chain_off + tile_idx(r)] : 0.f;
    }
  }
  if (!ut && a.prefix) store_tile(a.prefix + chain_off, St);
  put_tile(St);
  float g_next = 0.f;
  if (pairs) {
    issue_U(0);
    if (!ut) issue_Si(0);
    g_next = ut ? 0.f : a.g[pidx];
    store_U();
    if (nseg > 1) issue_U(1);
  }
  __syncthreads();

  for (int seg = 0; seg < nseg; ++seg) {
    refresh();
    // ---- seam window of this segment -----------------------------------------------
    if constexpr (SEAM) {
      float* sK = reinterpret_cast<float*>(smem + Cfg::OFF_WK);
      float* sQ = reinterpret_cast<float*>(smem + Cfg::OFF_WQ);
      float* sKz = reinterpret_cast<float*>(smem + Cfg::OFF_WKZ);
      float* sV = reinterpret_cast<float*>(smem + Cfg::OFF_WV);
      float* sR = reinterpret_cast<float*>(smem + Cfg::OFF_WR);
      float* sRec = reinterpret_cast<float*>(smem + Cfg::OFF_WSM);
      const float* sC = sRec;                  // [s][t]: Abar[t][s] exp(G_n - G_t)
      const float* sW2 = sRec + SUB * SUB;     // ((tril(Q K^T) o Gamma) Abar)[t][s]
      const float* sEG = sRec + 2 * SUB * SUB;  // exp(G_t); [SUB] = exp(G_n)
      const int n_sub = (a.w + SUB - 1) / SUB;
      for (int t0 = 0, sub = 0; t0 < a.w; t0 += SUB, ++sub) {
        refresh();
        const int n = min(SUB, a.w - t0);
        const size_t tok0 = (size_t)seg * a.w + t0;
        // W1: window tokens -> LDS (fp32), zero past n; the window's record
        for (int i = tid; i < 2 * SUB * (D / 8) + SUB * (COLS / 8); i += NTH) {
          float x[8];
          float* dst;
          if (i < 2 * SUB * (D / 8)) {
            const int which = i / (SUB * (D / 8)), j = i % (SUB * (D / 8));
            const int t = j / (D / 8), d8 = j % (D / 8);
            dst = (which ? sQ : sK) + t * D + 8 * d8;
            if (t < n) {
              load8<IN_F32>(which ? a.q : a.k, ((tok0 + t) * n_chain + chain) * D + 8 * d8, x);
            } else {
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) x[jj] = 0.f;
            }
          } else {
            const int j = i - 2 * SUB * (D / 8);
            const int t = j / (COLS / 8), c8 = j % (COLS / 8);
            dst = sV + t * COLS + 8 * c8;
            if (t < n) {
              load8<IN_F32>(a.v, ((tok0 + t) * n_chain + chain) * D + col0 + 8 * c8, x);
            } else {
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) x[jj] = 0.f;
            }
          }
          *reinterpret_cast<f32x4*>(dst) = f32x4{x[0], x[1], x[2], x[3]};
          *reinterpret_cast<f32x4*>(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
        }
        for (int i = tid; i < SEAM_REC_FLOATS; i += NTH)
          sRec[i] = a.wrec[((size_t)(seg * n_sub + sub) * n_chain + chain) * SEAM_REC_FLOATS + i];
        __syncthreads();
        // W4: Kz = Abar^T diag(exp(G_n - G)) K;  X = K S, P = Q S;  R = V - exp(G) X
        for (int i = tid; i < SUB * D; i += NTH) {
          const int s = i / D, d = i % D;
          float acc = 0.f;
#pragma unroll
          for (int t = 0; t < SUB; ++t) acc = fmaf(sC[s * SUB + t], sK[t * D + d], acc);
          sKz[i] = acc;
        }
        constexpr int NTC = (SUB * COLS + NTH - 1) / NTH;
        float P[NTC];
#pragma unroll
        for (int j = 0; j < NTC; ++j) {
          const int i = j * NTH + tid;
          P[j] = 0.f;
          if (i < SUB * COLS) {
            const int t = i / COLS, c = i % COLS;
            float xa = 0.f, pa = 0.f;
            const float* sc = sS + c * SP;
#pragma unroll 2
            for (int d = 0; d < D; d += 4) {
              const f32x4 sv = *reinterpret_cast<const f32x4*>(sc + d);
              const f32x4 kv = *reinterpret_cast<const f32x4*>(sK + t * D + d);
              const f32x4 qv = *reinterpret_cast<const f32x4*>(sQ + t * D + d);
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                xa = fmaf(kv[u], sv[u], xa);
                pa = fmaf(qv[u], sv[u], pa);
              }
            }
            P[j] = pa;
            sR[i] = sV[i] - sEG[t] * xa;
          }
        }
        __syncthreads();
        // W5: outputs and the new state from R
#pragma unroll
        for (int j = 0; j < NTC; ++j) {
          const int i = j * NTH + tid;
          if (i < SUB * COLS) {
            const int t = i / COLS, c = i % COLS;
            if (t < n) {
              float acc = sEG[t] * P[j];
#pragma unroll
              for (int s = 0; s < SUB; ++s)
                if (s <= t) acc = fmaf(sW2[t * SUB + s], sR[s * COLS + c], acc);
              a.o[((tok0 + t) * n_chain + chain) * D + col0 + c] = acc;
            }
          }
        }
        {
          const float eGn = sEG[SUB];
          for (int i = tid; i < COLS * (D / 16); i += NTH) {
            const int c = i / (D / 16), dq = i % (D / 16);
            float rr[SUB];
#pragma unroll
            for (int s = 0; s < SUB; ++s) rr[s] = sR[s * COLS + c];
            float* sc = sS + c * SP + 16 * dq;
            float m = 0.f;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
              f32x4 sv = *reinterpret_cast<const f32x4*>(sc + 4 * q4);
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const int d = 16 * dq + 4 * q4 + u;
                float acc = eGn * sv[u];
#pragma unroll
                for (int s = 0; s < SUB; ++s) acc = fmaf(sKz[s * D + d], rr[s], acc);
                sv[u] = acc;
                m = fmaxf(m, fabsf(acc));
              }
              *reinterpret_cast<f32x4*>(sc + 4 * q4) = sv;
            }
            sCM[dq * COLS + c] = m;
          }
        }
        __syncthreads();
      }
    }

    // ---- body pair: S <- exp(g) U S + S_B (or U_total <- U U_total) ----------------
    if (pairs) {
      refresh();
      const float gs = g_next;
      f32x16 T = zero16();
      {
        // column scale of the B operand (the lane's state column)
        float m = 0.f;
#pragma unroll
        for (int sl = 0; sl < NSLOT; ++sl) m = fmaxf(m, sCM[sl * COLS + tcol]);
        const int ec = split_exp(m);
        const float cs = ldexpf(1.f, -ec);
        const float* bcol = sS + tcol * SP + 8 * h;
        const f16_t* ah = sUh + (32 * rb + l32) * UP + 8 * h;
        const f16_t* al = sUl + (32 * rb + l32) * UP + 8 * h;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const f32x4 b0 = *reinterpret_cast<const f32x4*>(bcol + 16 * ks);
          const f32x4 b1 = *reinterpret_cast<const f32x4*>(bcol + 16 * ks + 4);
          const float bx[8] = {b0[0] * cs, b0[1] * cs, b0[2] * cs, b0[3] * cs,
                               b1[0] * cs, b1[1] * cs, b1[2] * cs, b1[3] * cs};
          f16x8 bh, bl;
          split_pair8(bx, bh, bl);
          const f16x8 fah = *reinterpret_cast<const f16x8*>(ah + 16 * ks);
          const f16x8 fal = *reinterpret_cast<const f16x8*>(al + 16 * ks);
          T = mfma32h(fal, bh, T);
          T = mfma32h(fah, bl, T);
          T = mfma32h(fah, bh, T);
          if (ks & 1) sched_fence();  // bounds how far ahead fragments are loaded
        }
        const float post = ldexpf(1.f, ec) * (ut ? 1.f : __expf(gs));
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = T[r] * sRF[32 * rb + acc_row(r, lane)] * post;
          St[r] = ut ? v : v + Si[r];
        }
      }
      __syncthreads();  // every wave is done with sU and the state
      put_tile(St);
      if (seg + 1 < nseg) {
        if (!ut && a.prefix) store_tile(a.prefix + (size_t)(seg + 1) * seg_stride + chain_off, St);
        store_U();
        if (!ut) {
          issue_Si(seg + 1);
          g_next = a.g[pidx + (size_t)(seg + 1) * n_chain];
        }
        if (seg + 2 < nseg) issue_U(seg + 2);
      }
      __syncthreads();
    }
  }

  // ---- results -----------------------------------------------------------------------
  // the state is in LDS (column-major): write it out row-major, coalesced
  float* dst = ut ? a.U_tot : a.S_out;
  for (int i = tid; i < D * COLS; i += NTH) {
    const int r = i / COLS, c = i % COLS;
    dst[chain_off + (size_t)r * D + col0 + c] = sS[c * SP + r];
  }
  if (!ut && a.g_tot && cgrp == 0 && tid == 0) {
    double acc = 0.0;
    for (int s = 0; s < nseg; ++s) acc += (double)a.g[pidx + (size_t)s * n_chain];
    a.g_tot[chain] = (float)acc;
  }
}

template <int D, int NCB, bool SEAM, bool IN_F32>
hipError_t launch_chain_t(const ChainArgs& a, bool want_ut, hipStream_t stream) {
  using Cfg = ChainCfg<D, NCB, SEAM>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&chain_kernel<D, NCB, SEAM, IN_F32>),
      hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
  if (attr != hipSuccess) return attr;
  const int nx = Cfg::NCG == 1 ? a.n_units : ((a.n_units + 7) / 8) * 8 * Cfg::NCG;
  hipLaunchKernelGGL((chain_kernel<D, NCB, SEAM, IN_F32>), dim3(nx, want_ut ? 2 : 1), dim3(Cfg::NTH), Cfg::LDS,
                     stream, a);
  return hipGetLastError();
}

// Few chains: split each over its column blocks (more workgroups, one per CU);
// many chains: one workgroup per chain (no duplicated U staging).
template <int D, bool SEAM, bool IN_F32>
hipError_t launch_chain_d(const ChainArgs& a, bool want_ut, hipStream_t stream) {
  constexpr int NCBT = D / 32;
  if (a.n_units * NCBT <= 256) return launch_chain_t<D, 1, SEAM, IN_F32>(a, want_ut, stream);
  return launch_chain_t<D, NCBT, SEAM, IN_F32>(a, want_ut, stream);
}

}  // namespace

namespace {
// Two-level schedule for few chains: about 128 (block, chain) units compose
// their blocks in parallel, then each chain composes its block pairs in order.
bool tree_plan(int d, int n_seg, int n_chain, bool prefix, int* blk_len, int* n_blocks) {
  if (prefix || n_seg < 8 || n_chain * (d / 32) > 256) return false;
  int nb = std::max(2, std::min(n_seg / 4, 128 / n_chain));
  const int bl = (n_seg + nb - 1) / nb;
  *blk_len = bl;
  *n_blocks = (n_seg + bl - 1) / bl;
  return *n_blocks >= 2;
}
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

size_t compose_workspace_bytes(int d, int n_seg, int n_chain, bool prefix) {
  int bl, nb;
  if (!tree_plan(d, n_seg, n_chain, prefix, &bl, &nb)) return 0;
  const size_t units = (size_t)nb * n_chain;
  return align256(units * 4) + 2 * units * d * d * 4;
}

hipError_t launch_compose_chain(int d, const ComposeArgs& c, void* ws, size_t ws_bytes, hipStream_t stream) {
  int bl, nb;
  const size_t need = compose_workspace_bytes(d, c.n_seg, c.n_chain, c.prefix != nullptr);
  if (need > 0 && ws != nullptr && ws_bytes >= need &&
      tree_plan(d, c.n_seg, c.n_chain, c.prefix != nullptr, &bl, &nb)) {
    const size_t units = (size_t)nb * c.n_chain;
    float* wg = reinterpret_cast<float*>(ws);
    float* wU = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(ws) + align256(units * 4));
    float* wS = wU + units * d * d;
    ChainArgs a1{};  // level 1: every (block, chain) from a zero state, with its U product and gate sum
    a1.g = c.g;
    a1.U = c.U;
    a1.S = c.S;
    a1.S_out = wS;
    a1.g_tot = wg;
    a1.U_tot = wU;
    a1.n_seg = c.n_seg;
    a1.n_chain = c.n_chain;
    a1.blk_len = bl;
    a1.n_units = (int)units;
    ChainArgs a2{};  // level 2: the block pairs of each chain in order
    a2.g = wg;
    a2.U = wU;
    a2.S = wS;
    a2.S_in = c.S_init;
    a2.S_out = c.S_out;
    a2.g_tot = c.g_tot;
    a2.U_tot = c.U_tot;
    a2.n_seg = nb;
    a2.n_chain = c.n_chain;
    a2.n_units = c.n_chain;
    hipError_t e;
    if (d == 128) {
      e = launch_chain_d<128, false, false>(a1, true, stream);
      if (e == hipSuccess) e = launch_chain_d<128, false, false>(a2, c.U_tot != nullptr, stream);
    } else if (d == 64) {
      e = launch_chain_d<64, false, false>(a1, true, stream);
      if (e == hipSuccess) e = launch_chain_d<64, false, false>(a2, c.U_tot != nullptr, stream);
    } else {
      e = hipErrorInvalidValue;
    }
    return e;
  }
  ChainArgs a{};
  a.n_units = c.n_chain;
  a.g = c.g;
  a.U = c.U;
  a.S = c.S;
  a.S_in = c.S_init;
  a.S_out = c.S_out;
  a.prefix = c.prefix;
  a.g_tot = c.g_tot;
  a.U_tot = c.U_tot;
  a.n_seg = c.n_seg;
  a.n_chain = c.n_chain;
  const bool ut = c.U_tot != nullptr;
  if (d == 128) return launch_chain_d<128, false, false>(a, ut, stream);
  if (d == 64) return launch_chain_d<64, false, false>(a, ut, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_seam_chain(int d, bool in_f32, const SeamArgs& s, hipStream_t stream) {
  ChainArgs a{};
  a.n_units = s.n_chain;
  a.g = s.bg;
  a.U = s.bU;
  a.S = s.bS;
  a.S_in = s.S_run;
  a.S_out = s.S_run;
  a.q = s.q;
  a.k = s.k;
  a.v = s.v;
  a.beta = s.beta;
  a.lg = s.lg;
  a.o = s.o;
  a.wrec = s.wrec;
  a.n_seg = s.n_seg;
  a.n_chain = s.n_chain;
  a.w = s.w;
  if (d == 128)
    return in_f32 ? launch_chain_d<128, true, true>(a, false, stream) : launch_chain_d<128, true, false>(a, false, stream);
  if (d == 64)
    return in_f32 ? launch_chain_d<64, true, true>(a, false, stream) : launch_chain_d<64, true, false>(a, false, stream);
  return hipErrorInvalidValue;
}

}  // namespace hypic
