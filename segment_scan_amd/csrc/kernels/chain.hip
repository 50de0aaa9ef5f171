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
// so a workgroup owns one unit (a chain, or a block of one chain's segments)
// and NCT 32-column tiles of its state.  It has one wave per 32-row block:
// wave rb keeps the state tiles at rows 32 rb .. 32 rb + 31 in MFMA
// accumulators for the whole chain, and computes the same rows of every
// product T = U S.  The workgroups of one unit take block ids that are equal
// modulo 8, so the round-robin dispatch puts them on one XCD, where they share
// its L2 copy of each U.
//
// Operands.  Products run on 32x32x16 fp16 MFMA with both fp32 operands as
// sums of NT fp16 terms (each the nearest fp16 of the remaining residual),
// keeping the term pairs i + j < NT: NT = 3 (six products) leaves about 2^-33
// of each operand, below fp32's own rounding, and is used wherever the pairs
// and tokens are fp32; NT = 2 (three products, about 2^-22) serves the seam
// step with bf16 tokens, whose outputs carry bf16 input precision anyway.
// U (fp32 in HBM) is the A operand: wave rb reads its 32 rows straight into
// registers one pair ahead (lane l: row 32 rb + l % 32, 8 consecutive k per
// 16-deep step), scales them by one power of two (from the largest magnitude
// among them) and splits each slice just before its products, reloading the
// slice with the next pair's values as soon as it is split.  The state is the
// B operand: after every update each wave splits its tiles once into
// column-major term arrays in LDS, each column scaled by a power of two from
// the column maxima the row-block waves leave behind, and every product reads
// its B fragments from there.
//
// Per seam window (sub-chunks of up to 8 tokens; the chunk form of the delta
// rule with start state S, gate prefix G within the sub-chunk, n tokens; the
// state-independent factors C, W2, exp(G) come from seam_prep.hip):
//   [X; P] = [K; Q] S                    one MFMA product per column block
//   R  = V - diag(exp(G)) X,  O = diag(exp(G)) P + W2 R,  R' = C^T R
//   S' = exp(G_n) S + K^T R'             a rank-8 MFMA update of every tile
#include <algorithm>

#include "common.h"
#include "split_f16.h"
#include "../launch.h"

// state tiles per workgroup of the d = 64 seam step with bf16 tokens (1 or 2)
#ifndef HYPIC_SEAM_NCT
#define HYPIC_SEAM_NCT 2
#endif

namespace hypic {

namespace {

constexpr int SUB = 8;  // window tokens per sub-chunk

template <int D, int NCT, int NT, bool SEAM, bool IN_F32>
struct ChainCfg {
  static constexpr int NRB = D / 32;          // waves: one per 32-row block
  static constexpr int NTH = 64 * NRB;
  static constexpr int COLS = 32 * NCT;       // state columns of a workgroup
  static constexpr int NCG = (D / 32) / NCT;  // workgroups (column groups) per unit
  static constexpr int KS = D / 16;           // 16-deep k steps of a product
  static constexpr int BP = D + 8;            // fp16 pitch of a split state column and a window row
  static constexpr int NTA = IN_F32 ? 2 : 1;  // fp16 terms of window key and query rows
  static constexpr int NTK = IN_F32 ? 3 : 1;  // bf16 terms of window keys in the update
  static constexpr int NTR = IN_F32 ? 3 : 2;  // bf16 terms of R' in the update
  static constexpr int RPP = SUB + 4;         // fp32 pitch of R' columns
  static constexpr int OFF_B = 0;                                // [NT][COLS][BP] f16
  static constexpr int OFF_CM = OFF_B + NT * COLS * BP * 2;      // [NRB][COLS] column maxima
  static constexpr int OFF_W = OFF_CM + NRB * COLS * 4;
  // window (SEAM): [K; Q] rows scaled and split to fp16, their scales, K^T in
  // bf16 terms, V of the group's columns, R' (column-major), the window record
  static constexpr int OFF_A = OFF_W;                            // [NTA][2 SUB][BP] f16
  static constexpr int OFF_AS = OFF_A + NTA * 2 * SUB * BP * 2;  // [2 SUB] f32
  static constexpr int OFF_KT = OFF_AS + 2 * SUB * 4;            // [NTK][D][SUB] bf16
  static constexpr int OFF_V = OFF_KT + NTK * D * SUB * 2;       // [SUB][COLS] f32
  static constexpr int OFF_RP = OFF_V + SUB * COLS * 4;          // [COLS][RPP] f32
  static constexpr int OFF_REC = OFF_RP + COLS * RPP * 4;
  static constexpr int LDS = SEAM ? OFF_REC + SEAM_REC_FLOATS * 4 : OFF_W;
  // window token chunks of 8 elements: K and Q rows, then V rows of the group's columns
  static constexpr int NWCH = 2 * SUB * (D / 8) + SUB * (COLS / 8);
  static constexpr int WPT = (NWCH + NTH - 1) / NTH;  // chunks per thread
  static_assert(NCG >= 1 && NCG * NCT == D / 32, "column groups");
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(2 * SUB * (D / 8) == NTH || !SEAM, "window rows: one chunk per thread");
};

struct ChainArgs {
  const float* g;     // pairs [n_seg, n_chain]; U, S [n_seg, n_chain, D, D]
  const float* U;
  const float* S;     // nullptr: no pairs (seam windows only)
  const float* S_in;  // [n_units, D, D] or nullptr (zero)
  float* S_out;       // may equal S_in
  float* prefix;      // compose: state before each segment, or nullptr
  float* g_tot;
  float* U_tot;
  const void* q;      // seam tokens [n_seg * w, n_chain, D]
  const void* k;
  const void* v;
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

// Waves per SIMD the register allocation must leave room for: the state
// tiles, the prefetched U slices and S_B tiles fit 2 waves (seam step) or 3
// (composition) without spills, and that many workgroups also fit the LDS of
// a CU, so more chains run at once (left to itself the compiler gives the seam
// step over 256 registers: one workgroup per CU).
template <int D, int NCT, int NT, bool SEAM, bool IN_F32>
constexpr int chain_min_waves() {
  return SEAM ? 2 : 3;
}

// PAIRS: the chain has cached pairs (always for composition; the seam step may
// run its windows alone)
template <int D, int NCT, int NT, bool SEAM, bool IN_F32, bool PAIRS>
__global__ __launch_bounds__(64 * (D / 32), (chain_min_waves<D, NCT, NT, SEAM, IN_F32>())) void chain_kernel(
    const ChainArgs a) {
  using Cfg = ChainCfg<D, NCT, NT, SEAM, IN_F32>;
  constexpr int NRB = Cfg::NRB, NTH = Cfg::NTH, COLS = Cfg::COLS, NCG = Cfg::NCG, KS = Cfg::KS;
  constexpr int BP = Cfg::BP, NTA = Cfg::NTA, NTK = Cfg::NTK, NTR = Cfg::NTR, RPP = Cfg::RPP;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  f16_t* sB = reinterpret_cast<f16_t*>(smem + Cfg::OFF_B);    // [term][col][k]
  float* sCM = reinterpret_cast<float*>(smem + Cfg::OFF_CM);  // [row block][col]

  // ---- which unit, which columns ---------------------------------------------------
  int unit, cgrp;
  if constexpr (NCG == 1) {
    unit = blockIdx.x;
    cgrp = 0;
  } else {
    const int blk8 = blockIdx.x / (8 * NCG), rem = blockIdx.x % (8 * NCG);
    cgrp = rem / 8;
    unit = blk8 * 8 + (rem % 8);
    if (unit >= a.n_units) return;  // padding of the unit count to a multiple of 8
  }
  const bool ut = blockIdx.y == 1;  // this workgroup composes U_total instead of S
  const int n_chain = a.n_chain;
  const int col0 = cgrp * COLS;     // first state column of the workgroup
  // pairs of this unit: index pidx + s * n_chain for its segments s < nseg
  const int blk = a.blk_len > 0 ? unit / n_chain : 0;
  const int chain = a.blk_len > 0 ? unit % n_chain : unit;
  const int pidx = a.blk_len > 0 ? blk * a.blk_len * n_chain + chain : unit;
  const int nseg = a.blk_len > 0 ? min(a.blk_len, a.n_seg - blk * a.blk_len) : a.n_seg;
  const size_t unit_off = (size_t)unit * D * D;  // outputs and start state: by unit
  const size_t pair_off = (size_t)pidx * D * D;
  const size_t seg_stride = (size_t)n_chain * D * D;
  constexpr bool pairs = PAIRS;

  // Lane-derived indices.  refresh() re-derives them from an opaque copy of the
  // thread id at the top of each phase, so that addresses built from them are
  // recomputed where used instead of being kept live through the whole loop.
  int tid, lane, rb, l32, h;
  auto refresh = [&]() {
    tid = opaque((int)threadIdx.x);
    lane = tid & 63;
    rb = tid >> 6;
    l32 = lane & 31;
    h = lane >> 5;
  };
  refresh();

  // ---- U of a pair: this wave's 32 rows as A fragments ------------------------------
  // slice ks of lane l: row 32 rb + l % 32, k = 16 ks + 8 (l / 32) + 0..7
  f32x4 ur[KS][2];
  auto u_src = [&](int s) {
    return reinterpret_cast<const f32x4*>(a.U + (size_t)s * seg_stride + pair_off) +
           ((size_t)(32 * rb + l32) * D + 8 * h) / 4;
  };
  auto issue_U = [&](int s) {
    const f32x4* p = u_src(s);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ur[ks][0] = p[4 * ks];
      ur[ks][1] = p[4 * ks + 1];
    }
  };

  // ---- the state tiles and their split -----------------------------------------------
  // tile ct of a [D][D] matrix at base: element r of this lane is row
  // 32 rb + 8 (r / 4) + 4 h + r % 4, column col0 + 32 ct + l32
  auto tile_ptr = [&](const float* base, int ct) {
    return base + (size_t)opaque(32 * rb + 4 * h) * D + col0 + 32 * ct + l32;
  };
  f32x16 St[NCT];  // the state
  f32x16 Si[NCT];  // S of the next pair
  auto issue_Si = [&](int s) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float* p = tile_ptr(a.S + (size_t)s * seg_stride + pair_off, ct);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) Si[ct][4 * q + j] = p[(8 * q + j) * D];
    }
  };
  auto store_tiles = [&](float* base) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float* p = const_cast<float*>(tile_ptr(base, ct));
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[(8 * q + j) * D] = St[ct][4 * q + j];
    }
  };
  // results (after the last segment): the tiles, from registers, and the gate sum
  auto store_results = [&]() {
    store_tiles((ut ? a.U_tot : a.S_out) + unit_off);
    if (!ut && a.g_tot && cgrp == 0 && threadIdx.x == 0) {
      double acc = 0.0;
      for (int s = 0; s < nseg; ++s) acc += (double)a.g[pidx + (size_t)s * n_chain];
      a.g_tot[unit] = (float)acc;
    }
  };
  // the wave's share of its columns' maxima
  auto put_cmax = [&]() {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(St[ct][r]));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (h == 0) sCM[rb * COLS + 32 * ct + l32] = m;
    }
  };
  // after a barrier: each column's exponent, and the tiles times f split into
  // the B arrays (f = exp(g) of the pair the split feeds, else 1)
  int ec[NCT];  // the lane's column of tile ct is stored as x f 2^-ec
  auto put_B = [&](float f) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int c = 32 * ct + l32;
      float m = 0.f;
#pragma unroll
      for (int s = 0; s < NRB; ++s) m = fmaxf(m, sCM[s * COLS + c]);
      ec[ct] = min(max(split_exp(m * f), -100), 100);
      const float sc = f * ldexpf(1.f, -ec[ct]);  // exact: f times a normal power of two
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float r[4];
        f16x4 tv[NT];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float x = St[ct][4 * q + j];
          tv[0][j] = (f16_t)mul_opaque(x, sc);
          if (NT > 1) r[j] = __builtin_fmaf(x, sc, -(float)tv[0][j]);
        }
#pragma unroll
        for (int i = 1; i < NT; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            tv[i][j] = (f16_t)r[j];
            if (i + 1 < NT) r[j] -= (float)tv[i][j];
          }
        const int off = c * BP + 32 * rb + 8 * q + 4 * h;
#pragma unroll
        for (int i = 0; i < NT; ++i) *reinterpret_cast<f16x4*>(sB + i * COLS * BP + off) = tv[i];
      }
    }
  };

  // ---- seam windows: staging and the two products ------------------------------------
  [[maybe_unused]] f16_t* sA = reinterpret_cast<f16_t*>(smem + Cfg::OFF_A);      // [NTA][2 SUB][BP]: K, Q rows
  [[maybe_unused]] float* sAS = reinterpret_cast<float*>(smem + Cfg::OFF_AS);    // 2^e of those rows
  [[maybe_unused]] bf16_t* sKt = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_KT);  // [NTK][D][SUB]
  [[maybe_unused]] float* sV = reinterpret_cast<float*>(smem + Cfg::OFF_V);      // [SUB][COLS]
  [[maybe_unused]] float* sRp = reinterpret_cast<float*>(smem + Cfg::OFF_RP);    // [COLS][RPP]
  [[maybe_unused]] float* sRec = reinterpret_cast<float*>(smem + Cfg::OFF_REC);
  const int n_sub = SEAM ? (a.w + SUB - 1) / SUB : 0;
  using Raw = uint4[IN_F32 ? 2 : 1];
  Raw wraw[Cfg::WPT];
  constexpr int RPT = (SEAM_REC_FLOATS + NTH - 1) / NTH;  // record floats per thread
  float wrec_r[RPT];
  // loads of window (seg, sub): chunk i < 2 SUB (D / 8) is 8 elements of a K
  // (t < SUB) or Q row, the rest 8 values of a V row of the group's columns
  // element offset of token tok0 + t of this chain: a uniform base plus a 32-bit
  // per-lane part (t < SUB, n_chain D < 2^31 / SUB)
  const uint32_t tok_stride = (uint32_t)n_chain * D;
  auto tok_base = [&](size_t tok0) { return (tok0 * n_chain + chain) * D; };
  auto issue_window = [&](int seg, int sub) {
    const int n = min(SUB, a.w - sub * SUB);
    const size_t base = tok_base((size_t)seg * a.w + sub * SUB);
#pragma unroll
    for (int k = 0; k < Cfg::WPT; ++k) {
      const int i = tid + k * NTH;
      int t = -1;
      const void* src = nullptr;
      uint32_t off = 0;
      if (i < 2 * SUB * (D / 8)) {
        const int row = i / (D / 8), d8 = i % (D / 8);
        t = row % SUB;
        src = row < SUB ? a.k : a.q;
        off = (uint32_t)t * tok_stride + 8 * d8;
      } else if (i < Cfg::NWCH) {
        const int j = i - 2 * SUB * (D / 8);
        t = j / (COLS / 8);
        src = a.v;
        off = (uint32_t)t * tok_stride + col0 + 8 * (j % (COLS / 8));
      }
#pragma unroll
      for (int u = 0; u < (IN_F32 ? 2 : 1); ++u) wraw[k][u] = make_uint4(0, 0, 0, 0);
      if (t >= 0 && t < n) {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(src) +
                                                        (base + off) * (IN_F32 ? 4 : 2));
#pragma unroll
        for (int u = 0; u < (IN_F32 ? 2 : 1); ++u) wraw[k][u] = p[u];
      }
    }
    const float* rec = a.wrec + ((size_t)(seg * n_sub + sub) * n_chain + chain) * SEAM_REC_FLOATS;
#pragma unroll
    for (int k = 0; k < RPT; ++k)
      if (tid + k * NTH < SEAM_REC_FLOATS) wrec_r[k] = rec[tid + k * NTH];
  };
  auto raw_to_f32 = [&](const Raw& r, float (&x)[8]) {
    if constexpr (IN_F32) {
      const uint32_t u[8] = {r[0].x, r[0].y, r[0].z, r[0].w, r[1].x, r[1].y, r[1].z, r[1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = __uint_as_float(u[j]);
    } else {
      const uint32_t u[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(u[j] << 16);
        x[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
      }
    }
  };
  // into LDS (every wave is past the previous window's products)
  auto stage_window = [&]() {
#pragma unroll
    for (int k = 0; k < Cfg::WPT; ++k) {
      const int i = tid + k * NTH;
      float x[8];
      raw_to_f32(wraw[k], x);
      if (i < 2 * SUB * (D / 8)) {
        // a K or Q row: scaled by the power of two of its maximum (the row's
        // D / 8 chunks are consecutive lanes), split to fp16
        const int row = i / (D / 8), d8 = i % (D / 8);
        float m = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
        m = dpp_max_step(m, 0);
        m = dpp_max_step(m, 1);
        m = dpp_max_step(m, 2);
        if (D / 8 >= 16) m = dpp_max_step(m, 3);
        const int e = min(max(split_exp(m), -100), 100);
        const HFrag<NTA> fa = split8h_scaled<NTA>(x, ldexpf(1.f, -e));
#pragma unroll
        for (int term = 0; term < NTA; ++term)
          *reinterpret_cast<f16x8*>(sA + (term * 2 * SUB + row) * BP + 8 * d8) = fa.t[term];
        if (d8 == 0) sAS[row] = ldexpf(1.f, e);
        if (row < SUB) {  // keys, transposed, in bf16 terms: [term][d][t]
          float r8[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) r8[j] = x[j];
#pragma unroll
          for (int term = 0; term < NTK; ++term)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              const bf16_t bv = (bf16_t)r8[j];
              sKt[(term * D + 8 * d8 + j) * SUB + row] = bv;
              r8[j] -= (float)bv;
            }
        }
      } else if (i < Cfg::NWCH) {
        const int j = i - 2 * SUB * (D / 8);
        float* dst = sV + (j / (COLS / 8)) * COLS + 8 * (j % (COLS / 8));
        *reinterpret_cast<f32x4*>(dst) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
      }
    }
#pragma unroll
    for (int k = 0; k < RPT; ++k)
      if (tid + k * NTH < SEAM_REC_FLOATS) sRec[tid + k * NTH] = wrec_r[k];
  };

  // ---- start state (one branch around all the loads, so they fly together) ---------
  if (!ut && a.S_in) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float* p = tile_ptr(a.S_in + unit_off, ct);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j) St[ct][4 * q + j] = p[(8 * q + j) * D];
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        St[ct][r] = (ut && 32 * rb + acc_row(r, lane) == col0 + 32 * ct + l32) ? 1.f : 0.f;
  }
  if (!ut && a.prefix) store_tiles(a.prefix + pair_off);  // prefix states follow the pairs' layout
  put_cmax();
  float g_next = 0.f;
  if (pairs) {
    issue_U(0);
    if (!ut) issue_Si(0);
    g_next = ut ? 0.f : a.g[pidx];
  }
  if constexpr (SEAM) issue_window(0, 0);
  __syncthreads();
  put_B((SEAM || !pairs) ? 1.f : expf(g_next));
  if constexpr (SEAM) stage_window();
  __syncthreads();

  for (int seg = 0; seg < nseg; ++seg) {
    // ---- seam window of this segment -----------------------------------------------
    if constexpr (SEAM) {
      for (int sub = 0; sub < n_sub; ++sub) {
        refresh();
        const int n = min(SUB, a.w - sub * SUB);
        const size_t obase = tok_base((size_t)seg * a.w + sub * SUB);
        // the next window's loads fly during this one and the body pair
        if (sub + 1 < n_sub) issue_window(seg, sub + 1);
        else if (seg + 1 < nseg) issue_window(seg + 1, 0);
        const float* sCt = sRec;              // [t][s]: Abar[t][s] exp(G_n - G_t)
        const float* sW2 = sRec + SUB * SUB;  // [t][s]: ((tril(Q K^T) o Gamma) Abar)[t][s]
        const float* sEG = sRec + 2 * SUB * SUB;  // exp(G_t); [SUB] = exp(G_n)
        // [X; P] = [K; Q] S on 16x16x32 MFMA: rows are the 8 keys and 8 queries,
        // one 16-column tile per wave (tiles ct16 = rb, rb + NRB, ... of the
        // group's 2 NCT); then [R'; W2 R] = [C^T; W2] R on one 16x16x16 MFMA
        // per tile, R in the B layout exactly where the X rows come out
#pragma unroll
        for (int ct16 = 0; ct16 < 2 * NCT; ++ct16) {
          if (ct16 % NRB != rb) continue;
          const int l16 = lane & 15, g = lane >> 4;
          const int col = 16 * ct16 + l16;  // the lane's column within the group
          f32x4 XP = f32x4{0.f, 0.f, 0.f, 0.f};
          const f16_t* pa = sA + l16 * BP + 8 * g;
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            HFrag<NTA> fa;
#pragma unroll
            for (int i = 0; i < NTA; ++i)
              fa.t[i] = *reinterpret_cast<const f16x8*>(pa + i * 2 * SUB * BP + 32 * ks);
            HFrag<NT> fb;
#pragma unroll
            for (int i = 0; i < NT; ++i)
              fb.t[i] = *reinterpret_cast<const f16x8*>(sB + (i * COLS + col) * BP + 32 * ks + 8 * g);
            mmah16<NTA, NT>(XP, fa, fb);
          }
          // the column's exponent: tile col / 32 of lane col % 32
          int ecc = ec[0];
#pragma unroll
          for (int ct = 1; ct < NCT; ++ct)
            if (ct16 / 2 == ct) ecc = ec[ct];
          const int ce = __shfl(ecc, col & 31, 64);
          // lane (l16, g): rows 4g + j of the tile -- X of token 4g + j (g < 2),
          // P of token 4(g - 2) + j (g >= 2); R = V - exp(G) X on the X lanes
          float v4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = 4 * g + j;  // 0..7 keys, 8..15 queries
            const int t = row & 7;
            const float x = ldexpf(XP[j], ce) * sAS[row];
            v4[j] = g < 2 ? sV[t * COLS + col] - sEG[t] * x : sEG[t] * x;  // R, or exp(G) P
          }
          // B = R (k = token 4g + j on the X lanes, zero on the P lanes), scaled
          // per column by a power of two and split into NT fp16 terms
          float m = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) m = fmaxf(m, g < 2 ? fabsf(v4[j]) : 0.f);
          m = fmaxf(m, __shfl_xor(m, 16, 64));
          // every lane of the column (the P lanes too) takes the X lanes' exponent
          const int er = __shfl(split_exp(m), l16, 64);
          float rb4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) rb4[j] = g < 2 ? ldexpf(v4[j], -er) : 0.f;
          // A = [C^T; W2] (row l16, k = 4g + j; zero for k >= 8)
          float a4[4] = {0.f, 0.f, 0.f, 0.f};
          if (g < 2) {
            const f32x4 av = *reinterpret_cast<const f32x4*>((l16 < 8 ? sCt + l16 * SUB : sW2 + (l16 - 8) * SUB) +
                                                             4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j) a4[j] = av[j];
          }
          f16x4 at[NT], bt[NT];
#pragma unroll
          for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              at[i][j] = (f16_t)a4[j];
              bt[i][j] = (f16_t)rb4[j];
              if (i + 1 < NT) {
                a4[j] -= (float)at[i][j];
                rb4[j] -= (float)bt[i][j];
              }
            }
          f32x4 RW = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s2 = NT - 1; s2 >= 0; --s2)
#pragma unroll
            for (int i = 0; i < NT; ++i)
              if (s2 - i >= 0 && s2 - i < NT)
                RW = __builtin_amdgcn_mfma_f32_16x16x16f16(at[i], bt[s2 - i], RW, 0, 0, 0);
          // rows 0..7 (lanes g < 2): R' of token 4g + j; rows 8..15 (g >= 2): W2 R
          if (g < 2) {
            f32x4 rp;
#pragma unroll
            for (int j = 0; j < 4; ++j) rp[j] = ldexpf(RW[j], er);
            *reinterpret_cast<f32x4*>(sRp + col * RPP + 4 * g) = rp;
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int t = 4 * (g - 2) + j;
              if (t < n) a.o[obase + (uint32_t)t * tok_stride + col0 + col] = v4[j] + ldexpf(RW[j], er);
            }
          }
        }
        __syncthreads();
        // S = exp(G_n) S + K^T R' on every tile (k = the 8 tokens; lanes of the
        // upper k half hold zeros)
        {
          const float eGn = sEG[SUB];
          Frag<NTK> fa;
          if (h == 0) {
#pragma unroll
            for (int term = 0; term < NTK; ++term)
              fa.t[term] = *reinterpret_cast<const bf16x8*>(sKt + (term * D + 32 * rb + l32) * SUB);
          } else {
#pragma unroll
            for (int term = 0; term < NTK; ++term) fa.t[term] = bf16x8{};
          }
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
            for (int r = 0; r < 16; ++r) St[ct][r] *= eGn;
            Frag<NTR> fb;
            if (h == 0) {
              const f32x4 r0 = *reinterpret_cast<const f32x4*>(sRp + (32 * ct + l32) * RPP);
              const f32x4 r1 = *reinterpret_cast<const f32x4*>(sRp + (32 * ct + l32) * RPP + 4);
              const float x[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
              fb = split8<NTR>(x);
            } else {
#pragma unroll
              for (int term = 0; term < NTR; ++term) fb.t[term] = bf16x8{};
            }
            mma<NTK, NTR>(St[ct], fa, fb);
          }
          put_cmax();
        }
        __syncthreads();
        put_B((sub + 1 == n_sub && pairs) ? expf(g_next) : 1.f);
        if (sub + 1 < n_sub) stage_window();
        __syncthreads();
      }
    }

    // ---- body pair: S <- exp(g) U S + S_B (or U_total <- U U_total) ----------------
    if (pairs) {
      refresh();
      const bool more = seg + 1 < nseg;
      // T = (U 2^-eu) (exp(g) S 2^-ec), then S = T 2^(eu + ec) + S_B
      float m = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(ur[ks][i][j]));
      const int eu = split_exp(wave_max_uniform(m));
      const float su = pow2_neg(eu);
      f32x16 T[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) T[ct] = zero16();
      const f32x4* nxt = u_src(more ? seg + 1 : seg);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x[j] = ur[ks][0][j];
          x[4 + j] = ur[ks][1][j];
        }
        HFrag<NT> fa = split8h_scaled<NT>(x, su);
        // (the split is complete before the slice's registers are reloaded)
#pragma unroll
        for (int i = 0; i < NT; ++i) asm volatile("" : "+v"(fa.t[i])::"memory");
        // the slice takes the next pair's values as soon as it is split (on the
        // last pair it reads this pair again, so no path keeps the old slice)
        ur[ks][0] = nxt[4 * ks];
        ur[ks][1] = nxt[4 * ks + 1];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const f16_t* pb = sB + (32 * ct + l32) * BP + 16 * ks + 8 * h;
          HFrag<NT> fb;
#pragma unroll
          for (int i = 0; i < NT; ++i) fb.t[i] = *reinterpret_cast<const f16x8*>(pb + i * COLS * BP);
          mmah<NT, NT>(T[ct], fa, fb);
        }
        sched_fence();  // bounds how far ahead fragments are loaded
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          St[ct][r] = ldexpf(T[ct][r], min(max(eu, -100), 100) + ec[ct]);
          if (!ut) St[ct][r] += Si[ct][r];
        }
      if (!more) store_results();
      if (more) {
        if (!ut) issue_Si(seg + 1);  // a whole step ahead
        put_cmax();
        if (!ut && a.prefix) store_tiles(a.prefix + (size_t)(seg + 1) * seg_stride + pair_off);
        if (!ut) g_next = a.g[pidx + (size_t)(seg + 1) * n_chain];
        __syncthreads();  // every wave is done with sB
        put_B((SEAM || ut) ? 1.f : expf(g_next));
        if constexpr (SEAM) stage_window();
        __syncthreads();
      }
    } else if constexpr (SEAM) {
      if (seg + 1 < nseg) {  // windows only: stage the next segment's first window
        stage_window();
        __syncthreads();
      } else {
        store_results();
      }
    }
  }
}


// =====================================================================================
// d = 128: one workgroup per unit, the whole state in MFMA accumulators
// =====================================================================================
// Work split.  Four waves; wave w keeps state columns 32w .. 32w+31, all 128
// rows, as four 32x32 accumulator tiles and uses them directly as the B
// operand of every product: elements 8m .. 8m+7 of a tile are a B fragment
// whose k order (rows 16m + 8(j >> 2) + 4h + (j & 3)) the A operand matches
// (common.h), so the state never goes through LDS and each column's scale is
// lane-local.  U is the A operand: each step wave rb splits rows 32 rb ..
// 32 rb + 31 (loaded into registers a step ahead, 1 KB per load instruction)
// into NT fp16 terms in LDS with one power of two per row block, and every
// wave reads all of U from there.  The split rows are stored with bits 2 and 3
// of k swapped inside each 16-wide block, so that an A fragment in the
// accumulator's k order is one 16-byte read.  Two workgroups share a CU (one
// split buffer and one window area each, about 80 KB of LDS): while one waits
// on a barrier, an LDS read or the S_B loads after its product, the other's
// MFMA and VALU work runs.  (One workgroup per CU with two split buffers, the
// next pair split between the MFMAs of the current product, measured 10 %
// slower on the seam step: per wave it issues the same VALU work and hides
// less of its waiting.)
//
// Seam windows (bf16 tokens): [X; P] = [K; Q] S on 32x32x16 MFMA (K rows 0..7,
// Q rows 8..15 of A; the upper 16 rows zero); each lane then holds X and P of
// four tokens of its column, takes the other four from its partner lane, and
// forms R = V - e^G X, R' = C^T R (lane half 0) or O = e^G P + W2 R (lane half
// 1) in fp32; S <- e^{G_n} S + K^T R' as a rank-8 bf16 MFMA update.
template <int NT, bool SEAM>
struct WideCfg {
  static constexpr int D = 128;
  static constexpr int NTH = 256;
  static constexpr int UP = D + 8;  // fp16 pitch of a split row: 272 bytes, 16-byte reads free of bank conflicts
  static constexpr int OFF_U = 0;                              // split U: [NT][D][UP] f16
  static constexpr int OFF_EU = OFF_U + NT * D * UP * 2;       // [4] int: row-block exponents
  // the window area:
  static constexpr int W_A = 0;                                // [2 SUB][UP] f16: K, Q rows, scaled
  static constexpr int W_AS = W_A + 2 * SUB * UP * 2;          // [2 SUB] f32: 2^e of those rows
  static constexpr int W_KT = W_AS + 2 * SUB * 4;              // [D][SUB] bf16: K^T
  static constexpr int W_V = W_KT + D * SUB * 2;               // [SUB][D] f32
  static constexpr int W_REC = W_V + SUB * D * 4;              // the window record
  static constexpr int WBUF = W_REC + SEAM_REC_FLOATS * 4;
  static constexpr int OFF_W = OFF_EU + 16;
  static constexpr int OFF_Z = OFF_W + WBUF;                   // a zero row, read by the lanes whose
  static constexpr int ZROW = UP * 2;                          // operand rows are padding
  static constexpr int LDS = SEAM ? OFF_Z + ZROW : OFF_W;
  static_assert(2 * LDS <= 160 * 1024, "two workgroups per CU");
};

template <int NT, bool SEAM, bool PAIRS>
__global__ __launch_bounds__(256, 2) void chain_wide_kernel(const ChainArgs a) {
  using Cfg = WideCfg<NT, SEAM>;
  constexpr int D = 128, UP = Cfg::UP;
  constexpr uint32_t MAT = D * D * 4;  // bytes of one [D][D] fp32 matrix
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  f16_t* sU = reinterpret_cast<f16_t*>(smem + Cfg::OFF_U);
  int* sEU = reinterpret_cast<int*>(smem + Cfg::OFF_EU);

  const int unit = blockIdx.x;
  const bool ut = blockIdx.y == 1;  // this workgroup composes U_total instead of S
  const int n_chain = a.n_chain;
  const int blk = a.blk_len > 0 ? unit / n_chain : 0;
  const int chain = a.blk_len > 0 ? unit % n_chain : unit;
  const int pidx = a.blk_len > 0 ? blk * a.blk_len * n_chain + chain : unit;
  const int nseg = a.blk_len > 0 ? min(a.blk_len, a.n_seg - blk * a.blk_len) : a.n_seg;
  const size_t unit_off = (size_t)unit * D * D;
  const size_t pair_off = (size_t)pidx * D * D;
  const size_t seg_stride = (size_t)n_chain * D * D;
  const int wv = wave_id_uniform();  // columns 32 wv .. (and U rows 32 wv .. for the split)

  // ---- the state tiles: element r of tile rt is row 32 rt + acc_row(r), column 32 wv + l32
  f32x16 St[4];
  auto tile_voff = [&]() {
    const int lane = opaque((int)threadIdx.x) & 63;
    return (uint32_t)(((4 * (lane >> 5)) * D + 32 * wv + (lane & 31)) * 4);
  };
  auto tile_soff = [](int rt, int r) { return (uint32_t)((32 * rt + 8 * (r >> 2) + (r & 3)) * D * 4); };
  auto load_tiles = [&](const float* base, f32x16 (&dst)[4]) {
    const auto rs = buffer_rsrc(base, MAT);
    const uint32_t vo = tile_voff();
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[rt][r] = __uint_as_float(buffer_load4(rs, vo, tile_soff(rt, r)));
  };
  auto store_tiles = [&](float* base) {
    const auto rs = buffer_rsrc(base, MAT);
    const uint32_t vo = tile_voff();
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) buffer_store4(St[rt][r], rs, vo, tile_soff(rt, r));
  };

  // ---- U of a pair: wave wv's rows, 16 loads of 1 KB (lane: row 32 wv + 2i + h, columns 4 l32 ..)
  f32x4 ur[16];
  auto issue_U = [&](int s) {
    const auto rs = buffer_rsrc(a.U + (size_t)s * seg_stride + pair_off, MAT);
    const int lane = opaque((int)threadIdx.x) & 63;
    const uint32_t vo = (uint32_t)(((lane >> 5) * D + 4 * (lane & 31)) * 4);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 v = buffer_load16(rs, vo, (uint32_t)((32 * wv + 2 * i) * D * 4));
      ur[i] = f32x4{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
    }
  };
  // split into LDS (NT fp16 terms, k permuted inside 16-blocks) with the row
  // block's power of two
  auto split_U = [&]() {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(ur[i][j]));
    const int eu = min(max(split_exp(wave_max_uniform(m)), -100), 100);
    if ((threadIdx.x & 63) == 0) sEU[wv] = eu;
    const float su = ldexpf(1.f, -eu);
    const int lane = opaque((int)threadIdx.x) & 63;
    const int c = lane & 31;
    f16_t* dst = sU + (32 * wv + (lane >> 5)) * UP + 16 * (c >> 2) + kperm(4 * (c & 3));
#pragma unroll
    for (int i = 0; i < 16; ++i) {  // slice i: rows 32 wv + 2 i + (lane >> 5)
      const H4<NT> f = split4h_scaled<NT>(ur[i], su);
#pragma unroll
      for (int t = 0; t < NT; ++t) *reinterpret_cast<f16x4*>(dst + (t * D + 2 * i) * UP) = f.t[t];
    }
  };

  // exponent of the lane's column: its 64 values and the partner lane's, times f
  auto col_exp = [&](float f) {
    float m = 0.f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(St[rt][r]));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    return min(max(split_exp(m * f), -100), 100);
  };
  // k step ks of the state as a one-term B fragment, times sc (the window
  // products feed outputs and updates of bf16-token precision)
  auto state_frag1 = [&](int ks, float sc) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = St[ks >> 1][8 * (ks & 1) + j];
    return split8h_scaled<1>(x, sc);
  };
  // k step ks of the state as an NT-term B fragment, times sc
  auto state_frag = [&](int ks, float sc) {
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = St[ks >> 1][8 * (ks & 1) + j];
    return split8h_scaled<NT>(x, sc);
  };

  // ---- body pair: S <- exp(g) U S + S_B (U_total <- U U_total) ----------------------
  // The product from the split U; then S_B of pair sb (sb < 0: none), its 64
  // loads in flight together.
  // Composition alone (one workgroup per CU when the chains are few): the
  // state's B fragments are formed half by half, so that each half of the
  // state registers takes S_B's tiles while the other half's product runs.
  auto body_split = [&](float f, int sb) {
    const int ec = col_exp(f);
    const float sc = f * ldexpf(1.f, -ec);
    // (sb < 0: a resource of no bytes, whose loads return zeros)
    const auto rs = buffer_rsrc(a.S + (size_t)max(sb, 0) * seg_stride + pair_off, sb >= 0 ? MAT : 0u);
    const uint32_t vo = tile_voff();
    f32x16 T[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) T[rt] = zero16();
    const int lane = opaque((int)threadIdx.x) & 63;
    const f16_t* pa = sU + (lane & 31) * UP + 8 * (lane >> 5);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {  // k steps 4 hf .. 4 hf + 3 read state tiles 2 hf, 2 hf + 1
      HFrag<NT> fb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) fb[k] = state_frag(4 * hf + k, sc);
#pragma unroll
      for (int rt = 2 * hf; rt < 2 * hf + 2; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) St[rt][r] = __uint_as_float(buffer_load4(rs, vo, tile_soff(rt, r)));
#pragma unroll
      for (int k = 0; k < 4; ++k) {
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          HFrag<NT> fa;
#pragma unroll
          for (int t = 0; t < NT; ++t)
            fa.t[t] = *reinterpret_cast<const f16x8*>(pa + (t * D + 32 * rt) * UP + 16 * (4 * hf + k));
          mmah<NT, NT>(T[rt], fa, fb[k]);
        }
        sched_fence();
      }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int e = sEU[rt] + ec;
#pragma unroll
      for (int r = 0; r < 16; ++r) St[rt][r] = ldexpf(T[rt][r], e) + St[rt][r];
    }
  };
  auto body = [&](float f, int sb) {
    const int ec = col_exp(f);
    const float sc = f * ldexpf(1.f, -ec);
    f32x16 T[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) T[rt] = zero16();
    const int lane = opaque((int)threadIdx.x) & 63;
    const f16_t* pa = sU + (lane & 31) * UP + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const HFrag<NT> fb = state_frag(ks, sc);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        HFrag<NT> fa;
#pragma unroll
        for (int t = 0; t < NT; ++t) fa.t[t] = *reinterpret_cast<const f16x8*>(pa + (t * D + 32 * rt) * UP + 16 * ks);
        mmah<NT, NT>(T[rt], fa, fb);
      }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int e = sEU[rt] + ec;
#pragma unroll
      for (int r = 0; r < 16; ++r) St[rt][r] = ldexpf(T[rt][r], e);
    }
    if (sb >= 0) {
      const auto rs = buffer_rsrc(a.S + (size_t)sb * seg_stride + pair_off, MAT);
      const uint32_t vo = tile_voff();
      f32x16 SB[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) SB[rt][r] = __uint_as_float(buffer_load4(rs, vo, tile_soff(rt, r)));
      sched_fence();
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) St[rt][r] += SB[rt][r];
    }
  };

  // ---- seam windows ------------------------------------------------------------------
  unsigned char* const warea = smem + Cfg::OFF_W;
  const int n_sub = SEAM ? (a.w + SUB - 1) / SUB : 1;
  const int n_win = SEAM ? n_sub * nseg : 0;  // windows in order: i = seg * n_sub + sub
  uint4 wraw[2];  // chunk tid: 8 values of a K (rows 0..7) or Q row; chunk 256 + tid: of a V row
  float wrec_r = 0.f;
  const uint32_t tok_stride = (uint32_t)n_chain * D;
  auto tok_base = [&](size_t tok0) { return (tok0 * n_chain + chain) * D; };
  auto issue_window = [&](int wi) {
    const int seg = wi / n_sub, sub = wi % n_sub;
    const int tid = opaque((int)threadIdx.x);
    const int n = min(SUB, a.w - sub * SUB);
    const size_t base = tok_base((size_t)seg * a.w + sub * SUB);
    const int row = tid >> 4, d8 = tid & 15, t = row & (SUB - 1);
    const uint16_t* src = reinterpret_cast<const uint16_t*>(row < SUB ? a.k : a.q);
    wraw[0] = t < n ? *reinterpret_cast<const uint4*>(src + base + (uint32_t)t * tok_stride + 8 * d8)
                    : make_uint4(0, 0, 0, 0);
    wraw[1] = make_uint4(0, 0, 0, 0);
    if (tid < SUB * (D / 8) && t < n)
      wraw[1] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.v) + base +
                                                (uint32_t)t * tok_stride + 8 * d8);
    const float* rec = a.wrec + ((size_t)(seg * n_sub + sub) * n_chain + chain) * SEAM_REC_FLOATS;
    if (tid < SEAM_REC_FLOATS) wrec_r = rec[tid];
  };
  auto stage_window = [&]() {
    f16_t* sA = reinterpret_cast<f16_t*>(warea + Cfg::W_A);
    float* sAS = reinterpret_cast<float*>(warea + Cfg::W_AS);
    uint16_t* sKt = reinterpret_cast<uint16_t*>(warea + Cfg::W_KT);
    float* sV = reinterpret_cast<float*>(warea + Cfg::W_V);
    float* sRec = reinterpret_cast<float*>(warea + Cfg::W_REC);
    const int tid = opaque((int)threadIdx.x);
    const int row = tid >> 4, d8 = tid & 15, t = row & (SUB - 1);
    const uint32_t u[4] = {wraw[0].x, wraw[0].y, wraw[0].z, wraw[0].w};
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(u[j] << 16);
      x[2 * j + 1] = __uint_as_float(u[j] & 0xffff0000u);
    }
    // a K or Q row scaled by the power of two of its maximum (the row's 16
    // chunks are one 16-lane DPP row), one fp16 term (exact for bf16 values)
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[j]));
    m = dpp_max_step(m, 0);
    m = dpp_max_step(m, 1);
    m = dpp_max_step(m, 2);
    m = dpp_max_step(m, 3);
    const int e = min(max(split_exp(m), -100), 100);
    const float s = ldexpf(1.f, -e);
    f16x4 lo, hi;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[j] = (f16_t)(x[j] * s);
      hi[j] = (f16_t)(x[4 + j] * s);
    }
    // columns 8 d8 + j of block d8 / 2 at positions kperm(8 (d8 & 1) + j)
    f16_t* dst = sA + row * UP + 16 * (d8 >> 1) + 4 * (d8 & 1);
    *reinterpret_cast<f16x4*>(dst) = lo;
    *reinterpret_cast<f16x4*>(dst + 8) = hi;
    if (d8 == 0) sAS[row] = ldexpf(1.f, e);
    if (row < SUB) {  // keys, transposed, as they are (bf16)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sKt[(8 * d8 + 2 * j) * SUB + t] = (uint16_t)(u[j] & 0xffffu);
        sKt[(8 * d8 + 2 * j + 1) * SUB + t] = (uint16_t)(u[j] >> 16);
      }
    }
    if (tid < SUB * (D / 8)) {  // values of token t, columns 8 d8 ..
      const uint32_t w[4] = {wraw[1].x, wraw[1].y, wraw[1].z, wraw[1].w};
      float* dv = sV + t * D + 8 * d8;
      *reinterpret_cast<f32x4*>(dv) = f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                                            __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
      *reinterpret_cast<f32x4*>(dv + 4) = f32x4{__uint_as_float(w[2] << 16), __uint_as_float(w[2] & 0xffff0000u),
                                                __uint_as_float(w[3] << 16), __uint_as_float(w[3] & 0xffff0000u)};
    }
    if (tid < SEAM_REC_FLOATS) sRec[tid] = wrec_r;
  };
  // one window sub-chunk of n tokens on the running state (LDS staged)
  // With fold (a body pair follows) the update is left as S + K^T R' / e^{G_n}
  // and e^{G_n} is returned for the body's state scale, saving the multiply of
  // every state element (unless e^{G_n} is so small that 1 / e^{G_n} could
  // overflow); else e^{G_n} is applied here and 1 returned.
  auto window = [&](int seg, int sub, bool fold) {
    const f16_t* sA = reinterpret_cast<const f16_t*>(warea + Cfg::W_A);
    const float* sAS = reinterpret_cast<const float*>(warea + Cfg::W_AS);
    const uint16_t* sKt = reinterpret_cast<const uint16_t*>(warea + Cfg::W_KT);
    const float* sV = reinterpret_cast<const float*>(warea + Cfg::W_V);
    const float* sRec = reinterpret_cast<const float*>(warea + Cfg::W_REC);
    const int n = min(SUB, a.w - sub * SUB);
    const int lane = opaque((int)threadIdx.x) & 63;
    const int h = lane >> 5, l32 = lane & 31;
    const int ec = col_exp(1.f);
    const float sc = ldexpf(1.f, -ec);
    f32x16 XP = zero16();
    {
      const f16_t* pa = (l32 < 2 * SUB ? sA + l32 * UP : reinterpret_cast<const f16_t*>(smem + Cfg::OFF_Z)) + 8 * h;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const HFrag<1> fb = state_frag1(ks, sc);
        HFrag<1> fa;
        fa.t[0] = *reinterpret_cast<const f16x8*>(pa + 16 * ks);
        mmah<1, 1>(XP, fa, fb);
      }
    }
    // elements j < 4: X of token 4h + j; elements 4 + j: P of token 4h + j
    const int c = 32 * wv + l32;
    const float cs = ldexpf(1.f, ec);
    float R4[4], P4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int t = 4 * h + j;
      const float eg = sRec[2 * SUB * SUB + t];
      R4[j] = sV[t * D + c] - eg * (XP[j] * cs * sAS[t]);
      P4[j] = eg * (XP[4 + j] * cs * sAS[SUB + t]);
    }
    float R8[SUB], EP[SUB];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float ro = __shfl_xor(R4[j], 32, 64), po = __shfl_xor(P4[j], 32, 64);
      R8[j] = h ? ro : R4[j];
      R8[4 + j] = h ? R4[j] : ro;
      EP[j] = h ? po : P4[j];
      EP[4 + j] = h ? P4[j] : po;
    }
    // lane half 0: R' = C^T R; lane half 1: O = e^G P + W2 R (fp32)
    float acc[SUB];
    const float* coef = sRec + (h ? SUB * SUB : 0);
#pragma unroll
    for (int t = 0; t < SUB; ++t) {
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(coef + t * SUB);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(coef + t * SUB + 4);
      float s = h ? EP[t] : 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        s = fmaf(c0[u], R8[u], s);
        s = fmaf(c1[u], R8[4 + u], s);
      }
      acc[t] = s;
    }
    if (h) {
      const size_t obase = tok_base((size_t)seg * a.w + sub * SUB);
#pragma unroll
      for (int t = 0; t < SUB; ++t)
        if (t < n) a.o[obase + (uint32_t)t * tok_stride + c] = acc[t];
    }
    // S <- exp(G_n) S + K^T R' (k = the 8 tokens in lane half 0; half 1 zeros)
    const float eGn = sRec[2 * SUB * SUB + SUB];
    const bool folded = fold && eGn >= 0x1p-60f;  // (uniform)
    const float rs = folded ? 1.f / eGn : 1.f;
    Frag<2> fb;
    {
      float x[8];
#pragma unroll
      for (int t = 0; t < SUB; ++t) x[t] = h ? 0.f : acc[t] * rs;
      fb = split8<2>(x);
    }
    if (!folded) {
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int r = 0; r < 16; ++r) St[rt][r] *= eGn;
    }
    const uint16_t* pk = h ? reinterpret_cast<const uint16_t*>(smem + Cfg::OFF_Z) : sKt + l32 * SUB;
    const int pk_step = h ? 0 : 32 * SUB;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      Frag<1> fa;
      fa.t[0] = *reinterpret_cast<const bf16x8*>(pk + rt * pk_step);
      mma<1, 2>(St[rt], fa, fb);
    }
    return folded ? eGn : 1.f;
  };

  // ---- start state, first loads --------------------------------------------------------
  if (!ut && a.S_in) {
    load_tiles(a.S_in + unit_off, St);
  } else {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        St[rt][r] = (ut && 32 * rt + acc_row(r, lane) == 32 * wv + (lane & 31)) ? 1.f : 0.f;
  }
  if (!ut && a.prefix) store_tiles(a.prefix + pair_off);  // prefix states follow the pairs' layout
  // Each step: stage the step's first window and split U (loaded a step ahead),
  // then the windows, then the body pair.  Window i + 1 is loaded while window
  // i is in use.
  if constexpr (SEAM) {
    if (threadIdx.x < Cfg::ZROW / 4) reinterpret_cast<float*>(smem + Cfg::OFF_Z)[threadIdx.x] = 0.f;
    issue_window(0);
  }
  // Composition from the zero state (U_total: the identity): the first step's
  // result is the first pair's S (U) itself, loaded instead of multiplied.
  int seg0 = 0;
  if constexpr (!SEAM) {
    if (PAIRS && (ut || !a.S_in) && nseg > 0) {
      load_tiles((ut ? a.U : a.S) + pair_off, St);
      seg0 = 1;
      if (nseg > 1 && !ut && a.prefix) store_tiles(a.prefix + seg_stride + pair_off);
    }
  }
  float g_cur = 0.f;
  if (PAIRS && seg0 < nseg) {
    issue_U(seg0);
    if (!ut) g_cur = a.g[pidx + (size_t)seg0 * n_chain];
  }
  for (int seg = seg0; seg < nseg; ++seg) {
    __syncthreads();  // every wave is done with the previous step's LDS
    // (the registers staged here were loaded a step ago; the next loads are
    // issued after them, so that no wait for these covers the new ones)
    if constexpr (SEAM) stage_window();
    if (PAIRS) split_U();
    const bool more = PAIRS && seg + 1 < nseg;
    const float g_nxt = (more && !ut) ? a.g[pidx + (size_t)(seg + 1) * n_chain] : 0.f;
    if (SEAM && seg * n_sub + 1 < n_win) issue_window(seg * n_sub + 1);
    if (more) issue_U(seg + 1);  // in flight during this step
    __syncthreads();
    float wfac = 1.f;  // gate factor the last window leaves to the body
    if constexpr (SEAM) {
      for (int sub = 0; sub < n_sub; ++sub) {
        const int wi = seg * n_sub + sub;
        wfac = window(seg, sub, PAIRS && sub + 1 == n_sub);
        if (sub + 1 < n_sub) {
          __syncthreads();
          stage_window();
          if (wi + 2 < n_win) issue_window(wi + 2);
          __syncthreads();
        }
      }
    }
    if (PAIRS) {
      if constexpr (SEAM) body(ut ? 1.f : expf(g_cur) * wfac, ut ? -1 : seg);
      else body_split(ut ? 1.f : expf(g_cur), ut ? -1 : seg);
      if (seg + 1 < nseg && !ut && a.prefix) store_tiles(a.prefix + (size_t)(seg + 1) * seg_stride + pair_off);
    }
    g_cur = g_nxt;
  }

  store_tiles((ut ? a.U_tot : a.S_out) + unit_off);
  if (!ut && a.g_tot && threadIdx.x == 0) {
    double acc = 0.0;
    for (int s = 0; s < nseg; ++s) acc += (double)a.g[pidx + (size_t)s * n_chain];
    a.g_tot[unit] = (float)acc;
  }
}

template <int NT, bool SEAM, bool PAIRS>
hipError_t launch_wide_p(const ChainArgs& a, bool want_ut, hipStream_t stream) {
  using Cfg = WideCfg<NT, SEAM>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&chain_wide_kernel<NT, SEAM, PAIRS>), hipFuncAttributeMaxDynamicSharedMemorySize,
      Cfg::LDS);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((chain_wide_kernel<NT, SEAM, PAIRS>), dim3(a.n_units, want_ut ? 2 : 1), dim3(Cfg::NTH),
                     Cfg::LDS, stream, a);
  return hipGetLastError();
}

template <int D, int NCT, int NT, bool SEAM, bool IN_F32, bool PAIRS>
hipError_t launch_chain_p(const ChainArgs& a, bool want_ut, hipStream_t stream) {
  using Cfg = ChainCfg<D, NCT, NT, SEAM, IN_F32>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&chain_kernel<D, NCT, NT, SEAM, IN_F32, PAIRS>),
      hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
  if (attr != hipSuccess) return attr;
  const int nx = Cfg::NCG == 1 ? a.n_units : ((a.n_units + 7) / 8) * 8 * Cfg::NCG;
  hipLaunchKernelGGL((chain_kernel<D, NCT, NT, SEAM, IN_F32, PAIRS>), dim3(nx, want_ut ? 2 : 1),
                     dim3(Cfg::NTH), Cfg::LDS, stream, a);
  return hipGetLastError();
}

template <int D, int NCT, int NT, bool SEAM, bool IN_F32>
hipError_t launch_chain_t(const ChainArgs& a, bool want_ut, hipStream_t stream) {
  if constexpr (SEAM) {
    if (a.S == nullptr) return launch_chain_p<D, NCT, NT, SEAM, IN_F32, false>(a, want_ut, stream);
  }
  return launch_chain_p<D, NCT, NT, SEAM, IN_F32, true>(a, want_ut, stream);
}

// Composition of fp32 pairs (three fp16 terms per operand): one 32-column tile
// per workgroup while the grid fits the CUs in one round (three such
// workgroups per CU), else two tiles (two workgroups per CU, each U slice
// split for twice the columns).
#ifndef HYPIC_COMPOSE_NCT1_MAX
#define HYPIC_COMPOSE_NCT1_MAX 768
#endif
template <int D>
hipError_t launch_compose_d(const ChainArgs& a, bool want_ut, hipStream_t stream) {
  // d = 128: two fp16 terms per operand.  With the leading term rounded once
  // (mul_opaque) the products carry about 2^-22 of each operand, below the
  // rounding of the matrix cores' own fp32 accumulation on these sums: composed
  // states of random fp32 pairs come out within about 1e-7 of the fp64
  // recurrence with two terms as with three.
  if constexpr (D == 128) return launch_wide_p<2, false, true>(a, want_ut, stream);
  if ((long)a.n_units * (D / 32) * (want_ut ? 2 : 1) <= HYPIC_COMPOSE_NCT1_MAX)
    return launch_chain_t<D, 1, 3, false, false>(a, want_ut, stream);
  return launch_chain_t<D, 2, 3, false, false>(a, want_ut, stream);
}

}  // namespace

namespace {
// Blocked schedule for few chains: about 256 (d = 128; d = 64: 128) (block,
// chain) units compose their blocks in parallel (two workgroups per CU with
// their U products).  Without prefix states the block pairs are then reduced
// pairwise, each level composing consecutive pairs two by two in parallel, down
// to two, which the last launch composes with the start state.  With prefix
// states each chain instead composes its block pairs in order, recording every
// block's start state, and a third level re-runs every block from its start
// state in parallel (a three-phase scan [hwlabs, section 세그먼트 누적 전이 연산자:
// the composition is associative]).
bool tree_plan(int d, int n_seg, int n_chain, bool /*prefix*/, int* blk_len, int* n_blocks) {
  if (n_seg < 8 || n_chain * (d / 32) > 256) return false;
  int nb = std::max(2, std::min(n_seg / 4, (d == 128 ? 256 : 128) / n_chain));
  const int bl = (n_seg + nb - 1) / nb;
  *blk_len = bl;
  *n_blocks = (n_seg + bl - 1) / bl;
  return *n_blocks >= 2;
}
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

// Pairs of `units` (g, U, S), 256-byte aligned parts.
size_t pairs_bytes(size_t units, int d) { return align256(units * 4) + 2 * units * d * d * 4; }

size_t compose_workspace_bytes(int d, int n_seg, int n_chain, bool prefix) {
  int bl, nb;
  if (!tree_plan(d, n_seg, n_chain, prefix, &bl, &nb)) return 0;
  const size_t units = (size_t)nb * n_chain;
  // the block pairs; with prefix states a start state per block, else the pairs
  // of the next level of the pairwise reduction
  return pairs_bytes(units, d) + (prefix ? units * d * d * 4 : pairs_bytes((size_t)((nb + 1) / 2) * n_chain, d));
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
    ChainArgs a2{};  // level 2: the block pairs of each chain in order (and each block's start state)
    float* wP = c.prefix ? wS + units * d * d : nullptr;
    a2.g = wg;
    a2.U = wU;
    a2.S = wS;
    a2.S_in = c.S_init;
    a2.S_out = c.S_out;
    a2.prefix = wP;
    a2.g_tot = c.g_tot;
    a2.U_tot = c.U_tot;
    a2.n_seg = nb;
    a2.n_chain = c.n_chain;
    a2.n_units = c.n_chain;
    // level 3 (prefix states only): every block again from its start state, in
    // parallel, emitting the state before each of its segments
    ChainArgs a3{};
    a3.g = c.g;
    a3.U = c.U;
    a3.S = c.S;
    a3.S_in = wP;
    a3.S_out = wS;  // the block pairs are spent by now
    a3.prefix = c.prefix;
    a3.n_seg = c.n_seg;
    a3.n_chain = c.n_chain;
    a3.blk_len = bl;
    a3.n_units = (int)units;
    auto launch = [&](const ChainArgs& x, bool want_ut) {
      return d == 128 ? launch_compose_d<128>(x, want_ut, stream)
                      : d == 64 ? launch_compose_d<64>(x, want_ut, stream) : hipErrorInvalidValue;
    };
    hipError_t e = launch(a1, true);
    if (!wP) {
      // no prefix states: the block pairs reduced pairwise (each level composes
      // consecutive pairs two by two, in parallel) until at most two are left
      float* g_cur = wg;
      float* U_cur = wU;
      float* S_cur = wS;
      unsigned char* nxt = reinterpret_cast<unsigned char*>(ws) + pairs_bytes(units, d);
      float* g_nx = reinterpret_cast<float*>(nxt);
      float* U_nx = reinterpret_cast<float*>(nxt + align256((size_t)((nb + 1) / 2) * c.n_chain * 4));
      float* S_nx = U_nx + (size_t)((nb + 1) / 2) * c.n_chain * d * d;
      int n = nb;
      while (e == hipSuccess && n > 2) {
        const int n2 = (n + 1) / 2;
        ChainArgs al{};
        al.g = g_cur;
        al.U = U_cur;
        al.S = S_cur;
        al.S_out = S_nx;
        al.g_tot = g_nx;
        al.U_tot = U_nx;
        al.n_seg = n;
        al.n_chain = c.n_chain;
        al.blk_len = 2;
        al.n_units = n2 * c.n_chain;
        e = launch(al, true);
        std::swap(g_cur, g_nx);
        std::swap(U_cur, U_nx);
        std::swap(S_cur, S_nx);
        n = n2;
      }
      a2.g = g_cur;
      a2.U = U_cur;
      a2.S = S_cur;
      a2.n_seg = n;
    }
    if (e == hipSuccess) e = launch(a2, c.U_tot != nullptr);
    if (e == hipSuccess && wP) e = launch(a3, false);
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
  if (d == 128) return launch_compose_d<128>(a, ut, stream);
  if (d == 64) return launch_compose_d<64>(a, ut, stream);
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
  a.o = s.o;
  a.wrec = s.wrec;
  a.n_seg = s.n_seg;
  a.n_chain = s.n_chain;
  a.w = s.w;
  // bf16 tokens: two fp16 terms per body operand (the outputs are of bf16
  // input precision); fp32 tokens: three
  constexpr int NCT64 = HYPIC_SEAM_NCT > 2 ? 2 : HYPIC_SEAM_NCT;
  if (d == 128) {
    if (in_f32) return launch_chain_t<128, 1, 3, true, true>(a, false, stream);
    return a.S == nullptr ? launch_wide_p<2, true, false>(a, false, stream)
                          : launch_wide_p<2, true, true>(a, false, stream);
  }
  if (d == 64)
    return in_f32 ? launch_chain_t<64, 1, 3, true, true>(a, false, stream)
                  : launch_chain_t<64, NCT64, 2, true, false>(a, false, stream);
  return hipErrorInvalidValue;
}

}  // namespace hypic
