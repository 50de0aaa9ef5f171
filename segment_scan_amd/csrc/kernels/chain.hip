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
// placed on one XCD and share its L2 copy of U).  Wave (rb, cb) keeps the
// 32 x 32 state tile at rows 32 rb, columns 32 cb of the group in MFMA
// accumulators for the whole chain.
//
// Operands.  Products run on 32x32x16 fp16 MFMA with both fp32 operands as
// hi + lo fp16 terms, keeping hi*hi + hi*lo + lo*hi: about 2^-22 relative, the
// fp32 class, in three products where three-term bf16 needs six.  Each U (fp32
// in HBM) is split once per workgroup into LDS, each row scaled by a power of
// two (a thread holds a contiguous piece of a row, so the row maximum is a
// short DPP reduction).  After every update the state is split once into
// column-major hi/lo arrays in LDS, each column scaled by a power of two from
// the column maxima the four row-block waves leave behind; every product then
// reads its B fragments from there.  The next pair's U and S tile are in
// flight during the current segment.
//
// Per seam window (sub-chunks of up to 8 tokens; the chunk form of the delta
// rule with start state S, gate prefix G within the sub-chunk, n tokens; the
// state-independent factors C, W2, exp(G) come from seam_prep.hip):
//   [X; P] = [K; Q] S                    one MFMA product per column block
//   R  = V - diag(exp(G)) X,  O = diag(exp(G)) P + W2 R,  R' = C^T R
//   S' = exp(G_n) S + K^T R'             a rank-8 MFMA update of every tile
#include <algorithm>

#include "common.h"
#include "../launch.h"

namespace hypic {

namespace {

constexpr int SUB = 8;  // window tokens per sub-chunk

template <int D, int NCB, bool SEAM, bool IN_F32>
struct ChainCfg {
  static constexpr int NRB = D / 32;          // row blocks (waves per column block)
  static constexpr int NW = NRB * NCB;        // waves
  static constexpr int NTH = 64 * NW;
  static constexpr int COLS = 32 * NCB;       // state columns of the workgroup
  static constexpr int NCG = (D / 32) / NCB;  // column groups per chain
  static constexpr int UP = D + 8;            // fp16 pitch of U rows, state columns, window rows
  static constexpr int TPR = NTH / D;         // threads per U row while staging
  static constexpr int LDU = D / TPR / 4;     // float4 of U per thread
  static constexpr int NTK = IN_F32 ? 3 : 1;  // bf16 terms of window keys in the update
  static constexpr int RPP = SUB + 4;         // fp32 pitch of R' columns
  static constexpr int OFF_UH = 0;
  static constexpr int OFF_UL = OFF_UH + D * UP * 2;
  static constexpr int OFF_BH = OFF_UL + D * UP * 2;
  static constexpr int OFF_BL = OFF_BH + COLS * UP * 2;
  static constexpr int OFF_CM = OFF_BL + COLS * UP * 2;  // column maxima per row block [NRB][COLS]
  static constexpr int OFF_RF = OFF_CM + NRB * COLS * 4;  // exponent of each U row
  static constexpr int OFF_W = OFF_RF + D * 4;
  // window (SEAM): [K; Q] rows scaled and split to fp16, their scales, K^T in
  // bf16 terms, V of the group's columns, R' (column-major), the window record
  static constexpr int OFF_AH = OFF_W;
  static constexpr int OFF_AL = OFF_AH + 2 * SUB * UP * 2;
  static constexpr int OFF_AS = OFF_AL + (IN_F32 ? 2 * SUB * UP * 2 : 0);
  static constexpr int OFF_KT = OFF_AS + 2 * SUB * 4;
  static constexpr int OFF_V = OFF_KT + NTK * D * SUB * 2;
  static constexpr int OFF_RP = OFF_V + SUB * COLS * 4;
  static constexpr int OFF_REC = OFF_RP + COLS * RPP * 4;
  static constexpr int LDS = SEAM ? OFF_REC + SEAM_REC_FLOATS * 4 : OFF_W;
  // window token chunks of 8 elements: K and Q rows, then V rows of the group
  static constexpr int NWCH = 2 * SUB * (D / 8) + SUB * (COLS / 8);
  static constexpr int WPT = (NWCH + NTH - 1) / NTH;  // chunks per thread
  static_assert(LDS <= 160 * 1024, "LDS budget");
  static_assert(TPR >= 2 && TPR <= 8 && LDU % 2 == 0, "U staging");
  static_assert(2 * SUB * (D / 8) <= NTH || !SEAM, "window rows: one chunk per thread");
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

// x (already scaled) -> fp16 hi and lo, both rounded to nearest:
// |x - hi| <= 2^-11 |x| and |x - hi - lo| <= 2^-22 |x| in fp16's normal range
__device__ __forceinline__ f32x4 mfma16h(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16_t hi_h(float x) { return (f16_t)x; }
__device__ __forceinline__ f16_t lo_h(float x, f16_t hi) { return (f16_t)(x - (float)hi); }

template <int D, int NCB, bool SEAM, bool IN_F32>
__global__ __launch_bounds__(64 * (D / 32) * NCB) void chain_kernel(const ChainArgs a) {
  using Cfg = ChainCfg<D, NCB, SEAM, IN_F32>;
  constexpr int NRB = Cfg::NRB, NTH = Cfg::NTH, COLS = Cfg::COLS, NCG = Cfg::NCG;
  constexpr int UP = Cfg::UP, TPR = Cfg::TPR, LDU = Cfg::LDU, NTK = Cfg::NTK, RPP = Cfg::RPP;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  f16_t* sUh = reinterpret_cast<f16_t*>(smem + Cfg::OFF_UH);
  f16_t* sUl = reinterpret_cast<f16_t*>(smem + Cfg::OFF_UL);
  f16_t* sBh = reinterpret_cast<f16_t*>(smem + Cfg::OFF_BH);  // [col][row]
  f16_t* sBl = reinterpret_cast<f16_t*>(smem + Cfg::OFF_BL);
  float* sCM = reinterpret_cast<float*>(smem + Cfg::OFF_CM);  // [row block][col]
  int* sRE = reinterpret_cast<int*>(smem + Cfg::OFF_RF);  // power-of-two exponent of each U row

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
    tcol = 32 * cb + l32;  // this lane's state column within the group
  };
  refresh();

  // ---- U: loads, then the split into LDS -----------------------------------------
  // thread t holds row t / TPR, float4 columns (t % TPR) + TPR i: the TPR
  // threads of a row read whole 128-byte lines with each load instruction
  f32x4 ureg[LDU];
  // (seam mode: in two halves, the first flying through the whole previous
  // segment, the second only through its product, which keeps the window phase
  // lighter; compose mode: whole, one segment ahead)
  auto issue_U = [&](int s, int i0, int i1) {
    const f32x4* src = reinterpret_cast<const f32x4*>(a.U + (size_t)s * seg_stride + pair_off) +
                       (tid / TPR) * (D / 4) + tid % TPR;
#pragma unroll
    for (int i = 0; i < LDU; ++i)
      if (i >= i0 && i < i1) ureg[i] = src[TPR * i];
  };
  auto store_U = [&]() {
    const int row = tid / TPR, c0 = 4 * (tid % TPR);
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < LDU; ++i)
      m = fmaxf(m, fmaxf(fmaxf(fabsf(ureg[i][0]), fabsf(ureg[i][1])), fmaxf(fabsf(ureg[i][2]), fabsf(ureg[i][3]))));
    m = dpp_max_step(m, 0);  // the row's TPR threads are consecutive lanes
    if (TPR >= 4) m = dpp_max_step(m, 1);
    if (TPR >= 8) m = dpp_max_step(m, 2);
    const int e = split_exp(m);
    const float s = ldexpf(1.f, -e);
#pragma unroll
    for (int i = 0; i < LDU; ++i) {
      f16x4 hv, lv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = ureg[i][j] * s;
        hv[j] = hi_h(x);
        lv[j] = lo_h(x, hv[j]);
      }
      *reinterpret_cast<f16x4*>(sUh + row * UP + c0 + 4 * TPR * i) = hv;
      *reinterpret_cast<f16x4*>(sUl + row * UP + c0 + 4 * TPR * i) = lv;
    }
    if (tid % TPR == 0) sRE[row] = e;
  };

  // ---- the state tile and its split ------------------------------------------------
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
  // the tile's share of its columns' maxima
  auto put_cmax = [&](const f32x16& t) {
    float m = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(t[r]));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    if (h == 0) sCM[rb * COLS + tcol] = m;
  };
  // after a barrier: the column's exponent, and the tile times f split into
  // the B arrays (f = exp(g) of the pair the split feeds, else 1)
  int ec = 0;  // the lane's column is stored as x f 2^-ec
  auto put_B = [&](const f32x16& t, float f) {
    float m = 0.f;
#pragma unroll
    for (int s = 0; s < NRB; ++s) m = fmaxf(m, sCM[s * COLS + tcol]);
    ec = split_exp(m * f);
    const float sc = ldexpf(1.f, -ec) * f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f16x4 hv, lv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = t[4 * q + j] * sc;
        hv[j] = hi_h(x);
        lv[j] = lo_h(x, hv[j]);
      }
      const int off = tcol * UP + 32 * rb + 8 * q + 4 * h;
      *reinterpret_cast<f16x4*>(sBh + off) = hv;
      *reinterpret_cast<f16x4*>(sBl + off) = lv;
    }
  };

  // ---- seam windows: staging and the two products ------------------------------------
  [[maybe_unused]] f16_t* sAh = reinterpret_cast<f16_t*>(smem + Cfg::OFF_AH);  // [2 SUB][UP]: K, Q rows
  [[maybe_unused]] f16_t* sAl = reinterpret_cast<f16_t*>(smem + Cfg::OFF_AL);
  [[maybe_unused]] float* sAS = reinterpret_cast<float*>(smem + Cfg::OFF_AS);     // 2^e of those rows
  [[maybe_unused]] bf16_t* sKt = reinterpret_cast<bf16_t*>(smem + Cfg::OFF_KT);   // [NTK][D][SUB]
  [[maybe_unused]] float* sV = reinterpret_cast<float*>(smem + Cfg::OFF_V);       // [SUB][COLS]
  [[maybe_unused]] float* sRp = reinterpret_cast<float*>(smem + Cfg::OFF_RP);     // [COLS][RPP]
  [[maybe_unused]] float* sRec = reinterpret_cast<float*>(smem + Cfg::OFF_REC);
  const int n_sub = SEAM ? (a.w + SUB - 1) / SUB : 0;
  using Raw = uint4[IN_F32 ? 2 : 1];
  Raw wraw[Cfg::WPT];
  constexpr int RPT = (SEAM_REC_FLOATS + NTH - 1) / NTH;  // record floats per thread
  float wrec_r[RPT];
  // loads of window (seg, sub): chunk i < 2 SUB (D / 8) is 8 elements of a K
  // (t < SUB) or Q row, the rest 8 values of a V row of the group's columns
  auto issue_window = [&](int seg, int sub) {
    const int n = min(SUB, a.w - sub * SUB);
    const size_t tok0 = (size_t)seg * a.w + sub * SUB;
#pragma unroll
    for (int k = 0; k < Cfg::WPT; ++k) {
      const int i = tid + k * NTH;
      int t = -1;
      const void* src = nullptr;
      size_t off = 0;
      if (i < 2 * SUB * (D / 8)) {
        const int row = i / (D / 8), d8 = i % (D / 8);
        t = row % SUB;
        src = row < SUB ? a.k : a.q;
        off = ((tok0 + t) * n_chain + chain) * D + 8 * d8;
      } else if (i < Cfg::NWCH) {
        const int j = i - 2 * SUB * (D / 8);
        t = j / (COLS / 8);
        src = a.v;
        off = ((tok0 + t) * n_chain + chain) * D + col0 + 8 * (j % (COLS / 8));
      }
#pragma unroll
      for (int u = 0; u < (IN_F32 ? 2 : 1); ++u) wraw[k][u] = make_uint4(0, 0, 0, 0);
      if (t >= 0 && t < n) {
        const uint4* p = reinterpret_cast<const uint4*>(reinterpret_cast<const unsigned char*>(src) +
                                                        off * (IN_F32 ? 4 : 2));
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
        const int e = split_exp(m);
        const float sc = ldexpf(1.f, -e);
        f16x8 hv, lv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float xs = x[j] * sc;
          hv[j] = hi_h(xs);
          lv[j] = lo_h(xs, hv[j]);
        }
        *reinterpret_cast<f16x8*>(sAh + row * UP + 8 * d8) = hv;
        if constexpr (IN_F32) *reinterpret_cast<f16x8*>(sAl + row * UP + 8 * d8) = lv;
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

  // ---- start state -----------------------------------------------------------------
  f32x16 St;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const size_t row = 32 * rb + acc_row(r, lane);
    if (ut) {
      St[r] = ((int)row == col0 + tcol) ? 1.f : 0.f;
    } else {
      St[r] = a.S_in ? a.S_in[chain_off + row * D + col0 + tcol] : 0.f;
    }
  }
  if (!ut && a.prefix) store_tile(a.prefix + pair_off, St);  // prefix states follow the pairs' layout
  put_cmax(St);
  float g_next = 0.f;
  if (pairs) {
    issue_U(0, 0, LDU);
    if (!ut) issue_Si(0);
    g_next = ut ? 0.f : a.g[pidx];
  }
  if constexpr (SEAM) issue_window(0, 0);
  __syncthreads();
  put_B(St, (SEAM || !pairs) ? 1.f : __expf(g_next));
  if (pairs) {
    store_U();
    if (nseg > 1) issue_U(1, 0, SEAM ? LDU / 2 : LDU);
  }
  if constexpr (SEAM) stage_window();
  __syncthreads();

  for (int seg = 0; seg < nseg; ++seg) {
    // ---- seam window of this segment -----------------------------------------------
    if constexpr (SEAM) {
      for (int sub = 0; sub < n_sub; ++sub) {
        refresh();
        const int n = min(SUB, a.w - sub * SUB);
        const size_t tok0 = (size_t)seg * a.w + sub * SUB;
        // the next window's loads fly during this one and the body pair
        if (sub + 1 < n_sub) issue_window(seg, sub + 1);
        else if (seg + 1 < nseg) issue_window(seg + 1, 0);
        const float* sCt = sRec;              // [t][s]: Abar[t][s] exp(G_n - G_t)
        const float* sW2 = sRec + SUB * SUB;  // [t][s]: ((tril(Q K^T) o Gamma) Abar)[t][s]
        const float* sEG = sRec + 2 * SUB * SUB;  // exp(G_t); [SUB] = exp(G_n)
        // W1: [X; P] = [K; Q] S for the column block (its first row-block wave),
        // on 16x16x32 MFMA: rows are the 8 keys and 8 queries, two 16-column tiles
        if (rb == 0) {
          const int l16 = lane & 15, g = lane >> 4;
          f32x4 XP[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
          const f16_t* pah = sAh + l16 * UP + 8 * g;
          const f16_t* pal = sAl + l16 * UP + 8 * g;
#pragma unroll
          for (int ks = 0; ks < D / 32; ++ks) {
            const f16x8 fah = *reinterpret_cast<const f16x8*>(pah + 32 * ks);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
              const int col = 32 * cb + 16 * ct + l16;
              const f16x8 fbh = *reinterpret_cast<const f16x8*>(sBh + col * UP + 32 * ks + 8 * g);
              const f16x8 fbl = *reinterpret_cast<const f16x8*>(sBl + col * UP + 32 * ks + 8 * g);
              XP[ct] = mfma16h(fah, fbl, XP[ct]);
              XP[ct] = mfma16h(fah, fbh, XP[ct]);
              if constexpr (IN_F32) {
                const f16x8 fal = *reinterpret_cast<const f16x8*>(pal + 32 * ks);
                XP[ct] = mfma16h(fal, fbh, XP[ct]);
              }
            }
            sched_fence();  // bounds how far ahead fragments are loaded
          }
          // lane (l16, g), tile ct: column 32 cb + 16 ct + l16, rows 4g + j: X of
          // token 4g + j (g < 2) or P of token 4(g - 2) + j (g >= 2).  Every lane
          // scales its rows; X lanes form R; P lanes gather the column's R and
          // emit the outputs and R'.
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) {
            const int col = 32 * cb + 16 * ct + l16;
            const float cs = ldexpf(1.f, __shfl(ec, (lane & 32) | (16 * ct + l16), 64));  // the column's exponent
            float v4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int row = 4 * g + j;  // 0..7 keys, 8..15 queries
              const int t = row & 7;
              const float x = XP[ct][j] * sAS[row] * cs;
              v4[j] = g < 2 ? sV[t * COLS + col] - sEG[t] * x : sEG[t] * x;  // R, or exp(G) P
            }
            float Ra[SUB];  // R of the column's 8 tokens, from its two X lane groups
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              Ra[j] = __shfl(v4[j], l16, 64);
              Ra[4 + j] = __shfl(v4[j], 16 + l16, 64);
            }
            if (g >= 2) {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int t = 4 * (g - 2) + j;
                const f32x4 w0 = *reinterpret_cast<const f32x4*>(sW2 + t * SUB);
                const f32x4 w1 = *reinterpret_cast<const f32x4*>(sW2 + t * SUB + 4);
                const f32x4 c0 = *reinterpret_cast<const f32x4*>(sCt + t * SUB);
                const f32x4 c1 = *reinterpret_cast<const f32x4*>(sCt + t * SUB + 4);
                const float w8[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
                const float c8[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
                float o = v4[j], rp = 0.f;
#pragma unroll
                for (int s = 0; s < SUB; ++s) {
                  o = fmaf(w8[s], Ra[s], o);  // W2 is lower triangular
                  rp = fmaf(c8[s], Ra[s], rp);
                }
                if (t < n) a.o[((tok0 + t) * n_chain + chain) * D + col0 + col] = o;
                sRp[col * RPP + t] = rp;
                sched_fence();  // one token's record rows in registers at a time
              }
            }
          }
        }
        __syncthreads();
        // W2: S = exp(G_n) S + K^T R' on every tile (k = the 8 tokens; lanes of
        // the upper k half hold zeros)
        {
          const float eGn = sEG[SUB];
#pragma unroll
          for (int r = 0; r < 16; ++r) St[r] *= eGn;
          Frag<NTK> fa;
          Frag<3> fb;
          if (h == 0) {
#pragma unroll
            for (int term = 0; term < NTK; ++term)
              fa.t[term] = *reinterpret_cast<const bf16x8*>(sKt + (term * D + 32 * rb + l32) * SUB);
            const f32x4 r0 = *reinterpret_cast<const f32x4*>(sRp + tcol * RPP);
            const f32x4 r1 = *reinterpret_cast<const f32x4*>(sRp + tcol * RPP + 4);
            const float x[8] = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
            fb = split8<3>(x);
          } else {
#pragma unroll
            for (int term = 0; term < NTK; ++term) fa.t[term] = bf16x8{};
#pragma unroll
            for (int term = 0; term < 3; ++term) fb.t[term] = bf16x8{};
          }
          mma<NTK, 3>(St, fa, fb);
          put_cmax(St);
        }
        __syncthreads();
        put_B(St, (sub + 1 == n_sub && pairs) ? __expf(g_next) : 1.f);
        if (sub + 1 < n_sub) stage_window();
        __syncthreads();
      }
    }

    // ---- body pair: S <- exp(g) U S + S_B (or U_total <- U U_total) ----------------
    if (pairs) {
      refresh();
      if (SEAM && seg + 1 < nseg) issue_U(seg + 1, LDU / 2, LDU);
      // T = U (exp(g) S) 2^-ec / 2^e_row (+ S_B 2^-ec / 2^e_row): in seam mode the
      // pair's state enters as the accumulator's start (all factors are powers of
      // two), which frees its registers during the product; in compose mode it is
      // added afterwards, which gives its loads the product's time to land
      f32x16 T;
      int er[16];  // the product's scale exponent per element (row and column)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        er[r] = sRE[32 * rb + acc_row(r, lane)] + ec;
        T[r] = (ut || !SEAM) ? 0.f : ldexpf(Si[r], -er[r]);
      }
      {
        const f16_t* ah = sUh + (32 * rb + l32) * UP + 8 * h;
        const f16_t* al = sUl + (32 * rb + l32) * UP + 8 * h;
        const f16_t* bh = sBh + tcol * UP + 8 * h;
        const f16_t* bl = sBl + tcol * UP + 8 * h;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const f16x8 fah = *reinterpret_cast<const f16x8*>(ah + 16 * ks);
          const f16x8 fal = *reinterpret_cast<const f16x8*>(al + 16 * ks);
          const f16x8 fbh = *reinterpret_cast<const f16x8*>(bh + 16 * ks);
          const f16x8 fbl = *reinterpret_cast<const f16x8*>(bl + 16 * ks);
          T = mfma32h(fal, fbh, T);
          T = mfma32h(fah, fbl, T);
          T = mfma32h(fah, fbh, T);
          sched_fence();  // bounds how far ahead fragments are loaded
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        St[r] = ldexpf(T[r], er[r]);
        if (!SEAM && !ut) St[r] += Si[r];
      }
      put_cmax(St);
      if (seg + 1 < nseg) {
        if (!ut && a.prefix) store_tile(a.prefix + (size_t)(seg + 1) * seg_stride + pair_off, St);
        if (!ut) g_next = a.g[pidx + (size_t)(seg + 1) * n_chain];
      }
      __syncthreads();  // every wave is done with sU and sB
      put_B(St, (SEAM || seg + 1 == nseg || ut) ? 1.f : __expf(g_next));
      if (seg + 1 < nseg) {
        store_U();
        if constexpr (SEAM) stage_window();
        // the next pair's loads, after the staging work of this interval
        if (!ut) issue_Si(seg + 1);
        if (seg + 2 < nseg) issue_U(seg + 2, 0, SEAM ? LDU / 2 : LDU);
      }
      __syncthreads();
    } else if constexpr (SEAM) {
      if (seg + 1 < nseg) {  // windows only: stage the next segment's first window
        stage_window();
        __syncthreads();
      }
    }
  }

  // ---- results: the tiles, from registers ------------------------------------------
  float* dst = ut ? a.U_tot : a.S_out;
  store_tile(dst + chain_off, St);
  if (!ut && a.g_tot && cgrp == 0 && tid == 0) {
    double acc = 0.0;
    for (int s = 0; s < nseg; ++s) acc += (double)a.g[pidx + (size_t)s * n_chain];
    a.g_tot[chain] = (float)acc;
  }
}

template <int D, int NCB, bool SEAM, bool IN_F32>
hipError_t launch_chain_t(const ChainArgs& a, bool want_ut, hipStream_t stream) {
  using Cfg = ChainCfg<D, NCB, SEAM, IN_F32>;
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
// many chains: one workgroup per chain (no duplicated U staging).  The seam
// step with fp32 tokens at d = 128 keeps two column blocks per workgroup, for
// its larger window staging to fit in LDS.
template <int D, bool SEAM, bool IN_F32>
hipError_t launch_chain_d(const ChainArgs& a, bool want_ut, hipStream_t stream) {
  constexpr int NCBT = (SEAM && IN_F32 && D == 128) ? 2 : D / 32;
  if (a.n_units * (D / 32) <= 256) return launch_chain_t<D, 1, SEAM, IN_F32>(a, want_ut, stream);
  return launch_chain_t<D, NCBT, SEAM, IN_F32>(a, want_ut, stream);
}

}  // namespace

namespace {
// Two-level schedule for few chains: about 128 (block, chain) units compose
// their blocks in parallel, then each chain composes its block pairs in order.
// With prefix states a third level re-runs every block from its start state in
// parallel (a three-phase scan [hwlabs, section 세그먼트 누적 전이 연산자: the
// composition is associative]).
bool tree_plan(int d, int n_seg, int n_chain, bool /*prefix*/, int* blk_len, int* n_blocks) {
  if (n_seg < 8 || n_chain * (d / 32) > 256) return false;
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
  return align256(units * 4) + (prefix ? 3 : 2) * units * d * d * 4;  // g, U, S (and start state) per block
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
    hipError_t e;
    if (d == 128) {
      e = launch_chain_d<128, false, false>(a1, true, stream);
      if (e == hipSuccess) e = launch_chain_d<128, false, false>(a2, c.U_tot != nullptr, stream);
      if (e == hipSuccess && wP) e = launch_chain_d<128, false, false>(a3, false, stream);
    } else if (d == 64) {
      e = launch_chain_d<64, false, false>(a1, true, stream);
      if (e == hipSuccess) e = launch_chain_d<64, false, false>(a2, c.U_tot != nullptr, stream);
      if (e == hipSuccess && wP) e = launch_chain_d<64, false, false>(a3, false, stream);
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
