// launch.h -- host-side launchers of the gfx950 kernels (internal to libhypic).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/hypic.h"

namespace hypic {

// Sets the calling thread's error message (printf format) and returns st; the
// message hypic_last_error reports.
hypic_status report_error(hypic_status st, const char* fmt, ...);

// Segments handled by one launch of a build kernel; their offsets travel by
// value in the kernel arguments (no device-side table to allocate).
constexpr int kMaxSegPerLaunch = 240;

// Slot i of a launch (workgroup row i) builds the segment of tokens
// [beg[i], end[i]) into output row out[i].  The host fills the slots in
// longest-processing-time order over the whole batch: all segments sorted by
// length, longest first (ties by index), launches taking consecutive runs of
// that order -- so in a ragged batch the longest units start first, in the
// first launch, and the short ones fill the tails.
struct SegTable {
  int32_t beg[kMaxSegPerLaunch];
  int32_t end[kMaxSegPerLaunch];
  int32_t out[kMaxSegPerLaunch];
  int n_seg;  // slots in this launch
  // 1: equal lengths and consecutive segments (slot i is segment out[0] + i,
  // tokens from beg[0] + i (end[0] - beg[0])), so kernels may skip the lookup
  int contiguous;
};

inline int seg_len(const SegTable& t, int s) { return t.end[s] - t.beg[s]; }
inline bool seg_uniform(const SegTable& t) { return t.contiguous != 0; }

// Composition fused into the delta build (hypic_seg_build_compose, fused
// schedule): the request's segments are the leaves of a binary tree per chain
// (leaf i at heap index P + i, node k over its children 2k and 2k + 1; a node
// whose right subtree holds no segment stands for its left child).  A build
// workgroup that has written its pair counts its arrival at the parent node;
// the last arrival composes the node's two children into the node's pair and
// moves up, the root's pair going to S_out, g_tot and U_tot.  No workgroup waits
// for another.
struct FuseArgs {
  int* cnt = nullptr;  // [P][n_chain] arrival counters, zero on entry (nullptr: not fused)
  float* g = nullptr;  // node pairs: g [P][n_chain], U and S [P][n_chain][d][d] (index k < P)
  float* U = nullptr;
  float* S = nullptr;
  float* S_out = nullptr;  // the root: S [n_chain][d][d], g [n_chain], U (or nullptr)
  float* g_tot = nullptr;
  float* U_tot = nullptr;
  int P = 0;      // leaves: a power of two >= n_seg
  int n_seg = 0;  // segments of the request
};

struct BuildArgs {
  const void* k;
  const void* v;
  const void* beta;
  const void* lg;
  float* g;
  float* U;
  float* S;
  int n_chain;
  int gate_per_chain;
  SegTable seg;
  FuseArgs fuse;  // delta build, two-kernel path only
};

struct ComposeArgs {
  const float* g;  // [n_seg, n_chain] or [n_seg, n_chain, d] (diag)
  const float* U;  // [n_seg, n_chain, d, d] (delta)
  const float* S;  // [n_seg, n_chain, d, d]
  const float* S_init;
  float* S_out;
  float* prefix;
  float* g_tot;
  float* U_tot;
  int n_seg;
  int n_chain;
  // Grouped composition (elementwise families): n_out outputs, output h composes
  // the n_seg consecutive pairs (h / n_chain) * n_seg + i, i < n_seg, of chain
  // h % n_chain.  n_out = n_chain is the plain composition of all pairs.
  int n_out;
};

struct SeamArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const void* lg;
  int gate_per_chain;
  const float* bg;  // body pairs (bS == nullptr: none)
  const float* bU;
  const float* bS;
  float* S_run;
  float* o;
  float* wg;  // window pairs (wS == nullptr: none)
  float* wU;
  float* wS;
  int n_seg;
  int w;
  int n_chain;
  const float* wrec;  // delta family: per-window records of seam_prep (see below)
};

// fam: 0 naive, 1 scalar, 2 diag, 3 delta.  d in {64, 128}.
hipError_t launch_build_sd(int fam, int d, bool in_f32, const BuildArgs& a, int n_blocks,
                           hipStream_t stream);
// Delta build.  For d = 128 with bf16 tokens and segments of at most
// kDelta2MaxSegLen tokens it runs as two kernels that hand per-chunk factors
// over through a caller workspace of build_delta_workspace() bytes; otherwise
// one kernel that needs no workspace (ws may then be NULL).
constexpr int kDelta2MaxSegLen = 2048;
size_t build_delta_workspace(int d, bool in_f32, const SegTable& seg, int n_chain);
hipError_t launch_build_delta(int d, bool in_f32, const BuildArgs& a, int n_blocks, void* ws,
                              hipStream_t stream);
// the single-kernel path for any size (no workspace)
hipError_t launch_build_delta_single(int d, bool in_f32, const BuildArgs& a, int n_blocks, hipStream_t stream);
// the two-kernel path (build_delta2.hip)
size_t delta2_workspace_bytes(const SegTable& seg, int n_chain);
hipError_t launch_build_delta2(const BuildArgs& a, void* ws, hipStream_t stream);
// zero n ints (the fused composition's counters) with a kernel, so the call can
// be captured into a graph
hipError_t launch_zero_ints(int* p, size_t n, hipStream_t stream);
hipError_t launch_compose_elem(int fam, int d, const ComposeArgs& a, hipStream_t stream);
// dense composition and the delta seam step on the column-split chain kernel (chain.hip)
// With a workspace of compose_workspace_bytes() (0 when the schedule does not
// apply), few-chain compositions without prefix states run in two levels.
size_t compose_workspace_bytes(int d, int n_seg, int n_chain, bool prefix);
hipError_t launch_compose_chain(int d, const ComposeArgs& a, void* ws, size_t ws_bytes, hipStream_t stream);
hipError_t launch_seam_chain(int d, bool in_f32, const SeamArgs& a, hipStream_t stream);
// Delta seam step: the state-independent part of every window (8-token
// sub-chunks) is formed first into a workspace of seam_workspace_bytes(), one
// record of SEAM_REC_FLOATS floats per (segment, sub-chunk, chain):
// C^T[8][8], W2[8][8], exp(G)[8], exp(G_n) (seam_prep.hip).
constexpr int SEAM_REC_FLOATS = 144;
size_t seam_workspace_bytes(int n_seg, int w, int n_chain);
hipError_t launch_seam_prep(int d, bool in_f32, const SeamArgs& a, float* ws, hipStream_t stream);
// seam step of the naive, scalar and diagonal families (seam_elem.hip)
hipError_t launch_seam_elem(int fam, int d, bool in_f32, const SeamArgs& a, hipStream_t stream);
// Chunk table of a two-kernel build launch: records are dense over the launch's
// 64-token chunks, record (base[s] + c) * n_chain + chain holding chunk c of
// segment s on that chain.
struct ChunkTable {
  int32_t base[kMaxSegPerLaunch + 1];  // chunks of the segments before s
};
inline int chunk_table(const SegTable& seg, ChunkTable* ct) {
  int n = 0;
  for (int s = 0; s < seg.n_seg; ++s) {
    if (ct) ct->base[s] = n;
    n += (seg_len(seg, s) + 63) / 64;
  }
  if (ct) ct->base[seg.n_seg] = n;
  return n;
}

// KDA build (build_kda.hip), built for d = 64 (bf16 or fp32 tokens) and d = 128
// (bf16 tokens).  With d = 128, bf16 tokens and segments of at most
// kDelta2MaxSegLen tokens it runs as a factor pass writing one record per
// (chunk, chain) into a workspace of kda_workspace_bytes() and the delta state
// pass in its KDA mode (build_delta2.hip); otherwise as one kernel without
// workspace (ws may then be NULL).
bool kda_build_supported(int d, bool in_f32);
size_t kda_workspace_bytes(int d, bool in_f32, const SegTable& seg, int n_chain);
hipError_t launch_build_kda(int d, bool in_f32, const BuildArgs& a, int n_blocks, void* ws, hipStream_t stream);
// Record of one (chunk, chain) of the KDA factor pass: the decayed keys
// Kb = K o e^H (fp16 [64][128]) and Kd = (K o e^(H_C - H))^T (fp16 [128][64]),
// X = (I + M)^-1 diag(b) (fp16 [64][64], each row scaled by a power of two) with
// the row scales, the value weights exp(mu_C - mu_t) [64], the row factors
// exp(G_C) and exp(G_C - mu_C) [128 each], and mu_C, exp(mu_C).
constexpr int KREC_KB = 0;
constexpr int KREC_KD = KREC_KB + 64 * 128 * 2;
constexpr int KREC_X = KREC_KD + 128 * 64 * 2;
constexpr int KREC_XS = KREC_X + 64 * 64 * 2;
constexpr int KREC_VF = KREC_XS + 64 * 4;
constexpr int KREC_RS = KREC_VF + 64 * 4;
constexpr int KREC_RU = KREC_RS + 128 * 4;
constexpr int KREC_M = KREC_RU + 128 * 4;
constexpr int KREC_BYTES = KREC_M + 16;
// the delta state pass in its KDA mode (build_delta2.hip), over the records of a factor pass
hipError_t launch_kda_state(const BuildArgs& a, const ChunkTable& ct, const void* ws, hipStream_t stream);
// seam step of the KDA family (seam_kda.hip): no workspace
hipError_t launch_seam_kda(int d, bool in_f32, const SeamArgs& a, hipStream_t stream);
// rotary re-rotation of n_seg x n_chain pairs in place (rerotate.hip): S <- R S,
// and U <- R U R^T when U is not NULL; pos: device [n_seg].
hipError_t launch_rerotate(int d, float* S, float* U, const int32_t* pos, int n_seg, int n_chain, double base,
                           hipStream_t stream);

}  // namespace hypic
