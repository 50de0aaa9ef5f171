// hypic_api.cpp -- the C ABI of include/hypic.h: host-side validation and
// dispatch to the gfx950 kernels.  Every argument check runs before any HIP
// call, so malformed calls are rejected without touching the device.
#include "../../include/hypic.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <numeric>
#include <string>
#include <vector>

#include "launch.h"

namespace {

thread_local std::string g_err;

hypic_status fail(hypic_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

hypic_status ok() {
  g_err.clear();
  return HYPIC_OK;
}

hypic_status hip_fail(hipError_t e, const char* what) {
  return fail(HYPIC_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

struct Range {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlaps(const Range& a, const Range& b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

// outputs must not overlap inputs or each other
hypic_status check_overlaps(const std::vector<Range>& ins, const std::vector<Range>& outs) {
  for (size_t i = 0; i < outs.size(); ++i) {
    for (const Range& r : ins)
      if (overlaps(outs[i], r)) return fail(HYPIC_E_INVALID, "output %s overlaps input %s", outs[i].name, r.name);
    for (size_t j = i + 1; j < outs.size(); ++j)
      if (overlaps(outs[i], outs[j]))
        return fail(HYPIC_E_INVALID, "outputs %s and %s overlap", outs[i].name, outs[j].name);
  }
  return HYPIC_OK;
}

hypic_status check_aligned(const void* p, const char* name) {
  if (((uintptr_t)p) & 15u) return fail(HYPIC_E_INVALID, "%s is not 16-byte aligned", name);
  return HYPIC_OK;
}

#define TRY(x)                           \
  do {                                   \
    hypic_status _st = (x);              \
    if (_st != HYPIC_OK) return _st;     \
  } while (0)

hypic_status check_common(int fam, int n_seg, int n_chain, int d_k, int d_v) {
  if (fam < HYPIC_NAIVE || fam > HYPIC_KDA) return fail(HYPIC_E_INVALID, "unknown family %d", fam);
  if (n_seg < 1) return fail(HYPIC_E_INVALID, "n_seg must be >= 1 (got %d)", n_seg);
  if (n_chain < 1) return fail(HYPIC_E_INVALID, "n_chain must be >= 1 (got %d)", n_chain);
  if (d_k < 1 || d_v < 1) return fail(HYPIC_E_INVALID, "d_k and d_v must be >= 1");
  if (d_k != d_v || (d_k != 64 && d_k != 128))
    return fail(HYPIC_E_UNSUPPORTED, "only d_k = d_v in {64, 128} is built (got %d, %d)", d_k, d_v);
  return HYPIC_OK;
}

size_t gate_len(int fam, int d) { return fam == HYPIC_DIAG ? (size_t)d : 1; }

// Families whose transition is a dense exp(g) U (pairs carry U).
bool dense(int fam) { return fam == HYPIC_DELTA || fam == HYPIC_KDA; }

// Validates the token inputs of a build or seam call and returns their byte ranges.
hypic_status check_tokens(int fam, const hypic_tokens* t, size_t n_tok, int n_chain, int d, bool need_q,
                          std::vector<Range>* ranges) {
  if (!t) return fail(HYPIC_E_INVALID, "token struct is NULL");
  if (t->dtype != HYPIC_F32 && t->dtype != HYPIC_BF16) return fail(HYPIC_E_INVALID, "unknown dtype %d", (int)t->dtype);
  const size_t es = t->dtype == HYPIC_F32 ? 4 : 2;
  const size_t rows = n_tok * (size_t)n_chain;
  if (!t->k) return fail(HYPIC_E_INVALID, "k is NULL");
  if (!t->v) return fail(HYPIC_E_INVALID, "v is NULL");
  if (need_q && !t->q) return fail(HYPIC_E_INVALID, "q is NULL");
  if (dense(fam)) {
    if (!t->beta) return fail(HYPIC_E_INVALID, "beta is required for the delta and KDA families");
  } else if (t->beta) {
    return fail(HYPIC_E_INVALID, "beta is only defined for the delta and KDA families");
  }
  if (fam == HYPIC_SCALAR || fam == HYPIC_DIAG || fam == HYPIC_KDA) {
    if (!t->log_gate) return fail(HYPIC_E_INVALID, "log_gate is required for this family");
  }
  if (fam == HYPIC_NAIVE && t->log_gate) return fail(HYPIC_E_INVALID, "log_gate must be NULL for the naive family");
  if (t->gate_per_chain && fam != HYPIC_SCALAR)
    return fail(HYPIC_E_INVALID, "gate_per_chain is only defined for the scalar family");
  TRY(check_aligned(t->k, "k"));
  TRY(check_aligned(t->v, "v"));
  if (need_q) TRY(check_aligned(t->q, "q"));
  if (t->beta) TRY(check_aligned(t->beta, "beta"));
  if (t->log_gate) TRY(check_aligned(t->log_gate, "log_gate"));
  ranges->push_back({t->k, rows * d * es, "k"});
  ranges->push_back({t->v, rows * d * es, "v"});
  if (need_q) ranges->push_back({t->q, rows * d * es, "q"});
  if (t->beta) ranges->push_back({t->beta, rows * es, "beta"});
  if (t->log_gate) {
    size_t bytes;
    if (fam == HYPIC_SCALAR && t->gate_per_chain)
      bytes = (size_t)n_chain * 4;
    else if (fam == HYPIC_DIAG || fam == HYPIC_KDA)
      bytes = rows * d * es;
    else
      bytes = rows * es;
    ranges->push_back({t->log_gate, bytes, "log_gate"});
  }
  return HYPIC_OK;
}

hypic_status check_cpairs(int fam, const hypic_cpairs* p, int n_seg, int n_chain, int d, const char* what,
                          std::vector<Range>* ranges) {
  const size_t units = (size_t)n_seg * n_chain;
  if (!p->S) return fail(HYPIC_E_INVALID, "%s.S is NULL", what);
  if (fam != HYPIC_NAIVE && !p->g) return fail(HYPIC_E_INVALID, "%s.g is NULL", what);
  if (dense(fam) && !p->U) return fail(HYPIC_E_INVALID, "%s.U is required for the delta and KDA families", what);
  if (!dense(fam) && p->U) return fail(HYPIC_E_INVALID, "%s.U is only defined for the delta and KDA families", what);
  TRY(check_aligned(p->S, "pairs.S"));
  if (p->g) TRY(check_aligned(p->g, "pairs.g"));
  if (p->U) TRY(check_aligned(p->U, "pairs.U"));
  ranges->push_back({p->S, units * d * d * 4, "pairs.S"});
  if (p->g) ranges->push_back({p->g, units * gate_len(fam, d) * 4, "pairs.g"});
  if (p->U) ranges->push_back({p->U, units * d * d * 4, "pairs.U"});
  return HYPIC_OK;
}

hypic_status check_offsets(int n_seg, const int32_t* seg_offsets) {
  if (!seg_offsets) return fail(HYPIC_E_INVALID, "seg_offsets is NULL");
  if (seg_offsets[0] != 0) return fail(HYPIC_E_INVALID, "seg_offsets[0] must be 0 (got %d)", seg_offsets[0]);
  for (int s = 0; s < n_seg; ++s)
    if (seg_offsets[s + 1] <= seg_offsets[s])
      return fail(HYPIC_E_INVALID, "seg_offsets must strictly increase (segment %d is empty or negative)", s);
  return HYPIC_OK;
}

// Launch plan of the build of segments [s0, s1) (segment s spans tokens
// [off[s], off[s + 1]); its output row is s) [youleyou, segment-parallelism
// paragraph: LPT scheduling of uneven segments]: the segments sorted by length,
// longest first (ties by index), and cut into launches of kMaxSegPerLaunch
// consecutive entries of that order.  The longest segments of the whole range
// start first, in the first launch, and the shortest end the last one.
std::vector<hypic::SegTable> plan_launches(const int32_t* off, int s0, int s1) {
  const int n = s1 - s0;
  std::vector<int> idx(n);
  std::iota(idx.begin(), idx.end(), s0);
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int x, int y) { return off[x + 1] - off[x] > off[y + 1] - off[y]; });
  constexpr int K = hypic::kMaxSegPerLaunch;
  std::vector<hypic::SegTable> plan((n + K - 1) / K);
  for (size_t l = 0; l < plan.size(); ++l) {
    hypic::SegTable& t = plan[l];
    const int q0 = (int)l * K, ns = std::min(K, n - q0);
    const int first = idx[q0], len0 = off[first + 1] - off[first];
    bool contiguous = true;
    for (int i = 0; i < ns; ++i) {
      const int sg = idx[q0 + i];
      t.beg[i] = off[sg];
      t.end[i] = off[sg + 1];
      t.out[i] = sg;
      contiguous = contiguous && sg == first + i && t.end[i] - t.beg[i] == len0;
    }
    t.n_seg = ns;
    t.contiguous = contiguous ? 1 : 0;
  }
  return plan;
}

// Workspace of a delta build: the largest any of its launches needs (launches
// run in stream order and reuse it).
size_t delta_workspace(int n_seg, const int32_t* seg_offsets, int n_chain, int d, bool f32) {
  size_t need = 0;
  for (const hypic::SegTable& t : plan_launches(seg_offsets, 0, n_seg))
    need = std::max(need, hypic::build_delta_workspace(d, f32, t, n_chain));
  return need;
}

// The same for the KDA build's factor records.
size_t kda_workspace(int n_seg, const int32_t* seg_offsets, int n_chain, int d, bool f32) {
  size_t need = 0;
  for (const hypic::SegTable& t : plan_launches(seg_offsets, 0, n_seg))
    need = std::max(need, hypic::kda_workspace_bytes(d, f32, t, n_chain));
  return need;
}

// Piece split of a naive / scalar / diagonal build with few units: each
// segment is cut into P pieces of whole 64-token chunks, built concurrently,
// and the pieces of every segment are joined by the composition law (the same
// law that joins segments) -- so few long segments still occupy the GPU.
// Returns P (1: no split).
int piece_count(int fam, int n_seg, const int32_t* seg_offsets, int n_chain) {
  if (dense(fam)) return 1;
  const long units = (long)n_seg * n_chain;
  int p = (int)std::min<long>(4, 512 / std::max<long>(units, 1));
  for (int s = 0; s < n_seg && p > 1; ++s) p = std::min(p, (seg_offsets[s + 1] - seg_offsets[s] + 63) / 64);
  return p >= 2 ? p : 1;
}

// Pieces: (g, S) of every (segment, piece, chain), then nothing else.
size_t piece_bytes(int fam, int n_seg, int P, int n_chain, int d) {
  const size_t pairs = (size_t)n_seg * P * n_chain;
  const size_t gbytes = pairs * gate_len(fam, d) * 4;
  return ((gbytes + 255) & ~(size_t)255) + pairs * d * d * 4;
}

size_t build_workspace(int fam, int n_seg, const int32_t* seg_offsets, int n_chain, int d, bool f32) {
  if (fam == HYPIC_DELTA) return delta_workspace(n_seg, seg_offsets, n_chain, d, f32);
  if (fam == HYPIC_KDA) return kda_workspace(n_seg, seg_offsets, n_chain, d, f32);
  const int P = piece_count(fam, n_seg, seg_offsets, n_chain);
  return P > 1 ? piece_bytes(fam, n_seg, P, n_chain, d) : 0;
}

// Launches the build of segments [s0, s1) of a validated batch (global segment
// indices; outputs at their places in `out`), over a workspace of at least
// build_workspace() bytes for those segments.
hypic_status build_range(int fam, int n_seg, const int32_t* seg_offsets, int s0, int s1, int n_chain, int d,
                         bool f32, const hypic_tokens* in, const hypic_pairs* out, void* workspace,
                         hipStream_t stream, const hypic::FuseArgs* fuse = nullptr) {
  (void)n_seg;
  hypic::BuildArgs a;
  if (fuse) a.fuse = *fuse;
  a.k = in->k;
  a.v = in->v;
  a.beta = in->beta;
  a.lg = in->log_gate;
  a.g = out->g;
  a.U = out->U;
  a.S = out->S;
  a.n_chain = n_chain;
  a.gate_per_chain = in->gate_per_chain ? 1 : 0;
  const int ns_all = s1 - s0;
  const int32_t* offs = seg_offsets + s0;  // offsets of the range (absolute token positions)
  const int P = piece_count(fam, ns_all, offs, n_chain);
  if (P > 1) {
    // build the pieces into the workspace, then compose each segment's pieces
    std::vector<int32_t> poff((size_t)ns_all * P + 1);
    for (int s = 0; s < ns_all; ++s) {
      const int nc = (offs[s + 1] - offs[s] + 63) / 64;
      for (int p = 0; p < P; ++p) poff[(size_t)s * P + p] = offs[s] + 64 * (int)((long)p * nc / P);
    }
    poff[(size_t)ns_all * P] = offs[ns_all];
    const size_t n_pairs = (size_t)ns_all * P * n_chain;
    float* pg = reinterpret_cast<float*>(workspace);
    float* pS = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(workspace) +
                                         ((n_pairs * gate_len(fam, d) * 4 + 255) & ~(size_t)255));
    a.g = pg;
    a.S = pS;
    for (const hypic::SegTable& t : plan_launches(poff.data(), 0, ns_all * P)) {
      a.seg = t;
      hipError_t e = hypic::launch_build_sd(fam, d, f32, a, t.n_seg * n_chain, stream);
      if (e != hipSuccess) return hip_fail(e, "hypic_seg_build launch");
    }
    hypic::ComposeArgs c{};
    c.g = pg;
    c.S = pS;
    c.S_out = out->S + (size_t)s0 * n_chain * d * d;
    c.g_tot = out->g + (size_t)s0 * n_chain * gate_len(fam, d);
    c.n_seg = P;
    c.n_chain = n_chain;
    c.n_out = ns_all * n_chain;
    hipError_t e = hypic::launch_compose_elem(fam, d, c, stream);
    if (e != hipSuccess) return hip_fail(e, "hypic_seg_build piece composition launch");
    return HYPIC_OK;
  }
  for (const hypic::SegTable& t : plan_launches(seg_offsets, s0, s1)) {
    a.seg = t;
    const int blocks = t.n_seg * n_chain;
    hipError_t e = (fam == HYPIC_DELTA) ? hypic::launch_build_delta(d, f32, a, blocks, workspace, stream)
                   : (fam == HYPIC_KDA) ? hypic::launch_build_kda(d, f32, a, blocks, workspace, stream)
                                        : hypic::launch_build_sd(fam, d, f32, a, blocks, stream);
    if (e != hipSuccess) return hip_fail(e, "hypic_seg_build launch");
  }
  return HYPIC_OK;
}

// ---- the cold request in one call: groups of segments built on the caller's
// stream, each group composed on a second stream while the next is built ------

// Segments per group: enough (segment, chain) units to fill the GPU once
// (two workgroups per CU of 256), at most kMaxGroups groups.
constexpr int kMaxGroups = 32;
#ifndef HYPIC_GROUP_UNITS
#define HYPIC_GROUP_UNITS 512
#endif
int group_len(int n_seg, int n_chain) {
  int len = std::max(1, (HYPIC_GROUP_UNITS + n_chain - 1) / n_chain);
  if ((n_seg + len - 1) / len > kMaxGroups) len = (n_seg + kMaxGroups - 1) / kMaxGroups;
  return len;
}

struct FusedLayout {
  int glen, n_grp;
  size_t build_ws, g_off, U_off, S_off, total;
  bool fused = false;  // fused schedule: counters at cnt_off, node pairs at g_off, U_off, S_off
  int P = 0;
  size_t cnt_off = 0;
};

// The fused schedule applies to the delta build's two-kernel path (d = 128, bf16
// tokens, segments of at most kDelta2MaxSegLen tokens), at least two segments
// and no start state; elsewhere the call runs the sequential schedule.
bool fused_applies(int fam, int n_seg, const int32_t* seg_offsets, int d, bool f32) {
  if (fam != HYPIC_DELTA || d != 128 || f32 || n_seg < 2) return false;
  for (int s = 0; s < n_seg; ++s)
    if (seg_offsets[s + 1] - seg_offsets[s] > hypic::kDelta2MaxSegLen) return false;
  return true;
}

// Sequential mode: one group (the whole batch), and the blocked composition's
// workspace after the build's.  Pipelined mode: groups, each group's pair.
FusedLayout fused_layout(int fam, int n_seg, const int32_t* seg_offsets, int n_chain, int d, bool f32, int mode,
                         bool has_init) {
  FusedLayout L;
  if (mode == HYPIC_BC_FUSED && !has_init && fused_applies(fam, n_seg, seg_offsets, d, f32)) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    L.fused = true;
    L.glen = n_seg;
    L.n_grp = 1;
    L.P = 1;
    while (L.P < n_seg) L.P *= 2;
    const size_t nodes = (size_t)L.P * n_chain;
    L.build_ws = build_workspace(fam, n_seg, seg_offsets, n_chain, d, f32);
    L.cnt_off = up(L.build_ws);
    L.g_off = L.cnt_off + up(nodes * 4);
    L.U_off = L.g_off + up(nodes * 4);
    L.S_off = L.U_off + nodes * d * d * 4;
    L.total = L.S_off + nodes * d * d * 4;
    return L;
  }
  if (mode != HYPIC_BC_PIPELINED) {
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    L.glen = n_seg;
    L.n_grp = 1;
    L.build_ws = build_workspace(fam, n_seg, seg_offsets, n_chain, d, f32);
    L.g_off = L.U_off = L.S_off = up(L.build_ws);
    L.total = L.g_off + (dense(fam) ? hypic::compose_workspace_bytes(d, n_seg, n_chain, false) : 0);
    return L;
  }
  L.glen = group_len(n_seg, n_chain);
  L.n_grp = (n_seg + L.glen - 1) / L.glen;
  L.build_ws = 0;
  for (int s0 = 0; s0 < n_seg; s0 += L.glen) {
    const int ns = std::min(L.glen, n_seg - s0);
    L.build_ws = std::max(L.build_ws, build_workspace(fam, ns, seg_offsets + s0, n_chain, d, f32));
  }
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t units = (size_t)L.n_grp * n_chain;
  L.g_off = up(L.build_ws);
  L.U_off = L.g_off + up(units * gate_len(fam, d) * 4);
  L.S_off = L.U_off + (dense(fam) ? up(units * d * d * 4) : 0);
  L.total = L.S_off + units * d * d * 4;
  return L;
}

// The second stream and the events of the calling host thread on the current
// device, created on first use and kept (default priority, non-blocking).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t ev[kMaxGroups + 1] = {};
};
hipError_t side_stream(SideStream** out) {
  static thread_local SideStream per_dev[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  SideStream& ss = per_dev[dev];
  if (!ss.s) {
    e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking);
    if (e != hipSuccess) return e;
    for (auto& ev : ss.ev) {
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e != hipSuccess) return e;
    }
  }
  *out = &ss;
  return hipSuccess;
}

// Ordered composition of n pairs per chain (flat single pass, no workspace).
hipError_t compose_range(int fam, int d, const float* g, const float* U, const float* S, int n, int n_chain,
                         const float* S_init, float* S_out, float* g_tot, float* U_tot, hipStream_t st) {
  hypic::ComposeArgs c{};
  c.g = g;
  c.U = U;
  c.S = S;
  c.S_init = S_init;
  c.S_out = S_out;
  c.g_tot = g_tot;
  c.U_tot = U_tot;
  c.n_seg = n;
  c.n_chain = n_chain;
  c.n_out = n_chain;
  return dense(fam) ? hypic::launch_compose_chain(d, c, nullptr, 0, st) : hypic::launch_compose_elem(fam, d, c, st);
}

}  // namespace

hypic_status hypic::report_error(hypic_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

extern "C" {

const char* hypic_last_error(void) { return g_err.c_str(); }

int hypic_abi_version(void) { return HYPIC_ABI_VERSION; }

hypic_status hypic_seg_build_workspace_size(hypic_family fam, int n_seg, const int32_t* seg_offsets, int n_chain,
                                            int d_k, int d_v, hypic_dtype dtype, size_t* bytes) {
  TRY(check_common(fam, n_seg, n_chain, d_k, d_v));
  TRY(check_offsets(n_seg, seg_offsets));
  if (dtype != HYPIC_F32 && dtype != HYPIC_BF16) return fail(HYPIC_E_INVALID, "unknown dtype %d", (int)dtype);
  if (!bytes) return fail(HYPIC_E_INVALID, "bytes is NULL");
  *bytes = build_workspace(fam, n_seg, seg_offsets, n_chain, d_k, dtype == HYPIC_F32);
  return ok();
}

hypic_status hypic_seg_build(hypic_family fam, int n_seg, const int32_t* seg_offsets, int n_chain, int d_k,
                             int d_v, const hypic_tokens* in, const hypic_pairs* out, void* workspace,
                             size_t workspace_bytes, void* stream) {
  TRY(check_common(fam, n_seg, n_chain, d_k, d_v));
  const int d = d_k;
  TRY(check_offsets(n_seg, seg_offsets));
  const size_t n_tok = (size_t)seg_offsets[n_seg];
  std::vector<Range> ins, outs;
  TRY(check_tokens(fam, in, n_tok, n_chain, d, false, &ins));
  if (!out) return fail(HYPIC_E_INVALID, "out is NULL");
  if (!out->S) return fail(HYPIC_E_INVALID, "out.S is NULL");
  if (!out->g) return fail(HYPIC_E_INVALID, "out.g is NULL");
  if (dense(fam) && !out->U) return fail(HYPIC_E_INVALID, "out.U is required for the delta and KDA families");
  if (!dense(fam) && out->U) return fail(HYPIC_E_INVALID, "out.U is only defined for the delta and KDA families");
  TRY(check_aligned(out->S, "out.S"));
  TRY(check_aligned(out->g, "out.g"));
  if (out->U) TRY(check_aligned(out->U, "out.U"));
  const size_t units = (size_t)n_seg * n_chain;
  outs.push_back({out->S, units * d * d * 4, "out.S"});
  outs.push_back({out->g, units * gate_len(fam, d) * 4, "out.g"});
  if (out->U) outs.push_back({out->U, units * d * d * 4, "out.U"});
  const bool f32 = in->dtype == HYPIC_F32;
  if (fam == HYPIC_KDA && !hypic::kda_build_supported(d, f32))
    return fail(HYPIC_E_UNSUPPORTED, "the KDA build is built for d = 64 and for d = 128 with bf16 tokens");
  const size_t ws_need = build_workspace(fam, n_seg, seg_offsets, n_chain, d, f32);
  if (ws_need > 0) {
    if (!workspace) return fail(HYPIC_E_INVALID, "workspace is NULL (%zu bytes required)", ws_need);
    if (workspace_bytes < ws_need)
      return fail(HYPIC_E_INVALID, "workspace too small: %zu bytes given, %zu required", workspace_bytes, ws_need);
    TRY(check_aligned(workspace, "workspace"));
    outs.push_back({workspace, ws_need, "workspace"});
  }
  TRY(check_overlaps(ins, outs));

  hypic_status st = build_range(fam, n_seg, seg_offsets, 0, n_seg, n_chain, d, f32, in, out, workspace,
                                (hipStream_t)stream);
  if (st != HYPIC_OK) return st;
  return ok();
}

hypic_status hypic_seg_build_compose_workspace_size(hypic_family fam, int n_seg, const int32_t* seg_offsets,
                                                    int n_chain, int d_k, int d_v, hypic_dtype dtype, int mode,
                                                    size_t* bytes) {
  TRY(check_common(fam, n_seg, n_chain, d_k, d_v));
  TRY(check_offsets(n_seg, seg_offsets));
  if (dtype != HYPIC_F32 && dtype != HYPIC_BF16) return fail(HYPIC_E_INVALID, "unknown dtype %d", (int)dtype);
  if (!bytes) return fail(HYPIC_E_INVALID, "bytes is NULL");
  if (mode != HYPIC_BC_SEQUENTIAL && mode != HYPIC_BC_PIPELINED && mode != HYPIC_BC_FUSED)
    return fail(HYPIC_E_INVALID, "unknown mode %d", mode);
  // (fused: enough also for the sequential schedule it runs when given a start state)
  const bool f32 = dtype == HYPIC_F32;
  *bytes = std::max(fused_layout(fam, n_seg, seg_offsets, n_chain, d_k, f32, mode, false).total,
                    fused_layout(fam, n_seg, seg_offsets, n_chain, d_k, f32, mode, true).total);
  return ok();
}

hypic_status hypic_seg_build_compose(hypic_family fam, int n_seg, const int32_t* seg_offsets, int n_chain, int d_k,
                                     int d_v, const hypic_tokens* in, const hypic_pairs* out, const float* S_init,
                                     float* S_out, float* g_total, float* U_total, int mode, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  TRY(check_common(fam, n_seg, n_chain, d_k, d_v));
  if (mode != HYPIC_BC_SEQUENTIAL && mode != HYPIC_BC_PIPELINED && mode != HYPIC_BC_FUSED)
    return fail(HYPIC_E_INVALID, "unknown mode %d", mode);
  const int d = d_k;
  TRY(check_offsets(n_seg, seg_offsets));
  const size_t n_tok = (size_t)seg_offsets[n_seg];
  std::vector<Range> ins, outs;
  TRY(check_tokens(fam, in, n_tok, n_chain, d, false, &ins));
  if (!out) return fail(HYPIC_E_INVALID, "out is NULL");
  if (!out->S) return fail(HYPIC_E_INVALID, "out.S is NULL");
  if (!out->g) return fail(HYPIC_E_INVALID, "out.g is NULL");
  if (dense(fam) && !out->U) return fail(HYPIC_E_INVALID, "out.U is required for the delta and KDA families");
  if (!dense(fam) && out->U) return fail(HYPIC_E_INVALID, "out.U is only defined for the delta and KDA families");
  if (!S_out) return fail(HYPIC_E_INVALID, "S_out is NULL");
  if (U_total && !dense(fam)) return fail(HYPIC_E_INVALID, "U_total is only defined for the delta and KDA families");
  TRY(check_aligned(out->S, "out.S"));
  TRY(check_aligned(out->g, "out.g"));
  if (out->U) TRY(check_aligned(out->U, "out.U"));
  TRY(check_aligned(S_out, "S_out"));
  if (S_init) TRY(check_aligned(S_init, "S_init"));
  if (g_total) TRY(check_aligned(g_total, "g_total"));
  if (U_total) TRY(check_aligned(U_total, "U_total"));
  const bool f32 = in->dtype == HYPIC_F32;
  if (fam == HYPIC_KDA && !hypic::kda_build_supported(d, f32))
    return fail(HYPIC_E_UNSUPPORTED, "the KDA build is built for d = 64 and for d = 128 with bf16 tokens");
  const size_t units = (size_t)n_seg * n_chain;
  const size_t sbytes = (size_t)n_chain * d * d * 4;
  outs.push_back({out->S, units * d * d * 4, "out.S"});
  outs.push_back({out->g, units * gate_len(fam, d) * 4, "out.g"});
  if (out->U) outs.push_back({out->U, units * d * d * 4, "out.U"});
  if (S_init && S_init != S_out) ins.push_back({S_init, sbytes, "S_init"});
  outs.push_back({S_out, sbytes, "S_out"});
  if (g_total) outs.push_back({g_total, (size_t)n_chain * gate_len(fam, d) * 4, "g_total"});
  if (U_total) outs.push_back({U_total, sbytes, "U_total"});
  const FusedLayout L = fused_layout(fam, n_seg, seg_offsets, n_chain, d, f32, mode, S_init != nullptr);
  if (L.total > 0 && !workspace) return fail(HYPIC_E_INVALID, "workspace is NULL (%zu bytes required)", L.total);
  if (workspace_bytes < L.total)
    return fail(HYPIC_E_INVALID, "workspace too small: %zu bytes given, %zu required", workspace_bytes, L.total);
  if (L.total > 0) {
    TRY(check_aligned(workspace, "workspace"));
    outs.push_back({workspace, L.total, "workspace"});
  }
  TRY(check_overlaps(ins, outs));

  hipStream_t sa = (hipStream_t)stream;
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  float* gg = reinterpret_cast<float*>(ws + L.g_off);
  float* gU = dense(fam) ? reinterpret_cast<float*>(ws + L.U_off) : nullptr;
  float* gS = reinterpret_cast<float*>(ws + L.S_off);
  const size_t gl = gate_len(fam, d);
  if (L.fused) {  // the build with the composition folded into its state pass
    hypic::FuseArgs f;
    f.cnt = reinterpret_cast<int*>(ws + L.cnt_off);
    f.g = gg;
    f.U = gU;
    f.S = gS;
    f.S_out = S_out;
    f.g_tot = g_total;
    f.U_tot = U_total;
    f.P = L.P;
    f.n_seg = n_seg;
    hipError_t e = hypic::launch_zero_ints(f.cnt, (size_t)L.P * n_chain, sa);
    if (e != hipSuccess) return hip_fail(e, "hypic_seg_build_compose counter reset");
    TRY(build_range(fam, n_seg, seg_offsets, 0, n_seg, n_chain, d, f32, in, out, workspace, sa, &f));
    return ok();
  }
  if (L.n_grp == 1) {  // build, then compose (blocked schedule when it applies), on the caller's stream
    TRY(build_range(fam, n_seg, seg_offsets, 0, n_seg, n_chain, d, f32, in, out, workspace, sa));
    hypic::ComposeArgs c{};
    c.g = out->g;
    c.U = out->U;
    c.S = out->S;
    c.S_init = S_init;
    c.S_out = S_out;
    c.g_tot = g_total;
    c.U_tot = U_total;
    c.n_seg = n_seg;
    c.n_chain = n_chain;
    c.n_out = n_chain;
    const size_t cws = mode == HYPIC_BC_SEQUENTIAL ? L.total - L.g_off : 0;
    hipError_t e = dense(fam) ? hypic::launch_compose_chain(d, c, cws ? ws + L.g_off : nullptr, cws, sa)
                              : hypic::launch_compose_elem(fam, d, c, sa);
    if (e != hipSuccess) return hip_fail(e, "hypic_seg_build_compose composition launch");
    return ok();
  }
  SideStream* side = nullptr;
  hipError_t e = side_stream(&side);
  if (e != hipSuccess) return hip_fail(e, "hypic_seg_build_compose second stream");
  for (int gi = 0; gi < L.n_grp; ++gi) {
    const int s0 = gi * L.glen, s1 = std::min(n_seg, s0 + L.glen);
    // group gi built on the caller's stream (in stream order after group gi - 1)
    TRY(build_range(fam, n_seg, seg_offsets, s0, s1, n_chain, d, f32, in, out, workspace, sa));
    e = hipEventRecord(side->ev[gi], sa);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->ev[gi], 0);
    if (e != hipSuccess) return hip_fail(e, "hypic_seg_build_compose event");
    // ... and composed into one pair per chain on the second stream, while the
    // caller's stream builds the next group
    const size_t p0 = (size_t)s0 * n_chain;
    e = compose_range(fam, d, out->g + p0 * gl, out->U ? out->U + p0 * d * d : nullptr, out->S + p0 * d * d,
                      s1 - s0, n_chain, nullptr, gS + (size_t)gi * n_chain * d * d, gg + (size_t)gi * n_chain * gl,
                      gU ? gU + (size_t)gi * n_chain * d * d : nullptr, side->s);
    if (e != hipSuccess) return hip_fail(e, "hypic_seg_build_compose group composition launch");
  }
  // join: the group pairs composed in order on the caller's stream
  e = hipEventRecord(side->ev[kMaxGroups], side->s);
  if (e == hipSuccess) e = hipStreamWaitEvent(sa, side->ev[kMaxGroups], 0);
  if (e != hipSuccess) return hip_fail(e, "hypic_seg_build_compose event");
  e = compose_range(fam, d, gg, gU, gS, L.n_grp, n_chain, S_init, S_out, g_total, U_total, sa);
  if (e != hipSuccess) return hip_fail(e, "hypic_seg_build_compose final composition launch");
  return ok();
}

hypic_status hypic_compose_workspace_size(hypic_family fam, int n_seg, int n_chain, int d_k, int d_v,
                                          int want_prefix, size_t* bytes) {
  TRY(check_common(fam, n_seg, n_chain, d_k, d_v));
  if (!bytes) return fail(HYPIC_E_INVALID, "bytes is NULL");
  *bytes = dense(fam) ? hypic::compose_workspace_bytes(d_k, n_seg, n_chain, want_prefix != 0) : 0;
  return ok();
}

hypic_status hypic_compose(hypic_family fam, int n_seg, int n_chain, int d_k, int d_v, const hypic_cpairs* in,
                           const float* S_init, float* S_out, float* prefix_states, float* g_total,
                           float* U_total, void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_common(fam, n_seg, n_chain, d_k, d_v));
  const int d = d_k;
  if (!in) return fail(HYPIC_E_INVALID, "in is NULL");
  std::vector<Range> ins, outs;
  TRY(check_cpairs(fam, in, n_seg, n_chain, d, "in", &ins));
  if (!S_out) return fail(HYPIC_E_INVALID, "S_out is NULL");
  if (U_total && !dense(fam))
    return fail(HYPIC_E_INVALID, "U_total is only defined for the delta and KDA families");
  TRY(check_aligned(S_out, "S_out"));
  if (S_init) TRY(check_aligned(S_init, "S_init"));
  if (prefix_states) TRY(check_aligned(prefix_states, "prefix_states"));
  if (g_total) TRY(check_aligned(g_total, "g_total"));
  if (U_total) TRY(check_aligned(U_total, "U_total"));
  const size_t sbytes = (size_t)n_chain * d * d * 4;
  // S_out may be exactly S_init (in-place); any other overlap is rejected
  if (S_init && S_init != S_out) ins.push_back({S_init, sbytes, "S_init"});
  outs.push_back({S_out, sbytes, "S_out"});
  if (prefix_states) outs.push_back({prefix_states, (size_t)n_seg * sbytes, "prefix_states"});
  if (g_total) outs.push_back({g_total, (size_t)n_chain * gate_len(fam, d) * 4, "g_total"});
  if (U_total) outs.push_back({U_total, (size_t)n_chain * d * d * 4, "U_total"});
  // (an in-place S_init is covered as S_out: it may overlap nothing else)
  const size_t ws_need =
      dense(fam) ? hypic::compose_workspace_bytes(d, n_seg, n_chain, prefix_states != nullptr) : 0;
  if (workspace && ws_need > 0) {
    if (workspace_bytes < ws_need)
      return fail(HYPIC_E_INVALID, "workspace too small: %zu bytes given, %zu required", workspace_bytes, ws_need);
    TRY(check_aligned(workspace, "workspace"));
    outs.push_back({workspace, ws_need, "workspace"});
  }
  TRY(check_overlaps(ins, outs));

  hypic::ComposeArgs a;
  a.g = in->g;
  a.U = in->U;
  a.S = in->S;
  a.S_init = S_init;
  a.S_out = S_out;
  a.prefix = prefix_states;
  a.g_tot = g_total;
  a.U_tot = U_total;
  a.n_seg = n_seg;
  a.n_chain = n_chain;
  a.n_out = n_chain;
  hipError_t e = dense(fam)
                     ? hypic::launch_compose_chain(d, a, ws_need > 0 ? workspace : nullptr, workspace_bytes,
                                                   (hipStream_t)stream)
                                      : hypic::launch_compose_elem(fam, d, a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hypic_compose launch");
  return ok();
}

hypic_status hypic_seam_step_workspace_size(hypic_family fam, int n_seg, int w, int n_chain, int d_k, int d_v,
                                            size_t* bytes) {
  TRY(check_common(fam, n_seg, n_chain, d_k, d_v));
  if (w < 1) return fail(HYPIC_E_INVALID, "w must be >= 1 (got %d)", w);
  if (!bytes) return fail(HYPIC_E_INVALID, "bytes is NULL");
  *bytes = fam == HYPIC_DELTA ? hypic::seam_workspace_bytes(n_seg, w, n_chain) : 0;
  return ok();
}

hypic_status hypic_seam_step(hypic_family fam, int n_seg, int w, int n_chain, int d_k, int d_v,
                             const hypic_tokens* seam, const hypic_cpairs* body, float* S_run, float* o_out,
                             const hypic_pairs* window_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  TRY(check_common(fam, n_seg, n_chain, d_k, d_v));
  const int d = d_k;
  if (w < 1) return fail(HYPIC_E_INVALID, "w must be >= 1 (got %d)", w);
  std::vector<Range> ins, outs;
  const size_t n_tok = (size_t)n_seg * w;
  TRY(check_tokens(fam, seam, n_tok, n_chain, d, true, &ins));
  if (body) TRY(check_cpairs(fam, body, n_seg, n_chain, d, "body", &ins));
  if (!S_run) return fail(HYPIC_E_INVALID, "S_run is NULL");
  if (!o_out) return fail(HYPIC_E_INVALID, "o_out is NULL");
  TRY(check_aligned(S_run, "S_run"));
  TRY(check_aligned(o_out, "o_out"));
  outs.push_back({S_run, (size_t)n_chain * d * d * 4, "S_run"});
  outs.push_back({o_out, n_tok * n_chain * d * 4, "o_out"});
  if (window_out) {
    if (!window_out->S || !window_out->g) return fail(HYPIC_E_INVALID, "window_out needs S and g");
    if (dense(fam) && !window_out->U)
      return fail(HYPIC_E_INVALID, "window_out.U is required for the delta and KDA families");
    if (!dense(fam) && window_out->U)
      return fail(HYPIC_E_INVALID, "window_out.U is only defined for the delta and KDA families");
    if (fam == HYPIC_KDA && !hypic::kda_build_supported(d, seam->dtype == HYPIC_F32))
      return fail(HYPIC_E_UNSUPPORTED, "KDA window pairs are built for d = 64 and for d = 128 with bf16 tokens");
    TRY(check_aligned(window_out->S, "window_out.S"));
    if (window_out->g) TRY(check_aligned(window_out->g, "window_out.g"));
    if (window_out->U) TRY(check_aligned(window_out->U, "window_out.U"));
    const size_t units = (size_t)n_seg * n_chain;
    outs.push_back({window_out->S, units * d * d * 4, "window_out.S"});
    if (window_out->g) outs.push_back({window_out->g, units * gate_len(fam, d) * 4, "window_out.g"});
    if (window_out->U) outs.push_back({window_out->U, units * d * d * 4, "window_out.U"});
  }
  const size_t ws_need = fam == HYPIC_DELTA ? hypic::seam_workspace_bytes(n_seg, w, n_chain) : 0;
  if (ws_need > 0) {
    if (!workspace) return fail(HYPIC_E_INVALID, "workspace is NULL (%zu bytes required)", ws_need);
    if (workspace_bytes < ws_need)
      return fail(HYPIC_E_INVALID, "workspace too small: %zu bytes given, %zu required", workspace_bytes, ws_need);
    TRY(check_aligned(workspace, "workspace"));
    outs.push_back({workspace, ws_need, "workspace"});
  }
  TRY(check_overlaps(ins, outs));
  const bool f32 = seam->dtype == HYPIC_F32;

  hypic::SeamArgs a;
  a.q = seam->q;
  a.k = seam->k;
  a.v = seam->v;
  a.beta = seam->beta;
  a.lg = seam->log_gate;
  a.gate_per_chain = seam->gate_per_chain ? 1 : 0;
  a.bg = body ? body->g : nullptr;
  a.bU = body ? body->U : nullptr;
  a.bS = body ? body->S : nullptr;
  a.S_run = S_run;
  a.o = o_out;
  a.wg = window_out ? window_out->g : nullptr;
  a.wU = window_out ? window_out->U : nullptr;
  a.wS = window_out ? window_out->S : nullptr;
  a.n_seg = n_seg;
  a.w = w;
  a.n_chain = n_chain;
  a.wrec = nullptr;
  hipError_t e;
  if (fam == HYPIC_DELTA) {
    float* rec = reinterpret_cast<float*>(workspace);
    e = hypic::launch_seam_prep(d, f32, a, rec, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hypic_seam_step window factor launch");
    a.wrec = rec;
    e = hypic::launch_seam_chain(d, f32, a, (hipStream_t)stream);
  } else if (fam == HYPIC_KDA) {
    e = hypic::launch_seam_kda(d, f32, a, (hipStream_t)stream);
  } else {
    e = hypic::launch_seam_elem(fam, d, f32, a, (hipStream_t)stream);
  }
  if (e != hipSuccess) return hip_fail(e, "hypic_seam_step launch");
  if (window_out) {
    // each window's own pair depends only on its tokens: the segment build of
    // the windows (segments of w tokens), on the single-kernel delta path
    hypic::BuildArgs b;
    b.k = seam->k;
    b.v = seam->v;
    b.beta = seam->beta;
    b.lg = seam->log_gate;
    b.g = window_out->g;
    b.U = window_out->U;
    b.S = window_out->S;
    b.n_chain = n_chain;
    b.gate_per_chain = seam->gate_per_chain ? 1 : 0;
    std::vector<int32_t> woff((size_t)n_seg + 1);
    for (int i = 0; i <= n_seg; ++i) woff[i] = i * w;
    for (const hypic::SegTable& t : plan_launches(woff.data(), 0, n_seg)) {
      b.seg = t;
      const int ns = t.n_seg;
      e = (fam == HYPIC_DELTA) ? hypic::launch_build_delta_single(d, f32, b, ns * n_chain, (hipStream_t)stream)
          : (fam == HYPIC_KDA) ? hypic::launch_build_kda(d, f32, b, ns * n_chain, nullptr, (hipStream_t)stream)
                               : hypic::launch_build_sd(fam, d, f32, b, ns * n_chain, (hipStream_t)stream);
      if (e != hipSuccess) return hip_fail(e, "hypic_seam_step window pairs launch");
    }
  }
  return ok();
}

hypic_status hypic_rerotate(hypic_family fam, int n_seg, int n_chain, int d_k, int d_v, const int32_t* positions,
                            double rope_base, const hypic_pairs* pairs, void* stream) {
  TRY(check_common(fam, n_seg, n_chain, d_k, d_v));
  const int d = d_k;
  if (fam == HYPIC_DIAG || fam == HYPIC_KDA)
    return fail(HYPIC_E_UNSUPPORTED, "a per-channel gate does not commute with the rotation");
  if (!(rope_base > 0.0) || !std::isfinite(rope_base))
    return fail(HYPIC_E_INVALID, "rope_base must be positive and finite");
  if (!positions) return fail(HYPIC_E_INVALID, "positions is NULL");
  if (!pairs) return fail(HYPIC_E_INVALID, "pairs is NULL");
  if (!pairs->S) return fail(HYPIC_E_INVALID, "pairs.S is NULL");
  if (fam == HYPIC_DELTA && !pairs->U) return fail(HYPIC_E_INVALID, "pairs.U is required for the delta family");
  if (fam != HYPIC_DELTA && pairs->U) return fail(HYPIC_E_INVALID, "pairs.U is only defined for the delta family");
  if ((int64_t)n_seg * n_chain * (pairs->U ? 2 : 1) > INT32_MAX)
    return fail(HYPIC_E_INVALID, "too many pairs for one launch (%d x %d)", n_seg, n_chain);
  TRY(check_aligned(pairs->S, "pairs.S"));
  if (pairs->U) TRY(check_aligned(pairs->U, "pairs.U"));
  const size_t mbytes = (size_t)n_seg * n_chain * d * d * 4;
  std::vector<Range> ins, outs;
  ins.push_back({positions, (size_t)n_seg * 4, "positions"});
  outs.push_back({pairs->S, mbytes, "pairs.S"});
  if (pairs->U) outs.push_back({pairs->U, mbytes, "pairs.U"});
  TRY(check_overlaps(ins, outs));
  hipError_t e = hypic::launch_rerotate(d, pairs->S, pairs->U, positions, n_seg, n_chain, rope_base,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hypic_rerotate launch");
  return ok();
}

}  // extern "C"
