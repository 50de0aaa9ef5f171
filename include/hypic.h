/*
 * hypic.h -- C ABI of the MI355X (gfx950) library for the linear-attention hot
 * path of position-independent caching: per-segment build of the cached pair
 * (T_C, S(C|0)), ordered composition of cached pairs, the seam-window step, and
 * the rotary re-rotation of cached pairs to a new position.
 *
 * Pages cited (by title):
 *   [youleyou] "小红书联合北大上交提出HYPIC，位置无关缓存降低首token延迟3.25倍" (youleyou.com)
 *   [hwlabs]   "HYPIC: 하이브리드 어텐션 LLM 서빙에서 포지션 독립적 캐싱으로 TTFT를 2.45배
 *              낮추는 방법" (llm-wiki.hwlabs.dev)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer, row-major, 16-byte aligned,
 *    allocated and owned by the caller.  The library never allocates or frees
 *    device memory and keeps no pointer after the call returns.  `seg_offsets`
 *    of hypic_seg_build (and of hypic_seg_build_workspace_size) is the only
 *    HOST pointer (the positions of hypic_rerotate are on the device).
 *    Scratch memory, where a call needs any, is a caller workspace sized by a
 *    query function.
 *  - Calls are asynchronous: HYPIC_OK means "validated and enqueued on
 *    `stream`" (a hipStream_t passed as void*; NULL = the null stream).  Results
 *    are ready once the stream reaches that point.
 *  - Arguments are validated on the host before anything is enqueued; a
 *    nonzero status means nothing was enqueued (except HYPIC_E_HIP, which
 *    reports a failed launch).  The library never aborts or throws.  The
 *    message of the last failure on the calling thread is in hypic_last_error().
 *  - Non-finite input values are not checked: NaN in gives NaN out.
 *  - Per head the state is S in R^{d_k x d_v} (d_v contiguous) and a token's
 *    output is o_t = S_t^T q_t, taken after the token's own update.  Layers and
 *    heads are folded into one "chain" index (chain = layer * heads + head).
 *  - Supported sizes: d_k = d_v = d with d in {64, 128}.  Other sizes return
 *    HYPIC_E_UNSUPPORTED.  The KDA build (and the KDA seam step's optional
 *    window pairs) is built for d = 64 and for d = 128 with bf16 tokens; the
 *    re-rotation is not defined for KDA (HYPIC_E_UNSUPPORTED); KDA pairs
 *    compose like DELTA pairs.
 *  - Token tensors are token-major, [n_tok, n_chain, d] (d contiguous);
 *    per-token scalars are [n_tok, n_chain].
 *
 * Families (per-token transition A_t and write weight b_t; the pages name the
 * families -- naive linear attention, RetNet, Mamba2, GLA, DeltaNet, GDN -- but
 * print no per-token formula, so the standard published forms are used):
 *   HYPIC_NAIVE  : A_t = I,                            b_t = 1
 *   HYPIC_SCALAR : A_t = exp(lg_t) I       (RetNet, Mamba2), b_t = 1
 *   HYPIC_DIAG   : A_t = diag(exp(lg_t))   (GLA),    b_t = 1
 *   HYPIC_DELTA  : A_t = exp(lg_t)(I - beta_t k_t k_t^T) (DeltaNet: lg = 0; GDN),
 *                  b_t = beta_t
 *   HYPIC_KDA    : A_t = (I - beta_t k_t k_t^T) diag(exp(lg_t)) (KDA: the delta rule
 *                  with one gate per key channel), b_t = beta_t
 *   and S_t = A_t S_{t-1} + b_t k_t v_t^T.  [youleyou, linear-layer paragraph] lists
 *   KDA among the families whose transition is a dense matrix.
 *
 * Cached pair layout (fp32).  The segment transition T_C = A_L ... A_1 is kept
 * factored so that it cannot underflow (the scalar gate commutes with the
 * Householder-like factors):
 *   T_C = exp(g) U  (NAIVE: g = 0, U = I; SCALAR: U = I; DELTA: U = prod(I - beta k k^T))
 *   T_C = diag(exp(g))  (DIAG: g has d_k entries)
 *   T_C = exp(g) U  (KDA: the channel gates do not commute with the erase factors,
 *                    so U is the dense product and g only a scale that keeps U in
 *                    range; only exp(g) U is defined, the split is the library's)
 *   g : [n_seg, n_chain]  (DIAG: [n_seg, n_chain, d_k])
 *   U : [n_seg, n_chain, d_k, d_k]  (DELTA and KDA; NULL for the other families)
 *   S : [n_seg, n_chain, d_k, d_v]  = S(C|0)
 */
#ifndef HYPIC_H
#define HYPIC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYPIC_ABI_VERSION 8

typedef enum {
  HYPIC_OK = 0,
  HYPIC_E_INVALID = 1,     /* malformed arguments; nothing enqueued */
  HYPIC_E_UNSUPPORTED = 2, /* well-formed but not built (size, dtype/family combination) */
  HYPIC_E_HIP = 3          /* the HIP runtime reported an error at launch */
} hypic_status;

typedef enum { HYPIC_NAIVE = 0, HYPIC_SCALAR = 1, HYPIC_DIAG = 2, HYPIC_DELTA = 3, HYPIC_KDA = 4 } hypic_family;

typedef enum { HYPIC_F32 = 0, HYPIC_BF16 = 1 } hypic_dtype;

/* Token inputs (device pointers).  `dtype` applies to q, k, v, beta and
 * log_gate, except that a per-chain SCALAR gate is always fp32. */
typedef struct {
  hypic_dtype dtype;
  const void* q;        /* [n_tok, n_chain, d_k]; seam step only (NULL for builds) */
  const void* k;        /* [n_tok, n_chain, d_k] */
  const void* v;        /* [n_tok, n_chain, d_v] */
  const void* beta;     /* [n_tok, n_chain]; DELTA and KDA, NULL otherwise */
  const void* log_gate; /* natural log of the gate, <= 0:
                           SCALAR: [n_tok, n_chain], or fp32 [n_chain] if gate_per_chain (RetNet)
                           DIAG, KDA: [n_tok, n_chain, d_k]
                           DELTA : [n_tok, n_chain], or NULL (DeltaNet, gate = 1)
                           NAIVE : NULL */
  int gate_per_chain;   /* SCALAR only: 1 = one constant gate per chain */
} hypic_tokens;

/* Cached pairs written by the library (layout above). */
typedef struct {
  float* g;
  float* U;
  float* S;
} hypic_pairs;

/* Cached pairs read by the library (layout above). */
typedef struct {
  const float* g;
  const float* U;
  const float* S;
} hypic_cpairs;

/*
 * hypic_seg_build -- build (T_C, S(C|0)) of every (segment, chain) unit.
 *
 * [youleyou, linear-layer paragraph]: T_C is the product of all per-token
 * transition matrices of the segment and S(C|0) its final state from a zero
 * start; both depend only on the segment's own tokens, so every unit is built
 * independently and all of them run concurrently.
 * [hwlabs, section 병렬 콜드 프리필]: a segment may itself be split into pieces
 * joined by composition; inside a unit the kernels run 64-token chunks joined
 * the same way.
 *
 *   fam          family (above).
 *   n_seg        number of segments, >= 1.
 *   seg_offsets  HOST array of n_seg + 1 token offsets: segment s is tokens
 *                [seg_offsets[s], seg_offsets[s+1]); seg_offsets[0] = 0 and the
 *                offsets strictly increase (every segment has >= 1 token).
 *                Segment lengths may differ (ragged batches).
 *   n_chain      chains (layers x heads), >= 1.
 *   d_k, d_v     head sizes (d_k = d_v in {64, 128}).
 *   in           token inputs; q is ignored.
 *   out          g, S required; U required for DELTA (NULL otherwise).  Every
 *                output element is written.
 *   workspace    device scratch of at least workspace_bytes bytes, as returned
 *                by hypic_seg_build_workspace_size for the same fam, n_seg,
 *                seg_offsets, n_chain, d_k, d_v and in->dtype; may be NULL when
 *                that size is 0.  Its contents on entry are ignored and on exit
 *                undefined; it is in use until the stream passes the call, so
 *                calls that overlap in time need workspaces of their own.
 *   stream       hipStream_t or NULL.
 * Errors: HYPIC_E_INVALID for NULL required pointers, misaligned pointers,
 * bad offsets, a field that does not match the family, outputs or workspace
 * that overlap inputs or each other, or a workspace smaller than required;
 * HYPIC_E_UNSUPPORTED for other sizes.
 */
hypic_status hypic_seg_build(hypic_family fam, int n_seg, const int32_t* seg_offsets, int n_chain,
                             int d_k, int d_v, const hypic_tokens* in, const hypic_pairs* out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * hypic_seg_build_workspace_size -- bytes of workspace hypic_seg_build needs.
 *
 *  - DELTA with d = 128 and bf16 tokens (segments up to 2048 tokens): per
 *    64-token chunk and chain the chunk's WY factor (8,704 bytes), i.e. about
 *    136 bytes per token and chain.
 *  - KDA with d = 128 and bf16 tokens (segments up to 2048 tokens): per
 *    64-token chunk and chain a 42,512-byte factor record (the chunk's two
 *    decayed key copies and X as fp16, its gate factors), about 664 bytes per
 *    token and chain.
 *  - NAIVE, SCALAR, DIAG when there are few (segment, chain) units (at most
 *    256) and every segment has at least two 64-token chunks: the segments are
 *    built as P = min(4, 512 / units, shortest segment's chunks) pieces of whole
 *    chunks, joined by the composition law [youleyou, linear-layer paragraph];
 *    the workspace holds the pieces' pairs: g (padded to 256 bytes) and S.
 *  - 0 otherwise.
 * Arguments as for hypic_seg_build (seg_offsets is validated the same way);
 * *bytes receives the size.  Enqueues nothing.
 */
hypic_status hypic_seg_build_workspace_size(hypic_family fam, int n_seg, const int32_t* seg_offsets,
                                            int n_chain, int d_k, int d_v, hypic_dtype dtype,
                                            size_t* bytes);

/*
 * hypic_compose -- ordered composition of cached pairs along every chain.
 *
 * [youleyou, linear-layer paragraph]: S(C1.C2) = T(C2) S(C1) + S(C2), i.e.
 * left-multiply by T_C and add; [hwlabs, section 세그먼트 누적 전이 연산자]:
 * T_ABC = T_C T_B T_A and e_ABC = T_C (T_B e_A + e_B) + e_C.
 * For i = 0 .. n_seg-1 (index order): S <- T_i S + S_i, starting from S_init.
 *
 *   in             pairs [n_seg, n_chain, ...] (layout above); U for DELTA and KDA.
 *   S_init         [n_chain, d_k, d_v] or NULL (zero start).
 *   S_out          [n_chain, d_k, d_v]; may be the same pointer as S_init
 *                  (in-place update), no other overlap.
 *   prefix_states  NULL or [n_seg, n_chain, d_k, d_v]: the running state
 *                  BEFORE segment i (prefix_states[0] = S_init or 0).
 *   g_total        NULL or [n_chain] (DIAG: [n_chain, d_k]): sum of g_i.
 *   U_total        NULL or [n_chain, d_k, d_k] (DELTA, KDA): U_{n-1} ... U_0.
 *                  With S_init = NULL, (g_total, U_total, S_out) is the pair
 *                  of the concatenated segments.
 *   workspace      NULL, or device scratch of workspace_bytes bytes, at least
 *                  hypic_compose_workspace_size(); contents ignored on entry and
 *                  undefined on exit, in use until the stream passes the call.
 *                  For the DELTA and KDA families with few chains (at most 256 / (d / 32))
 *                  and at least 8 segments it lets the composition run as a
 *                  scan: blocks of consecutive segments are composed in
 *                  parallel (by associativity, [hwlabs, section 세그먼트 누적
 *                  전이 연산자]); without prefix_states the block pairs are then
 *                  reduced pairwise in parallel levels down to two; with them
 *                  each chain composes its block pairs in order and every block
 *                  is run again from its start state in parallel to emit them.
 *                  The result equals the single-pass one up to rounding.
 * Errors as for hypic_seg_build (a workspace that is smaller than required or
 * overlaps another argument is HYPIC_E_INVALID).
 */
hypic_status hypic_compose(hypic_family fam, int n_seg, int n_chain, int d_k, int d_v,
                           const hypic_cpairs* in, const float* S_init, float* S_out,
                           float* prefix_states, float* g_total, float* U_total,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * hypic_seg_build_compose -- a cold request in one call: every (segment, chain)
 * pair built as by hypic_seg_build, and every chain's pairs composed in index
 * order as by hypic_compose.
 *
 * [youleyou, segment-parallelism paragraph]: cold segments are prefilled in
 * parallel by scatter workers and a combine worker composes their results in
 * order, the combine step overlapping the scatter; [hwlabs, section 병렬 콜드
 * 프리필]: the pieces are joined by operator composition.  Two schedules:
 *   HYPIC_BC_SEQUENTIAL  every pair built in one pass, then composed (the
 *                        blocked scan of hypic_compose where it applies), all
 *                        on the caller's stream;
 *   HYPIC_BC_PIPELINED   the segments built in groups of consecutive segments
 *                        (enough units to fill the GPU once); each group, once
 *                        built, composed into one pair per chain on a second
 *                        stream of the library while the caller's stream builds
 *                        the next group; the group pairs then composed in order
 *                        on the caller's stream.  The second stream waits only
 *                        on events recorded on the caller's stream, and the
 *                        caller's stream on it before the last composition, so
 *                        the call is ordered on `stream` like any other (and can
 *                        be captured into a graph from it).  The library creates
 *                        that stream and its events once per host thread and
 *                        device, on the first call.
 *   HYPIC_BC_FUSED       the composition folded into the build: the segments
 *                        are the leaves of a binary tree per chain, and a build
 *                        workgroup that has written its pair counts its arrival
 *                        at the parent node (a device-wide atomic counter); the
 *                        last arrival composes the node's two children and moves
 *                        up, so composition overlaps the build with no workgroup
 *                        waiting on another.  It applies to the delta family at
 *                        d = 128 with bf16 tokens, segments of at most 2048
 *                        tokens, two or more segments and no S_init; elsewhere
 *                        the call runs the sequential schedule.  Calls that
 *                        overlap on one workspace race.
 * On one MI355X the sequential schedule is the faster at the 32k-token cold
 * request's shape (the two phases share the CUs' slots when overlapped).
 *
 *   out            the built pairs, as for hypic_seg_build.
 *   S_init, S_out, g_total, U_total   as for hypic_compose (no prefix states).
 *   mode           HYPIC_BC_SEQUENTIAL, HYPIC_BC_PIPELINED or HYPIC_BC_FUSED.
 *   workspace      device scratch of at least
 *                  hypic_seg_build_compose_workspace_size() bytes for `mode`
 *                  (NULL allowed when that is 0): the build's workspace, then
 *                  the composition's (sequential), each group's pair
 *                  (pipelined), or the tree's counters and node pairs (fused).
 *                  Contents ignored on entry, undefined on exit.
 * The pairs equal those of hypic_seg_build; S_out, g_total and U_total equal
 * those of hypic_compose up to the rounding of the grouping.
 * Errors as for hypic_seg_build and hypic_compose.
 */
enum { HYPIC_BC_SEQUENTIAL = 0, HYPIC_BC_PIPELINED = 1, HYPIC_BC_FUSED = 2 };
hypic_status hypic_seg_build_compose(hypic_family fam, int n_seg, const int32_t* seg_offsets, int n_chain,
                                     int d_k, int d_v, const hypic_tokens* in, const hypic_pairs* out,
                                     const float* S_init, float* S_out, float* g_total, float* U_total, int mode,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* hypic_seg_build_compose_workspace_size -- bytes of workspace that call needs
 * for the schedule `mode` (other arguments as for
 * hypic_seg_build_workspace_size; may be 0 in the sequential mode); enqueues
 * nothing. */
hypic_status hypic_seg_build_compose_workspace_size(hypic_family fam, int n_seg, const int32_t* seg_offsets,
                                                    int n_chain, int d_k, int d_v, hypic_dtype dtype, int mode,
                                                    size_t* bytes);

/*
 * hypic_compose_workspace_size -- bytes of workspace that enable the blocked
 * schedule of hypic_compose for these sizes (0: not used): per (block, chain)
 * its g, U and S, and with want_prefix = 0 the pairs of the first reduction
 * level (half as many), with want_prefix = 1 (prefix_states will be requested)
 * each block's start state instead.  *bytes receives the size; enqueues nothing.
 */
hypic_status hypic_compose_workspace_size(hypic_family fam, int n_seg, int n_chain, int d_k, int d_v,
                                          int want_prefix, size_t* bytes);

/*
 * hypic_seam_step -- advance the running state through each segment's seam
 * window, emitting the window tokens' outputs, then apply the segment's cached
 * body pair.
 *
 * [youleyou, full-attention paragraph]: the first w tokens of each reused
 * segment (default w = 8) are kept out of its cache entry and recomputed under
 * the full prefix; to do so the linear layers compute the window's own T and S
 * on the fly, advance the running state, and forward each seam token's output
 * to the full-attention layer above.
 * For each segment i in order: for its w window tokens t (rows i*w .. i*w+w-1
 * of the seam tensors) S <- A_t S + b_t k_t v_t^T and o_t = S^T q_t; then, if
 * body pairs are given, S <- T_{B_i} S + S_{B_i}.
 *
 *   n_seg, w       segments and window length (w >= 1).
 *   seam           window tokens [n_seg * w, n_chain, d] (q required).
 *   body           NULL (windows only) or cached body pairs [n_seg, n_chain, ...].
 *   S_run          [n_chain, d_k, d_v], read and overwritten with the final state.
 *   o_out          [n_seg * w, n_chain, d_v] fp32.
 *   window_out     NULL, or each window's own pair (T_W, S(W|0)), the pair a
 *                  segment build of the window tokens would give: g [n_seg,
 *                  n_chain] (DIAG: [.., d_k]) and S [n_seg, n_chain, d_k, d_v]
 *                  required, U [n_seg, n_chain, d_k, d_k] for DELTA only.  It
 *                  satisfies S_after = T_W S_before + S(W|0) for each window.
 *   workspace      device scratch of at least workspace_bytes bytes, as returned
 *                  by hypic_seam_step_workspace_size for the same fam, n_seg, w
 *                  and n_chain; may be NULL when that size is 0.  Contents
 *                  ignored on entry and undefined on exit; in use until the
 *                  stream passes the call.
 * Errors as for hypic_seg_build.
 */
hypic_status hypic_seam_step(hypic_family fam, int n_seg, int w, int n_chain, int d_k, int d_v,
                             const hypic_tokens* seam, const hypic_cpairs* body, float* S_run,
                             float* o_out, const hypic_pairs* window_out, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * hypic_seam_step_workspace_size -- bytes of workspace hypic_seam_step needs.
 *
 * Only the DELTA family uses one: the part of each window's update that does
 * not depend on the running state (the window's inverse factor and gate
 * weights, 576 bytes per 8-token sub-window and chain) is formed for all
 * windows at once before the ordered pass.  Other families return 0.
 * *bytes receives the size; enqueues nothing.
 */
hypic_status hypic_seam_step_workspace_size(hypic_family fam, int n_seg, int w, int n_chain, int d_k,
                                            int d_v, size_t* bytes);

/*
 * hypic_seam_step_noalloc -- hypic_seam_step for callers that cannot allocate
 * device memory: code under HIP graph capture, serving loops and harnesses that
 * forbid allocation.  The delta family's window records (see
 * hypic_seam_step_workspace_size) go to a fixed scratch array of
 * HYPIC_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on, from the first call there until the process ends, instead of a caller
 * workspace.
 *
 * Arguments, layouts, results and errors as hypic_seam_step without the
 * workspace.  Limit: the workspace size hypic_seam_step_workspace_size reports
 * for the call must not exceed HYPIC_NOALLOC_SCRATCH_BYTES (576 bytes per
 * 8-token sub-window and chain; the 100k-token warm request, 196 segments x
 * 480 chains with w = 8, needs 54 MB); a larger call returns HYPIC_E_INVALID
 * and enqueues nothing.  Other families use no scratch.
 * Calls no allocating routine.  Every call on one GPU uses that GPU's single
 * array: calls whose work overlaps on one GPU (on other streams, or from other
 * host threads without ordering) race on it and give undefined results; calls
 * ordered on one stream are safe.  Each call writes every record it reads, so
 * nothing is cleared between calls.  The first call on a device looks up the
 * array's device address with that device current (HYPIC_E_HIP if that fails).
 */
#define HYPIC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hypic_status hypic_seam_step_noalloc(hypic_family fam, int n_seg, int w, int n_chain, int d_k, int d_v,
                                     const hypic_tokens* seam, const hypic_cpairs* body, float* S_run,
                                     float* o_out, const hypic_pairs* window_out, void* stream);

/*
 * hypic_rerotate -- move cached pairs to a new position under rotary position
 * encoding, in place.
 *
 * [youleyou, linear-layer paragraph]: for linear layers whose keys carry a
 * rotary encoding, a cached segment reused at another position is aligned
 * exactly by re-rotating its state.  The pages give no formula; the reading
 * implemented: keys carry the RoFormer encoding -- the pairs (2i, 2i+1) of the
 * d_k axis turned by the angle pos * theta_i, theta_i = rope_base^(-2i/d_k) --
 * at positions counted from the segment's first token when the pair was
 * built.  Reused with its first token at position p, every key becomes R(p) k,
 * every per-token transition R(p) A_t R(p)^T and every write R(p) k v^T, so
 *   DELTA:         U <- R(p) U R(p)^T   (g unchanged)
 *   every family:  S <- R(p) S
 * NAIVE and SCALAR transitions are multiples of I and do not change.  A DIAG
 * transition does not stay diagonal under R(p) (unless its gates agree within
 * each pair), so that family returns HYPIC_E_UNSUPPORTED.
 *
 *   positions   DEVICE [n_seg] int32: the offset p of segment s, any sign.
 *               Rotations add (R(a) R(b) = R(a + b)), so a pair already moved
 *               to p0 and rotated by p ends at p0 + p.
 *   rope_base   the rotary base, positive and finite (e.g. 10000).
 *   pairs       S [n_seg, n_chain, d_k, d_v] (required) and U [n_seg, n_chain,
 *               d_k, d_k] (DELTA only, NULL otherwise) are updated in place; g
 *               is neither read nor written (may be NULL).
 * The angles and their cosines and sines are formed in fp64 on the device (so
 * offsets far beyond 2^24 tokens keep full accuracy); the rotation is fp32.
 * Errors as for hypic_compose; positions overlapping S or U is HYPIC_E_INVALID.
 */
hypic_status hypic_rerotate(hypic_family fam, int n_seg, int n_chain, int d_k, int d_v,
                            const int32_t* positions, double rope_base, const hypic_pairs* pairs,
                            void* stream);

/* Message of the last failed call on this thread ("" if none).  The string is
 * owned by the library and valid until the next call on this thread. */
const char* hypic_last_error(void);

/* HYPIC_ABI_VERSION of the loaded library. */
int hypic_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HYPIC_H */
