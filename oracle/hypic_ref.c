/*
 * hypic_ref.c -- the oracle: a plain, slow, fp64 CPU statement of what the
 * linear-attention hot path of position-independent caching computes.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header, table or helper with the HIP
 * library; it reads its inputs as fp64 values (bf16/fp32 inputs converted
 * exactly by the caller) and writes fp64 results.
 *
 * Pages cited (by title):
 *   [youleyou]  "小红书联合北大上交提出HYPIC，位置无关缓存降低首token延迟3.25倍"
 *               (youleyou.com), the paragraphs on linear layers, on full-attention
 *               layers (seam window) and on segment parallelism.
 *   [xix]       "Xiaohongshu, die Peking-Universität und die Shanghai Jiao Tong
 *               University stellen HYPIC vor ..." (xix.ai), the same paragraphs.
 *   [hwlabs]    "HYPIC: 하이브리드 어텐션 LLM 서빙에서 포지션 독립적 캐싱으로 TTFT를
 *               2.45배 낮추는 방법" (llm-wiki.hwlabs.dev), section
 *               "세그먼트 누적 전이 연산자" (h_out = T_S h_in + e_S and the
 *               three-segment composition T_ABC, e_ABC).
 *
 * What the pages fix, restated:
 *   - Each linear-attention token applies a transition matrix to the state and
 *     adds its own write; a segment's transition operator T_C is the ordered
 *     product of its per-token transition matrices, and S(C|0) is the final
 *     state from a zero start [youleyou, linear layers; hwlabs, h_out = T h_in + e].
 *   - Both depend only on the segment's own tokens, and concatenation composes
 *     as S(C1.C2) = T(C2) S(C1) + S(C2), T(C1.C2) = T(C2) T(C1)
 *     [youleyou, linear layers; hwlabs, T_ABC = T_C T_B T_A].
 *   - Plain addition of zero-start states is exact only for naive linear
 *     attention (T = I) [youleyou, linear layers].
 *   - At reuse the first w tokens of each segment (the seam window) are run
 *     through the layer on the running state, emitting each token's output,
 *     and the cached pair covers the rest of the segment [youleyou,
 *     full-attention paragraph].
 *
 * Readings taken where the pages are silent (the pages name the families
 * RetNet, Mamba2, GLA, DeltaNet, GDN, KDA but print no per-token formula):
 *   state S is d_k x d_v, the output of a token is o_t = S_t^T q_t taken after
 *   the token's own update, and the per-token update is
 *     naive : S <- S + k v^T
 *     scalar: S <- a_t S + k v^T                       (RetNet, Mamba2)
 *     diag  : S <- diag(alpha_t) S + k v^T             (GLA)
 *     delta : S <- a_t (I - beta_t k k^T) S + beta_t k v^T   (DeltaNet a=1, GDN)
 *     kda   : S <- (I - beta_t k k^T) diag(alpha_t) S + beta_t k v^T   (KDA:
 *             the delta rule with one gate per key channel)
 *   with a_t = exp(log_gate_t).  The transition operator is kept factored as
 *   T = exp(g) * U (scalar/delta: g scalar; diag: T = diag(exp(g)), U = I;
 *   delta: U = prod (I - beta k k^T)) so that it cannot underflow; the scalar
 *   gate commutes with the Householder-like factors, so the factorisation is
 *   exact.  For KDA the per-channel gates do not commute with the erase
 *   factors, so T = exp(g) U is a dense product whose scalar g is only a scale:
 *   each token moves its largest channel gate into g.  Only the product
 *   exp(g) U is defined; a different split of it is an equal pair.
 *
 * Layouts (row-major, fp64):
 *   tokens  k, v, q : [n_tok, n_chain, d]   (token-major, d contiguous)
 *   beta            : [n_tok, n_chain]
 *   log_gate        : scalar/delta [n_tok, n_chain] (or [n_chain] when
 *                     gate_per_chain), diag/kda [n_tok, n_chain, d_k], else NULL
 *   pairs g         : [n_seg, n_chain] (diag: [n_seg, n_chain, d_k])
 *   pairs U         : [n_seg, n_chain, d_k, d_k] (delta and kda)
 *   pairs S, states : [.., n_chain, d_k, d_v]
 *
 * Rotary re-rotation (hypic_ref_rerotate, below): the pages name a state
 * re-rotation step for linear layers that carry rotary position encoding but
 * give no formula; the reading taken is stated at that function.
 *
 * Parity pins (see the tests): brute-force matrix products on tiny inputs,
 * the composition law against straight recurrence over the concatenation,
 * re-rotation against a build from keys rotated at the new positions,
 * closed forms of the scalar and diagonal families, the one-token and
 * overwrite cases of the delta rule, Householder orthogonality, and the size
 * of the naive-addition error on a slow-decay head.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { REF_NAIVE = 0, REF_SCALAR = 1, REF_DIAG = 2, REF_DELTA = 3, REF_KDA = 4 };

/* Families whose transition is a dense matrix, kept as T = exp(g) U. */
#define REF_DENSE(fam) ((fam) == REF_DELTA || (fam) == REF_KDA)

#define REF_OK 0
#define REF_EINVAL 1
#define REF_ENOMEM 2

/* Per-chain view of one token's inputs. */
typedef struct {
  const double* k;   /* d_k */
  const double* v;   /* d_v */
  double beta;       /* delta only */
  double lg;         /* scalar/delta log gate (0 when absent) */
  const double* lgv; /* diag and KDA per-channel log gates (d_k) */
} tok_t;

static tok_t get_tok(int fam, int t, int h, int n_chain, int dk, int dv,
                     const double* k, const double* v, const double* beta,
                     const double* lg, int gate_per_chain) {
  tok_t x;
  x.k = k + ((size_t)t * n_chain + h) * dk;
  x.v = v + ((size_t)t * n_chain + h) * dv;
  x.beta = REF_DENSE(fam) ? beta[(size_t)t * n_chain + h] : 1.0;
  x.lg = 0.0;
  x.lgv = NULL;
  if (fam == REF_SCALAR) {
    x.lg = gate_per_chain ? lg[h] : lg[(size_t)t * n_chain + h];
  } else if (fam == REF_DELTA && lg != NULL) {
    x.lg = lg[(size_t)t * n_chain + h];
  } else if (fam == REF_DIAG || fam == REF_KDA) {
    x.lgv = lg + ((size_t)t * n_chain + h) * dk;
  }
  return x;
}

/* U <- (I - beta k k^T) U, one rank-1 step, column by column. */
static void erase_rank1(int dk, const tok_t* x, double* U) {
  for (int j = 0; j < dk; ++j) {
    double dot = 0.0;
    for (int i = 0; i < dk; ++i) dot += x->k[i] * U[(size_t)i * dk + j];
    for (int i = 0; i < dk; ++i) U[(size_t)i * dk + j] -= x->beta * x->k[i] * dot;
  }
}

/*
 * One token of the recurrence applied to the state S (d_k x d_v) and, when
 * requested, to the factored transition (g, U) accumulated so far:
 * S <- A_t S + b_t k v^T,  T <- A_t T  [youleyou, linear layers: T_C is the
 * product of the per-token transition matrices].  `work` holds d_v doubles.
 */
static void token_step(int fam, int dk, int dv, const tok_t* x, double* S,
                       double* g, double* U, double* work) {
  int i, j;
  switch (fam) {
    case REF_NAIVE:
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] += x->k[i] * x->v[j];
      break;
    case REF_SCALAR: {
      double a = exp(x->lg);
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
          S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + x->k[i] * x->v[j];
      if (g) g[0] += x->lg;
      break;
    }
    case REF_DIAG:
      for (i = 0; i < dk; ++i) {
        double a = exp(x->lgv[i]);
        for (j = 0; j < dv; ++j)
          S[(size_t)i * dv + j] = a * S[(size_t)i * dv + j] + x->k[i] * x->v[j];
        if (g) g[i] += x->lgv[i];
      }
      break;
    case REF_DELTA: {
      double a = exp(x->lg);
      /* work = k^T S  (row vector over d_v) */
      for (j = 0; j < dv; ++j) work[j] = 0.0;
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) work[j] += x->k[i] * S[(size_t)i * dv + j];
      /* S <- a (S - beta k (k^T S)) + beta k v^T */
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) {
          double s = S[(size_t)i * dv + j];
          S[(size_t)i * dv + j] =
              a * (s - x->beta * x->k[i] * work[j]) + x->beta * x->k[i] * x->v[j];
        }
      if (U) erase_rank1(dk, x, U);
      if (g) g[0] += x->lg;
      break;
    }
    case REF_KDA: {
      /* S <- (I - beta k k^T) diag(alpha) S + beta k v^T: decay each row
       * (channel) of S first, then the delta-rule erase and write. */
      for (i = 0; i < dk; ++i) {
        const double a = exp(x->lgv[i]);
        for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
      }
      for (j = 0; j < dv; ++j) work[j] = 0.0;
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) work[j] += x->k[i] * S[(size_t)i * dv + j];
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j)
          S[(size_t)i * dv + j] += x->beta * x->k[i] * (x->v[j] - work[j]);
      if (U) {
        /* T = exp(g) U and T <- (I - beta k k^T) diag(alpha) T.  The largest
         * channel gate m of the token moves into g, so U is scaled by
         * diag(exp(lg - m)) <= 1 and cannot overflow. */
        double m = x->lgv[0];
        for (i = 1; i < dk; ++i)
          if (x->lgv[i] > m) m = x->lgv[i];
        for (i = 0; i < dk; ++i) {
          const double a = exp(x->lgv[i] - m);
          for (j = 0; j < dk; ++j) U[(size_t)i * dk + j] *= a;
        }
        erase_rank1(dk, x, U);
        if (g) g[0] += m;
      }
      break;
    }
  }
}

static int fam_ok(int fam) { return fam >= REF_NAIVE && fam <= REF_KDA; }

/* Per-chain gate accumulators live on the stack; d_k is bounded accordingly. */
#define REF_MAX_D 4096

static int gate_len(int fam, int dk) { return fam == REF_DIAG ? dk : 1; }

static void set_identity(double* U, int d) {
  memset(U, 0, sizeof(double) * (size_t)d * d);
  for (int i = 0; i < d; ++i) U[(size_t)i * d + i] = 1.0;
}

/*
 * Segment build: for every (segment, chain) unit, start from T = I, S = 0 and
 * run the unit's tokens in order; emit the factored T_C and S(C|0)
 * [youleyou, linear layers: both are fixed by the segment's own tokens and are
 * cached together at its first prefill].
 *   offsets: n_seg + 1 token offsets, offsets[0] = 0, strictly increasing.
 *   U_out may be NULL (it is only defined for the delta family).
 */
int hypic_ref_build(int fam, int n_seg, const int32_t* offsets, int n_chain, int dk,
                    int dv, const double* k, const double* v, const double* beta,
                    const double* lg, int gate_per_chain, double* g_out, double* U_out,
                    double* S_out, int n_threads) {
  if (!fam_ok(fam) || n_seg < 1 || n_chain < 1 || dk < 1 || dv < 1 || dk > REF_MAX_D || !offsets || !k ||
      !v || !g_out || !S_out)
    return REF_EINVAL;
  if (REF_DENSE(fam) && !beta) return REF_EINVAL;
  if ((fam == REF_SCALAR || fam == REF_DIAG || fam == REF_KDA) && !lg) return REF_EINVAL;
  if (offsets[0] != 0) return REF_EINVAL;
  for (int s = 0; s < n_seg; ++s)
    if (offsets[s + 1] <= offsets[s]) return REF_EINVAL;
  const int gl = gate_len(fam, dk);
  const long n_units = (long)n_seg * n_chain;
  int status = REF_OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
  for (long u = 0; u < n_units; ++u) {
    const int s = (int)(u / n_chain), h = (int)(u % n_chain);
    double* work = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
    double* U = REF_DENSE(fam) ? (double*)malloc(sizeof(double) * (size_t)dk * dk) : NULL;
    if (!work || (REF_DENSE(fam) && !U)) {
      status = REF_ENOMEM;
      free(work);
      free(U);
      continue;
    }
    double* S = S_out + (size_t)u * dk * dv;
    double* g = g_out + (size_t)u * gl;
    memset(S, 0, sizeof(double) * (size_t)dk * dv);
    for (int i = 0; i < gl; ++i) g[i] = 0.0;
    if (U) set_identity(U, dk);
    for (int t = offsets[s]; t < offsets[s + 1]; ++t) {
      tok_t x = get_tok(fam, t, h, n_chain, dk, dv, k, v, beta, lg, gate_per_chain);
      token_step(fam, dk, dv, &x, S, g, U, work);
    }
    if (U && U_out) memcpy(U_out + (size_t)u * dk * dk, U, sizeof(double) * (size_t)dk * dk);
    free(work);
    free(U);
  }
  return status;
}

/*
 * Apply one cached transition to a state: S <- T S with T = exp(g) U (delta),
 * diag(exp(g)) (diag), exp(g) I (scalar) or I (naive).  `tmp` holds d_k*d_v.
 */
static void apply_T(int fam, int dk, int dv, const double* g, const double* U, double* S,
                    double* tmp) {
  int i, j, l;
  switch (fam) {
    case REF_NAIVE:
      break;
    case REF_SCALAR: {
      double a = exp(g[0]);
      for (i = 0; i < dk * dv; ++i) S[i] *= a;
      break;
    }
    case REF_DIAG:
      for (i = 0; i < dk; ++i) {
        double a = exp(g[i]);
        for (j = 0; j < dv; ++j) S[(size_t)i * dv + j] *= a;
      }
      break;
    case REF_DELTA:
    case REF_KDA: {
      double a = exp(g[0]);
      for (i = 0; i < dk; ++i)
        for (j = 0; j < dv; ++j) {
          double acc = 0.0;
          for (l = 0; l < dk; ++l) acc += U[(size_t)i * dk + l] * S[(size_t)l * dv + j];
          tmp[(size_t)i * dv + j] = a * acc;
        }
      memcpy(S, tmp, sizeof(double) * (size_t)dk * dv);
      break;
    }
  }
}

/*
 * Ordered composition of cached pairs along each chain: for i = 0..n_seg-1,
 * S <- T_i S + S_i, starting from S_init (or zero)
 * [youleyou, linear layers: left-multiply by T_C, then add;
 *  hwlabs, e_ABC = T_C (T_B e_A + e_B) + e_C].
 *   prefix (optional): the running state before each segment.
 *   g_tot, U_tot (optional): the transition of the whole concatenation,
 *   g = sum g_i and U = U_{n-1} ... U_0 [hwlabs, T_ABC = T_C T_B T_A].
 */
int hypic_ref_compose(int fam, int n_seg, int n_chain, int dk, int dv, const double* g,
                      const double* U, const double* S, const double* S_init, double* S_out,
                      double* prefix, double* g_tot, double* U_tot, int n_threads) {
  if (!fam_ok(fam) || n_seg < 1 || n_chain < 1 || dk < 1 || dv < 1 || dk > REF_MAX_D || !g ||
      !S || !S_out)
    return REF_EINVAL;
  if (REF_DENSE(fam) && !U) return REF_EINVAL;
  const int gl = gate_len(fam, dk);
  int status = REF_OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
  for (int h = 0; h < n_chain; ++h) {
    const size_t sz = (size_t)dk * dv;
    double* cur = (double*)malloc(sizeof(double) * sz);
    double* tmp = (double*)malloc(sizeof(double) * sz);
    double* ut = (U_tot && REF_DENSE(fam)) ? (double*)malloc(sizeof(double) * (size_t)dk * dk * 2) : NULL;
    if (!cur || !tmp || (U_tot && REF_DENSE(fam) && !ut)) {
      status = REF_ENOMEM;
      free(cur);
      free(tmp);
      free(ut);
      continue;
    }
    if (S_init)
      memcpy(cur, S_init + (size_t)h * sz, sizeof(double) * sz);
    else
      memset(cur, 0, sizeof(double) * sz);
    double gacc[REF_MAX_D];
    for (int i = 0; i < gl; ++i) gacc[i] = 0.0;
    if (ut) set_identity(ut, dk);
    for (int s = 0; s < n_seg; ++s) {
      const size_t pu = (size_t)s * n_chain + h;
      if (prefix) memcpy(prefix + pu * sz, cur, sizeof(double) * sz);
      apply_T(fam, dk, dv, g + pu * gl, REF_DENSE(fam) ? U + pu * dk * dk : NULL, cur, tmp);
      const double* Si = S + pu * sz;
      for (size_t e = 0; e < sz; ++e) cur[e] += Si[e];
      for (int i = 0; i < gl; ++i) gacc[i] += g[pu * gl + i];
      if (ut) {
        /* ut <- U_s ut */
        const double* Us = U + pu * dk * dk;
        double* nt = ut + (size_t)dk * dk;
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < dk; ++j) {
            double acc = 0.0;
            for (int l = 0; l < dk; ++l) acc += Us[(size_t)i * dk + l] * ut[(size_t)l * dk + j];
            nt[(size_t)i * dk + j] = acc;
          }
        memcpy(ut, nt, sizeof(double) * (size_t)dk * dk);
      }
    }
    memcpy(S_out + (size_t)h * sz, cur, sizeof(double) * sz);
    if (g_tot)
      for (int i = 0; i < gl; ++i) g_tot[(size_t)h * gl + i] = gacc[i];
    if (U_tot && ut) memcpy(U_tot + (size_t)h * dk * dk, ut, sizeof(double) * (size_t)dk * dk);
    free(cur);
    free(tmp);
    free(ut);
  }
  return status;
}

/*
 * Seam-window step at reuse: for each segment i in order, run its w window
 * tokens through the recurrence on the running state, emitting
 * o_t = S_t^T q_t after each token, then apply the segment's cached body pair,
 * S <- T_B S + S_B [youleyou, full-attention paragraph: the linear layers
 * compute the window's own T and S on the fly, advance the running state and
 * hand each seam token's output upward].
 *   Window tokens are rows i*w .. i*w+w-1 of q/k/v/beta/log_gate.
 *   body_S == NULL means no body pairs (windows only).
 *   wg/wU/wS (optional): each window's own factored pair (T_W, S(W|0)).
 */
int hypic_ref_seam(int fam, int n_seg, int w, int n_chain, int dk, int dv, const double* q,
                   const double* k, const double* v, const double* beta, const double* lg,
                   int gate_per_chain, const double* body_g, const double* body_U,
                   const double* body_S, double* S_run, double* o_out, double* wg, double* wU,
                   double* wS, int n_threads) {
  if (!fam_ok(fam) || n_seg < 1 || w < 1 || n_chain < 1 || dk < 1 || dv < 1 || dk > REF_MAX_D ||
      !q || !k ||
      !v || !S_run || !o_out)
    return REF_EINVAL;
  if (REF_DENSE(fam) && !beta) return REF_EINVAL;
  if ((fam == REF_SCALAR || fam == REF_DIAG || fam == REF_KDA) && !lg) return REF_EINVAL;
  if (body_S && (!body_g || (REF_DENSE(fam) && !body_U))) return REF_EINVAL;
  const int gl = gate_len(fam, dk);
  int status = REF_OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
  for (int h = 0; h < n_chain; ++h) {
    const size_t sz = (size_t)dk * dv;
    double* S = S_run + (size_t)h * sz;
    double* tmp = (double*)malloc(sizeof(double) * sz);
    double* work = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
    double* pS = (double*)malloc(sizeof(double) * sz);
    double* pU = (double*)malloc(sizeof(double) * (size_t)dk * dk);
    if (!tmp || !work || !pS || !pU) {
      status = REF_ENOMEM;
      free(tmp);
      free(work);
      free(pS);
      free(pU);
      continue;
    }
    for (int s = 0; s < n_seg; ++s) {
      double pg[REF_MAX_D];
      for (int i = 0; i < gl; ++i) pg[i] = 0.0;
      memset(pS, 0, sizeof(double) * sz);
      set_identity(pU, dk);
      for (int j = 0; j < w; ++j) {
        const int t = s * w + j;
        tok_t x = get_tok(fam, t, h, n_chain, dk, dv, k, v, beta, lg, gate_per_chain);
        token_step(fam, dk, dv, &x, S, NULL, NULL, work);
        if (wS || wU || wg) token_step(fam, dk, dv, &x, pS, pg, REF_DENSE(fam) ? pU : NULL, work);
        const double* qt = q + ((size_t)t * n_chain + h) * dk;
        double* ot = o_out + ((size_t)t * n_chain + h) * dv;
        for (int c = 0; c < dv; ++c) {
          double acc = 0.0;
          for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + c] * qt[i];
          ot[c] = acc;
        }
      }
      const size_t pu = (size_t)s * n_chain + h;
      if (wS) memcpy(wS + pu * sz, pS, sizeof(double) * sz);
      if (wU && REF_DENSE(fam)) memcpy(wU + pu * dk * dk, pU, sizeof(double) * (size_t)dk * dk);
      if (wg)
        for (int i = 0; i < gl; ++i) wg[pu * gl + i] = pg[i];
      if (body_S) {
        apply_T(fam, dk, dv, body_g + pu * gl, REF_DENSE(fam) ? body_U + pu * dk * dk : NULL,
                S, tmp);
        const double* Sb = body_S + pu * sz;
        for (size_t e = 0; e < sz; ++e) S[e] += Sb[e];
      }
    }
    free(tmp);
    free(work);
    free(pS);
    free(pU);
  }
  return status;
}

/*
 * Straight recurrence over n_tok tokens from S_init (or zero): the "full
 * recompute" that composition must reproduce.  Optionally emits every token's
 * output o_t = S_t^T q_t.
 */
int hypic_ref_sequential(int fam, int n_tok, int n_chain, int dk, int dv, const double* q,
                         const double* k, const double* v, const double* beta,
                         const double* lg, int gate_per_chain, const double* S_init,
                         double* S_out, double* o_out, int n_threads) {
  if (!fam_ok(fam) || n_tok < 0 || n_chain < 1 || dk < 1 || dv < 1 || !k || !v || !S_out)
    return REF_EINVAL;
  if (REF_DENSE(fam) && !beta) return REF_EINVAL;
  if ((fam == REF_SCALAR || fam == REF_DIAG || fam == REF_KDA) && !lg) return REF_EINVAL;
  if (o_out && !q) return REF_EINVAL;
  int status = REF_OK;
#pragma omp parallel for schedule(dynamic, 1) num_threads(n_threads > 0 ? n_threads : 1)
  for (int h = 0; h < n_chain; ++h) {
    const size_t sz = (size_t)dk * dv;
    double* S = S_out + (size_t)h * sz;
    double* work = (double*)malloc(sizeof(double) * (size_t)(dv > dk ? dv : dk));
    if (!work) {
      status = REF_ENOMEM;
      continue;
    }
    if (S_init)
      memcpy(S, S_init + (size_t)h * sz, sizeof(double) * sz);
    else
      memset(S, 0, sizeof(double) * sz);
    for (int t = 0; t < n_tok; ++t) {
      tok_t x = get_tok(fam, t, h, n_chain, dk, dv, k, v, beta, lg, gate_per_chain);
      token_step(fam, dk, dv, &x, S, NULL, NULL, work);
      if (o_out) {
        const double* qt = q + ((size_t)t * n_chain + h) * dk;
        double* ot = o_out + ((size_t)t * n_chain + h) * dv;
        for (int c = 0; c < dv; ++c) {
          double acc = 0.0;
          for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + c] * qt[i];
          ot[c] = acc;
        }
      }
    }
    free(work);
  }
  return status;
}

/*
 * State re-rotation of cached pairs to a new position [youleyou, linear-layer
 * paragraph: for linear layers with RoPE a "state re-rotation" patch aligns a
 * cached segment exactly; the pages give no formula].  Reading taken: keys
 * carry the rotary encoding of RoFormer -- pairs (2i, 2i+1) of the d_k axis
 * rotated by the angle pos * theta_i, theta_i = base^(-2i/d_k) -- at their
 * position within the segment when the pair was cached.  Reused with its first
 * token at offset p, every key becomes R(p) R(t) k = R(p) k_cached, so each
 * per-token transition a (I - beta k k^T) becomes R(p) A_t R(p)^T and each write
 * R(p) k v^T; hence
 *     T' = R(p) T R(p)^T,   S'(C|0) = R(p) S(C|0).
 * For the naive and scalar families T is a multiple of I and stays put; for the
 * delta family U <- R U R^T (g unchanged).  A diagonal transition does not stay
 * diagonal under R (unless its gates agree within each pair), so that family
 * is refused.  delta[s] is segment s's offset p (any sign); pairs are updated
 * in place.  Plain dense products with the explicit rotation matrix.
 */
static void rope_matrix(double* R, int dk, long p, double base) {
  for (int i = 0; i < dk * dk; ++i) R[i] = 0.0;
  for (int i = 0; i < dk / 2; ++i) {
    const double theta = pow(base, -2.0 * i / dk);
    const double ang = (double)p * theta;
    const double c = cos(ang), sn = sin(ang);
    R[(2 * i) * dk + 2 * i] = c;
    R[(2 * i) * dk + 2 * i + 1] = -sn;
    R[(2 * i + 1) * dk + 2 * i] = sn;
    R[(2 * i + 1) * dk + 2 * i + 1] = c;
  }
}

int hypic_ref_rerotate(int fam, int n_seg, int n_chain, int dk, int dv, const int32_t* delta, double base,
                       double* U, double* S, int n_threads) {
  if (!fam_ok(fam) || fam == REF_DIAG || fam == REF_KDA || dk < 2 || dk % 2 || !S || !delta || !(base > 0.0)) return 1;
  if (fam == REF_DELTA && !U) return 1;
  int status = 0;
#pragma omp parallel num_threads(n_threads > 0 ? n_threads : 1)
  {
    double* R = (double*)malloc(sizeof(double) * dk * dk);
    double* tmp = (double*)malloc(sizeof(double) * dk * (dk > dv ? dk : dv));
    if (!R || !tmp) {
#pragma omp atomic write
      status = 2;
    } else {
#pragma omp for schedule(dynamic)
      for (long u = 0; u < (long)n_seg * n_chain; ++u) {
        rope_matrix(R, dk, delta[u / n_chain], base);
        double* Su = S + (size_t)u * dk * dv;  /* S <- R S */
        for (int i = 0; i < dk; ++i)
          for (int c = 0; c < dv; ++c) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += R[i * dk + j] * Su[(size_t)j * dv + c];
            tmp[(size_t)i * dv + c] = acc;
          }
        memcpy(Su, tmp, sizeof(double) * dk * dv);
        if (fam == REF_DELTA) {  /* U <- R U R^T */
          double* Uu = U + (size_t)u * dk * dk;
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dk; ++c) {
              double acc = 0.0;
              for (int j = 0; j < dk; ++j) acc += R[i * dk + j] * Uu[(size_t)j * dk + c];
              tmp[(size_t)i * dk + c] = acc;
            }
          for (int i = 0; i < dk; ++i)
            for (int c = 0; c < dk; ++c) {
              double acc = 0.0;
              for (int j = 0; j < dk; ++j) acc += tmp[(size_t)i * dk + j] * R[c * dk + j];
              Uu[(size_t)i * dk + c] = acc;
            }
        }
      }
    }
    free(R);
    free(tmp);
  }
  return status;
}

int hypic_ref_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
