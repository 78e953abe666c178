/*
 * moe_oracle.c -- plain, slow CPU oracle for one MoE layer's expert computation.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file: only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no source with the HIP library.
 *
 * Every floating-point step runs in IEEE double (the pages fix no precision);
 * inputs given in fp32 or bf16 are upcast exactly by the caller.  Loops are the
 * plain definitions: a per-token loop over the token's selected experts, with no
 * blocking, fusion or reordering.  OpenMP only splits independent tokens (or,
 * for dW, independent experts); each output is produced by exactly one thread in
 * a fixed order, so results do not depend on the thread count.
 *
 * What is computed, and where the pages describe it:
 *  - routing of each token to k of E experts, and token dispatch into per-expert
 *    groups of rows: npu-train issue #14 "[MoE] Hot experts on RNGD during
 *    training (host dispatch, device expert graphs)", sections Evidence (k = 1..8
 *    experts per token) and Proposal (routing and dispatch, rows grouped per
 *    expert, results scattered back);
 *  - expert forward, backward dx (LoRA, experts frozen) and dW (full
 *    fine-tuning): issue #14, sections Proposal and Scope;
 *  - saved forward activations reused by backward: npu-train pull request #44,
 *    section Changes (HostMLP keep_graph);
 *  - the router's logits and its backward with the selection held fixed
 *    (issue #14, sections Proposal and Done when);
 *  - retention quotas, per-pair selection within quotas, physical compaction and
 *    a backward restricted to the retained token-expert pairs: LRMoE
 *    (arXiv:2610.37720), abstract.
 * The pages print no formula.  The readings taken here (softmax over the k
 * selected logits, SwiGLU experts without biases, ties to the lower index,
 * retained pairs summed without rescaling) are listed with the design notes.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

static double sigmoid(double z) { return 1.0 / (1.0 + exp(-z)); }

/* ------------------------------------------------------------------------- */
/* Router logits  l[t,e] = sum_h x[t,h] * Wr[h,e]  (the router forward; also
 * builds the routing inputs of the tiny fp32 layer).                         */
void oracle_router_logits(int T, int H, int E, const double* x, const double* Wr, double* logits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int h = 0; h < H; ++h) s += x[(size_t)t * H + h] * Wr[(size_t)h * E + e];
      logits[(size_t)t * E + e] = s;
    }
}

/* ------------------------------------------------------------------------- */
/* Router backward with the selection held fixed (issue #14, Proposal: routing
 * precedes dispatch; Done when: the device path matches the host path in
 * outputs and gradients).  The weights are the softmax over the k selected
 * logits (the reading of oracle_route_topk), so with g_j = dL/dw[t,j] the chain
 * rule through that softmax gives
 *     dl[t, idx_j] = w_j * (g_j - sum_i w_i g_i),   dl[t, e] = 0 otherwise,
 * and through l = x Wr:
 *     dWr[h,e]      = sum_t x[t,h] * dl[t,e]
 *     dx_router[t,h] = sum_e dl[t,e] * Wr[h,e].
 * Each output is one plain sum in index order.                               */
void oracle_router_backward(int T, int H, int E, int k, const double* x, const double* Wr, const int32_t* idx,
                            const double* w, const double* dg, double* dlogits, double* dWr, double* dx_router) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += w[(size_t)t * k + j] * dg[(size_t)t * k + j];
    for (int e = 0; e < E; ++e) dlogits[(size_t)t * E + e] = 0.0;
    for (int j = 0; j < k; ++j) {
      const size_t p = (size_t)t * k + j;
      dlogits[(size_t)t * E + idx[p]] = w[p] * (dg[p] - s);
    }
  }
#pragma omp parallel for schedule(static)
  for (int h = 0; h < H; ++h)
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int t = 0; t < T; ++t) s += x[(size_t)t * H + h] * dlogits[(size_t)t * E + e];
      dWr[(size_t)h * E + e] = s;
    }
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int h = 0; h < H; ++h) {
      double s = 0.0;
      for (int e = 0; e < E; ++e) s += dlogits[(size_t)t * E + e] * Wr[(size_t)h * E + e];
      dx_router[(size_t)t * H + h] = s;
    }
}

/* ------------------------------------------------------------------------- */
/* Top-k routing (issue #14, Evidence/Proposal).  For each token the experts are
 * ordered by (logit descending, expert index ascending) -- a full stable sort,
 * written as an insertion sort -- and the first k are kept.  Weights are the
 * softmax over the k selected logits:
 *     w[t,j] = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 * which equals a softmax over all E renormalised to the selected k.
 * The pages say nothing of NaN logits.  Reading taken: a NaN ranks above every
 * number (the order of torch's sort and top-k), NaNs among themselves by the
 * lower expert index; a token with a NaN logit then selects it first and all
 * its weights are NaN.  +0.0 and -0.0 are equal.                             */
static int ranks_above(double a, double b) {
  if (isnan(a)) return !isnan(b);
  if (isnan(b)) return 0;
  return a > b;
}

void oracle_route_topk(int T, int E, int k, const double* logits, int32_t* idx, double* w) {
#pragma omp parallel
  {
    int* order = (int*)malloc(sizeof(int) * (size_t)E);
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
      const double* l = logits + (size_t)t * E;
      for (int e = 0; e < E; ++e) {
        /* insert e after every earlier expert whose logit l[e] does not rank above */
        int pos = e;
        while (pos > 0 && ranks_above(l[e], l[order[pos - 1]])) {
          order[pos] = order[pos - 1];
          --pos;
        }
        order[pos] = e;
      }
      double denom = 0.0;
      for (int j = 0; j < k; ++j) denom += exp(l[order[j]] - l[order[0]]);
      for (int j = 0; j < k; ++j) {
        idx[(size_t)t * k + j] = order[j];
        w[(size_t)t * k + j] = exp(l[order[j]] - l[order[0]]) / denom;
      }
    }
    free(order);
  }
}

/* ------------------------------------------------------------------------- */
/* Dispatch (issue #14, Proposal: rows grouped per expert).  Pair id p = t*k+j.
 * For each expert in ascending order, append every pair routed to it in
 * ascending p.  perm[s] is the pair at sorted position s; inv_perm inverts it.
 * Returns 0, or -1 if an index is out of range.                              */
int oracle_dispatch(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                    int32_t* perm, int32_t* inv_perm) {
  const int64_t N = (int64_t)T * k;
  for (int64_t p = 0; p < N; ++p)
    if (idx[p] < 0 || idx[p] >= E) return -1;
  int64_t s = 0;
  for (int e = 0; e < E; ++e) {
    offsets[e] = (int32_t)s;
    for (int64_t p = 0; p < N; ++p)
      if (idx[p] == e) perm[s++] = (int32_t)p;
    counts[e] = (int32_t)(s - offsets[e]);
  }
  offsets[E] = (int32_t)s;
  for (int64_t q = 0; q < N; ++q) inv_perm[perm[q]] = (int32_t)q;
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Pair scores for the quota selection (LRMoE abstract: retention guided by
 * each pair's contribution to the expert update).  The pages leave the metric
 * open; the one taken here is available before any backward GEMM: the
 * Frobenius norm of pair p's rank-one term in dW_down,
 *     score_p = || a_p (w_p dy_t)^T ||_F = w_p * ||a_p||_2 * ||dy_t||_2,
 * with a_p the pair's SwiGLU activation [F] and t its token.                 */
void oracle_pair_scores(int T, int H, int F, int k, const double* a_pairs, const double* dy, const double* w,
                        double* score) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    double sdy = 0.0;
    for (int h = 0; h < H; ++h) sdy += dy[(size_t)t * H + h] * dy[(size_t)t * H + h];
    for (int j = 0; j < k; ++j) {
      const size_t p = (size_t)t * k + j;
      double sa = 0.0;
      for (int f = 0; f < F; ++f) sa += a_pairs[p * F + f] * a_pairs[p * F + f];
      score[p] = w[p] * sqrt(sa) * sqrt(sdy);
    }
  }
}

/* Quota from a memory budget (LRMoE abstract: quotas planned from the memory a
 * node has for backward work).  A retained row holds dO [H], dh [2F], dX [H] and
 * the compacted copy of x [H], plus h [2F] when the forward's pre-activations
 * are kept and a [F] when dW is computed, each of elem_bytes.  The cap is the
 * largest per-expert quota whose worst case (every expert at its cap) fits:
 *     cap = floor(budget / (E * row_bytes)),  at most ceil(T k / E);
 * -1 when not even one row per expert fits.                                 */
int64_t oracle_quota_cap_for_budget(int T, int H, int F, int E, int k, int elem_bytes, int with_dw, int keep_graph,
                                    double budget_bytes) {
  const double row_bytes = (double)elem_bytes * (3.0 * H + 2.0 * F + (keep_graph ? 2.0 * F : 0.0) +
                                                 (with_dw ? (double)F : 0.0));
  const double cap = floor(budget_bytes / ((double)E * row_bytes));
  if (cap < 1.0) return -1;
  const int64_t most = ((int64_t)T * k + E - 1) / E;
  return cap < (double)most ? (int64_t)cap : most;
}

/* ------------------------------------------------------------------------- */
/* Retention quota (LRMoE abstract: quotas planned during forward).  The
 * per-expert quota is q_e = min(count_e, cap) with cap = ceil(rho * T * k / E);
 * rho = 1 is evaluated in integers.                                          */
int64_t oracle_quota_cap(int T, int E, int k, double rho) {
  if (rho == 1.0) return ((int64_t)T * k + E - 1) / E;
  return (int64_t)ceil(rho * (double)T * (double)k / (double)E);
}

typedef struct {
  double score;
  int32_t p;
} scored_pair;

static int by_score_desc_p_asc(const void* a, const void* b) {
  const scored_pair* x = (const scored_pair*)a;
  const scored_pair* y = (const scored_pair*)b;
  if (x->score > y->score) return -1;
  if (x->score < y->score) return 1;
  return (x->p < y->p) ? -1 : (x->p > y->p);
}

/* Selection within quotas and physical compaction (LRMoE abstract).  The score
 * of pair p is score[p] (pair-indexed).  Each expert keeps its q_e pairs with
 * the largest (score, then lower p); kept pairs stay in ascending p within the
 * expert.  Outputs: kept_counts[E], kept_offsets[E+1], kept_perm[R] (pair id),
 * kept_src[R] (position in the uncompacted sorted order), kept_inv[N]
 * (compacted position, or -1 when dropped), retained[N] (0/1).  Returns R.   */
int64_t oracle_compact(int T, int E, int k, const int32_t* counts, const int32_t* offsets,
                       const int32_t* perm, const double* score, double rho, int32_t* kept_counts,
                       int32_t* kept_offsets, int32_t* kept_perm, int32_t* kept_src, int32_t* kept_inv,
                       uint8_t* retained) {
  const int64_t N = (int64_t)T * k;
  const int64_t cap = oracle_quota_cap(T, E, k, rho);
  for (int64_t p = 0; p < N; ++p) {
    retained[p] = 0;
    kept_inv[p] = -1;
  }
  int64_t r = 0;
  for (int e = 0; e < E; ++e) {
    const int n = counts[e];
    const int64_t q = n < cap ? n : cap;
    scored_pair* list = (scored_pair*)malloc(sizeof(scored_pair) * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < n; ++i) {
      list[i].p = perm[offsets[e] + i];
      list[i].score = score[list[i].p];
    }
    qsort(list, (size_t)n, sizeof(scored_pair), by_score_desc_p_asc);
    for (int64_t i = 0; i < q; ++i) retained[list[i].p] = 1;
    free(list);
    kept_offsets[e] = (int32_t)r;
    for (int i = 0; i < n; ++i) {
      const int32_t p = perm[offsets[e] + i];
      if (retained[p]) {
        kept_perm[r] = p;
        kept_src[r] = offsets[e] + i;
        kept_inv[p] = (int32_t)r;
        ++r;
      }
    }
    kept_counts[e] = (int32_t)(r - kept_offsets[e]);
  }
  kept_offsets[E] = (int32_t)r;
  return r;
}

/* ------------------------------------------------------------------------- */
/* One SwiGLU expert on one token row (issue #14, Proposal: expert forward):
 *   hg[f] = sum_h x[h] Wg[e,h,f],  hu[f] = sum_h x[h] Wu[e,h,f]
 *   a[f]  = silu(hg[f]) * hu[f],   silu(z) = z * sigmoid(z)
 *   o[h]  = sum_f a[f] Wd[e,f,h]
 * Weights are row-major Wg, Wu [E,H,F] and Wd [E,F,H].                       */
static void expert_forward(int H, int F, const double* xt, const double* Wg, const double* Wu,
                           const double* Wd, double* hg, double* hu, double* a, double* o) {
  for (int f = 0; f < F; ++f) {
    double sg = 0.0, su = 0.0;
    for (int h = 0; h < H; ++h) {
      sg += xt[h] * Wg[(size_t)h * F + f];
      su += xt[h] * Wu[(size_t)h * F + f];
    }
    hg[f] = sg;
    hu[f] = su;
    a[f] = sg * sigmoid(sg) * su;
  }
  for (int h = 0; h < H; ++h) {
    double s = 0.0;
    for (int f = 0; f < F; ++f) s += a[f] * Wd[(size_t)f * H + h];
    o[h] = s;
  }
}

/* Forward of the layer for a list of tokens (all tokens when toks == NULL):
 *   y[t,:] = sum_{j ascending} w[t,j] * Expert_{idx[t,j]}(x[t,:])
 * Optional pair-indexed intermediates: hg, hu, a [N,F] and o [N,H].          */
void oracle_forward(int T, int H, int F, int E, int k, const double* x, const int32_t* idx,
                    const double* w, const double* Wg, const double* Wu, const double* Wd, int n_tok,
                    const int32_t* toks, double* y, double* hg_out, double* hu_out, double* a_out,
                    double* o_out) {
  (void)E;
  const int count = toks ? n_tok : T;
#pragma omp parallel
  {
    double* hg = (double*)malloc(sizeof(double) * (size_t)F);
    double* hu = (double*)malloc(sizeof(double) * (size_t)F);
    double* a = (double*)malloc(sizeof(double) * (size_t)F);
    double* o = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < count; ++i) {
      const int t = toks ? toks[i] : i;
      const double* xt = x + (size_t)t * H;
      double* yt = y + (size_t)t * H;
      for (int h = 0; h < H; ++h) yt[h] = 0.0;
      for (int j = 0; j < k; ++j) {
        const int64_t p = (int64_t)t * k + j;
        const int e = idx[p];
        expert_forward(H, F, xt, Wg + (size_t)e * H * F, Wu + (size_t)e * H * F,
                       Wd + (size_t)e * F * H, hg, hu, a, o);
        for (int h = 0; h < H; ++h) yt[h] += w[p] * o[h];
        if (hg_out) memcpy(hg_out + (size_t)p * F, hg, sizeof(double) * (size_t)F);
        if (hu_out) memcpy(hu_out + (size_t)p * F, hu, sizeof(double) * (size_t)F);
        if (a_out) memcpy(a_out + (size_t)p * F, a, sizeof(double) * (size_t)F);
        if (o_out) memcpy(o_out + (size_t)p * H, o, sizeof(double) * (size_t)H);
      }
    }
    free(hg);
    free(hu);
    free(a);
    free(o);
  }
}

/* Backward of one pair with routing held fixed (issue #14, Proposal/Scope:
 * backward dx, and dW for full fine-tuning).  With dO = w * dy[t]:
 *   dA[f]  = sum_h dO[h] Wd[e,f,h]
 *   dHg[f] = dA[f] * hu[f] * s * (1 + hg[f] * (1 - s)),  s = sigmoid(hg[f])
 *   dHu[f] = dA[f] * hg[f] * s
 *   dX[h]  = sum_f dHg[f] Wg[e,h,f] + dHu[f] Wu[e,h,f]
 * (d/dz silu(z) = s * (1 + z * (1 - s)).)                                     */
static void expert_backward(int H, int F, double wp, const double* dyt, const double* Wg,
                            const double* Wu, const double* Wd, const double* hg, const double* hu,
                            double* dO, double* dHg, double* dHu, double* dX) {
  for (int h = 0; h < H; ++h) dO[h] = wp * dyt[h];
  for (int f = 0; f < F; ++f) {
    double dA = 0.0;
    for (int h = 0; h < H; ++h) dA += dO[h] * Wd[(size_t)f * H + h];
    const double s = sigmoid(hg[f]);
    dHg[f] = dA * hu[f] * s * (1.0 + hg[f] * (1.0 - s));
    dHu[f] = dA * hg[f] * s;
  }
  for (int h = 0; h < H; ++h) {
    double sx = 0.0;
    for (int f = 0; f < F; ++f) sx += dHg[f] * Wg[(size_t)h * F + f] + dHu[f] * Wu[(size_t)h * F + f];
    dX[h] = sx;
  }
}

/* Input gradient and router-weight gradient for a list of tokens (all when
 * toks == NULL).  dg[t,j] = <dy[t], o_p> for every pair; dx[t] sums dX over the
 * token's retained pairs only (retained == NULL keeps every pair), in
 * ascending j.  Optional pair-indexed intermediates: dO [N,H], dh [N,2F] laid
 * out as [dHg | dHu], dX [N,H]; rows of dropped pairs are left untouched.      */
void oracle_backward(int T, int H, int F, int E, int k, const double* x, const int32_t* idx,
                     const double* w, const double* Wg, const double* Wu, const double* Wd,
                     const double* dy, const uint8_t* retained, int n_tok, const int32_t* toks,
                     double* dx, double* dg, double* dO_out, double* dh_out, double* dX_out) {
  (void)E;
  const int count = toks ? n_tok : T;
#pragma omp parallel
  {
    double* hg = (double*)malloc(sizeof(double) * (size_t)F);
    double* hu = (double*)malloc(sizeof(double) * (size_t)F);
    double* a = (double*)malloc(sizeof(double) * (size_t)F);
    double* o = (double*)malloc(sizeof(double) * (size_t)H);
    double* dO = (double*)malloc(sizeof(double) * (size_t)H);
    double* dHg = (double*)malloc(sizeof(double) * (size_t)F);
    double* dHu = (double*)malloc(sizeof(double) * (size_t)F);
    double* dX = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int i = 0; i < count; ++i) {
      const int t = toks ? toks[i] : i;
      const double* xt = x + (size_t)t * H;
      const double* dyt = dy + (size_t)t * H;
      double* dxt = dx + (size_t)t * H;
      for (int h = 0; h < H; ++h) dxt[h] = 0.0;
      for (int j = 0; j < k; ++j) {
        const int64_t p = (int64_t)t * k + j;
        const int e = idx[p];
        const double* wg = Wg + (size_t)e * H * F;
        const double* wu = Wu + (size_t)e * H * F;
        const double* wd = Wd + (size_t)e * F * H;
        expert_forward(H, F, xt, wg, wu, wd, hg, hu, a, o);
        double g = 0.0;
        for (int h = 0; h < H; ++h) g += dyt[h] * o[h];
        dg[p] = g;
        if (retained && !retained[p]) continue;
        expert_backward(H, F, w[p], dyt, wg, wu, wd, hg, hu, dO, dHg, dHu, dX);
        for (int h = 0; h < H; ++h) dxt[h] += dX[h];
        if (dO_out) memcpy(dO_out + (size_t)p * H, dO, sizeof(double) * (size_t)H);
        if (dh_out) {
          memcpy(dh_out + (size_t)p * 2 * F, dHg, sizeof(double) * (size_t)F);
          memcpy(dh_out + (size_t)p * 2 * F + F, dHu, sizeof(double) * (size_t)F);
        }
        if (dX_out) memcpy(dX_out + (size_t)p * H, dX, sizeof(double) * (size_t)H);
      }
    }
    free(hg);
    free(hu);
    free(a);
    free(o);
    free(dO);
    free(dHg);
    free(dHu);
    free(dX);
  }
}

/* Full weight gradients of every expert (issue #14, Scope: dW for full FT),
 * summed over the retained pairs routed to it, in ascending p:
 *   dWd[e,f,h] = sum_p a_p[f] dO_p[h]
 *   dWg[e,h,f] = sum_p x_t[h] dHg_p[f],  dWu[e,h,f] = sum_p x_t[h] dHu_p[f]
 * An expert with no retained pair gets exact zeros.  Parallel over experts.  */
void oracle_backward_dw(int T, int H, int F, int E, int k, const double* x, const int32_t* idx,
                        const double* w, const double* Wg, const double* Wu, const double* Wd,
                        const double* dy, const uint8_t* retained, double* dWg, double* dWu,
                        double* dWd) {
  const int64_t N = (int64_t)T * k;
#pragma omp parallel
  {
    double* hg = (double*)malloc(sizeof(double) * (size_t)F);
    double* hu = (double*)malloc(sizeof(double) * (size_t)F);
    double* a = (double*)malloc(sizeof(double) * (size_t)F);
    double* o = (double*)malloc(sizeof(double) * (size_t)H);
    double* dO = (double*)malloc(sizeof(double) * (size_t)H);
    double* dHg = (double*)malloc(sizeof(double) * (size_t)F);
    double* dHu = (double*)malloc(sizeof(double) * (size_t)F);
    double* dX = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(dynamic, 1)
    for (int e = 0; e < E; ++e) {
      double* gWg = dWg + (size_t)e * H * F;
      double* gWu = dWu + (size_t)e * H * F;
      double* gWd = dWd + (size_t)e * F * H;
      memset(gWg, 0, sizeof(double) * (size_t)H * F);
      memset(gWu, 0, sizeof(double) * (size_t)H * F);
      memset(gWd, 0, sizeof(double) * (size_t)F * H);
      const double* wg = Wg + (size_t)e * H * F;
      const double* wu = Wu + (size_t)e * H * F;
      const double* wd = Wd + (size_t)e * F * H;
      for (int64_t p = 0; p < N; ++p) {
        if (idx[p] != e) continue;
        if (retained && !retained[p]) continue;
        const double* xt = x + (size_t)(p / k) * H;
        const double* dyt = dy + (size_t)(p / k) * H;
        expert_forward(H, F, xt, wg, wu, wd, hg, hu, a, o);
        expert_backward(H, F, w[p], dyt, wg, wu, wd, hg, hu, dO, dHg, dHu, dX);
        for (int f = 0; f < F; ++f)
          for (int h = 0; h < H; ++h) gWd[(size_t)f * H + h] += a[f] * dO[h];
        for (int h = 0; h < H; ++h)
          for (int f = 0; f < F; ++f) {
            gWg[(size_t)h * F + f] += xt[h] * dHg[f];
            gWu[(size_t)h * F + f] += xt[h] * dHu[f];
          }
      }
    }
    free(hg);
    free(hu);
    free(a);
    free(o);
    free(dO);
    free(dHg);
    free(dHu);
    free(dX);
  }
}

/* Single entries of the weight gradients, one by one, for layers too large to
 * differentiate whole.  Query i asks for matrix mat[i] (0 = dW_gate[e,r,c],
 * 1 = dW_up[e,r,c], 2 = dW_down[e,r,c]) of expert e[i]; the sum runs over the
 * expert's retained pairs in ascending p with the same per-pair terms as
 * oracle_backward_dw, evaluating only the feature that the entry needs.       */
void oracle_dw_entries(int T, int H, int F, int E, int k, const double* x, const int32_t* idx,
                       const double* w, const double* Wg, const double* Wu, const double* Wd,
                       const double* dy, const uint8_t* retained, int n_q, const int32_t* q_e,
                       const int32_t* q_mat, const int32_t* q_r, const int32_t* q_c, double* out) {
  (void)E;
  const int64_t N = (int64_t)T * k;
#pragma omp parallel for schedule(dynamic, 1)
  for (int i = 0; i < n_q; ++i) {
    const int e = q_e[i], mat = q_mat[i], r = q_r[i], c = q_c[i];
    const double* wg = Wg + (size_t)e * H * F;
    const double* wu = Wu + (size_t)e * H * F;
    const double* wd = Wd + (size_t)e * F * H;
    /* feature index f of the entry: dW_down[f,h] -> f = r; dW_gate/up[h,f] -> f = c */
    const int f = (mat == 2) ? r : c;
    double acc = 0.0;
    for (int64_t p = 0; p < N; ++p) {
      if (idx[p] != e) continue;
      if (retained && !retained[p]) continue;
      const double* xt = x + (size_t)(p / k) * H;
      const double* dyt = dy + (size_t)(p / k) * H;
      double hg = 0.0, hu = 0.0;
      for (int h = 0; h < H; ++h) {
        hg += xt[h] * wg[(size_t)h * F + f];
        hu += xt[h] * wu[(size_t)h * F + f];
      }
      const double s = sigmoid(hg);
      if (mat == 2) {
        const double a = hg * s * hu;
        acc += a * (w[p] * dyt[c]);
      } else {
        double dA = 0.0;
        for (int h = 0; h < H; ++h) dA += (w[p] * dyt[h]) * wd[(size_t)f * H + h];
        const double d = (mat == 0) ? dA * hu * s * (1.0 + hg * (1.0 - s)) : dA * hg * s;
        acc += xt[r] * d;
      }
    }
    out[i] = acc;
  }
}

/* ------------------------------------------------------------------------- */
/* fp8 storage of frozen expert weights.  The experts are frozen in the LoRA
 * step (issue #14, Scope) and their weights stay resident on the device
 * (issue #14, Proposal), so they can be stored once in 8 bits.  The pages fix
 * no format; the element format is OCP 8-bit floating point E4M3 ("E4M3FN":
 * 1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
 * infinities, S.1111.111 = NaN, largest finite 448), and each expert keeps one
 * power-of-two scale shared by its W_gate and W_up (and one for W_down).
 *
 * Decoding is the format's definition. */
double oracle_e4m3_decode(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* Encoding: round to nearest, ties to the even mantissa, values beyond 448 in
 * magnitude saturate to 448, NaN to S.1111.111.  Every step below is exact in
 * double for the inputs it receives, so rint() alone decides the rounding. */
uint8_t oracle_e4m3_encode(double v) {
  if (isnan(v)) return 0x7F;
  const uint8_t sign = signbit(v) ? 0x80 : 0x00;
  const double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) {  /* subnormal range: multiples of 2^-9 (8 * 2^-9 is the smallest normal) */
    const int q = (int)rint(ldexp(a, 9));
    return sign | (uint8_t)q;
  }
  int e2;
  const double f = frexp(a, &e2); /* a = f 2^e2, f in [0.5, 1) */
  int e = e2 - 1;                   /* a = (2 f) 2^e, 2 f in [1, 2) */
  int m = (int)rint((2.0 * f - 1.0) * 8.0);
  if (m == 8) {
    m = 0;
    ++e;
  }
  const int code = ((e + 7) << 3) | m;
  return sign | (uint8_t)(code > 0x7E ? 0x7E : code);
}

/* The scale of one expert: the smallest power of two s with amax <= 448 s,
 * amax the largest magnitude over the expert's matrices (s = 1 when all are
 * zero).  Returns log2(s). */
int oracle_fp8_scale_exp(double amax) {
  if (!(amax > 0.0)) return 0;
  int k;
  (void)frexp(amax, &k);
  k -= 9; /* a start near the answer (448 is just under 2^9); the loops make it exact */
  while (448.0 * ldexp(1.0, k) < amax) ++k;
  while (448.0 * ldexp(1.0, k - 1) >= amax) --k;
  return k;
}

/* Quantize E experts' matrices: w0 [E][n0] and optionally w1 [E][n1] share
 * one scale per expert; q = E4M3(w / s), scale[e] = s. */
void oracle_quantize_fp8(int E, int64_t n0, const double* w0, int64_t n1, const double* w1, uint8_t* q0, uint8_t* q1,
                         double* scale) {
  for (int e = 0; e < E; ++e) {
    double amax = 0.0;
    for (int64_t i = 0; i < n0; ++i) amax = fmax(amax, fabs(w0[(size_t)e * n0 + i]));
    if (w1)
      for (int64_t i = 0; i < n1; ++i) amax = fmax(amax, fabs(w1[(size_t)e * n1 + i]));
    const int k = oracle_fp8_scale_exp(amax);
    scale[e] = ldexp(1.0, k);
    for (int64_t i = 0; i < n0; ++i) q0[(size_t)e * n0 + i] = oracle_e4m3_encode(ldexp(w0[(size_t)e * n0 + i], -k));
    if (w1)
      for (int64_t i = 0; i < n1; ++i) q1[(size_t)e * n1 + i] = oracle_e4m3_encode(ldexp(w1[(size_t)e * n1 + i], -k));
  }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------------- */
/* Round to the nearest bf16 value (8 significant bits, ties to even; bf16 has
 * fp32's exponent range, so below 2^-126 the quantum is fixed at 2^-133).    */
static double round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  if (fabs(v) < ldexp(1.0, -126)) return ldexp(nearbyint(ldexp(v, 133)), -133);
  int ex;
  const double m = frexp(v, &ex); /* v = m 2^ex, 0.5 <= |m| < 1 */
  return ldexp(nearbyint(ldexp(m, 8)), ex - 8);
}

/* Expert forward on fp8 (E4M3) operands: the grouped GEMMs run on the fp8
 * matrix cores (LRMoE abstract: variable-size grouped GEMMs; the pages fix no
 * precision).  Reading taken: every operand of both products is E4M3 with one
 * power-of-two scale per row of activations (per token for x, per pair for a)
 * and per expert for the weights (the rule of oracle_quantize_fp8), products
 * accumulated exactly; the SwiGLU output is stored in bf16 as in the bf16 path
 * and that stored value is what gets quantized for the down product.  Per token
 * t and slot j (e = idx[t,j]), on the decoded inputs xd [T,H] and weights Wgd,
 * Wud [E,H,F], Wdd [E,F,H]:
 *     hg[f] = sum_h xd[t,h] Wgd[e,h,f],  hu[f] = sum_h xd[t,h] Wud[e,h,f]
 *     a16[f] = bf16(silu(hg[f]) hu[f])
 *     s = 2^oracle_fp8_scale_exp(max_f |a16[f]|),  aq[f] = E4M3(a16[f] / s)
 *     o[h] = sum_f decode(aq[f]) s Wdd[e,f,h],   y[t,h] += w[t,j] o[h]  (j ascending)
 * Outputs (pair-indexed p = t k + j, each optional): hg, hu, a16 [N,F]; aq
 * [N,F] codes and ascale [N]; o [N,H].                                       */
void oracle_forward_fp8(int T, int H, int F, int E, int k, const double* xd, const int32_t* idx, const double* w,
                        const double* Wgd, const double* Wud, const double* Wdd, double* y, double* hg_out,
                        double* hu_out, double* a_out, uint8_t* aq_out, double* ascale_out, double* o_out) {
  (void)E;
#pragma omp parallel
  {
    double* hg = (double*)malloc(sizeof(double) * (size_t)F);
    double* hu = (double*)malloc(sizeof(double) * (size_t)F);
    double* a = (double*)malloc(sizeof(double) * (size_t)F);
    uint8_t* q = (uint8_t*)malloc((size_t)F);
    double* o = (double*)malloc(sizeof(double) * (size_t)H);
#pragma omp for schedule(static)
    for (int t = 0; t < T; ++t) {
      for (int h = 0; h < H; ++h) y[(size_t)t * H + h] = 0.0;
      for (int j = 0; j < k; ++j) {
        const size_t p = (size_t)t * k + j;
        const int e = idx[p];
        const double* wg = Wgd + (size_t)e * H * F;
        const double* wu = Wud + (size_t)e * H * F;
        const double* wd = Wdd + (size_t)e * F * H;
        for (int f = 0; f < F; ++f) {
          double sg = 0.0, su = 0.0;
          for (int h = 0; h < H; ++h) {
            sg += xd[(size_t)t * H + h] * wg[(size_t)h * F + f];
            su += xd[(size_t)t * H + h] * wu[(size_t)h * F + f];
          }
          hg[f] = sg;
          hu[f] = su;
          a[f] = round_bf16(sg / (1.0 + exp(-sg)) * su);
        }
        double amax = 0.0;
        for (int f = 0; f < F; ++f) amax = fmax(amax, fabs(a[f]));
        const int ks = oracle_fp8_scale_exp(amax);
        for (int f = 0; f < F; ++f) q[f] = oracle_e4m3_encode(ldexp(a[f], -ks));
        for (int h = 0; h < H; ++h) {
          double sum = 0.0;
          for (int f = 0; f < F; ++f) sum += ldexp(oracle_e4m3_decode(q[f]), ks) * wd[(size_t)f * H + h];
          o[h] = sum;
          y[(size_t)t * H + h] += w[p] * sum;
        }
        if (hg_out)
          for (int f = 0; f < F; ++f) hg_out[p * F + f] = hg[f];
        if (hu_out)
          for (int f = 0; f < F; ++f) hu_out[p * F + f] = hu[f];
        if (a_out)
          for (int f = 0; f < F; ++f) a_out[p * F + f] = a[f];
        if (aq_out)
          for (int f = 0; f < F; ++f) aq_out[p * F + f] = q[f];
        if (ascale_out) ascale_out[p] = ldexp(1.0, ks);
        if (o_out)
          for (int h = 0; h < H; ++h) o_out[p * H + h] = o[h];
      }
    }
    free(hg);
    free(hu);
    free(a);
    free(q);
    free(o);
  }
}

