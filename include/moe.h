/*
 * moe.h -- C ABI of libmoe: one MoE layer's expert computation in training on
 * one AMD Instinct MI355X (gfx950), as hand-written HIP kernels.
 *
 * The path (pages: npu-train issue #14 "[MoE] Hot experts on RNGD during
 * training (host dispatch, device expert graphs)", sections Evidence, Proposal
 * and Scope; npu-train pull request #44, section Changes; LRMoE,
 * arXiv:2610.37720, abstract):
 *
 *   moe_router_fwd          router logits = x W_r
 *   moe_route_topk          router logits -> top-k experts and weights per token
 *   moe_dispatch            token-expert pairs -> rows contiguous per expert
 *   moe_grouped_swiglu_fwd  SwiGLU expert MLP over every expert's rows (ragged
 *                           grouped GEMM); keeps the activations backward needs
 *   moe_grouped_swiglu_fwd_gather  the same with the rows gathered on load
 *   moe_grouped_swiglu_recompute  the forward's pre-activations again, for a
 *                           forward that did not keep them
 *   moe_combine             router-weighted sum of each token's expert rows
 *   moe_compact_pairs       keep at most a quota of pairs per expert and gather
 *                           their rows into smaller contiguous buffers
 *   moe_grouped_bwd_dx      input gradient (experts frozen) + routing-weight
 *                           gradient, over all or only the retained pairs
 *   moe_pair_scores         per-pair scores for the quota selection
 *   moe_grouped_bwd_dw      expert weight gradients (full fine-tuning)
 *   moe_router_bwd          router gradients (logits, W_r, the router's share
 *                           of dx) from the routing-weight gradient
 *   moe_quantize_weights_fp8, moe_grouped_swiglu_fwd_fp8w,
 *   moe_grouped_bwd_dx_fp8w frozen expert weights stored once in fp8 (E4M3),
 *                           and the forward and dx backward reading them
 *
 * Conventions for every call:
 *  - Pointers marked (device) are device pointers owned by the caller; the
 *    library allocates no memory and keeps no pointer after a call returns
 *    (its one device array, moe_dispatch_noalloc's workspace, is static).
 *  - `stream` is a hipStream_t (NULL = the default stream).  A call only
 *    enqueues work on it: no device synchronisation, no device-to-host copy.
 *    Data-dependent sizes (row counts, offsets, the retained total) stay on the
 *    device; the host passes capacities only.
 *  - Arguments are validated before anything is enqueued; on any error nothing
 *    is enqueued and the status says why (moe_last_error() has the detail).
 *  - dtype: MOE_F32 or MOE_BF16 for activations and weights (all of one call
 *    are of that dtype); logits, routing weights, scores and dg are always
 *    fp32; indices int32.  Accumulation is fp32; bf16 results are rounded to
 *    nearest even once, at the store.
 *  - Layouts are row-major.  Pair id p = t*k + j (token t, slot j of its top-k).
 *    Expert weights: W_gate and W_up [E, H, F], W_down [E, F, H].
 *  - Limits: 1 <= k <= E <= 256, k <= 16, T*k < 2^31, H and F multiples of 8
 *    (any dtype; widths that are not multiples of the kernels' tiles run on
 *    the same kernels with the reduction and column tails masked).
 *  - Results are deterministic: the same inputs on the same GPU give bitwise
 *    identical outputs (no order-dependent atomics).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, k > E, ... */
  MOE_ERR_UNSUPPORTED = 2,        /* outside the limits above */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4                 /* a HIP launch failed; see moe_last_error() */
} moe_status;

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Static text for a status code. */
const char* moe_status_string(int status);
/* Detail of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);
/* ABI version, currently 8. */
int moe_abi_version(void);

/* Kernel launches made so far by library calls from the calling thread (a
 * debug counter; it never resets).  Every call launches a fixed number of
 * kernels given by its arguments alone (a call rejected by validation
 * launches none); with Nk = T*k pairs, R = max_rows and B = 1 when experts
 * of 256 rows and more get the 256-row kernel for a product (bf16, the
 * expert-row bound of the call and R both >= 256), else 0:
 *   moe_route_topk                          1
 *   moe_dispatch, moe_dispatch_noalloc      (Nk <= 1024 ? 1 : 3) + (x_sorted ? 1 : 0)
 *   moe_grouped_swiglu_fwd[_gather]         R = 0: 0; bf16: 2 + 2 B with the
 *                                           bound max_expert_rows; fp32: 2
 *   moe_grouped_swiglu_fwd_fp8w             R = 0: 0; else 2
 *   moe_grouped_swiglu_recompute            R = 0: 0; bf16: 1 + B; fp32: 1
 *   moe_combine                             1
 *   moe_grouped_bwd_dx                      2 + (R > 0 ? 2 + B + B_dA : 0), bound min(R, T),
 *                                           B_dA = B when F >= 1024, else 0
 *                                           (fp32 and fp8 weights: B = B_dA = 0)
 *   moe_grouped_bwd_dw                      bf16: 2; fp32: 1
 *   moe_compact_pairs[_cap]                 2 + (any row source given ? 1 : 0)
 *   moe_pair_scores, moe_quantize_weights_fp8, moe_quantize_rows_fp8,
 *   moe_transpose_fp8                       1
 *   moe_grouped_swiglu_fwd_fp8              R = 0: 0; else 3
 *   moe_router_fwd                          1, plus 1 when its workspace is used
 *   moe_router_bwd                          3, plus 1 when its dW_r reduction is split
 * These counts are what a HIP graph of a layer step captures. */
int64_t moe_launch_count(void);

/* Kernels that moe_profile_kernel can bracket with events. */
typedef enum moe_kernel {
  MOE_K_ROUTE = 0,         /* moe_route_topk */
  MOE_K_DISPATCH_ROWS = 1, /* the row copy of moe_dispatch */
  MOE_K_GEMM_GATEUP = 2,   /* gate/up GEMM + SwiGLU of moe_grouped_swiglu_fwd */
  MOE_K_GEMM_DOWN = 3,     /* down GEMM of moe_grouped_swiglu_fwd */
  MOE_K_COMBINE = 4,       /* moe_combine, and the dx sum of moe_grouped_bwd_dx */
  MOE_K_GRAD_ROWS = 5,     /* dO rows and dg of moe_grouped_bwd_dx */
  MOE_K_GEMM_DA = 6,       /* dA GEMM + SwiGLU backward of moe_grouped_bwd_dx */
  MOE_K_GEMM_DX = 7,       /* dX GEMM of moe_grouped_bwd_dx */
  MOE_K_GEMM_DW = 8,       /* moe_grouped_bwd_dw */
  MOE_K_COMPACT = 9,       /* the selection kernel of moe_compact_pairs */
  MOE_K_ROUTER_FWD = 10,   /* moe_router_fwd */
  MOE_K_ROUTER_DW = 11,    /* the dW_r GEMM of moe_router_bwd */
  MOE_K_COUNT = 12
} moe_kernel;

/* Profiling hook.  Arms a one-shot request on the calling thread: the next
 * launch of `kernel` made from this thread (one or more kernel dispatches)
 * carries the events in its own dispatches -- the first dispatch records
 * `start_event` as it begins, every dispatch records `stop_event` as it ends --
 * so hipEventElapsedTime(start, stop) is that kernel's duration and no extra
 * packet is queued between kernels; a launch that dispatches nothing records
 * both on its stream.  Both events are hipEvent_t created by the caller, with
 * timing enabled; NULL events disarm.  Several kernels may be armed at once.
 * Results of the calls are unaffected. */
int moe_profile_kernel(int kernel, void* start_event, void* stop_event);

/* Fork point between the input gradient and the weight gradients (issue #14,
 * Scope: dW for full fine-tuning reads the same dO and dh rows as dx).  Arms a
 * one-shot request on the calling thread: the next moe_grouped_bwd_dx or
 * moe_grouped_bwd_dx_fp8w call made from this thread records `event` (a
 * hipEvent_t created by the caller) on its stream as soon as dO_rows and
 * dh_rows are complete, that is after the dA GEMM and before the dX GEMM.  A
 * moe_grouped_bwd_dw launched on another stream that waits for the event then
 * runs alongside dX and the dx sum; the caller joins the streams afterwards.
 * The next call takes the request whatever its outcome (one that fails
 * records nothing).  NULL disarms.  Results are unaffected.  Returns MOE_OK. */
int moe_signal_dh_ready(void* event);

/* Workspace (device bytes) that moe_router_fwd and moe_router_bwd need for T
 * tokens, hidden size H and E experts: fp32 partial sums of the long
 * reductions (at most ~8.5 MB; 0 when no reduction is split).  Host-only. */
size_t moe_router_workspace_bytes(int T, int H, int E);

/* Router logits (issue #14, Proposal: routing precedes dispatch):
 *   logits[t,e] = sum_h x[t,h] W_r[h,e]
 * accumulated in fp32 in one fixed order.  x [T, H] and w_r [H, E] of `dtype`
 * (device); logits [T, E] fp32 (device, out); workspace (device) of at least
 * moe_router_workspace_bytes(T, H, E) bytes (may be NULL when that is 0).
 * 1 <= E <= 256; H a multiple of 8. */
int moe_router_fwd(int T, int H, int E, int dtype, const void* x, const void* w_r, float* logits, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Top-k routing (issue #14, Evidence and Proposal: each token is routed to k
 * of E experts).  For token t the experts are ranked by logit descending, equal
 * logits by lower expert index (+0.0 equals -0.0); topk_idx[t, 0..k) lists the
 * first k in that order.  The weights are the softmax over the k selected
 * logits,
 *   topk_w[t,j] = exp(l_j - l_0) / sum_i exp(l_i - l_0).
 * NaN logits (the pages say nothing of them) rank above every number, NaNs
 * among themselves by lower index, so topk_idx always holds k distinct experts;
 * a token with a NaN logit gets NaN weights.
 * logits [T, E] fp32 (device); topk_idx [T, k] int32 (device, out);
 * topk_w [T, k] fp32 (device, out). */
int moe_route_topk(int T, int E, int k, const float* logits, int32_t* topk_idx, float* topk_w,
                   void* stream);

/* Workspace bytes moe_dispatch needs for T tokens, E experts, top-k. */
size_t moe_dispatch_workspace_bytes(int T, int E, int k);

/* Dispatch (issue #14, Proposal: rows gathered per expert; here on the GPU).
 * A stable counting sort of the N = T*k pairs by expert:
 *   counts[e]   pairs routed to expert e;  offsets = exclusive scan, offsets[E] = N
 *   perm[s]     pair id at sorted position s, ascending p within each expert
 *   inv_perm[p] sorted position of pair p
 *   x_sorted[s] = x[perm[s] / k]  (exact copy; skipped when x_sorted is NULL)
 * topk_idx [T, k] int32 (device, values in [0, E)); x [T, H] (device);
 * counts [E], offsets [E+1], perm [N], inv_perm [N] int32 (device, out);
 * x_sorted [N, H] (device, out, may be NULL together with x);
 * workspace (device) of at least moe_dispatch_workspace_bytes(T, E, k). */
int moe_dispatch(int T, int H, int E, int k, int dtype, const int32_t* topk_idx, const void* x,
                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* x_sorted,
                 void* workspace, size_t workspace_bytes, void* stream);

/* moe_dispatch for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, kernels and results as moe_dispatch, without the workspace: the
 * dispatch workspace is an array the library holds on every GPU it runs on,
 * until the process ends, of moe_dispatch_noalloc_max_workspace() bytes
 * (4 MiB).  A call whose moe_dispatch_workspace_bytes(T, E, k) exceeds that is
 * rejected with MOE_ERR_UNSUPPORTED before anything is enqueued (4 MiB holds
 * T*k up to 4194304 pairs at E = 128, 2097152 at E = 256).  The call allocates
 * nothing; its first call on a device looks up the array's device address
 * once.  Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (on different streams, or from host threads without an
 * order between them) race and give wrong results; calls on one stream are
 * ordered and safe.  Nothing in the array needs clearing between calls. */
int moe_dispatch_noalloc(int T, int H, int E, int k, int dtype, const int32_t* topk_idx, const void* x,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* x_sorted,
                         void* stream);
/* Bytes of the library-held dispatch workspace of moe_dispatch_noalloc.
 * Host-only. */
size_t moe_dispatch_noalloc_max_workspace(void);

/* SwiGLU expert forward as a ragged grouped GEMM (issue #14, Proposal: expert
 * forward graphs; pull request #44, Changes: forward keeps the activations that
 * backward reuses).  For each expert e, over its rows s in
 * [offsets[e], offsets[e+1]):
 *   hg = x_sorted[s] W_gate[e],  hu = x_sorted[s] W_up[e]        (length F)
 *   a  = silu(hg) * hu,  silu(z) = z / (1 + exp(-z))
 *   o_sorted[s] = a W_down[e]                                      (length H)
 * h_save[s] = [hg | hu] ([rows, 2F]) and a_save[s] = a ([rows, F]) are kept for
 * backward.  offsets [E+1] int32 (device); max_rows >= offsets[E] is a host
 * capacity (T*k) used only to size the launch; max_expert_rows >= 0 is a host
 * bound on one expert's row count used only to pick kernels (T for rows from
 * moe_dispatch, since top-k picks distinct experts per token; max_rows when
 * unknown): a bound below an actual count costs speed, never correctness,
 * and results do not depend on it beyond rounding; x_sorted [rows, H],
 * w_gate/w_up [E, H, F], w_down [E, F, H] (device); h_save, a_save, o_sorted
 * (device, out).  h_save may be NULL: the forward then keeps no pre-activations
 * and the backward recomputes them with moe_grouped_swiglu_recompute (pull
 * request #44, Changes and Compatibility and limits: keep_graph=False restores
 * the recompute path).  Rows of empty experts: nothing. */
int moe_grouped_swiglu_fwd(int H, int F, int E, int max_rows, int max_expert_rows, int dtype,
                           const int32_t* offsets,
                           const void* x_sorted, const void* w_gate, const void* w_up,
                           const void* w_down, void* h_save, void* a_save, void* o_sorted,
                           void* stream);

/* The expert forward with the gate/up product's rows gathered on load: row s
 * of expert e's rows reads x[perm[s] / k] instead of a materialized x_sorted[s]
 * (so moe_dispatch can skip its row copy: x_sorted = NULL there).  Everything
 * else as moe_grouped_swiglu_fwd, whose outputs it reproduces bit for bit.
 * x [T, H] (device); perm [T*k] int32 from moe_dispatch (device). */
int moe_grouped_swiglu_fwd_gather(int H, int F, int E, int k, int max_rows, int max_expert_rows, int dtype,
                                  const int32_t* offsets, const void* x, const int32_t* perm, const void* w_gate,
                                  const void* w_up, const void* w_down, void* h_save, void* a_save, void* o_sorted,
                                  void* stream);

/* The gate/up half of the expert forward over given rows, for the recompute
 * path (pull request #44, Background and Changes: without kept activations
 * the backward first recomputes the forward):
 *   h_rows[s] = [x_rows[s] W_gate[e] | x_rows[s] W_up[e]],  a_rows[s] = silu(hg) * hu
 * for the rows s of every expert e in offsets.  With the same offsets and row
 * capacities as a moe_grouped_swiglu_fwd call it gives that call's h_save and
 * a_save bit for bit.  Arguments as in moe_grouped_swiglu_fwd; x_rows [rows,
 * H] (device), or with x_src != NULL gathered on load: row s is
 * x_rows[x_src[s] / x_div] (x_src [rows] int32, device; 1 <= x_div <= 16; e.g.
 * the token matrix x with the pair ids perm or kept_perm and x_div = k);
 * h_rows [rows, 2F] (device, out); a_rows [rows, F] (device, out) or NULL. */
int moe_grouped_swiglu_recompute(int H, int F, int E, int max_rows, int max_expert_rows, int dtype,
                                 const int32_t* offsets, const void* x_rows, const int32_t* x_src, int x_div,
                                 const void* w_gate, const void* w_up, void* h_rows, void* a_rows, void* stream);

/* Router-weighted combine (issue #14, Proposal: results scattered back):
 *   out[t] = sum_{j = 0..k-1, inv[t*k+j] >= 0} w[t,j] * rows[inv[t*k+j]]
 * accumulated in fp32 in ascending j and rounded once.  With topk_w == NULL the
 * weight is 1 (this sums expert input-gradients into dx).  rows [*, H]
 * (device); inv [T*k] int32 (device; -1 skips the pair); topk_w [T, k] fp32
 * (device) or NULL; out [T, H] (device, out). */
int moe_combine(int T, int H, int k, int dtype, const void* rows, const int32_t* inv,
                const float* topk_w, void* out, void* stream);

/* Backward dx with routing held fixed (issue #14, Proposal and Scope: expert
 * backward dx, LoRA with frozen experts; LRMoE abstract: backward over the
 * retained, compacted pairs only).  Rows are either all pairs (offsets, inv
 * from moe_dispatch; h_rows = h_save) or the retained ones (kept_offsets,
 * kept_inv from moe_compact_pairs; h_rows = h_kept, or h_rows = h_save read
 * through h_src = kept_src without the compacted copy).  For each pair p with
 * r = inv[p] >= 0 (t = p / k):
 *   dO_rows[r]  = w[p] * dy[t]                                      [R, H]
 *   dA          = dO_rows[r] W_down[e]^T                             (length F)
 *   dh_rows[r]  = [dHg | dHu],  s = sigmoid(hg):                     [R, 2F]
 *                 dHg = dA * hu * s * (1 + hg * (1 - s)),  dHu = dA * hg * s
 *   dX_rows[r]  = dHg W_gate[e]^T + dHu W_up[e]^T                    [R, H]
 *   dx[t]       = sum_{j ascending, inv[t*k+j] >= 0} dX_rows[inv[t*k+j]]
 * and, when dg != NULL, for every pair (retained or not)
 *   dg[p] = <dy[p / k], o_sorted[inv_all[p]]>  (fp32).
 * offsets [E+1], inv [T*k] int32 (device; every row r < offsets[E] is the
 * image of exactly one pair); dy [T, H];
 * topk_w [T, k] fp32; h_rows [max_rows, 2F], or with h_src != NULL row r's
 * pre-activations are h_rows[h_src[r]] (h_src [max_rows] int32, device);
 * weights as in the forward; inv_all [T*k] and o_sorted [T*k, H] (device,
 * only read when dg != NULL); dO_rows, dh_rows, dX_rows [max_rows, *],
 * dx [T, H] (device, out). */
int moe_grouped_bwd_dx(int T, int H, int F, int E, int k, int max_rows, int dtype,
                       const int32_t* offsets, const int32_t* inv,
                       const void* dy, const float* topk_w, const void* h_rows, const int32_t* h_src,
                       const void* w_gate, const void* w_up, const void* w_down, const int32_t* inv_all,
                       const void* o_sorted, float* dg, void* dO_rows, void* dh_rows,
                       void* dX_rows, void* dx, void* stream);

/* ---- fp8 storage of frozen expert weights --------------------------------
 * In the LoRA step the experts are frozen (issue #14, Scope) and their weights
 * stay resident on the device (issue #14, Proposal), so they can be stored once
 * in 8 bits; the GEMMs then read half the weight bytes, which is what bounds
 * them when experts have few rows.  Element format: OCP 8-bit floating point
 * E4M3 (bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN,
 * largest finite 448).  Every expert has one power-of-two scale s: the
 * smallest with amax <= 448 s over all of that expert's matrices quantized
 * together (W_gate and W_up share one scale; W_down has its own).  The stored
 * code is E4M3(w / s), rounded to nearest with ties to the even mantissa
 * (w / s is exact); the weight the GEMMs use is decode(code) * s, exactly. */

/* Quantize E experts' bf16 matrices w0 [E][n0] and, when given, w1 [E][n1]
 * with one scale per expert shared by both: q0 [E][n0], q1 [E][n1] uint8
 * codes and scale [E] fp32 (device, out).  n0, n1 multiples of 8 (n1 = 0 and
 * w1 = q1 = NULL for a single matrix); w0/w1 16-byte aligned, q0/q1 8-byte
 * aligned (device).  One workgroup per expert; run once per set of weights. */
int moe_quantize_weights_fp8(int E, int64_t n0, int64_t n1, const void* w0, const void* w1, uint8_t* q0,
                             uint8_t* q1, float* scale, void* stream);

/* moe_grouped_swiglu_fwd with fp8 weights: wq_gate/wq_up [E, H, F] and
 * wq_down [E, F, H] E4M3 codes (device, 8-byte aligned) with per-expert scales
 * s_gu (of W_gate and W_up) and s_down [E] fp32 (device), as written by
 * moe_quantize_weights_fp8.  Activations and outputs are bf16.  perm = NULL:
 * x_rows is x_sorted [rows, H]; otherwise x_rows is x [T, H] and row s reads
 * x[perm[s] / k] (as moe_grouped_swiglu_fwd_gather).  Every expert, whatever
 * its row count, runs on the weight-streaming kernel (16-row tiles), the
 * regime where the weight bytes bound the GEMM.  The products are exactly
 * those of moe_grouped_swiglu_fwd on the decoded weights decode(q) * s, up to
 * the order of the fp32 sums. */
int moe_grouped_swiglu_fwd_fp8w(int H, int F, int E, int k, int max_rows, const int32_t* offsets,
                                const void* x_rows, const int32_t* perm, const uint8_t* wq_gate,
                                const uint8_t* wq_up, const uint8_t* wq_down, const float* s_gu,
                                const float* s_down, void* h_save, void* a_save, void* o_sorted,
                                void* stream);

/* moe_grouped_bwd_dx with fp8 weights (arguments as there, dtype bf16, and the
 * weights as in moe_grouped_swiglu_fwd_fp8w). */
int moe_grouped_bwd_dx_fp8w(int T, int H, int F, int E, int k, int max_rows, const int32_t* offsets,
                            const int32_t* inv, const void* dy, const float* topk_w, const void* h_rows,
                            const int32_t* h_src, const uint8_t* wq_gate, const uint8_t* wq_up, const uint8_t* wq_down,
                            const float* s_gu, const float* s_down, const int32_t* inv_all,
                            const void* o_sorted, float* dg, void* dO_rows, void* dh_rows, void* dX_rows,
                            void* dx, void* stream);

/* ---- the forward on the fp8 matrix cores ----------------------------------
 * The expert forward's two grouped GEMMs on E4M3 x E4M3 operands
 * (v_mfma_scale_f32_32x32x64_f8f6f4, twice the bf16 rate; LRMoE abstract:
 * variable-size grouped GEMMs; the pages fix no precision).  Every operand row
 * carries one power-of-two scale (the rule of moe_quantize_weights_fp8): per
 * token for x, per expert for the weights (W_gate and W_up sharing one), per
 * row for the SwiGLU output; products are accumulated in fp32 and multiplied
 * by the two scales (exact).  The SwiGLU output is stored in bf16 (a_save) and
 * that stored value is quantized for the down product.  H and F multiples of
 * 16.  Forward only. */

/* Per-row fp8 storage of bf16 activations x [rows, cols] (device, 16-byte
 * aligned; cols a multiple of 8): q [rows, cols] E4M3 codes (device, 8-byte
 * aligned, out) and scale [rows] fp32 (device, out), the smallest power of two
 * s with max_j |x[r,j]| <= 448 s, codes E4M3(x / s) rounded to nearest even,
 * saturating.  One wave per row. */
int moe_quantize_rows_fp8(int rows, int cols, const void* x, uint8_t* q, float* scale, void* stream);

/* out[e][c][r] = in[e][r][c] for E matrices of rows x cols bytes (device,
 * 16-byte aligned, distinct buffers; rows and cols multiples of 16): the
 * K-major copy of fp8 weight codes that moe_grouped_swiglu_fwd_fp8 reads
 * (W_gate, W_up [E,H,F] -> [E,F,H]; W_down [E,F,H] -> [E,H,F]). */
int moe_transpose_fp8(int E, int rows, int cols, const uint8_t* in, uint8_t* out, void* stream);

/* The expert forward on fp8 operands, over every expert's rows s in
 * [offsets[e], offsets[e+1]) (all on 256-row tiles):
 *   hg, hu = xd[s] W_gate_d[e], xd[s] W_up_d[e]       (d: decoded codes x scale)
 *   a_save[s] = bf16(silu(hg) hu),  h_save[s] = [hg | hu] (bf16; h_save may be NULL)
 *   aq[s], a_scale[s] = moe_quantize_rows_fp8 of a_save[s]
 *   o_sorted[s] = ad[s] W_down_d[e]                     (bf16)
 * xq [*, H] codes with x_scale [*] (device): with perm == NULL row s is xq[s]
 * (rows of x_sorted, quantized); otherwise xq holds the token rows and row s
 * is xq[perm[s] / k] (perm [T*k] from moe_dispatch, 1 <= k <= 16).  wt_gate,
 * wt_up [E, F, H] and wt_down [E, H, F]: K-major codes (moe_transpose_fp8 of
 * moe_quantize_weights_fp8's), with s_gu, s_down [E] (device).  h_save
 * [max_rows, 2F], a_save [max_rows, F] bf16; aq [max_rows, F] uint8 and
 * a_scale [max_rows] fp32 (device, out: the down product's input);
 * o_sorted [max_rows, H] bf16 (device, out).  max_rows = offsets[E] (every
 * row is quantized).  Codes, a_save and xq 16-byte aligned. */
int moe_grouped_swiglu_fwd_fp8(int H, int F, int E, int k, int max_rows, const int32_t* offsets, const uint8_t* xq,
                               const float* x_scale, const int32_t* perm, const uint8_t* wt_gate,
                               const uint8_t* wt_up, const uint8_t* wt_down, const float* s_gu, const float* s_down,
                               void* h_save, void* a_save, uint8_t* aq, float* a_scale, void* o_sorted,
                               void* stream);

/* Expert weight gradients (issue #14, Scope: dW for full fine-tuning), over the
 * rows r of each expert e (all pairs or the retained ones):
 *   dW_gate[e] = sum_r x_rows[r]^T dHg[r],  dW_up[e] = sum_r x_rows[r]^T dHu[r]
 *   dW_down[e] = sum_r a_rows[r]^T dO_rows[r]
 * in fp32, rounded once to the weight dtype; overwritten, not accumulated; an
 * expert without rows gets exact zeros.  offsets [E+1] int32 (device);
 * x_rows [*, H], a_rows [*, F], dO_rows [*, H], dh_rows [*, 2F] (device);
 * dw_gate, dw_up [E, H, F], dw_down [E, F, H] (device, out).  Rows gathered on
 * load: with x_src != NULL row r of x is x_rows[x_src[r] / x_div] (e.g. the
 * token matrix x, x_src = perm or kept_perm, x_div = k; 1 <= x_div <= 16), and
 * with a_src != NULL row r of a is a_rows[a_src[r]] (e.g. a_save with
 * a_src = kept_src); x_src, a_src [max_rows] int32 (device) or NULL.  The
 * results do not depend on whether rows are gathered. */
int moe_grouped_bwd_dw(int H, int F, int E, int max_rows, int dtype, const int32_t* offsets,
                       const void* x_rows, const int32_t* x_src, int x_div, const void* a_rows,
                       const int32_t* a_src, const void* dO_rows, const void* dh_rows, void* dw_gate,
                       void* dw_up, void* dw_down, void* stream);

/* Router backward with the selection held fixed (issue #14, Proposal and Done
 * when: the gradients of the device path match the host path's).  The weights
 * being the softmax over the k selected logits, with g = dg (dL/dtopk_w, from
 * moe_grouped_bwd_dx) and s_t = sum_j topk_w[t,j] g[t,j]:
 *   dlogits[t, topk_idx[t,j]] = topk_w[t,j] (g[t,j] - s_t), other entries 0
 *   dw_r = x^T dlogits                       [H, E], overwritten
 *   dx   = dlogits w_r^T  (+ dx if dx_accumulate != 0)   [T, H]
 * all accumulated in fp32 and rounded once to `dtype`.  x [T, H], w_r [H, E]
 * of `dtype` (device); topk_idx [T, k] int32 (device, distinct experts per
 * token, as moe_route_topk gives); topk_w, dg [T, k] fp32 (device); dlogits
 * [T, E] fp32 (device, out); dw_r [H, E] and dx [T, H] of `dtype` (device;
 * dx read too when accumulating); workspace as for moe_router_fwd. */
int moe_router_bwd(int T, int H, int E, int k, int dtype, const void* x, const void* w_r, const int32_t* topk_idx,
                   const float* topk_w, const float* dg, float* dlogits, void* dw_r, void* dx, int dx_accumulate,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Quota cap used by moe_compact_pairs: ceil(rho * T * k / E) (integer
 * arithmetic when rho == 1, else evaluated in double).  Host-only. */
int64_t moe_quota_cap(int T, int E, int k, double rho);

/* Selection within retention quotas and physical compaction (LRMoE abstract:
 * quotas, a per-pair score, selection within quotas, compaction into smaller
 * buffers for variable-size grouped GEMMs).  Expert e keeps its
 * q_e = min(counts[e], moe_quota_cap(T, E, k, rho)) pairs of largest score,
 * equal scores to the lower pair id; kept pairs stay in ascending pair id.
 *   kept_counts[e] = q_e, kept_offsets = exclusive scan (kept_offsets[E] = R)
 *   kept_perm[r] pair id, kept_src[r] its position in the uncompacted order,
 *   kept_inv[p] compacted position or -1 when dropped
 *   x_kept[r] = x_sorted[kept_src[r]], a_kept[r] = a_save[..], h_kept[r] = h_save[..]
 * The row gathers are skipped for NULL sources.  counts [E], offsets [E+1],
 * perm [T*k] int32 and score [T*k] fp32 (device, pair-indexed, finite);
 * kept_counts [E], kept_offsets [E+1], kept_inv [T*k] int32 (device, out);
 * kept_perm and kept_src int32 (device, out) and x_kept, a_kept, h_kept
 * (device, out) hold at least min(T*k, E*cap) entries or rows, cap =
 * moe_quota_cap(T, E, k, rho) (the given cap for moe_compact_pairs_cap), of
 * which the first R (<= that bound) are written. */
int moe_compact_pairs(int T, int H, int F, int E, int k, int dtype, double rho,
                      const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                      const float* score, int32_t* kept_counts, int32_t* kept_offsets,
                      int32_t* kept_perm, int32_t* kept_src, int32_t* kept_inv,
                      const void* x_sorted, const void* a_save, const void* h_save, void* x_kept,
                      void* a_kept, void* h_kept, void* stream);

/* The same selection and compaction with the per-expert quota given directly
 * (cap >= 1; a cap above T*k means no pair is dropped), e.g. from
 * moe_quota_cap_for_budget. */
int moe_compact_pairs_cap(int T, int H, int F, int E, int k, int dtype, int cap,
                      const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                      const float* score, int32_t* kept_counts, int32_t* kept_offsets,
                      int32_t* kept_perm, int32_t* kept_src, int32_t* kept_inv,
                      const void* x_sorted, const void* a_save, const void* h_save, void* x_kept,
                      void* a_kept, void* h_kept, void* stream);

/* Quota cap from a memory budget for the backward's per-row buffers (LRMoE
 * abstract: quotas planned from the memory a node can spend).  A retained row
 * holds dO [H], dh [2F], dX [H] and its compacted x [H], plus h [2F] when
 * keep_graph and a [F] when with_dw, all of `dtype`; the cap is the largest
 * per-expert quota whose worst case (every expert at its cap) fits:
 *   floor(budget_bytes / (E * row_bytes)), at most ceil(T k / E);
 * -1 when not even one row per expert fits or an argument is invalid.
 * Host-only. */
int64_t moe_quota_cap_for_budget(int T, int H, int F, int E, int k, int dtype, int with_dw, int keep_graph,
                                 size_t budget_bytes);

/* Pair scores for the quota selection (LRMoE abstract: retention by each
 * pair's contribution to the expert update; the pages leave the metric open).
 * The metric here is known before any backward GEMM: the Frobenius norm of
 * pair p's rank-one term in dW_down,
 *   score[p] = topk_w[p] * ||a_save[inv_perm[p]]||_2 * ||dy[p / k]||_2
 * (0 for a pair without a row), sums of squares in fp32.  inv_perm [T*k] int32,
 * topk_w [T*k] fp32, a_save [*, F], dy [T, H] of `dtype` (device); score
 * [T*k] fp32 (device, out). */
int moe_pair_scores(int T, int H, int F, int k, int dtype, const int32_t* inv_perm, const float* topk_w,
                    const void* a_save, const void* dy, float* score, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
