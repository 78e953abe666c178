// moe_route.hip -- top-k routing, one wavefront per token.
//
// Routing of each token to k of E experts (npu-train issue #14, sections
// Evidence and Proposal).  Ranking: logit descending, equal logits to the lower
// expert index (+0.0 and -0.0 compare equal), a NaN above every number (NaNs
// among themselves by index).  Weights: softmax over the k selected logits
// with the largest one subtracted (NaN for a token with a NaN logit).
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

namespace {

// Total-order key of a logit: larger key = ranks first.  -0.0 maps to the key
// of +0.0 and every NaN to the largest key, so the ranks of one token's logits
// are always a permutation of 0..E-1.
__device__ __forceinline__ uint32_t rank_key(float v) {
  if (v != v) return 0xffffffffu;
  const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Order key of (logit key, expert index) in one 64-bit word: the logit key
// above the complemented index, so a larger word ranks first and equal logit
// keys fall to the lower index; one 64-bit compare per pair of logits.
__device__ __forceinline__ uint64_t order_key(uint32_t key, int e) {
  return ((uint64_t)key << 32) | (uint32_t)~e;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// One wavefront per token; lane l holds the logits of experts l + 64 i
// (i < SLOTS = ceil(E / 64)).  Every lane computes the rank of each of its
// logits under the order above by comparing its order key with all E keys of
// the token (read back from LDS as broadcasts); the ranks are distinct, and a
// logit of rank r < k is the token's r-th selection.  The comparisons are the
// kernel's work (VALU-bound: the packed 64-bit key halves the instructions per
// comparison, 36.7 -> 22.4 us at 16384 tokens, 8.1 -> 5.3 us at 128).  The
// weights are the softmax over the k selected logits, shifted by the largest
// one.
template <int SLOTS>
__global__ __launch_bounds__(256) void route_topk_kernel(int T, int E, int k, const float* __restrict__ logits,
                                                         int32_t* __restrict__ idx, float* __restrict__ w) {
  __shared__ __attribute__((aligned(16))) uint64_t s_l[4][kMaxExperts];  // order keys
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits; only this wave's LDS row is used below
  const float* lt = logits + (size_t)t * E;
  float v[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) v[i] = lt[min(lane + 64 * i, E - 1)];  // in bounds, no branch
  const int E2 = (E + 1) & ~1;
  uint64_t key[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int e = lane + 64 * i;
    key[i] = order_key(rank_key(v[i]), e);
    // an entry E (E odd) holds logit key 0 below every real logit's (a real
    // key is at least that of -inf, 0x007fffff): it never ranks first
    if (e < E2) s_l[wv][e] = (e < E) ? key[i] : order_key(0u, e);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // the wave's LDS writes before its reads
  int rank[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) rank[i] = 0;
#pragma unroll 4
  for (int j = 0; j < E2; j += 2) {
    const uint64_t q0 = s_l[wv][j], q1 = s_l[wv][j + 1];
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) rank[i] += (q0 > key[i] ? 1 : 0) + (q1 > key[i] ? 1 : 0);
  }
  float top = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < SLOTS; ++i)
    if (lane + 64 * i < E) top = fmaxf(top, v[i]);
  top = wave_max(top);
  float ex[SLOTS], part = 0.0f;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const bool sel = lane + 64 * i < E && rank[i] < k;
    ex[i] = sel ? expf(v[i] - top) : 0.0f;
    part += ex[i];
  }
  const float denom = wave_sum(part);
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    if (lane + 64 * i < E && rank[i] < k) {
      idx[(size_t)t * k + rank[i]] = lane + 64 * i;
      w[(size_t)t * k + rank[i]] = ex[i] / denom;
    }
  }
}

}  // namespace

hipError_t launch_route_topk(int T, int E, int k, const float* logits, int32_t* idx, float* w,
                             hipStream_t stream) {
  const dim3 grid((T + 3) / 4), block(256);
  switch ((E + 63) / 64) {
    case 1: MOE_LAUNCH(route_topk_kernel<1>, grid, block, 0, stream, T, E, k, logits, idx, w); break;
    case 2: MOE_LAUNCH(route_topk_kernel<2>, grid, block, 0, stream, T, E, k, logits, idx, w); break;
    case 3: MOE_LAUNCH(route_topk_kernel<3>, grid, block, 0, stream, T, E, k, logits, idx, w); break;
    default: MOE_LAUNCH(route_topk_kernel<4>, grid, block, 0, stream, T, E, k, logits, idx, w); break;
  }
  return hipGetLastError();
}

}  // namespace moe
