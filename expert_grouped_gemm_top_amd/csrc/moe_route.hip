// moe_route.hip -- top-k routing, one wavefront per token.
//
// Routing of each token to k of E experts (npu-train issue #14, sections
// Evidence and Proposal).  Ranking: logit descending, equal logits to the lower
// expert index (+0.0 and -0.0 compare equal).  Weights: softmax over the k
// selected logits with the largest one subtracted.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kPerLane = kMaxExperts / kWave;  // logits held per lane (E <= 256)

// (va, ia) ranks before (vb, ib)?
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__global__ __launch_bounds__(256) void route_topk_kernel(int T, int E, int k, const float* __restrict__ logits,
                                                         int32_t* __restrict__ idx, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave exits together
  const float* lt = logits + (size_t)t * E;
  float v[kPerLane];
  bool live[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    const int e = lane + i * kWave;
    live[i] = e < E;
    v[i] = live[i] ? lt[e] : 0.0f;
  }
  float sel_v = 0.0f;  // lane j (< k) keeps the j-th selected logit
  int sel_e = 0;
  float top = 0.0f;
  for (int j = 0; j < k; ++j) {
    // lane-local best among the experts not taken yet
    float bv = 0.0f;
    int be = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const int e = lane + i * kWave;
      if (live[i] && (be == 0x7fffffff || ranks_before(v[i], e, bv, be))) {
        bv = v[i];
        be = e;
      }
    }
    // wave arg-max under the same order (butterfly: every lane ends with the winner)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, kWave);
      const int oe = __shfl_xor(be, o, kWave);
      if (oe != 0x7fffffff && (be == 0x7fffffff || ranks_before(ov, oe, bv, be))) {
        bv = ov;
        be = oe;
      }
    }
    if (j == 0) top = bv;
    if (lane == j) {
      sel_v = bv;
      sel_e = be;
    }
    // retire the winner in its owning lane
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
      if (lane + i * kWave == be) live[i] = false;
  }
  const float ex = (lane < k) ? expf(sel_v - top) : 0.0f;
  const float denom = wave_sum(ex);
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel_e;
    w[(size_t)t * k + lane] = ex / denom;
  }
}

}  // namespace

hipError_t launch_route_topk(int T, int E, int k, const float* logits, int32_t* idx, float* w,
                             hipStream_t stream) {
  const int blocks = (T + 3) / 4;
  hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(256), 0, stream, T, E, k, logits, idx, w);
  return hipGetLastError();
}

}  // namespace moe
