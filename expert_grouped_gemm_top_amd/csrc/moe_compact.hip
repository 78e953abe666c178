// moe_compact.hip -- selection of retained pairs within per-expert quotas and
// their compaction (LRMoE, arXiv:2610.37720, abstract: quotas planned in the
// forward pass, a per-pair score, selection within the quotas, and physical
// compaction into smaller buffers for variable-size grouped GEMMs).
//
// One workgroup per expert.  Expert e keeps q_e = min(n_e, cap) pairs: the ones
// with the largest score, equal scores to the lower pair id.  That order is a
// total order on the 64-bit key  (orderable(score) << 32) | ~p , so the kept
// set is { key >= the q_e-th largest key }.  The threshold key is found by an
// 8-pass MSB-first radix select (256-bin LDS histograms; the counts do not
// depend on the order of the LDS atomics).  A block prefix scan over the
// expert's pairs in sorted order then writes the kept pairs in ascending p.
// kept_offsets follows from the counts alone (q_e depends only on n_e), so
// every workgroup computes its own base with one block scan.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

namespace {

__device__ __forceinline__ uint64_t pair_key(float score, int32_t p) {
  if (score == 0.0f) score = 0.0f;  // -0 ranks equal to +0
  uint32_t u = __float_as_uint(score);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~(uint32_t)p);
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ a, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) a[i] = v;
}

__global__ __launch_bounds__(256) void compact_select_kernel(int E, int cap, const int32_t* __restrict__ counts,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ perm,
                                                             const float* __restrict__ score,
                                                             int32_t* __restrict__ kept_counts,
                                                             int32_t* __restrict__ kept_offsets,
                                                             int32_t* __restrict__ kept_perm,
                                                             int32_t* __restrict__ kept_src,
                                                             int32_t* __restrict__ kept_inv) {
  __shared__ int s_tmp[4];
  __shared__ int s_hist[256];
  __shared__ int s_pick[2];
  const int e = blockIdx.x, tid = threadIdx.x;
  // kept base of this expert: exclusive scan of min(n_e', cap)
  const int qv = (tid < E) ? min(counts[tid], cap) : 0;
  int total;
  const int kbase_t = block256_exclusive_scan(qv, s_tmp, total);
  if (tid == e) {
    kept_counts[e] = qv;
    kept_offsets[e] = kbase_t;
    s_pick[0] = kbase_t;
  }
  if (e == 0 && tid == 0) kept_offsets[E] = total;
  __syncthreads();
  const int kbase = s_pick[0];
  const int off = offsets[e];
  const int n = offsets[e + 1] - off;
  const int q = min(n, cap);
  __syncthreads();
  if (q == n) {
    for (int i = tid; i < n; i += 256) {
      const int32_t p = perm[off + i];
      kept_perm[kbase + i] = p;
      kept_src[kbase + i] = off + i;
      kept_inv[p] = kbase + i;
    }
    return;
  }
  // radix select of the q-th largest key, most significant byte first
  uint64_t prefix = 0, mask = 0;
  int remaining = q;  // rank (1-based, from the top) still to find within the prefix class
  for (int shift = 56; shift >= 0; shift -= 8) {
    s_hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const int32_t p = perm[off + i];
      const uint64_t key = pair_key(score[p], p);
      if ((key & mask) == prefix) atomicAdd(&s_hist[(int)((key >> shift) & 0xffu)], 1);
    }
    __syncthreads();
    // thread t looks at bin 255 - t; count of keys in higher bins = exclusive scan
    const int cnt = s_hist[255 - tid];
    int tot;
    const int above = block256_exclusive_scan(cnt, s_tmp, tot);
    if (above < remaining && remaining <= above + cnt) {
      s_pick[0] = 255 - tid;
      s_pick[1] = remaining - above;
    }
    __syncthreads();
    prefix |= (uint64_t)s_pick[0] << shift;
    mask |= (uint64_t)0xffu << shift;
    remaining = s_pick[1];
    __syncthreads();
  }
  const uint64_t thr = prefix;  // the q-th largest key; keep key >= thr
  int run = 0;
  for (int i0 = 0; i0 < n; i0 += 256) {
    const int i = i0 + tid;
    int32_t p = 0;
    int keep = 0;
    if (i < n) {
      p = perm[off + i];
      keep = pair_key(score[p], p) >= thr;
    }
    int tot;
    const int pos = block256_exclusive_scan(keep, s_tmp, tot);
    if (i < n) {
      if (keep) {
        kept_perm[kbase + run + pos] = p;
        kept_src[kbase + run + pos] = off + i;
        kept_inv[p] = kbase + run + pos;
      } else {
        kept_inv[p] = -1;
      }
    }
    run += tot;
  }
}

}  // namespace

hipError_t launch_fill_i32(int32_t* a, int64_t n, int32_t v, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, n, v);
  return hipGetLastError();
}

hipError_t launch_compact(int64_t N, int E, int cap, const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                          const float* score, int32_t* kept_counts, int32_t* kept_offsets, int32_t* kept_perm,
                          int32_t* kept_src, int32_t* kept_inv, hipStream_t stream) {
  (void)N;
  hipLaunchKernelGGL(compact_select_kernel, dim3(E), dim3(256), 0, stream, E, cap, counts, offsets, perm, score,
                     kept_counts, kept_offsets, kept_perm, kept_src, kept_inv);
  return hipGetLastError();
}

}  // namespace moe
