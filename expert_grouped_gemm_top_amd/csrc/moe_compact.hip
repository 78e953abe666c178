// moe_compact.hip -- selection of retained pairs within per-expert quotas and
// their compaction (LRMoE, arXiv:2610.37720, abstract: quotas planned in the
// forward pass, a per-pair score, selection within the quotas, and physical
// compaction into smaller buffers for variable-size grouped GEMMs).
//
// One workgroup per expert.  Expert e keeps q_e = min(n_e, cap) pairs: the ones
// with the largest score, equal scores to the lower pair id.  That order is a
// total order on the 64-bit key  (orderable(score) << 32) | ~p , so the kept
// set is { key >= the q_e-th largest key }.  The threshold key is found by an
// MSB-first radix select of up to 8 passes (256-bin LDS histograms; the counts
// do not depend on the order of the LDS atomics), ending early once the q-th
// key's bin is kept whole.  A block prefix scan over the
// expert's pairs in sorted order then writes the kept pairs in ascending p.
// Up to kLdsPairs pairs, the expert's pair ids and score keys are gathered
// into LDS once (eight independent loads per thread in flight) and every pass
// runs out of LDS; larger experts re-read them from memory in each pass.
// kept_offsets follows from the counts alone (q_e depends only on n_e), so
// every workgroup computes its own base with one block scan.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kLdsPairs = 16384;  // pairs whose id and score key fit the workgroup's LDS (128 KiB)
constexpr int kUnroll = 8;        // independent loads per thread in flight

// Score -> unsigned key with the same order (-0 ranks equal to +0).
__device__ __forceinline__ uint32_t score_key(float score) {
  if (score == 0.0f) score = 0.0f;
  const uint32_t u = __float_as_uint(score);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t pair_key(float score, int32_t p) {
  return ((uint64_t)score_key(score) << 32) | (uint32_t)(~(uint32_t)p);
}

__device__ __forceinline__ uint64_t lds_key(const uint32_t* s_khi, const int32_t* s_p, int i) {
  return ((uint64_t)s_khi[i] << 32) | (uint32_t)(~(uint32_t)s_p[i]);
}

// The key threshold from a 256-bin histogram pass: thread t looks at bin
// 255 - t; the keys in higher bins are an exclusive scan.  Updates the prefix
// class and the rank still to find within it.  Returns true (uniformly) when
// the rank is the last of its bin: every key of the bin is then kept, so the
// prefix with its lower bits zero is already the threshold and the remaining
// passes are skipped (with real-valued scores the q-th key is usually alone in
// its bin after two or three passes).
__device__ __forceinline__ bool radix_pick(const int* s_hist, int* s_tmp, int* s_pick, int shift, uint64_t& prefix,
                                           uint64_t& mask, int& remaining) {
  const int tid = threadIdx.x;
  const int cnt = s_hist[255 - tid];
  int tot;
  const int above = block256_exclusive_scan(cnt, s_tmp, tot);
  if (above < remaining && remaining <= above + cnt) {
    s_pick[0] = 255 - tid;
    s_pick[1] = remaining - above;
    s_pick[2] = cnt;
  }
  __syncthreads();
  prefix |= (uint64_t)s_pick[0] << shift;
  mask |= (uint64_t)0xffu << shift;
  remaining = s_pick[1];
  const bool whole_bin = s_pick[1] == s_pick[2];
  __syncthreads();
  return whole_bin;
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
  __shared__ int s_pick[3];
  extern __shared__ __attribute__((aligned(16))) uint32_t s_pairs[];  // [kLdsPairs] keys, then [kLdsPairs] ids
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
    for (int i0 = 0; i0 < n; i0 += 256 * kUnroll) {
      int32_t pv[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int i = i0 + 256 * j + tid;
        pv[j] = i < n ? perm[off + i] : 0;
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int i = i0 + 256 * j + tid;
        if (i < n) {
          kept_perm[kbase + i] = pv[j];
          kept_src[kbase + i] = off + i;
          kept_inv[pv[j]] = kbase + i;
        }
      }
    }
    return;
  }
  if (n <= kLdsPairs) {
    uint32_t* s_khi = s_pairs;
    int32_t* s_p = reinterpret_cast<int32_t*>(s_pairs + kLdsPairs);
    for (int i0 = 0; i0 < n; i0 += 256 * kUnroll) {
      int32_t pv[kUnroll];
      float sv[kUnroll];
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int i = i0 + 256 * j + tid;
        pv[j] = i < n ? perm[off + i] : 0;
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int i = i0 + 256 * j + tid;
        sv[j] = i < n ? score[pv[j]] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < kUnroll; ++j) {
        const int i = i0 + 256 * j + tid;
        if (i < n) {
          s_p[i] = pv[j];
          s_khi[i] = score_key(sv[j]);
        }
      }
    }
    __syncthreads();
    uint64_t prefix = 0, mask = 0;
    int remaining = q;
    for (int shift = 56; shift >= 0; shift -= 8) {
      s_hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += 256) {
        const uint64_t key = lds_key(s_khi, s_p, i);
        if ((key & mask) == prefix) atomicAdd(&s_hist[(int)((key >> shift) & 0xffu)], 1);
      }
      __syncthreads();
      if (radix_pick(s_hist, s_tmp, s_pick, shift, prefix, mask, remaining)) break;
    }
    // kept pairs in ascending order: thread t takes the contiguous chunk
    // [t c, (t + 1) c) and its place follows from a scan of the chunk counts
    const int c = (n + 255) / 256, i_lo = min(n, tid * c), i_hi = min(n, i_lo + c);
    int cnt = 0;
    for (int i = i_lo; i < i_hi; ++i) cnt += lds_key(s_khi, s_p, i) >= prefix ? 1 : 0;
    int tot;
    int pos = kbase + block256_exclusive_scan(cnt, s_tmp, tot);
    for (int i = i_lo; i < i_hi; ++i) {
      const int32_t p = s_p[i];
      if (lds_key(s_khi, s_p, i) >= prefix) {
        kept_perm[pos] = p;
        kept_src[pos] = off + i;
        kept_inv[p] = pos;
        ++pos;
      } else {
        kept_inv[p] = -1;
      }
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
    if (radix_pick(s_hist, s_tmp, s_pick, shift, prefix, mask, remaining)) break;
  }
  const uint64_t thr = prefix;  // keep key >= thr: exactly the q largest keys
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
  MOE_LAUNCH(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, n, v);
  return hipGetLastError();
}

hipError_t launch_compact(int64_t N, int E, int cap, const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                          const float* score, int32_t* kept_counts, int32_t* kept_offsets, int32_t* kept_perm,
                          int32_t* kept_src, int32_t* kept_inv, hipStream_t stream) {
  (void)N;
  const size_t lds = 2 * kLdsPairs * sizeof(uint32_t);
  // dynamic LDS above 64 KiB must be allowed explicitly, once per device
  static PerDeviceOnce lds_once;
  hipError_t err = allow_dynamic_lds(lds_once, (const void*)compact_select_kernel, lds);
  if (err != hipSuccess) return err;
  MOE_LAUNCH(compact_select_kernel, dim3(E), dim3(256), lds, stream, E, cap, counts, offsets, perm, score,
                     kept_counts, kept_offsets, kept_perm, kept_src, kept_inv);
  return hipGetLastError();
}

}  // namespace moe
