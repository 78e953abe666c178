// moe_dispatch.hip -- stable counting sort of token-expert pairs by expert,
// and the copy of token rows into rows contiguous per expert.
//
// Dispatch of tokens into per-expert groups of rows (npu-train issue #14,
// section Proposal), done on the GPU instead of the host.  Pair p = t*k + j
// goes to expert idx[p]; within an expert pairs keep ascending p, so the
// permutation is unique and bit-reproducible.
//
// Kernels (all on the caller's stream):
//   hist  per block of 1024 pairs: expert histogram in LDS     (order-free LDS atomics)
//   scan  one block: offsets = exclusive scan of counts, and every block's base
//         (the blocks split into ranges summed by separate threads)
//   rank  per block: stable rank of each pair among equal experts, from
//         ballots on the bits of the expert id and popcounts below the lane,
//         plus per-wave running bases in LDS; writes perm and inv_perm
//   rows  per token: read x[t] once, write its k copies to x_sorted
// With a single block of pairs (N <= 1024) hist, scan and rank run fused in one
// workgroup.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kPairsPerWave = 256;
constexpr int kPairsPerBlock = 4 * kPairsPerWave;

__device__ __forceinline__ int expert_bits(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

__global__ __launch_bounds__(256) void dispatch_hist_kernel(int64_t N, int E, const int32_t* __restrict__ idx,
                                                            int32_t* __restrict__ ws_hist) {
  __shared__ int s_cnt[kMaxExperts];
  const int tid = threadIdx.x;
  if (tid < E) s_cnt[tid] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * kPairsPerBlock;
  for (int i = tid; i < kPairsPerBlock; i += 256) {
    const int64_t p = p0 + i;
    if (p < N) {
      const int e = idx[p];
      if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
    }
  }
  __syncthreads();
  if (tid < E) ws_hist[(size_t)blockIdx.x * E + tid] = s_cnt[tid];
}

// One block.  ws_base[b][e] = offsets[e] + pairs of expert e in blocks before
// b.  The blocks are split into `parts` ranges (parts x E <= 256 threads);
// thread (part, e) sums its range, the part sums and the expert totals are
// scanned in LDS, then the thread writes its range's running bases.  Loads
// are issued kUnroll at a time so that their latencies overlap.
constexpr int kScanUnroll = 8;
__global__ __launch_bounds__(256) void dispatch_scan_kernel(int nblocks, int E, const int32_t* __restrict__ ws_hist,
                                                            int32_t* __restrict__ ws_base, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int s_tmp[4];
  __shared__ int s_part[4][kMaxExperts];
  const int tid = threadIdx.x;
  const int parts = min(4, 256 / E);
  const bool active = tid < parts * E;
  const int e = active ? tid % E : 0, part = active ? tid / E : 0;
  const int lo = (int)((int64_t)part * nblocks / parts), hi = (int)((int64_t)(part + 1) * nblocks / parts);
  int sum = 0;
  if (active)
    for (int b0 = lo; b0 < hi; b0 += kScanUnroll) {
      int v[kScanUnroll];
#pragma unroll
      for (int j = 0; j < kScanUnroll; ++j) v[j] = (b0 + j < hi) ? ws_hist[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanUnroll; ++j) sum += v[j];
    }
  if (active) s_part[part][e] = sum;
  __syncthreads();
  int tot = 0;
  if (tid < E)
    for (int q = 0; q < parts; ++q) tot += s_part[q][tid];
  int total;
  const int off = block256_exclusive_scan(tid < E ? tot : 0, s_tmp, total);
  if (tid < E) {
    counts[tid] = tot;
    offsets[tid] = off;
    int run = off;
    for (int q = 0; q < parts; ++q) {  // part sums -> part bases
      const int c = s_part[q][tid];
      s_part[q][tid] = run;
      run += c;
    }
  }
  if (tid == 0) offsets[E] = total;
  __syncthreads();
  if (active) {
    int run = s_part[part][e];
    for (int b0 = lo; b0 < hi; b0 += kScanUnroll) {
      int v[kScanUnroll];
#pragma unroll
      for (int j = 0; j < kScanUnroll; ++j) v[j] = (b0 + j < hi) ? ws_hist[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kScanUnroll; ++j)
        if (b0 + j < hi) {
          ws_base[(size_t)(b0 + j) * E + e] = run;
          run += v[j];
        }
    }
  }
}

// FUSED: this is the only block; counts/offsets are produced here.
template <bool FUSED>
__global__ __launch_bounds__(256) void dispatch_rank_kernel(int64_t N, int E, const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ ws_base,
                                                            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm) {
  __shared__ int s_cnt[4][kMaxExperts];   // per-wave histograms, then per-wave running bases
  __shared__ int s_tmp[4];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t pw = (int64_t)blockIdx.x * kPairsPerBlock + (int64_t)w * kPairsPerWave;
  for (int i = tid; i < 4 * kMaxExperts; i += 256) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  for (int c = 0; c < kPairsPerWave; c += kWave) {
    const int64_t p = pw + c + lane;
    if (p < N) {
      const int e = idx[p];
      if (e >= 0 && e < E) atomicAdd(&s_cnt[w][e], 1);
    }
  }
  __syncthreads();
  // thread e turns the four wave histograms into running bases
  int base = 0;
  if (FUSED) {
    int tot = 0;
    if (tid < E) tot = s_cnt[0][tid] + s_cnt[1][tid] + s_cnt[2][tid] + s_cnt[3][tid];
    int total;
    base = block256_exclusive_scan(tot, s_tmp, total);
    if (tid < E) {
      counts[tid] = tot;
      offsets[tid] = base;
    }
    if (tid == 0) offsets[E] = total;
  } else if (tid < E) {
    base = ws_base[(size_t)blockIdx.x * E + tid];
  }
  if (tid < E) {
    const int c0 = s_cnt[0][tid], c1 = s_cnt[1][tid], c2 = s_cnt[2][tid];
    s_cnt[0][tid] = base;
    s_cnt[1][tid] = base + c0;
    s_cnt[2][tid] = base + c0 + c1;
    s_cnt[3][tid] = base + c0 + c1 + c2;
  }
  __syncthreads();
  const int nbits = expert_bits(E);
  const uint64_t lt = lanemask_lt();
  for (int c = 0; c < kPairsPerWave; c += kWave) {
    const int64_t p = pw + c + lane;
    int e = (p < N) ? idx[p] : -1;
    const bool ok = e >= 0 && e < E;
    if (!ok) e = 0;
    uint64_t peers = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    if (ok) {
      const int s = s_cnt[w][e] + rank;
      perm[s] = (int32_t)p;
      inv_perm[p] = s;
    } else if (p < N) {
      inv_perm[p] = -1;  // out-of-range expert id: the pair is dropped
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    if (ok && (peers & lt) == 0) s_cnt[w][e] += __popcll(peers);  // lowest lane of each group
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  }
}

// Row copy x_sorted[inv_perm[t k + j]] = x[t].  Work item = (token, run of
// 256 16-byte chunks of its row); workgroups take items in a grid-stride loop
// and load the next item's chunk and destinations before storing the current
// one, so each lane has a load in flight while it stores (a workgroup per
// token left every lane waiting one memory latency before its stores).  Every
// chunk of x[t] is read once and written to the k sorted positions of the
// token's pairs.
constexpr int kRowCopyBlocks = 16384;  // workgroups of the row copy at most

__global__ __launch_bounds__(256) void dispatch_rows_kernel(int T, int k, int row_chunks, const u32x4* __restrict__ x,
                                                            const int32_t* __restrict__ inv_perm,
                                                            u32x4* __restrict__ x_sorted) {
  const int groups = (row_chunks + 255) / 256;
  const int64_t items = (int64_t)T * groups;
  int64_t i = blockIdx.x;
  if (i >= items) return;
  struct Item {
    int64_t t;
    int c;
    u32x4 v;
    int dst[kMaxTopK];
  };
  auto fetch = [&](int64_t it, Item& d) {
    d.t = it / groups;
    d.c = (int)(it - d.t * groups) * 256 + (int)threadIdx.x;
    // x is read once here (the GEMMs read x_sorted): non-temporal
    if (d.c < row_chunks) d.v = __builtin_nontemporal_load(x + d.t * row_chunks + d.c);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) d.dst[j] = (j < k) ? inv_perm[d.t * k + j] : -1;
  };
  Item cur, nxt;
  fetch(i, cur);
  for (;;) {
    const int64_t in = i + gridDim.x;
    if (in < items) fetch(in, nxt);
    if (cur.c < row_chunks) {
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j)
        if (j < k && cur.dst[j] >= 0) x_sorted[(size_t)cur.dst[j] * row_chunks + cur.c] = cur.v;
    }
    if (in >= items) break;
    i = in;
    cur = nxt;
  }
}

}  // namespace

// Library-owned dispatch workspace for callers that cannot allocate device
// memory (moe_dispatch_noalloc).  Every GPU the library runs on holds its own
// copy until the process ends.  Host code must use the device address that
// hipGetSymbolAddress returns for it (dispatch_scratch below), never the
// array's name, which on the host is only a stand-in for the symbol.
// Nothing in it needs to start at zero: the histogram kernel writes every
// entry it uses before the scan reads it, and the scan writes every base the
// rank kernel reads.
static __device__ __align__(256) unsigned char scratch[kDispatchScratchBytes];

hipError_t dispatch_scratch(void** out) {
  static PerDeviceOnce once;
  static void* addr[PerDeviceOnce::kDevices];
  void* fresh = nullptr;
  hipError_t err = once.run([&](int dev) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e == hipSuccess) {
      fresh = p;
      if (dev >= 0 && dev < PerDeviceOnce::kDevices) addr[dev] = p;
    }
    return e;
  });
  if (err != hipSuccess) return err;
  int dev = 0;
  if ((err = hipGetDevice(&dev)) != hipSuccess) return err;
  *out = (dev >= 0 && dev < PerDeviceOnce::kDevices) ? addr[dev] : fresh;
  return *out != nullptr ? hipSuccess : hipErrorInvalidSymbol;
}

size_t dispatch_workspace_bytes(int64_t N, int E) {
  const int64_t nblocks = (N + kPairsPerBlock - 1) / kPairsPerBlock;
  if (nblocks <= 1) return 0;
  return (size_t)(2 * nblocks * E) * sizeof(int32_t);
}

hipError_t launch_dispatch_index(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                                 int32_t* perm, int32_t* inv_perm, void* ws, hipStream_t stream) {
  const int64_t N = (int64_t)T * k;
  const int64_t nblocks = (N + kPairsPerBlock - 1) / kPairsPerBlock;
  if (nblocks <= 1) {
    MOE_LAUNCH(dispatch_rank_kernel<true>, dim3(1), dim3(256), 0, stream, N, E, idx, nullptr, counts, offsets,
                       perm, inv_perm);
  } else {
    int32_t* hist = (int32_t*)ws;
    int32_t* base = hist + nblocks * E;
    MOE_LAUNCH(dispatch_hist_kernel, dim3((unsigned)nblocks), dim3(256), 0, stream, N, E, idx, hist);
    MOE_LAUNCH(dispatch_scan_kernel, dim3(1), dim3(256), 0, stream, (int)nblocks, E, hist, base, counts,
                       offsets);
    MOE_LAUNCH(dispatch_rank_kernel<false>, dim3((unsigned)nblocks), dim3(256), 0, stream, N, E, idx, base,
                       counts, offsets, perm, inv_perm);
  }
  return hipGetLastError();
}

hipError_t launch_dispatch_rows(int T, int H, int k, int esize, const void* x, const int32_t* inv_perm, void* x_sorted,
                                hipStream_t stream) {
  const int row_chunks = (int)((int64_t)H * esize / 16);
  const int64_t items = (int64_t)T * ((row_chunks + 255) / 256);
  const int64_t want = (items + 1) / 2;  // two items per workgroup: one load in flight under the other's stores
  const int grid = (int)(want < kRowCopyBlocks ? want : kRowCopyBlocks);
  if (grid <= 0) return hipSuccess;
  MOE_LAUNCH(dispatch_rows_kernel, dim3(grid), dim3(256), 0, stream, T, k, row_chunks, (const u32x4*)x,
                     inv_perm, (u32x4*)x_sorted);
  return hipGetLastError();
}

}  // namespace moe
