// moe_common.h -- device-side helpers shared by the gfx950 kernels of libmoe.
//
// Element storage: activations and weights are either fp32 or bf16 (held as
// uint16_t bit patterns).  Every accumulation is fp32; bf16 values are produced
// only at stores, rounded to nearest even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kMaxExperts = 256; // expert ids fit in 8 bits; one thread per expert in a 256-wide block
constexpr int kMaxTopK = 16;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) { return f2bf(lo) | (f2bf(hi) << 16); }

__device__ __forceinline__ float sigmoidf_fast(float z) { return 1.0f / (1.0f + __expf(-z)); }

// 64 bytes of zeros in device memory, never written: the load source of every
// 16-byte operand chunk that lies past the end of a reduction (K not a multiple
// of the stage depth), so that such chunks contribute nothing and the loads
// stay unpredicated (direct global->LDS loads cannot be zeroed in flight).
static __device__ __attribute__((aligned(64))) uint32_t kZeroChunk[16];
__device__ __forceinline__ const uint16_t* zero_chunk() { return reinterpret_cast<const uint16_t*>(kZeroChunk); }

// ---- wave-level primitives -------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  // bit i set for every lane i below the calling lane (v_mbcnt based)
  const int l = __lane_id();
  return (l == 0) ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int l = __lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (l >= o) v += u;
  }
  return v;
}

// Exclusive scan over a 256-thread block; `total` receives the block sum.
// s_tmp needs 4 ints of shared memory.
__device__ __forceinline__ int block256_exclusive_scan(int v, int* s_tmp, int& total) {
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int inc = wave_inclusive_scan(v);
  if (l == 63) s_tmp[w] = inc;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) base += (i < w) ? s_tmp[i] : 0;
  total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
  __syncthreads();
  return base + inc - v;
}

// ---- ragged per-expert tile schedule ---------------------------------------
// Given device offsets[0..E] (rows of expert e are [offsets[e], offsets[e+1])),
// every workgroup derives the prefix of per-expert tile counts ceil(n_e / rows)
// itself and finds the (expert, tile) that a linear tile id falls on.  No host
// synchronisation and no padding of experts to a fixed bucket.
struct TileSlot {
  int expert;      // -1 when the id is past the last real tile
  int tile;        // tile index within the expert
  int row_begin;   // first row of the tile
  int rows;        // rows in this tile (1..tile_rows)
  int expert_rows; // n_e
};

// Block-level part: s_start[e] = first tile id of expert e, s_start[E] = total;
// s_off = offsets.  s_start and s_off need kMaxExperts + 1 ints, s_tmp 4 ints.
// Must be called by all 256 threads of the block.
// Only experts with min_rows <= n_e < max_rows get tiles (the others are served
// by a kernel tuned for their row count).
__device__ __forceinline__ void build_tile_starts(const int32_t* __restrict__ offsets, int E, int tile_rows,
                                                  int* s_start, int* s_off, int* s_tmp, int min_rows = 0,
                                                  int max_rows = 0x7fffffff) {
  const int tid = threadIdx.x;
  for (int i = tid; i <= E; i += 256) s_off[i] = offsets[i];  // E + 1 entries: 257 at E = 256
  __syncthreads();
  int n_tiles = 0;
  if (tid < E) {
    const int n = s_off[tid + 1] - s_off[tid];
    if (n >= min_rows && n < max_rows) n_tiles = (n + tile_rows - 1) / tile_rows;
  }
  int total;
  const int start = block256_exclusive_scan(n_tiles, s_tmp, total);
  if (tid < E) s_start[tid] = start;
  if (tid == 0) s_start[E] = total;
  __syncthreads();
}

// XCD-aware order.  Workgroups are dealt round-robin to the 8 XCDs, each with
// its own L2.  Map workgroup `wg` of a launch segment to a work item so that
// every XCD walks a contiguous range of the `real` items (neighbouring items
// share rows or weights and then meet in one L2), while the real items stay
// spread evenly over the XCDs when the grid was sized for more items than
// exist.  A bijection on [0, real & ~7); the identity elsewhere.
__device__ __forceinline__ int xcd_item(int wg, int real) {
  const int r8 = real & ~7;
  if (wg >= r8) return wg;
  return (wg & 7) * (r8 >> 3) + (wg >> 3);
}

// Per-thread part: the slot of `tile_id` (binary search over s_start).
__device__ __forceinline__ TileSlot lookup_tile(const int* s_start, const int* s_off, int E, int tile_rows,
                                                int tile_id) {
  TileSlot s;
  if (tile_id >= s_start[E]) {
    s.expert = -1;
    s.tile = s.row_begin = s.rows = s.expert_rows = 0;
    return s;
  }
  int lo = 0, hi = E;  // invariant: s_start[lo] <= tile_id < s_start[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_start[mid] <= tile_id) lo = mid; else hi = mid;
  }
  s.expert = lo;
  s.tile = tile_id - s_start[lo];
  s.expert_rows = s_off[lo + 1] - s_off[lo];
  s.row_begin = s_off[lo] + s.tile * tile_rows;
  const int left = s_off[lo + 1] - s.row_begin;
  s.rows = left < tile_rows ? left : tile_rows;
  return s;
}

}  // namespace moe
