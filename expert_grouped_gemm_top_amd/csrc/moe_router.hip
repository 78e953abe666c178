// moe_router.hip -- the router in front of the expert path: logits = x W_r, and
// its backward with the top-k selection held fixed.
//
// Routing precedes dispatch (npu-train issue #14, section Proposal), and the
// device path has to match the host path in gradients as well as outputs
// (issue #14, section Done when).  With the weights the softmax over the k
// selected logits, g_j = dL/dw[t,j] and s_t = sum_j w[t,j] g_j:
//     dlogits[t, idx_j] = w_j (g_j - s_t),  dlogits[t, e] = 0 otherwise,
//     dW_r = x^T dlogits,   dx += dlogits W_r^T.
//
// The three products are small next to the experts' (E columns against k * 3F).
// In bf16 layers they run on the 16x16x32 bf16 matrix core: 64 x 64 output
// tiles, four waves of 16 rows, operands staged through LDS as [row][k] bf16
// whatever their layout in memory; the fp32 operand (dlogits) enters as two
// bf16 parts, hi = bf16(v) and lo = bf16(v - hi), multiplied separately, so
// its precision is kept to ~2^-16.  fp32 layers use a tiled fp32 kernel:
// 128 x 128 output tiles, reduction depth 16 per LDS stage, 8 x 8 outputs per
// thread.  Two of the products have few outputs and a long reduction
// (logits: T x E over H; dW_r: H x E over T), so the reduction is cut into S
// slices run by separate workgroups that write fp32 partial tiles to the
// caller's workspace; a second kernel adds the S partials of each output in
// slice order and rounds once.  Every output is thus reduced in one fixed
// order (deterministic, no atomics).
#include <algorithm>
#include <type_traits>

#include "moe_common.h"
#include "moe_launch.h"
#include "moe_lds32.h"

namespace moe {

namespace {

constexpr int kRBK = 16;  // LDS depth
// Output tiles are TILE x TILE (64 or 128), TILE / 16 x TILE / 16 outputs per thread.

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf2f(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return (uint16_t)f2bf(v); }

// C[M,N] (+)= sum_k A(m,k) B(k,n).  A(m,k) = a[m*lda + k] when A_KC (k
// contiguous), else a[k*lda + m]; B(k,n) = b[n*ldb + k] when B_KC, else
// b[k*ldb + n].  C is row-major with leading dimension N; ACC adds the product
// to C's current contents (one rounding of the sum).  With slices > 1,
// workgroup z reduces k in [z*kslice, (z+1)*kslice) and writes its fp32 partial
// tile to part + z*M*N instead (C, ACC unused).
template <int TILE, typename TA, typename TB, typename TC, bool A_KC, bool B_KC, bool ACC>
__global__ __launch_bounds__(256) void router_gemm_kernel(int M, int N, int K, const TA* __restrict__ a, int lda,
                                                          const TB* __restrict__ b, int ldb, TC* __restrict__ c,
                                                          int kslice, float* __restrict__ part) {
  constexpr int kRBM = TILE, kRBN = TILE, TPT = TILE / 16;
  __shared__ __attribute__((aligned(16))) float s_a[kRBK][kRBM];
  __shared__ __attribute__((aligned(16))) float s_b[kRBK][kRBN];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.x * kRBM, n0 = blockIdx.y * kRBN;
  const int kb0 = blockIdx.z * kslice, kb1 = min(K, kb0 + kslice);
  // thread (tx, ty) owns rows 64 (i / 4) + 4 ty + i % 4 and columns
  // 64 (j / 4) + 4 tx + j % 4 (i, j < TPT): its LDS reads are float4s that
  // neighbouring threads take from neighbouring addresses
  float acc[TPT][TPT] = {};
  for (int k0 = kb0; k0 < kb1; k0 += kRBK) {
#pragma unroll
    for (int i = 0; i < kRBM * kRBK / 256; ++i) {
      const int q = tid + 256 * i;  // element of the 128 x 16 tile
      // walk the contiguous index fastest so that neighbouring threads read
      // neighbouring addresses
      const int mm = A_KC ? q / kRBK : q % kRBM, kk = A_KC ? q % kRBK : q / kRBM;
      const int m = m0 + mm, k = k0 + kk;
      float v = 0.0f;
      if (m < M && k < kb1) v = to_f32<TA>(A_KC ? a[(size_t)m * lda + k] : a[(size_t)k * lda + m]);
      s_a[kk][mm] = v;
      const int nn = B_KC ? q / kRBK : q % kRBN, kb = B_KC ? q % kRBK : q / kRBN;
      const int n = n0 + nn, kq = k0 + kb;
      float u = 0.0f;
      if (n < N && kq < kb1) u = to_f32<TB>(B_KC ? b[(size_t)n * ldb + kq] : b[(size_t)kq * ldb + n]);
      s_b[kb][nn] = u;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRBK; ++kk) {
      float av[TPT], bv[TPT];
#pragma unroll
      for (int h = 0; h < TPT / 4; ++h) {
        const f32x4 a4 = *(const f32x4*)&s_a[kk][64 * h + 4 * ty];
        const f32x4 b4 = *(const f32x4*)&s_b[kk][64 * h + 4 * tx];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          av[4 * h + u] = a4[u];
          bv[4 * h + u] = b4[u];
        }
      }
#pragma unroll
      for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int j = 0; j < TPT; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < TPT; ++i) {
    const int m = m0 + 64 * (i / 4) + 4 * ty + i % 4;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int n = n0 + 64 * (j / 4) + 4 * tx + j % 4;
      if (n >= N) continue;
      if (part != nullptr) {
        part[((size_t)blockIdx.z * M + m) * N + n] = acc[i][j];
      } else {
        TC* p = c + (size_t)m * N + n;
        const float v = ACC ? to_f32<TC>(*p) + acc[i][j] : acc[i][j];
        *p = from_f32<TC>(v);
      }
    }
  }
}

// The same product on the 16x16x32 bf16 matrix core (at least one operand bf16;
// an fp32 operand is split into bf16 hi and lo parts).  Workgroup = 64 x 64
// outputs, wave w owns rows 16 w .. 16 w + 15 and four 16-column blocks; the
// reduction advances kMK at a time.  Each thread moves kRuns runs of eight
// consecutive elements of each operand per k-step (a 16-byte load each, two
// for fp32), loaded one k-step ahead, and writes each to LDS as one 16-byte
// chunk in the operand's own memory order: [row][k] when k is contiguous in
// memory, else [k][row], whose fragments are read with the gfx950 transpose
// read ds_read_b64_tr_b16.  The output tile is staged through LDS so that
// every row leaves as 16-byte stores.  Same slicing and epilogue contract as router_gemm_kernel.
constexpr int kMT = 64, kMK = 32;  // (k-steps of 64 measured slower: fewer workgroups fit a CU)
constexpr int kRuns = kMT * kMK / (256 * 8);  // runs of eight elements per thread and operand tile
constexpr int kKcPitch = kMK + 8;  // [row][k] tiles: 80-byte rows
constexpr int kRcPitch = kMT + 8;  // [k][row] tiles: 144-byte rows (the 4 k rows of a transpose read hit distinct banks)
constexpr int kPart = kMT * kKcPitch;  // elements of one bf16 tile part (either layout)
constexpr int kCPitch = kMT + 4;       // fp32 output staging, floats per row
static_assert(kMK * kRcPitch <= kPart, "tile part size");

__device__ __forceinline__ f32x4 mfma16(u32x4 first, u32x4 second, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, first), __builtin_bit_cast(bf16x8, second),
                                                  acc, 0, 0, 0);
}

// Eight consecutive elements p[o * ld + c + j], j < 8, of an operand as fp32
// (zero where o >= olim or c + j >= clim): one 16-byte load (two for fp32)
// when the run is whole and aligned, else element by element.
template <typename T>
__device__ __forceinline__ void load_run(const T* __restrict__ p, int ld, int o, int olim, int c, int clim,
                                         float (&v)[8]) {
  const T* src = p + (size_t)(o < olim ? o : 0) * ld + c;
  if (o < olim && c + 8 <= clim && ((uintptr_t)src & 15) == 0) {
    if constexpr (std::is_same<T, float>::value) {
      const f32x4 lo = *(const f32x4*)src, hi = *(const f32x4*)(src + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] = lo[j];
        v[4 + j] = hi[j];
      }
    } else {
      const u32x4 r = *(const u32x4*)src;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf2f(r[j] & 0xffffu);
        v[2 * j + 1] = bf2f(r[j] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (o < olim && c + j < clim) ? to_f32<T>(src[j]) : 0.0f;
  }
}

// Run q (= thread + 256 i) of a 64 x kMK operand tile: KC (k contiguous) row
// q / (kMK / 8), k 8 (q % (kMK / 8)) .. + 7; otherwise k q / 8, rows
// 8 (q % 8) .. + 7.
static_assert(kMT == 64 && kMK % 32 == 0 && kRuns >= 1, "run mapping");
constexpr int kKcRuns = kMK / 8;  // runs per row of a KC tile
template <bool KC>
__device__ __forceinline__ int run_row(int q) { return KC ? q / kKcRuns : 8 * (q & 7); }
template <bool KC>
__device__ __forceinline__ int run_k(int q) { return KC ? 8 * (q % kKcRuns) : q >> 3; }

// The run as bf16 into part 0 of the tile (and, SPLIT, the residuals v - hi
// into part 1), one 16-byte chunk each.
template <bool KC, bool SPLIT>
__device__ __forceinline__ void store_run(uint16_t* s, int q, const float (&v)[8]) {
  const int off = KC ? run_row<KC>(q) * kKcPitch + run_k<KC>(q) : run_k<KC>(q) * kRcPitch + run_row<KC>(q);
  u32x4 hi, lo;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t h0 = f2bf(v[2 * j]), h1 = f2bf(v[2 * j + 1]);
    hi[j] = h0 | (h1 << 16);
    if constexpr (SPLIT) lo[j] = f2bf(v[2 * j] - bf2f(h0)) | (f2bf(v[2 * j + 1] - bf2f(h1)) << 16);
  }
  *(u32x4*)&s[off] = hi;
  if constexpr (SPLIT) *(u32x4*)&s[kPart + off] = lo;
}

// 16x16x32 fragment of tile rows row0 .. row0 + 15 and k k0 .. k0 + 31: lane
// l gets row row0 + l % 16, k k0 + 8 (l / 16) .. + 7.  From a [k][row] tile by
// two transpose reads: in 16-lane group G, lane r points at k row
// k0 + 8 G + 4 h + r / 4 and rows row0 + 4 (r % 4) .. + 3, and receives the 4 k
// of row row0 + r.
template <bool KC>
__device__ __forceinline__ u32x4 frag(const uint16_t* s, int row0, int k0) {
  const int l = __lane_id();
  if constexpr (KC) {
    return *(const u32x4*)&s[(row0 + (l & 15)) * kKcPitch + k0 + 8 * (l >> 4)];
  } else {
    const int G = l >> 4, r = l & 15;
    v4i16 q[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
      q[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(lds_void*)&s[(k0 + 8 * G + 4 * h + (r >> 2)) * kRcPitch + row0 + 4 * (r & 3)]);
    return u32x4{(uint32_t)(uint16_t)q[0][0] | ((uint32_t)(uint16_t)q[0][1] << 16),
                 (uint32_t)(uint16_t)q[0][2] | ((uint32_t)(uint16_t)q[0][3] << 16),
                 (uint32_t)(uint16_t)q[1][0] | ((uint32_t)(uint16_t)q[1][1] << 16),
                 (uint32_t)(uint16_t)q[1][2] | ((uint32_t)(uint16_t)q[1][3] << 16)};
  }
}

// Sixteen consecutive outputs of row m from the staging row, written (and for
// ACC added to the current contents) as 16-byte runs when whole and aligned.
template <typename TC, bool ACC>
__device__ __forceinline__ void store_out(TC* __restrict__ dst, const float* src, int cols) {
  constexpr int V = 16 / sizeof(TC);  // outputs per 16-byte chunk
  if (cols >= 16 && ((uintptr_t)dst & 15) == 0) {
#pragma unroll
    for (int q = 0; q < 16 / V; ++q) {
      if constexpr (std::is_same<TC, float>::value) {
        f32x4 o = *(const f32x4*)&src[4 * q];
        if constexpr (ACC) o += *(const f32x4*)&dst[4 * q];
        *(f32x4*)&dst[4 * q] = o;
      } else {
        u32x4 o;
        u32x4 cur;
        if constexpr (ACC) cur = *(const u32x4*)&dst[8 * q];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float v0 = src[8 * q + 2 * j], v1 = src[8 * q + 2 * j + 1];
          if constexpr (ACC) {
            v0 += bf2f(cur[j] & 0xffffu);
            v1 += bf2f(cur[j] >> 16);
          }
          o[j] = f2bf(v0) | (f2bf(v1) << 16);
        }
        *(u32x4*)&dst[8 * q] = o;
      }
    }
  } else {
    for (int j = 0; j < 16 && j < cols; ++j) {
      const float v = ACC ? to_f32<TC>(dst[j]) + src[j] : src[j];
      dst[j] = from_f32<TC>(v);
    }
  }
}

template <typename TA, typename TB, typename TC, bool A_KC, bool B_KC, bool ACC>
__global__ __launch_bounds__(256) void router_mfma_kernel(int M, int N, int K, const TA* __restrict__ a, int lda,
                                                          const TB* __restrict__ b, int ldb, TC* __restrict__ c,
                                                          int kslice, float* __restrict__ part) {
  constexpr bool SA = std::is_same<TA, float>::value, SB = std::is_same<TB, float>::value;  // split operands
  static_assert(!(SA && SB), "one operand is bf16");
  constexpr int PA = SA ? 2 : 1, PB = SB ? 2 : 1;
  constexpr int kOpBytes = (PA + PB) * kPart * 2, kOutBytes = kMT * kCPitch * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kOpBytes > kOutBytes ? kOpBytes : kOutBytes];
  uint16_t* s_a = (uint16_t*)smem;
  uint16_t* s_b = s_a + PA * kPart;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int m0 = blockIdx.x * kMT, n0 = blockIdx.y * kMT;
  const int kb0 = blockIdx.z * kslice, kb1 = min(K, kb0 + kslice);
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ra[kRuns][8], rb[kRuns][8];  // the next k-step's runs, loaded while this one computes
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kRuns; ++i) {
      const int q = tid + 256 * i;
      const int ar = m0 + run_row<A_KC>(q), ak = k0 + run_k<A_KC>(q);
      if constexpr (A_KC) load_run(a, lda, ar, M, ak, kb1, ra[i]);
      else load_run(a, lda, ak, kb1, ar, M, ra[i]);
      const int br = n0 + run_row<B_KC>(q), bk = k0 + run_k<B_KC>(q);
      if constexpr (B_KC) load_run(b, ldb, br, N, bk, kb1, rb[i]);
      else load_run(b, ldb, bk, kb1, br, N, rb[i]);
    }
  };
  if (kb0 < kb1) gload(kb0);
  for (int k0 = kb0; k0 < kb1; k0 += kMK) {
#pragma unroll
    for (int i = 0; i < kRuns; ++i) {
      store_run<A_KC, SA>(s_a, tid + 256 * i, ra[i]);
      store_run<B_KC, SB>(s_b, tid + 256 * i, rb[i]);
    }
    __syncthreads();
    if (k0 + kMK < kb1) gload(k0 + kMK);
#pragma unroll
    for (int ks = 0; ks < kMK; ks += 32) {
      const u32x4 af = frag<A_KC>(s_a, 16 * w, ks);
      u32x4 al;
      if constexpr (SA) al = frag<A_KC>(s_a + kPart, 16 * w, ks);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 bf = frag<B_KC>(s_b, 16 * j, ks);
        acc[j] = mfma16(af, bf, acc[j]);
        if constexpr (SA) acc[j] = mfma16(al, bf, acc[j]);
        if constexpr (SB) acc[j] = mfma16(af, frag<B_KC>(s_b + kPart, 16 * j, ks), acc[j]);
      }
    }
    __syncthreads();
  }
  // register rr of lane l in block j: tile row 16 w + 4 (l / 16) + rr, column
  // 16 j + l % 16 -> staging; then thread t writes row t / 4, columns
  // 16 (t % 4) .. + 15
  float* s_c = (float*)smem;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) s_c[(16 * w + 4 * (l >> 4) + rr) * kCPitch + 16 * j + (l & 15)] = acc[j][rr];
  __syncthreads();
  const int r = tid >> 2, c0 = 16 * (tid & 3);
  const int m = m0 + r, n = n0 + c0;
  if (m >= M || n >= N) return;
  const float* src = &s_c[r * kCPitch + c0];
  if (part != nullptr) store_out<float, false>(part + ((size_t)blockIdx.z * M + m) * N + n, src, N - n);
  else store_out<TC, ACC>(c + (size_t)m * N + n, src, N - n);
}

// c[i] = sum_{z < slices} part[z*MN + i], z ascending, rounded once.
template <typename TC>
__global__ __launch_bounds__(256) void router_sum_slices_kernel(int64_t MN, int slices, const float* __restrict__ part,
                                                                TC* __restrict__ c) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < MN; i += (int64_t)gridDim.x * 256) {
    float v = 0.0f;
    for (int z = 0; z < slices; ++z) v += part[z * MN + i];
    c[i] = from_f32<TC>(v);
  }
}

// One wavefront per token: s = sum_j w_j g_j (wave tree), then every lane
// writes its experts' entries of the token's dlogits row exactly once.
__global__ __launch_bounds__(256) void router_dlogits_kernel(int T, int E, int k, const int32_t* __restrict__ idx,
                                                             const float* __restrict__ w, const float* __restrict__ dg,
                                                             float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // whole wave
  const size_t p = (size_t)t * k + (lane < k ? lane : k - 1);
  const int32_t e_l = idx[p];
  const float w_l = w[p], g_l = dg[p];
  const float s = wave_sum(lane < k ? w_l * g_l : 0.0f);
  const float d_l = w_l * (g_l - s);
  for (int e = lane; e < E; e += kWave) {
    float v = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int ej = __builtin_amdgcn_readlane(e_l, j);
      const float dj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d_l), j));
      if (ej == e) v = dj;
    }
    dl[(size_t)t * E + e] = v;
  }
}

// Reduction slices of an M x N x K product: enough workgroups to cover the
// chip (about kTargetGroups), each slice a multiple of the LDS depth.
constexpr int64_t kTargetGroups = 512;
constexpr int kMinSlice = 128;

int64_t slices_for(int64_t tiles, int K, bool may_split) {
  if (!may_split) return 1;
  int64_t s = (kTargetGroups + tiles - 1) / tiles;
  s = std::min<int64_t>(s, (K + kMinSlice - 1) / kMinSlice);
  return std::max<int64_t>(s, 1);
}

// 128 x 128 tiles when they (with their reduction slices) give enough
// workgroups to cover the chip, else 64 x 64
int tile_of(int M, int N, int K, bool may_split) {
  const int64_t t128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
  return t128 * slices_for(t128, K, may_split) >= 256 ? 128 : 64;
}

// (the matrix-core kernel takes the same slices over its 64 x 64 tiles; a
// chip-sized grid of workgroups that walk the tiles measured slower)
int64_t slice_count(int M, int N, int K, bool may_split = true) {
  const int tile = tile_of(M, N, K, may_split);
  const int64_t tiles = (int64_t)((M + tile - 1) / tile) * ((N + tile - 1) / tile);
  return slices_for(tiles, K, may_split);
}

int slice_length(int K, int64_t slices) {
  // a multiple of both kernels' reduction step (16 and 32)
  const int64_t per = (K + slices - 1) / slices;
  return (int)((per + kMK - 1) / kMK * kMK);
}

size_t split_bytes(int M, int N, int K) {
  const int64_t s = slice_count(M, N, K);
  return s > 1 ? (size_t)s * M * N * sizeof(float) : 0;
}

// Plain launch (one slice) or the sliced reduction through `ws`.
template <typename TA, typename TB, typename TC, bool A_KC, bool B_KC, bool ACC>
hipError_t gemm(int M, int N, int K, const void* a, int lda, const void* b, int ldb, void* c, float* ws,
                bool may_split, hipStream_t stream) {
  const int64_t slices = slice_count(M, N, K, may_split);
  const int kslice = slices > 1 ? slice_length(K, slices) : K;
  const int64_t used = (K + kslice - 1) / kslice;  // slices that hold some k
  const int tile = tile_of(M, N, K, may_split);
  const dim3 grid((M + tile - 1) / tile, (N + tile - 1) / tile, (unsigned)(slices > 1 ? used : 1));
  float* part = slices > 1 ? ws : nullptr;
  if constexpr (!std::is_same<TA, float>::value || !std::is_same<TB, float>::value) {
    // bf16 layer: the matrix core, 64 x 64 tiles
    const dim3 mgrid((M + kMT - 1) / kMT, (N + kMT - 1) / kMT, grid.z);
    MOE_LAUNCH((router_mfma_kernel<TA, TB, TC, A_KC, B_KC, ACC>), mgrid, dim3(256), 0, stream, M, N, K,
                       (const TA*)a, lda, (const TB*)b, ldb, (TC*)c, kslice, part);
  } else if (tile == 128)
    MOE_LAUNCH((router_gemm_kernel<128, TA, TB, TC, A_KC, B_KC, ACC>), grid, dim3(256), 0, stream, M, N, K,
                       (const TA*)a, lda, (const TB*)b, ldb, (TC*)c, kslice, part);
  else
    MOE_LAUNCH((router_gemm_kernel<64, TA, TB, TC, A_KC, B_KC, ACC>), grid, dim3(256), 0, stream, M, N, K,
                       (const TA*)a, lda, (const TB*)b, ldb, (TC*)c, kslice, part);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || slices == 1) return err;
  const int64_t MN = (int64_t)M * N;
  const int64_t blocks = std::min<int64_t>((MN + 255) / 256, 4096);
  MOE_LAUNCH((router_sum_slices_kernel<TC>), dim3((unsigned)blocks), dim3(256), 0, stream, MN, (int)used,
                     (const float*)ws, (TC*)c);
  return hipGetLastError();
}

template <typename T>
hipError_t router_bwd_typed(int T_, int H, int E, int k, const void* x, const void* w_r, const int32_t* idx,
                            const float* w, const float* dg, float* dl, void* dw_r, void* dx, bool dx_acc,
                            float* ws, hipStream_t stream) {
  MOE_LAUNCH(router_dlogits_kernel, dim3((T_ + 3) / 4), dim3(256), 0, stream, T_, E, k, idx, w, dg, dl);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // dW_r [H,E] = x^T dl: A(h,t) = x[t*H + h], B(t,e) = dl[t*E + e]; reduction over T
  err = gemm<T, float, T, false, false, false>(H, E, T_, x, H, dl, E, dw_r, ws, true, stream);
  if (err != hipSuccess) return err;
  // dx [T,H] (+)= dl W_r^T: A(t,e) = dl[t*E + e], B(e,h) = w_r[h*E + e]; reduction over E only
  if (dx_acc) return gemm<float, T, T, true, true, true>(T_, H, E, dl, E, w_r, E, dx, nullptr, false, stream);
  return gemm<float, T, T, true, true, false>(T_, H, E, dl, E, w_r, E, dx, nullptr, false, stream);
}

}  // namespace

size_t router_workspace_bytes(int T, int H, int E) {
  return std::max(split_bytes(T, E, H), split_bytes(H, E, T));
}

hipError_t launch_router_fwd(int T, int H, int E, int esize, const void* x, const void* w_r, float* logits, void* ws,
                             hipStream_t stream) {
  // logits [T,E] = x W_r: A(t,h) = x[t*H + h], B(h,e) = w_r[h*E + e]; reduction over H
  if (esize == 4)
    return gemm<float, float, float, true, false, false>(T, E, H, x, H, w_r, E, logits, (float*)ws, true, stream);
  return gemm<uint16_t, uint16_t, float, true, false, false>(T, E, H, x, H, w_r, E, logits, (float*)ws, true, stream);
}

hipError_t launch_router_bwd(int T, int H, int E, int k, int esize, const void* x, const void* w_r,
                             const int32_t* idx, const float* w, const float* dg, float* dlogits, void* dw_r,
                             void* dx, bool dx_accumulate, void* ws, hipStream_t stream) {
  if (esize == 4)
    return router_bwd_typed<float>(T, H, E, k, x, w_r, idx, w, dg, dlogits, dw_r, dx, dx_accumulate, (float*)ws,
                                   stream);
  return router_bwd_typed<uint16_t>(T, H, E, k, x, w_r, idx, w, dg, dlogits, dw_r, dx, dx_accumulate, (float*)ws,
                                    stream);
}

}  // namespace moe
