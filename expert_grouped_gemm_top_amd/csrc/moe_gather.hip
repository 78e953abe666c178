// moe_gather.hip -- HBM-bound row kernels around the grouped GEMMs:
//   combine   out[t] = sum_j w[t,j] * rows[inv[t*k+j]]     (router-weighted combine;
//             with unit weight it sums expert input-gradients into dx)
//   dO / dg   dO_rows[inv[p]] = w[p] * dy[t];  dg[p] = <dy[t], o_sorted[inv_all[p]]>
//   gather    compacted copies of kept rows (x, a, h) by source position
// Results are scattered back per token and weighted by the router (npu-train
// issue #14, section Proposal); the backward restricted to retained pairs and
// the physical compaction follow the LRMoE abstract.
//
// Every thread moves 8 elements (16 B of bf16, 32 B of fp32) per step; a token
// row is read once and its k expert rows are gathered with full-row coalesced
// loads.  Sums run in fp32 in ascending j and are rounded once.
#include <algorithm>

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

namespace {

template <typename T>
struct Vec8;
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float* v) {
    const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  // the same, for data this step reads once (non-temporal hint)
  static __device__ __forceinline__ void load_once(const float* p, float* v) {
    const f32x4 a = __builtin_nontemporal_load((const f32x4*)p), b = __builtin_nontemporal_load((const f32x4*)(p + 4));
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
};
template <>
struct Vec8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* v) { unpack(*(const u32x4*)p, v); }
  static __device__ __forceinline__ void load_once(const uint16_t* p, float* v) {
    unpack(__builtin_nontemporal_load((const u32x4*)p), v);
  }
  static __device__ __forceinline__ void unpack(const u32x4 a, float* v) {
    v[0] = bf_lo(a.x); v[1] = bf_hi(a.x); v[2] = bf_lo(a.y); v[3] = bf_hi(a.y);
    v[4] = bf_lo(a.z); v[5] = bf_hi(a.z); v[6] = bf_lo(a.w); v[7] = bf_hi(a.w);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    *(u32x4*)p = u32x4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])};
  }
};

// The k pair slots of a token are handled with KP >= k compile-time slots
// (KP a power of two); every row load is issued before any of them is used.
// Slots past k and skipped pairs (inv < 0) load a harmless in-bounds address
// (the token's own row of another tensor) and are masked out by a select, so
// the loads need no branches and stay in flight together.

// One thread per (token, 16-byte chunk of the row).  HAS_W: router weights
// given (else every weight is 1).
template <typename T, int KP, bool HAS_W>
__global__ __launch_bounds__(128) void combine_kernel(int Tn, int H, int k, const T* __restrict__ rows,
                                                      const int32_t* __restrict__ inv, const float* __restrict__ w,
                                                      T* __restrict__ out) {
  const int chunks = H / 8;
  const int64_t items = (int64_t)Tn * chunks;
  for (int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; it < items; it += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(it / chunks), c = (int)(it % chunks);
    int src[KP];
    float wt[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      const size_t p = (size_t)t * k + (j < k ? j : k - 1);  // in bounds: loads need no branch
      const int32_t iv = inv[p];
      src[j] = (j < k) ? iv : -1;
      wt[j] = HAS_W ? w[p] : 1.0f;
    }
    T* orow = out + (size_t)t * H + c * 8;
    float v[KP][8];
#pragma unroll
    for (int j = 0; j < KP; ++j)
      Vec8<T>::load_once(src[j] >= 0 ? rows + (size_t)src[j] * H + c * 8 : (const T*)orow, v[j]);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < KP; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = (src[j] >= 0) ? acc[i] + wt[j] * v[j][i] : acc[i];
    Vec8<T>::store(orow, acc);
  }
}

// One block per token (dg needs a block-wide dot product per pair).  DG: dg is
// wanted (o_sorted and inv_all are then valid; a pair without a row reads row 0
// and is masked).
template <typename T, int KP, bool DG>
__global__ __launch_bounds__(256) void grad_rows_kernel(int Tn, int H, int k, const T* __restrict__ dy,
                                                        const float* __restrict__ w, const int32_t* __restrict__ inv,
                                                        T* __restrict__ dO_rows, const int32_t* __restrict__ inv_all,
                                                        const T* __restrict__ o_sorted, float* __restrict__ dg) {
  __shared__ float s_part[4][KP];
  const int chunks = H / 8;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  for (int t = blockIdx.x; t < Tn; t += gridDim.x) {
    // lane j of every wave fetches slot j's indices (one load per array, all
    // in flight together); the slots are then broadcast from those lanes
    const size_t pl = (size_t)t * k + (lane < k ? lane : k - 1);
    const int32_t inv_l = inv[pl];
    const float w_l = w[pl];
    const int32_t ia_l = DG ? inv_all[pl] : -1;
    int dst[KP], osrc[KP];
    float wt[KP], dot[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      dst[j] = (j < k) ? __builtin_amdgcn_readlane(inv_l, j) : -1;
      wt[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), j));
      osrc[j] = (DG && j < k) ? __builtin_amdgcn_readlane(ia_l, j) : -1;
      dot[j] = 0.0f;
    }
    const T* dyrow = dy + (size_t)t * H;
    for (int c = tid; c < chunks; c += 256) {
      float g[8];
      Vec8<T>::load_once(dyrow + c * 8, g);
      float o[KP][8];
      if constexpr (DG) {
#pragma unroll
        for (int j = 0; j < KP; ++j)
          Vec8<T>::load_once(o_sorted + (size_t)(osrc[j] >= 0 ? osrc[j] : 0) * H + c * 8, o[j]);
      }
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        if (dst[j] >= 0) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = wt[j] * g[i];
          Vec8<T>::store(dO_rows + (size_t)dst[j] * H + c * 8, v);
        }
        if constexpr (DG) {
          float s = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) s += g[i] * o[j][i];
          dot[j] += (osrc[j] >= 0) ? s : 0.0f;
        }
      }
    }
    if constexpr (DG) {
#pragma unroll
      for (int j = 0; j < KP; ++j) {
        const float s = wave_sum(dot[j]);
        if (lane == 0) s_part[wv][j] = s;
      }
      __syncthreads();
      if (tid < k) dg[(size_t)t * k + tid] = s_part[0][tid] + s_part[1][tid] + s_part[2][tid] + s_part[3][tid];
      __syncthreads();
    }
  }
}

// Pair scores for the quota selection: score[p] = w[p] * ||a_p|| * ||dy_t||,
// the Frobenius norm of pair p's rank-one term in dW_down (a_p = the pair's
// row of a_save, found through inv_perm; a pair without a row scores 0).  One
// block per token; sums of squares in fp32, reduced in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void pair_scores_kernel(int Tn, int H, int F, int k, const int32_t* __restrict__ inv,
                                                          const float* __restrict__ w, const T* __restrict__ a_rows,
                                                          const T* __restrict__ dy, float* __restrict__ score) {
  __shared__ float s_part[4];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  auto block_sum = [&](float v) {
    v = wave_sum(v);
    if (lane == 0) s_part[wv] = v;
    __syncthreads();
    const float r = s_part[0] + s_part[1] + s_part[2] + s_part[3];
    __syncthreads();
    return r;
  };
  for (int t = blockIdx.x; t < Tn; t += gridDim.x) {
    float q = 0.0f;
    for (int c = tid; c < H / 8; c += 256) {
      float v[8];
      Vec8<T>::load(dy + (size_t)t * H + c * 8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) q += v[i] * v[i];
    }
    const float ndy = sqrtf(block_sum(q));
    for (int j = 0; j < k; ++j) {
      const size_t p = (size_t)t * k + j;
      const int r = inv[p];
      float sa = 0.0f;
      if (r >= 0)
        for (int c = tid; c < F / 8; c += 256) {
          float v[8];
          Vec8<T>::load(a_rows + (size_t)r * F + c * 8, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) sa += v[i] * v[i];
        }
      const float na = sqrtf(block_sum(sa));
      if (tid == 0) score[p] = (r >= 0) ? w[p] * na * ndy : 0.0f;
    }
  }
}

// Row r < R = kept_offsets[E]: copy 16-byte chunks of up to three row sources.
__global__ __launch_bounds__(256) void gather_rows_kernel(const int32_t* __restrict__ R_ptr,
                                                          const int32_t* __restrict__ src, int max_rows,
                                                          const u32x4* __restrict__ a_src, u32x4* __restrict__ a_dst,
                                                          int a_chunks, const u32x4* __restrict__ b_src,
                                                          u32x4* __restrict__ b_dst, int b_chunks,
                                                          const u32x4* __restrict__ c_src, u32x4* __restrict__ c_dst,
                                                          int c_chunks) {
  const int R = *R_ptr;
  for (int r = blockIdx.x; r < R && r < max_rows; r += gridDim.x) {
    const size_t s = (size_t)src[r];
    if (a_src)
      for (int c = threadIdx.x; c < a_chunks; c += 256) a_dst[(size_t)r * a_chunks + c] = a_src[s * a_chunks + c];
    if (b_src)
      for (int c = threadIdx.x; c < b_chunks; c += 256) b_dst[(size_t)r * b_chunks + c] = b_src[s * b_chunks + c];
    if (c_src)
      for (int c = threadIdx.x; c < c_chunks; c += 256) c_dst[(size_t)r * c_chunks + c] = c_src[s * c_chunks + c];
  }
}

inline int token_grid(int T) { return T < 16384 ? T : 16384; }


template <typename T, int KP>
void launch_combine_kp(int T_, int H, int k, const void* rows, const int32_t* inv, const float* w, void* out,
                       hipStream_t stream) {
  const int64_t items = (int64_t)T_ * (H / 8);
  const int64_t blocks = std::min<int64_t>((items + 127) / 128, 65536);
  if (w != nullptr)
    MOE_LAUNCH((combine_kernel<T, KP, true>), dim3((unsigned)blocks), dim3(128), 0, stream, T_, H, k,
                       (const T*)rows, inv, w, (T*)out);
  else
    MOE_LAUNCH((combine_kernel<T, KP, false>), dim3((unsigned)blocks), dim3(128), 0, stream, T_, H, k,
                       (const T*)rows, inv, w, (T*)out);
}

template <typename T, int KP>
void launch_grad_rows_kp(int T_, int H, int k, const void* dy, const float* w, const int32_t* inv, void* dO_rows,
                         const int32_t* inv_all, const void* o_sorted, float* dg, hipStream_t stream) {
  if (dg != nullptr)
    MOE_LAUNCH((grad_rows_kernel<T, KP, true>), dim3(token_grid(T_)), dim3(256), 0, stream, T_, H, k,
                       (const T*)dy, w, inv, (T*)dO_rows, inv_all, (const T*)o_sorted, dg);
  else
    MOE_LAUNCH((grad_rows_kernel<T, KP, false>), dim3(token_grid(T_)), dim3(256), 0, stream, T_, H, k,
                       (const T*)dy, w, inv, (T*)dO_rows, inv_all, (const T*)o_sorted, dg);
}

// k -> the smallest power-of-two slot count KP >= k (k <= 16)
template <typename T, template <typename, int> class L, typename... A>
void dispatch_kp(int k, A... a) {
  if (k <= 1) L<T, 1>::run(a...);
  else if (k <= 2) L<T, 2>::run(a...);
  else if (k <= 4) L<T, 4>::run(a...);
  else if (k <= 8) L<T, 8>::run(a...);
  else L<T, 16>::run(a...);
}

template <typename T, int KP>
struct CombineL {
  static void run(int T_, int H, int k, const void* rows, const int32_t* inv, const float* w, void* out,
                  hipStream_t s) {
    launch_combine_kp<T, KP>(T_, H, k, rows, inv, w, out, s);
  }
};
template <typename T, int KP>
struct GradRowsL {
  static void run(int T_, int H, int k, const void* dy, const float* w, const int32_t* inv, void* dO_rows,
                  const int32_t* inv_all, const void* o_sorted, float* dg, hipStream_t s) {
    launch_grad_rows_kp<T, KP>(T_, H, k, dy, w, inv, dO_rows, inv_all, o_sorted, dg, s);
  }
};

}  // namespace

hipError_t launch_combine(int T, int H, int k, int esize, const void* rows, const int32_t* inv, const float* w,
                          void* out, hipStream_t stream) {
  if (esize == 4)
    dispatch_kp<float, CombineL>(k, T, H, k, rows, inv, w, out, stream);
  else
    dispatch_kp<uint16_t, CombineL>(k, T, H, k, rows, inv, w, out, stream);
  return hipGetLastError();
}

hipError_t launch_grad_rows(int T, int H, int k, int esize, const void* dy, const float* w, const int32_t* inv,
                            void* dO_rows, const int32_t* inv_all, const void* o_sorted, float* dg,
                            hipStream_t stream) {
  if (esize == 4)
    dispatch_kp<float, GradRowsL>(k, T, H, k, dy, w, inv, dO_rows, inv_all, o_sorted, dg, stream);
  else
    dispatch_kp<uint16_t, GradRowsL>(k, T, H, k, dy, w, inv, dO_rows, inv_all, o_sorted, dg, stream);
  return hipGetLastError();
}

hipError_t launch_pair_scores(int T, int H, int F, int k, int esize, const int32_t* inv, const float* w,
                              const void* a_rows, const void* dy, float* score, hipStream_t stream) {
  if (esize == 4)
    MOE_LAUNCH(pair_scores_kernel<float>, dim3(token_grid(T)), dim3(256), 0, stream, T, H, F, k, inv, w,
                       (const float*)a_rows, (const float*)dy, score);
  else
    MOE_LAUNCH(pair_scores_kernel<uint16_t>, dim3(token_grid(T)), dim3(256), 0, stream, T, H, F, k, inv, w,
                       (const uint16_t*)a_rows, (const uint16_t*)dy, score);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const int32_t* R_ptr, const int32_t* src, int max_rows, const void* a_src, void* a_dst,
                              int a_bytes, const void* b_src, void* b_dst, int b_bytes, const void* c_src,
                              void* c_dst, int c_bytes, hipStream_t stream) {
  if (max_rows <= 0) return hipSuccess;
  const int grid = max_rows < 65536 ? max_rows : 65536;
  MOE_LAUNCH(gather_rows_kernel, dim3(grid), dim3(256), 0, stream, R_ptr, src, max_rows,
                     (const u32x4*)a_src, (u32x4*)a_dst, a_bytes / 16, (const u32x4*)b_src, (u32x4*)b_dst,
                     b_bytes / 16, (const u32x4*)c_src, (u32x4*)c_dst, c_bytes / 16);
  return hipGetLastError();
}

}  // namespace moe
