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
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *(f32x4*)p = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
  }
};
template <>
struct Vec8<uint16_t> {
  static __device__ __forceinline__ void load(const uint16_t* p, float* v) {
    const u32x4 a = *(const u32x4*)p;
    v[0] = bf_lo(a.x); v[1] = bf_hi(a.x); v[2] = bf_lo(a.y); v[3] = bf_hi(a.y);
    v[4] = bf_lo(a.z); v[5] = bf_hi(a.z); v[6] = bf_lo(a.w); v[7] = bf_hi(a.w);
  }
  static __device__ __forceinline__ void store(uint16_t* p, const float* v) {
    *(u32x4*)p = u32x4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])};
  }
};

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(int Tn, int H, int k, const T* __restrict__ rows,
                                                      const int32_t* __restrict__ inv, const float* __restrict__ w,
                                                      T* __restrict__ out) {
  const int chunks = H / 8;
  for (int t = blockIdx.x; t < Tn; t += gridDim.x) {
    int src[kMaxTopK];
    float wt[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      src[j] = (j < k) ? inv[(size_t)t * k + j] : -1;
      wt[j] = (j < k && w != nullptr) ? w[(size_t)t * k + j] : 1.0f;
    }
    for (int c = threadIdx.x; c < chunks; c += 256) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k && src[j] >= 0) {
          float v[8];
          Vec8<T>::load(rows + (size_t)src[j] * H + c * 8, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += wt[j] * v[i];
        }
      }
      Vec8<T>::store(out + (size_t)t * H + c * 8, acc);
    }
  }
}

// One block per token.  dg needs a block-wide dot product per pair.
template <typename T>
__global__ __launch_bounds__(256) void grad_rows_kernel(int Tn, int H, int k, const T* __restrict__ dy,
                                                        const float* __restrict__ w, const int32_t* __restrict__ inv,
                                                        T* __restrict__ dO_rows, const int32_t* __restrict__ inv_all,
                                                        const T* __restrict__ o_sorted, float* __restrict__ dg) {
  __shared__ float s_part[4][kMaxTopK];
  const int chunks = H / 8;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  for (int t = blockIdx.x; t < Tn; t += gridDim.x) {
    int dst[kMaxTopK], osrc[kMaxTopK];
    float wt[kMaxTopK], dot[kMaxTopK];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      const size_t p = (size_t)t * k + j;
      dst[j] = (j < k) ? inv[p] : -1;
      wt[j] = (j < k) ? w[p] : 0.0f;
      osrc[j] = (j < k && dg != nullptr) ? inv_all[p] : -1;
      dot[j] = 0.0f;
    }
    for (int c = tid; c < chunks; c += 256) {
      float g[8];
      Vec8<T>::load(dy + (size_t)t * H + c * 8, g);
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k && dst[j] >= 0) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = wt[j] * g[i];
          Vec8<T>::store(dO_rows + (size_t)dst[j] * H + c * 8, v);
        }
        if (j < k && osrc[j] >= 0) {
          float o[8];
          Vec8<T>::load(o_sorted + (size_t)osrc[j] * H + c * 8, o);
          float s = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; ++i) s += g[i] * o[i];
          dot[j] += s;
        }
      }
    }
    if (dg != nullptr) {
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        if (j < k) {
          const float s = wave_sum(dot[j]);
          if (lane == 0) s_part[wv][j] = s;
        }
      }
      __syncthreads();
      if (tid < k) dg[(size_t)t * k + tid] = s_part[0][tid] + s_part[1][tid] + s_part[2][tid] + s_part[3][tid];
      __syncthreads();
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

}  // namespace

hipError_t launch_combine(int T, int H, int k, int esize, const void* rows, const int32_t* inv, const float* w,
                          void* out, hipStream_t stream) {
  if (esize == 4)
    hipLaunchKernelGGL(combine_kernel<float>, dim3(token_grid(T)), dim3(256), 0, stream, T, H, k,
                       (const float*)rows, inv, w, (float*)out);
  else
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3(token_grid(T)), dim3(256), 0, stream, T, H, k,
                       (const uint16_t*)rows, inv, w, (uint16_t*)out);
  return hipGetLastError();
}

hipError_t launch_grad_rows(int T, int H, int k, int esize, const void* dy, const float* w, const int32_t* inv,
                            void* dO_rows, const int32_t* inv_all, const void* o_sorted, float* dg,
                            hipStream_t stream) {
  if (esize == 4)
    hipLaunchKernelGGL(grad_rows_kernel<float>, dim3(token_grid(T)), dim3(256), 0, stream, T, H, k,
                       (const float*)dy, w, inv, (float*)dO_rows, inv_all, (const float*)o_sorted, dg);
  else
    hipLaunchKernelGGL(grad_rows_kernel<uint16_t>, dim3(token_grid(T)), dim3(256), 0, stream, T, H, k,
                       (const uint16_t*)dy, w, inv, (uint16_t*)dO_rows, inv_all, (const uint16_t*)o_sorted, dg);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const int32_t* R_ptr, const int32_t* src, int max_rows, const void* a_src, void* a_dst,
                              int a_bytes, const void* b_src, void* b_dst, int b_bytes, const void* c_src,
                              void* c_dst, int c_bytes, hipStream_t stream) {
  if (max_rows <= 0) return hipSuccess;
  const int grid = max_rows < 65536 ? max_rows : 65536;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(grid), dim3(256), 0, stream, R_ptr, src, max_rows,
                     (const u32x4*)a_src, (u32x4*)a_dst, a_bytes / 16, (const u32x4*)b_src, (u32x4*)b_dst,
                     b_bytes / 16, (const u32x4*)c_src, (u32x4*)c_dst, c_bytes / 16);
  return hipGetLastError();
}

}  // namespace moe
