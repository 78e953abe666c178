// moe_fp8.hip -- one-time fp8 storage of frozen expert weights, and the
// per-row quantization of activation rows for the fp8 matrix-core forward.
//
// In the LoRA step the experts are frozen (npu-train issue #14, section Scope)
// and their weights stay resident on the device (issue #14, section Proposal),
// so they can be stored once in 8 bits and widened in the GEMMs.  Element
// format: OCP 8-bit floating point E4M3 (1 sign, 4 exponent bits with bias 7,
// 3 mantissa bits, subnormals, no infinities, S.1111.111 = NaN, largest finite
// 448).  Each expert has one power-of-two scale s, the smallest with
// amax <= 448 s over all of that expert's matrices given together (W_gate and
// W_up share one), so w / s is exact and so is the product with s afterwards.
//
// One workgroup per expert: a block max of |w| over its matrices, then every
// element w -> E4M3(w / s), rounded to nearest with ties to the even mantissa.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

namespace {

// log2 of the smallest power of two s with amax <= 448 s (0 for amax = 0).
__device__ int fp8_scale_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  int k = (int)((__float_as_uint(amax) >> 23) & 0xff) - 127 - 8;  // near the answer; the loops make it exact
  while (448.0f * __builtin_ldexpf(1.0f, k) < amax) ++k;
  while (448.0f * __builtin_ldexpf(1.0f, k - 1) >= amax) --k;
  return k;
}

// E4M3 code of v (exact input); saturates beyond 448 in magnitude.
__device__ uint32_t e4m3_encode(float v) {
  if (v != v) return 0x7f;
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const float a = __builtin_fabsf(v);
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0x1p-6f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);  // multiples of 2^-9; 8 is 2^-6
  const uint32_t ab = bits & 0x7fffffffu;
  int e = (int)(ab >> 23) - 127;        // a = 1.m * 2^e, e >= -6
  const uint32_t m23 = ab & 0x7fffffu;
  uint32_t m = m23 >> 20;               // round the 23-bit mantissa to 3 bits, ties to even
  const uint32_t rest = m23 & 0xfffffu;
  if (rest > 0x80000u || (rest == 0x80000u && (m & 1u))) ++m;
  if (m == 8u) {
    m = 0u;
    ++e;
  }
  const uint32_t code = (uint32_t)((e + 7) << 3) | m;
  return sign | (code > 0x7eu ? 0x7eu : code);
}

__device__ __forceinline__ float bf_to_f(uint32_t h) { return __uint_as_float(h << 16); }

__device__ float block_max(float v, float* s_red) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) s_red[w] = v;
  __syncthreads();
  float m = s_red[0];
  for (int i = 1; i < 4; ++i) m = fmaxf(m, s_red[i]);
  __syncthreads();
  return m;
}

// amax over one expert's matrix (8 elements per load)
__device__ float chunk_amax(const u32x4* w, int64_t chunks) {
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < chunks; i += 256) {
    const u32x4 v = w[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(__builtin_fabsf(bf_to_f(v[j] & 0xffffu)), __builtin_fabsf(bf_to_f(v[j] >> 16))));
  }
  return m;
}

__device__ void chunk_quantize(const u32x4* w, u32x2* q, int64_t chunks, int k) {
  for (int64_t i = threadIdx.x; i < chunks; i += 256) {
    const u32x4 v = w[i];
    u32x2 out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t h = (b & 1) ? (v[2 * j + (b >> 1)] >> 16) : (v[2 * j + (b >> 1)] & 0xffffu);
        word |= e4m3_encode(__builtin_ldexpf(bf_to_f(h), -k)) << (8 * b);
      }
      out[j] = word;
    }
    q[i] = out;
  }
}

__global__ __launch_bounds__(256) void quantize_fp8_kernel(int64_t n0, int64_t n1, const uint16_t* __restrict__ w0,
                                                           const uint16_t* __restrict__ w1, uint8_t* __restrict__ q0,
                                                           uint8_t* __restrict__ q1, float* __restrict__ scale) {
  __shared__ float s_red[4];
  const int e = blockIdx.x;
  const u32x4* a0 = (const u32x4*)(w0 + (size_t)e * n0);
  const u32x4* a1 = w1 ? (const u32x4*)(w1 + (size_t)e * n1) : nullptr;
  float m = chunk_amax(a0, n0 / 8);
  if (a1) m = fmaxf(m, chunk_amax(a1, n1 / 8));
  const float amax = block_max(m, s_red);
  const int k = fp8_scale_exp(amax);
  if (threadIdx.x == 0) scale[e] = __builtin_ldexpf(1.0f, k);
  chunk_quantize(a0, (u32x2*)(q0 + (size_t)e * n0), n0 / 8, k);
  if (a1) chunk_quantize(a1, (u32x2*)(q1 + (size_t)e * n1), n1 / 8, k);
}

// Activation rows (token rows, SwiGLU outputs): one wave per row, each row
// its own "expert" of the rule above.  A row is read twice, for its max and
// then to encode it (the second read hits the cache); no barriers, so rows of
// a few thousand elements do not leave the CU waiting on workgroup
// synchronization.
constexpr int kRowsPerBlock = 4;

__global__ __launch_bounds__(64 * kRowsPerBlock) void quantize_rows_fp8_kernel(int64_t rows, int64_t cols,
                                                                            const uint16_t* __restrict__ x,
                                                                            uint8_t* __restrict__ q,
                                                                            float* __restrict__ scale) {
  const int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (r >= rows) return;  // wave-uniform
  const int l = threadIdx.x & 63;
  const int64_t chunks = cols / 8;
  const u32x4* src = (const u32x4*)(x + r * cols);
  float m = 0.0f;
  for (int64_t i = l; i < chunks; i += kWave) {
    const u32x4 v = src[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) m = fmaxf(m, fmaxf(__builtin_fabsf(bf_to_f(v[j] & 0xffffu)), __builtin_fabsf(bf_to_f(v[j] >> 16))));
  }
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
  const int k = fp8_scale_exp(m);
  if (l == 0) scale[r] = __builtin_ldexpf(1.0f, k);
  u32x2* dst = (u32x2*)(q + r * cols);
  for (int64_t i = l; i < chunks; i += kWave) {
    const u32x4 v = src[i];
    u32x2 out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t word = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint32_t h = (b & 1) ? (v[2 * j + (b >> 1)] >> 16) : (v[2 * j + (b >> 1)] & 0xffffu);
        word |= e4m3_encode(__builtin_ldexpf(bf_to_f(h), -k)) << (8 * b);
      }
      out[j] = word;
    }
    dst[i] = out;
  }
}

}  // namespace

hipError_t launch_quantize_rows_fp8(int64_t rows, int64_t cols, const uint16_t* x, uint8_t* q, float* scale,
                                    hipStream_t stream) {
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (blocks <= 0) return hipSuccess;
  MOE_LAUNCH(quantize_rows_fp8_kernel, dim3((unsigned)blocks), dim3(64 * kRowsPerBlock), 0, stream, rows, cols, x, q,
             scale);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(int E, int64_t n0, int64_t n1, const uint16_t* w0, const uint16_t* w1, uint8_t* q0,
                               uint8_t* q1, float* scale, hipStream_t stream) {
  MOE_LAUNCH(quantize_fp8_kernel, dim3((unsigned)E), dim3(256), 0, stream, n0, n1, w0, w1, q0, q1, scale);
  return hipGetLastError();
}

}  // namespace moe
