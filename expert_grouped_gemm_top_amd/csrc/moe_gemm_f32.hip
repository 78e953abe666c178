// moe_gemm_f32.hip -- the same ragged grouped GEMMs for fp32 activations and
// weights (expert forward, backward dx and dW: npu-train issue #14, sections
// Proposal and Scope).
//
// fp32 layers in this path are small (a 128-wide hidden size and 64-wide
// experts); on MI355X the fp32 matrix and vector peaks are the same
// (157.3 TFLOP/s), so these kernels use plain fp32 FMAs: one thread per output
// element, a 64-wide LDS-staged strip of the reduced dimension at a time.
// Ragged row counts come from the device offsets exactly as in the bf16 path.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

namespace {

__device__ __forceinline__ int expert_of_row(const int32_t* s_off, int E, int row) {
  int lo = 0, hi = E;  // s_off[lo] <= row < s_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_off[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

// grid: x = rows (up to max_rows), y = column blocks of 256 threads
template <int MODE>
__global__ __launch_bounds__(256) void row_gemm_f32_kernel(RowGemmArgs g) {
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ float s_a[64];
  const int tid = threadIdx.x;
  for (int i = tid; i <= g.E; i += 256) s_off[i] = g.offsets[i];  // E + 1 entries: 257 at E = 256
  __syncthreads();
  const int row = blockIdx.x;
  if (row >= s_off[g.E]) return;
  const int e = expert_of_row(s_off, g.E, row);
  const int H = g.H, F = g.F;
  const int ncols = (MODE == kGemmGateUp || MODE == kGemmDA) ? F : H;
  const int K = (MODE == kGemmGateUp || MODE == kGemmDA) ? H : (MODE == kGemmDown ? F : 2 * F);
  const int col = blockIdx.y * 256 + tid;
  const bool ok = col < ncols;
  const float* A = (const float*)g.a + a_row_of(g, row) * K;
  const float* w0 = (const float*)g.w0;
  const float* w1 = (const float*)g.w1;
  float s0 = 0.0f, s1 = 0.0f;
  for (int k0 = 0; k0 < K; k0 += 64) {
    __syncthreads();
    if (tid < 64 && k0 + tid < K) s_a[tid] = A[k0 + tid];
    __syncthreads();
    const int kn = (K - k0) < 64 ? (K - k0) : 64;
    if (!ok) continue;
    for (int kk = 0; kk < kn; ++kk) {
      const int k = k0 + kk;
      const float a = s_a[kk];
      if (MODE == kGemmGateUp) {
        s0 += a * w0[((size_t)e * H + k) * F + col];
        s1 += a * w1[((size_t)e * H + k) * F + col];
      } else if (MODE == kGemmDown) {
        s0 += a * w0[((size_t)e * F + k) * H + col];
      } else if (MODE == kGemmDA) {
        s0 += a * w0[((size_t)e * F + col) * H + k];
      } else {
        s0 += (k < F) ? a * w0[((size_t)e * H + col) * F + k] : a * w1[((size_t)e * H + col) * F + (k - F)];
      }
    }
  }
  if (!ok) return;
  if (MODE == kGemmGateUp) {
    if (g.out0 != nullptr) {
      float* h = (float*)g.out0 + (size_t)row * 2 * F;
      h[col] = s0;
      h[F + col] = s1;
    }
    if (g.out1 != nullptr) ((float*)g.out1)[(size_t)row * F + col] = s0 / (1.0f + expf(-s0)) * s1;
  } else if (MODE == kGemmDA) {
    const float* h = (const float*)g.h + h_row_of(g, row) * 2 * F;
    const float hg = h[col], hu = h[F + col];
    const float sg = 1.0f / (1.0f + expf(-hg));
    float* d = (float*)g.out0 + (size_t)row * 2 * F;
    d[col] = s0 * hu * sg * (1.0f + hg * (1.0f - sg));
    d[F + col] = s0 * hg * sg;
  } else {
    ((float*)g.out0)[(size_t)row * H + col] = s0;
  }
}

// grid: x = output elements / 256 per expert, y = expert.  Job 1: [dW_gate|dW_up]
// (H x 2F) = x^T [dHg|dHu]; job 2: dW_down (F x H) = a^T dO.
__global__ __launch_bounds__(256) void dw_f32_kernel(DwArgs g) {
  const int e = blockIdx.y;
  const int H = g.H, F = g.F;
  const int64_t job1 = (int64_t)H * 2 * F;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= job1 + (int64_t)F * H) return;
  const int row0 = g.offsets[e], n_e = g.offsets[e + 1] - row0;
  const float *P, *Q;
  int ldp, ldq, m, n;
  const int32_t* pmap;  // gathered rows of the left operand, or NULL
  int pdiv;
  float* out;
  if (i < job1) {
    m = (int)(i / (2 * F));
    n = (int)(i - (int64_t)m * 2 * F);
    P = (const float*)g.x; ldp = H;
    pmap = g.x_map;
    pdiv = g.x_div;
    Q = (const float*)g.dh; ldq = 2 * F;
    out = (n < F) ? (float*)g.dwg + ((size_t)e * H + m) * F + n : (float*)g.dwu + ((size_t)e * H + m) * F + (n - F);
  } else {
    const int64_t j = i - job1;
    m = (int)(j / H);
    n = (int)(j - (int64_t)m * H);
    P = (const float*)g.a; ldp = F;
    pmap = g.a_map;
    pdiv = 1;
    Q = (const float*)g.dO; ldq = H;
    out = (float*)g.dwd + ((size_t)e * F + m) * H + n;
  }
  float s = 0.0f;
  for (int r = 0; r < n_e; ++r) {
    const int64_t pr = pmap != nullptr ? (int64_t)(pmap[row0 + r] / pdiv) : (int64_t)(row0 + r);
    s += P[(size_t)pr * ldp + m] * Q[(size_t)(row0 + r) * ldq + n];
  }
  *out = s;
}

}  // namespace

hipError_t launch_row_gemm_f32(int mode, const RowGemmArgs& g, int max_rows, hipStream_t stream) {
  if (max_rows <= 0) return hipSuccess;
  const int ncols = (mode == kGemmGateUp || mode == kGemmDA) ? g.F : g.H;
  const dim3 grid((unsigned)max_rows, (unsigned)((ncols + 255) / 256));
  switch (mode) {
    case kGemmGateUp: MOE_LAUNCH(row_gemm_f32_kernel<kGemmGateUp>, grid, dim3(256), 0, stream, g); break;
    case kGemmDown: MOE_LAUNCH(row_gemm_f32_kernel<kGemmDown>, grid, dim3(256), 0, stream, g); break;
    case kGemmDA: MOE_LAUNCH(row_gemm_f32_kernel<kGemmDA>, grid, dim3(256), 0, stream, g); break;
    default: MOE_LAUNCH(row_gemm_f32_kernel<kGemmDX>, grid, dim3(256), 0, stream, g); break;
  }
  return hipGetLastError();
}

hipError_t launch_dw_f32(DwArgs g, hipStream_t stream) {
  const int64_t outputs = (int64_t)3 * g.H * g.F;
  const dim3 grid((unsigned)((outputs + 255) / 256), (unsigned)g.E);
  MOE_LAUNCH(dw_f32_kernel, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace moe
