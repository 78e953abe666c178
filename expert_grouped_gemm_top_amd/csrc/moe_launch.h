// moe_launch.h -- internal launchers behind the C ABI (include/moe.h).  Each
// returns the HIP status of its launches; the ABI layer validates arguments
// before any of them is called.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

namespace moe {

// Per-device set-up run once per GPU, safe when several host threads make
// their first call at the same time.  A failed attempt is not recorded, so the
// next call tries again.  Devices past kDevices run the set-up on every call.
class PerDeviceOnce {
 public:
  static constexpr int kDevices = 64;
  template <typename Fn>
  hipError_t run(Fn&& fn) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kDevices) return fn(dev);
    if (done_[dev].load(std::memory_order_acquire)) return hipSuccess;
    std::lock_guard<std::mutex> lock(mu_);
    if (done_[dev].load(std::memory_order_relaxed)) return hipSuccess;
    err = fn(dev);
    if (err == hipSuccess) done_[dev].store(true, std::memory_order_release);
    return err;
  }

 private:
  std::atomic<bool> done_[kDevices] = {};
  std::mutex mu_;
};

// Allows `kern` dynamic LDS of `bytes` (needed above 64 KiB) on the current
// device, once per device per `once`.
inline hipError_t allow_dynamic_lds(PerDeviceOnce& once, const void* kern, size_t bytes) {
  return once.run([&](int) { return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes); });
}

// Every kernel launch of the library goes through MOE_LAUNCH, which counts it
// on the calling thread (moe_launch_count) and then launches it.  While the
// profiling hook has armed a pair of events for a phase (moe_profile_kernel),
// the launches of that phase carry them in their own dispatch: the first one
// records `start` as it begins, every one records `stop` as it ends (the last
// one's end stands), so timing a kernel adds no packet to the stream between
// kernels (separate event records around the phase had cost the LoRA step
// ~8 us, 1.7 %).
void note_launch();
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();  // this thread's armed events

template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, size_t shmem, hipStream_t stream, Args... args) {
  note_launch();
  LaunchEvents& ev = launch_events();
  if (ev.stop == nullptr) {
    hipLaunchKernelGGL(kernel, grid, block, shmem, stream, args...);
  } else {
    hipExtLaunchKernelGGL(kernel, grid, block, (std::uint32_t)shmem, stream, ev.start, ev.stop, 0u, args...);
    ev.start = nullptr;  // the phase's first launch took it
  }
}
#define MOE_LAUNCH(...) ::moe::launch_kernel(__VA_ARGS__)

constexpr int kMaxExpertsHost = 256;  // expert ids fit in 8 bits
enum RowGemmMode { kGemmGateUp = 0, kGemmDown = 1, kGemmDA = 2, kGemmDX = 3 };

// Row GEMM regimes by an expert's row count n_e: n_e < kMidTileMinRows -> streaming
// kernel (16-row wave tiles); up to big_gemm_min_rows(...) -> 128 x 128 LDS
// tiles; above -> 256 x 256 LDS tiles fed by direct global->LDS loads.
constexpr int kMidTileMinRows = 32;
constexpr int kBigTileMinRows = 256;
constexpr int kNoBigTiles = 0x40000000;  // above every row count

// Pointers of one row-ragged grouped GEMM.  Element type is bf16 (uint16_t
// bits) or fp32 depending on the launcher; all buffers are device memory.
//   GATEUP: a = x rows [R,H], w0 = W_gate, w1 = W_up, out0 = h [R,2F], out1 = a [R,F]
//   DOWN:   a = a rows [R,F], w0 = W_down, out0 = o [R,H]
//   DA:     a = dO rows [R,H], w0 = W_down, h = h rows [R,2F], out0 = dh [R,2F]
//   DX:     a = dh rows [R,2F], w0 = W_gate, w1 = W_up, out0 = dX [R,H]
struct RowGemmArgs {
  const int32_t* offsets;
  int E, H, F;
  const uint16_t* a;
  const uint16_t* w0;
  const uint16_t* w1;
  const uint16_t* h;
  uint16_t* out0;
  uint16_t* out1;
  const int32_t* a_map;  // when set, row s of `a` is a[a_map[s] / a_div] (rows gathered on load)
  int a_div;
  const int32_t* h_map;  // DA: when set, the saved pre-activations of row s are h[h_map[s]]
  int big_min_rows;   // set by launch_row_gemm_bf16: experts from this row count take the 256-row kernel
  int stream_ksplit;  // set by launch_row_gemm_bf16: reduction split of the skinny-expert kernel (1, 2 or 4)
  // fp8 weights (launch_row_gemm_fp8w): w0 / w1 point at E4M3 bytes, and every
  // product of expert e is multiplied by wscale[e] (the scale of the weights
  // it reads)
  const float* wscale;
};

struct DwArgs {
  const int32_t* offsets;
  int E, H, F;
  const uint16_t* x;   // [R,H], or gathered: row s is x[x_map[s] / x_div]
  const uint16_t* a;   // [R,F], or gathered: row s is a[a_map[s]]
  const int32_t* x_map;
  int x_div;
  const int32_t* a_map;
  const uint16_t* dO;  // [R,H]
  const uint16_t* dh;  // [R,2F]
  uint16_t* dwg;       // [E,H,F]
  uint16_t* dwu;       // [E,H,F]
  uint16_t* dwd;       // [E,F,H]
};

// Pointers of one grouped GEMM of the forward on fp8 (E4M3) codes; every
// operand row is K-contiguous codes, every product scaled by the activation
// row's scale times the expert's.
//   GATEUP: a = x codes [*, H] (row s is a[a_map[s] / a_div] when a_map is
//           set), w0 / w1 = W_gate^T / W_up^T codes [E][F][H], out0 = h [R,2F]
//           (or NULL), out1 = a [R,F] (bf16)
//   DOWN:   a = SwiGLU-output codes [R,F], w0 = W_down^T codes [E][H][F], out0 = o [R,H] (bf16)
struct Fp8GemmArgs {
  const int32_t* offsets;
  int E, H, F;
  const uint8_t* a;
  const int32_t* a_map;
  int a_div;
  const float* ascale;  // per source row of a
  const uint8_t* w0;
  const uint8_t* w1;
  const float* wscale;  // per expert
  uint16_t* out0;
  uint16_t* out1;
};

// Source row of operand row s of a row GEMM.
__device__ __forceinline__ int64_t a_row_of(const RowGemmArgs& g, int s) {
  return g.a_map != nullptr ? (int64_t)(g.a_map[s] / g.a_div) : (int64_t)s;
}

// Row of the saved pre-activations that row s of a dA product reads.
__device__ __forceinline__ int64_t h_row_of(const RowGemmArgs& g, int64_t s) {
  return g.h_map != nullptr ? (int64_t)g.h_map[s] : s;
}

hipError_t launch_route_topk(int T, int E, int k, const float* logits, int32_t* idx, float* w, hipStream_t stream);

size_t dispatch_workspace_bytes(int64_t N, int E);
// Size of the library-owned dispatch workspace of moe_dispatch_noalloc (per GPU).
constexpr size_t kDispatchScratchBytes = (size_t)4 << 20;
// Device address of that workspace on the current device (looked up once per
// device).
hipError_t dispatch_scratch(void** out);
hipError_t launch_dispatch_index(int T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                                 int32_t* perm, int32_t* inv_perm, void* ws, hipStream_t stream);
hipError_t launch_dispatch_rows(int T, int H, int k, int esize, const void* x, const int32_t* inv_perm, void* x_sorted,
                                hipStream_t stream);

hipError_t launch_combine(int T, int H, int k, int esize, const void* rows, const int32_t* inv, const float* w,
                          void* out, hipStream_t stream);
hipError_t launch_grad_rows(int T, int H, int k, int esize, const void* dy, const float* w, const int32_t* inv,
                            void* dO_rows, const int32_t* inv_all, const void* o_sorted, float* dg,
                            hipStream_t stream);
hipError_t launch_pair_scores(int T, int H, int F, int k, int esize, const int32_t* inv, const float* w,
                              const void* a_rows, const void* dy, float* score, hipStream_t stream);
hipError_t launch_gather_rows(const int32_t* R_ptr, const int32_t* src, int max_rows, const void* a_src, void* a_dst,
                              int a_bytes, const void* b_src, void* b_dst, int b_bytes, const void* c_src,
                              void* c_dst, int c_bytes, hipStream_t stream);

// max_expert_rows bounds one expert's row count (a hint for kernel choice only:
// experts above it are still computed, on the 128-row tiles)
hipError_t launch_row_gemm_bf16(int mode, const RowGemmArgs& g, int max_rows, int max_expert_rows,
                                hipStream_t stream);
hipError_t launch_dw_bf16(const DwArgs& g, hipStream_t stream);
// Row GEMMs with fp8 (E4M3) weights and bf16 activations: every expert, whatever
// its row count, on the streaming kernel.
hipError_t launch_row_gemm_fp8w(int mode, const RowGemmArgs& g, int max_rows, hipStream_t stream);
// E4M3 codes of `rows` rows of `cols` bf16 values, one power-of-two scale per
// row (moe_fp8.hip).
hipError_t launch_quantize_rows_fp8(int64_t rows, int64_t cols, const uint16_t* x, uint8_t* q, float* scale,
                                    hipStream_t stream);
// Per-expert fp8 storage of w0 [E][n0] and w1 [E][n1] (w1 may be NULL) with one
// power-of-two scale per expert.
hipError_t launch_quantize_fp8(int E, int64_t n0, int64_t n1, const uint16_t* w0, const uint16_t* w1, uint8_t* q0,
                               uint8_t* q1, float* scale, hipStream_t stream);
hipError_t launch_big_gemm_bf16(int mode, const RowGemmArgs& g, int max_rows, hipStream_t stream);
// fp8 forward products (kGemmGateUp, kGemmDown), every expert on 256 x 256 tiles.
hipError_t launch_gemm_fp8(int mode, const Fp8GemmArgs& g, int max_rows, hipStream_t stream);
// out[e][c][r] = in[e][r][c] (bytes; rows and cols multiples of 16).
hipError_t launch_transpose_u8(int E, int rows, int cols, const uint8_t* in, uint8_t* out, hipStream_t stream);
// Row count from which an expert takes the 256-row kernel for this product and
// shape; kNoBigTiles where that kernel does not apply.
int big_gemm_min_rows(int mode, int H, int F);
hipError_t launch_row_gemm_f32(int mode, const RowGemmArgs& g, int max_rows, hipStream_t stream);
hipError_t launch_dw_f32(DwArgs g, hipStream_t stream);

size_t router_workspace_bytes(int T, int H, int E);
hipError_t launch_router_fwd(int T, int H, int E, int esize, const void* x, const void* w_r, float* logits, void* ws,
                             hipStream_t stream);
hipError_t launch_router_bwd(int T, int H, int E, int k, int esize, const void* x, const void* w_r,
                             const int32_t* idx, const float* w, const float* dg, float* dlogits, void* dw_r,
                             void* dx, bool dx_accumulate, void* ws, hipStream_t stream);

hipError_t launch_fill_i32(int32_t* a, int64_t n, int32_t v, hipStream_t stream);
hipError_t launch_compact(int64_t N, int E, int cap, const int32_t* counts, const int32_t* offsets, const int32_t* perm,
                          const float* score, int32_t* kept_counts, int32_t* kept_offsets, int32_t* kept_perm,
                          int32_t* kept_src, int32_t* kept_inv, hipStream_t stream);

}  // namespace moe
