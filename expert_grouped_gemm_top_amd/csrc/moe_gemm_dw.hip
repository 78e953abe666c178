// moe_gemm_dw.hip -- expert weight gradients in bf16 on the 32x32x16 matrix
// core (full fine-tuning: npu-train issue #14, section Scope), reduced over
// each expert's own ragged row count (LRMoE abstract):
//   [dW_gate | dW_up][e] (H x 2F) = x_rows^T [dHg | dHu]   over the rows of e
//   dW_down[e]           (F x H)  = a_rows^T dO_rows
//
// Workgroup = one 256 x 256 output tile of one expert, eight waves of 128 x 64.
// Both operands are row-major over the reduced index (the expert's rows), so
// both land in LDS as [64 rows][256 columns] stages through direct
// global->LDS loads (two stages in flight) and both MFMA fragments come from
// the transposing LDS read.  Rows past the expert's last one are loaded from
// its last row and zeroed in LDS before use.  Every output is reduced in row
// order by one workgroup (deterministic, no atomics); an expert without rows
// stores exact zeros.  Workgroups take experts in order of decreasing row
// count, so the longest reductions start first.
#include <algorithm>

#include "moe_common.h"
#include "moe_launch.h"
#include "moe_lds32.h"

namespace moe {

namespace {

constexpr int kDwBM = 256, kDwBN = 256, kDwBK = 64;  // tile rows (of dW), columns, rows reduced per stage
constexpr int kDwWaves = 8, kDwWM = 2;               // waves, waves along the tile rows
constexpr int kDwTM = kDwBM / kDwWM;                 // 128 tile rows per wave
constexpr int kDwTN = kDwBN / (kDwWaves / kDwWM);    // 64 tile columns per wave
constexpr int kDwMI = kDwTM / 32, kDwNJ = kDwTN / 32;
constexpr int kDwPitch = kDwBM * 2;                    // bytes per reduced row of a stage tile
constexpr int kDwTileBytes = kDwBK * kDwPitch;         // 32 KiB per operand and stage
constexpr int kDwStageBytes = 2 * kDwTileBytes;
constexpr int kDwStages = 2;
constexpr int kDwIns = kDwTileBytes / 1024 / kDwWaves;  // direct loads per wave, operand and stage
static_assert(kDwBM == kDwBN, "one stage layout for both operands");
static_assert(kDwIns * 1024 * kDwWaves == kDwTileBytes, "loads cover the tile");

struct DwShape {
  int nt1, tiles1;  // gate/up: column tiles, all tiles
  int nt2;          // down: column tiles
  int tiles;        // tiles per expert
};

__host__ __device__ inline DwShape dw_shape(int H, int F) {
  DwShape s;
  const int mt1 = (H + kDwBM - 1) / kDwBM;
  s.nt1 = (2 * F + kDwBN - 1) / kDwBN;
  s.tiles1 = mt1 * s.nt1;
  const int mt2 = (F + kDwBM - 1) / kDwBM;
  s.nt2 = (H + kDwBN - 1) / kDwBN;
  s.tiles = s.tiles1 + mt2 * s.nt2;
  return s;
}

__global__ __launch_bounds__(64 * kDwWaves, 1) void dw_bf16_kernel(DwArgs g) {
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_expert;
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l32 = l & 31, hk = l >> 5;
  const int wm = w % kDwWM, wn = w / kDwWM;
  const int H = g.H, F = g.F, E = g.E;
  const DwShape sh = dw_shape(H, F);

  // ---- which expert: rank of this workgroup's expert in decreasing row count
  const int rank = blockIdx.x / sh.tiles, t = blockIdx.x - rank * sh.tiles;
  static_assert(64 * kDwWaves > kMaxExperts, "every offsets entry has a thread");
  if (tid <= E) s_off[tid] = g.offsets[tid];
  __syncthreads();
  if (tid < E) {
    const int n = s_off[tid + 1] - s_off[tid];
    int r = 0;
    for (int e2 = 0; e2 < E; ++e2) {
      const int n2 = s_off[e2 + 1] - s_off[e2];
      r += (n2 > n || (n2 == n && e2 < tid)) ? 1 : 0;
    }
    if (r == rank) s_expert = tid;
  }
  __syncthreads();
  const int e = s_expert;
  const int row0 = s_off[e], n_e = s_off[e + 1] - row0;

  // ---- the product this tile belongs to
  const uint16_t *P, *Q;
  int ldp, ldq, M, N, mt, nt;
  if (t < sh.tiles1) {  // [dW_gate | dW_up] = x^T [dHg | dHu]
    mt = t / sh.nt1;
    nt = t - mt * sh.nt1;
    P = g.x; ldp = H; M = H;
    Q = g.dh; ldq = 2 * F; N = 2 * F;
  } else {              // dW_down = a^T dO
    const int tt = t - sh.tiles1;
    mt = tt / sh.nt2;
    nt = tt - mt * sh.nt2;
    P = g.a; ldp = F; M = F;
    Q = g.dO; ldq = H; N = H;
  }
  const int m0 = mt * kDwBM, n0 = nt * kDwBN;

  // ---- loader: instruction i of wave w fills reduced rows 2 (kDwIns w + i) + hk
  // of a stage; LDS position l32 of a row holds the 8-column chunk
  // l32 ^ nn_swz(row).  Chunks past the matrix edge read column 0 (their
  // results are never stored).
  const uint16_t* p_col[kDwIns];
  const uint16_t* q_col[kDwIns];
  int krow[kDwIns];
#pragma unroll
  for (int i = 0; i < kDwIns; ++i) {
    const int k = 2 * (kDwIns * w + i) + hk;
    const int ch = l32 ^ nn_swz(k);
    const int pc = m0 + 8 * ch, qc = n0 + 8 * ch;
    krow[i] = k;
    p_col[i] = P + (size_t)row0 * ldp + (pc < M ? pc : 0);
    q_col[i] = Q + (size_t)row0 * ldq + (qc < N ? qc : 0);
  }
  auto issue = [&](int s) {
    unsigned char* st = s_dyn + (s % kDwStages) * kDwStageBytes;
#pragma unroll
    for (int i = 0; i < kDwIns; ++i) {
      int r = s * kDwBK + krow[i];
      r = r < n_e ? r : n_e - 1;  // past the expert's rows: its last row, zeroed before use
      g2lds(p_col[i] + (size_t)r * ldp, st + 1024 * (kDwIns * w + i));
      g2lds(q_col[i] + (size_t)r * ldq, st + kDwTileBytes + 1024 * (kDwIns * w + i));
    }
  };

  f32x16 acc[kDwMI][kDwNJ];
#pragma unroll
  for (int i = 0; i < kDwMI; ++i)
#pragma unroll
    for (int j = 0; j < kDwNJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto compute = [&](int s) {
    const unsigned char* st = s_dyn + (s % kDwStages) * kDwStageBytes;
#pragma unroll
    for (int sub = 0; sub < kDwBK / 16; ++sub) {
      u32x4 fa[kDwMI], fb[kDwNJ];
#pragma unroll
      for (int i = 0; i < kDwMI; ++i) fa[i] = tr_frag32(st, kDwPitch, sub, kDwTM * wm + 32 * i);
#pragma unroll
      for (int j = 0; j < kDwNJ; ++j) fb[j] = tr_frag32(st + kDwTileBytes, kDwPitch, sub, kDwTN * wn + 32 * j);
#pragma unroll
      for (int j = 0; j < kDwNJ; ++j)
#pragma unroll
        for (int i = 0; i < kDwMI; ++i) acc[i][j] = mfma32(fb[j], fa[i], acc[i][j]);
    }
  };

  const int steps = (n_e + kDwBK - 1) / kDwBK;
  if (steps > 0) issue(0);
  for (int s = 0; s < steps; ++s) {
    wait_vmcnt<0>();  // this wave's loads of stage s (the only stage in flight)
    barrier_no_fence();
    if (s + 1 < steps) issue(s + 1);
    const int valid = n_e - s * kDwBK;
    if (valid < kDwBK) {
      // last stage: zero the rows past the expert's end in both operand tiles
      unsigned char* st = s_dyn + (s % kDwStages) * kDwStageBytes;
      for (int c = tid; c < 2 * kDwBK * (kDwPitch / 16); c += 64 * kDwWaves) {
        const int op = c / (kDwBK * (kDwPitch / 16));
        const int rr = (c / (kDwPitch / 16)) % kDwBK;
        if (rr >= valid) *(u32x4*)(st + op * kDwTileBytes + rr * kDwPitch + 16 * (c % (kDwPitch / 16))) = u32x4{0, 0, 0, 0};
      }
      __syncthreads();
    }
    compute(s);
  }

  // ---- epilogue.  acc[i][j] register r -> tile row kDwTM wm + 32 i + l32,
  // tile column kDwTN wn + 32 j + 8 q + 4 hk + (0..3) with q = r / 4.
#pragma unroll
  for (int i = 0; i < kDwMI; ++i) {
    const int m = m0 + kDwTM * wm + 32 * i + l32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < kDwNJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + kDwTN * wn + 32 * j + 8 * q + 4 * hk;
        if (n >= N) continue;
        uint16_t* dst;
        if (t < sh.tiles1) dst = (n < F) ? g.dwg + ((size_t)e * H + m) * F + n : g.dwu + ((size_t)e * H + m) * F + (n - F);
        else dst = g.dwd + ((size_t)e * F + m) * H + n;
        *(u32x2*)dst = u32x2{pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                             pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
      }
  }
}

}  // namespace

hipError_t launch_dw_bf16(const DwArgs& g, hipStream_t stream) {
  const DwShape sh = dw_shape(g.H, g.F);
  const int64_t blocks = (int64_t)g.E * sh.tiles;
  const size_t lds = (size_t)kDwStages * kDwStageBytes;
  // dynamic LDS above 64 KiB must be allowed explicitly, once per device
  static bool attr_set[64] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= 64 || !attr_set[dev]) {
    err = hipFuncSetAttribute((const void*)dw_bf16_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < 64) attr_set[dev] = true;
  }
  hipLaunchKernelGGL(dw_bf16_kernel, dim3((unsigned)blocks), dim3(64 * kDwWaves), lds, stream, g);
  return hipGetLastError();
}

}  // namespace moe
