// moe_gemm_bf16.hip -- ragged grouped GEMMs of the SwiGLU experts in bf16 on
// gfx950 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
//
// Expert forward, backward dx and dW (npu-train issue #14, sections Proposal
// and Scope), run as variable-size grouped GEMMs over each expert's own row
// count (LRMoE abstract), with no padding of experts to a fixed bucket.
//
// Row GEMMs (M = the expert's rows, ragged; K, N = feature sizes):
//   GATEUP  [n_e,H] x [W_gate|W_up][e] (W [H,F], N-contiguous)  -> h=[hg|hu], a=silu(hg)*hu
//   DOWN    [n_e,F] x W_down[e]        (W [F,H], N-contiguous)  -> o
//   DA      [n_e,H] x W_down[e]^T      (W [F,H], K-contiguous)  -> dh=[dHg|dHu] (SwiGLU backward)
//   DX      [n_e,2F] x [W_gate|W_up][e]^T (K-contiguous)        -> dX
// Each workgroup owns one 32-row tile of one expert (found on the device from
// the offsets, see find_row_tile) and one block of output columns; its four
// waves split K four ways, stream operands straight from global memory into
// MFMA registers (no LDS round trip: at the routed row counts of these layers
// the weights are read once and are the traffic that bounds the kernel), and
// reduce their fp32 partial tiles through LDS before the fused epilogue.
//
// Operand mapping inside a wave (lane l: c = l % 16, g = l / 16):
//   A (rows, K-contiguous): lane loads 8 consecutive k (k0 + 8g ..) of row c.
//   B columns are split into 8 interleaved sub-tiles: MFMA number jj covers
//   columns 8c + jj (c = 0..15).  N-contiguous weights: the lane loads rows
//   k0 + 8g + (0..7) x columns 8c .. 8c+7 (16 B each) and transposes the 8x8
//   bf16 block in registers; K-contiguous weights: one 16 B load per column.
//   The MFMA runs with B as its first operand, so lane (c, g) ends up holding
//   row c and columns 32g + (0..31) of the tile: contiguous output segments.
//
// dW GEMM (K = the expert's rows, ragged):
//   dW_gate|dW_up [H, 2F] = x_rows^T [dHg|dHu],  dW_down [F, H] = a_rows^T dO_rows
// Workgroup = one 128x128 output tile of one expert; both operands are
// row-major over the reduced index, so each lane loads 8 rows x 4 columns and
// transposes them in registers.  The reduction runs in a fixed order over all
// of the expert's rows (deterministic, no atomics); an empty expert stores
// exact zeros.
#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

namespace {

constexpr int kTileRows = 32;  // rows of one expert per workgroup tile
constexpr int kRedPitch = 132; // fp32 pitch of the LDS reduction tile (128 + 4)

// ---- register transposes of bf16 blocks -------------------------------------
// rows[r] holds 8 bf16 (columns 0..7) of row r; returns the 8 k-values (rows
// 0..7) of column jj packed as an MFMA operand.
__device__ __forceinline__ u32x4 column_of_8x8(const u32x4* rows, int jj) {
  const int d = jj >> 1;
  u32x4 f;
  if ((jj & 1) == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) f[q] = (rows[2 * q][d] & 0xffffu) | (rows[2 * q + 1][d] << 16);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) f[q] = (rows[2 * q][d] >> 16) | (rows[2 * q + 1][d] & 0xffff0000u);
  }
  return f;
}

// rows[r] holds 4 bf16 (columns 0..3) of row r; column jj (0..3) of the 8x4 block.
__device__ __forceinline__ u32x4 column_of_8x4(const u32x2* rows, int jj) {
  const int d = jj >> 1;
  u32x4 f;
  if ((jj & 1) == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) f[q] = (rows[2 * q][d] & 0xffffu) | (rows[2 * q + 1][d] << 16);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) f[q] = (rows[2 * q][d] >> 16) | (rows[2 * q + 1][d] & 0xffff0000u);
  }
  return f;
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 first, u32x4 second, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, first), __builtin_bit_cast(bf16x8, second),
                                                  acc, 0, 0, 0);
}

// ---- row GEMMs --------------------------------------------------------------
template <int MODE>
struct RowGemmShape;
// K (reduced length), columns per block, whether the weights are N-contiguous
template <>
struct RowGemmShape<kGemmGateUp> { static constexpr bool kNN = true; };
template <>
struct RowGemmShape<kGemmDown> { static constexpr bool kNN = true; };
template <>
struct RowGemmShape<kGemmDA> { static constexpr bool kNN = false; };
template <>
struct RowGemmShape<kGemmDX> { static constexpr bool kNN = false; };

template <int MODE>
__device__ __forceinline__ int row_gemm_K(const RowGemmArgs& g) {
  return (MODE == kGemmGateUp || MODE == kGemmDA) ? g.H : (MODE == kGemmDown ? g.F : 2 * g.F);
}

template <int MODE>
__global__ __launch_bounds__(256, 2) void row_gemm_bf16_kernel(RowGemmArgs g) {
  constexpr bool NN = RowGemmShape<MODE>::kNN;
  __shared__ int s_start[kMaxExperts + 1], s_off[kMaxExperts + 1], s_tmp[4];
  __shared__ float s_red[4][kTileRows][kRedPitch];

  const TileSlot ts = find_row_tile(g.offsets, g.E, kTileRows, blockIdx.x, s_start, s_off, s_tmp);
  if (ts.expert < 0) return;  // uniform across the workgroup
  const int e = ts.expert;
  const int nb = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, gq = l >> 4;
  const int H = g.H, F = g.F;
  const int K = row_gemm_K<MODE>(g);
  const int Kq = K / 4;
  const int k_begin = w * Kq;
  const int steps = Kq / 32;
  const int ms = (ts.rows + 15) >> 4;  // 16-row sub-tiles with real rows: 1 or 2

  const uint16_t* __restrict__ A = (const uint16_t*)g.a;
  const uint16_t* a_ptr[2];
  bool a_ok[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = 16 * i + c;
    a_ok[i] = m < ts.rows;
    a_ptr[i] = A + (size_t)(ts.row_begin + (a_ok[i] ? m : 0)) * K + k_begin + 8 * gq;
  }

  // B operand base pointer and strides
  const uint16_t* b_ptr;
  size_t b_step;  // elements per K-step of 32
  size_t b_sub;   // NN: elements between the 8 rows a lane loads; NT: between the 8 columns
  if (MODE == kGemmGateUp) {
    const uint16_t* W = (c < 8) ? g.w0 : g.w1;
    b_ptr = W + (size_t)e * H * F + (size_t)(k_begin + 8 * gq) * F + nb * 64 + 8 * (c & 7);
    b_step = (size_t)32 * F;
    b_sub = F;
  } else if (MODE == kGemmDown) {
    b_ptr = g.w0 + (size_t)e * F * H + (size_t)(k_begin + 8 * gq) * H + nb * 128 + 8 * c;
    b_step = (size_t)32 * H;
    b_sub = H;
  } else if (MODE == kGemmDA) {
    b_ptr = g.w0 + (size_t)e * F * H + (size_t)(nb * 128 + 8 * c) * H + k_begin + 8 * gq;
    b_step = 32;
    b_sub = H;
  } else {  // DX: waves 0,1 reduce over dHg (W_gate), waves 2,3 over dHu (W_up)
    const uint16_t* W = (w < 2) ? g.w0 : g.w1;
    const int kloc = k_begin - ((w < 2) ? 0 : F);
    b_ptr = W + (size_t)e * H * F + (size_t)(nb * 128 + 8 * c) * F + kloc + 8 * gq;
    b_step = 32;
    b_sub = F;
  }

  f32x4 acc[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load = [&](int s, u32x4* bq, u32x4* aq) {
    const uint16_t* bp = b_ptr + (size_t)s * b_step;
#pragma unroll
    for (int r = 0; r < 8; ++r) bq[r] = *(const u32x4*)(bp + (size_t)r * b_sub);
#pragma unroll
    for (int i = 0; i < 2; ++i) aq[i] = a_ok[i] ? *(const u32x4*)(a_ptr[i] + (size_t)s * 32) : u32x4{0u, 0u, 0u, 0u};
  };
  auto compute = [&](const u32x4* bq, const u32x4* aq) {
    u32x4 bf[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) bf[jj] = NN ? column_of_8x8(bq, jj) : bq[jj];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[0][jj] = mfma_bf16(bf[jj], aq[0], acc[0][jj]);
    if (ms > 1) {
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) acc[1][jj] = mfma_bf16(bf[jj], aq[1], acc[1][jj]);
    }
  };

  u32x4 bA[8], aA[2], bB[8], aB[2];
  load(0, bA, aA);
  int s = 0;
  for (; s + 2 <= steps; s += 2) {
    load(s + 1, bB, aB);
    compute(bA, aA);
    if (s + 2 < steps) load(s + 2, bA, aA);
    compute(bB, aB);
  }
  if (s < steps) compute(bA, aA);

  // partial tiles -> LDS: lane (c, gq) holds row 16i + c, columns 32gq + 8r + jj
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float* dst = &s_red[w][16 * i + c][32 * gq + 8 * r];
      *(f32x4*)dst = f32x4{acc[i][0][r], acc[i][1][r], acc[i][2][r], acc[i][3][r]};
      *(f32x4*)(dst + 4) = f32x4{acc[i][4][r], acc[i][5][r], acc[i][6][r], acc[i][7][r]};
    }
  __syncthreads();

  // epilogue: thread -> one row, 16 (or 8+8) columns of the block
  const int row = tid >> 3, q = tid & 7;
  if (row >= ts.rows) return;
  const size_t grow = (size_t)ts.row_begin + row;
  if (MODE == kGemmGateUp) {
    float hg[8], hu[8], av[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hg[i] = s_red[0][row][8 * q + i] + s_red[1][row][8 * q + i] + s_red[2][row][8 * q + i] + s_red[3][row][8 * q + i];
      hu[i] = s_red[0][row][64 + 8 * q + i] + s_red[1][row][64 + 8 * q + i] + s_red[2][row][64 + 8 * q + i] +
              s_red[3][row][64 + 8 * q + i];
      av[i] = hg[i] * sigmoidf_fast(hg[i]) * hu[i];
    }
    const int f = nb * 64 + 8 * q;
    uint16_t* hrow = g.out0 + grow * 2 * F;
    *(u32x4*)(hrow + f) = u32x4{pack_bf2(hg[0], hg[1]), pack_bf2(hg[2], hg[3]), pack_bf2(hg[4], hg[5]), pack_bf2(hg[6], hg[7])};
    *(u32x4*)(hrow + F + f) = u32x4{pack_bf2(hu[0], hu[1]), pack_bf2(hu[2], hu[3]), pack_bf2(hu[4], hu[5]), pack_bf2(hu[6], hu[7])};
    *(u32x4*)(g.out1 + grow * F + f) =
        u32x4{pack_bf2(av[0], av[1]), pack_bf2(av[2], av[3]), pack_bf2(av[4], av[5]), pack_bf2(av[6], av[7])};
  } else {
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v[i] = s_red[0][row][16 * q + i] + s_red[1][row][16 * q + i] + s_red[2][row][16 * q + i] + s_red[3][row][16 * q + i];
    const int col = nb * 128 + 16 * q;
    if (MODE == kGemmDA) {
      // SwiGLU backward with the saved pre-activations hg, hu
      const uint16_t* hrow = g.h + grow * 2 * F;
      const u32x4 g0 = *(const u32x4*)(hrow + col), g1 = *(const u32x4*)(hrow + col + 8);
      const u32x4 u0 = *(const u32x4*)(hrow + F + col), u1 = *(const u32x4*)(hrow + F + col + 8);
      float dg[16], du[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t gw = (i < 8) ? g0[(i & 7) >> 1] : g1[(i & 7) >> 1];
        const uint32_t uw = (i < 8) ? u0[(i & 7) >> 1] : u1[(i & 7) >> 1];
        const float hg = (i & 1) ? bf_hi(gw) : bf_lo(gw);
        const float hu = (i & 1) ? bf_hi(uw) : bf_lo(uw);
        const float sg = sigmoidf_fast(hg);
        dg[i] = v[i] * hu * sg * (1.0f + hg * (1.0f - sg));
        du[i] = v[i] * hg * sg;
      }
      uint16_t* drow = g.out0 + grow * 2 * F;
      *(u32x4*)(drow + col) = u32x4{pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]), pack_bf2(dg[4], dg[5]), pack_bf2(dg[6], dg[7])};
      *(u32x4*)(drow + col + 8) =
          u32x4{pack_bf2(dg[8], dg[9]), pack_bf2(dg[10], dg[11]), pack_bf2(dg[12], dg[13]), pack_bf2(dg[14], dg[15])};
      *(u32x4*)(drow + F + col) =
          u32x4{pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]), pack_bf2(du[4], du[5]), pack_bf2(du[6], du[7])};
      *(u32x4*)(drow + F + col + 8) =
          u32x4{pack_bf2(du[8], du[9]), pack_bf2(du[10], du[11]), pack_bf2(du[12], du[13]), pack_bf2(du[14], du[15])};
    } else {
      uint16_t* orow = g.out0 + grow * H + col;  // DOWN: o rows, DX: dX rows (both [rows, H])
      *(u32x4*)orow = u32x4{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7])};
      *(u32x4*)(orow + 8) =
          u32x4{pack_bf2(v[8], v[9]), pack_bf2(v[10], v[11]), pack_bf2(v[12], v[13]), pack_bf2(v[14], v[15])};
    }
  }
}

// ---- dW GEMM ------------------------------------------------------------------
__global__ __launch_bounds__(256, 2) void dw_bf16_kernel(DwArgs g) {
  const int e = blockIdx.x / g.tiles_per_expert;
  const int t = blockIdx.x - e * g.tiles_per_expert;
  const int H = g.H, F = g.F;
  const int row0 = g.offsets[e];
  const int n_e = g.offsets[e + 1] - row0;
  const uint16_t *P, *Q;
  int ldp, ldq, mt, nt;
  uint16_t* out;
  int ldo, out_col0;
  if (t < g.tiles_job1) {  // [dW_gate | dW_up] = x^T [dHg | dHu]
    const int ntn = (2 * F) / 128;
    mt = t / ntn;
    nt = t - mt * ntn;
    P = g.x; ldp = H;
    Q = g.dh; ldq = 2 * F;
    const bool up = nt * 128 >= F;
    out = (up ? g.dwu : g.dwg) + (size_t)e * H * F;
    ldo = F;
    out_col0 = up ? -F : 0;
  } else {                 // dW_down = a^T dO
    const int tt = t - g.tiles_job1;
    const int ntn = H / 128;
    mt = tt / ntn;
    nt = tt - mt * ntn;
    P = g.a; ldp = F;
    Q = g.dO; ldq = H;
    out = g.dwd + (size_t)e * F * H;
    ldo = H;
    out_col0 = 0;
  }
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, gq = l >> 4;
  const int mb = mt * 128 + (w & 1) * 64;
  const int nb = nt * 128 + (w >> 1) * 64;
  const uint16_t* p_ptr = P + (size_t)(row0 + 8 * gq) * ldp + mb + 4 * c;
  const uint16_t* q_ptr = Q + (size_t)(row0 + 8 * gq) * ldq + nb + 4 * c;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = (n_e + 31) / 32;
  auto load = [&](int s, u32x2* pq, u32x2* qq) {
    const int rbase = 32 * s + 8 * gq;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const bool ok = rbase + r < n_e;
      pq[r] = ok ? *(const u32x2*)(p_ptr + (size_t)(32 * s + r) * ldp) : u32x2{0u, 0u};
      qq[r] = ok ? *(const u32x2*)(q_ptr + (size_t)(32 * s + r) * ldq) : u32x2{0u, 0u};
    }
  };
  auto compute = [&](const u32x2* pq, const u32x2* qq) {
    u32x4 pf[4], qf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pf[j] = column_of_8x4(pq, j);
      qf[j] = column_of_8x4(qq, j);
    }
#pragma unroll
    for (int ja = 0; ja < 4; ++ja)
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) acc[ja][jb] = mfma_bf16(qf[jb], pf[ja], acc[ja][jb]);
  };

  if (steps > 0) {
    u32x2 pA[8], qA[8], pB[8], qB[8];
    load(0, pA, qA);
    int s = 0;
    for (; s + 2 <= steps; s += 2) {
      load(s + 1, pB, qB);
      compute(pA, qA);
      if (s + 2 < steps) load(s + 2, pA, qA);
      compute(pB, qB);
    }
    if (s < steps) compute(pA, qA);
  }

  // lane (c, gq) holds rows mb + 4c + ja and columns nb + 16gq + 4r + jb
#pragma unroll
  for (int ja = 0; ja < 4; ++ja) {
    uint16_t* orow = out + (size_t)(mb + 4 * c + ja) * ldo + nb + 16 * gq + out_col0;
    u32x4 lo, hi;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      lo[2 * r] = pack_bf2(acc[ja][0][r], acc[ja][1][r]);
      lo[2 * r + 1] = pack_bf2(acc[ja][2][r], acc[ja][3][r]);
      hi[2 * r] = pack_bf2(acc[ja][0][r + 2], acc[ja][1][r + 2]);
      hi[2 * r + 1] = pack_bf2(acc[ja][2][r + 2], acc[ja][3][r + 2]);
    }
    *(u32x4*)orow = lo;
    *(u32x4*)(orow + 8) = hi;
  }
}

}  // namespace

hipError_t launch_row_gemm_bf16(int mode, const RowGemmArgs& g, int max_rows, hipStream_t stream) {
  const int64_t tiles = ((int64_t)max_rows + (int64_t)g.E * (kTileRows - 1)) / kTileRows;
  if (tiles <= 0) return hipSuccess;
  int nblocks;
  switch (mode) {
    case kGemmGateUp: nblocks = g.F / 64; break;
    case kGemmDA: nblocks = g.F / 128; break;
    default: nblocks = g.H / 128; break;
  }
  const dim3 grid((unsigned)tiles, (unsigned)nblocks);
  switch (mode) {
    case kGemmGateUp: hipLaunchKernelGGL(row_gemm_bf16_kernel<kGemmGateUp>, grid, dim3(256), 0, stream, g); break;
    case kGemmDown: hipLaunchKernelGGL(row_gemm_bf16_kernel<kGemmDown>, grid, dim3(256), 0, stream, g); break;
    case kGemmDA: hipLaunchKernelGGL(row_gemm_bf16_kernel<kGemmDA>, grid, dim3(256), 0, stream, g); break;
    default: hipLaunchKernelGGL(row_gemm_bf16_kernel<kGemmDX>, grid, dim3(256), 0, stream, g); break;
  }
  return hipGetLastError();
}

hipError_t launch_dw_bf16(DwArgs g, hipStream_t stream) {
  g.tiles_job1 = (g.H / 128) * ((2 * g.F) / 128);
  g.tiles_per_expert = g.tiles_job1 + (g.F / 128) * (g.H / 128);
  const int64_t blocks = (int64_t)g.E * g.tiles_per_expert;
  hipLaunchKernelGGL(dw_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g);
  return hipGetLastError();
}

}  // namespace moe
