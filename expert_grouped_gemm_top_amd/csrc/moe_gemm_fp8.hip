// moe_gemm_fp8.hip -- the expert forward's grouped GEMMs on the gfx950 fp8
// matrix core (v_mfma_scale_f32_32x32x64_f8f6f4: E4M3 x E4M3, fp32 accumulate,
// twice the bf16 rate).
//
// Variable-size grouped GEMMs (LRMoE abstract) of the SwiGLU experts (npu-train
// issue #14, section Proposal), forward only, every expert on 256 x 256 tiles
// (rows of one expert x output columns), ragged row tails included:
//   GATEUP  xq rows [s][H] x [W_gate^T | W_up^T][e] ([F][H] codes each) -> h=[hg|hu], a=silu(hg)*hu (bf16)
//   DOWN    aq rows [s][F] x W_down^T[e] ([H][F] codes)                 -> o (bf16)
// Both operands are K-contiguous codes (the weights transposed once, see
// moe_transpose_fp8), so both tiles land in LDS as [row][128 k] by direct
// global->LDS loads and every fragment is two 16-byte reads: lane l of a
// 32x32x64 operand holds row (or column) l % 32 and k 32 (l / 32) .. + 31.
// Each product is scaled in the epilogue by the activation row's and the
// expert's power-of-two scales (exact).  Chunks past the reduction or the
// output edge load from a zero chunk; columns past the edge are not stored.
#include <algorithm>

#include "moe_common.h"
#include "moe_launch.h"
#include "moe_lds32.h"

namespace moe {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kF8BM = 256, kF8BN = 256, kF8BK = 128;  // rows, columns, k (bytes) per stage
constexpr int kF8Waves = 8, kF8WM = 2;               // waves as 2 (rows) x 4 (columns), each 128 x 64
constexpr int kF8Stages = 2;
constexpr int kF8TM = kF8BM / kF8WM, kF8TN = kF8BN / (kF8Waves / kF8WM);
constexpr int kF8MI = kF8TM / 32, kF8NJ = kF8TN / 32;
constexpr int kF8ABytes = kF8BM * kF8BK, kF8BBytes = kF8BN * kF8BK;
constexpr int kF8StageBytes = kF8ABytes + kF8BBytes;
constexpr int kF8AIns = kF8ABytes / 1024 / kF8Waves, kF8BIns = kF8BBytes / 1024 / kF8Waves;
constexpr int kF8Ins = kF8AIns + kF8BIns;
constexpr int kF8CPR = kF8BK / 16;  // 16-byte chunks per tile row
static_assert(kF8CPR == 8, "chunk swizzle key row & 7");

// LDS position of chunk `c` of tile row `row`: XOR by (row >> 1) & 7, so that
// the 16-byte reads of 16 consecutive 128-byte rows (two rows per 256 bytes of
// banks) fall in distinct bank groups (measured: no bank-conflict cycles; the
// key row & 7 left rows r and r + 8 in the same banks).
__device__ __forceinline__ int f8_swz(int row, int c) { return c ^ ((row >> 1) & 7); }

// D = first x second + D, fp8 operands (32 bytes per lane), unit scales
// (E8M0 127 = 2^0): the operands' power-of-two scales are applied afterwards.
__device__ __forceinline__ f32x16 mfma_fp8(const u32x4 (&first)[2], const u32x4 (&second)[2], f32x16 acc) {
  const i32x8 a = {(int)first[0][0], (int)first[0][1], (int)first[0][2], (int)first[0][3],
                   (int)first[1][0], (int)first[1][1], (int)first[1][2], (int)first[1][3]};
  const i32x8 b = {(int)second[0][0], (int)second[0][1], (int)second[0][2], (int)second[0][3],
                   (int)second[1][0], (int)second[1][1], (int)second[1][2], (int)second[1][3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc, 0, 0, 0, 127, 0, 127);
}

// 16 B from sbase + voff straight into LDS at lds_base + 16 * lane: the
// 64-bit base in scalar registers (wave-uniform), a 32-bit offset per lane,
// which holds one vector register per load address instead of two.
__device__ __forceinline__ void g2lds_off(const void* sbase, uint32_t voff, void* lds_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds)
      : "memory");
}

// wave-uniform pointer held in scalar registers
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// OFF32: whole-tile shapes (the reduction a multiple of kF8BK, the output
// width one of kF8BN: no chunk past an edge) whose operands lie within 4 GiB
// of their base (activation codes, and one expert's weight matrix): loads
// address by base + 32-bit offset, and the next stage's loads go out in two
// halves, A before the stage's first MFMA run and B before its second.
template <int MODE, bool OFF32>
__global__ __launch_bounds__(64 * kF8Waves, 1) void big_gemm_fp8_kernel(Fp8GemmArgs g) {
  static_assert(MODE == kGemmGateUp || MODE == kGemmDown, "forward products only");
  __shared__ int s_start[kMaxExperts + 1], s_off[kMaxExperts + 1], s_tmp[4];
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;

  // ---- schedule: every expert with rows, ceil(n_e / 256) row tiles each
  if (tid <= g.E) s_off[tid] = g.offsets[tid];  // 512 threads > E + 1
  __syncthreads();
  {
    int n_tiles = 0;
    if (tid < g.E) n_tiles = (s_off[tid + 1] - s_off[tid] + kF8BM - 1) / kF8BM;
    const int wv = tid >> 6;
    const int inc = wave_inclusive_scan(n_tiles);
    if (wv < 4 && l == 63) s_tmp[wv] = inc;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < 4; ++i) base += (i < wv) ? s_tmp[i] : 0;
    if (tid < g.E) s_start[tid] = base + inc - n_tiles;
    if (tid == 0) s_start[g.E] = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    __syncthreads();
  }
  const int H = g.H, F = g.F;
  const int ncols = MODE == kGemmGateUp ? 2 * F : H;  // virtual output columns (gate/up interleaved)
  const int nblk = (ncols + kF8BN - 1) / kF8BN;
  const int item = xcd_item(blockIdx.x, s_start[g.E] * nblk);
  if (item >= s_start[g.E] * nblk) return;
  int lo = 0, hi = g.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_start[mid] * nblk <= item) lo = mid; else hi = mid;
  }
  // groups of up to 4 row tiles x all column blocks, column-major within a group
  const int tiles_e = s_start[lo + 1] - s_start[lo];
  const int li = item - s_start[lo] * nblk;
  const int grp = li / (4 * nblk);
  const int gm = min(4, tiles_e - 4 * grp);
  const int within = li - grp * 4 * nblk;
  const int mt = 4 * grp + within % gm;
  const int nb = within / gm;
  const TileSlot ts = lookup_tile(s_start, s_off, g.E, kF8BM, s_start[lo] + mt);
  const int e = ts.expert;
  const int K = MODE == kGemmGateUp ? H : F;  // bytes (codes) per operand row
  const int wm = w % kF8WM, wn = w / kF8WM;
  const int l32 = l & 31, hk = l >> 5;

  // ---- loaders: an instruction covers 8 tile rows (8 lanes x 16 B each)
  const uint8_t* a_src[kF8AIns];
  int a_k[kF8AIns];
#pragma unroll
  for (int i = 0; i < kF8AIns; ++i) {
    const int row = 8 * (kF8AIns * w + i) + l / 8;
    const int c = f8_swz(row, l % 8);  // LDS position l % 8 of this row holds chunk c
    const int r = row < ts.rows ? row : ts.rows - 1;
    const int s = ts.row_begin + r;
    const int64_t src_row = g.a_map != nullptr ? (int64_t)(g.a_map[s] / g.a_div) : (int64_t)s;
    a_k[i] = 16 * c;
    a_src[i] = g.a + src_row * K + 16 * c;
  }
  const uint8_t* b_src[kF8BIns];
  int b_k[kF8BIns];
  bool b_ok[kF8BIns];
#pragma unroll
  for (int i = 0; i < kF8BIns; ++i) {
    const int row = 8 * (kF8BIns * w + i) + l / 8;  // virtual output column within the block
    const int c = f8_swz(row, l % 8);
    const uint8_t* Wt;
    int n;
    if (MODE == kGemmGateUp) {
      // 8-column chunks alternate W_gate / W_up over the same 8 features
      const int vchunk = row >> 3;
      n = nb * (kF8BN / 2) + 8 * (vchunk >> 1) + (row & 7);  // feature
      b_ok[i] = n < F;
      Wt = ((vchunk & 1) ? g.w1 : g.w0) + (size_t)e * F * H;
    } else {
      n = nb * kF8BN + row;
      b_ok[i] = n < H;
      Wt = g.w0 + (size_t)e * H * F;
    }
    b_k[i] = 16 * c;
    b_src[i] = Wt + (size_t)(b_ok[i] ? n : 0) * K + 16 * c;
  }
  // OFF32 addressing: bases in scalar registers, offsets per lane
  // B instructions i and i + 2 read the same chunk position of weight rows
  // b_step bytes apart (8 features on for gate/up, 16 output columns for down),
  // so two offsets per lane serve all four.
  static_assert(kF8BIns == 4, "B offsets: instructions 0, 1 and their successors two on");
  uint32_t a_off[kF8AIns], b_off[2];
  const uint32_t b_step = (uint32_t)K * (MODE == kGemmGateUp ? 8u : 16u);
  const uint8_t* a_base = uniform_ptr(g.a);
  const uint8_t* b_base0 = uniform_ptr(g.w0 + (size_t)e * F * H);
  const uint8_t* b_base1 = uniform_ptr((MODE == kGemmGateUp ? g.w1 : g.w0) + (size_t)e * F * H);
  if constexpr (OFF32) {
#pragma unroll
    for (int i = 0; i < kF8AIns; ++i) a_off[i] = (uint32_t)(a_src[i] - g.a);
    // gate/up: instruction i reads W_up when i is odd (its 8-row chunk index 4 w + i)
    b_off[0] = (uint32_t)(b_src[0] - b_base0);
    b_off[1] = (uint32_t)(b_src[1] - (MODE == kGemmGateUp ? b_base1 : b_base0));
  }
  auto issue_a = [&](int s) {
    unsigned char* st = s_dyn + (s % kF8Stages) * kF8StageBytes;
    const int k0 = s * kF8BK;
#pragma unroll
    for (int i = 0; i < kF8AIns; ++i) {
      if constexpr (OFF32) {
        g2lds_off(a_base, a_off[i] + (uint32_t)k0, st + 1024 * (kF8AIns * w + i));
      } else {
        const void* src = k0 + a_k[i] < K ? (const void*)(a_src[i] + k0) : (const void*)zero_chunk();
        g2lds(src, st + 1024 * (kF8AIns * w + i));
      }
    }
  };
  auto issue_b = [&](int s) {
    unsigned char* st = s_dyn + (s % kF8Stages) * kF8StageBytes;
    const int k0 = s * kF8BK;
#pragma unroll
    for (int i = 0; i < kF8BIns; ++i) {
      if constexpr (OFF32) {
        g2lds_off((MODE == kGemmGateUp && (i & 1)) ? b_base1 : b_base0,
                  b_off[i & 1] + (i >> 1) * b_step + (uint32_t)k0, st + kF8ABytes + 1024 * (kF8BIns * w + i));
      } else {
        const void* src = (b_ok[i] && k0 + b_k[i] < K) ? (const void*)(b_src[i] + k0) : (const void*)zero_chunk();
        g2lds(src, st + kF8ABytes + 1024 * (kF8BIns * w + i));
      }
    }
  };
  auto issue = [&](int s) { issue_a(s); issue_b(s); };

  f32x16 acc[kF8MI][kF8NJ];
#pragma unroll
  for (int i = 0; i < kF8MI; ++i)
#pragma unroll
    for (int j = 0; j < kF8NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  struct Frags {
    u32x4 a[kF8MI][2];
    u32x4 b[kF8NJ][2];
  };
  // fragments of sub-step `sub` (64 k) of the stage in LDS buffer `st`:
  // 16-byte chunks 4 sub + 2 hk and + 1 of the lane's row / column
  auto read_frags = [&](const unsigned char* st, int sub, Frags& fr) {
    const unsigned char* sb = st + kF8ABytes;
    const int c0 = 4 * sub + 2 * hk;
#pragma unroll
    for (int i = 0; i < kF8MI; ++i) {
      const int row = kF8TM * wm + 32 * i + l32;
#pragma unroll
      for (int h = 0; h < 2; ++h) fr.a[i][h] = *(const u32x4*)(st + row * kF8BK + 16 * f8_swz(row, c0 + h));
    }
#pragma unroll
    for (int j = 0; j < kF8NJ; ++j) {
      const int row = kF8TN * wn + 32 * j + l32;
#pragma unroll
      for (int h = 0; h < 2; ++h) fr.b[j][h] = *(const u32x4*)(sb + row * kF8BK + 16 * f8_swz(row, c0 + h));
    }
  };
  auto mfmas = [&](const Frags& fr) {
#pragma unroll
    for (int j = 0; j < kF8NJ; ++j)
#pragma unroll
      for (int i = 0; i < kF8MI; ++i) acc[i][j] = mfma_fp8(fr.b[j], fr.a[i], acc[i][j]);
  };
  // one sub-step's MFMAs with the next sub-step's fragment reads woven in
  auto mfmas_interleaved = [&](const Frags& cur, const unsigned char* st, int next_sub, Frags& nxt) {
    __builtin_amdgcn_s_setprio(1);
    if (next_sub >= 0) read_frags(st, next_sub, nxt);
    mfmas(cur);
#pragma unroll
    for (int q = 0; q < kF8MI * kF8NJ; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads (one fragment)
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  const int steps = (K + kF8BK - 1) / kF8BK;
  static_assert(kF8Stages == 2 && kF8BK == 128, "two stage buffers of two sub-steps");
  // Stage handoff before the last sub-step: stage s is waited for and the
  // workgroup synchronized while stage s - 1's last fragments are in
  // registers, so stage s's first fragments are read under stage s - 1's last
  // MFMAs (no fragment-read bubble at stage starts).  After that barrier every
  // wave is done reading stage s - 1's buffer, which then takes stage s + 1.
  issue(0);
  wait_vmcnt<0>();
  barrier_no_fence();
  if (steps > 1) issue(1);
  Frags f0, f1;
  read_frags(s_dyn, 0, f0);
  mfmas_interleaved(f0, s_dyn, 1, f1);
  auto stage_sync = [&] {
    wait_vmcnt<0>();                      // stage s has landed (the only loads in flight)
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of stage s - 1 are done
    barrier_no_fence();                   // ... and every wave's: its buffer can take stage s + 1
  };
  if constexpr (OFF32) {
    // stages 1 .. steps - 2 load the next stage in two halves; the last one
    // loads nothing and is peeled off: with a branch around each half inside
    // the loop, the compiler placed both halves ahead of the first MFMA run
    for (int s = 1; s < steps - 1; ++s) {
      const unsigned char* st = s_dyn + (s & 1) * kF8StageBytes;
      stage_sync();
      issue_a(s + 1);
      mfmas_interleaved(f1, st, 0, f0);   // stage s - 1's last sub-step, stage s's first fragments
      issue_b(s + 1);
      mfmas_interleaved(f0, st, 1, f1);
    }
    if (steps > 1) {
      const unsigned char* st = s_dyn + ((steps - 1) & 1) * kF8StageBytes;
      stage_sync();
      mfmas_interleaved(f1, st, 0, f0);
      mfmas_interleaved(f0, st, 1, f1);
    }
  } else {
    for (int s = 1; s < steps; ++s) {
      const unsigned char* st = s_dyn + (s & 1) * kF8StageBytes;
      stage_sync();
      if (s + 1 < steps) issue(s + 1);
      mfmas_interleaved(f1, st, 0, f0);   // stage s - 1's last sub-step, stage s's first fragments
      mfmas_interleaved(f0, st, 1, f1);
    }
  }
  mfmas_interleaved(f1, s_dyn, -1, f0);

  // ---- epilogue: acc[i][j] register r -> activation row TM wm + 32 i + l32,
  // virtual column TN wn + 32 j + 8 q + 4 hk + (0..3), q = r / 4; scaled by
  // the row's and the expert's power-of-two scales.  The bf16 results are
  // staged in the idle stage buffers as [row][columns] (16-byte chunk c of
  // row r at chunk c ^ (r & 15)) and leave as 16-byte lanes of contiguous row
  // runs; storing the MFMA layout's 8-byte pieces straight to memory touches
  // 32 rows per instruction.  Gate/up: round 1 stages [hg | hu], round 2 the
  // SwiGLU output a.
  const float sw = g.wscale[e];
  float sc[kF8MI];  // scale of each of this lane's rows (rows past the tile: any finite value, never stored)
#pragma unroll
  for (int i = 0; i < kF8MI; ++i) {
    const int s = ts.row_begin + min(kF8TM * wm + 32 * i + l32, ts.rows - 1);
    const int64_t src_row = g.a_map != nullptr ? (int64_t)(g.a_map[s] / g.a_div) : (int64_t)s;
    sc[i] = g.ascale[src_row] * sw;
  }
  constexpr int FT = MODE == kGemmGateUp ? kF8BN / 2 : kF8BN;  // columns of one staged matrix
  constexpr int PITCH = 2 * FT, CH = FT / 8;
  static_assert(CH >= 16 && (MODE == kGemmGateUp ? 2 : 1) * kF8BM * PITCH <= kF8Stages * kF8StageBytes, "staging");
  auto put = [&](unsigned char* m, int row, int col, u32x2 v) {  // 4 bf16 at columns col .. col + 3
    *(u32x2*)(m + row * PITCH + 16 * ((col >> 3) ^ (row & 15)) + 2 * (col & 7)) = v;
  };
  auto sync_lds = [] {
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS accesses are done
    barrier_no_fence();                   // ... and every wave's
  };
  sync_lds();  // every wave is done reading the stage buffers
  if (MODE == kGemmGateUp) {
    unsigned char* sg = s_dyn;                  // hg, then a
    unsigned char* su = s_dyn + kF8BM * PITCH;  // hu
    const int fb = (kF8BN / 2) * nb;            // first feature of the tile
    // a, packed to bf16 up front, so that the accumulators are dead once h is staged
    u32x2 apk[kF8MI][kF8NJ][2];
#pragma unroll
    for (int i = 0; i < kF8MI; ++i)
#pragma unroll
      for (int j = 0; j < kF8NJ; ++j)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float av[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const float hgv = acc[i][j][8 * p + e2] * sc[i], huv = acc[i][j][8 * p + 4 + e2] * sc[i];
            av[e2] = hgv * sigmoidf_fast(hgv) * huv;
          }
          apk[i][j][p] = u32x2{pack_bf2(av[0], av[1]), pack_bf2(av[2], av[3])};
        }
    if (g.out0 != nullptr) {
#pragma unroll
      for (int i = 0; i < kF8MI; ++i)
#pragma unroll
        for (int j = 0; j < kF8NJ; ++j)
#pragma unroll
          for (int p = 0; p < 2; ++p) {
            const int row = kF8TM * wm + 32 * i + l32, fl = (kF8TN * wn + 32 * j) / 2 + 8 * p + 4 * hk;
            const f32x16& a = acc[i][j];
            put(sg, row, fl, u32x2{pack_bf2(a[8 * p] * sc[i], a[8 * p + 1] * sc[i]),
                                   pack_bf2(a[8 * p + 2] * sc[i], a[8 * p + 3] * sc[i])});
            put(su, row, fl, u32x2{pack_bf2(a[8 * p + 4] * sc[i], a[8 * p + 5] * sc[i]),
                                   pack_bf2(a[8 * p + 6] * sc[i], a[8 * p + 7] * sc[i])});
          }
      sync_lds();
      for (int it = tid; it < 2 * kF8BM * CH; it += 64 * kF8Waves) {
        const int row = it / (2 * CH), c2 = it % (2 * CH), up = c2 >= CH, c = up ? c2 - CH : c2;
        const int f = fb + 8 * c;
        if (row < ts.rows && f < F)  // F is a multiple of 8: a chunk is all in or all out
          *(u32x4*)(g.out0 + ((size_t)ts.row_begin + row) * 2 * F + (up ? F : 0) + f) =
              *(const u32x4*)((up ? su : sg) + row * PITCH + 16 * (c ^ (row & 15)));
      }
      sync_lds();
    }
#pragma unroll
    for (int i = 0; i < kF8MI; ++i)
#pragma unroll
      for (int j = 0; j < kF8NJ; ++j)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          put(sg, kF8TM * wm + 32 * i + l32, (kF8TN * wn + 32 * j) / 2 + 8 * p + 4 * hk, apk[i][j][p]);
    sync_lds();
    for (int it = tid; it < kF8BM * CH; it += 64 * kF8Waves) {
      const int row = it / CH, c = it % CH, f = fb + 8 * c;
      if (row < ts.rows && f < F)
        *(u32x4*)(g.out1 + ((size_t)ts.row_begin + row) * F + f) = *(const u32x4*)(sg + row * PITCH + 16 * (c ^ (row & 15)));
    }
  } else {
#pragma unroll
    for (int i = 0; i < kF8MI; ++i)
#pragma unroll
      for (int j = 0; j < kF8NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          put(s_dyn, kF8TM * wm + 32 * i + l32, kF8TN * wn + 32 * j + 8 * q + 4 * hk,
              u32x2{pack_bf2(acc[i][j][4 * q] * sc[i], acc[i][j][4 * q + 1] * sc[i]),
                    pack_bf2(acc[i][j][4 * q + 2] * sc[i], acc[i][j][4 * q + 3] * sc[i])});
    sync_lds();
    for (int it = tid; it < kF8BM * CH; it += 64 * kF8Waves) {
      const int row = it / CH, c = it % CH, col = nb * kF8BN + 8 * c;
      if (row < ts.rows && col < H)  // H is a multiple of 8
        *(u32x4*)(g.out0 + ((size_t)ts.row_begin + row) * H + col) = *(const u32x4*)(s_dyn + row * PITCH + 16 * (c ^ (row & 15)));
    }
  }
}

template <int MODE>
hipError_t launch_fp8_mode(const Fp8GemmArgs& g, int max_rows, hipStream_t stream) {
  const int64_t N = max_rows, E = g.E;
  const int64_t tiles = (N + E * (kF8BM - 1)) / kF8BM;
  const int ncols = MODE == kGemmGateUp ? 2 * g.F : g.H;
  const int64_t wgs = ((tiles * ((ncols + kF8BN - 1) / kF8BN) + 7) / 8) * 8;
  if (wgs <= 0) return hipSuccess;
  const size_t lds = (size_t)kF8Stages * kF8StageBytes;
  const int64_t K = MODE == kGemmGateUp ? g.H : g.F;
  // whole tiles, and every operand byte within 4 GiB of its base: the rows of
  // a (at most max_rows of them, gathered or not) and one expert's weights
  // (the down product only: gate/up measured no faster with the split issue)
  const bool off32 = MODE == kGemmDown && K % kF8BK == 0 && ncols % kF8BN == 0 && N * K < ((int64_t)1 << 32) &&
                     (int64_t)g.H * g.F < ((int64_t)1 << 32);
  auto kern = big_gemm_fp8_kernel<MODE, false>;
  if constexpr (MODE == kGemmDown) {
    if (off32) kern = big_gemm_fp8_kernel<MODE, true>;
  }
  static PerDeviceOnce lds_once[2];
  hipError_t err = allow_dynamic_lds(lds_once[off32 ? 1 : 0], (const void*)kern, lds);
  if (err != hipSuccess) return err;
  MOE_LAUNCH(kern, dim3((unsigned)wgs), dim3(64 * kF8Waves), lds, stream, g);
  return hipGetLastError();
}

// out[e][c][r] = in[e][r][c] for bytes; 64 x 64 tiles through LDS (rows and
// columns multiples of 16).
__global__ __launch_bounds__(256) void transpose_u8_kernel(int rows, int cols, const uint8_t* __restrict__ in,
                                                           uint8_t* __restrict__ out) {
  __shared__ uint8_t s_t[64][64 + 16];
  const int e = blockIdx.z, r0 = blockIdx.y * 64, c0 = blockIdx.x * 64, tid = threadIdx.x;
  const uint8_t* src = in + (size_t)e * rows * cols;
  uint8_t* dst = out + (size_t)e * rows * cols;
  {
    const int r = tid >> 2, c = 16 * (tid & 3);
    if (r0 + r < rows && c0 + c < cols) {
      const u32x4 v = *(const u32x4*)(src + (size_t)(r0 + r) * cols + c0 + c);
      *(u32x4*)&s_t[r][c] = v;
    }
  }
  __syncthreads();
  {
    const int c = tid >> 2, r = 16 * (tid & 3);  // output row (input column) c, 16 input rows from r
    if (c0 + c < cols && r0 + r < rows) {
      uint32_t wv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) word |= (uint32_t)s_t[r + 4 * q + b][c] << (8 * b);
        wv[q] = word;
      }
      *(u32x4*)(dst + (size_t)(c0 + c) * rows + r0 + r) = u32x4{wv[0], wv[1], wv[2], wv[3]};
    }
  }
}

}  // namespace

hipError_t launch_gemm_fp8(int mode, const Fp8GemmArgs& g, int max_rows, hipStream_t stream) {
  return mode == kGemmGateUp ? launch_fp8_mode<kGemmGateUp>(g, max_rows, stream)
                             : launch_fp8_mode<kGemmDown>(g, max_rows, stream);
}

hipError_t launch_transpose_u8(int E, int rows, int cols, const uint8_t* in, uint8_t* out, hipStream_t stream) {
  const dim3 grid((unsigned)((cols + 63) / 64), (unsigned)((rows + 63) / 64), (unsigned)E);
  MOE_LAUNCH(transpose_u8_kernel, grid, dim3(256), 0, stream, rows, cols, in, out);
  return hipGetLastError();
}

}  // namespace moe
