// moe_gemm_big.hip -- row GEMMs of the SwiGLU experts for experts with many
// rows (>= 256), where the grouped GEMM is bound by the matrix cores.
//
// The four products of the row GEMMs (expert forward and backward dx:
// npu-train issue #14, sections Proposal and Scope; variable-size grouped
// GEMMs: LRMoE abstract), tiled for gfx950:
//   * workgroup tile BM rows x BN columns, waves laid out WM x (NW / WM), each
//     wave a grid of 32 x 32 blocks on v_mfma_f32_32x32x16_bf16
//     (on gfx950 it sustains ~2.4 PFLOP/s where the 16x16x32 form stops near
//     1.4 PFLOP/s);
//   * operands move global -> LDS with global_load_lds_dwordx4 (no register
//     staging), several K-stages of BK in flight;
//   * K-contiguous operands (activation rows, backward weights) land as
//     [row][BK] rows with the 16-byte chunks XOR-swizzled per row, keys that
//     measured conflict-free for 16-byte fragment reads of 16 consecutive rows;
//   * N-contiguous weights (forward) land as [32 k][BN] and are read with the
//     gfx950 transpose read ds_read_b64_tr_b16: lane r of a 16-lane group
//     points at row r / 4, column quad r % 4, and receives 4 consecutive k of
//     one column -- half of a 32x32x16 B fragment; 64-byte chunk groups are
//     XOR-swizzled by 4 (k & 3) so the rows of one read fall in distinct banks;
//   * rows past the tile's real rows re-read the tile's last row: they only
//     produce output rows that are never stored;
//   * dA's SwiGLU backward needs the saved pre-activations of every output:
//     its tile is staged through the idle stage buffers so that h is read and
//     dh written as 16-byte runs of one row.
#include <algorithm>

#include "moe_common.h"
#include "moe_launch.h"
#include "moe_lds32.h"

namespace moe {

namespace {

template <int MODE>
struct BigShape {
  static constexpr bool kNN = (MODE == kGemmGateUp || MODE == kGemmDown);
};

template <int MODE>
__host__ __device__ inline int big_out_cols(int H, int F) {
  return MODE == kGemmGateUp ? 2 * F : (MODE == kGemmDA ? F : H);
}

template <int MODE>
__host__ __device__ inline int big_reduction(int H, int F) {
  return (MODE == kGemmGateUp || MODE == kGemmDA) ? H : (MODE == kGemmDown ? F : 2 * F);
}

// K-contiguous tile rows of BK elements (CPR 16-byte chunks): swizzled chunk
// position, so that the 16-byte fragment reads of 16 consecutive rows hit
// distinct bank groups (the LDS serves 256 bytes of banks at once: 64-byte
// rows, key (row >> 2) & 3, so rows r, r + 4, r + 8, r + 12 -- same offset
// within 256 bytes -- take distinct chunks; 128-byte rows, key (row >> 1) & 7
// -- the key row & 7 had rows r and r + 8 collide, measured as 10 % of the
// kernel's cycles in bank conflicts, now none).
template <int CPR>
__device__ __forceinline__ int kc_swz(int row, int chunk) {
  return CPR == 4 ? (chunk ^ ((row >> 2) & 3)) : (chunk ^ ((row >> 1) & 7));
}

// Tile of BM rows x BN columns, reduction depth BK per stage, NW waves laid out
// WM x (NW / WM); STAGES stages resident in LDS; WPC workgroups per CU.
// TAIL: the reduction length is not a multiple of BK, or the output width not
// one of BN (or, for dX, F not one of BK): every direct load then picks its
// source per stage, and 16-byte chunks past the reduction or the output edge
// come from a chunk of zeros; output columns past the edge are not stored.
template <int MODE, int BM, int BN, int BK, int NW, int WM, int STAGES, int WPC, bool TAIL>
__global__ __launch_bounds__(64 * NW, WPC) void big_gemm_bf16_kernel(RowGemmArgs g) {
  constexpr bool NN = BigShape<MODE>::kNN;
  const int kMinRows = g.big_min_rows;  // experts with at least this many rows use this kernel
  constexpr int WNW = NW / WM;          // waves along N
  constexpr int TM = BM / WM;           // rows per wave
  constexpr int TN = BN / WNW;          // columns per wave
  constexpr int MI = TM / 32, NJ = TN / 32;
  constexpr int CPR = BK / 8;           // 16-byte chunks per K-contiguous row
  constexpr int A_BYTES = BM * BK * 2;
  constexpr int B_BYTES = BN * BK * 2;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int A_INS = A_BYTES / 1024 / NW;  // direct loads per wave per stage
  constexpr int B_INS = B_BYTES / 1024 / NW;
  constexpr int INS = A_INS + B_INS;
  static_assert(A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0, "tile / wave split");
  static_assert(MI >= 1 && NJ >= 1, "wave tile");
  __shared__ int s_start[kMaxExperts + 1], s_off[kMaxExperts + 1], s_tmp[4];
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];

  // schedule (the builder needs 256 threads; larger workgroups run it on the first 256)
  static_assert(NW == 4 || 64 * NW > kMaxExperts, "every offsets entry has a thread");
  if (NW == 4) {
    build_tile_starts(g.offsets, g.E, BM, s_start, s_off, s_tmp, kMinRows);
  } else {
    const bool first = threadIdx.x < 256;
    if (threadIdx.x <= g.E) s_off[threadIdx.x] = g.offsets[threadIdx.x];  // 64 NW >= 512 > E threads
    __syncthreads();
    int n_tiles = 0;
    if (first && threadIdx.x < g.E) {
      const int n = s_off[threadIdx.x + 1] - s_off[threadIdx.x];
      if (n >= kMinRows) n_tiles = (n + BM - 1) / BM;
    }
    // exclusive scan by the first four waves
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const int inc = wave_inclusive_scan(n_tiles);
    if (w < 4 && l == 63) s_tmp[w] = inc;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < 4; ++i) base += (i < w) ? s_tmp[i] : 0;
    if (first && threadIdx.x < g.E) s_start[threadIdx.x] = base + inc - n_tiles;
    if (threadIdx.x == 0) s_start[g.E] = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    __syncthreads();
  }
  const int H = g.H, F = g.F;
  const int nblk = (big_out_cols<MODE>(H, F) + BN - 1) / BN;
  const int item = xcd_item(blockIdx.x, s_start[g.E] * nblk);
  if (item >= s_start[g.E] * nblk) return;
  int lo = 0, hi = g.E;  // expert of this item
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
  const TileSlot ts = lookup_tile(s_start, s_off, g.E, BM, s_start[lo] + mt);
  const int e = ts.expert;
  const int K = big_reduction<MODE>(H, F);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w % WM, wn = w / WM;
  const int l32 = l & 31, hk = l >> 5;  // MFMA row/column and k-group of this lane

  // ---- loader: 1 KiB per direct-load instruction
  // A (K-contiguous rows of 2 BK bytes): instruction covers 64 / CPR rows
  const uint16_t* a_src[A_INS];
  int a_k[A_INS];  // k offset of this lane's chunk within a stage
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int row = (64 / CPR) * (A_INS * w + i) + l / CPR;
    const int chunk = kc_swz<CPR>(row, l % CPR);  // LDS position l % CPR holds this chunk
    const int r = row < ts.rows ? row : ts.rows - 1;
    a_k[i] = 8 * chunk;
    a_src[i] = g.a + a_row_of(g, ts.row_begin + r) * K + 8 * chunk;
  }
  const uint16_t* b_src[B_INS];
  const uint16_t* b_hi[B_INS];  // DX: the same rows in W_up for k >= F
  int b_k[B_INS];               // NN: k row of this lane within a stage; NT: k offset of its chunk
  bool b_ok[B_INS];             // the chunk's columns (NN) or weight row (NT) lie inside the output
  size_t b_kstride;             // elements per k for NN (row stride), 1 for NT
  if (NN) {
    // [BK k][BN]: a k row is BN/8 chunks; instruction covers 512 / BN k rows
    constexpr int ROWS_PER_INS = 512 / BN;
    b_kstride = (MODE == kGemmGateUp) ? F : H;
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      const int k = ROWS_PER_INS * (B_INS * w + i) + l / (BN / 8);
      const int pos = l % (BN / 8);
      const int vchunk = pos ^ nn_swz(k);  // virtual 8-column chunk stored at pos
      const uint16_t* W;
      int col;
      if (MODE == kGemmGateUp) {
        // virtual chunks alternate W_gate / W_up over the same 8 features
        W = ((vchunk & 1) ? g.w1 : g.w0) + (size_t)e * H * F;
        col = nb * (BN / 2) + 8 * (vchunk >> 1);
        b_ok[i] = col < F;
      } else {
        W = g.w0 + (size_t)e * F * H;
        col = nb * BN + 8 * vchunk;
        b_ok[i] = col < H;
      }
      b_k[i] = k;
      b_src[i] = W + (size_t)k * b_kstride + (b_ok[i] ? col : 0);
      b_hi[i] = b_src[i];
    }
  } else {
    b_kstride = 1;
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      const int row = (64 / CPR) * (B_INS * w + i) + l / CPR;  // output column within the tile
      const int chunk = kc_swz<CPR>(row, l % CPR);
      const int n = nb * BN + row;
      b_k[i] = 8 * chunk;
      if (MODE == kGemmDA) {
        // W_down [F,H]: output column n is weight row n
        b_ok[i] = n < F;
        b_src[i] = g.w0 + (size_t)e * F * H + (size_t)(b_ok[i] ? n : 0) * H + 8 * chunk;
        b_hi[i] = b_src[i];
      } else {
        b_ok[i] = n < H;
        const size_t nrow = (size_t)(b_ok[i] ? n : 0) * F;
        // DX: k < F from W_gate, k >= F from W_up
        b_src[i] = g.w0 + (size_t)e * H * F + nrow + 8 * chunk;
        b_hi[i] = g.w1 + (size_t)e * H * F + nrow + 8 * chunk;
      }
    }
  }

  // loads [lo, hi) of stage s in the order A (A_INS), then B (B_INS)
  auto issue_part = [&](int s, int lo, int hi) {
    unsigned char* st = s_dyn + (s % STAGES) * STAGE_BYTES;
    const int k0 = s * BK;
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
      if (i < lo || i >= hi) continue;
      const uint16_t* src = a_src[i] + k0;
      if (TAIL && k0 + a_k[i] >= K) src = zero_chunk();
      g2lds(src, st + 1024 * (A_INS * w + i));
    }
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
      if (A_INS + i < lo || A_INS + i >= hi) continue;
      const uint16_t* src;
      if (NN) {
        src = b_src[i] + (size_t)k0 * b_kstride;
        if (TAIL && (!b_ok[i] || k0 + b_k[i] >= K)) src = zero_chunk();
      } else if (!TAIL) {
        src = (MODE == kGemmDX && k0 >= F) ? b_hi[i] + (k0 - F) : b_src[i] + k0;
      } else {
        const int k = k0 + b_k[i];  // chunks never straddle F (a multiple of 8)
        src = (MODE == kGemmDX && k >= F) ? b_hi[i] + (k0 - F) : b_src[i] + k0;
        if (!b_ok[i] || k >= K) src = zero_chunk();
      }
      g2lds(src, st + A_BYTES + 1024 * (B_INS * w + i));
    }
  };
  auto issue = [&](int s) { issue_part(s, 0, INS); };

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  struct Frags {
    u32x4 a[MI];
    u32x4 b[NJ];
  };
  // fragments of sub-step `sub` (16 k) of the stage in LDS buffer `st`
  auto read_frags = [&](const unsigned char* st, int sub, Frags& fr) {
    const unsigned char* sb = st + A_BYTES;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = TM * wm + 32 * i + l32;
      fr.a[i] = *(const u32x4*)(st + row * (2 * BK) + 16 * kc_swz<CPR>(row, 2 * sub + hk));
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (NN) {
        fr.b[j] = tr_frag32(sb, BN * 2, sub, TN * wn + 32 * j);
      } else {
        const int row = TN * wn + 32 * j + l32;
        fr.b[j] = *(const u32x4*)(sb + row * (2 * BK) + 16 * kc_swz<CPR>(row, 2 * sub + hk));
      }
    }
  };
  auto mfmas = [&](const Frags& fr) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < MI; ++i) acc[i][j] = mfma32(fr.b[j], fr.a[i], acc[i][j]);
  };
  // Sub-steps are software-pipelined: the fragments of sub-step t+1 are read
  // from LDS while the MFMAs of sub-step t run.  One sub-step's MFMAs, with
  // the next sub-step's fragment reads woven between them one for one, at
  // raised wave priority.
  auto mfmas_interleaved = [&](const Frags& cur, const unsigned char* st, int next_sub, Frags& nxt) {
    __builtin_amdgcn_s_setprio(1);
    if (next_sub >= 0) read_frags(st, next_sub, nxt);
    mfmas(cur);
#pragma unroll
    for (int q = 0; q < MI * NJ; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };

  const int steps = (K + BK - 1) / BK;
  static_assert(STAGES == 2 && (BK / 16) % 2 == 0, "two stage buffers, an even number of sub-steps per stage");
  // Stage handoff before the last sub-step: stage s + 1 is waited for and the
  // workgroup synchronized while stage s's last fragments are in registers,
  // so the next stage's first fragments are read under the last MFMAs of this
  // one (no fragment-read bubble at stage starts).  After that barrier every
  // wave is done reading stage s's buffer, which then takes stage s + 2.
  issue(0);
  wait_vmcnt<0>();
  barrier_no_fence();
  if (steps > 1) issue(1);
  {
    constexpr int SUBS = BK / 16;
    Frags f0, f1;
    // sub-steps 0 .. SUBS-2 of the stage in `st`, starting with f0 holding
    // sub-step 0; leaves f1 holding sub-step SUBS-1 (read, not yet used)
    auto stage_body = [&](const unsigned char* st) {
#pragma unroll
      for (int t = 0; t + 2 < SUBS; t += 2) {
        mfmas_interleaved(f0, st, t + 1, f1);
        mfmas_interleaved(f1, st, t + 2, f0);
      }
      mfmas_interleaved(f0, st, SUBS - 1, f1);
    };
    read_frags(s_dyn, 0, f0);
    stage_body(s_dyn);
    // The next stage's loads go out in two halves, before this stage's first
    // two MFMA runs.  Issued all at once after the barrier, they made every
    // wave stall on the full memory-instruction queue with the matrix pipes
    // idle (measured with cycle counters: 30-40 % of a wave's time spent
    // issuing them); spreading them over all four runs leaves the last ones
    // too little time to land.
    static_assert(SUBS == 4, "four MFMA runs per stage");
    for (int s = 1; s < steps; ++s) {
      const unsigned char* st = s_dyn + (s & 1) * STAGE_BYTES;
      wait_vmcnt<0>();                      // stage s has landed (the only loads in flight)
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of stage s - 1 are done
      barrier_no_fence();                   // ... and every wave's: its buffer can take stage s + 1
      const bool more = s + 1 < steps;
      if (more) issue_part(s + 1, 0, INS / 2);
      mfmas_interleaved(f1, st, 0, f0);     // stage s - 1's last sub-step, stage s's first fragments
      if (more) issue_part(s + 1, INS / 2, INS);
      mfmas_interleaved(f0, st, 1, f1);
      mfmas_interleaved(f1, st, 2, f0);
      mfmas_interleaved(f0, st, 3, f1);
    }
    mfmas_interleaved(f1, s_dyn, -1, f0);
  }

  // ---- epilogue.  acc[i][j] register r -> row TM wm + 32 i + l32, tile
  // column TN wn + 32 j + 8 q + 4 hk + e with q = r / 4, e = r % 4.
  if constexpr (MODE == kGemmDA) {
    // dA -> dh = [dHg | dHu] through the SwiGLU backward.  The fp32 tile goes
    // to LDS in two halves of HC = BN / 2 columns (the stage buffers hold
    // one), each read back as 8 consecutive columns of one row per thread, so
    // h is read and dh written as contiguous row segments.  16-byte chunk c
    // of staged row r sits at chunk c ^ (r & 15): the MFMA-layout writes (16
    // rows, one chunk) touch 16 distinct bank groups, and so do the row reads
    // (HC = 64: two rows of opposite parity per 16 lanes; HC = 128: one row,
    // odd chunk first in the upper 8 lanes).
    constexpr int HC = BN / 2;
    static_assert(BM * HC * 4 <= STAGES * STAGE_BYTES && WNW % 2 == 0 && (HC == 64 || HC == 128), "dA staging");
    float* s_f = reinterpret_cast<float*>(s_dyn);
    auto staged = [&](int row, int chunk) { return s_f + row * HC + 4 * (chunk ^ (row & 15)); };
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's last fragment reads are done
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      barrier_no_fence();  // every wave is done with the stage buffers / the previous half
      if (wn / (WNW / 2) == half) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int row = TM * wm + 32 * i + l32;
              const int col = TN * (wn % (WNW / 2)) + 32 * j + 8 * q + 4 * hk;
              *(f32x4*)staged(row, col >> 2) =
                  f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the staged values are written
      barrier_no_fence();
      constexpr int C8 = HC / 8;  // 8-column groups per staged row
#pragma unroll 2
      for (int it = tid; it < BM * C8; it += 64 * NW) {
        const int row = it / C8, c8 = it % C8;
        const int f = nb * BN + half * HC + 8 * c8;  // feature of the group's first column
        if (row >= ts.rows || (TAIL && f >= F)) continue;  // F is a multiple of 8: a group is all in or all out
        const int first = 2 * c8 + (HC == 128 ? ((c8 >> 3) & 1) : 0);
        const f32x4 d_first = *(const f32x4*)staged(row, first);
        const f32x4 d_second = *(const f32x4*)staged(row, first ^ 1);
        const f32x4 d_lo = (first & 1) ? d_second : d_first, d_hi = (first & 1) ? d_first : d_second;
        const int64_t grow = (int64_t)ts.row_begin + row;
        const uint16_t* hrow = g.h + h_row_of(g, grow) * 2 * F;
        const u32x4 hg = *(const u32x4*)(hrow + f), hu = *(const u32x4*)(hrow + F + f);
        float dg[8], du[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const float da = c < 4 ? d_lo[c] : d_hi[c - 4];
          const float hgv = (c & 1) ? bf_hi(hg[c >> 1]) : bf_lo(hg[c >> 1]);
          const float huv = (c & 1) ? bf_hi(hu[c >> 1]) : bf_lo(hu[c >> 1]);
          const float sg = sigmoidf_fast(hgv);
          dg[c] = da * huv * sg * (1.0f + hgv * (1.0f - sg));
          du[c] = da * hgv * sg;
        }
        uint16_t* drow = g.out0 + grow * 2 * F;
        *(u32x4*)(drow + f) = u32x4{pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3]), pack_bf2(dg[4], dg[5]),
                                    pack_bf2(dg[6], dg[7])};
        *(u32x4*)(drow + F + f) = u32x4{pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3]), pack_bf2(du[4], du[5]),
                                        pack_bf2(du[6], du[7])};
      }
    }
    return;
  }
  // The other products leave through LDS too: the MFMA layout gives a lane 4
  // consecutive columns of one row per register quad, and storing those 8
  // bytes straight to memory touches 32 rows per instruction (measured: the
  // stores took 12-29 % of these kernels' time).  The bf16 results are staged
  // in the idle stage buffers as [row][columns] with 16-byte chunk c of row r
  // at chunk c ^ (r & 15) (16 consecutive rows of one chunk land in distinct
  // bank groups), then leave as whole 16-byte lanes of contiguous row runs.
  // Gate/up: round 1 stages [hg | hu] of the tile's BN / 2 features (the h
  // output), round 2 the SwiGLU output a, computed from the fp32 sums.
  {
    constexpr int FT = MODE == kGemmGateUp ? BN / 2 : BN;  // columns of one staged matrix
    constexpr int PITCH = 2 * FT;                          // bytes per staged row
    constexpr int CH = FT / 8;                             // 16-byte chunks per staged row
    static_assert(CH >= 16 && (MODE == kGemmGateUp ? 2 : 1) * BM * PITCH <= STAGES * STAGE_BYTES, "staging");
    auto put = [&](unsigned char* m, int row, int col, u32x2 v) {  // 4 bf16 at columns col .. col + 3
      *(u32x2*)(m + row * PITCH + 16 * ((col >> 3) ^ (row & 15)) + 2 * (col & 7)) = v;
    };
    // every staged chunk of every staged matrix goes out: items = BM x CH per matrix
    auto drain = [&](const unsigned char* m, uint16_t* out, int ld, int col0, int ncols) {
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's staging writes are done
      barrier_no_fence();                   // ... and every wave's
#pragma unroll 4
      for (int it = tid; it < BM * CH; it += 64 * NW) {
        const int row = it / CH, c = it % CH;
        const int col = col0 + 8 * c;
        if (row < ts.rows && (!TAIL || col < ncols))  // ncols is a multiple of 8: a chunk is all in or all out
          *(u32x4*)(out + ((size_t)ts.row_begin + row) * ld + col) =
              *(const u32x4*)(m + row * PITCH + 16 * (c ^ (row & 15)));
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's reads of the staged rows are done
      barrier_no_fence();                   // ... and every wave's: the buffers can be staged again
    };
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's last fragment reads are done
    barrier_no_fence();                   // ... and every wave's: the stage buffers are free
    if constexpr (MODE == kGemmGateUp) {
      // register 8 p + e of acc[i][j] -> hg, register 8 p + 4 + e -> hu, of
      // tile feature (TN wn + 32 j) / 2 + 8 p + 4 hk + e
      unsigned char* sg = s_dyn;                 // hg, then a
      unsigned char* su = s_dyn + BM * PITCH;    // hu
      const int fb = (BN / 2) * nb;              // first feature of the tile
      if (g.out0 != nullptr) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const int row = TM * wm + 32 * i + l32, fl = (TN * wn + 32 * j) / 2 + 8 * p + 4 * hk;
              put(sg, row, fl, u32x2{pack_bf2(acc[i][j][8 * p], acc[i][j][8 * p + 1]),
                                     pack_bf2(acc[i][j][8 * p + 2], acc[i][j][8 * p + 3])});
              put(su, row, fl, u32x2{pack_bf2(acc[i][j][8 * p + 4], acc[i][j][8 * p + 5]),
                                     pack_bf2(acc[i][j][8 * p + 6], acc[i][j][8 * p + 7])});
            }
        // hg and hu of one row leave together: chunks 0 .. CH-1 of sg, then of su
        __builtin_amdgcn_s_waitcnt(0xc07f);
        barrier_no_fence();
#pragma unroll 4
        for (int it = tid; it < 2 * BM * CH; it += 64 * NW) {
          const int row = it / (2 * CH), c2 = it % (2 * CH), up = c2 >= CH, c = up ? c2 - CH : c2;
          const int f = fb + 8 * c;
          if (row < ts.rows && (!TAIL || f < F))
            *(u32x4*)(g.out0 + ((size_t)ts.row_begin + row) * 2 * F + (up ? F : 0) + f) =
                *(const u32x4*)((up ? su : sg) + row * PITCH + 16 * (c ^ (row & 15)));
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);
        barrier_no_fence();
      }
      if (g.out1 != nullptr) {
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const int row = TM * wm + 32 * i + l32, fl = (TN * wn + 32 * j) / 2 + 8 * p + 4 * hk;
              float av[4];
#pragma unroll
              for (int e2 = 0; e2 < 4; ++e2) {
                const float hgv = acc[i][j][8 * p + e2], huv = acc[i][j][8 * p + 4 + e2];
                av[e2] = hgv * sigmoidf_fast(hgv) * huv;
              }
              put(sg, row, fl, u32x2{pack_bf2(av[0], av[1]), pack_bf2(av[2], av[3])});
            }
        drain(sg, g.out1, F, fb, F);
      }
    } else {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            put(s_dyn, TM * wm + 32 * i + l32, TN * wn + 32 * j + 8 * q + 4 * hk,
                u32x2{pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                      pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])});
      drain(s_dyn, g.out0, H, nb * BN, H);
    }
  }
}


// dA takes the 256-row kernel only for F of at least this many features: with
// fewer than four 256-column blocks per row tile its tiles are too few to
// fill the chip, and the 128-row tiles measured faster (F = 768: dA 251 ->
// 268 us at qwen3_ft_t4096; F = 1408: 1289 -> 1214 us at glm45air_t8192).
constexpr int kBigDaMinF = 1024;

template <int MODE, int BM, int BN, int BK, int NW, int WM, int STAGES, int WPC>
struct BigCfg {
  static int min_rows(int, int F) { return (MODE == kGemmDA && F < kBigDaMinF) ? kNoBigTiles : kBigTileMinRows; }

  template <bool TAIL>
  static hipError_t launch_as(const RowGemmArgs& g, int64_t wgs, hipStream_t stream) {
    const size_t lds = (size_t)STAGES * (BM + BN) * BK * 2;
    auto kern = big_gemm_bf16_kernel<MODE, BM, BN, BK, NW, WM, STAGES, WPC, TAIL>;
    // dynamic LDS above 64 KiB must be allowed explicitly, once per device
    static PerDeviceOnce lds_once;
    hipError_t err = allow_dynamic_lds(lds_once, (const void*)kern, lds);
    if (err != hipSuccess) return err;
    MOE_LAUNCH(kern, dim3((unsigned)wgs), dim3(64 * NW), lds, stream, g);
    return hipGetLastError();
  }

  static hipError_t launch(const RowGemmArgs& g, int max_rows, hipStream_t stream) {
    const int64_t N = max_rows, E = g.E;
    const int64_t big_experts = std::min<int64_t>(E, N / g.big_min_rows);
    if (big_experts == 0) return hipSuccess;
    const int64_t tiles = (N + big_experts * (BM - 1)) / BM;
    const int cols = big_out_cols<MODE>(g.H, g.F);
    const int64_t wgs = ((tiles * ((cols + BN - 1) / BN) + 7) / 8) * 8;
    const int K = big_reduction<MODE>(g.H, g.F);
    const bool tail = K % BK != 0 || cols % BN != 0 || (MODE == kGemmDX && g.F % BK != 0);
    return tail ? launch_as<true>(g, wgs, stream) : launch_as<false>(g, wgs, stream);
  }
};

template <int MODE>
using Big = BigCfg<MODE, 256, 256, 64, 8, 2, 2, 1>;  // BM, BN, BK, waves, waves along M, stages, workgroups per CU

}  // namespace

int big_gemm_min_rows(int mode, int H, int F) {
  switch (mode) {
    case kGemmGateUp: return Big<kGemmGateUp>::min_rows(H, F);
    case kGemmDown: return Big<kGemmDown>::min_rows(H, F);
    case kGemmDA: return Big<kGemmDA>::min_rows(H, F);
    default: return Big<kGemmDX>::min_rows(H, F);
  }
}

hipError_t launch_big_gemm_bf16(int mode, const RowGemmArgs& g, int max_rows, hipStream_t stream) {
  switch (mode) {
    case kGemmGateUp: return Big<kGemmGateUp>::launch(g, max_rows, stream);
    case kGemmDown: return Big<kGemmDown>::launch(g, max_rows, stream);
    case kGemmDA: return Big<kGemmDA>::launch(g, max_rows, stream);
    default: return Big<kGemmDX>::launch(g, max_rows, stream);
  }
}

}  // namespace moe
