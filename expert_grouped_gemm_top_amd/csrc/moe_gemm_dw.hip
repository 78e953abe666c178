// moe_gemm_dw.hip -- expert weight gradients in bf16 on the 32x32x16 matrix
// core (full fine-tuning: npu-train issue #14, section Scope), reduced over
// each expert's own ragged row count (LRMoE abstract):
//   [dW_gate | dW_up][e] (H x 2F) = x_rows^T [dHg | dHu]   over the rows of e
//   dW_down[e]           (F x H)  = a_rows^T dO_rows
//
// Workgroup = one BM x BN output tile of one expert, waves of 128 x 64.  Both
// operands are row-major over the reduced index (the expert's rows), so both
// land in LDS as [BK rows][tile columns] stages through direct global->LDS
// loads and both MFMA fragments come from the transposing LDS read.  Rows past
// the expert's last one are loaded from its last row and zeroed in LDS before
// use.  Every output is reduced in row order by one workgroup (deterministic,
// no atomics); an expert without rows stores exact zeros.
//
// Experts with at most one stage of rows (BK, empty ones included) are left to
// dw_small_bf16_kernel: their tiles are bound by their stores and by the
// workgroup's own latency, so they run on 128 x 128 tiles with 32 KiB of LDS,
// several workgroups per CU, instead of one 256 x 256 workgroup per CU.
//
// Work order: workgroups take experts in order of decreasing row count, so the
// longest reductions start first; the tiles of one expert are dealt to the 8
// XCDs in contiguous runs (tiles next to each other share an operand block,
// which then stays in that XCD's L2).  The output tile is staged through LDS
// so that every store is a full 16-byte lane of a contiguous row segment; the
// stores carry the non-temporal hint, since nothing in the step reads dW
// (measured: dW 615 -> 595 us at qwen3_ft_t4096, 684 -> 660 us at
// qwen3_compact_t16384).
#include <algorithm>
#include <type_traits>

#include "moe_common.h"
#include "moe_launch.h"
#include "moe_lds32.h"

namespace moe {

namespace {


template <int BN_, int WAVES_, int BK_, int STAGES_, int OCC_>
struct DwCfg {
  static constexpr int BM = 256, BN = BN_, BK = BK_, WAVES = WAVES_, STAGES = STAGES_, OCC = OCC_;
  static constexpr int WM = 2;                       // waves along the tile rows
  static constexpr int TM = BM / WM;                 // 128 tile rows per wave
  static constexpr int TN = BN / (WAVES / WM);       // tile columns per wave
  static constexpr int MI = TM / 32, NJ = TN / 32;
  static constexpr int PITCH_P = 2 * BM, PITCH_Q = 2 * BN;  // bytes per reduced row of a stage tile
  static constexpr int TILE_P = BK * PITCH_P, TILE_Q = BK * PITCH_Q;
  static constexpr int STAGE_BYTES = TILE_P + TILE_Q;
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
  static constexpr int INS_P = TILE_P / 1024 / WAVES, INS_Q = TILE_Q / 1024 / WAVES;  // direct loads per wave
  static constexpr int INS = INS_P + INS_Q;
  static_assert(TN == 64 && TM == 128, "waves of 128 x 64");
  static_assert(INS_P * 1024 * WAVES == TILE_P && INS_Q * 1024 * WAVES == TILE_Q, "loads cover the tiles");
  static_assert(STAGES >= 2 && STAGES <= 4 && 2 * INS < 64, "waits cover up to two stages issued ahead");
  static_assert(BM * BN * 2 <= LDS_BYTES, "the output tile fits the stage buffers");
  static_assert(64 * WAVES >= kMaxExperts, "every expert has a thread in the ranking");
};
using Cfg = DwCfg<256, 8, 64, 2, 1>;  // 256 x 256 tiles, 8 waves, 64-deep stages, 2 stages, 1 workgroup per CU
constexpr int kSmallMaxRows = Cfg::BK;  // experts with at most this many rows go to the small-expert kernel

struct DwShape {
  int nt1, tiles1;  // gate/up: column tiles, all tiles
  int nt2;          // down: column tiles
  int tiles;        // tiles per expert
};

__host__ __device__ inline DwShape dw_shape(int H, int F) {
  DwShape s;
  const int mt1 = (H + Cfg::BM - 1) / Cfg::BM;
  s.nt1 = (2 * F + Cfg::BN - 1) / Cfg::BN;
  s.tiles1 = mt1 * s.nt1;
  const int mt2 = (F + Cfg::BM - 1) / Cfg::BM;
  s.nt2 = (H + Cfg::BN - 1) / Cfg::BN;
  s.tiles = s.tiles1 + mt2 * s.nt2;
  return s;
}

// Workgroups per expert: the tiles rounded up to a multiple of the 8 XCDs.
__host__ __device__ inline int dw_slots(const DwShape& s) { return (s.tiles + 7) & ~7; }

// 16-byte direct loads of one operand's stage tile, `cpr` chunks per reduced
// row; LDS position p of row k holds the chunk p ^ nn_swz(k).  Row r of the
// expert is row row0 + r of the operand, or, with a row map, row
// map[row0 + r] / div (rows gathered on load).
template <int INS_N>
struct DwLoader {
  const uint16_t* col[INS_N];
  int krow[INS_N];
  __device__ void init(const uint16_t* base, int c0, int ncols, int cpr, int w, int l) {
#pragma unroll
    for (int i = 0; i < INS_N; ++i) {
      const int k = (64 / cpr) * (INS_N * w + i) + l / cpr;
      const int c = c0 + 8 * ((l % cpr) ^ nn_swz(k));
      krow[i] = k;
      col[i] = base + (c < ncols ? c : 0);  // chunks past the matrix edge read column 0 (never stored)
    }
  }
  __device__ void issue(int s, int row0, int n_e, int ld, unsigned char* tile, int w) const {
#pragma unroll
    for (int i = 0; i < INS_N; ++i) {
      int r = s * Cfg::BK + krow[i];
      r = r < n_e ? r : n_e - 1;  // past the expert's rows: its last row, zeroed before use
      g2lds(col[i] + (size_t)(row0 + r) * ld, tile + 1024 * (INS_N * w + i));
    }
  }
  // Mapped rows: the map entries of this lane's loads of stage s, read one
  // stage ahead of their use (ordinary loads that land while the previous
  // stage computes; nothing reads them before the next issue, which follows
  // the two-stage wait, so no wait is spent on them).
  __device__ void rows_of(int s, int row0, int n_e, const int32_t* map, int* pent) const {
#pragma unroll
    for (int i = 0; i < INS_N; ++i) {
      int r = s * Cfg::BK + krow[i];
      r = r < n_e ? r : n_e - 1;
      pent[i] = map[row0 + r];
    }
  }
  __device__ void issue_rows(const int* pent, int div, int ld, unsigned char* tile, int w) const {
#pragma unroll
    for (int i = 0; i < INS_N; ++i) g2lds(col[i] + (size_t)(pent[i] / div) * ld, tile + 1024 * (INS_N * w + i));
  }
};

__global__ __launch_bounds__(64 * Cfg::WAVES, Cfg::OCC) void dw_bf16_kernel(DwArgs g) {
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_rank[kMaxExperts];
  __shared__ int s_expert, s_nbig;
  extern __shared__ __attribute__((aligned(16))) unsigned char s_dyn[];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l32 = l & 31, hk = l >> 5;
  const int wm = w % Cfg::WM, wn = w / Cfg::WM;
  const int H = g.H, F = g.F, E = g.E;
  const DwShape sh = dw_shape(H, F);

  // ---- work item: expert rank and tile.  Workgroup b runs on XCD b % 8; the
  // j-th slot of XCD x within an expert's run of workgroups takes tile
  // x * slots / 8 + j.
  const int slots = dw_slots(sh);
  const int rank = blockIdx.x / slots, traw = blockIdx.x - rank * slots;
  const int t = (traw & 7) * (slots >> 3) + (traw >> 3);
  if (t >= sh.tiles) return;

  // ---- which expert has that rank in decreasing row count (ties: lower id
  // first).  Each expert's rank is summed from `parts` threads' partial counts.
  for (int i = tid; i <= E; i += 64 * Cfg::WAVES) s_off[i] = g.offsets[i];
  if (tid == 0) s_nbig = 0;
  __syncthreads();
  if (tid < E) {
    s_cnt[tid] = s_off[tid + 1] - s_off[tid];
    s_rank[tid] = 0;
    if (s_cnt[tid] > kSmallMaxRows) atomicAdd(&s_nbig, 1);
  }
  __syncthreads();
  // the experts ranked past the large ones are the small-expert kernel's
  if (rank >= s_nbig) return;
  {
    const int parts = (64 * Cfg::WAVES) / E;
    if (tid < parts * E) {
      const int ee = tid % E, part = tid / E;
      const int n = s_cnt[ee];
      const int lo = part * E / parts, hi = (part + 1) * E / parts;
      int r = 0;
      for (int e2 = lo; e2 < hi; ++e2) {
        const int n2 = s_cnt[e2];
        r += (n2 > n || (n2 == n && e2 < ee)) ? 1 : 0;
      }
      atomicAdd(&s_rank[ee], r);
    }
  }
  __syncthreads();
  if (tid < E && s_rank[tid] == rank) s_expert = tid;
  __syncthreads();
  const int e = s_expert;
  const int row0 = s_off[e], n_e = s_off[e + 1] - row0;

  // ---- the product this tile belongs to
  const uint16_t *P, *Q;
  const int32_t* pmap;  // gathered rows of the left operand, or NULL
  int ldp, ldq, M, N, mt, nt, pdiv;
  if (t < sh.tiles1) {  // [dW_gate | dW_up] = x^T [dHg | dHu]
    mt = t / sh.nt1;
    nt = t - mt * sh.nt1;
    P = g.x; ldp = H; M = H;
    pmap = g.x_map; pdiv = g.x_div;
    Q = g.dh; ldq = 2 * F; N = 2 * F;
  } else {              // dW_down = a^T dO
    const int tt = t - sh.tiles1;
    mt = tt / sh.nt2;
    nt = tt - mt * sh.nt2;
    P = g.a; ldp = F; M = F;
    pmap = g.a_map; pdiv = 1;
    Q = g.dO; ldq = H; N = H;
  }
  const int m0 = mt * Cfg::BM, n0 = nt * Cfg::BN;

  DwLoader<Cfg::INS_P> lp;
  DwLoader<Cfg::INS_Q> lq;
  lp.init(P, m0, M, Cfg::PITCH_P / 16, w, l);
  lq.init(Q, n0, N, Cfg::PITCH_Q / 16, w, l);
  static_assert(Cfg::STAGES == 2, "mapped rows are read one stage ahead, inside the two-stage wait");
  int pent[Cfg::INS_P];  // map entries of the next stage to issue
  // MAPPED is a compile-time switch so that the two pipelines are separate
  // loops: pending map loads of one never make the other wait
  auto issue = [&](int s, auto mapped) {
    unsigned char* st = s_dyn + (s % Cfg::STAGES) * Cfg::STAGE_BYTES;
    if constexpr (decltype(mapped)::value) {
      lp.issue_rows(pent, pdiv, ldp, st, w);
      if ((s + 1) * Cfg::BK < n_e) lp.rows_of(s + 1, row0, n_e, pmap, pent);
    } else {
      lp.issue(s, row0, n_e, ldp, st, w);
    }
    lq.issue(s, row0, n_e, ldq, st + Cfg::TILE_P, w);
  };

  f32x16 acc[Cfg::MI][Cfg::NJ];
#pragma unroll
  for (int i = 0; i < Cfg::MI; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  struct Frags {
    u32x4 a[Cfg::MI];
    u32x4 b[Cfg::NJ];
  };
  auto read_frags = [&](const unsigned char* st, int sub, Frags& fr) {
#pragma unroll
    for (int i = 0; i < Cfg::MI; ++i) fr.a[i] = tr_frag32(st, Cfg::PITCH_P, sub, Cfg::TM * wm + 32 * i);
#pragma unroll
    for (int j = 0; j < Cfg::NJ; ++j) fr.b[j] = tr_frag32(st + Cfg::TILE_P, Cfg::PITCH_Q, sub, Cfg::TN * wn + 32 * j);
  };
  auto mfmas = [&](const Frags& fr) {
#pragma unroll
    for (int j = 0; j < Cfg::NJ; ++j)
#pragma unroll
      for (int i = 0; i < Cfg::MI; ++i) acc[i][j] = mfma32(fr.b[j], fr.a[i], acc[i][j]);
  };
  // one sub-step's MFMAs with the next sub-step's fragment reads woven in
  auto mfmas_interleaved = [&](const Frags& cur, const unsigned char* st, int next_sub, Frags& nxt) {
    __builtin_amdgcn_s_setprio(1);
    if (next_sub >= 0) read_frags(st, next_sub, nxt);
    mfmas(cur);
#pragma unroll
    for (int q = 0; q < Cfg::MI * Cfg::NJ; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two LDS reads (one transposed fragment)
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto compute = [&](int s) {
    const unsigned char* st = s_dyn + (s % Cfg::STAGES) * Cfg::STAGE_BYTES;
    constexpr int SUBS = Cfg::BK / 16;
    Frags f0, f1;
    read_frags(st, 0, f0);
#pragma unroll
    for (int u = 0; u < SUBS; u += 2) {
      mfmas_interleaved(f0, st, u + 1 < SUBS ? u + 1 : -1, f1);
      if (u + 1 < SUBS) mfmas_interleaved(f1, st, u + 2 < SUBS ? u + 2 : -1, f0);
    }
  };

  const int steps = (n_e + Cfg::BK - 1) / Cfg::BK;
  auto pipeline = [&](auto mapped) {
    if constexpr (decltype(mapped)::value) lp.rows_of(0, row0, n_e, pmap, pent);
#pragma unroll
    for (int s = 0; s < Cfg::STAGES - 1; ++s)
      if (s < steps) issue(s, mapped);
    for (int s = 0; s < steps; ++s) {
      // stage s has landed once at most (stages issued after it) x INS loads remain
      const int ahead = min(Cfg::STAGES - 2, steps - 1 - s);
      if (ahead >= 2) wait_vmcnt<2 * Cfg::INS>();
      else if (ahead == 1) wait_vmcnt<Cfg::INS>();
      else wait_vmcnt<0>();
      barrier_no_fence();
      if (s + Cfg::STAGES - 1 < steps) issue(s + Cfg::STAGES - 1, mapped);
      const int valid = n_e - s * Cfg::BK;
      if (valid < Cfg::BK) {
        // last stage: zero the rows past the expert's end in both operand tiles
        unsigned char* st = s_dyn + (s % Cfg::STAGES) * Cfg::STAGE_BYTES;
        for (int c = tid; c < Cfg::STAGE_BYTES / 16; c += 64 * Cfg::WAVES) {
          const bool in_q = c >= Cfg::TILE_P / 16;
          const int rr = in_q ? (c - Cfg::TILE_P / 16) / (Cfg::PITCH_Q / 16) : c / (Cfg::PITCH_P / 16);
          if (rr >= valid) *(u32x4*)(st + 16 * c) = u32x4{0, 0, 0, 0};
        }
        __syncthreads();
      }
      compute(s);
    }
  };
  if (pmap != nullptr) pipeline(std::true_type{});
  else pipeline(std::false_type{});

  // ---- epilogue, staged through LDS.  acc[i][j] register r -> tile row
  // TM wm + 32 i + l32, tile column TN wn + 32 j + 8 q + 4 hk + (0..3) with
  // q = r / 4.  LDS row m holds the tile row, its 16-byte chunk c at position
  // c ^ (m % CPR).
  constexpr int CPR = Cfg::BN / 8;
  __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
  for (int i = 0; i < Cfg::MI; ++i) {
    const int m = Cfg::TM * wm + 32 * i + l32;
#pragma unroll
    for (int j = 0; j < Cfg::NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = (Cfg::TN * wn + 32 * j + 8 * q) >> 3;
        *(u32x2*)(s_dyn + m * (2 * Cfg::BN) + 16 * (c ^ (m % CPR)) + 8 * hk) =
            u32x2{pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]), pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
      }
  }
  __syncthreads();
  constexpr int kRowsPerWave = Cfg::BM / Cfg::WAVES, kRowsPerIns = 64 / CPR;
#pragma unroll
  for (int it = 0; it < kRowsPerWave / kRowsPerIns; ++it) {
    const int m = kRowsPerWave * w + kRowsPerIns * it + l / CPR, c = l % CPR;
    const int gm = m0 + m, gn = n0 + 8 * c;
    if (gm < M && gn < N) {
      const u32x4 v = *(const u32x4*)(s_dyn + m * (2 * Cfg::BN) + 16 * (c ^ (m % CPR)));
      uint16_t* dst;
      if (t < sh.tiles1) dst = (gn < F) ? g.dwg + ((size_t)e * H + gm) * F + gn : g.dwu + ((size_t)e * H + gm) * F + (gn - F);
      else dst = g.dwd + ((size_t)e * F + gm) * H + gn;
      __builtin_nontemporal_store(v, (u32x4*)dst);  // nothing in the step reads dW again
    }
  }
}

// ---- experts with at most one stage of rows ---------------------------------
// Workgroup = one 128 x 128 output tile of one such expert, four waves of
// 64 x 64 on the 32x32x16 matrix core; both operand blocks ([rows][128
// columns], 16 KiB each) come in with direct global->LDS loads and are read
// with the transposing LDS read, as in the large-expert kernel; only the
// 16-row sub-steps that hold rows of the expert are multiplied (the rows past
// its end within them are zeroed); an expert without rows stores zeros.  The
// output tile is staged through the operand buffers for full 16-byte row
// stores.  32 KiB of LDS lets several workgroups share a CU, so one tile's
// loads and stores overlap another's.  Work order: the j-th small expert (in
// id order) takes the j-th run of workgroups, each workgroup kSmallTpw
// consecutive tiles (one schedule for several tiles), the runs dealt to the 8
// XCDs in contiguous blocks like the large-expert kernel's tiles.
constexpr int kSmallBM = 128, kSmallBN = 128;
constexpr int kSmallPitch = 2 * kSmallBN;            // bytes per reduced row of either operand block
constexpr int kSmallTile = Cfg::BK * kSmallPitch;    // 16 KiB
constexpr int kSmallIns = kSmallTile / 1024 / 4;     // direct loads per wave per operand
constexpr int kSmallTpw = 4;          // consecutive tiles of one expert per workgroup

struct DwSmallShape {
  int nt1, tiles1;  // gate/up: column tiles, all tiles
  int nt2;          // down: column tiles
  int tiles;        // tiles per expert
};

// Tiles cover the outputs; the last row or column tile of a product is partial
// when H or F is not a multiple of 128 (its loads past the edge read column 0,
// its stores past the edge are skipped).
__host__ __device__ inline DwSmallShape dw_small_shape(int H, int F) {
  DwSmallShape s;
  s.nt1 = (2 * F + kSmallBN - 1) / kSmallBN;
  s.tiles1 = ((H + kSmallBM - 1) / kSmallBM) * s.nt1;
  s.nt2 = (H + kSmallBN - 1) / kSmallBN;
  s.tiles = s.tiles1 + ((F + kSmallBM - 1) / kSmallBM) * s.nt2;
  return s;
}

// Workgroups per expert: its tiles in runs of kSmallTpw, rounded up to a multiple of the 8 XCDs.
__host__ __device__ inline int dw_small_slots(const DwSmallShape& s) {
  return ((s.tiles + kSmallTpw - 1) / kSmallTpw + 7) & ~7;
}

__global__ __launch_bounds__(256, 3) void dw_small_bf16_kernel(DwArgs g) {
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_list[kMaxExperts];
  __shared__ int s_tmp[4];
  __shared__ __attribute__((aligned(16))) unsigned char s_t[2 * kSmallTile];  // P | Q, then the output tile
  static_assert(kSmallBM * kSmallBN * 2 == 2 * kSmallTile, "the output tile fills the operand buffers");
  static_assert(kSmallIns * 1024 * 4 == kSmallTile && 64 / (kSmallPitch / 16) * kSmallIns * 4 == Cfg::BK,
                "four waves load the BK rows of a block");
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, l32 = l & 31, hk = l >> 5;
  const int wm = w & 1, wn = w >> 1;
  const int H = g.H, F = g.F, E = g.E;
  const DwSmallShape sh = dw_small_shape(H, F);
  const int slots = dw_small_slots(sh);
  const int unit = blockIdx.x / slots, traw = blockIdx.x - unit * slots;
  const int t_first = ((traw & 7) * (slots >> 3) + (traw >> 3)) * kSmallTpw;
  if (t_first >= sh.tiles) return;  // uniform across the workgroup
  const int t_end = min(t_first + kSmallTpw, sh.tiles);

  // the small experts in id order
  for (int i = tid; i <= E; i += 256) s_off[i] = g.offsets[i];
  __syncthreads();
  const int small = (tid < E && s_off[tid + 1] - s_off[tid] <= kSmallMaxRows) ? 1 : 0;
  int n_small;
  const int pos = block256_exclusive_scan(small, s_tmp, n_small);
  if (small) s_list[pos] = tid;
  __syncthreads();
  if (unit >= n_small) return;
  const int e = s_list[unit];
  const int row0 = s_off[e], n_e = s_off[e + 1] - row0;

  for (int t = t_first; t < t_end; ++t) {
    // the product this tile belongs to
    const uint16_t *P, *Q;
    const int32_t* pmap;
    int ldp, ldq, M, N, mt, nt, pdiv;
    if (t < sh.tiles1) {  // [dW_gate | dW_up] = x^T [dHg | dHu]
      mt = t / sh.nt1;
      nt = t - mt * sh.nt1;
      P = g.x; ldp = H; M = H;
      pmap = g.x_map; pdiv = g.x_div;
      Q = g.dh; ldq = 2 * F; N = 2 * F;
    } else {              // dW_down = a^T dO
      const int tt = t - sh.tiles1;
      mt = tt / sh.nt2;
      nt = tt - mt * sh.nt2;
      P = g.a; ldp = F; M = F;
      pmap = g.a_map; pdiv = 1;
      Q = g.dO; ldq = H; N = H;
    }
    const int m0 = mt * kSmallBM, n0 = nt * kSmallBN;

    f32x16 acc[2][2];
  #pragma unroll
    for (int i = 0; i < 2; ++i)
  #pragma unroll
      for (int j = 0; j < 2; ++j)
  #pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    if (n_e > 0) {
      DwLoader<kSmallIns> lp, lq;
      lp.init(P, m0, M, kSmallPitch / 16, w, l);
      lq.init(Q, n0, N, kSmallPitch / 16, w, l);
      if (pmap != nullptr) {
        int pent[kSmallIns];
        lp.rows_of(0, row0, n_e, pmap, pent);
        lp.issue_rows(pent, pdiv, ldp, s_t, w);
      } else {
        lp.issue(0, row0, n_e, ldp, s_t, w);
      }
      lq.issue(0, row0, n_e, ldq, s_t + kSmallTile, w);
      wait_vmcnt<0>();
      barrier_no_fence();
      const int used = (n_e + 15) & ~15;  // rows of the sub-steps that hold rows of the expert
      if (n_e < used) {
        for (int c = tid; c < 2 * kSmallTile / 16; c += 256) {
          const int rr = (c & (kSmallTile / 16 - 1)) / (kSmallPitch / 16);
          if (rr >= n_e && rr < used) *(u32x4*)(s_t + 16 * c) = u32x4{0, 0, 0, 0};
        }
        __syncthreads();
      }
      for (int sub = 0; sub < used / 16; ++sub) {
        u32x4 fa[2], fb[2];
  #pragma unroll
        for (int i = 0; i < 2; ++i) fa[i] = tr_frag32(s_t, kSmallPitch, sub, 64 * wm + 32 * i);
  #pragma unroll
        for (int j = 0; j < 2; ++j) fb[j] = tr_frag32(s_t + kSmallTile, kSmallPitch, sub, 64 * wn + 32 * j);
  #pragma unroll
        for (int j = 0; j < 2; ++j)
  #pragma unroll
          for (int i = 0; i < 2; ++i) acc[i][j] = mfma32(fb[j], fa[i], acc[i][j]);
      }
    }

    // epilogue, staged through the operand buffers.  acc[i][j] register r ->
    // tile row 64 wm + 32 i + l32, tile column 64 wn + 32 j + 8 q + 4 hk +
    // (0..3), q = r / 4; LDS row m holds the tile row, its 16-byte chunk c at
    // position c ^ (m % 16).
    __syncthreads();  // every wave is done with the operand blocks
  #pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = 64 * wm + 32 * i + l32;
  #pragma unroll
      for (int j = 0; j < 2; ++j)
  #pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = (64 * wn + 32 * j + 8 * q) >> 3;
          *(u32x2*)(s_t + m * kSmallPitch + 16 * (c ^ (m & 15)) + 8 * hk) =
              u32x2{pack_bf2(acc[i][j][4 * q], acc[i][j][4 * q + 1]), pack_bf2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
        }
    }
    __syncthreads();
  #pragma unroll
    for (int it = 0; it < 8; ++it) {  // a wave stores 32 rows, 4 per instruction
      const int m = 32 * w + 4 * it + (l >> 4), c = l & 15;
      const int gm = m0 + m, gn = n0 + 8 * c;
      if (gm < M && gn < N) {
        const u32x4 v = *(const u32x4*)(s_t + m * kSmallPitch + 16 * (c ^ (m & 15)));
        uint16_t* dst;
        if (t < sh.tiles1) dst = (gn < F) ? g.dwg + ((size_t)e * H + gm) * F + gn : g.dwu + ((size_t)e * H + gm) * F + (gn - F);
        else dst = g.dwd + ((size_t)e * F + gm) * H + gn;
        __builtin_nontemporal_store(v, (u32x4*)dst);  // nothing in the step reads dW again
      }
    }
    __syncthreads();  // the next tile's loads overwrite the staged tile
  }
}

}  // namespace

hipError_t launch_dw_bf16(const DwArgs& g, hipStream_t stream) {
  // experts with at most one stage of rows (empty ones included)
  const DwSmallShape ss = dw_small_shape(g.H, g.F);
  const int64_t sblocks = (int64_t)g.E * dw_small_slots(ss);
  MOE_LAUNCH(dw_small_bf16_kernel, dim3((unsigned)sblocks), dim3(256), 0, stream, g);
  hipError_t serr = hipGetLastError();
  if (serr != hipSuccess) return serr;
  // the others
  const DwShape sh = dw_shape(g.H, g.F);
  const int64_t blocks = (int64_t)g.E * dw_slots(sh);
  const size_t lds = (size_t)Cfg::LDS_BYTES;
  // dynamic LDS above 64 KiB must be allowed explicitly, once per device
  static PerDeviceOnce lds_once;
  hipError_t err = allow_dynamic_lds(lds_once, (const void*)dw_bf16_kernel, lds);
  if (err != hipSuccess) return err;
  MOE_LAUNCH(dw_bf16_kernel, dim3((unsigned)blocks), dim3(64 * Cfg::WAVES), lds, stream, g);
  return hipGetLastError();
}

}  // namespace moe
