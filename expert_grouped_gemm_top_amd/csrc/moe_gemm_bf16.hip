// moe_gemm_bf16.hip -- ragged grouped GEMMs of the SwiGLU experts in bf16 on
// gfx950 matrix cores (v_mfma_f32_16x16x32_bf16, fp32 accumulate): the
// skinny-expert and mid-size regimes of the row GEMMs.
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
// One launch covers two regimes, both scheduled on the device from the
// offsets (build_tile_starts / lookup_tile):
//   * experts with fewer than 32 rows: every wave streams one 16-row tile x one
//     column block straight from memory (the weights are the traffic), with
//     an optional split of K between waves of a workgroup;
//   * experts with 32 .. big_min_rows rows: 128 x 128 workgroup tiles staged
//     through double-buffered, swizzled LDS.
// Experts with more rows run in the 256-row kernel of moe_gemm_big.hip.
// In every case the MFMA takes the weights as its first operand, so a lane
// ends up holding one output row and contiguous columns, and the epilogue
// (SwiGLU forward or backward) is applied from registers.

#include <algorithm>

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {

namespace {

// Reduction split of the skinny-expert kernel per product, 4 bits each
// (GATEUP, DOWN, DA, DX from the low end): 1, 2 or 4 waves per column block
// (measured: gate/up and dA gain from 2, down and dX from none).
constexpr int kStreamSplitK = 0x1212;

constexpr int kFewRows = 128;  // below this many rows in all, the streaming kernel splits K four ways
                               // and reads its weights with ordinary (temporal) loads
constexpr int kTileRows = 16;  // rows of one expert per wave tile of the streaming kernel (one MFMA row block)
constexpr int kBigRows = kMidTileMinRows;  // experts with at least this many rows use an LDS-tiled kernel
constexpr int kTBM = 128;      // LDS-tiled kernel: rows per workgroup tile
constexpr int kTBN = 128;      //   output columns per workgroup tile
constexpr int kTBK = 64;       //   reduction depth per stage
constexpr int kTPitch = kTBK;  // LDS row pitch (elements); 16-byte chunks XOR-swizzled by row & 7

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

// 8 fp8 (E4M3) weights -> 8 bf16, exactly (an E4M3 value has at most 4
// significant bits): the hardware conversion to fp32, then the upper half of
// each fp32.  Element order is kept: byte b of the input is element b.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 fp8x8_to_bf16(u32x2 q) {
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[h], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q[h], true);
    r[2 * h] = __builtin_amdgcn_perm(__float_as_uint(lo.y), __float_as_uint(lo.x), 0x07060302u);
    r[2 * h + 1] = __builtin_amdgcn_perm(__float_as_uint(hi.y), __float_as_uint(hi.x), 0x07060302u);
  }
  return r;
}

// Weight element and 8-element load of the streaming kernel: bf16, or fp8
// bytes widened to bf16 just before use.
template <bool W8>
struct WeightFmt {
  using Elem = uint16_t;
  using Vec = u32x4;
  static __device__ __forceinline__ u32x4 widen(u32x4 v) { return v; }
};
template <>
struct WeightFmt<true> {
  using Elem = uint8_t;
  using Vec = u32x2;
  static __device__ __forceinline__ u32x4 widen(u32x2 v) { return fp8x8_to_bf16(v); }
};

// Weight load of the streaming kernel.  Each weight is read once per call,
// so with NONTEMP the load carries the non-temporal hint: the weight stream
// then keeps out of the caches' way (measured at the LoRA shape: gate/up
// 149 -> 137 us, dX 144 -> 136 us, the step 0.47 -> 0.44 ms, also with the
// caches flushed between steps).  Decode-sized batches (fewer than kFewRows
// rows, a few thousand waves in flight) measured slower with it (gate/up
// 65 -> 73 us) and keep ordinary loads.
template <bool NONTEMP, typename T>
__device__ __forceinline__ T load_weights(const T* p) {
  if constexpr (NONTEMP) return __builtin_nontemporal_load(p);
  else return *p;
}

// ---- row GEMMs --------------------------------------------------------------
// N-contiguous weights (GATEUP, DOWN): a wave covers 128 output columns; per
// K-step of 32 a lane loads 8 rows x 16 B, so one load instruction reads 4 rows
// x 256 contiguous bytes.  K-contiguous weights (DA, DX): a wave covers 64
// output columns; per K-stage of 128 one load instruction again reads 4 rows x
// 256 contiguous bytes, and the stage is turned into MFMA fragments through
// LDS.
template <int MODE>
struct RowGemmShape;
template <>
struct RowGemmShape<kGemmGateUp> { static constexpr bool kNN = true; };
template <>
struct RowGemmShape<kGemmDown> { static constexpr bool kNN = true; };
template <>
struct RowGemmShape<kGemmDA> { static constexpr bool kNN = false; };
template <>
struct RowGemmShape<kGemmDX> { static constexpr bool kNN = false; };

template <int MODE>
__host__ __device__ constexpr int row_gemm_cols() { return RowGemmShape<MODE>::kNN ? 128 : 64; }

// column blocks of one expert tile (the last one partial when the output width
// is not a multiple of the block; its columns past the edge are never stored)
template <int MODE>
__host__ __device__ inline int row_gemm_blocks(int H, int F) {
  return MODE == kGemmGateUp ? (F + 63) / 64
                             : (MODE == kGemmDown ? (H + 127) / 128 : (MODE == kGemmDA ? (F + 63) / 64 : (H + 63) / 64));
}

// Column blocks of the streaming kernel.  With fp8 weights the gate/up wave
// covers 128 features of both matrices (its loads then read 128-byte runs of
// each weight row; 64 features per wave left 64-byte runs, which read
// memory at 4.5 TB/s where 128-byte runs read 6.2).
template <int MODE, bool W8>
__host__ __device__ inline int stream_blocks(int H, int F) {
  return (W8 && MODE == kGemmGateUp) ? (F + 127) / 128 : row_gemm_blocks<MODE>(H, F);
}

// Output columns of a row GEMM (gate/up: features, each a gate and an up column).
template <int MODE>
__host__ __device__ inline int row_gemm_cols(int H, int F) {
  return (MODE == kGemmGateUp || MODE == kGemmDA) ? F : H;
}

// Per-wave tile schedule of the row GEMMs (the streaming kernel and the
// 128-row tiles): the same tile prefix as
// build_tile_starts / lookup_tile (experts with min_rows <= n_e < max_rows,
// ceil(n_e / tile_rows) tiles each, in expert order), derived by every wave
// on its own from offsets[0..E] with a wave scan and a ballot: no LDS and no
// workgroup barrier before the first weight loads.  Lane l covers experts
// 4 l .. 4 l + 3 (E <= 256).
struct WaveTiles {
  int off[5];   // offsets[4 l .. 4 l + 4], clamped at E
  int cnt[4];   // tiles of those experts
  int excl;     // tiles of the experts before 4 l
  int total;    // tiles of all experts
};

__device__ __forceinline__ WaveTiles wave_tile_prefix(const int32_t* __restrict__ offsets, int E, int tile_rows,
                                                      int min_rows, int max_rows) {
  WaveTiles t;
  const int l = __lane_id();
#pragma unroll
  for (int i = 0; i < 5; ++i) t.off[i] = offsets[min(4 * l + i, E)];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int n = t.off[i + 1] - t.off[i];  // 0 past E (both ends clamped)
    t.cnt[i] = (n >= min_rows && n < max_rows) ? (n + tile_rows - 1) / tile_rows : 0;
    sum += t.cnt[i];
  }
  const int inc = wave_inclusive_scan(sum);
  t.excl = inc - sum;
  t.total = __shfl(inc, kWave - 1, kWave);
  return t;
}

// The slot of a wave-uniform tile id (expert -1 past the last tile).
__device__ __forceinline__ TileSlot wave_lookup_tile(const WaveTiles& t, int tile_rows, int tile_id) {
  TileSlot s;
  const int l = __lane_id();
  int start = t.excl, ex = -1, tl = 0, rb = 0, nr = 0, ne = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (tile_id >= start && tile_id < start + t.cnt[i]) {
      ex = 4 * l + i;
      tl = tile_id - start;
      ne = t.off[i + 1] - t.off[i];
      rb = t.off[i] + tl * tile_rows;
      nr = min(t.off[i + 1] - rb, tile_rows);
    }
    start += t.cnt[i];
  }
  const uint64_t hit = __ballot(ex >= 0);
  if (hit == 0) {
    s.expert = -1;
    s.tile = s.row_begin = s.rows = s.expert_rows = 0;
    return s;
  }
  const int src = __ffsll((unsigned long long)hit) - 1;  // the one lane whose range holds tile_id
  s.expert = __shfl(ex, src, kWave);
  s.tile = __shfl(tl, src, kWave);
  s.row_begin = __shfl(rb, src, kWave);
  s.rows = __shfl(nr, src, kWave);
  s.expert_rows = __shfl(ne, src, kWave);
  return s;
}

//
// With a reduction split of S = 2 or 4 (g.stream_ksplit), a workgroup takes
// 4 / S adjacent column blocks of one tile and each block's reduction is cut
// into S parts run by S waves; the partial sums of parts 1.. are added to part
// 0's through LDS in part order.  That multiplies the waves streaming weights
// when there are too few tiles to fill the chip.
//
// W8: the weights are fp8 (E4M3) bytes, widened to bf16 in registers right
// before the MFMA, and the products of expert e are scaled by g.wscale[e]; the
// kernel then takes every expert, whatever its row count.
// NONTEMP: weight loads with the non-temporal hint (load_weights).
template <int MODE, bool W8, bool NONTEMP>
__device__ __forceinline__ void stream_gemm(const RowGemmArgs& g, int wg, unsigned char* lds) {
  constexpr bool NN = RowGemmShape<MODE>::kNN;
  using WF = WeightFmt<W8>;
  using WE = typename WF::Elem;
  using WV = typename WF::Vec;
  const WaveTiles wt = wave_tile_prefix(g.offsets, g.E, kTileRows, 0, W8 ? kNoBigTiles : kBigRows);

  const int H = g.H, F = g.F;
  // fp8 gate/up: a wave takes 128 features, MFMAs 0..7 on W_gate, 8..15 on W_up
  constexpr bool WIDE = W8 && MODE == kGemmGateUp;
  constexpr int NACC = WIDE ? 16 : (NN ? 8 : 4);  // accumulators in use
  const int nblk = stream_blocks<MODE, W8>(H, F);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, c = l & 15, gq = l >> 4;
  const int ks = g.stream_ksplit;  // 1, 2 or 4
  const bool split = ks > 1;
  const int cpw = 4 / ks;  // column blocks per workgroup
  // work item of this wave: (tile, column block); the waves of a workgroup take
  // adjacent column blocks of the same tile (when split, nblk is a multiple of
  // cpw, so all blocks of a workgroup fall on one tile).  Workgroups are taken
  // in XCD order, so a tile's activation rows are fetched into one L2.
  const int real_wgs = (wt.total * nblk + cpw - 1) / cpw;
  const int item = xcd_item(wg, real_wgs) * cpw + (w % cpw);
  const int kpart = w / cpw;
  const TileSlot ts = wave_lookup_tile(wt, kTileRows, item / nblk);
  // uniform across the wave, and across the workgroup when split (before its barrier)
  if (ts.expert < 0) return;
  const int nb = item % nblk;
  const int e = ts.expert;
  const int K = (MODE == kGemmGateUp || MODE == kGemmDA) ? H : (MODE == kGemmDown ? F : 2 * F);
  const int Kp = K / ks;  // reduction length of this wave, from k_begin
  const int k_begin = kpart * Kp;

  const bool a_ok = c < ts.rows;
  const uint16_t* __restrict__ A = (const uint16_t*)g.a;
  // rows past the tile read the tile's last row (always valid) and are zeroed at use
  const uint16_t* a_row = A + a_row_of(g, ts.row_begin + (a_ok ? c : ts.rows - 1)) * K + k_begin;

  f32x4 acc[WIDE ? 16 : 8];
#pragma unroll
  for (int j = 0; j < (WIDE ? 16 : 8); ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero4 = {0u, 0u, 0u, 0u};

  if constexpr (WIDE) {
    // lane c reads 8 features f = 128 nb + 8 c of W_gate and of W_up at rows
    // k0 + 8 gq + (0..7): 16 lanes read 128 contiguous bytes of one weight row
    // (features past the edge read feature 0: never stored)
    const int f = nb * 128 + 8 * c;
    const size_t wofs = (size_t)e * H * F + (f < F ? f : 0) + (size_t)k_begin * F;
    const WE* g_first = (const WE*)g.w0 + wofs;
    const WE* u_first = (const WE*)g.w1 + wofs;
    const uint16_t* a_ptr = a_row + 8 * gq;
    const int steps = (Kp + 31) / 32, last = steps - 1;
    auto load = [&](int s, WV* bq, u32x4& aq) {
      const bool kin = s * 32 + 8 * gq < Kp;
      const size_t ofs = kin ? (size_t)(s * 32 + 8 * gq) * F : 0;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        bq[r] = load_weights<NONTEMP>((const WV*)(g_first + ofs + (size_t)r * F));
        bq[8 + r] = load_weights<NONTEMP>((const WV*)(u_first + ofs + (size_t)r * F));
      }
      aq = *(const u32x4*)(kin ? a_ptr + (size_t)s * 32 : zero_chunk());
    };
    auto compute = [&](const WV* bq, const u32x4& aq) {
      const u32x4 av = a_ok ? aq : zero4;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        u32x4 bw[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) bw[r] = WF::widen(bq[8 * m + r]);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc[8 * m + jj] = mfma_bf16(column_of_8x8(bw, jj), av, acc[8 * m + jj]);
      }
    };
    WV b0[16], b1[16], b2[16];
    u32x4 a0, a1, a2;
    load(0, b0, a0);
    load(min(1, last), b1, a1);
    for (int s = 0; s < steps; s += 3) {
      load(min(s + 2, last), b2, a2);
      __builtin_amdgcn_sched_barrier(0);
      compute(b0, a0);
      __builtin_amdgcn_sched_barrier(0);
      load(min(s + 3, last), b0, a0);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < steps) compute(b1, a1);
      __builtin_amdgcn_sched_barrier(0);
      load(min(s + 4, last), b1, a1);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 2 < steps) compute(b2, a2);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (NN) {
    // B operand: lane c reads columns [col, col+8) of rows k0 + 8gq + (0..7)
    // (columns past the output edge read column 0: never stored)
    const WE* b_ptr;
    size_t ldb;
    if (MODE == kGemmGateUp) {
      // even lanes read W_gate, odd lanes W_up, at the same 8 features f
      const WE* W = (const WE*)((c & 1) ? g.w1 : g.w0);
      const int f = nb * 64 + 8 * (c >> 1);
      b_ptr = W + (size_t)e * H * F + (f < F ? f : 0);
      ldb = F;
    } else {
      const int col = nb * 128 + 8 * c;
      b_ptr = (const WE*)g.w0 + (size_t)e * F * H + (col < H ? col : 0);
      ldb = H;
    }
    const WE* b_first = b_ptr + (size_t)k_begin * ldb;  // rows k_begin .. k_begin + 7 (Kp >= 8)
    b_ptr = b_first + (size_t)(8 * gq) * ldb;
    const uint16_t* a_ptr = a_row + 8 * gq;
    // the last step may run past Kp (Kp a multiple of 8, not of 32): a lane
    // whose 8 k of that step lie past it reads the first 8 weight rows and a
    // zero activation chunk, so they add nothing
    const int steps = (Kp + 31) / 32, last = steps - 1;
    auto load = [&](int s, WV* bq, u32x4& aq) {
      const bool kin = s * 32 + 8 * gq < Kp;
      const WE* bp = kin ? b_ptr + (size_t)s * 32 * ldb : b_first;
#pragma unroll
      for (int r = 0; r < 8; ++r) bq[r] = load_weights<NONTEMP>((const WV*)(bp + (size_t)r * ldb));
      aq = *(const u32x4*)(kin ? a_ptr + (size_t)s * 32 : zero_chunk());
    };
    auto compute = [&](const WV* bq, const u32x4& aq) {
      const u32x4 av = a_ok ? aq : zero4;
      u32x4 bw[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) bw[r] = WF::widen(bq[r]);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) acc[jj] = mfma_bf16(column_of_8x8(bw, jj), av, acc[jj]);
    };
    WV b0[8], b1[8], b2[8];
    u32x4 a0, a1, a2;
    load(0, b0, a0);
    load(min(1, last), b1, a1);
    for (int s = 0; s < steps; s += 3) {
      load(min(s + 2, last), b2, a2);
      __builtin_amdgcn_sched_barrier(0);
      compute(b0, a0);
      __builtin_amdgcn_sched_barrier(0);
      load(min(s + 3, last), b0, a0);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < steps) compute(b1, a1);
      __builtin_amdgcn_sched_barrier(0);
      load(min(s + 4, last), b1, a1);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 2 < steps) compute(b2, a2);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // K-contiguous weights, stage = 64 weight rows x 128 k.  One load
    // instruction reads 4 rows x 256 contiguous bytes (16 lanes per row); the
    // stage goes through this wave's 16 KiB of LDS (16-byte chunks XOR-swizzled
    // by row & 15) and comes back as MFMA fragments: lane (c, gq) takes weight
    // rows c + 16 jj, k chunks 4 gq + q, matching its activation chunks.
    // Lanes read chunks other lanes wrote: the LDS operations of one wave
    // complete in order, so a wave barrier with a wavefront-scope fence (which
    // emits no instruction) after the stage's writes, and again before the
    // next stage overwrites it, is all the ordering needed; it keeps the
    // compiler from moving a read above the writes or a write above the reads.
    const int lrow = l >> 4, lchunk = l & 15;
    const WE* w_lo;  // rows for k in [0, Kw)
    const WE* w_hi;  // DX only: rows for k in [F, 2F)
    size_t ldw;
    int Kw;
    const int Nw = MODE == kGemmDA ? F : H;  // weight rows (output columns)
    if (MODE == kGemmDA) {
      w_lo = (const WE*)g.w0 + (size_t)e * F * H;
      w_hi = w_lo;
      ldw = H;
      Kw = K;
    } else {
      w_lo = (const WE*)g.w0 + (size_t)e * H * F;
      w_hi = (const WE*)g.w1 + (size_t)e * H * F;
      ldw = F;
      Kw = F;
    }
    unsigned char* xs = lds + w * 16384;
    const uint16_t* a_ptr = a_row + 32 * gq;
    // The last stage may run past Kp (a multiple of 8, not of 128): this lane's
    // chunk (8 k) past the end reads columns 0..7 of the weights and the
    // activation chunks past it read zeros.  Weight rows past the output edge read row 0
    // (never stored).  A chunk never straddles Kw (F is a multiple of 8).
    const int stages = (Kp + 127) / 128, last = stages - 1;
    const int row0 = nb * 64 + lrow;
    auto load = [&](int s, WV* bq, u32x4* aq) {
      const int k = k_begin + s * 128 + 8 * lchunk;  // this lane's weight chunk
      const WE* wp = (k < Kw) ? w_lo + k : (k < K ? w_hi + (k - Kw) : w_lo);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int n = row0 + 4 * i;
        bq[i] = load_weights<NONTEMP>((const WV*)(wp + (size_t)(n < Nw ? n : 0) * ldw));
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ka = s * 128 + 32 * gq + 8 * q;
        aq[q] = *(const u32x4*)(ka < Kp ? a_ptr + (size_t)s * 128 + 8 * q : zero_chunk());
      }
    };
    auto wave_sync = [] {
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    };
    auto compute = [&](const WV* bq, const u32x4* aq) {
      wave_sync();  // the previous stage's reads before these writes
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 4 * i + lrow;
        *(u32x4*)(xs + row * 256 + 16 * (lchunk ^ (row & 15))) = WF::widen(bq[i]);
      }
      wave_sync();  // every lane's writes before any lane's reads
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 av = a_ok ? aq[q] : zero4;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const u32x4 bv = *(const u32x4*)(xs + (c + 16 * jj) * 256 + 16 * ((4 * gq + q) ^ c));
          acc[jj] = mfma_bf16(bv, av, acc[jj]);
        }
      }
    };
    WV b0[16], b1[16];
    u32x4 a0[4], a1[4];
    load(0, b0, a0);
    for (int s = 0; s < stages; s += 2) {
      load(min(s + 1, last), b1, a1);
      __builtin_amdgcn_sched_barrier(0);
      compute(b0, a0);
      __builtin_amdgcn_sched_barrier(0);
      load(min(s + 2, last), b0, a0);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < stages) compute(b1, a1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (split) {
    // parts 1.. -> each into its own wave's LDS area (for K-contiguous weights
    // the one only it has used for its stages); part 0 adds them in part order
    // a wave's partials go to its own area: 8 KiB (N-contiguous weights use no
    // other LDS here; 16 KiB for the fp8 gate/up wave) or the 16 KiB of its
    // K-contiguous stages
    constexpr int kRedBytes = NN ? NACC * kWave * 16 : 16384;
    if (kpart > 0) {
      f32x4* red = reinterpret_cast<f32x4*>(lds + w * kRedBytes);
#pragma unroll
      for (int j = 0; j < NACC; ++j) red[j * kWave + l] = acc[j];
    }
    __syncthreads();
    if (kpart > 0) return;
    for (int p = 1; p < ks; ++p) {
      const f32x4* red = reinterpret_cast<const f32x4*>(lds + (w + p * cpw) * kRedBytes);
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j] = acc[j] + red[j * kWave + l];
    }
  }

  if constexpr (W8) {  // the weights' scale: a power of two, so the product is exact
    const float sc = g.wscale[e];
#pragma unroll
    for (int j = 0; j < NACC; ++j) acc[j] = acc[j] * sc;
  }

  // epilogue straight from registers: lane (c, gq) owns tile row c
  if (!a_ok) return;
  const size_t grow = (size_t)ts.row_begin + c;
  if constexpr (WIDE) {
    // MFMA jj (W_gate) and 8 + jj (W_up), register r: feature
    // f = 128 nb + 32 gq + 8 r + jj
    uint16_t* hrow = g.out0 + grow * 2 * F;
    uint16_t* arow = g.out1 + grow * F;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int f = nb * 128 + 32 * gq + 8 * r;
      if (f >= F) break;  // features past the edge
      float G[8], U[8], V[8];
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        G[jj] = acc[jj][r];
        U[jj] = acc[8 + jj][r];
        V[jj] = G[jj] * sigmoidf_fast(G[jj]) * U[jj];
      }
      if (g.out0 != nullptr) {
        *(u32x4*)(hrow + f) = u32x4{pack_bf2(G[0], G[1]), pack_bf2(G[2], G[3]), pack_bf2(G[4], G[5]), pack_bf2(G[6], G[7])};
        *(u32x4*)(hrow + F + f) =
            u32x4{pack_bf2(U[0], U[1]), pack_bf2(U[2], U[3]), pack_bf2(U[4], U[5]), pack_bf2(U[6], U[7])};
      }
      if (g.out1 != nullptr)
        *(u32x4*)(arow + f) = u32x4{pack_bf2(V[0], V[1]), pack_bf2(V[2], V[3]), pack_bf2(V[4], V[5]), pack_bf2(V[6], V[7])};
    }
  } else if (MODE == kGemmGateUp) {
    // MFMA jj, register r: gate (r even) / up (r odd) of feature
    // f = 64 nb + 16 gq + 8 (r >> 1) + jj
    float hg[16], hu[16], av[16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        hg[8 * h + jj] = acc[jj][2 * h];
        hu[8 * h + jj] = acc[jj][2 * h + 1];
      }
#pragma unroll
    for (int i = 0; i < 16; ++i) av[i] = hg[i] * sigmoidf_fast(hg[i]) * hu[i];
    const int f = nb * 64 + 16 * gq;
    uint16_t* hrow = g.out0 + grow * 2 * F;
    uint16_t* arow = g.out1 + grow * F;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (f + 8 * h >= F) break;  // features past the edge
      const float* G = hg + 8 * h;
      const float* U = hu + 8 * h;
      const float* V = av + 8 * h;
      if (g.out0 != nullptr) {
        *(u32x4*)(hrow + f + 8 * h) =
            u32x4{pack_bf2(G[0], G[1]), pack_bf2(G[2], G[3]), pack_bf2(G[4], G[5]), pack_bf2(G[6], G[7])};
        *(u32x4*)(hrow + F + f + 8 * h) =
            u32x4{pack_bf2(U[0], U[1]), pack_bf2(U[2], U[3]), pack_bf2(U[4], U[5]), pack_bf2(U[6], U[7])};
      }
      if (g.out1 != nullptr)
        *(u32x4*)(arow + f + 8 * h) =
            u32x4{pack_bf2(V[0], V[1]), pack_bf2(V[2], V[3]), pack_bf2(V[4], V[5]), pack_bf2(V[6], V[7])};
    }
  } else if (MODE == kGemmDown) {
    // MFMA jj, register r: column 128 nb + 32 gq + 8 r + jj
    const int col0 = nb * 128 + 32 * gq;
    uint16_t* orow = g.out0 + grow * H + col0;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (col0 + 8 * r < H)
        *(u32x4*)(orow + 8 * r) = u32x4{pack_bf2(acc[0][r], acc[1][r]), pack_bf2(acc[2][r], acc[3][r]),
                                        pack_bf2(acc[4][r], acc[5][r]), pack_bf2(acc[6][r], acc[7][r])};
  } else {
    // MFMA jj, register r: column 64 nb + 16 jj + 4 gq + r
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int col = nb * 64 + 16 * jj + 4 * gq;
      if (col >= row_gemm_cols<MODE>(H, F)) continue;  // past the edge (4 columns, all or none)
      if (MODE == kGemmDA) {
        // SwiGLU backward with the saved pre-activations hg, hu
        const uint16_t* hrow = g.h + h_row_of(g, grow) * 2 * F;
        const u32x2 gw = *(const u32x2*)(hrow + col), uw = *(const u32x2*)(hrow + F + col);
        float dg[4], du[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float hgv = (r & 1) ? bf_hi(gw[r >> 1]) : bf_lo(gw[r >> 1]);
          const float huv = (r & 1) ? bf_hi(uw[r >> 1]) : bf_lo(uw[r >> 1]);
          const float sg = sigmoidf_fast(hgv);
          dg[r] = acc[jj][r] * huv * sg * (1.0f + hgv * (1.0f - sg));
          du[r] = acc[jj][r] * hgv * sg;
        }
        uint16_t* drow = g.out0 + grow * 2 * F;
        *(u32x2*)(drow + col) = u32x2{pack_bf2(dg[0], dg[1]), pack_bf2(dg[2], dg[3])};
        *(u32x2*)(drow + F + col) = u32x2{pack_bf2(du[0], du[1]), pack_bf2(du[2], du[3])};
      } else {
        *(u32x2*)(g.out0 + grow * H + col) =
            u32x2{pack_bf2(acc[jj][0], acc[jj][1]), pack_bf2(acc[jj][2], acc[jj][3])};
      }
    }
  }
}

// ---- LDS-tiled row GEMM for experts with many rows ---------------------------
// Workgroup tile: 128 rows of one expert x 128 output columns, four waves as
// 2 x 2 of 64 x 64; the reduction advances 64 at a time through double-buffered
// LDS tiles, so each weight tile read from memory serves 128 rows and each row
// tile serves 128 columns.  Operand tiles are stored [row][k] (k contiguous):
// activations are copied as they are, K-contiguous weights likewise, and
// N-contiguous weights are transposed in registers (8 k x 4 columns per
// thread) on the way in.  Column c of a wave's 64 is kept in LDS row
// 16 (c % 4) + c / 4, so that after the MFMA (weights as the first operand) a
// lane owns 16 consecutive output columns; for gate/up, LDS rows alternate
// W_gate / W_up features so each lane owns hg and hu of the same 8 features.
template <int MODE>
__host__ __device__ inline int tile_gemm_blocks(int H, int F) {
  return MODE == kGemmGateUp ? (2 * F + kTBN - 1) / kTBN : (MODE == kGemmDA ? (F + kTBN - 1) / kTBN : (H + kTBN - 1) / kTBN);
}

template <int MODE>
__device__ __forceinline__ void tile_gemm(const RowGemmArgs& g, int wg, uint16_t* s_a, uint16_t* s_b) {
  constexpr bool NN = RowGemmShape<MODE>::kNN;
  // the schedule, per wave (identical in every wave of the workgroup)
  const WaveTiles wt = wave_tile_prefix(g.offsets, g.E, kTBM, kBigRows, g.big_min_rows);
  const int H = g.H, F = g.F;
  const int nblk = tile_gemm_blocks<MODE>(H, F);
  const int item = xcd_item(wg, wt.total * nblk);
  // Items of one expert are walked in groups of up to 8 row tiles x all column
  // blocks, column-major inside a group, so the workgroups resident together
  // share both row tiles and weight tiles.
  if (item >= wt.total * nblk) return;  // uniform across the workgroup
  // the expert whose tiles hold tile id item / nblk, its first tile id and tiles
  const TileSlot first = wave_lookup_tile(wt, kTBM, item / nblk);
  const int start_e = item / nblk - first.tile;
  const int tiles_e = (first.expert_rows + kTBM - 1) / kTBM;
  const int li = item - start_e * nblk;
  const int grp = li / (8 * nblk);
  const int gm = min(8, tiles_e - 8 * grp);
  const int within = li - grp * 8 * nblk;
  const int mt = 8 * grp + within % gm;
  const int nb = within / gm;
  TileSlot ts;
  ts.expert = first.expert;
  ts.tile = mt;
  ts.expert_rows = first.expert_rows;
  ts.row_begin = first.row_begin + (mt - first.tile) * kTBM;
  ts.rows = min(first.expert_rows - mt * kTBM, kTBM);
  const int e = ts.expert;
  const int K = (MODE == kGemmGateUp || MODE == kGemmDA) ? H : (MODE == kGemmDown ? F : 2 * F);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lm = l & 15, gq = l >> 4;
  const int wm = w & 1, wn = w >> 1;
  const uint16_t* __restrict__ A = g.a;

  // ---- loader assignments
  // A: 128 rows x 8 chunks of 16 B; thread handles chunks tid + 256 i
  const uint16_t* a_src[4];
  bool a_ok[4];
  int a_dst[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ch = tid + 256 * i, row = ch >> 3, kc = ch & 7;
    a_ok[i] = row < ts.rows;
    a_src[i] = A + a_row_of(g, ts.row_begin + (a_ok[i] ? row : ts.rows - 1)) * K + 8 * kc;
    a_dst[i] = row * kTPitch + 8 * (kc ^ (row & 7));
  }
  // B, N-contiguous: thread -> 8 k-rows (8 kb .. 8 kb + 7) x 4 columns of one matrix
  // B, K-contiguous: thread -> 4 chunks (16 B) of weight rows
  // Columns (weight rows) past the output edge read column (row) 0 and are
  // never stored; k chunks past K read the first 8 k (N-contiguous) or column
  // 0 (K-contiguous) of the weights against zero activation chunks.
  const uint16_t* b_src[4];
  int b_dst[4];
  size_t ldb = 0;
  const uint16_t* b_lo = nullptr;  // K-contiguous: expert base for k < Kw (W_down for DA, W_gate for DX)
  const uint16_t* b_hi = nullptr;  // DX: W_up for F <= k < 2F
  int kb = 0;
  if (NN) {
    kb = tid >> 5;
    const int cb = tid & 31;
    const int bw = cb >> 4, cq = cb & 15;  // wave column block, quad within it
    const uint16_t* W;
    int gcol;
    if (MODE == kGemmGateUp) {
      W = (cq & 1) ? g.w1 : g.w0;
      gcol = nb * 64 + 32 * bw + 4 * (cq >> 1);
      if (gcol >= F) gcol = 0;
      ldb = F;
      W += (size_t)e * H * F;
    } else {
      W = g.w0 + (size_t)e * F * H;
      gcol = nb * 128 + 64 * bw + 4 * cq;
      if (gcol >= H) gcol = 0;
      ldb = H;
    }
    b_src[0] = W + gcol;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 64 * bw + 16 * i + cq;
      b_dst[i] = row * kTPitch + 8 * (kb ^ (row & 7));
    }
  } else {
    const int Nw = MODE == kGemmDA ? F : H;
    if (MODE == kGemmDA) {
      b_lo = g.w0 + (size_t)e * F * H;
      ldb = H;
    } else {
      b_lo = g.w0 + (size_t)e * H * F;
      b_hi = g.w1 + (size_t)e * H * F;
      ldb = F;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i, nl = ch >> 3;
      const int n = nb * kTBN + nl;
      const int bw = nl >> 6, nw = nl & 63;
      const int brow = 64 * bw + 16 * (nw & 3) + (nw >> 2);
      b_dst[i] = brow * kTPitch + 8 * ((ch & 7) ^ (brow & 7));
      b_src[i] = b_lo + (size_t)(n < Nw ? n : 0) * ldb;  // row start; the k offset is added per step
    }
  }

  // global -> register staging of one K-step
  struct Stage {
    u32x4 a[4];
    u32x2 bn[8];
    u32x4 bt[4];
  };
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  const int steps = (K + kTBK - 1) / kTBK;
  auto gload = [&](int s, Stage& st) {
    const int k0 = s * kTBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + 8 * ((tid + 256 * i) & 7);
      st.a[i] = *(const u32x4*)(k < K ? a_src[i] + k0 : zero_chunk());
    }
    if (NN) {
      const int kr = k0 + 8 * kb < K ? k0 + 8 * kb : 0;
#pragma unroll
      for (int r = 0; r < 8; ++r) st.bn[r] = *(const u32x2*)(b_src[0] + (size_t)(kr + r) * ldb);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = k0 + 8 * ((tid + 256 * i) & 7);
        const uint16_t* src;
        if (MODE == kGemmDX)
          src = k < F ? b_src[i] + k : (k < K ? b_src[i] - b_lo + b_hi + (k - F) : b_src[i]);
        else
          src = k < K ? b_src[i] + k : b_src[i];
        st.bt[i] = *(const u32x4*)src;
      }
    }
  };
  auto lstore = [&](int buf, const Stage& st) {
    uint16_t* sa = s_a + buf * (kTBM * kTPitch);
    uint16_t* sb = s_b + buf * (kTBN * kTPitch);
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4*)(sa + a_dst[i]) = a_ok[i] ? st.a[i] : z4;
    if (NN) {
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4*)(sb + b_dst[i]) = column_of_8x4(st.bn, i);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4*)(sb + b_dst[i]) = st.bt[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    // rows 64 wm + 16 i + lm (A) / 64 wn + 16 j + lm (B): row & 7 == lm & 7
    const uint16_t* sa = s_a + buf * (kTBM * kTPitch) + (64 * wm + lm) * kTPitch;
    const uint16_t* sb = s_b + buf * (kTBN * kTPitch) + (64 * wn + lm) * kTPitch;
#pragma unroll
    for (int kh = 0; kh < kTBK / 32; ++kh) {
      const int pos = 8 * ((4 * kh + gq) ^ (lm & 7));
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const u32x4*)(sa + 16 * i * kTPitch + pos);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = *(const u32x4*)(sb + 16 * j * kTPitch + pos);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(bf[j], af[i], acc[i][j]);
    }
  };

  // one register stage: step s+1's loads are in flight while step s is
  // multiplied out of LDS
  Stage st;
  gload(0, st);
  lstore(0, st);
  __syncthreads();
  for (int s = 0; s < steps; ++s) {
    if (s + 1 < steps) gload(s + 1, st);
    compute(s & 1);
    if (s + 1 < steps) lstore((s + 1) & 1, st);
    __syncthreads();
  }

  // epilogue: acc[ia][jb] register r -> row 64 wm + 16 ia + lm, virtual column
  // (c' = 4 gq + r, jb)
#pragma unroll
  for (int ia = 0; ia < 4; ++ia) {
    const int row = 64 * wm + 16 * ia + lm;
    if (row >= ts.rows) continue;
    const size_t grow = (size_t)ts.row_begin + row;
    if (MODE == kGemmGateUp) {
      // r even: gate, r odd: up, of feature 64 nb + 32 wn + 8 gq + 4 (r >> 1) + jb
      float hg[8], hu[8], av[8];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          hg[4 * h + jb] = acc[ia][jb][2 * h];
          hu[4 * h + jb] = acc[ia][jb][2 * h + 1];
        }
#pragma unroll
      for (int i = 0; i < 8; ++i) av[i] = hg[i] * sigmoidf_fast(hg[i]) * hu[i];
      const int f = nb * 64 + 32 * wn + 8 * gq;
      if (f >= F) continue;  // features past the edge (8 of them, all or none)
      if (g.out0 != nullptr) {
        uint16_t* hrow = g.out0 + grow * 2 * F;
        *(u32x4*)(hrow + f) =
            u32x4{pack_bf2(hg[0], hg[1]), pack_bf2(hg[2], hg[3]), pack_bf2(hg[4], hg[5]), pack_bf2(hg[6], hg[7])};
        *(u32x4*)(hrow + F + f) =
            u32x4{pack_bf2(hu[0], hu[1]), pack_bf2(hu[2], hu[3]), pack_bf2(hu[4], hu[5]), pack_bf2(hu[6], hu[7])};
      }
      if (g.out1 != nullptr)
        *(u32x4*)(g.out1 + grow * F + f) =
            u32x4{pack_bf2(av[0], av[1]), pack_bf2(av[2], av[3]), pack_bf2(av[4], av[5]), pack_bf2(av[6], av[7])};
    } else {
      // column 128 nb + 64 wn + 16 gq + 4 r + jb
      float v[16];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) v[4 * r + jb] = acc[ia][jb][r];
      const int col = nb * kTBN + 64 * wn + 16 * gq;
      const int ncols = row_gemm_cols<MODE>(H, F);
      if (col >= ncols) continue;  // past the edge; col + 8 .. + 15 are checked below
      const bool hi_ok = col + 8 < ncols;
      if (MODE == kGemmDA) {
        const uint16_t* hrow = g.h + h_row_of(g, grow) * 2 * F;
        const int col1 = hi_ok ? col + 8 : col;  // the second 8 columns, when inside
        const u32x4 g0 = *(const u32x4*)(hrow + col), g1 = *(const u32x4*)(hrow + col1);
        const u32x4 u0 = *(const u32x4*)(hrow + F + col), u1 = *(const u32x4*)(hrow + F + col1);
        float dgv[16], duv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t gw = (i < 8) ? g0[(i & 7) >> 1] : g1[(i & 7) >> 1];
          const uint32_t uw = (i < 8) ? u0[(i & 7) >> 1] : u1[(i & 7) >> 1];
          const float hgv = (i & 1) ? bf_hi(gw) : bf_lo(gw);
          const float huv = (i & 1) ? bf_hi(uw) : bf_lo(uw);
          const float sg = sigmoidf_fast(hgv);
          dgv[i] = v[i] * huv * sg * (1.0f + hgv * (1.0f - sg));
          duv[i] = v[i] * hgv * sg;
        }
        uint16_t* drow = g.out0 + grow * 2 * F;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && !hi_ok) break;
          const float* G = dgv + 8 * h;
          const float* U = duv + 8 * h;
          *(u32x4*)(drow + col + 8 * h) =
              u32x4{pack_bf2(G[0], G[1]), pack_bf2(G[2], G[3]), pack_bf2(G[4], G[5]), pack_bf2(G[6], G[7])};
          *(u32x4*)(drow + F + col + 8 * h) =
              u32x4{pack_bf2(U[0], U[1]), pack_bf2(U[2], U[3]), pack_bf2(U[4], U[5]), pack_bf2(U[6], U[7])};
        }
      } else {
        uint16_t* orow = g.out0 + grow * H + col;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && !hi_ok) break;
          const float* V = v + 8 * h;
          *(u32x4*)(orow + 8 * h) =
              u32x4{pack_bf2(V[0], V[1]), pack_bf2(V[2], V[3]), pack_bf2(V[4], V[5]), pack_bf2(V[6], V[7])};
        }
      }
    }
  }
}

// One launch serves both regimes: workgroups [0, n_stream) run the streaming
// kernel over experts with fewer than kBigRows rows, the rest run the LDS-tiled
// kernel over the others.  Both schedules are derived on the device.
template <int MODE, bool NONTEMP>
__global__ __launch_bounds__(256, 2) void row_gemm_bf16_kernel(RowGemmArgs g, int n_stream, int n_tile) {
  // 64 KiB: the tiled kernel's double-buffered A and B tiles, or the streaming
  // kernel's four per-wave areas (16 KiB of stages, or 8 KiB of split partial
  // sums for N-contiguous weights)
  __shared__ __attribute__((aligned(16))) uint16_t s_ab[2 * kTBM * kTPitch + 2 * kTBN * kTPitch];
  static_assert(sizeof(s_ab) == 4 * 16384, "streaming kernel: 16 KiB of LDS per wave");
  if ((int)blockIdx.x < n_stream)
    stream_gemm<MODE, false, NONTEMP>(g, blockIdx.x, reinterpret_cast<unsigned char*>(s_ab));
  else
    tile_gemm<MODE>(g, blockIdx.x - n_stream, s_ab, s_ab + 2 * kTBM * kTPitch);
}

// fp8 weights: every expert on the streaming kernel (one wave per 16-row tile
// and column block), so weight bytes are read once per 16 rows.  Down needs
// only 8 KiB of LDS per wave (split partial sums), which lets more workgroups
// share a CU.
template <int MODE, bool NONTEMP>
__global__ __launch_bounds__(256, 2) void row_gemm_fp8w_kernel(RowGemmArgs g) {
  // per wave: 8 KiB of split partial sums (down), 16 KiB (gate/up: twice the
  // columns) or 16 KiB of stages (K-contiguous weights)
  __shared__ __attribute__((aligned(16))) unsigned char s_lds[MODE == kGemmDown ? 4 * 8192 : 4 * 16384];
  stream_gemm<MODE, true, NONTEMP>(g, blockIdx.x, s_lds);
}

// Reduction split of the streaming kernel for this product and row count.
template <int MODE, bool W8>
int stream_split(const RowGemmArgs& g, int64_t N) {
  const int K = (MODE == kGemmGateUp || MODE == kGemmDA) ? g.H : (MODE == kGemmDown ? g.F : 2 * g.F);
  const int kstep = RowGemmShape<MODE>::kNN ? 32 : 128;  // whole K-steps in each part
  // decode-sized batches (a handful of rows in all) have too few tiles to keep
  // the chip's memory busy: split every product four ways
  int ks = N < kFewRows ? 4 : (kStreamSplitK >> (4 * MODE)) & 0xf;
  while (ks > 1 && (K % (ks * kstep) != 0 || stream_blocks<MODE, W8>(g.H, g.F) % (4 / ks) != 0)) ks /= 2;
  return ks;
}

}  // namespace

template <int MODE>
hipError_t launch_row_gemm_fp8w_mode(const RowGemmArgs& args, int max_rows, hipStream_t stream) {
  RowGemmArgs g = args;
  g.big_min_rows = kNoBigTiles;
  const int64_t N = max_rows, E = g.E;
  const int64_t tiles = (N + E * (kTileRows - 1)) / kTileRows;
  g.stream_ksplit = stream_split<MODE, true>(g, N);
  const int64_t grid = (tiles * stream_blocks<MODE, true>(g.H, g.F) * g.stream_ksplit + 3) / 4;
  if (grid <= 0) return hipSuccess;
  auto kern = N >= kFewRows ? row_gemm_fp8w_kernel<MODE, true> : row_gemm_fp8w_kernel<MODE, false>;
  MOE_LAUNCH(kern, dim3((unsigned)grid), dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_row_gemm_fp8w(int mode, const RowGemmArgs& g, int max_rows, hipStream_t stream) {
  switch (mode) {
    case kGemmGateUp: return launch_row_gemm_fp8w_mode<kGemmGateUp>(g, max_rows, stream);
    case kGemmDown: return launch_row_gemm_fp8w_mode<kGemmDown>(g, max_rows, stream);
    case kGemmDA: return launch_row_gemm_fp8w_mode<kGemmDA>(g, max_rows, stream);
    default: return launch_row_gemm_fp8w_mode<kGemmDX>(g, max_rows, stream);
  }
}

template <int MODE>
hipError_t launch_row_gemm_mode(const RowGemmArgs& args, int max_rows, int max_expert_rows, hipStream_t stream) {
  RowGemmArgs g = args;
  g.big_min_rows = big_gemm_min_rows(MODE, g.H, g.F);
  if (max_expert_rows < g.big_min_rows) g.big_min_rows = kNoBigTiles;  // no launch of a kernel with no work
  const int64_t N = max_rows, E = g.E;
  // streaming kernel: experts with n_e < kBigRows, ceil(n_e / 16) tiles each
  const int64_t small_tiles = std::min<int64_t>((N + E * (kTileRows - 1)) / kTileRows,
                                                 E * ((kBigRows - 1 + kTileRows - 1) / kTileRows));
  g.stream_ksplit = stream_split<MODE, false>(g, N);
  const int64_t n_stream = (small_tiles * row_gemm_blocks<MODE>(g.H, g.F) * g.stream_ksplit + 3) / 4;
  // tiled kernel: experts with kBigRows <= n_e < g.big_min_rows, ceil(n_e / 128) tiles each
  const int64_t big_experts = std::min<int64_t>(E, N / kBigRows);
  const int64_t big_tiles = std::min<int64_t>((N + big_experts * (kTBM - 1)) / kTBM,
                                              big_experts * ((g.big_min_rows + kTBM - 2) / kTBM));
  const int64_t n_tile = (big_experts == 0) ? 0 : ((big_tiles * tile_gemm_blocks<MODE>(g.H, g.F) + 7) / 8) * 8;
  const int64_t grid = n_stream + n_tile;
  if (grid <= 0) return hipSuccess;
  auto kern = N >= kFewRows ? row_gemm_bf16_kernel<MODE, true> : row_gemm_bf16_kernel<MODE, false>;
  MOE_LAUNCH(kern, dim3((unsigned)grid), dim3(256), 0, stream, g, (int)n_stream, (int)n_tile);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_big_gemm_bf16(MODE, g, max_rows, stream);
}

hipError_t launch_row_gemm_bf16(int mode, const RowGemmArgs& g, int max_rows, int max_expert_rows,
                                hipStream_t stream) {
  switch (mode) {
    case kGemmGateUp: return launch_row_gemm_mode<kGemmGateUp>(g, max_rows, max_expert_rows, stream);
    case kGemmDown: return launch_row_gemm_mode<kGemmDown>(g, max_rows, max_expert_rows, stream);
    case kGemmDA: return launch_row_gemm_mode<kGemmDA>(g, max_rows, max_expert_rows, stream);
    default: return launch_row_gemm_mode<kGemmDX>(g, max_rows, max_expert_rows, stream);
  }
}


}  // namespace moe
