// moe_lds32.h -- device helpers shared by the LDS-tiled gfx950 GEMM kernels
// built on the 32x32x16 bf16 matrix core: direct global->LDS loads, a
// fence-free workgroup barrier, counted waits, and transposed fragment reads
// from N-contiguous ([k][column]) LDS tiles.
#pragma once

#include "moe_common.h"

namespace moe {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef float f32x16 __attribute__((ext_vector_type(16)));

// D = first x second + D on the 32x32x16 bf16 matrix core.  Lane l supplies
// row (first) / column (second) l % 32 and k-group l / 32 (8 consecutive k);
// register r of lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__device__ __forceinline__ f32x16 mfma32(u32x4 first, u32x4 second, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, first), __builtin_bit_cast(bf16x8, second),
                                                  acc, 0, 0, 0);
}

// 16 B from global straight into LDS at lds_base + 16 * lane (lds_base
// wave-uniform).
// Issued as inline assembly so that the compiler does not see an LDS write in
// flight: it would otherwise wait for every outstanding direct load before the
// next LDS read, whichever buffer that read touches, and no stage could load
// while another is computed.  Completion is the caller's business (wait_vmcnt
// and a barrier before the stage is read).
__device__ __forceinline__ void g2lds(const void* src, void* lds_base) {
  // m0 carries the LDS address; its previous value is restored for the compiler
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)lds_base);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(src), "s"(lds)
      : "memory");
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would make the compiler wait for every outstanding global load (including
// the stages still meant to be in flight).  LDS data written by the direct
// loads is made complete explicitly with wait_vmcnt before this barrier; the
// asm clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // s_waitcnt vmcnt(N); expcnt and lgkmcnt left unconstrained
  static_assert(N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// k row of an N-contiguous tile -> XOR on the 16-byte chunk index (keeps the
// 4-chunk groups one transpose read covers aligned)
__device__ __forceinline__ int nn_swz(int k) { return 4 * (k & 3); }

// 32x32x16 operand fragment from an N-contiguous LDS tile ([k][column], row
// pitch `pitch` bytes, 16-byte chunks swizzled by nn_swz(k)): MFMA row/column
// index = tile column col_base + (0..31), k = 16 sub + (0..15).  Uses the
// gfx950 transpose read ds_read_b64_tr_b16: within each 16-lane group G, lane
// r points at k row 8 (G >> 1) + 4 h + (r >> 2) and columns 16 (G & 1) +
// 4 (r & 3) .. + 3, and receives 4 consecutive k of one column (half of the
// lane's 8 k).
__device__ __forceinline__ u32x4 tr_frag32(const unsigned char* tile, int pitch, int sub, int col_base) {
  const int l = __lane_id(), G = l >> 4, r = l & 15;
  const int col = col_base + 16 * (G & 1) + 4 * (r & 3);
  v4i16 part[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = 16 * sub + 8 * (G >> 1) + 4 * h + (r >> 2);
    const int chunk = (col >> 3) ^ nn_swz(k);
    part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(tile + k * pitch + 16 * chunk + 2 * (col & 7)));
  }
  return u32x4{(uint32_t)(uint16_t)part[0][0] | ((uint32_t)(uint16_t)part[0][1] << 16),
               (uint32_t)(uint16_t)part[0][2] | ((uint32_t)(uint16_t)part[0][3] << 16),
               (uint32_t)(uint16_t)part[1][0] | ((uint32_t)(uint16_t)part[1][1] << 16),
               (uint32_t)(uint16_t)part[1][2] | ((uint32_t)(uint16_t)part[1][3] << 16)};
}

}  // namespace moe
