// Dictionary tiles for the MFMA sweeps (screening and the full-dictionary yardstick).
//
// A tile is 16 consecutive atoms.  It is copied global -> LDS by direct-to-LDS loads whose
// lanes read the rows contiguously (one load moves 1 KB, four lanes a 64-byte segment), then
// every lane reads its MFMA fragment (row lane % 16, 16-byte chunk 4 i + lane / 16) back from
// the wave's stage.  The stage keeps chunk c of row r at position c ^ swz(r), so the 16 rows
// of a fragment read fall in distinct LDS banks.  A tile's 16x16 products per vector block
// land as 4 accumulators per lane: vector lane % 16 of the block, atoms 4 (lane / 16) + e.
#pragma once

#include "common.h"

namespace fadkv {
namespace tile {

typedef float float4_t __attribute__((ext_vector_type(4)));

template <int DT, int D> struct Geo {
  static constexpr int ROWB = D * Elem<DT>::bytes;   // bytes per row
  static constexpr int CPR = ROWB / 16;              // 16-byte chunks per row
  static constexpr int CH = CPR / 4;                 // chunks per lane per row (fragment steps)
  static constexpr int LOADS = ROWB / 64;            // 1 KB loads per 16-row tile
  static constexpr int STAGE = 16 * CPR;             // 16-byte slots per wave stage
};

// stage position of chunk c in row r is c ^ swz(r): 16 rows reading the same chunk hit 16
// distinct 16-byte bank groups (rows of 256 or 512 bytes: low 4 bits of r; rows of 128
// bytes: two rows share a 256-byte bank window, so bits 1..3 of r)
template <int CPR> __device__ __forceinline__ int swz(int r) {
  if constexpr (CPR >= 16) return r & 15;
  else return (r >> 1) & (CPR - 1);
}

// 16 bytes per lane global -> LDS (lane L writes LDS bytes [lds + 16 L, lds + 16 L + 16)).
// Written as assembly so that the compiler does not treat the copy as an LDS store that
// every later LDS access must wait for: the sweep orders the stage by hand (wait_vmem before
// the fragment reads, wait_lds before the stage is refilled), and the histogram and boundary
// regions never overlap the stages.  M0 holds the LDS address; one wait state after writing it.
// M0 is otherwise unused by these kernels (no LDS DMA builtins, no indexed register moves),
// so clobbering it cannot break a value the compiler keeps there; a CPU test checks the
// generated code for any other M0 use.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// per-lane 64-bit address
__device__ __forceinline__ void copy16_to_lds(const void *gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}
// wave-uniform 64-bit base + per-lane 32-bit offset
__device__ __forceinline__ void copy16_to_lds(const void *base, uint32_t off, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
}

// Tile t is rows 16 t .. 16 t + 15; load j, lane L moves stage slot 64 j + L, which holds
// row (64 j + L) / CPR, chunk ((64 j + L) % CPR) ^ swz(row).  tile_offsets gives the lane's
// byte offsets inside a tile; a tile that ends past N takes the clamped path (rows >= N read
// row N - 1, whose scores are discarded).
template <int DT, int D>
__device__ __forceinline__ void tile_offsets(int lane, uint32_t (&off)[Geo<DT, D>::LOADS]) {
  using G = Geo<DT, D>;
#pragma unroll
  for (int j = 0; j < G::LOADS; ++j) {
    const int slot = 64 * j + lane;
    const int row = slot / G::CPR;
    const int chunk = (slot % G::CPR) ^ swz<G::CPR>(row);
    off[j] = (uint32_t)(row * G::ROWB + chunk * 16);
  }
}

template <int DT, int D>
__device__ __forceinline__ void issue_tile(const uint8_t *dict_atoms, int N, int t, int lane,
                                           const uint32_t (&off)[Geo<DT, D>::LOADS],
                                           uint32_t stage_lds) {
  using G = Geo<DT, D>;
  if (t * 16 + 16 <= N) {
    const uint8_t *tile = uniform_ptr(dict_atoms + (size_t)t * 16 * G::ROWB);
#pragma unroll
    for (int j = 0; j < G::LOADS; ++j) copy16_to_lds(tile, off[j], stage_lds + 1024u * j);
  } else {
#pragma unroll
    for (int j = 0; j < G::LOADS; ++j) {
      const int slot = 64 * j + lane;
      const int row = slot / G::CPR;
      const int chunk = (slot % G::CPR) ^ swz<G::CPR>(row);
      int grow = t * 16 + row;
      grow = grow < N ? grow : N - 1;
      copy16_to_lds(dict_atoms + (size_t)grow * G::ROWB + chunk * 16, stage_lds + 1024u * j);
    }
  }
}

// s_waitcnt vmcnt(0) / lgkmcnt(0) (gfx9 encoding; the other counters left at their maximum)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// acc += the 16x16 products of one tile with both vector blocks
template <int DT, int D>
__device__ __forceinline__ void tile_mma(const uint4 (&a)[Geo<DT, D>::CH],
                                         const uint4 (&b)[2][Geo<DT, D>::CH], float4_t &acc0,
                                         float4_t &acc1) {
#pragma unroll
  for (int i = 0; i < Geo<DT, D>::CH; ++i) {
    if constexpr (DT == DT_F16) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a[i]),
                                                    __builtin_bit_cast(half8_t, b[0][i]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a[i]),
                                                    __builtin_bit_cast(half8_t, b[1][i]), acc1, 0, 0, 0);
    } else if constexpr (DT == DT_BF16) {
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[i]),
                                                     __builtin_bit_cast(bf16x8_t, b[0][i]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[i]),
                                                     __builtin_bit_cast(bf16x8_t, b[1][i]), acc1, 0, 0, 0);
    } else {
      // fp32: one k element per lane and instruction; element e of the chunk at step e
      const uint32_t av[4] = {a[i].x, a[i].y, a[i].z, a[i].w};
      const uint32_t b0[4] = {b[0][i].x, b[0][i].y, b[0][i].z, b[0][i].w};
      const uint32_t b1[4] = {b[1][i].x, b[1][i].y, b[1][i].z, b[1][i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av[e]), __uint_as_float(b0[e]), acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av[e]), __uint_as_float(b1[e]), acc1, 0, 0, 0);
      }
    }
  }
}

// 16x16 scores of one tile for both vector blocks
template <int DT, int D>
__device__ __forceinline__ void tile_scores(const uint4 (&a)[Geo<DT, D>::CH],
                                            const uint4 (&b)[2][Geo<DT, D>::CH], float4_t &acc0,
                                            float4_t &acc1) {
  acc0 = float4_t{0.f, 0.f, 0.f, 0.f};
  acc1 = acc0;
  tile_mma<DT, D>(a, b, acc0, acc1);
}

}  // namespace tile
}  // namespace fadkv
