// LDS tiles for the gfx950 kernels: the XOR swizzle of 16-byte chunks and
// the direct HBM -> LDS copies (global_load_lds) that fill them.
//
// A [64][DP] bf16 tile stores 16-byte chunk c of row r at chunk c ^ swz(r),
// which keeps both 16-byte operand reads (8 consecutive rows, one chunk) and
// 8-byte transposing reads (4 consecutive rows, two adjacent chunks) free of
// bank conflicts.
#pragma once
#include <hip/hip_runtime.h>

#include "ta_device.h"

namespace ta {
namespace {

__device__ __forceinline__ int perm_row(int r) { return (r & ~31) | swap23(r & 31); }

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// Element offset of (row, col) in a swizzled [64][DP] bf16 tile (col % 4 == 0).
template <int DP>
__device__ __forceinline__ int toff(int row, int col) {
  constexpr int CH = DP / 8;
  return row * DP + ((((col >> 3) ^ swz(row)) & (CH - 1)) << 3) + (col & 7);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void glb_void;

#if TA_DMA_ASM
// The copies are issued as inline assembly. The compiler models an LDS copy
// in flight as an unordered event on the counter LDS reads share, so with
// the builtin every LDS operand wait behind a copy becomes a full wait (no
// read-ahead at all while the next tile is being copied). Written this way
// the compiler does not see the copies: the kernels that use them wait for
// them themselves (s_waitcnt vmcnt(0), then a barrier, before a copied tile
// is read, and a barrier after the last read of a buffer before it is
// refilled). The instruction writes no register; m0 holds the LDS address
// and is set in the same statement (one wait state before its use).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
// Each lane copies 16 bytes from g to (wave-uniform) dst + 16 * lane.
__device__ __forceinline__ void dma16(const void* g, void* dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr(dst))
               : "memory", "m0");
}
// Each lane copies 4 bytes from g to (wave-uniform) dst + 4 * lane.
__device__ __forceinline__ void dma4(const void* g, void* dst) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_addr(dst))
               : "memory", "m0");
}
#pragma clang diagnostic pop
#else
// Each lane copies 16 bytes from g to (wave-uniform) dst + 16 * lane.
__device__ __forceinline__ void dma16(const void* g, void* dst) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)dst, 16, 0, 0);
}
// Each lane copies 4 bytes from g to (wave-uniform) dst + 4 * lane.
__device__ __forceinline__ void dma4(const void* g, void* dst) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, (lds_void*)dst, 4, 0, 0);
}
#endif
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Copies 64 head-major rows [row0 + rowmap(r)] of a [*][DP] bf16 array into a
// swizzled LDS tile. Each wave issues DP/32 16-byte-per-lane instructions;
// every lane's offset inside the 64-row block is fixed, so it is computed once.
template <int DP, bool PERM, int NW = 4>
struct TileDma {
  static constexpr int CH = DP / 8;                // 16-byte chunks per row (= instructions per tile)
  static constexpr int NI = (CH + NW - 1) / NW;    // instructions per wave (the last may be idle)
  int off[NI];
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int p = (w + NW * j) * 64 + lane;
      const int r = min(p / CH, 63);
      const int c = ((p % CH) ^ swz(r)) & (CH - 1);
      off[j] = (PERM ? perm_row(r) : r) * DP + 8 * c;
    }
  }
  // rows: the global address of row row0 of the source; w: wave index (uniform)
  __device__ __forceinline__ void issue(const bf16* rows, bf16* tile, int w) const {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if (w + NW * j < CH) dma16(rows + off[j], tile + (w + NW * j) * 512);
  }
};

__device__ __forceinline__ bf16x8 lds128(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

}  // namespace
}  // namespace ta
