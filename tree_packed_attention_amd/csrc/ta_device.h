// Device-side helpers for the gfx950 kernels: vector types, bf16 packing,
// MFMA wrappers and the lane layouts the kernels rely on.
//
// Lane layouts of the bf16 matrix instructions used here (wave64):
//   v_mfma_f32_32x32x16_bf16  D[32x32] = A[32x16] * B[16x32] + C
//     A: lane l holds row m = l % 32, k = 8 * (l / 32) + s, s = 0..7
//     B: lane l holds col n = l % 32, k = 8 * (l / 32) + s
//     C/D: lane l holds col n = l % 32, reg i holds row 8*(i/4) + 4*(l/32) + i%4
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane j receives
//   element (j % 4) of the 8-byte row that lane 4*r + j/4 addressed, r = 0..3.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ta {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row permutation inside a 32-row MFMA block: swapping bits 2 and 3 makes the
// C-layout rows a lane holds for one 16-wide k step contiguous. It is its own
// inverse.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Transposing 8-byte LDS read (see the layout note above).
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat(const bf16x4& a, const bf16x4& b) {
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// 8 consecutive elements of a row as bf16 (float inputs are rounded).
__device__ __forceinline__ bf16x8 load8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ bf16x8 load8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  bf16x8 r;
  r[0] = (bf16)a[0]; r[1] = (bf16)a[1]; r[2] = (bf16)a[2]; r[3] = (bf16)a[3];
  r[4] = (bf16)b[0]; r[5] = (bf16)b[1]; r[6] = (bf16)b[2]; r[7] = (bf16)b[3];
  return r;
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 r;
#pragma unroll
  for (int s = 0; s < 8; ++s) r[s] = (bf16)0.0f;
  return r;
}

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Maps a launch-order block index to a logical work index so that blocks the
// hardware sends to the same XCD (round-robin over 8) get consecutive logical
// indices and share that XCD's L2. A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int per = n / 8;
  const int full = per * 8;
  if (b >= full) return b;
  return (b % 8) * per + b / 8;
}

}  // namespace ta
