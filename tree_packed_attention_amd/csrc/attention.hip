// Tree-masked flash attention for gfx950: RoPE at depth positions, tile plan
// from subtree ends, forward with online softmax, backward dQ and dK/dV.
//
// Visibility: key j is visible to query i iff j <= i < subtree_end[j]. In a
// preorder layout the descendants of j are the packed indices (j, se[j]), so
// this is the ancestor-or-self rule of the "Trie packing" page (Step 2) and of
// "Tree Training" §3.2 (attend iff j <= i and both lie on one root-to-leaf
// path), expressed with O(T) metadata instead of a (T, T) mask.
//
// Layouts (all tiles staged in LDS in natural row-major order):
//   q, o, dout, dq  [T][Hq][D] (caller, bf16 or f32)
//   k, v, dk, dv    [T][Hkv][D]
//   lse             [Hq][T] f32
// workspace:
//   qr [Hq][Tp][DP], kr [Hkv][Tp][DP]  bf16, RoPE applied, rows >= T and
//                                       columns >= D zero (DP = max(D, 32))
//   cs [Tp][D/2] float2                  cos / sin of every token's angles
//   kmm64 [nk64] int2, kmm128 [nk128]   min / max subtree end per key tile
//   qcount [nq], qlist [nq][nk64]       non-empty key tiles per query tile
//                                       (2 * tile + full flag), ascending
//   dd [Hq][Tp] f32                      rowsum(dO * O) for the backward
//
// Products use v_mfma_f32_32x32x16_bf16 with float32 accumulation. The
// forward and dQ kernels work on S^T (keys x queries): each lane then owns
// one query column, so softmax statistics reduce inside the lane plus one
// exchange with the lane 32 away, and the probabilities feed the next MFMA
// as its B operand without any data movement (key rows are fed to the first
// MFMA in bit-2/bit-3 swapped order so the C layout matches the B layout).
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "ta_device.h"
#include "profile.h"
#include "ta_error.h"
#include "tree_attn.h"

namespace ta {
namespace {

constexpr int kFwdBQ = 128;   // query rows per forward / dQ workgroup (4 waves x 32)
constexpr int kFwdBK = 64;    // keys per forward / dQ iteration
constexpr int kBwdBK = 128;   // keys per dK/dV workgroup (4 waves x 32)
constexpr int kBwdBQ = 64;    // query rows per dK/dV iteration
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int perm_row(int r) { return (r & ~31) | swap23(r & 31); }

// Key (or query) index, inside a 64-row tile, of C register i of M-block mb
// for lane group lg, when the A operand rows were fed in swap23 order.
__device__ __forceinline__ int c_row(int mb, int i, int lg) {
  return 32 * mb + 16 * (i >> 3) + 8 * lg + 4 * ((i >> 2) & 1) + (i & 3);
}

// ------------------------------------------------------------------------
// Prep: RoPE on q and k into the padded head-major workspace, and the cos /
// sin table. Angles are formed and reduced in float64, then evaluated in
// float32 on [-pi, pi].
template <typename Tin>
__global__ __launch_bounds__(256) void rope_prep_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                        const int* __restrict__ pos, int T, int Tp, int Hq,
                                                        int Hkv, int D, int DP, float theta,
                                                        bf16* __restrict__ qr, bf16* __restrict__ kr,
                                                        float2* __restrict__ cs) {
  __shared__ float2 tab[64];
  const int t = blockIdx.x;
  const int half = D / 2;
  if ((int)threadIdx.x < half) {
    float c = 1.0f, s = 0.0f;
    if (t < T && theta > 0.0f) {
      const double inv = exp2(-2.0 * (double)threadIdx.x / (double)D * log2((double)theta));
      const double ang = (double)pos[t] * inv;
      const double twopi = 6.283185307179586476925286766559;
      const double r = ang - rint(ang / twopi) * twopi;
      sincosf((float)r, &s, &c);
    }
    tab[threadIdx.x] = make_float2(c, s);
    cs[(size_t)t * half + threadIdx.x] = make_float2(c, s);
  }
  __syncthreads();
  const int H = Hq + Hkv;
  const int per_head = DP / 2;  // pairs (kk, kk + half) for kk < half; zero fill beyond D
  for (int idx = threadIdx.x; idx < H * per_head; idx += blockDim.x) {
    const int h = idx / per_head;
    const int kk = idx % per_head;
    const Tin* src;
    bf16* dst;
    if (h < Hq) {
      src = q + ((size_t)t * Hq + h) * D;
      dst = qr + ((size_t)h * Tp + t) * DP;
    } else {
      src = k + ((size_t)t * Hkv + (h - Hq)) * D;
      dst = kr + ((size_t)(h - Hq) * Tp + t) * DP;
    }
    if (kk < half) {
      float x1 = 0.0f, x2 = 0.0f;
      if (t < T) {
        x1 = to_f32(src[kk]);
        x2 = to_f32(src[kk + half]);
      }
      const float2 c = tab[kk];
      dst[kk] = (bf16)(x1 * c.x - x2 * c.y);
      dst[kk + half] = (bf16)(x2 * c.x + x1 * c.y);
    } else {
      // DP > D only for D = 16: columns D..DP-1 are zero padding
      dst[D + 2 * (kk - half)] = (bf16)0.0f;
      dst[D + 2 * (kk - half) + 1] = (bf16)0.0f;
    }
  }
}

// Per key tile: min and max subtree end (keys past T count as 0).
__global__ __launch_bounds__(256) void tile_minmax_kernel(const int* __restrict__ se, int T, int BK, int nk,
                                                          int2* __restrict__ out) {
  const int kt = blockIdx.x * blockDim.x + threadIdx.x;
  if (kt >= nk) return;
  int mn = INT_MAX, mx = 0;
  for (int j = kt * BK; j < kt * BK + BK; ++j) {
    const int s = j < T ? se[j] : 0;
    mn = min(mn, s);
    mx = max(mx, s);
  }
  out[kt] = make_int2(mn, mx);
}

// One wave per query tile: the compacted, ascending list of key tiles that
// hold at least one visible pair. Keys of tile kt cover [j0, max se) without
// gaps (every key's interval starts inside the tile), so the tile meets query
// rows [i0, i1) iff j0 <= i1 - 1 and max se > i0.
__global__ __launch_bounds__(64) void q_plan_kernel(const int2* __restrict__ kmm, int T, int BQ, int BK, int nk,
                                                    int* __restrict__ counts, int* __restrict__ lists) {
  const int qt = blockIdx.x;
  const int lane = threadIdx.x;
  const int i0 = qt * BQ;
  const int i1 = min(i0 + BQ, T);
  const int nkc = min(nk, (i1 - 1) / BK + 1);
  int* out = lists + (size_t)qt * nk;
  int n = 0;
  for (int base = 0; base < nkc; base += 64) {
    const int kt = base + lane;
    bool ne = false;
    int full = 0;
    if (kt < nkc) {
      const int2 m = kmm[kt];
      ne = m.y > i0;
      full = (kt * BK + BK - 1 <= i0) && (m.x >= i1);
    }
    const uint64_t mask = __ballot(ne);
    const int off = __popcll(mask & ((1ull << lane) - 1ull));
    if (ne) out[n + off] = 2 * kt + full;
    n += __popcll(mask);
  }
  if (lane == 0) counts[qt] = n;
}

// Loads 8 elements [c, c+8) of a caller row; zero past the row end or for
// rows past T.
template <typename Tio>
__device__ __forceinline__ bf16x8 load_row8(const Tio* rowp, bool row_ok, int c, int D) {
  return (row_ok && c < D) ? load8(rowp + c) : zero8();
}

// ------------------------------------------------------------------------
// Forward. One workgroup = 128 query rows of one head (4 waves x 32 rows),
// looping over the query tile's non-empty 64-key tiles.
template <int DP, typename Tio>
__global__ __launch_bounds__(256) void attn_fwd_kernel(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const Tio* __restrict__ v,
    const int* __restrict__ se, const int* __restrict__ counts, const int* __restrict__ lists, int T, int Tp,
    int Hq, int Hkv, int nq, int nk, float sl2, Tio* __restrict__ o, float* __restrict__ lse) {
  constexpr int D = DP == 32 ? 16 : DP;  // head dim (16 is padded to 32 for the MFMA shapes)
  constexpr int BK = kFwdBK;
  constexpr int KS = DP / 16;   // k steps of S^T = K' Q'^T
  constexpr int NDB = DP / 32;  // 32-wide d blocks of O^T
  constexpr int SK = DP + 8;    // LDS row strides (elements)
  constexpr int SV = DP + 16;
  __shared__ __attribute__((aligned(16))) bf16 ks_[BK * SK];
  __shared__ __attribute__((aligned(16))) bf16 vs_[BK * SV];
  __shared__ int ses[BK];

  const int G = Hq / Hkv;
  const int lid = xcd_remap(blockIdx.x, nq * Hq);
  const int gq = lid % G;
  const int hk = (lid / G) % Hkv;
  const int qt = lid / (G * Hkv);
  const int h = hk * G + gq;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  const int qrow = qt * kFwdBQ + 32 * w + lc;

  bf16x8 qop[KS];
  {
    const bf16* qb = qr + ((size_t)h * Tp + qrow) * DP + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) qop[s] = load8(qb + 16 * s);
  }
  f32x16 acc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) acc[b] = f32x16{};
  float m2 = kNegInf, lsum = 0.0f;

  const int cnt = counts[qt];
  const int* lst = lists + (size_t)qt * nk;
  const bf16* kbase = kr + (size_t)hk * Tp * DP;

  for (int it = 0; it < cnt; ++it) {
    const int e = lst[it];
    const int kt = e >> 1;
    const bool full = e & 1;
    const int j0 = kt * BK;
    __syncthreads();
    for (int vi = tid; vi < BK * DP / 8; vi += 256) {
      const int r = vi / (DP / 8), c = 8 * (vi % (DP / 8));
      *reinterpret_cast<bf16x8*>(ks_ + perm_row(r) * SK + c) = load8(kbase + (size_t)(j0 + r) * DP + c);
      const int j = j0 + r;
      *reinterpret_cast<bf16x8*>(vs_ + r * SV + c) =
          load_row8(v + ((size_t)j * Hkv + hk) * D, j < T, c, D);
    }
    if (tid < BK) ses[tid] = (j0 + tid < T) ? se[j0 + tid] : 0;
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16{};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(ks_ + (32 * mb + lc) * SK + 16 * st + 8 * lg);
        s[mb] = mfma32x32x16(a, qop[st], s[mb]);
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float x = s[mb][i] * sl2;
        if (!full) {
          const int kk = c_row(mb, i, lg);
          const bool vis = (j0 + kk <= qrow) && (qrow < ses[kk]);
          x = vis ? x : kNegInf;
        }
        s[mb][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(m2, mx);
    const float muse = (mnew == kNegInf) ? 0.0f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m2 - muse);
    m2 = mnew;
    float ps = 0.0f;
    bf16x8 pb[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[mb][i] - muse);
        ps += p;
        pb[2 * mb + (i >> 3)][i & 7] = (bf16)p;
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] *= alpha;

#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const bf16* pa = vs_ + (16 * t + 8 * lg + ((lane & 15) >> 2)) * SV + 32 * b + 16 * ((lane >> 4) & 1) +
                         4 * (lane & 3);
        const bf16x8 a = cat(lds_read_tr(pa), lds_read_tr(pa + 4 * SV));
        acc[b] = mfma32x32x16(a, pb[t], acc[b]);
      }
  }

  const float lt = lsum + __shfl_xor(lsum, 32);
  if (qrow < T) {
    const float inv = 1.0f / lt;
    Tio* orow = o + ((size_t)qrow * Hq + h) * D;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 32 * b + 8 * (i >> 2) + 4 * lg + (i & 3);
        if (d < D) orow[d] = from_f32<Tio>(acc[b][i] * inv);
      }
    if (lg == 0) lse[(size_t)h * T + qrow] = (m2 + log2f(lt)) * kLn2;
  }
}

// ------------------------------------------------------------------------
// Backward dQ. Same shape as the forward: a workgroup owns 128 query rows of
// one head and loops over their non-empty key tiles. It first forms
// D_i = dO_i . O_i from the dO operand registers it holds anyway and stores
// it for the dK/dV kernel.
//   S^T = K' Q'^T,  P^T = exp2(S^T * scale*log2e - lse*log2e)
//   dP^T = V dO^T,  dS^T = P^T (dP^T - D)
//   dQ'^T += K'^T dS^T  (A operand read transposed from the K' tile)
// then dQ = R(pos)^T * scale * dQ'.
template <int DP, typename Tio>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const Tio* __restrict__ v,
    const Tio* __restrict__ o, const Tio* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ dd, const int* __restrict__ se, const int* __restrict__ counts,
    const int* __restrict__ lists, const float2* __restrict__ cs, int T, int Tp, int Hq, int Hkv, int nq,
    int nk, float sl2, float scale, Tio* __restrict__ dq) {
  constexpr int D = DP == 32 ? 16 : DP;
  constexpr int BK = kFwdBK;
  constexpr int KS = DP / 16;
  constexpr int NDB = DP / 32;
  constexpr int SK = DP + 8;
  __shared__ __attribute__((aligned(16))) bf16 ks_[BK * SK];
  __shared__ __attribute__((aligned(16))) bf16 vs_[BK * SK];
  __shared__ int ses[BK];

  const int G = Hq / Hkv;
  const int lid = xcd_remap(blockIdx.x, nq * Hq);
  const int gq = lid % G;
  const int hk = (lid / G) % Hkv;
  const int qt = lid / (G * Hkv);
  const int h = hk * G + gq;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  const int qrow = qt * kFwdBQ + 32 * w + lc;
  const bool qok = qrow < T;

  bf16x8 qop[KS], dop[KS];
  float dval = 0.0f;
  {
    const bf16* qb = qr + ((size_t)h * Tp + qrow) * DP + 8 * lg;
    const size_t roff = ((size_t)(qok ? qrow : 0) * Hq + h) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qop[s] = load8(qb + 16 * s);
      dop[s] = load_row8(dout + roff, qok, 16 * s + 8 * lg, D);
      const bf16x8 ov = load_row8(o + roff, qok, 16 * s + 8 * lg, D);
#pragma unroll
      for (int e = 0; e < 8; ++e) dval += (float)dop[s][e] * (float)ov[e];
    }
  }
  dval += __shfl_xor(dval, 32);
  if (lg == 0) dd[(size_t)h * Tp + qrow] = dval;
  const float lse2 = qok ? lse[(size_t)h * T + qrow] * kLog2e : 0.0f;

  f32x16 acc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) acc[b] = f32x16{};

  const int cnt = counts[qt];
  const int* lst = lists + (size_t)qt * nk;
  const bf16* kbase = kr + (size_t)hk * Tp * DP;

  for (int it = 0; it < cnt; ++it) {
    const int e = lst[it];
    const int kt = e >> 1;
    const bool full = e & 1;
    const int j0 = kt * BK;
    __syncthreads();
    for (int vi = tid; vi < BK * DP / 8; vi += 256) {
      const int r = vi / (DP / 8), c = 8 * (vi % (DP / 8));
      const int pr = perm_row(r);
      *reinterpret_cast<bf16x8*>(ks_ + pr * SK + c) = load8(kbase + (size_t)(j0 + r) * DP + c);
      const int j = j0 + r;
      *reinterpret_cast<bf16x8*>(vs_ + pr * SK + c) = load_row8(v + ((size_t)j * Hkv + hk) * D, j < T, c, D);
    }
    if (tid < BK) ses[tid] = (j0 + tid < T) ? se[j0 + tid] : 0;
    __syncthreads();

    f32x16 s[2], dp[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16{};
      dp[mb] = f32x16{};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const int off = (32 * mb + lc) * SK + 16 * st + 8 * lg;
        s[mb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(ks_ + off), qop[st], s[mb]);
        dp[mb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(vs_ + off), dop[st], dp[mb]);
      }
    }
    bf16x8 db8[4];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = __builtin_amdgcn_exp2f(s[mb][i] * sl2 - lse2);
        if (!full) {
          const int kk = c_row(mb, i, lg);
          const bool vis = (j0 + kk <= qrow) && (qrow < ses[kk]);
          p = vis ? p : 0.0f;
        }
        db8[2 * mb + (i >> 3)][i & 7] = (bf16)(p * (dp[mb][i] - dval));
      }
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // K'^T operand: rows d = 32b + lane%32, k slots = keys 16t + 8lg + s
        const int kb = 16 * t + 8 * lg;
        const bf16* pa = ks_ + (perm_row(kb) + ((lane & 15) >> 2)) * SK + 32 * b + 16 * ((lane >> 4) & 1) +
                         4 * (lane & 3);
        const bf16* pb = ks_ + (perm_row(kb + 4) + ((lane & 15) >> 2)) * SK + 32 * b + 16 * ((lane >> 4) & 1) +
                         4 * (lane & 3);
        const bf16x8 a = cat(lds_read_tr(pa), lds_read_tr(pb));
        acc[b] = mfma32x32x16(a, db8[t], acc[b]);
      }
  }

  if (qok) {
    // lane holds dQ'^T column qrow, rows d = 32b + 8(i/4) + 4lg + i%4; the
    // RoPE partner d + D/2 sits in the same lane (D/2 is a multiple of 8).
    constexpr int half = D / 2;
    const float2* csr = cs + (size_t)qrow * half;
    Tio* out = dq + ((size_t)qrow * Hq + h) * D;
    float g[NDB * 16];
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) g[16 * b + i] = acc[b][i] * scale;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int d = 32 * b + 8 * (i >> 2) + 4 * lg + (i & 3);
        if (d < half) {
          // partner register: d + half = 32 b' + 8 a' + 4 lg + (i & 3)
          const int dp2 = d + half;
          const int b2 = dp2 >> 5, a2 = (dp2 & 31) >> 3;
          const float g1 = g[16 * b + i];
          const float g2 = g[16 * b2 + 4 * a2 + (i & 3)];
          const float2 c = csr[d];
          out[d] = from_f32<Tio>(g1 * c.x + g2 * c.y);
          out[dp2] = from_f32<Tio>(g2 * c.x - g1 * c.y);
        }
      }
  }
}

// ------------------------------------------------------------------------
// Backward dK / dV. One workgroup owns 128 keys of one kv head (4 waves x 32
// keys, K' and V rows held in registers) and loops over the query blocks its
// keys can see, for every query head of the group. The visible queries of a
// key tile form the contiguous range [j0, max se), so no list is needed.
//   S = Q' K'^T, P = exp2(S*scale*log2e - lse*log2e), dP = dO V^T
//   dS = P (dP - D);  dV += P^T dO;  dK' += dS^T Q'
// The accumulators never leave registers until the epilogue, which rotates
// dK back (R(pos)^T) through an LDS transpose and writes both once.
template <int DP, typename Tio>
__global__ __launch_bounds__(256) void attn_bwd_dkdv_kernel(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const Tio* __restrict__ v,
    const Tio* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dd,
    const int* __restrict__ se, const int2* __restrict__ kmm, const float2* __restrict__ cs, int T, int Tp,
    int Hq, int Hkv, int nkb, float sl2, float scale, Tio* __restrict__ dk, Tio* __restrict__ dv) {
  constexpr int D = DP == 32 ? 16 : DP;
  constexpr int BQ = kBwdBQ;
  constexpr int KS = DP / 16;
  constexpr int NDB = DP / 32;
  constexpr int SQ = DP + 8;
  constexpr int SE = DP + 4;  // epilogue f32 row stride
  constexpr int kTileBytes = 2 * BQ * SQ * 2;
  constexpr int kEpiBytes = 4 * 32 * SE * 4;
  constexpr int kSmem = kTileBytes > kEpiBytes ? kTileBytes : kEpiBytes;
  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmem];
  __shared__ __attribute__((aligned(16))) float lse_s[BQ];
  __shared__ __attribute__((aligned(16))) float dd_s[BQ];
  bf16* qs_ = reinterpret_cast<bf16*>(smem);
  bf16* ds_ = qs_ + BQ * SQ;

  const int G = Hq / Hkv;
  const int lid = xcd_remap(blockIdx.x, nkb * Hkv);
  const int kt = lid % nkb;
  const int hk = lid / nkb;

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  const int j0 = kt * kBwdBK;
  const int key = j0 + 32 * w + lc;
  const bool kok = key < T;
  const int myse = kok ? se[key] : 0;

  bf16x8 kop[KS], vop[KS];
  {
    const bf16* kb = kr + ((size_t)hk * Tp + key) * DP + 8 * lg;
    const Tio* vb = v + ((size_t)(kok ? key : 0) * Hkv + hk) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kop[s] = load8(kb + 16 * s);
      vop[s] = load_row8(vb, kok, 16 * s + 8 * lg, D);
    }
  }
  f32x16 acck[NDB], accv[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) {
    acck[b] = f32x16{};
    accv[b] = f32x16{};
  }

  const int2 mm = kmm[kt];
  const int qb_lo = j0 / BQ;
  const int qb_hi = (mm.y + BQ - 1) / BQ;

  for (int gq = 0; gq < G; ++gq) {
    const int h = hk * G + gq;
    const bf16* qbase = qr + (size_t)h * Tp * DP;
    for (int qb = qb_lo; qb < qb_hi; ++qb) {
      const int i0 = qb * BQ;
      const int i1 = min(i0 + BQ, T);
      const bool full = (j0 + kBwdBK - 1 <= i0) && (mm.x >= i1);
      __syncthreads();
      for (int vi = tid; vi < BQ * DP / 8; vi += 256) {
        const int r = vi / (DP / 8), c = 8 * (vi % (DP / 8));
        const int pr = perm_row(r);
        const int i = i0 + r;
        *reinterpret_cast<bf16x8*>(qs_ + pr * SQ + c) = load8(qbase + (size_t)i * DP + c);
        *reinterpret_cast<bf16x8*>(ds_ + pr * SQ + c) =
            load_row8(dout + ((size_t)(i < T ? i : 0) * Hq + h) * D, i < T, c, D);
      }
      if (tid < BQ) {
        const int i = i0 + tid;
        lse_s[tid] = i < T ? lse[(size_t)h * T + i] * kLog2e : 0.0f;
        dd_s[tid] = dd[(size_t)h * Tp + i];
      }
      __syncthreads();

#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          const int off = (32 * mb + lc) * SQ + 16 * st + 8 * lg;
          s = mfma32x32x16(*reinterpret_cast<const bf16x8*>(qs_ + off), kop[st], s);
          dp = mfma32x32x16(*reinterpret_cast<const bf16x8*>(ds_ + off), vop[st], dp);
        }
        // C register i <-> query row c_row(mb, i, lg) of this block; lane <-> key
        bf16x8 pa[2], sa[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qi = c_row(mb, i, lg);
          float p = __builtin_amdgcn_exp2f(s[i] * sl2 - lse_s[qi]);
          if (!full) {
            const int iq = i0 + qi;
            p = (key <= iq && iq < myse) ? p : 0.0f;
          }
          pa[i >> 3][i & 7] = (bf16)p;
          sa[i >> 3][i & 7] = (bf16)(p * (dp[i] - dd_s[qi]));
        }
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const int qb0 = 32 * mb + 16 * t2 + 8 * lg;  // natural query row of slot 0
#pragma unroll
          for (int b = 0; b < NDB; ++b) {
            const int col = 32 * b + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            const int r0 = perm_row(qb0) + ((lane & 15) >> 2);
            const int r1 = perm_row(qb0 + 4) + ((lane & 15) >> 2);
            const bf16x8 bdo = cat(lds_read_tr(ds_ + r0 * SQ + col), lds_read_tr(ds_ + r1 * SQ + col));
            accv[b] = mfma32x32x16(pa[t2], bdo, accv[b]);
            const bf16x8 bq = cat(lds_read_tr(qs_ + r0 * SQ + col), lds_read_tr(qs_ + r1 * SQ + col));
            acck[b] = mfma32x32x16(sa[t2], bq, acck[b]);
          }
        }
      }
    }
  }

  // Epilogue: stage each wave's 32 x DP block in LDS as [key][d] f32.
  __syncthreads();
  float* ep = reinterpret_cast<float*>(smem) + w * 32 * SE;
  constexpr int half = D / 2;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 8 * (i >> 2) + 4 * lg + (i & 3);
        ep[r * SE + 32 * b + lc] = pass == 0 ? acck[b][i] * scale : accv[b][i];
      }
    __syncthreads();
    for (int r = 0; r < 32; ++r) {
      const int j = j0 + 32 * w + r;
      if (j >= T) break;
      const float* er = ep + r * SE;
      if (pass == 0) {
        Tio* out = dk + ((size_t)j * Hkv + hk) * D;
        const float2* csr = cs + (size_t)j * half;
        for (int kk = lane; kk < half; kk += 64) {
          const float g1 = er[kk], g2 = er[kk + half];
          const float2 c = csr[kk];
          out[kk] = from_f32<Tio>(g1 * c.x + g2 * c.y);
          out[kk + half] = from_f32<Tio>(g2 * c.x - g1 * c.y);
        }
      } else {
        Tio* out = dv + ((size_t)j * Hkv + hk) * D;
        for (int c = lane; c < D; c += 64) out[c] = from_f32<Tio>(er[c]);
      }
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------------
// Host side
struct AttnLayout {
  int T, Tp, Hq, Hkv, D, DP, nq, nk64, nk128;
  size_t off_qr, off_kr, off_cs, off_kmm64, off_kmm128, off_qcount, off_qlist, off_dd, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

AttnLayout make_layout(int T, int Hq, int Hkv, int D, bool with_bwd) {
  AttnLayout L{};
  L.T = T;
  L.Tp = (T + kFwdBQ - 1) / kFwdBQ * kFwdBQ;
  L.Hq = Hq;
  L.Hkv = Hkv;
  L.D = D;
  L.DP = D < 32 ? 32 : D;
  L.nq = L.Tp / kFwdBQ;
  L.nk64 = (T + kFwdBK - 1) / kFwdBK;
  L.nk128 = (T + kBwdBK - 1) / kBwdBK;
  size_t o = 0;
  L.off_qr = o;
  o = align256(o + (size_t)Hq * L.Tp * L.DP * 2);
  L.off_kr = o;
  o = align256(o + (size_t)Hkv * L.Tp * L.DP * 2);
  L.off_cs = o;
  o = align256(o + (size_t)L.Tp * (D / 2) * 8);
  L.off_kmm64 = o;
  o = align256(o + (size_t)L.nk64 * 8);
  L.off_kmm128 = o;
  o = align256(o + (size_t)L.nk128 * 8);
  L.off_qcount = o;
  o = align256(o + (size_t)L.nq * 4);
  L.off_qlist = o;
  o = align256(o + (size_t)L.nq * L.nk64 * 4);
  L.off_dd = o;
  if (with_bwd) o = align256(o + (size_t)Hq * L.Tp * 4);
  L.total = o;
  return L;
}

int validate_shape(const char* fn, int T, int Hq, int Hkv, int d) {
  if (T < 1 || T > (1 << 22)) return fail(TA_EINVAL, "%s: T must be in [1, 2^22] (got %d)", fn, T);
  if (Hq < 1 || Hkv < 1 || Hq > 256 || Hq % Hkv != 0)
    return fail(TA_EINVAL, "%s: need 1 <= Hkv, Hq <= 256 and Hq %% Hkv == 0 (got Hq=%d Hkv=%d)", fn, Hq, Hkv);
  if (d != 16 && d != 64 && d != 128) return fail(TA_EUNSUPPORTED, "%s: head dim %d not in {16, 64, 128}", fn, d);
  return TA_OK;
}

int check_launch(const char* fn) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TA_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return TA_OK;
}

template <typename Tio>
int run_prep(const AttnLayout& L, const void* q, const void* k, const int* pos, const int* se, float theta,
             char* ws, hipStream_t st) {
  {
  ProfScope ps("rope_prep", st);
  hipLaunchKernelGGL(rope_prep_kernel<Tio>, dim3(L.Tp), dim3(256), 0, st, static_cast<const Tio*>(q),
                     static_cast<const Tio*>(k), pos, L.T, L.Tp, L.Hq, L.Hkv, L.D, L.DP, theta,
                     reinterpret_cast<bf16*>(ws + L.off_qr), reinterpret_cast<bf16*>(ws + L.off_kr),
                     reinterpret_cast<float2*>(ws + L.off_cs));
  }
  ProfScope ps("tile_plan", st);
  hipLaunchKernelGGL(tile_minmax_kernel, dim3((L.nk64 + 255) / 256), dim3(256), 0, st, se, L.T, kFwdBK, L.nk64,
                     reinterpret_cast<int2*>(ws + L.off_kmm64));
  hipLaunchKernelGGL(tile_minmax_kernel, dim3((L.nk128 + 255) / 256), dim3(256), 0, st, se, L.T, kBwdBK,
                     L.nk128, reinterpret_cast<int2*>(ws + L.off_kmm128));
  hipLaunchKernelGGL(q_plan_kernel, dim3(L.nq), dim3(64), 0, st, reinterpret_cast<const int2*>(ws + L.off_kmm64),
                     L.T, kFwdBQ, kFwdBK, L.nk64, reinterpret_cast<int*>(ws + L.off_qcount),
                     reinterpret_cast<int*>(ws + L.off_qlist));
  return check_launch("prep");
}

template <int DP, typename Tio>
int run_fwd(const AttnLayout& L, const void* v, const int* se, float sl2, void* o, float* lse, char* ws,
            hipStream_t st) {
  ProfScope ps("attn_fwd", st);
  hipLaunchKernelGGL((attn_fwd_kernel<DP, Tio>), dim3(L.nq * L.Hq), dim3(256), 0, st,
                     reinterpret_cast<const bf16*>(ws + L.off_qr), reinterpret_cast<const bf16*>(ws + L.off_kr),
                     static_cast<const Tio*>(v), se, reinterpret_cast<const int*>(ws + L.off_qcount),
                     reinterpret_cast<const int*>(ws + L.off_qlist), L.T, L.Tp, L.Hq, L.Hkv, L.nq, L.nk64,
                     sl2, static_cast<Tio*>(o), lse);
  return check_launch("tree_attn_fwd");
}

template <int DP, typename Tio>
int run_bwd(const AttnLayout& L, const void* v, const void* o, const float* lse, const void* dout, const int* se,
            float sl2, float scale, void* dq, void* dk, void* dv, char* ws, hipStream_t st) {
  {
  ProfScope ps("attn_bwd_dq", st);
  hipLaunchKernelGGL((attn_bwd_dq_kernel<DP, Tio>), dim3(L.nq * L.Hq), dim3(256), 0, st,
                     reinterpret_cast<const bf16*>(ws + L.off_qr), reinterpret_cast<const bf16*>(ws + L.off_kr),
                     static_cast<const Tio*>(v), static_cast<const Tio*>(o), static_cast<const Tio*>(dout), lse,
                     reinterpret_cast<float*>(ws + L.off_dd), se,
                     reinterpret_cast<const int*>(ws + L.off_qcount), reinterpret_cast<const int*>(ws + L.off_qlist),
                     reinterpret_cast<const float2*>(ws + L.off_cs), L.T, L.Tp, L.Hq, L.Hkv, L.nq, L.nk64,
                     sl2, scale, static_cast<Tio*>(dq));
  }
  ProfScope ps("attn_bwd_dkdv", st);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DP, Tio>), dim3(L.nk128 * L.Hkv), dim3(256), 0, st,
                     reinterpret_cast<const bf16*>(ws + L.off_qr), reinterpret_cast<const bf16*>(ws + L.off_kr),
                     static_cast<const Tio*>(v), static_cast<const Tio*>(dout), lse,
                     reinterpret_cast<const float*>(ws + L.off_dd), se,
                     reinterpret_cast<const int2*>(ws + L.off_kmm128), reinterpret_cast<const float2*>(ws + L.off_cs),
                     L.T, L.Tp, L.Hq, L.Hkv, L.nk128, sl2, scale, static_cast<Tio*>(dk),
                     static_cast<Tio*>(dv));
  return check_launch("tree_attn_bwd");
}

}  // namespace
}  // namespace ta

using namespace ta;

extern "C" size_t tree_attn_workspace_bytes(int32_t T, int32_t Hq, int32_t Hkv, int32_t d, int32_t with_bwd) {
  if (T < 1 || Hq < 1 || Hkv < 1 || d < 1) return 0;
  return make_layout(T, Hq, Hkv, d, with_bwd != 0).total;
}

extern "C" int tree_attn_fwd(const void* q, const void* k, const void* v, ta_dtype dt, int32_t T, int32_t Hq,
                             int32_t Hkv, int32_t d, const int32_t* pos, const int32_t* subtree_end,
                             float softmax_scale, float rope_theta, void* o, float* lse, void* workspace,
                             size_t ws_bytes, void* stream) {
  clear_error();
  if (int rc = validate_shape("tree_attn_fwd", T, Hq, Hkv, d)) return rc;
  if (!q || !k || !v || !pos || !subtree_end || !o || !lse || !workspace)
    return fail(TA_EINVAL, "tree_attn_fwd: NULL pointer argument");
  if (dt != TA_BF16 && dt != TA_F32) return fail(TA_EINVAL, "tree_attn_fwd: bad dtype %d", (int)dt);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TA_EINVAL, "tree_attn_fwd: workspace must be 256-byte aligned");
  if (!(rope_theta >= 0.0f)) return fail(TA_EINVAL, "tree_attn_fwd: rope_theta must be >= 0");
  const AttnLayout L = make_layout(T, Hq, Hkv, d, false);
  if (ws_bytes < L.total)
    return fail(TA_EINVAL, "tree_attn_fwd: workspace too small (%zu < %zu bytes)", ws_bytes, L.total);
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)d);
  const float sl2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int rc = dt == TA_BF16 ? run_prep<bf16>(L, q, k, pos, subtree_end, rope_theta, ws, st)
                         : run_prep<float>(L, q, k, pos, subtree_end, rope_theta, ws, st);
  if (rc) return rc;
  if (dt == TA_BF16) {
    if (L.DP == 32) return run_fwd<32, bf16>(L, v, subtree_end, sl2, o, lse, ws, st);
    if (L.DP == 64) return run_fwd<64, bf16>(L, v, subtree_end, sl2, o, lse, ws, st);
    return run_fwd<128, bf16>(L, v, subtree_end, sl2, o, lse, ws, st);
  }
  if (L.DP == 32) return run_fwd<32, float>(L, v, subtree_end, sl2, o, lse, ws, st);
  if (L.DP == 64) return run_fwd<64, float>(L, v, subtree_end, sl2, o, lse, ws, st);
  return run_fwd<128, float>(L, v, subtree_end, sl2, o, lse, ws, st);
}

extern "C" int tree_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, ta_dtype dt, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                             const int32_t* pos, const int32_t* subtree_end, float softmax_scale, float rope_theta,
                             int32_t flags, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                             void* stream) {
  clear_error();
  if (int rc = validate_shape("tree_attn_bwd", T, Hq, Hkv, d)) return rc;
  if (!q || !k || !v || !o || !lse || !dout || !pos || !subtree_end || !dq || !dk || !dv || !workspace)
    return fail(TA_EINVAL, "tree_attn_bwd: NULL pointer argument");
  if (dt != TA_BF16 && dt != TA_F32) return fail(TA_EINVAL, "tree_attn_bwd: bad dtype %d", (int)dt);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TA_EINVAL, "tree_attn_bwd: workspace must be 256-byte aligned");
  if (!(rope_theta >= 0.0f)) return fail(TA_EINVAL, "tree_attn_bwd: rope_theta must be >= 0");
  if (flags & ~TA_REUSE_PREP) return fail(TA_EINVAL, "tree_attn_bwd: unknown flags 0x%x", flags);
  const AttnLayout L = make_layout(T, Hq, Hkv, d, true);
  if (ws_bytes < L.total)
    return fail(TA_EINVAL, "tree_attn_bwd: workspace too small (%zu < %zu bytes)", ws_bytes, L.total);
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)d);
  const float sl2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (!(flags & TA_REUSE_PREP)) {
    int rc = dt == TA_BF16 ? run_prep<bf16>(L, q, k, pos, subtree_end, rope_theta, ws, st)
                           : run_prep<float>(L, q, k, pos, subtree_end, rope_theta, ws, st);
    if (rc) return rc;
  }
  if (dt == TA_BF16) {
    if (L.DP == 32) return run_bwd<32, bf16>(L, v, o, lse, dout, subtree_end, sl2, scale, dq, dk, dv, ws, st);
    if (L.DP == 64) return run_bwd<64, bf16>(L, v, o, lse, dout, subtree_end, sl2, scale, dq, dk, dv, ws, st);
    return run_bwd<128, bf16>(L, v, o, lse, dout, subtree_end, sl2, scale, dq, dk, dv, ws, st);
  }
  if (L.DP == 32) return run_bwd<32, float>(L, v, o, lse, dout, subtree_end, sl2, scale, dq, dk, dv, ws, st);
  if (L.DP == 64) return run_bwd<64, float>(L, v, o, lse, dout, subtree_end, sl2, scale, dq, dk, dv, ws, st);
  return run_bwd<128, float>(L, v, o, lse, dout, subtree_end, sl2, scale, dq, dk, dv, ws, st);
}
