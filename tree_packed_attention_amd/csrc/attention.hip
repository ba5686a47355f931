// Tree-masked flash attention for gfx950: RoPE at depth positions, tile plan
// from subtree ends, forward with online softmax, backward dQ and dK/dV.
//
// Visibility: key j is visible to query i iff j <= i < subtree_end[j]. In a
// preorder layout the descendants of j are the packed indices (j, se[j]), so
// this is the ancestor-or-self rule of the "Trie packing" page (Step 2) and of
// "Tree Training" §3.2 (attend iff j <= i and both lie on one root-to-leaf
// path), expressed with O(T) metadata instead of a (T, T) mask.
//
// Layouts:
//   q, o, dout, dq  [T][Hq][D] (caller, bf16 or f32)
//   k, v, dk, dv    [T][Hkv][D]
//   lse             [Hq][T] f32
// workspace (Tp = T rounded up to 256, DP = max(D, 32); padding is zero):
//   status (one int at offset 0)         device-side data errors of the last prep
//   qr [Hq][Tp][DP], kr, vr [Hkv][Tp][DP]  bf16; q, k rotated by RoPE
//   sep [Tp]                             subtree ends, 0 past T
//   cs [Tp][D/2] float2                  cos / sin of every token's angles
//   kmm64 [nk64], kmm128 [nk128] int2    min / max subtree end per key tile
//   sbmax [nk64 / 64]                    max subtree end per 4096-key superblock
//   qcount, qfull, qorder [nq]           non-empty and full 64-key tiles per
//                                        128-row query tile, work order (the
//                                        tile lists themselves are built per
//                                        workgroup in LDS: O(T) plan storage)
//   kwork, korder [nk128]                query blocks per 128-key tile; scratch
//   cdesc [nk128 + 32] int4              dK/dV chunks, heaviest first
//   ktcut [32] int4                      the cut tiles: {tile, chunks, first slot}
//   dd, l2 [Hq][Tp] f32                  -rowsum(dO * O) and -lse / scale
//   dor [Hq][Tp][DP] bf16                dO, head-major (written by dQ pass)
//   kpart [64][Hkv][8][DP/8][64][4] f32  dK/dV partial sums of cut tiles
//
// Products use v_mfma_f32_32x32x16_bf16 with float32 accumulation. The
// forward and dQ kernels work on S^T (keys x queries): each lane then owns
// one query column, so softmax statistics reduce inside the lane plus one
// exchange with the lane 32 away, and the probabilities feed the next MFMA
// as its B operand without any data movement (the key rows of a tile sit in
// LDS in bit-2/bit-3 swapped order so that the C layout of the first product
// matches the B layout of the second).
//
// Tiles move HBM -> LDS with global_load_lds_dwordx4 (no register staging),
// double buffered: the loads for tile i+1 are in flight while tile i is
// computed. Each 64-row tile is stored without padding; 16-byte chunk c of
// row r sits at chunk c ^ swz(r), which keeps both the 16-byte operand reads
// (8 consecutive rows, one chunk) and the transposing 8-byte reads (4
// consecutive rows, two adjacent chunks) free of bank conflicts.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>

#include "profile.h"
#include "ta_device.h"
#ifndef TA_DMA_ASM
#define TA_DMA_ASM 1
#endif
#include "ta_lds.h"
#include "ta_error.h"
#include "tree_attn.h"

// Build-time scheduling knobs (defaults are the measured best).
#ifndef TA_IGLP
#define TA_IGLP -1  // >= 0: __builtin_amdgcn_iglp_opt(TA_IGLP) in the tile bodies
#endif
#ifndef TA_FWD_WAVES
#define TA_FWD_WAVES 4  // forward workgroup: TA_FWD_WAVES waves x 32 query rows
#endif
// LDS operand reads issued this many reads ahead of the MFMAs that use them
// (0: left to the compiler), per kernel
#ifndef TA_LA_FWD
#define TA_LA_FWD 0
#endif
#ifndef TA_LA_DQ
#define TA_LA_DQ 4
#endif
#ifndef TA_LA_DKDV
#define TA_LA_DKDV 4
#endif

namespace ta {
namespace {

__device__ __forceinline__ void sched_hint() {
#if TA_IGLP >= 0
  __builtin_amdgcn_iglp_opt(TA_IGLP);
#endif
}

// Issue order for one straight-line product: the first L LDS reads, then
// after each MFMA the next reads in turn, so every operand is requested
// about L reads before the MFMA that consumes it instead of just before it
// (the compiler's default under register pressure). MF MFMAs and RD LDS
// reads in all; the region is the enclosing basic block.
template <int MF, int RD, int PER>
struct LdsAheadTail {
  static __device__ __forceinline__ void emit() {
    if constexpr (MF > 0) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      constexpr int r = RD < PER ? RD : PER;
      if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
      LdsAheadTail<MF - 1, RD - r, PER>::emit();
    }
  }
};
template <int L, int MF, int RD>
__device__ __forceinline__ void lds_ahead() {
  if constexpr (L > 0) {
    constexpr int pre = L < RD ? L : RD;
    constexpr int per = (RD + MF - 1) / MF;
    __builtin_amdgcn_sched_group_barrier(0x100, pre, 0);
    LdsAheadTail<MF, RD - pre, per>::emit();
  }
}

constexpr int kFwdBQ = 128;  // query rows per forward / dQ workgroup (4 waves x 32)
constexpr int kFwdBK = 64;   // keys per forward / dQ iteration
constexpr int kBwdBK = 128;  // keys per dK/dV workgroup (4 waves x 32)
constexpr int kBwdBQ = 64;   // query rows per dK/dV iteration
constexpr float kNegInf = -__builtin_inff();
// Lazy rescaling: the running maximum used as the softmax reference is only
// raised when a tile's maximum exceeds it by more than 2^8 (log2 units), so
// probabilities stay <= 256 and the O accumulator is rarely touched.
constexpr float kRescaleLog2 = 8.0f;


// Per-lane element offsets into a swizzled [64][DP] tile, computed once:
//   op[k]: 16-byte operand read of LDS row lc (+32 mb), columns 16k + 8lg
//   tr[b]: transposed read of rows 4lg + (lane%16)/4 (+16 t, +8, +32 mb),
//          columns 32b + 16((lane/16)%2) + 4(lane%4)
// The swizzle of a row depends only on its low 3 bits, which the row
// offsets added at the call sites (multiples of 8) leave unchanged.
template <int DP>
struct SwzAddr {
  int op[DP / 16];
  int tr[DP / 32];
  __device__ __forceinline__ void init(int lane) {
    const int lg = lane >> 5, lc = lane & 31;
#pragma unroll
    for (int k = 0; k < DP / 16; ++k) op[k] = toff<DP>(lc, 16 * k + 8 * lg);
#pragma unroll
    for (int b = 0; b < DP / 32; ++b)
      tr[b] = toff<DP>(4 * lg + ((lane & 15) >> 2), 32 * b + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));
  }
};

// ------------------------------------------------------------------------
// Prep: RoPE on q and k, the padded bf16 copy of v, the padded subtree ends
// and the cos / sin table. Angles are formed and reduced in float64, then
// evaluated in float32 on [-pi, pi]. One workgroup per token; each thread
// rotates 8-element chunks (kk .. kk+7 with their partners kk+half ..) with
// 16-byte loads and stores.
__device__ __forceinline__ void load8f(const bf16* p, float* x) {
  const bf16x8 v = load8(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void load8f(const float* p, float* x) {  // rotated in float, rounded once
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[e] = a[e];
    x[4 + e] = b[e];
  }
}

// Status word at the start of the workspace: bits of data errors only the
// device can see. It is cleared at the start of every prep pass and read by
// tree_attn_workspace_status.
constexpr int kStatusSubtreeEnd = 1;  // a subtree end outside (i, T] was clamped
__global__ __launch_bounds__(64) void status_reset_kernel(int* __restrict__ status) {
  if (threadIdx.x == 0) *status = 0;
}

// cos / sin of the RoPE angle of position p for rotation pair k (dims k and
// k + D/2): angle = p * theta^(-2k/D), formed and reduced in float64, then
// evaluated in float32 on [-pi, pi]. theta <= 0: no rotation. Shared by the
// prep, the gateway export and the gateway relay, so all rotate bitwise alike.
__device__ __forceinline__ float2 rope_cs(int p, int k, int D, float theta) {
  float c = 1.0f, s = 0.0f;
  if (theta > 0.0f) {
    const double inv = exp2(-2.0 * (double)k / (double)D * log2((double)theta));
    const double ang = (double)p * inv;
    const double twopi = 6.283185307179586476925286766559;
    const double r = ang - rint(ang / twopi) * twopi;
    sincosf((float)r, &s, &c);
  }
  return make_float2(c, s);
}
// (x1, x2) -> R (x1, x2) and its transpose, with explicit fused multiply-adds
// so every kernel rounds alike
__device__ __forceinline__ void rope_rot(float x1, float x2, float2 cs, float& y1, float& y2) {
  y1 = fmaf(x1, cs.x, -x2 * cs.y);
  y2 = fmaf(x2, cs.x, x1 * cs.y);
}
__device__ __forceinline__ void rope_rot_t(float g1, float g2, float2 cs, float& y1, float& y2) {
  y1 = fmaf(g1, cs.x, g2 * cs.y);
  y2 = fmaf(g2, cs.x, -g1 * cs.y);
}

template <typename Tin>
__global__ __launch_bounds__(256) void rope_prep_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                                                        const Tin* __restrict__ v, const int* __restrict__ pos,
                                                        const int* __restrict__ se, const Tin* __restrict__ k_past,
                                                        const Tin* __restrict__ v_past,
                                                        const unsigned char* __restrict__ past_vis, int Lp, int Lq,
                                                        int pos_offset, int T, int Tp, int Hq, int Hkv, int D,
                                                        int DP, float theta, bf16* __restrict__ qr,
                                                        bf16* __restrict__ kr, bf16* __restrict__ vr,
                                                        int* __restrict__ sep, float2* __restrict__ cs,
                                                        int* __restrict__ status) {
  // Row t of the combined sequence (T = Lq + own tokens, padded to Tp):
  //   t <  Lp        a cached row: key and value copied as given (the key is
  //                  already rotated), no query; visible to every own query
  //                  (subtree end T) when past_vis[t], else to none (t)
  //   Lp <= t < Lq   padding: zeros, visible to none
  //   Lq <= t < T    own token i = t - Lq at position pos_offset + pos[i]
  //   t >= T         padding
  __shared__ float2 tab[64];
  const int t = blockIdx.x;
  const int half = D / 2;
  const bool own = t >= Lq && t < T;
  const int i = t - Lq;
  if ((int)threadIdx.x < half) {
    const float2 c = own ? rope_cs(pos_offset + pos[i], threadIdx.x, D, theta) : make_float2(1.0f, 0.0f);
    tab[threadIdx.x] = c;
    cs[(size_t)t * half + threadIdx.x] = c;
  }
  if (threadIdx.x == 0) {
    int e = 0;
    if (own) {
      // a subtree end lies in (i, number of own tokens]; any other value is
      // clamped into that range (and reported in the status word), so every
      // tile bound derived from it stays inside the workspace and every row
      // sees at least itself
      const int raw = se[i];
      const int c = min(max(raw, i + 1), T - Lq);
      if (c != raw) atomicOr(status, kStatusSubtreeEnd);
      e = c + Lq;
    } else if (t < Lp)
      e = past_vis[t] ? T : t;
    else if (t < Lq)
      e = t;
    sep[t] = e;
  }
  __syncthreads();
  const int H = Hq + 2 * Hkv;
  const int nc = half / 8;  // 8-element chunks per half row
  for (int idx = threadIdx.x; idx < H * nc; idx += blockDim.x) {
    const int h = idx / nc;
    const int kk = 8 * (idx % nc);
    const Tin* src = nullptr;
    bf16* dst;
    bool rotate = own;
    if (h < Hq) {
      if (own) src = q + ((size_t)i * Hq + h) * D;
      dst = qr + ((size_t)h * Tp + t) * DP;
    } else if (h < Hq + Hkv) {
      const int hk = h - Hq;
      if (own)
        src = k + ((size_t)i * Hkv + hk) * D;
      else if (t < Lp)
        src = k_past + ((size_t)t * Hkv + hk) * D;
      dst = kr + ((size_t)hk * Tp + t) * DP;
    } else {
      const int hk = h - Hq - Hkv;
      if (own)
        src = v + ((size_t)i * Hkv + hk) * D;
      else if (t < Lp)
        src = v_past + ((size_t)t * Hkv + hk) * D;
      dst = vr + ((size_t)hk * Tp + t) * DP;
      rotate = false;
    }
    float x1[8], x2[8];
    if (src) {
      load8f(src + kk, x1);
      load8f(src + kk + half, x2);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x1[e] = x2[e] = 0.0f;
    }
    bf16x8 y1, y2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (rotate) {
        float r1, r2;
        rope_rot(x1[e], x2[e], tab[kk + e], r1, r2);
        y1[e] = (bf16)r1;
        y2[e] = (bf16)r2;
      } else {
        y1[e] = (bf16)x1[e];
        y2[e] = (bf16)x2[e];
      }
    }
    *reinterpret_cast<bf16x8*>(dst + kk) = y1;
    *reinterpret_cast<bf16x8*>(dst + kk + half) = y2;
    // DP > D only for D = 16: columns D..DP-1 are zero padding
    if (DP > D && kk == 0) {
      *reinterpret_cast<bf16x8*>(dst + D) = zero8();
      *reinterpret_cast<bf16x8*>(dst + D + 8) = zero8();
    }
  }
}

// Per key tile: min and max subtree end (keys past T count as 0), for the
// 64-key tiles of the forward / dQ pass and the 128-key tiles of the dK/dV
// pass, whose work (the number of 64-row query blocks from row Lq on it can
// see) is also recorded.
__device__ __forceinline__ int2 wave_minmax(int2 m) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    m.x = min(m.x, __shfl_xor(m.x, o));
    m.y = max(m.y, __shfl_xor(m.y, o));
  }
  return m;
}
// One wave per 128-key tile (and its two 64-key halves); subtree ends past T
// count as 0, so a tile holding the end of the sequence is never "full".
__global__ __launch_bounds__(256) void tile_minmax_kernel(const int* __restrict__ se, int T, int Lq, int nk64,
                                                          int nk128, int2* __restrict__ kmm64,
                                                          int2* __restrict__ kmm128, int* __restrict__ work) {
  const int kt = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (kt >= nk128) return;
  const int lane = threadIdx.x & 63;
  const int ja = kt * kBwdBK + lane, jb = ja + kFwdBK;
  const int sa = ja < T ? se[ja] : 0, sb = jb < T ? se[jb] : 0;
  const int2 ma = wave_minmax(make_int2(sa, sa)), mb = wave_minmax(make_int2(sb, sb));
  if (lane == 0) {
    kmm64[2 * kt] = ma;
    if (2 * kt + 1 < nk64) kmm64[2 * kt + 1] = mb;
    const int2 m = make_int2(min(ma.x, mb.x), max(ma.y, mb.y));
    kmm128[kt] = m;
    work[kt] = max((m.y + kBwdBQ - 1) / kBwdBQ - max(kt * kBwdBK, Lq) / kBwdBQ, 0);  // queries start at Lq
  }
}

// Superblocks of kSbTiles key tiles (4096 keys): the largest subtree end of
// each, so the list builder skips 64 empty key tiles with one comparison.
constexpr int kSbTiles = 64;
constexpr int kListCap = 256;  // entries of one round of a workgroup's tile list
// One wave per superblock.
__global__ __launch_bounds__(256) void sb_max_kernel(const int2* __restrict__ kmm64, int nk64, int nsb,
                                                     int* __restrict__ sbmax) {
  const int sb = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (sb >= nsb) return;
  const int lane = threadIdx.x & 63;
  const int kt = sb * kSbTiles + lane;
  int m = kt < nk64 ? kmm64[kt].y : 0;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = max(m, __shfl_xor(m, o));
  if (lane == 0) sbmax[sb] = m;
}

// The non-empty key tiles of query rows [i0, i1), ascending from tile
// `resume` on, written by one wave as entries 2 * tile + full into list
// (at most kListCap). Keys of tile kt cover [j0, max se) without gaps (every
// key's interval starts inside the tile), so the tile meets the rows iff
// j0 <= i1 - 1 (kt < nkc) and max se > i0; it is full iff j1 - 1 <= i0 and
// min se >= i1. (Cached rows visible to all queries span [j, T) and masked
// ones nothing, so for the query rows, which start at Lq after all cached
// rows, the same test holds.) Returns the number of entries; resume becomes
// the tile to continue from (nkc when the list is complete). Empty
// superblocks cost one comparison, so the work is O(nkc / 4096 + entries).
__device__ __forceinline__ int build_tile_list(const int2* __restrict__ kmm, const int* __restrict__ sbmax, int i0,
                                               int i1, int nkc, int& resume, int* list, int lane) {
  const int nsb = (nkc + kSbTiles - 1) / kSbTiles;
  int n = 0;
  int kt = resume;
  while (kt < nkc && n < kListCap) {
    int sb = kt / kSbTiles;
    const uint64_t smask = __ballot(sb + lane < nsb && sbmax[sb + lane] > i0);
    if (smask == 0) {
      kt = (sb + 64) * kSbTiles;
      continue;
    }
    sb += __builtin_ctzll(smask);
    kt = max(kt, sb * kSbTiles);
    const int t = sb * kSbTiles + lane;
    bool ne = false;
    int full = 0;
    if (t >= kt && t < nkc) {
      const int2 m = kmm[t];
      ne = m.y > i0;
      full = (t * kFwdBK + kFwdBK - 1 <= i0) && (m.x >= i1);
    }
    const uint64_t mask = __ballot(ne);
    const int off = n + __popcll(mask & ((1ull << lane) - 1ull));
    if (ne && off < kListCap) list[off] = 2 * t + full;
    const int total = n + __popcll(mask);
    kt = (sb + 1) * kSbTiles;
    if (total > kListCap) {
      // the first tile that did not fit is where the next round starts
      const uint64_t first_out = __ballot(ne && off == kListCap);
      kt = sb * kSbTiles + __builtin_ctzll(first_out);
      n = kListCap;
      break;
    }
    n = total;
  }
  resume = min(kt, nkc);
  return n;
}

// One wave per query tile: how many key tiles the forward and dQ passes
// visit for it (the lists build_tile_list gives them) and how many of those
// are full; the counts order the query tiles and are what
// tree_attn_plan_counts reports.
__global__ __launch_bounds__(64) void q_count_kernel(const int2* __restrict__ kmm, const int* __restrict__ sbmax,
                                                     int T, int Lq, int nk, int* __restrict__ counts,
                                                     int* __restrict__ fulls) {
  __shared__ int list[kListCap];
  const int qt = blockIdx.x;
  const int lane = threadIdx.x;
  const int i0 = qt * kFwdBQ;
  if (i0 < Lq || i0 >= T) {  // rows before Lq (cached keys) and padding rows have no queries
    if (lane == 0) counts[qt] = fulls[qt] = 0;
    return;
  }
  const int i1 = min(i0 + kFwdBQ, T);
  const int nkc = min(nk, (i1 - 1) / kFwdBK + 1);
  int resume = 0, n = 0, nf = 0;
  while (resume < nkc) {
    const int m = build_tile_list(kmm, sbmax, i0, i1, nkc, resume, list, lane);
    for (int e = lane; e < m; e += 64) nf += list[e] & 1;
    n += m;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) nf += __shfl_xor(nf, o);
  if (lane == 0) {
    counts[qt] = n;
    fulls[qt] = nf;
  }
}

// Tile indices sorted by work, heaviest first (counting sort on the work
// clipped to 1023). The order within one work value is arbitrary; it only
// affects scheduling, never results.
// Run by one workgroup of 1024 threads.
__device__ __forceinline__ void order_tiles(const int* __restrict__ work, int n, int* __restrict__ order) {
  __shared__ int hist[1024];
  __shared__ int scan[1024];
  const int t = threadIdx.x;
  hist[t] = 0;
  __syncthreads();
  for (int i = t; i < n; i += blockDim.x) atomicAdd(&hist[min(work[i], 1023)], 1);
  __syncthreads();
  // start of each bin, heaviest bin first: an inclusive scan over bins in
  // descending order (thread t holds bin 1023 - t), made exclusive
  const int cnt = hist[1023 - t];
  int v = cnt;
  for (int o = 1; o < 1024; o <<= 1) {
    scan[t] = v;
    __syncthreads();
    if (t >= o) v += scan[t - o];
    __syncthreads();
  }
  hist[1023 - t] = v - cnt;
  __syncthreads();
  for (int i = t; i < n; i += blockDim.x) order[atomicAdd(&hist[min(work[i], 1023)], 1)] = i;
}

// dK/dV work split. The work of a 128-key tile is W = G * (its query blocks)
// iterations of one workgroup. In a tree the root's keys see every query
// below them, so a few tiles can carry many times the average and, as single
// workgroups, finish long after the rest. Let total be the sum of W over the
// tiles of one kv head and C = max(ceil(total / kDkdvSlots), kMinChunk),
// kDkdvSlots being the dK/dV workgroups one XCD holds at a time (32 CUs x 1):
// a tile with W > C is cut into S = ceil(W / C) chunks of consecutive
// iterations, every other tile is one chunk. Each chunk of a cut tile writes
// its float32 dK / dV accumulators to a partial-sum slot of its own; a second
// kernel adds the S slots of each cut tile in slot order (the same order on
// every run) and writes the tile's gradients as an uncut tile does.
// Bounds: sum over cut tiles of (S - 1) < total / C <= kDkdvSlots, so there
// are fewer than nk128 + kDkdvSlots chunks; a cut tile has W >= C + 1, so
// fewer than kDkdvSlots tiles are cut and they use fewer than
// 2 * kDkdvSlots slots.
constexpr int kDkdvSlots = 32;
constexpr int kMinChunk = 64;  // a chunk's fixed cost (operand loads, epilogue) is a few iterations
constexpr int kSplitSlots = 2 * kDkdvSlots;

__device__ __forceinline__ int chunk_count(int W, int C) { return W > C ? (W + C - 1) / C : 1; }

// Run by one workgroup of 1024 threads. Lists the chunks heaviest first (counting sort on the
// chunk size relative to C, 1024 bins): cdesc[c] = {tile, index s within the
// tile, S, first slot of the tile (-1 when S = 1)}, then {-1, 0, 0, 0} up to
// ncmax; and the cut tiles, ktcut[i] = {tile, S, first slot, 0}, then
// {-1, 0, 0, 0} up to kDkdvSlots. korder is scratch (nk ints).
__device__ __forceinline__ void chunk_plan(const int* __restrict__ work, int nk, int G, int* __restrict__ korder,
                                           int4* __restrict__ cdesc, int ncmax, int4* __restrict__ ktcut) {
  __shared__ int hist[1024];
  __shared__ int scan[1024];
  __shared__ long long part[16];
  __shared__ int4 sums[1024];
  const int t = threadIdx.x;
  long long s = 0;
  for (int i = t; i < nk; i += blockDim.x) s += (long long)G * work[i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if ((t & 63) == 0) part[t >> 6] = s;
  hist[t] = 0;
  __syncthreads();
  long long total = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) total += part[i];
  // W <= 256 * 2^16 (heads x query blocks), so C fits an int once clipped there
  const int C = (int)min(max((total + kDkdvSlots - 1) / kDkdvSlots, (long long)kMinChunk), (long long)(1 << 25));
  auto bin_of = [&](int i) {
    const int W = G * work[i];
    const int S = chunk_count(W, C);
    return (int)((long long)((W + S - 1) / S) * 1023 / C);
  };
  for (int i = t; i < nk; i += blockDim.x) atomicAdd(&hist[bin_of(i)], 1);
  __syncthreads();
  const int cnt = hist[1023 - t];
  int v = cnt;
  for (int o = 1; o < 1024; o <<= 1) {
    scan[t] = v;
    __syncthreads();
    if (t >= o) v += scan[t - o];
    __syncthreads();
  }
  hist[1023 - t] = v - cnt;
  __syncthreads();
  for (int i = t; i < nk; i += blockDim.x) korder[atomicAdd(&hist[bin_of(i)], 1)] = i;
  __syncthreads();
  // chunks, slots and cut tiles before each position of the order: thread t
  // owns the positions [p0, p1)
  const int per = (nk + 1023) / 1024;
  const int p0 = min(t * per, nk), p1 = min(p0 + per, nk);
  int4 mine = make_int4(0, 0, 0, 0);
  for (int p = p0; p < p1; ++p) {
    const int S = chunk_count(G * work[korder[p]], C);
    mine.x += S;
    mine.y += S > 1 ? S : 0;
    mine.z += S > 1 ? 1 : 0;
  }
  int4 acc = mine;
  for (int o = 1; o < 1024; o <<= 1) {
    sums[t] = acc;
    __syncthreads();
    if (t >= o) {
      acc.x += sums[t - o].x;
      acc.y += sums[t - o].y;
      acc.z += sums[t - o].z;
    }
    __syncthreads();
  }
  int c = acc.x - mine.x, slot = acc.y - mine.y, ci = acc.z - mine.z;
  for (int p = p0; p < p1; ++p) {
    const int kt = korder[p];
    const int S = chunk_count(G * work[kt], C);
    // running out of slots or cut-tile entries is not reached (see the
    // bounds above); the tile would then be one chunk and its other
    // positions idle
    const bool cut = S > 1 && slot + S <= kSplitSlots && ci < kDkdvSlots;
    for (int q = 0; q < S && c < ncmax; ++q, ++c)
      cdesc[c] = cut ? make_int4(kt, q, S, slot) : (q == 0 ? make_int4(kt, 0, 1, -1) : make_int4(-1, 0, 0, 0));
    if (S > 1) {
      if (ci < kDkdvSlots) ktcut[ci] = cut ? make_int4(kt, S, slot, 0) : make_int4(-1, 0, 0, 0);
      slot += S;
      ++ci;
    }
  }
  if (t == 1023) sums[0] = acc;
  __syncthreads();
  for (int i = sums[0].x + t; i < ncmax; i += blockDim.x) cdesc[i] = make_int4(-1, 0, 0, 0);
  for (int i = sums[0].z + t; i < kDkdvSlots; i += blockDim.x) ktcut[i] = make_int4(-1, 0, 0, 0);
}

// Workgroup 0 orders the query tiles for the forward and dQ passes,
// workgroup 1 plans the dK/dV chunks.
__global__ __launch_bounds__(1024) void order_kernel(const int* __restrict__ qcount, int nq, int* __restrict__ qorder,
                                                     const int* __restrict__ kwork, int nk, int G,
                                                     int* __restrict__ korder, int4* __restrict__ cdesc, int ncmax,
                                                     int4* __restrict__ ktcut) {
  if (blockIdx.x == 0)
    order_tiles(qcount, nq, qorder);
  else
    chunk_plan(kwork, nk, G, korder, cdesc, ncmax, ktcut);
}

// Stores 8 floats as elements [0, 8) of a caller row (one 16- or 32-byte
// store; the row start is 16-byte aligned).
__device__ __forceinline__ void store_row8(bf16* p, const float* f) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)f[e];
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void store_row8(float* p, const float* f) {
  *reinterpret_cast<f32x4*>(p) = f32x4{f[0], f[1], f[2], f[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
}

// Loads 8 elements [c, c+8) of a caller row; zero past the row end or for
// rows past T.
template <typename Tio>
__device__ __forceinline__ bf16x8 load_row8(const Tio* rowp, bool row_ok, int c, int D) {
  return (row_ok && c < D) ? load8(rowp + c) : zero8();
}

// ------------------------------------------------------------------------
// Forward. One workgroup = 128 query rows of one head (kFwdWaves waves x
// kNB 32-row column blocks), looping over the query tile's non-empty 64-key
// tiles. With kNB = 2 every K' / V operand read from LDS would feed two MFMAs,
// but one wave per SIMD then hides too little latency; 4 waves x 32 rows at
// two waves per SIMD is faster on gfx950.
//
// LDS: the K' tile (read only as 16-byte operands) uses rows padded to DP + 8
// elements, which is conflict-free and keeps every read address an immediate
// offset from one per-lane base; the V tile (read only transposed) uses the
// XOR swizzle, whose 8 distinct per-lane bases are computed once.
constexpr int kFwdWaves = TA_FWD_WAVES;
constexpr int kNB = 1;  // 32-query column blocks per wave
constexpr int kFwdRows = 32 * kNB * kFwdWaves;  // query rows per forward workgroup

struct FwdState {
  float mref, lsum;
};

// DMA of one padded 64-row tile (row stride DP + 8): a flat copy of
// 64 * (DP/8 + 1) 16-byte positions; a padding position copies any valid chunk.
template <int DP, bool PERM, int NW>
struct PadTileDma {
  static constexpr int RC = DP / 8 + 1;                // 16-byte positions per padded row
  static constexpr int NINS = RC;                      // 64 * RC positions / 64 lanes
  static constexpr int NI = (NINS + NW - 1) / NW;      // instructions per wave (last may be partial)
  int off[NI];
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int p = (w + NW * j) * 64 + lane;
      const int r = min(p / RC, 63);
      const int c = p % RC;
      off[j] = (PERM ? perm_row(r) : r) * DP + (c < DP / 8 ? 8 * c : 0);
    }
  }
  __device__ __forceinline__ void issue(const bf16* rows, bf16* tile, int w) const {
#pragma unroll
    for (int j = 0; j < NI; ++j)
      if (w + NW * j < NINS) dma16(rows + off[j], tile + (w + NW * j) * 512);
  }
};

template <int DP>
struct FwdAddr {
  int k;          // element offset of this lane's first K' operand in a padded tile
  int v[2][DP / 32];  // element offsets of the transposed V reads, per (half, d block), t = 0
};

template <int DP>
__device__ __forceinline__ void fwd_issue(const PadTileDma<DP, true, kFwdWaves>& kd,
                                          const TileDma<DP, false, kFwdWaves>& vd, const bf16* kg, const bf16* vg,
                                          const int* sep, int j0, bf16* kb, bf16* vb, int* sb, int w, int lane) {
  kd.issue(kg + (size_t)j0 * DP, kb, w);
  vd.issue(vg + (size_t)j0 * DP, vb, w);
  if (w == 0) dma4(sep + j0 + lane, sb);
}

// One key tile for both column blocks: S^T = K' Q'^T, mask, lazy-rescaled
// online softmax, O^T += V^T P^T.
template <int DP>
__device__ __forceinline__ void fwd_tile(const bf16* kb, const bf16* vb, const int* sb, bool full, int j0,
                                         const int* qrow, int lg, const FwdAddr<DP>& ad, float sl2,
                                         const bf16x8 (*qop)[DP / 16], f32x16 (*acc)[DP / 32], FwdState* st) {
  constexpr int KS = DP / 16;
  constexpr int NDB = DP / 32;
  constexpr int SKP = DP + 8;
  sched_hint();
  f32x16 s[2][kNB];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) s[mb][nb] = f32x16{};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const bf16x8 a = lds128(kb + ad.k + 32 * mb * SKP + 16 * k);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) s[mb][nb] = mfma32x32x16(a, qop[nb][k], s[mb][nb]);
    }
  }
  lds_ahead<TA_LA_FWD, 2 * KS * kNB, 2 * KS>();
  if (!full) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int kk0 = 32 * mb + 16 * (q4 >> 1) + 8 * lg + 4 * (q4 & 1);
        const int4 s4 = *reinterpret_cast<const int4*>(sb + kk0);
        const int sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int nb = 0; nb < kNB; ++nb) {
            const bool vis = (j0 + kk0 + b <= qrow[nb]) & (qrow[nb] < sv[b]);
            s[mb][nb][4 * q4 + b] = vis ? s[mb][nb][4 * q4 + b] : kNegInf;
          }
      }
  }
  bf16x8 pb[kNB][4];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    float mx = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[mb][nb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mt2 = mx * sl2;
    if (__any(mt2 > st[nb].mref + kRescaleLog2)) {
      const float mnew = fmaxf(st[nb].mref, mt2);
      const float alpha = (st[nb].mref == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(st[nb].mref - mnew);
      st[nb].mref = mnew;
      st[nb].lsum *= alpha;
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nb][b][i] *= alpha;
    }
    const float nmu = (st[nb].mref == kNegInf) ? 0.0f : -st[nb].mref;
    float ps = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[mb][nb][i], sl2, nmu));
        ps += p;
        pb[nb][2 * mb + (i >> 3)][i & 7] = (bf16)p;
      }
    st[nb].lsum += ps;
  }
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // rows 16t + 8lg + (lane%16)/4 (+4): the 16t part only moves whole rows
      const bf16x8 a = cat(lds_read_tr(vb + ad.v[0][b] + 16 * t * DP), lds_read_tr(vb + ad.v[1][b] + 16 * t * DP));
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[nb][b] = mfma32x32x16(a, pb[nb][t], acc[nb][b]);
    }
}

template <int DP, typename Tio>
__global__ __launch_bounds__(64 * kFwdWaves, 8 / kFwdWaves) void attn_fwd_kernel(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ vr,
    const int* __restrict__ sep, const int2* __restrict__ kmm, const int* __restrict__ sbmax,
    const int* __restrict__ order, int T, int Lq, int Tp, int Hq, int Hkv, int nq, int nk, float sl2,
    Tio* __restrict__ o, float* __restrict__ lse) {
  // Row indices are those of the combined sequence: Lq cached / padding rows
  // (keys only, no queries) and then the packed tokens; T = Lq + own tokens.
  constexpr int D = DP == 32 ? 16 : DP;  // head dim (16 is padded to 32 for the MFMA shapes)
  constexpr int KS = DP / 16;            // k steps of S^T = K' Q'^T
  constexpr int NDB = DP / 32;           // 32-wide d blocks of O^T
  constexpr int TILE = 64 * DP;
  constexpr int KTILE = 64 * (DP + 8);
  // two buffers per operand as separate objects, so the compiler can tell
  // the tile being computed from the one being loaded
  __shared__ __attribute__((aligned(1024))) bf16 kb0[KTILE];
  __shared__ __attribute__((aligned(1024))) bf16 kb1[KTILE];
  __shared__ __attribute__((aligned(1024))) bf16 vb0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vb1[TILE];
  __shared__ __attribute__((aligned(256))) int sb0[64];
  __shared__ __attribute__((aligned(256))) int sb1[64];
  __shared__ int lst[kListCap + 2];  // this round's key tiles, their count, the next round's start

  const int G = Hq / Hkv;
  // kv-head-major: consecutive workgroups (one XCD's share) work on one kv
  // head, the G query heads of a query tile side by side, so K' / V tiles
  // are reused from that XCD's L2; query tiles in heaviest-first order
  const int lid = xcd_remap(blockIdx.x, nq * Hq);
  const int gq = lid % G;
  const int hk = lid / (G * nq);
  const int qt = order[(lid / G) % nq];
  const int h = hk * G + gq;
  if (qt * kFwdRows < Lq || qt * kFwdRows >= T) return;  // cached rows or padding: no queries

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  int qrow[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) qrow[nb] = qt * kFwdRows + 32 * kNB * w + 32 * nb + lc;
  PadTileDma<DP, true, kFwdWaves> kd;
  TileDma<DP, false, kFwdWaves> vd;
  kd.init(w, lane);
  vd.init(w, lane);
  FwdAddr<DP> ad;
  ad.k = lc * (DP + 8) + 8 * lg;
#pragma unroll
  for (int hi = 0; hi < 2; ++hi)
#pragma unroll
    for (int b = 0; b < NDB; ++b)
      ad.v[hi][b] = toff<DP>(8 * lg + ((lane & 15) >> 2) + 4 * hi, 32 * b + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  bf16x8 qop[kNB][KS];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const bf16* qb = qr + ((size_t)h * Tp + qrow[nb]) * DP + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) qop[nb][s] = load8(qb + 16 * s);
  }
  f32x16 acc[kNB][NDB];
  FwdState st[kNB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    st[nb] = FwdState{kNegInf, 0.0f};
#pragma unroll
    for (int b = 0; b < NDB; ++b) acc[nb][b] = f32x16{};
  }

  const bf16* kg = kr + (size_t)hk * Tp * DP;
  const bf16* vg = vr + (size_t)hk * Tp * DP;
  // The Q' operands are waited for before the loop: the compiler does not see
  // the tile copies (inline assembly), and a wait for these loads placed at
  // their first use inside the loop would also drain the copies in flight.
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(qop[nb][s]));

  // this wave's own rows [r0, r1): a key tile can be empty or full for them
  // even when it is partial for the whole query tile
  const int r0 = qt * kFwdRows + 32 * kNB * w;
  const int r1 = min(r0 + 32 * kNB, T);
  auto wave_tile = [&](int e, const bf16* kb, const bf16* vb, const int* sb) {
    const int kt = e >> 1;
    const int j0 = kt * kFwdBK;
    const int2 m = kmm[kt];
    if (r0 >= r1 || j0 > r1 - 1 || m.y <= r0) return;  // nothing visible to this wave
    const bool full = (e & 1) || ((j0 + kFwdBK - 1 <= r0) && (m.x >= r1));
    fwd_tile<DP>(kb, vb, sb, full, j0, qrow, lg, ad, sl2, qop, acc, st);
  };
  // the query tile's non-empty key tiles, kListCap per round
  const int i0 = qt * kFwdRows, i1 = min(i0 + kFwdRows, T);
  const int nkc = min(nk, (i1 - 1) / kFwdBK + 1);
  int resume = 0;
  for (;;) {
    if (w == 0) {
      const int n = build_tile_list(kmm, sbmax, i0, i1, nkc, resume, lst, lane);
      if (lane == 0) {
        lst[kListCap] = n;
        lst[kListCap + 1] = resume;
      }
    }
    __syncthreads();
    const int cnt = lst[kListCap];
    resume = lst[kListCap + 1];
    if (cnt > 0) fwd_issue<DP>(kd, vd, kg, vg, sep, (lst[0] >> 1) * kFwdBK, kb0, vb0, sb0, w, lane);
    for (int it = 0; it < cnt; it += 2) {
      {
        const int e = lst[it];
        wait_dma();
        __syncthreads();
        if (it + 1 < cnt) fwd_issue<DP>(kd, vd, kg, vg, sep, (lst[it + 1] >> 1) * kFwdBK, kb1, vb1, sb1, w, lane);
        wave_tile(e, kb0, vb0, sb0);
      }
      if (it + 1 < cnt) {
        const int e = lst[it + 1];
        wait_dma();
        __syncthreads();
        if (it + 2 < cnt) fwd_issue<DP>(kd, vd, kg, vg, sep, (lst[it + 2] >> 1) * kFwdBK, kb0, vb0, sb0, w, lane);
        wave_tile(e, kb1, vb1, sb1);
      }
    }
    if (resume >= nkc) break;
    __syncthreads();  // every wave is done with this round's list and tiles
  }

#pragma unroll
  for (int nb = 0; nb < kNB; ++nb) {
    const float lt = st[nb].lsum + __shfl_xor(st[nb].lsum, 32);
    if (qrow[nb] < T) {
      const float inv = 1.0f / lt;
      Tio* orow = o + ((size_t)(qrow[nb] - Lq) * Hq + h) * D;
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int d = 32 * b + 8 * (i >> 2) + 4 * lg + (i & 3);
          if (d < D) orow[d] = from_f32<Tio>(acc[nb][b][i] * inv);
        }
      const float mu = (st[nb].mref == kNegInf) ? 0.0f : st[nb].mref;
      if (lg == 0) lse[(size_t)h * (T - Lq) + (qrow[nb] - Lq)] = (mu + log2f(lt)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------------
// Backward dQ. Same shape as the forward: a workgroup owns 128 query rows of
// one head and loops over their non-empty key tiles.
//   S^T = K' Q'^T,  P^T = exp2(S^T * scale*log2e - lse*log2e)
//   dP^T = V dO^T,  dS^T = P^T (dP^T - D)
//   dQ'^T += K'^T dS^T  (A operand read transposed from the K' tile)
// then dQ = R(pos)^T * scale * dQ'. Before the loop it forms
// D_i = dO_i . O_i from the dO registers it holds anyway, and stores D,
// lse * log2(e) and a bf16 head-major copy of dO for the dK/dV kernel.
template <int DP>
__device__ __forceinline__ void dq_tile(const bf16* kb, const bf16* vb, const int* sb, bool full, int j0, int qrow,
                                        int lg, const SwzAddr<DP>& ad, float sl2, float lse2, float dval,
                                        const bf16x8* qop, const bf16x8* dop, f32x16* acc) {
  constexpr int KS = DP / 16;
  constexpr int NDB = DP / 32;
  sched_hint();
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const int off = ad.op[k] + 32 * mb * DP;
      s = mfma32x32x16(lds128(kb + off), qop[k], s);
      dp = mfma32x32x16(lds128(vb + off), dop[k], dp);
    }
    lds_ahead<TA_LA_DQ, 2 * KS, 2 * KS>();
    bf16x8 db8[2];
    if (full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -lse2));
        db8[i >> 3][i & 7] = (bf16)(p * (dp[i] - dval));
      }
    } else {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int kk0 = 32 * mb + 16 * (q4 >> 1) + 8 * lg + 4 * (q4 & 1);
        const int4 s4 = *reinterpret_cast<const int4*>(sb + kk0);
        const int sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * q4 + b;
          const bool vis = (j0 + kk0 + b <= qrow) & (qrow < sv[b]);
          const float p = vis ? __builtin_amdgcn_exp2f(fmaf(s[i], sl2, -lse2)) : 0.0f;
          db8[i >> 3][i & 7] = (bf16)(p * (dp[i] - dval));
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        // K'^T operand: rows d = 32b + lane%32, k slots = keys 32mb + 16t2 + 8lg + s
        const int r0 = (32 * mb + 16 * t2) * DP;
        const bf16x8 a = cat(lds_read_tr(kb + ad.tr[b] + r0), lds_read_tr(kb + ad.tr[b] + r0 + 8 * DP));
        acc[b] = mfma32x32x16(a, db8[t2], acc[b]);
      }
    lds_ahead<TA_LA_DQ, 2 * NDB, 4 * NDB>();
  }
}

template <int DP, typename Tio>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ vr,
    const Tio* __restrict__ o, const Tio* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ dd, float* __restrict__ l2, bf16* __restrict__ dor, const int* __restrict__ sep,
    const int2* __restrict__ kmm, const int* __restrict__ sbmax, const int* __restrict__ order,
    const float2* __restrict__ cs, int T, int Lq, int Tp, int Hq, int Hkv, int nq, int nk, float sl2, float scale,
    Tio* __restrict__ dq) {
  // Row indices are those of the combined sequence (Lq cached / padding
  // rows, then the packed tokens; T = Lq + own tokens). o, dout, lse and dq
  // hold the own rows only.
  constexpr int D = DP == 32 ? 16 : DP;
  constexpr int KS = DP / 16;
  constexpr int NDB = DP / 32;
  constexpr int TILE = 64 * DP;
  __shared__ __attribute__((aligned(1024))) bf16 kb0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 kb1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vb0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 vb1[TILE];
  __shared__ __attribute__((aligned(256))) int sb0[64];
  __shared__ __attribute__((aligned(256))) int sb1[64];
  __shared__ int lst[kListCap + 2];  // this round's key tiles, their count, the next round's start

  const int G = Hq / Hkv;
  // kv-head-major: consecutive workgroups (one XCD's share) work on one kv
  // head, the G query heads of a query tile side by side, so K' / V tiles
  // are reused from that XCD's L2; query tiles in heaviest-first order
  const int lid = xcd_remap(blockIdx.x, nq * Hq);
  const int gq = lid % G;
  const int hk = lid / (G * nq);
  const int qt = order[(lid / G) % nq];
  const int h = hk * G + gq;
  if (qt * kFwdBQ < Lq) return;  // a tile of cached rows: no queries (Lq is a multiple of the tile)

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  const int qrow = qt * kFwdBQ + 32 * w + lc;
  const bool qok = qrow < T;
  const int own = qrow - Lq;  // row in o, dout, lse and dq
  TileDma<DP, true> td;
  td.init(w, lane);
  SwzAddr<DP> ad;
  ad.init(lane);

  bf16x8 qop[KS], dop[KS];
  float dval = 0.0f;
  {
    // every load of the row is issued before any is used
    const bf16* qb = qr + ((size_t)h * Tp + qrow) * DP + 8 * lg;
    bf16* dob = dor + ((size_t)h * Tp + qrow) * DP + 8 * lg;
    const size_t roff = ((size_t)(qok ? own : 0) * Hq + h) * D;
    bf16x8 ov[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qop[s] = load8(qb + 16 * s);
      dop[s] = load_row8(dout + roff, qok, 16 * s + 8 * lg, D);
      ov[s] = load_row8(o + roff, qok, 16 * s + 8 * lg, D);
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      *reinterpret_cast<bf16x8*>(dob + 16 * s) = dop[s];
#pragma unroll
      for (int e = 0; e < 8; ++e) dval += (float)dop[s][e] * (float)ov[s][e];
    }
  }
  dval += __shfl_xor(dval, 32);
  const float lse_row = qok ? lse[(size_t)h * (T - Lq) + own] : 0.0f;
  const float lse2 = lse_row * kLog2e;
  if (lg == 0) {
    dd[(size_t)h * Tp + qrow] = -dval;
    l2[(size_t)h * Tp + qrow] = qok ? -lse_row / scale : 0.0f;
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) acc[b] = f32x16{};

  const bf16* kg = kr + (size_t)hk * Tp * DP;
  const bf16* vg = vr + (size_t)hk * Tp * DP;
  auto issue = [&](int j, bf16* kb, bf16* vb, int* sb) {
    td.issue(kg + (size_t)j * DP, kb, w);
    td.issue(vg + (size_t)j * DP, vb, w);
    if (w == 0) dma4(sep + j + lane, sb);
  };

  // the query tile's non-empty key tiles, kListCap per round (no rows past T:
  // an empty list)
  const int i0 = qt * kFwdBQ, i1 = min(i0 + kFwdBQ, T);
  const int nkc = i0 < T ? min(nk, (i1 - 1) / kFwdBK + 1) : 0;
  int resume = 0;
  for (;;) {
    if (w == 0) {
      const int n = build_tile_list(kmm, sbmax, i0, i1, nkc, resume, lst, lane);
      if (lane == 0) {
        lst[kListCap] = n;
        lst[kListCap + 1] = resume;
      }
    }
    __syncthreads();
    const int cnt = lst[kListCap];
    resume = lst[kListCap + 1];
    if (cnt > 0) issue((lst[0] >> 1) * kFwdBK, kb0, vb0, sb0);
    for (int it = 0; it < cnt; it += 2) {
      {
        const int e = lst[it];
        wait_dma();
        __syncthreads();
        if (it + 1 < cnt) issue((lst[it + 1] >> 1) * kFwdBK, kb1, vb1, sb1);
        dq_tile<DP>(kb0, vb0, sb0, e & 1, (e >> 1) * kFwdBK, qrow, lg, ad, sl2, lse2, dval, qop, dop, acc);
      }
      if (it + 1 < cnt) {
        const int e = lst[it + 1];
        wait_dma();
        __syncthreads();
        if (it + 2 < cnt) issue((lst[it + 2] >> 1) * kFwdBK, kb0, vb0, sb0);
        dq_tile<DP>(kb1, vb1, sb1, e & 1, (e >> 1) * kFwdBK, qrow, lg, ad, sl2, lse2, dval, qop, dop, acc);
      }
    }
    if (resume >= nkc) break;
    __syncthreads();  // every wave is done with this round's list and tiles
  }

  // Epilogue through LDS. The lane holds dQ'^T column qrow, rows
  // d = 32b + 8(i/4) + 4lg + i%4; per-lane stores of single elements would
  // touch a cache line per lane. Each wave stages its 32 rows scaled, as
  // [d][row] float32, in one tile buffer (the tiles are no longer read), then
  // a lane forms its row's output 8 columns at a time with the RoPE partner
  // d + D/2 (R(pos)^T) and writes 16-byte pieces.
  static_assert(DP * 32 * 4 <= TILE * 2, "a wave's dQ' rows must fit in one tile buffer");
  __syncthreads();
  float* ep = reinterpret_cast<float*>(w < 2 ? (w == 0 ? kb0 : kb1) : (w == 2 ? vb0 : vb1));
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) ep[(32 * b + 8 * (i >> 2) + 4 * lg + (i & 3)) * 32 + lc] = acc[b][i] * scale;
  __syncthreads();
  if (qok) {
    constexpr int half = D / 2;
    constexpr int NP = half / 8;  // 8-column pieces per half row
    const float2* csr = cs + (size_t)qrow * half;
    Tio* out = dq + ((size_t)own * Hq + h) * D;
    for (int c = lg; c < NP; c += 2) {
      const int d0 = 8 * c;
      float o1[8], o2[8];
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        rope_rot_t(ep[(d0 + s2) * 32 + lc], ep[(d0 + half + s2) * 32 + lc], csr[d0 + s2], o1[s2], o2[s2]);
      }
      store_row8(out + d0, o1);
      store_row8(out + d0 + half, o2);
    }
  }
}

// ------------------------------------------------------------------------
// dK / dV epilogue of one 128-key tile, dK (pass 0) then dV (pass 1): the
// waves holding that gradient (m = 1 holds dK', m = 0 dV) stage their 32 x DP
// block in LDS as [key][d] float32, one of the four tile buffers per key
// slice, then all waves write 16 keys each: dK rotated back (R(pos)^T) and
// scaled, cached rows to dk_past / dv_past in float32 (added when acc_past),
// padding rows skipped. Called by all eight waves with the buffers free.
template <int DP, typename Tio>
__device__ __forceinline__ void dkdv_epilogue(const f32x16* acc, bf16* qb0, bf16* qb1, bf16* ob0, bf16* ob1, int j0,
                                              int hk, int T, int Lq, int Lp, int Hkv, float scale,
                                              const float2* __restrict__ cs, Tio* __restrict__ dk,
                                              Tio* __restrict__ dv, float* __restrict__ dk_past,
                                              float* __restrict__ dv_past, int acc_past) {
  constexpr int D = DP == 32 ? 16 : DP;
  constexpr int NDB = DP / 32;
  constexpr int SE = DP;  // f32 row stride: 32 rows x DP floats = one tile buffer
  static_assert(32 * SE * 4 <= 64 * DP * 2, "a key slice's epilogue block must fit in one tile buffer");
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = w & 3, m = w >> 2;
  const int lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  constexpr int half = D / 2;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    if (m == 1 - pass) {
      float* ep = reinterpret_cast<float*>(ks < 2 ? (ks == 0 ? qb0 : qb1) : (ks == 2 ? ob0 : ob1));
      const float mul = pass == 0 ? scale : 1.0f;
#pragma unroll
      for (int b = 0; b < NDB; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 8 * (i >> 2) + 4 * lg + (i & 3);
          ep[r * SE + 32 * b + lc] = acc[b][i] * mul;
        }
    }
    __syncthreads();
    for (int rr = 0; rr < 16; ++rr) {
      const int r = 16 * w + rr;  // key row within the workgroup's 128
      const int j = j0 + r;
      if (j >= T) break;
      if (j >= Lp && j < Lq) continue;  // padding after the cached rows
      const bf16* eb = (r >> 5) < 2 ? ((r >> 5) == 0 ? qb0 : qb1) : ((r >> 5) == 2 ? ob0 : ob1);
      const float* er = reinterpret_cast<const float*>(eb) + (r & 31) * SE;
      if (j < Lp) {
        // cached rows: their keys came in rotated, so dK is left unrotated
        float* out = (pass == 0 ? dk_past : dv_past) + ((size_t)j * Hkv + hk) * D;
        for (int c = lane; c < D; c += 64) out[c] = acc_past ? out[c] + er[c] : er[c];
      } else if (pass == 0) {
        Tio* out = dk + ((size_t)(j - Lq) * Hkv + hk) * D;
        const float2* csr = cs + (size_t)j * half;
        for (int kk = lane; kk < half; kk += 64) {
          float y1, y2;
          rope_rot_t(er[kk], er[kk + half], csr[kk], y1, y2);
          out[kk] = from_f32<Tio>(y1);
          out[kk + half] = from_f32<Tio>(y2);
        }
      } else {
        Tio* out = dv + ((size_t)(j - Lq) * Hkv + hk) * D;
        for (int c = lane; c < D; c += 64) out[c] = from_f32<Tio>(er[c]);
      }
    }
    __syncthreads();
  }
}

// Backward dK / dV. One workgroup owns 128 keys of one kv head and loops over
// the 64-row query blocks those keys can see, for every query head of the
// group. The visible queries of a key tile form the contiguous range
// [j0, max se), so no list is needed.
//   S = Q' K'^T, P = exp2(S*scale*log2e - lse*log2e), dP = dO V^T
//   dS = P (dP - D);  dV += P^T dO;  dK' += dS^T Q'
// Eight waves: key slice ks = w % 4 (32 keys) x role m = w / 4; both waves of
// a slice sit on the same SIMD. The m = 0 wave holds the slice's K' rows,
// computes S and P for all 64 rows and accumulates dV; the m = 1 wave holds
// the V rows, computes dP, takes P (bf16, as the dV product uses it) from
// its partner through LDS, forms dS and accumulates dK. Both run the same
// MFMA sequence on different operands: 32 MFMAs per block, one 32 x DP
// accumulator and one operand set per wave, all in VGPRs. The epilogue
// rotates dK back (R(pos)^T) through an LDS transpose and writes both once;
// no atomics, so results are reproducible.
constexpr int kDkdvWaves = 8;

// role 0: x = S - lse/scale = Q' K'^T + rowv (rowv holds -lse/scale);
// role 1: x = dP - D = dO V^T + rowv (rowv holds -D). The accumulators
// start at the per-row value, read from LDS straight into them.
// C register i of block mb <-> query row 32mb + 16(i/8) + 8lg + 4((i/4)%2) + i%4; lane <-> key.
__device__ __forceinline__ void dkdv_rows(const float* rowv, int lg, f32x16* x) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v = *reinterpret_cast<const float4*>(rowv + 32 * mb + 16 * (q4 >> 1) + 8 * lg + 4 * (q4 & 1));
      x[mb][4 * q4 + 0] = v.x;
      x[mb][4 * q4 + 1] = v.y;
      x[mb][4 * q4 + 2] = v.z;
      x[mb][4 * q4 + 3] = v.w;
    }
}

template <int DP>
__device__ __forceinline__ void dkdv_tile(const bf16* xs, const bf16* ys, f32x16* x, bool full, int m, int rel_lo,
                                          int rel_hi, int lg, const SwzAddr<DP>& ad, float sl2, const bf16x8* op,
                                          bf16x8* xch, f32x16* acc) {
  constexpr int KS = DP / 16;
  constexpr int NDB = DP / 32;
  sched_hint();
  // role 0's products and softmax go first on the SIMD
  if (m == 0) __builtin_amdgcn_s_setprio(2);
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) x[mb] = mfma32x32x16(lds128(xs + ad.op[k] + 32 * mb * DP), op[k], x[mb]);
  lds_ahead<TA_LA_DKDV, 2 * KS, 2 * KS>();
  // a[2 mb + t2] is the A operand (keys x 16 query rows) of the second product.
  bf16x8 a[4];
  if (m == 0) {
    // P = exp2(x * scale * log2(e)); this lane's key sees block rows
    // [rel_lo, rel_hi): row 8lg + c, c a compile-time constant, is compared
    // with the bounds shifted by 8lg
    const int lo8 = rel_lo - 8 * lg, hi8 = rel_hi - 8 * lg;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c0 = 32 * mb + 16 * (q4 >> 1) + 4 * (q4 & 1);
        float p[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) p[b] = __builtin_amdgcn_exp2f(x[mb][4 * q4 + b] * sl2);
        if (!full) {
#pragma unroll
          for (int b = 0; b < 4; ++b) p[b] = ((c0 + b >= lo8) & (c0 + b < hi8)) ? p[b] : 0.0f;
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) a[2 * mb + (q4 >> 1)][4 * (q4 & 1) + b] = (bf16)p[b];
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) xch[64 * j] = a[j];
    // the priority stays raised through the exponentials, which the dP-wave
    // waits for
    __builtin_amdgcn_s_setprio(0);
  }
  // the P hand-over orders LDS only: the next block's copies stay in flight
  // (__syncthreads would wait for them here)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (m == 1) {
    // dS = P (dP - D), P from the partner
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = xch[64 * j];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = 2 * mb + (i >> 3), e = i & 7;
        a[j][e] = (bf16)((float)a[j][e] * x[mb][i]);
      }
  }
  // role 0: dV += P^T dO (ys = dO tile); role 1: dK' += dS^T Q' (ys = Q' tile)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      // natural query rows 32mb + 16t2 + 8lg + s sit in LDS rows
      // 32mb + 16t2 + 4lg + (s / 4) * 8 + s % 4 (perm_row order)
      const int r0 = (32 * mb + 16 * t2) * DP;
#pragma unroll
      for (int b = 0; b < NDB; ++b) {
        const bf16x8 bt = cat(lds_read_tr(ys + ad.tr[b] + r0), lds_read_tr(ys + ad.tr[b] + r0 + 8 * DP));
        acc[b] = mfma32x32x16(a[2 * mb + t2], bt, acc[b]);
      }
    }
  lds_ahead<TA_LA_DKDV, 4 * NDB, 8 * NDB>();
}

template <int DP, typename Tio>
__global__ __launch_bounds__(64 * kDkdvWaves) void attn_bwd_dkdv_kernel(
    const bf16* __restrict__ qr, const bf16* __restrict__ kr, const bf16* __restrict__ vr,
    const bf16* __restrict__ dor, const float* __restrict__ l2, const float* __restrict__ dd,
    const int* __restrict__ sep, const int2* __restrict__ kmm, const int4* __restrict__ cdesc, int ncmax,
    float* __restrict__ kpart, const float2* __restrict__ cs, int T, int Lq, int Lp, int Tp,
    int Hq, int Hkv, float sl2, float scale, Tio* __restrict__ dk, Tio* __restrict__ dv, float* __restrict__ dk_past,
    float* __restrict__ dv_past, int acc_past) {
  // Key rows are those of the combined sequence: Lp cached rows (gradients to
  // dk_past / dv_past in float32, added to their contents when acc_past),
  // padding up to Lq, then the packed tokens (dk, dv); T = Lq + own tokens.
  // Queries exist from row Lq on. A workgroup runs one chunk of the work
  // split (chunk_plan) for one kv head.
  constexpr int BQ = kBwdBQ;
  constexpr int KS = DP / 16;
  constexpr int NDB = DP / 32;
  constexpr int TILE = 64 * DP;
  __shared__ __attribute__((aligned(1024))) bf16 qb0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 qb1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 ob0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 ob1[TILE];
  __shared__ __attribute__((aligned(256))) float lb0[BQ];
  __shared__ __attribute__((aligned(256))) float lb1[BQ];
  __shared__ __attribute__((aligned(256))) float db0[BQ];
  __shared__ __attribute__((aligned(256))) float db1[BQ];
  // P exchange: [key slice][4 operands][lane] 16 bytes
  __shared__ __attribute__((aligned(1024))) bf16x8 xb[4 * 4 * 64];

  const int G = Hq / Hkv;
  const int lid = xcd_remap(blockIdx.x, ncmax * Hkv);
  const int4 cd = cdesc[lid % ncmax];  // {tile, chunk, chunks of the tile, first partial-sum slot}
  const int hk = lid / ncmax;
  if (cd.x < 0) return;  // an unused chunk position (uniform over the workgroup)
  const int kt = cd.x;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ks = w & 3, m = w >> 2;
  const int lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  const int j0 = kt * kBwdBK;
  const int key = j0 + 32 * ks + lc;
  const int myse = sep[key];
  // Only the role-1 waves load query blocks: role 0 is the critical path
  // (its P feeds role 1's dS), so it starts its products right after the
  // barrier instead of waiting behind its share of the load issue.
  TileDma<DP, true, 4> td;
  td.init(w & 3, lane);
  SwzAddr<DP> ad;
  ad.init(lane);
  bf16x8* xch = xb + ks * 256 + lane;

  // role 0 holds K' rows, role 1 V rows, as MFMA B operands
  bf16x8 op[KS];
  {
    const bf16* ob = (m == 0 ? kr : vr) + ((size_t)hk * Tp + key) * DP + 8 * lg;
#pragma unroll
    for (int s = 0; s < KS; ++s) op[s] = load8(ob + 16 * s);
    // waited for here, not at their first use inside the loop, where the
    // wait would also drain the tile copies in flight (the compiler does
    // not see them)
#pragma unroll
    for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(op[s]));
  }
  f32x16 acc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) acc[b] = f32x16{};

  const int2 mm = kmm[kt];
  const int qb_lo = max(j0, Lq) / BQ;
  const int nqb = max((mm.y + BQ - 1) / BQ - qb_lo, 0);
  // this chunk's iterations [it0, n_it) of the tile's G * nqb
  const int it0 = (int)((long long)G * nqb * cd.y / cd.z);
  const int n_it = (int)((long long)G * nqb * (cd.y + 1) / cd.z);

  // iteration it covers query head hk * G + it / nqb, block qb_lo + it % nqb;
  // (hh, qq) track that pair for the block being loaded next
  int hh = nqb > 0 ? it0 / nqb : 0, qq = nqb > 0 ? it0 % nqb : 0;
  auto issue = [&](bf16* qs_, bf16* ds_, float* lsb, float* dlb) {
    const int h = hk * G + hh;
    const int i0 = (qb_lo + qq) * BQ;
    if (m == 1) {
      td.issue(qr + ((size_t)h * Tp + i0) * DP, qs_, w & 3);
      td.issue(dor + ((size_t)h * Tp + i0) * DP, ds_, w & 3);
      if (w == 4) dma4(l2 + (size_t)h * Tp + i0 + lane, lsb);
      if (w == 5) dma4(dd + (size_t)h * Tp + i0 + lane, dlb);
    }
    if (++qq == nqb) {
      qq = 0;
      ++hh;
    }
  };
  auto tile = [&](int cq, const bf16* qs_, const bf16* ds_, f32x16* x) {
    const int i0 = (qb_lo + cq) * BQ;
    const bool full = (j0 + kBwdBK - 1 <= i0) && (mm.x >= min(i0 + BQ, T));
    dkdv_tile<DP>(m == 0 ? qs_ : ds_, m == 0 ? ds_ : qs_, x, full, m, key - i0, myse - i0, lg, ad, sl2, op, xch, acc);
  };
  // Two query blocks in LDS (the one computed, the one loaded), as separate
  // arrays and an unrolled pair of iterations so the compiler can tell them
  // apart.
  int cq = qq;  // block index (within the head) of the block being computed
  if (it0 < n_it) issue(qb0, ob0, lb0, db0);
  // The per-row values are read before the next block's copies are issued:
  // an LDS read right after the issue would make the compiler wait for the
  // copies (it cannot tell the buffers apart).
  for (int it = it0; it < n_it; it += 2) {
    {
      wait_dma();
      __syncthreads();
      f32x16 x[2];
      dkdv_rows(m == 0 ? lb0 : db0, lg, x);
      if (it + 1 < n_it) issue(qb1, ob1, lb1, db1);
      tile(cq, qb0, ob0, x);
      if (++cq == nqb) cq = 0;
    }
    if (it + 1 < n_it) {
      wait_dma();
      __syncthreads();
      f32x16 x[2];
      dkdv_rows(m == 0 ? lb1 : db1, lg, x);
      if (it + 2 < n_it) issue(qb0, ob0, lb0, db0);
      tile(cq, qb1, ob1, x);
      if (++cq == nqb) cq = 0;
    }
  }

  if (cd.z > 1) {
    // a chunk of a cut tile: its accumulators go to its partial-sum slot,
    // laid out [slot][kv head][wave][register / 4][lane][4]; dkdv_reduce_kernel
    // adds the tile's slots and writes the gradients
    f32x4* mine = reinterpret_cast<f32x4*>(kpart) + (((size_t)(cd.w + cd.y) * Hkv + hk) * kDkdvWaves + w) * (NDB * 4 * 64) + lane;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        mine[(4 * b + i4) * 64] = f32x4{acc[b][4 * i4], acc[b][4 * i4 + 1], acc[b][4 * i4 + 2], acc[b][4 * i4 + 3]};
    return;
  }
  __syncthreads();  // every wave is done with the tile buffers
  dkdv_epilogue<DP, Tio>(acc, qb0, qb1, ob0, ob1, j0, hk, T, Lq, Lp, Hkv, scale, cs, dk, dv, dk_past, dv_past,
                         acc_past);
}

// The cut tiles of the dK/dV work split: workgroup (i, kv head) adds the S
// partial sums of cut tile i in slot order, each wave the slot blocks of its
// own (key slice, role), and writes the tile's gradients.
template <int DP, typename Tio>
__global__ __launch_bounds__(64 * kDkdvWaves) void dkdv_reduce_kernel(
    const int4* __restrict__ ktcut, const float* __restrict__ kpart, const float2* __restrict__ cs, int T, int Lq,
    int Lp, int Hkv, float scale, Tio* __restrict__ dk, Tio* __restrict__ dv, float* __restrict__ dk_past,
    float* __restrict__ dv_past, int acc_past) {
  constexpr int NDB = DP / 32;
  constexpr int TILE = 64 * DP;
  __shared__ __attribute__((aligned(1024))) bf16 sb0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sb1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sb2[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sb3[TILE];
  const int4 ct = ktcut[blockIdx.x % kDkdvSlots];  // {tile, chunks, first slot}
  const int hk = blockIdx.x / kDkdvSlots;
  if (ct.x < 0) return;  // uniform over the workgroup
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  f32x16 acc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) acc[b] = f32x16{};
  for (int c = 0; c < ct.y; ++c) {
    const f32x4* src =
        reinterpret_cast<const f32x4*>(kpart) + (((size_t)(ct.z + c) * Hkv + hk) * kDkdvWaves + w) * (NDB * 4 * 64) + lane;
    // all of the slot's loads first, then the adds
    f32x4 t[NDB * 4];
#pragma unroll
    for (int q = 0; q < NDB * 4; ++q) t[q] = src[q * 64];
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[b][i] += t[4 * b + (i >> 2)][i & 3];
  }
  dkdv_epilogue<DP, Tio>(acc, sb0, sb1, sb2, sb3, ct.x * kBwdBK, hk, T, Lq, Lp, Hkv, scale, cs, dk, dv, dk_past,
                         dv_past, acc_past);
}

// ------------------------------------------------------------------------
// Partition-boundary hand-over ("Tree Training" App. B.2 and B.5). Export:
// rows[r] of a partition's own tokens become cached row r of a child's
// gateway, the key rotated at that token's position (pos_offset + pos), the
// value as is. Relay: the float32 gradients of cached row r flow back into
// that token's dk (through R^T) and dv, added in float32 and rounded once.
// One workgroup per listed row; a row index outside [0, T) exports zeros and
// relays nothing.
template <typename Tio>
__global__ __launch_bounds__(256) void gw_export_kernel(const Tio* __restrict__ k, const Tio* __restrict__ v,
                                                        const int* __restrict__ pos, const int* __restrict__ rows,
                                                        int T, int Hkv, int D, int pos_offset, float theta,
                                                        Tio* __restrict__ k_past, Tio* __restrict__ v_past) {
  __shared__ float2 tab[64];
  const int r = blockIdx.x;
  const int j = rows[r];
  const bool ok = j >= 0 && j < T;
  const int half = D / 2;
  if ((int)threadIdx.x < half) tab[threadIdx.x] = ok ? rope_cs(pos_offset + pos[j], threadIdx.x, D, theta)
                                                     : make_float2(1.0f, 0.0f);
  __syncthreads();
  for (int idx = threadIdx.x; idx < Hkv * half; idx += blockDim.x) {
    const int hk = idx / half, kk = idx % half;
    const size_t src = ((size_t)(ok ? j : 0) * Hkv + hk) * D, dst = ((size_t)r * Hkv + hk) * D;
    float y1 = 0.0f, y2 = 0.0f, v1 = 0.0f, v2 = 0.0f;
    if (ok) {
      rope_rot(to_f32(k[src + kk]), to_f32(k[src + kk + half]), tab[kk], y1, y2);
      v1 = to_f32(v[src + kk]);
      v2 = to_f32(v[src + kk + half]);
    }
    k_past[dst + kk] = from_f32<Tio>(y1);
    k_past[dst + kk + half] = from_f32<Tio>(y2);
    v_past[dst + kk] = from_f32<Tio>(v1);
    v_past[dst + kk + half] = from_f32<Tio>(v2);
  }
}

template <typename Tio>
__global__ __launch_bounds__(256) void gw_relay_kernel(const float* __restrict__ dk_past,
                                                       const float* __restrict__ dv_past,
                                                       const int* __restrict__ pos, const int* __restrict__ rows,
                                                       int T, int Hkv, int D, int pos_offset, float theta,
                                                       Tio* __restrict__ dk, Tio* __restrict__ dv) {
  __shared__ float2 tab[64];
  const int r = blockIdx.x;
  const int j = rows[r];
  if (j < 0 || j >= T) return;  // uniform over the workgroup
  const int half = D / 2;
  if ((int)threadIdx.x < half) tab[threadIdx.x] = rope_cs(pos_offset + pos[j], threadIdx.x, D, theta);
  __syncthreads();
  for (int idx = threadIdx.x; idx < Hkv * half; idx += blockDim.x) {
    const int hk = idx / half, kk = idx % half;
    const size_t src = ((size_t)r * Hkv + hk) * D, dst = ((size_t)j * Hkv + hk) * D;
    float g1, g2;
    rope_rot_t(dk_past[src + kk], dk_past[src + kk + half], tab[kk], g1, g2);
    dk[dst + kk] = from_f32<Tio>(to_f32(dk[dst + kk]) + g1);
    dk[dst + kk + half] = from_f32<Tio>(to_f32(dk[dst + kk + half]) + g2);
    dv[dst + kk] = from_f32<Tio>(to_f32(dv[dst + kk]) + dv_past[src + kk]);
    dv[dst + kk + half] = from_f32<Tio>(to_f32(dv[dst + kk + half]) + dv_past[src + kk + half]);
  }
}

// ------------------------------------------------------------------------
// Host side
// Workspace layout. Rows are those of the combined sequence: Lp cached rows
// padded to Lq (a multiple of the 128-row query tile), then the T packed
// tokens; Tc = Lq + T rows in all, padded to Tp.
struct AttnLayout {
  int T, Lp, Lq, Tc, Tp, Hq, Hkv, D, DP, nq, nk64, nk128;
  int nsb, ncmax;
  size_t off_status, off_qr, off_kr, off_vr, off_sep, off_cs, off_kmm64, off_kmm128, off_sbmax, off_qcount, off_qfull,
      off_qorder;
  size_t off_kwork, off_korder, off_cdesc, off_ktcut, off_dd, off_l2, off_dor, off_kpart, total;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

AttnLayout make_layout(int T, int Lp, int Hq, int Hkv, int D, bool with_bwd) {
  AttnLayout L{};
  L.T = T;
  L.Lp = Lp;
  L.Lq = (Lp + kFwdBQ - 1) / kFwdBQ * kFwdBQ;
  L.Tc = L.Lq + T;
  L.Tp = (L.Tc + 255) / 256 * 256;  // a multiple of every query tile size
  L.Hq = Hq;
  L.Hkv = Hkv;
  L.D = D;
  L.DP = D < 32 ? 32 : D;
  L.nq = L.Tp / kFwdBQ;
  L.nk64 = (L.Tc + kFwdBK - 1) / kFwdBK;
  L.nk128 = (L.Tc + kBwdBK - 1) / kBwdBK;
  L.nsb = (L.nk64 + kSbTiles - 1) / kSbTiles;
  L.ncmax = L.nk128 + kDkdvSlots;
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.off_status = take(4);  // always offset 0
  L.off_qr = take((size_t)Hq * L.Tp * L.DP * 2);
  L.off_kr = take((size_t)Hkv * L.Tp * L.DP * 2);
  L.off_vr = take((size_t)Hkv * L.Tp * L.DP * 2);
  L.off_sep = take((size_t)L.Tp * 4);
  L.off_cs = take((size_t)L.Tp * (D / 2) * 8);
  L.off_kmm64 = take((size_t)L.nk64 * 8);
  L.off_kmm128 = take((size_t)L.nk128 * 8);
  L.off_sbmax = take((size_t)L.nsb * 4);
  L.off_qcount = take((size_t)L.nq * 4);
  L.off_qfull = take((size_t)L.nq * 4);
  L.off_qorder = take((size_t)L.nq * 4);
  L.off_kwork = take((size_t)L.nk128 * 4);
  L.off_korder = take((size_t)L.nk128 * 4);
  L.off_cdesc = take((size_t)L.ncmax * 16);
  L.off_ktcut = take((size_t)kDkdvSlots * 16);
  if (with_bwd) {
    L.off_dd = take((size_t)Hq * L.Tp * 4);
    L.off_l2 = take((size_t)Hq * L.Tp * 4);
    L.off_dor = take((size_t)Hq * L.Tp * L.DP * 2);
    L.off_kpart = take((size_t)kSplitSlots * Hkv * kDkdvWaves * (L.DP / 2) * 64 * 4);
  }
  L.total = o;
  return L;
}

constexpr int kMaxRows = 1 << 22;

int validate_shape(const char* fn, int T, int Lp, int Hq, int Hkv, int d) {
  if (T < 1 || T > kMaxRows) return fail(TA_EINVAL, "%s: T must be in [1, 2^22] (got %d)", fn, T);
  if (Lp < 0 || Lp > kMaxRows - T - kFwdBQ)
    return fail(TA_EINVAL, "%s: past_len must be in [0, 2^22 - T - 128] (got %d)", fn, Lp);
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

template <typename T>
T* at(char* ws, size_t off) {
  return reinterpret_cast<T*>(ws + off);
}

// The cached rows of a child partition (none: Lp = 0).
struct Past {
  const void* k = nullptr;
  const void* v = nullptr;
  const unsigned char* vis = nullptr;
  int pos_offset = 0;
  float* dk = nullptr;
  float* dv = nullptr;
  int accumulate = 0;
};

template <typename Tio>
int run_prep(const AttnLayout& L, const void* q, const void* k, const void* v, const int* pos, const int* se,
             const Past& past, float theta, char* ws, hipStream_t st) {
  {
    ProfScope ps("rope_prep", st);
    hipLaunchKernelGGL(status_reset_kernel, dim3(1), dim3(64), 0, st, at<int>(ws, L.off_status));
    hipLaunchKernelGGL(rope_prep_kernel<Tio>, dim3(L.Tp), dim3(256), 0, st, static_cast<const Tio*>(q),
                       static_cast<const Tio*>(k), static_cast<const Tio*>(v), pos, se,
                       static_cast<const Tio*>(past.k), static_cast<const Tio*>(past.v), past.vis, L.Lp, L.Lq,
                       past.pos_offset, L.Tc, L.Tp, L.Hq, L.Hkv, L.D, L.DP, theta, at<bf16>(ws, L.off_qr),
                       at<bf16>(ws, L.off_kr), at<bf16>(ws, L.off_vr), at<int>(ws, L.off_sep),
                       at<float2>(ws, L.off_cs), at<int>(ws, L.off_status));
  }
  ProfScope ps("tile_plan", st);
  static_assert(kFwdRows == kFwdBQ, "the forward shares the dQ pass's query-tile plan");
  static_assert(kBwdBK == 2 * kFwdBK, "a 128-key tile is two 64-key tiles");
  hipLaunchKernelGGL(tile_minmax_kernel, dim3((L.nk128 + 3) / 4), dim3(256), 0, st, at<const int>(ws, L.off_sep),
                     L.Tc, L.Lq, L.nk64, L.nk128, at<int2>(ws, L.off_kmm64), at<int2>(ws, L.off_kmm128),
                     at<int>(ws, L.off_kwork));
  hipLaunchKernelGGL(sb_max_kernel, dim3((L.nsb + 3) / 4), dim3(256), 0, st, at<const int2>(ws, L.off_kmm64), L.nk64,
                     L.nsb, at<int>(ws, L.off_sbmax));
  hipLaunchKernelGGL(q_count_kernel, dim3(L.nq), dim3(64), 0, st, at<const int2>(ws, L.off_kmm64),
                     at<const int>(ws, L.off_sbmax), L.Tc, L.Lq, L.nk64, at<int>(ws, L.off_qcount),
                     at<int>(ws, L.off_qfull));
  hipLaunchKernelGGL(order_kernel, dim3(2), dim3(1024), 0, st, at<const int>(ws, L.off_qcount), L.nq,
                     at<int>(ws, L.off_qorder), at<const int>(ws, L.off_kwork), L.nk128, L.Hq / L.Hkv,
                     at<int>(ws, L.off_korder), at<int4>(ws, L.off_cdesc), L.ncmax, at<int4>(ws, L.off_ktcut));
  return check_launch("prep");
}

template <int DP, typename Tio>
int run_fwd(const AttnLayout& L, float sl2, void* o, float* lse, char* ws, hipStream_t st) {
  ProfScope ps("attn_fwd", st);
  hipLaunchKernelGGL((attn_fwd_kernel<DP, Tio>), dim3(L.nq * L.Hq), dim3(64 * kFwdWaves), 0, st,
                     at<const bf16>(ws, L.off_qr), at<const bf16>(ws, L.off_kr), at<const bf16>(ws, L.off_vr),
                     at<const int>(ws, L.off_sep), at<const int2>(ws, L.off_kmm64), at<const int>(ws, L.off_sbmax),
                     at<const int>(ws, L.off_qorder), L.Tc, L.Lq, L.Tp, L.Hq, L.Hkv, L.nq, L.nk64, sl2,
                     static_cast<Tio*>(o), lse);
  return check_launch("tree_attn_fwd");
}

template <int DP, typename Tio>
int run_bwd(const AttnLayout& L, const void* o, const float* lse, const void* dout, float sl2, float scale,
            void* dq, void* dk, void* dv, const Past& past, char* ws, hipStream_t st) {
  {
    ProfScope ps("attn_bwd_dq", st);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<DP, Tio>), dim3(L.nq * L.Hq), dim3(256), 0, st,
                       at<const bf16>(ws, L.off_qr), at<const bf16>(ws, L.off_kr), at<const bf16>(ws, L.off_vr),
                       static_cast<const Tio*>(o), static_cast<const Tio*>(dout), lse, at<float>(ws, L.off_dd),
                       at<float>(ws, L.off_l2), at<bf16>(ws, L.off_dor), at<const int>(ws, L.off_sep),
                       at<const int2>(ws, L.off_kmm64), at<const int>(ws, L.off_sbmax),
                       at<const int>(ws, L.off_qorder), at<const float2>(ws, L.off_cs), L.Tc, L.Lq, L.Tp, L.Hq,
                       L.Hkv, L.nq, L.nk64, sl2, scale, static_cast<Tio*>(dq));
  }
  ProfScope ps("attn_bwd_dkdv", st);
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<DP, Tio>), dim3(L.ncmax * L.Hkv), dim3(64 * kDkdvWaves), 0, st,
                     at<const bf16>(ws, L.off_qr), at<const bf16>(ws, L.off_kr), at<const bf16>(ws, L.off_vr),
                     at<const bf16>(ws, L.off_dor), at<const float>(ws, L.off_l2), at<const float>(ws, L.off_dd),
                     at<const int>(ws, L.off_sep), at<const int2>(ws, L.off_kmm128), at<const int4>(ws, L.off_cdesc),
                     L.ncmax, at<float>(ws, L.off_kpart), at<const float2>(ws, L.off_cs), L.Tc, L.Lq, L.Lp, L.Tp,
                     L.Hq, L.Hkv, sl2, scale, static_cast<Tio*>(dk), static_cast<Tio*>(dv), past.dk, past.dv,
                     past.accumulate);
  hipLaunchKernelGGL((dkdv_reduce_kernel<DP, Tio>), dim3(kDkdvSlots * L.Hkv), dim3(64 * kDkdvWaves), 0, st,
                     at<const int4>(ws, L.off_ktcut), at<const float>(ws, L.off_kpart), at<const float2>(ws, L.off_cs),
                     L.Tc, L.Lq, L.Lp, L.Hkv, scale, static_cast<Tio*>(dk), static_cast<Tio*>(dv), past.dk, past.dv,
                     past.accumulate);
  return check_launch("tree_attn_bwd");
}

// Shared by the plain and the partition-boundary entry points.
int attn_fwd(const char* fn, const void* q, const void* k, const void* v, ta_dtype dt, int T, int Hq, int Hkv, int d,
             const int* pos, const int* se, const Past& past, int Lp, float softmax_scale, float rope_theta, void* o,
             float* lse, void* workspace, size_t ws_bytes, void* stream) {
  if (int rc = validate_shape(fn, T, Lp, Hq, Hkv, d)) return rc;
  if (!q || !k || !v || !pos || !se || !o || !lse || !workspace) return fail(TA_EINVAL, "%s: NULL pointer argument", fn);
  if (Lp > 0 && (!past.k || !past.v || !past.vis)) return fail(TA_EINVAL, "%s: NULL past pointer argument", fn);
  if (dt != TA_BF16 && dt != TA_F32) return fail(TA_EINVAL, "%s: bad dtype %d", fn, (int)dt);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (Lp > 0 && (!aligned16(past.k) || !aligned16(past.v))))
    return fail(TA_EINVAL, "%s: q, k, v (and k_past, v_past) must be 16-byte aligned", fn);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TA_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  if (!(rope_theta >= 0.0f)) return fail(TA_EINVAL, "%s: rope_theta must be >= 0", fn);
  if (past.pos_offset < 0) return fail(TA_EINVAL, "%s: pos_offset must be >= 0", fn);
  const AttnLayout L = make_layout(T, Lp, Hq, Hkv, d, false);
  if (ws_bytes < L.total) return fail(TA_EINVAL, "%s: workspace too small (%zu < %zu bytes)", fn, ws_bytes, L.total);
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)d);
  const float sl2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int rc = dt == TA_BF16 ? run_prep<bf16>(L, q, k, v, pos, se, past, rope_theta, ws, st)
                         : run_prep<float>(L, q, k, v, pos, se, past, rope_theta, ws, st);
  if (rc) return rc;
  if (dt == TA_BF16) {
    if (L.DP == 32) return run_fwd<32, bf16>(L, sl2, o, lse, ws, st);
    if (L.DP == 64) return run_fwd<64, bf16>(L, sl2, o, lse, ws, st);
    return run_fwd<128, bf16>(L, sl2, o, lse, ws, st);
  }
  if (L.DP == 32) return run_fwd<32, float>(L, sl2, o, lse, ws, st);
  if (L.DP == 64) return run_fwd<64, float>(L, sl2, o, lse, ws, st);
  return run_fwd<128, float>(L, sl2, o, lse, ws, st);
}

int attn_bwd(const char* fn, const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, ta_dtype dt, int T, int Hq, int Hkv, int d, const int* pos, const int* se,
             const Past& past, int Lp, float softmax_scale, float rope_theta, int flags, void* dq, void* dk, void* dv,
             void* workspace, size_t ws_bytes, void* stream) {
  if (int rc = validate_shape(fn, T, Lp, Hq, Hkv, d)) return rc;
  if (!q || !k || !v || !o || !lse || !dout || !pos || !se || !dq || !dk || !dv || !workspace)
    return fail(TA_EINVAL, "%s: NULL pointer argument", fn);
  if (Lp > 0 && (!past.k || !past.v || !past.vis || !past.dk || !past.dv))
    return fail(TA_EINVAL, "%s: NULL past pointer argument", fn);
  if (dt != TA_BF16 && dt != TA_F32) return fail(TA_EINVAL, "%s: bad dtype %d", fn, (int)dt);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      (Lp > 0 && (!aligned16(past.k) || !aligned16(past.v))))
    return fail(TA_EINVAL, "%s: q, k, v, o, dout (and k_past, v_past) must be 16-byte aligned", fn);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TA_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  if (!(rope_theta >= 0.0f)) return fail(TA_EINVAL, "%s: rope_theta must be >= 0", fn);
  if (past.pos_offset < 0) return fail(TA_EINVAL, "%s: pos_offset must be >= 0", fn);
  if (flags & ~(TA_REUSE_PREP | TA_ACCUMULATE_PAST)) return fail(TA_EINVAL, "%s: unknown flags 0x%x", fn, flags);
  const AttnLayout L = make_layout(T, Lp, Hq, Hkv, d, true);
  if (ws_bytes < L.total) return fail(TA_EINVAL, "%s: workspace too small (%zu < %zu bytes)", fn, ws_bytes, L.total);
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)d);
  const float sl2 = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (!(flags & TA_REUSE_PREP)) {
    int rc = dt == TA_BF16 ? run_prep<bf16>(L, q, k, v, pos, se, past, rope_theta, ws, st)
                           : run_prep<float>(L, q, k, v, pos, se, past, rope_theta, ws, st);
    if (rc) return rc;
  }
  if (dt == TA_BF16) {
    if (L.DP == 32) return run_bwd<32, bf16>(L, o, lse, dout, sl2, scale, dq, dk, dv, past, ws, st);
    if (L.DP == 64) return run_bwd<64, bf16>(L, o, lse, dout, sl2, scale, dq, dk, dv, past, ws, st);
    return run_bwd<128, bf16>(L, o, lse, dout, sl2, scale, dq, dk, dv, past, ws, st);
  }
  if (L.DP == 32) return run_bwd<32, float>(L, o, lse, dout, sl2, scale, dq, dk, dv, past, ws, st);
  if (L.DP == 64) return run_bwd<64, float>(L, o, lse, dout, sl2, scale, dq, dk, dv, past, ws, st);
  return run_bwd<128, float>(L, o, lse, dout, sl2, scale, dq, dk, dv, past, ws, st);
}

}  // namespace
}  // namespace ta

using namespace ta;

extern "C" size_t tree_attn_workspace_bytes(int32_t T, int32_t Hq, int32_t Hkv, int32_t d, int32_t with_bwd) {
  if (T < 1 || T > kMaxRows || Hq < 1 || Hkv < 1 || d < 1) return 0;
  return make_layout(T, 0, Hq, Hkv, d, with_bwd != 0).total;
}

extern "C" int tree_attn_fwd(const void* q, const void* k, const void* v, ta_dtype dt, int32_t T, int32_t Hq,
                             int32_t Hkv, int32_t d, const int32_t* pos, const int32_t* subtree_end,
                             float softmax_scale, float rope_theta, void* o, float* lse, void* workspace,
                             size_t ws_bytes, void* stream) {
  clear_error();
  return attn_fwd("tree_attn_fwd", q, k, v, dt, T, Hq, Hkv, d, pos, subtree_end, Past{}, 0, softmax_scale,
                  rope_theta, o, lse, workspace, ws_bytes, stream);
}

extern "C" int tree_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, ta_dtype dt, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                             const int32_t* pos, const int32_t* subtree_end, float softmax_scale, float rope_theta,
                             int32_t flags, void* dq, void* dk, void* dv, void* workspace, size_t ws_bytes,
                             void* stream) {
  clear_error();
  if (flags & TA_ACCUMULATE_PAST) return fail(TA_EINVAL, "tree_attn_bwd: TA_ACCUMULATE_PAST needs cached rows");
  return attn_bwd("tree_attn_bwd", q, k, v, o, lse, dout, dt, T, Hq, Hkv, d, pos, subtree_end, Past{}, 0,
                  softmax_scale, rope_theta, flags, dq, dk, dv, workspace, ws_bytes, stream);
}

extern "C" int tree_attn_workspace_status(const void* workspace, int32_t* status, void* stream) {
  clear_error();
  if (!workspace || !status) return fail(TA_EINVAL, "tree_attn_workspace_status: NULL pointer argument");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(status, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(TA_EHIP, "tree_attn_workspace_status: %s", hipGetErrorString(hipGetLastError()));
  return TA_OK;
}

extern "C" int tree_attn_plan_counts(const void* workspace, size_t ws_bytes, int32_t T, int32_t past_len, int32_t Hq,
                                     int32_t Hkv, int32_t d, int32_t n_qtiles, int32_t* nonempty, int32_t* full,
                                     void* stream) {
  clear_error();
  if (int rc = validate_shape("tree_attn_plan_counts", T, past_len, Hq, Hkv, d)) return rc;
  if (!workspace || !nonempty || !full) return fail(TA_EINVAL, "tree_attn_plan_counts: NULL pointer argument");
  const AttnLayout L = make_layout(T, past_len, Hq, Hkv, d, false);
  if (ws_bytes < L.total)
    return fail(TA_EINVAL, "tree_attn_plan_counts: workspace too small (%zu < %zu bytes)", ws_bytes, L.total);
  if (n_qtiles != L.nq)
    return fail(TA_EINVAL, "tree_attn_plan_counts: n_qtiles must be %d (got %d)", L.nq, n_qtiles);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char* ws = static_cast<const char*>(workspace);
  if (hipMemcpyAsync(nonempty, ws + L.off_qcount, (size_t)L.nq * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(full, ws + L.off_qfull, (size_t)L.nq * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return fail(TA_EHIP, "tree_attn_plan_counts: %s", hipGetErrorString(hipGetLastError()));
  return TA_OK;
}

extern "C" size_t tree_attn_gw_workspace_bytes(int32_t T, int32_t past_len, int32_t Hq, int32_t Hkv, int32_t d,
                                               int32_t with_bwd) {
  if (T < 1 || T > kMaxRows || past_len < 0 || past_len > kMaxRows - T - kFwdBQ || Hq < 1 || Hkv < 1 || d < 1)
    return 0;
  return make_layout(T, past_len, Hq, Hkv, d, with_bwd != 0).total;
}

extern "C" int tree_attn_gw_fwd(const void* q, const void* k, const void* v, ta_dtype dt, int32_t T, int32_t Hq,
                                int32_t Hkv, int32_t d, const int32_t* pos, const int32_t* subtree_end,
                                int32_t pos_offset, const void* k_past, const void* v_past,
                                const uint8_t* past_visible, int32_t past_len, float softmax_scale, float rope_theta,
                                void* o, float* lse, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  Past past;
  past.k = k_past;
  past.v = v_past;
  past.vis = past_visible;
  past.pos_offset = pos_offset;
  return attn_fwd("tree_attn_gw_fwd", q, k, v, dt, T, Hq, Hkv, d, pos, subtree_end, past, past_len, softmax_scale,
                  rope_theta, o, lse, workspace, ws_bytes, stream);
}

extern "C" int tree_attn_gw_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                const void* dout, ta_dtype dt, int32_t T, int32_t Hq, int32_t Hkv, int32_t d,
                                const int32_t* pos, const int32_t* subtree_end, int32_t pos_offset,
                                const void* k_past, const void* v_past, const uint8_t* past_visible,
                                int32_t past_len, float softmax_scale, float rope_theta, int32_t flags, void* dq,
                                void* dk, void* dv, float* dk_past, float* dv_past, void* workspace,
                                size_t ws_bytes, void* stream) {
  clear_error();
  Past past;
  past.k = k_past;
  past.v = v_past;
  past.vis = past_visible;
  past.pos_offset = pos_offset;
  past.dk = dk_past;
  past.dv = dv_past;
  past.accumulate = (flags & TA_ACCUMULATE_PAST) ? 1 : 0;
  return attn_bwd("tree_attn_gw_bwd", q, k, v, o, lse, dout, dt, T, Hq, Hkv, d, pos, subtree_end, past, past_len,
                  softmax_scale, rope_theta, flags, dq, dk, dv, workspace, ws_bytes, stream);
}

namespace ta {
namespace {
int gw_rows_check(const char* fn, ta_dtype dt, int32_t T, int32_t Hkv, int32_t d, int32_t n_rows) {
  if (T < 1 || T > kMaxRows) return fail(TA_EINVAL, "%s: T must be in [1, 2^22] (got %d)", fn, T);
  if (Hkv < 1 || Hkv > 256) return fail(TA_EINVAL, "%s: Hkv must be in [1, 256] (got %d)", fn, Hkv);
  if (d != 16 && d != 64 && d != 128) return fail(TA_EUNSUPPORTED, "%s: head dim %d not in {16, 64, 128}", fn, d);
  if (n_rows < 0 || n_rows > kMaxRows) return fail(TA_EINVAL, "%s: n_rows must be in [0, 2^22] (got %d)", fn, n_rows);
  if (dt != TA_BF16 && dt != TA_F32) return fail(TA_EINVAL, "%s: bad dtype %d", fn, (int)dt);
  return TA_OK;
}
}  // namespace
}  // namespace ta

extern "C" int tree_attn_gw_export(const void* k, const void* v, ta_dtype dt, int32_t T, int32_t Hkv, int32_t d,
                                   const int32_t* pos, int32_t pos_offset, float rope_theta, const int32_t* rows,
                                   int32_t n_rows, void* k_past, void* v_past, void* stream) {
  clear_error();
  const char* fn = "tree_attn_gw_export";
  if (int rc = gw_rows_check(fn, dt, T, Hkv, d, n_rows)) return rc;
  if (!k || !v || !pos || !rows || !k_past || !v_past) return fail(TA_EINVAL, "%s: NULL pointer argument", fn);
  if (!(rope_theta >= 0.0f)) return fail(TA_EINVAL, "%s: rope_theta must be >= 0", fn);
  if (pos_offset < 0) return fail(TA_EINVAL, "%s: pos_offset must be >= 0", fn);
  if (n_rows == 0) return TA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ProfScope ps("gw_export", st);
  if (dt == TA_BF16)
    hipLaunchKernelGGL(gw_export_kernel<bf16>, dim3(n_rows), dim3(256), 0, st, static_cast<const bf16*>(k),
                       static_cast<const bf16*>(v), pos, rows, T, Hkv, d, pos_offset, rope_theta,
                       static_cast<bf16*>(k_past), static_cast<bf16*>(v_past));
  else
    hipLaunchKernelGGL(gw_export_kernel<float>, dim3(n_rows), dim3(256), 0, st, static_cast<const float*>(k),
                       static_cast<const float*>(v), pos, rows, T, Hkv, d, pos_offset, rope_theta,
                       static_cast<float*>(k_past), static_cast<float*>(v_past));
  return check_launch(fn);
}

extern "C" int tree_attn_gw_relay(const float* dk_past, const float* dv_past, const int32_t* rows, int32_t n_rows,
                                  ta_dtype dt, int32_t T, int32_t Hkv, int32_t d, const int32_t* pos,
                                  int32_t pos_offset, float rope_theta, void* dk, void* dv, void* stream) {
  clear_error();
  const char* fn = "tree_attn_gw_relay";
  if (int rc = gw_rows_check(fn, dt, T, Hkv, d, n_rows)) return rc;
  if (!dk_past || !dv_past || !rows || !pos || !dk || !dv) return fail(TA_EINVAL, "%s: NULL pointer argument", fn);
  if (!(rope_theta >= 0.0f)) return fail(TA_EINVAL, "%s: rope_theta must be >= 0", fn);
  if (pos_offset < 0) return fail(TA_EINVAL, "%s: pos_offset must be >= 0", fn);
  if (n_rows == 0) return TA_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  ProfScope ps("gw_relay", st);
  if (dt == TA_BF16)
    hipLaunchKernelGGL(gw_relay_kernel<bf16>, dim3(n_rows), dim3(256), 0, st, dk_past, dv_past, pos, rows, T, Hkv,
                       d, pos_offset, rope_theta, static_cast<bf16*>(dk), static_cast<bf16*>(dv));
  else
    hipLaunchKernelGGL(gw_relay_kernel<float>, dim3(n_rows), dim3(256), 0, st, dk_past, dv_past, pos, rows, T, Hkv,
                       d, pos_offset, rope_theta, static_cast<float*>(dk), static_cast<float*>(dv));
  return check_launch(fn);
}
