// Tree-correct SSM pieces for gfx950: the depthwise causal conv1d over each
// token's ancestor chain, and the gated delta rule with the state routed
// along the tree.
//
// "Tree Training" §3.2 (SSM Layers, Eq. 10 and 11) and App. A.2-A.3: in the
// DFS layout the tokens just before a child chunk belong to a sibling branch,
// so a chunk must take its conv context and its initial recurrent state from
// its parent. Both reduce to following par[t]:
//   conv   a_t = b + sum_{n<K} w[:, K-1-n] x_{anc_n(t)},  y_t = act(a_t)
//   delta  h_t = alpha_t (I - beta_t k_t k_t^T) h_{par(t)} + beta_t k_t v_t^T,
//          o_t = h_t^T q_t,  alpha_t = exp(g_t)
//
// Conv: a workgroup takes a tile of tokens and every thread 8 channels. The
// tile's rows and the K-1 rows before it are loaded up front; one thread per
// token lists its K-1 ancestors in LDS (walking parents read into LDS for the
// tile window), and taps whose ancestor is not the row before are loaded
// apart. A tile on a chain (every tap's ancestor is t - m) skips the
// per-tap checks. The backward forms g = dy * act'(a) once, gathers dx_j over
// the descendants of j at most K-1 levels below it (listed per token in LDS
// by a walk of the preorder range (j, se[j]) that jumps over every deeper
// subtree; on a chain they are j + 1 .. j + K - 1 and come from a tile of g
// rows), and reduces dw / db over token blocks in a fixed order.
//
// Gated delta rule, per v-head, in chunks of <= 64 tokens inside tree nodes
// (the host plan, tree_gdn_plan, gives chunk ranges, chunk parents and the
// chain / level schedule):
//   1. prep (all chunks at once): gc = in-chunk cumulative log decay,
//      M = strictly-lower (beta k) k^T * exp(gc_i - gc_j) (bf16 MFMA),
//      T = (I + M)^-1 in float32 by 16 x 16 blocks, [u | w] = T [beta v |
//      beta k exp(gc)] (bf16 MFMA)
//   2. state (one launch per level; a workgroup walks one chain): starting
//      from the parent's end state, per chunk h0 is stored, vn = u - w h0
//      and h = exp(gc_last) h0 + kd^T vn with kd = k exp(gc_last - gc), both
//      bf16 MFMA with float32 accumulators that carry h from chunk to chunk;
//      the next chunk's w, kd^T and u stream into LDS (direct HBM -> LDS
//      copies, double buffered) while the current one is computed
//   3. output (all chunks at once): o = (q exp(gc)) h0 + (q k^T * exp(gc_i -
//      gc_j), j <= i) vn
// The start state of a chunk's first child chunk is the chunk's end state, so
// a chain that starts under chunk p loads the stored start state of p + 1.
// The backward (tree_gdn_bwd) runs the same routing in reverse: see the
// section "gated delta rule, backward" below.
//
// Workspace (chunk-local, rows past a chunk's length are zero):
//   gc  [Hv][nc][64] f32        (past the chunk length: the last value)
//   u   [Hv][nc][64][dv] f32
//   w   [Hv][nc][64][dk] bf16   (columns in swap23 order within each 16)
//   kd  [Hv][nc][dk][64] bf16   (k^T exp(gc_last - gc), zero past the length)
//   vnt [Hv][nc] x (dv x 64) bf16, column-grouped (vn^T; cr_off below)
//   h0  [nc][Hv] x (dv x dk) bf16, column-grouped (start state of each chunk)
//   tt  [Hv][nc][64][64] bf16   ((I + M)^-1 transposed, for the backward)
#include <hip/hip_runtime.h>

#include <cstdint>

#include "profile.h"
#include "ta_device.h"
#include "ta_error.h"
#include "ta_lds.h"
#include "tree_attn.h"

namespace ta {
namespace {

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ void ld8f(const bf16* p, float* f) {
  const bf16x8 v = load8(p);
#pragma unroll
  for (int s = 0; s < 8; ++s) f[s] = (float)v[s];
}
__device__ __forceinline__ void ld8f(const float* p, float* f) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    f[s] = a[s];
    f[4 + s] = b[s];
  }
}
__device__ __forceinline__ void st8f(bf16* p, const float* f) {
  bf16x8 v;
#pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = (bf16)f[s];
  *reinterpret_cast<bf16x8*>(p) = v;
}
__device__ __forceinline__ void st8f(float* p, const float* f) {
  f32x4 a, b;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    a[s] = f[s];
    b[s] = f[4 + s];
  }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

// Logistic function from the hardware exp2 and reciprocal (each about 1 ulp in
// float32): the full-precision expf and IEEE division would make the conv
// kernels instruction-bound. Large |a| saturates to 0 or 1 (exp2 overflows to
// inf, whose reciprocal is 0).
__device__ __forceinline__ float sigmoidf(float a) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-a * 1.4426950408889634f));
}

// Workgroup barrier that orders LDS only: global loads in flight stay in
// flight (__syncthreads also waits for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- tree conv

constexpr int kConvThreads = 256;
constexpr int kConvMaxK = 8;
constexpr int kConvTB = 16;          // tokens per forward / dx workgroup
constexpr int kConvTokBlock = 128;   // tokens per dw / db partial (g pass)
constexpr int kConvMaxDesc = 48;     // listed descendants per token in the dx pass

// Ancestor table of tokens [t0, t0 + N): anc[i][m] = m-th ancestor of
// t0 + i (m < K), -1 past a root or for tokens past T. The parents of the
// window [t0 - (kConvMaxK - 1), t0 + N) are read in one parallel pass into
// pl (LDS, N + kConvMaxK - 1 entries); one thread per token then walks its
// parents there, reading HBM only where a node's first token points outside
// the window. All threads of the workgroup call it (it holds a barrier).
// A parent precedes its child in preorder; any other value (malformed
// metadata) is read as "no parent", so ancestor walks always move to lower
// indices and stay in bounds.
__device__ __forceinline__ int sane_parent(int p, int t) { return (p >= 0 && p < t) ? p : -1; }

template <int N>
__device__ __forceinline__ void conv_ancestors(const int* __restrict__ par, int t0, int T, int K,
                                               int (*anc)[kConvMaxK], int* pl) {
  const int base = t0 - (kConvMaxK - 1);
  for (int r = threadIdx.x; r < N + kConvMaxK - 1; r += blockDim.x) {
    const int t = base + r;
    pl[r] = (t >= 0 && t < T) ? sane_parent(par[t], t) : -1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < N; i += blockDim.x) {
    int s = t0 + i < T ? t0 + i : -1;
#pragma unroll
    for (int m = 0; m < kConvMaxK; ++m) {
      if (m < K) {
        anc[i][m] = s;
        if (s >= 0) s = s >= base ? pl[s - base] : sane_parent(par[s], s);
      }
    }
  }
}

// Whether every tap of the tokens [t0, t0 + n) in the ancestor table is on a
// chain (anc[i][m] = t0 + i - m for m < K) and every token is below T: then
// the kernels take all inputs from the tile without per-tap checks.
__device__ __forceinline__ bool conv_tile_is_chain(const int (*anc)[kConvMaxK], int t0, int n, int T, int K) {
  bool ok = true;
  if (threadIdx.x < n) {
    const int i = threadIdx.x;
    ok = t0 + i < T;
#pragma unroll
    for (int m = 0; m < kConvMaxK; ++m)
      if (m < K) ok = ok && anc[i][m] == t0 + i - m;
  }
  return __syncthreads_and(ok) != 0;
}

// weights of channels c0..c0+7 in tap order m (tap m multiplies the m-th ancestor)
// With K = 4 and a 16-byte aligned w, the 8 channels' taps are 32
// consecutive floats, read as eight 16-byte loads: per-element loads touch a
// different cache line in every lane and kept the texture unit busy.
template <int KM>
__device__ __forceinline__ void conv_weights(const float* __restrict__ w, int c0, int K, float (*wr)[8]) {
  if (KM >= 4 && K == 4 && (reinterpret_cast<uintptr_t>(w) & 15) == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const f32x4 f = *reinterpret_cast<const f32x4*>(w + (size_t)(c0 + e) * 4);
#pragma unroll
      for (int m = 0; m < 4; ++m) wr[m][e] = f[3 - m];
#pragma unroll
      for (int m = 4; m < KM; ++m) wr[m][e] = 0.0f;
    }
    return;
  }
#pragma unroll
  for (int m = 0; m < KM; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) wr[m][e] = m < K ? w[(size_t)(c0 + e) * K + (K - 1 - m)] : 0.0f;
}

// Eight channels of one row, kept in the input precision.
template <typename Tio>
struct Raw8;
template <>
struct Raw8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = load8(p); }
  __device__ __forceinline__ void zero() { v = zero8(); }
  __device__ __forceinline__ void get(float* f) const {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (float)v[e];
  }
};
template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = f32x4{}; }
  __device__ __forceinline__ void get(float* f) const {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = a[e];
      f[4 + e] = b[e];
    }
  }
};

// A tile of kConvTB consecutive tokens [t0, t0 + kConvTB) and the KM - 1
// rows before it, loaded up front (independent loads). On a chain (every
// token of a node but its first) the m-th ancestor of t is t - m, which the
// tile holds; other taps are loaded.
template <typename Tio, int KM>
struct ConvTile {
  static constexpr int NR = kConvTB + KM - 1;
  Raw8<Tio> rows[NR];  // rows[r] = x_{t0 - (KM - 1) + r}
  __device__ __forceinline__ void load(const Tio* __restrict__ x, int t0, int T, int C, int c0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int t = t0 - (KM - 1) + r;
      if (t >= 0 && t < T)
        rows[r].load(x + (size_t)t * C + c0);
      else
        rows[r].zero();
    }
  }
  // The same rows without branches: a row outside [0, T) is read from a
  // clamped row and zeroed by fix_edges once it has arrived. Every thread
  // then issues the same loads, so a wait for a load issued before them
  // (the window's parents) leaves them in flight.
  __device__ __forceinline__ void load_all(const Tio* __restrict__ x, int t0, int T, int C, int c0) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int t = min(max(t0 - (KM - 1) + r, 0), T - 1);
      rows[r].load(x + (size_t)t * C + c0);
    }
  }
  __device__ __forceinline__ void fix_edges(int t0, int T) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int t = t0 - (KM - 1) + r;
      if (t < 0 || t >= T) rows[r].zero();
    }
  }
  // a_i += sum over taps of w_m x_{t-m}, for a tile whose every tap is on a
  // chain (the m-th ancestor of t is t - m): all inputs are in the tile
  __device__ __forceinline__ void chain_taps(int i, int K, const float (*wr)[8], float* a) const {
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      if (m < K) {
        float xv[8];
        rows[i + KM - 1 - m].get(xv);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = fmaf(wr[m][e], xv[e], a[e]);
      }
    }
  }
  // input of tap m of tile token i (ancestor s, -1 past a root)
  __device__ __forceinline__ void tap(const Tio* __restrict__ x, int s, int t, int i, int m, int C, int c0,
                                      float* xv) const {
    if (s < 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xv[e] = 0.0f;
    } else if (s == t - m) {
      rows[i + KM - 1 - m].get(xv);
    } else {
      ld8f(x + (size_t)s * C + c0, xv);
    }
  }
};

template <typename Tio, int KM>
__global__ __launch_bounds__(kConvThreads) void conv_fwd_kernel(const Tio* __restrict__ x, const float* __restrict__ w,
                                                                const float* __restrict__ bias,
                                                                const int* __restrict__ par, int T, int C, int K,
                                                                int act, Tio* __restrict__ y) {
  constexpr int NWIN = kConvTB + kConvMaxK - 1;  // tokens whose parents are staged in LDS
  static_assert(NWIN <= 64, "the window's parents are loaded and walked by wave 0");
  __shared__ int anc[kConvTB][kConvMaxK];
  __shared__ int pl[NWIN];
  __shared__ int chain_all;
  const int t0 = blockIdx.x * kConvTB;
  const int c0 = (blockIdx.y * kConvThreads + threadIdx.x) * 8;
  const bool cok = c0 < C;
  const int cl = cok ? c0 : C - 8;  // in-bounds channels for the threads past C (their results are dropped)
  // The window's parents are requested first and the rows, weights and bias
  // after them, all unconditionally: waiting for the parents leaves the rest
  // in flight through the ancestor walk.
  const int base = t0 - (kConvMaxK - 1);
  const int tw = base + (int)threadIdx.x;
  const int pv = par[min(max(tw, 0), T - 1)];
  ConvTile<Tio, KM> tile;
  float wr[KM][8], br[8];
  tile.load_all(x, t0, T, C, cl);
  conv_weights<KM>(w, cl, K, wr);
#pragma unroll
  for (int e = 0; e < 8; ++e) br[e] = bias ? bias[cl + e] : 0.0f;
  if (threadIdx.x < NWIN) pl[threadIdx.x] = (tw >= 0 && tw < T) ? sane_parent(pv, tw) : -1;
  lds_barrier();
  // one thread per token lists its ancestors (HBM only where a walk leaves
  // the window) and checks that every tap lies on a chain
  if (threadIdx.x < 64) {
    bool ok = true;
    if ((int)threadIdx.x < kConvTB) {
      const int i = threadIdx.x;
      int s = t0 + i < T ? t0 + i : -1;
      ok = t0 + i < T;
#pragma unroll
      for (int m = 0; m < kConvMaxK; ++m) {
        if (m < K) {
          anc[i][m] = s;
          ok = ok && s == t0 + i - m;
          if (s >= 0) s = s >= base ? pl[s - base] : sane_parent(par[s], s);
        }
      }
    }
    const bool all = __all(ok);
    if (threadIdx.x == 0) chain_all = all ? 1 : 0;
  }
  lds_barrier();
  const bool chain = chain_all != 0;
  if (!cok) return;
  tile.fix_edges(t0, T);
  if (chain) {
#pragma unroll
    for (int i = 0; i < kConvTB; ++i) {
      float a[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = br[e];
      tile.chain_taps(i, K, wr, a);
      if (act) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = a[e] * sigmoidf(a[e]);
      }
      st8f(y + (size_t)(t0 + i) * C + c0, a);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < kConvTB; ++i) {
    const int t = t0 + i;
    if (t < T) {
      float a[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = br[e];
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        if (m < K) {
          float xv[8];
          tile.tap(x, anc[i][m], t, i, m, C, c0, xv);
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = fmaf(wr[m][e], xv[e], a[e]);
        }
      }
      if (act) {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = a[e] * sigmoidf(a[e]);
      }
      st8f(y + (size_t)t * C + c0, a);
    }
  }
}

// g = dy * act'(a) for a block of kConvTokBlock tokens, plus that block's
// partial sums of dw (per tap) and db (from g in float32). g itself is kept
// in the input precision for the dx pass.
template <typename Tio, int KM>
__global__ __launch_bounds__(kConvThreads) void conv_bwd_g_kernel(
    const Tio* __restrict__ x, const Tio* __restrict__ dy, const float* __restrict__ w,
    const float* __restrict__ bias, const int* __restrict__ par, int T, int C, int K, int act, Tio* __restrict__ gbuf,
    float* __restrict__ part) {
  __shared__ int anc[kConvTokBlock][kConvMaxK];
  __shared__ int pl[kConvTokBlock + kConvMaxK - 1];
  const int tb = blockIdx.x * kConvTokBlock;
  const int c0 = (blockIdx.y * kConvThreads + threadIdx.x) * 8;
  float wr[KM][8], br[8];
  if (c0 < C) {
    conv_weights<KM>(w, c0, K, wr);
#pragma unroll
    for (int e = 0; e < 8; ++e) br[e] = bias ? bias[c0 + e] : 0.0f;
  }
  conv_ancestors<kConvTokBlock>(par, tb, T, K, anc, pl);
  __syncthreads();
  const bool chain = conv_tile_is_chain(anc, tb, kConvTokBlock, T, K);
  if (c0 >= C) return;
  float dw[KM][8], db[8];
#pragma unroll
  for (int m = 0; m < KM; ++m)
#pragma unroll
    for (int e = 0; e < 8; ++e) dw[m][e] = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) db[e] = 0.0f;
  for (int sub = 0; sub < kConvTokBlock; sub += kConvTB) {
    const int ts = tb + sub;
    if (ts >= T) break;
    ConvTile<Tio, KM> tile;
    tile.load(x, ts, T, C, c0);
    // dy one token ahead, from a clamped (always valid) row, so its load is
    // issued before the current token's g store: stores share the wait
    // counter with loads, and a load issued after a store waits for it too
    Raw8<Tio> dcur, dnext;
    dcur.load(dy + (size_t)min(ts, T - 1) * C + c0);
#pragma unroll
    for (int i = 0; i < kConvTB; ++i) {
      const int t = ts + i;
      if (i + 1 < kConvTB) dnext.load(dy + (size_t)min(t + 1, T - 1) * C + c0);
      if (t < T) {
        float a[8], g[8], xt[KM][8];
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = br[e];
#pragma unroll
        for (int m = 0; m < KM; ++m) {
          if (m < K) {
            // a chain block takes every input from the tile, without per-tap checks
            if (chain)
              tile.rows[i + KM - 1 - m].get(xt[m]);
            else
              tile.tap(x, anc[sub + i][m], t, i, m, C, c0, xt[m]);
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = fmaf(wr[m][e], xt[m][e], a[e]);
          }
        }
        dcur.get(g);
        if (act) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float sg = sigmoidf(a[e]);
            g[e] *= sg * (1.0f + a[e] * (1.0f - sg));
          }
        }
        st8f(gbuf + (size_t)t * C + c0, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) db[e] += g[e];
#pragma unroll
        for (int m = 0; m < KM; ++m)
          if (m < K) {
#pragma unroll
            for (int e = 0; e < 8; ++e) dw[m][e] = fmaf(g[e], xt[m][e], dw[m][e]);
          }
      }
      dcur = dnext;
    }
  }
  // partials [block][c][K + 1]: taps in weight order (index K-1-m), then db
  float* pp = part + ((size_t)blockIdx.x * C + c0) * (K + 1);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
#pragma unroll
    for (int m = 0; m < KM; ++m)
      if (m < K) pp[(size_t)e * (K + 1) + (K - 1 - m)] = dw[m][e];
    pp[(size_t)e * (K + 1) + K] = db[e];
  }
}

// dx_j = sum_{t: anc_m(t) = j, m < K} w[:, K-1-m] g_t. The descendants of j
// are the preorder range (j, se[j]); depth below j is pos[t] - pos[j]; a
// token K or more levels down is skipped together with its subtree. One
// thread per token lists (token, depth) pairs in LDS; a token with more than
// kConvMaxDesc of them is walked again by the channel threads.
template <typename Tio, int KM>
__global__ __launch_bounds__(kConvThreads) void conv_bwd_dx_kernel(const Tio* __restrict__ gbuf,
                                                                   const float* __restrict__ w,
                                                                   const int* __restrict__ pos,
                                                                   const int* __restrict__ se, int T, int C, int K,
                                                                   Tio* __restrict__ dx) {
  constexpr int NWIN = kConvTB + kConvMaxK;  // pos / se of [t0, t0 + NWIN) staged in LDS
  __shared__ int dlist[kConvTB][kConvMaxDesc];
  __shared__ int dcount[kConvTB];
  __shared__ int pw[NWIN], sw[NWIN];
  __shared__ int chain_all;
  static_assert(NWIN <= 64 && kConvTB <= 64, "the window is staged and walked by wave 0");
  const int t0 = blockIdx.x * kConvTB;
  const int c0 = (blockIdx.y * kConvThreads + threadIdx.x) * 8;
  const int cl = c0 < C ? c0 : C - 8;  // in-bounds channels for the threads past C (their results are dropped)
  // The window's pos / se first, then (unconditionally, from clamped rows)
  // the g rows a chain tile needs: waiting for the window leaves the g rows
  // in flight through the walk, whose barriers order LDS only.
  const int tw = min(t0 + (int)threadIdx.x, T - 1);
  const int pv = pos[tw], sv = se[tw];
  ConvTile<Tio, KM> gt;  // gt.rows[r] = g_{t0 + r}
  gt.load_all(gbuf, t0 + KM - 1, T, C, cl);
  float wr[KM][8];
  conv_weights<KM>(w, cl, K, wr);
  if (threadIdx.x < NWIN) {
    const bool in = t0 + (int)threadIdx.x < T;
    pw[threadIdx.x] = in ? pv : 0;
    sw[threadIdx.x] = in ? sv : 0;
  }
  lds_barrier();
  // the walk reads LDS inside the window and HBM past it
  auto pos_at = [&](int t) { return t - t0 < NWIN ? pw[t - t0] : pos[t]; };
  auto se_at = [&](int t) { return t - t0 < NWIN ? sw[t - t0] : se[t]; };
  for (int i = threadIdx.x; i < kConvTB; i += blockDim.x) {
    const int j = t0 + i;
    int cnt = 0;
    if (j < T) {
      // subtree ends are clamped into (t, T] and depths below 1 are skipped,
      // so malformed metadata can neither leave [0, T) nor stall the walk
      const int pj = pw[i], end = min(max(sw[i], j + 1), T);
      int t = j + 1;
      while (t < end) {
        const int dd = pos_at(t) - pj;
        if (dd < K) {
          if (dd >= 1) {
            if (cnt < kConvMaxDesc) dlist[i][cnt] = (t << 3) | dd;
            ++cnt;
          }
          ++t;
        } else {
          t = max(se_at(t), t + 1);
        }
      }
    }
    dcount[i] = cnt;
  }
  // chain tile: every token j has exactly the descendants j + 1 .. j + K - 1
  // (depths 1 .. K - 1) within K - 1 levels, so dx_j = sum_m w_m g_{j+m}
  // from a tile of g rows loaded up front
  // (the walk's threads are wave 0's: its own dlist / dcount writes are seen
  // in order, and the other waves wait at the barrier below)
  if (threadIdx.x < 64) {
    bool ch = true;
    if ((int)threadIdx.x < kConvTB) {
      const int i = threadIdx.x, j = t0 + i;
      ch = j < T && dcount[i] == K - 1;
      for (int q = 0; q < K - 1 && ch; ++q) ch = dlist[i][q] == (((j + q + 1) << 3) | (q + 1));
    }
    const bool all = __all(ch);
    if (threadIdx.x == 0) chain_all = all ? 1 : 0;
  }
  lds_barrier();
  const bool chain = chain_all != 0;
  if (c0 >= C) return;
  if (chain) {
    gt.fix_edges(t0 + KM - 1, T);
#pragma unroll
    for (int i = 0; i < kConvTB; ++i) {
      float acc[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int m = 0; m < KM; ++m) {
        if (m < K) {
          float g[8];
          gt.rows[i + m].get(g);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(wr[m][e], g[e], acc[e]);
        }
      }
      st8f(dx + (size_t)(t0 + i) * C + c0, acc);
    }
    return;
  }
  const int n = min(kConvTB, T - t0);
  for (int i = 0; i < n; ++i) {
    const int j = t0 + i;
    float acc[8], g[8];
    ld8f(gbuf + (size_t)j * C + c0, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = wr[0][e] * g[e];
    const int cnt = dcount[i];
    if (cnt <= kConvMaxDesc) {
      for (int q = 0; q < cnt; ++q) {
        const int code = dlist[i][q];
        const int t = code >> 3, dd = code & 7;
        ld8f(gbuf + (size_t)t * C + c0, g);
#pragma unroll
        for (int m = 1; m < KM; ++m)
          if (m == dd) {
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = fmaf(wr[m][e], g[e], acc[e]);
          }
      }
    } else {
      const int pj = pos[j], end = min(max(se[j], j + 1), T);
      int t = j + 1;
      while (t < end) {
        const int dd = pos[t] - pj;
        if (dd < K) {
          if (dd >= 1) {
            ld8f(gbuf + (size_t)t * C + c0, g);
#pragma unroll
            for (int m = 1; m < KM; ++m)
              if (m == dd) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(wr[m][e], g[e], acc[e]);
              }
          }
          ++t;
        } else {
          t = max(se[t], t + 1);
        }
      }
    }
    st8f(dx + (size_t)j * C + c0, acc);
  }
}

// Fixed-order sum of the per-block partials [nblk][C][K + 1]: one thread
// per (channel, tap) value, reading consecutive values across the block's
// threads; eight running sums over block residues, added in a fixed order.
__global__ __launch_bounds__(256) void conv_bwd_reduce_kernel(const float* __restrict__ part, int nblk, int C, int K,
                                                              float* __restrict__ dw, float* __restrict__ db) {
  const int V = C * (K + 1);
  const int vi = blockIdx.x * blockDim.x + threadIdx.x;
  if (vi >= V) return;
  float acc[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) acc[r] = 0.0f;
  int b = 0;
  for (; b + 8 <= nblk; b += 8)
#pragma unroll
    for (int r = 0; r < 8; ++r) acc[r] += part[(size_t)(b + r) * V + vi];
  for (int r = 0; b < nblk; ++b, ++r) acc[r] += part[(size_t)b * V + vi];
  const float sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  const int c = vi / (K + 1), n = vi % (K + 1);
  if (n < K)
    dw[(size_t)c * K + n] = sum;
  else if (db)
    db[c] = sum;
}

// ---------------------------------------------------------------- gated delta rule

constexpr int kCh = 64;  // chunk rows (the plan's chunk size is at most this)

struct GdnLayout {
  size_t gc, u, w, kt, vnt, h0, tt, total;
};

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

GdnLayout gdn_layout(int H, int Hv, int dk, int dv, int nc) {
  GdnLayout L{};
  size_t o = 0;
  L.gc = o;
  o = al256(o + (size_t)Hv * nc * kCh * 4);
  L.u = o;
  o = al256(o + (size_t)Hv * nc * kCh * dv * 4);
  L.w = o;
  o = al256(o + (size_t)Hv * nc * kCh * dk * 2);
  L.kt = o;
  o = al256(o + (size_t)Hv * nc * dk * kCh * 2);
  L.vnt = o;
  o = al256(o + (size_t)Hv * nc * dv * kCh * 2);
  L.h0 = o;
  o = al256(o + (size_t)nc * Hv * dv * dk * 2);
  L.tt = o;
  o = al256(o + (size_t)Hv * nc * kCh * kCh * 2);
  L.total = o;
  return L;
}

// Backward workspace, after the forward's (chunk-local like it):
//   dvlt [Hv][nc] x (dv x 64) f32, column-grouped   (P^T dO)^T
//   kgl  [Hv][nc][64][dk] bf16   k e^(gl - gc), swap23 columns
//   qgt  [Hv][nc][dk][64] bf16   (q e^gc)^T
//   wt   [Hv][nc][dk][64] bf16   w^T
//   dot  [Hv][nc] x (dv x 64) bf16, column-grouped  dO^T
//   dvnt [Hv][nc] x (dv x 64) bf16, column-grouped   dvn^T
//   dhe  [nc][Hv] x (dv x dk) bf16, column-grouped   end-state gradient of each chunk
//   dwt  [Hv][nc] x (dk x 64) bf16, column-grouped   dw^T
//   dgca [Hv][nc][64] f32        decay gradient, output / state part
//   dka  [H][nc][64][dk] f32     dk, output / state part
//   dhead [nch][Hv][dv][dk] f32  start-state gradient of each chain, transposed
struct GdnBwdLayout {
  size_t dvlt, kgl, qgt, wt, dot, dvnt, dhe, dwt, dgca, dka, dhead, total;
};

GdnBwdLayout gdn_bwd_layout(int H, int Hv, int dk, int dv, int nc, int nch) {
  GdnBwdLayout L{};
  size_t o = gdn_layout(H, Hv, dk, dv, nc).total;
  const size_t hn = (size_t)Hv * nc;
  auto take = [&](size_t* at, size_t bytes) {
    *at = o;
    o = al256(o + bytes);
  };
  take(&L.dvlt, hn * dv * kCh * 4);
  take(&L.kgl, hn * kCh * dk * 2);
  take(&L.qgt, hn * dk * kCh * 2);
  take(&L.wt, hn * dk * kCh * 2);
  take(&L.dot, hn * dv * kCh * 2);
  take(&L.dvnt, hn * dv * kCh * 2);
  take(&L.dhe, hn * dv * dk * 2);
  take(&L.dwt, hn * dk * kCh * 2);
  take(&L.dgca, hn * kCh * 4);
  take(&L.dka, (size_t)H * nc * kCh * dk * 4);
  take(&L.dhead, (size_t)nch * Hv * dv * dk * 4);
  L.total = o;
  return L;
}

// Column-grouped layout of the chunk states and of the transposed chunk rows
// (h0 and dh_end: columns dv, rows dk; vn^T and dvn^T: columns dv, rows the
// chunk's 64): 32-column groups, then 32-row blocks, 8-row groups, the 32
// columns and 8 rows. A wave's stores from MFMA C registers (lane = column,
// 4 consecutive rows) are contiguous 512-byte runs, and 8 consecutive rows
// of a column are 16 contiguous bytes. Offset of (column e, row r) within
// one C x R block:
template <int R>
__device__ __forceinline__ int cr_off(int e, int r) {
  return (((e >> 5) * (R / 32) + (r >> 5)) * 4 + ((r & 31) >> 3)) * 256 + (e & 31) * 8 + (r & 7);
}

// A C x R block in the column-grouped layout into LDS rows of stride ls
// (l[e * ls + r]), read in its memory order (coalesced): issue() starts the
// loads, commit() stores them.
template <int C, int R, int NT>
struct CrTileLoad {
  static_assert((C * R / 8) % NT == 0, "whole rounds of the workgroup's threads");
  static constexpr int N = C * R / 8 / NT;
  bf16x8 x[N];
  __device__ __forceinline__ void issue(const bf16* __restrict__ g, int tid) {
#pragma unroll
    for (int it = 0; it < N; ++it) x[it] = load8(g + (size_t)(tid + NT * it) * 8);
  }
  __device__ __forceinline__ void commit(bf16* l, int ls, int tid) const {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int idx = tid + NT * it;
      const int ec = idx & 31, gg = (idx >> 5) & 3, rb = (idx >> 7) % (R / 32), eg = (idx >> 7) / (R / 32);
      *reinterpret_cast<bf16x8*>(l + (32 * eg + ec) * ls + 32 * rb + 8 * gg) = x[it];
    }
  }
};

// T = (I + M)^-1 for a unit lower-triangular 64 x 64 system, by 16 x 16
// blocks: T_ii = (I + M_ii)^-1 by forward substitution (one lane per
// column), then T_ij = -T_ii sum_{j <= q < i} M_iq T_qj one block diagonal
// at a time. mval(r, q) returns M[r][q] (read for q < r only); ts is
// cleared here. All 256 threads of the workgroup take part; ts is complete
// when it returns.
template <class MV>
__device__ __forceinline__ void unit_lower_inverse(MV mval, float (*ts)[kCh + 4], float (*pscr)[16][17], int tid) {
  const int wv = tid >> 6, lane = tid & 63;
  for (int idx = tid; idx < kCh * (kCh + 4); idx += 256) (&ts[0][0])[idx] = 0.0f;
  __syncthreads();
  if (wv == 0) {
    const int bd = 16 * (lane >> 4), j = lane & 15;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == j ? 1.0f : 0.0f;
#pragma unroll
      for (int q = 0; q < r; ++q) acc = fmaf(-mval(bd + r, bd + q), x[q], acc);
      x[r] = acc;
      ts[bd + r][bd + j] = acc;
    }
  }
  __syncthreads();
  const int er = tid >> 4, ec = tid & 15;  // element (row, column) of a 16 x 16 block
#pragma unroll
  for (int d = 1; d < 4; ++d) {
    float part[3];
#pragma unroll
    for (int bi = 0; bi < 4 - d; ++bi) {
      const int bi_ = bi + d, bj = bi;
      float acc = 0.0f;
      for (int q = 16 * bj; q < 16 * bi_; ++q) acc = fmaf(mval(16 * bi_ + er, q), ts[q][16 * bj + ec], acc);
      part[bi] = acc;
    }
    // every thread holds its element of each partial sum; exchange them through LDS
#pragma unroll
    for (int bi = 0; bi < 4 - d; ++bi) pscr[bi][er][ec] = part[bi];
    __syncthreads();
#pragma unroll
    for (int bi = 0; bi < 4 - d; ++bi) {
      const int bi_ = bi + d, bj = bi;
      float acc = 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) acc = fmaf(ts[16 * bi_ + er][16 * bi_ + q], pscr[bi][q][ec], acc);
      ts[16 * bi_ + er][16 * bj + ec] = -acc;
    }
    __syncthreads();
  }
}

// Stage 1: per (chunk, v-head). 256 threads.
//   gc, beta, the decay to the chunk end; M = strictly-lower (beta k) k^T *
//   exp(gc_i - gc_j) (bf16 MFMA); T = (I + M)^-1 in float32 by 16 x 16
//   blocks; then [u | w] = T [beta v | beta k e^gc] as a bf16 MFMA product
//   with the right-hand side transposed in LDS.
template <int DK, int DV>
struct PrepLds {
  static constexpr int NCOL = DK + DV;      // right-hand-side columns
  static constexpr int KS_B = kCh * (DK + 8) * 2;
  static constexpr int TS_B = kCh * (kCh + 4) * 4;
  static constexpr int KT_B = KS_B > TS_B ? KS_B : TS_B;  // k rows, then T (same storage)
};

template <int DK, int DV, typename Tin>
__global__ __launch_bounds__(256) void gdn_prep_kernel(const Tin* __restrict__ k, const Tin* __restrict__ v,
                                                       const float* __restrict__ g, const float* __restrict__ beta,
                                                       const int* __restrict__ cstart, const int* __restrict__ clen,
                                                       int nc, int H, int Hv, float* __restrict__ gcw,
                                                       float* __restrict__ u, bf16* __restrict__ wp,
                                                       bf16* __restrict__ kt, bf16* __restrict__ tt) {
  typedef PrepLds<DK, DV> PL;
  constexpr int NCOL = PL::NCOL;
  __shared__ float gcs[kCh];
  __shared__ float bs[kCh];
  __shared__ float dec[kCh];
  __shared__ float egs[kCh];
  __shared__ __attribute__((aligned(16))) float Ms[kCh][kCh + 4];
  __shared__ __attribute__((aligned(16))) char kt_raw[PL::KT_B];
  __shared__ __attribute__((aligned(16))) bf16 rt[NCOL][kCh + 8];  // right-hand side, transposed
  __shared__ float pscr[3][16][17];                                 // partial sums of the block inverse
  bf16 (*ks)[DK + 8] = reinterpret_cast<bf16 (*)[DK + 8]>(kt_raw);
  float (*ts)[kCh + 4] = reinterpret_cast<float (*)[kCh + 4]>(kt_raw);
  const int c = blockIdx.x, hv = blockIdx.y;
  const int hk = hv / (Hv / H);
  const int t0 = cstart[c], L = clen[c];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  // every HBM read of the chunk is issued here, before any is used: k rows
  // (thread: rows tid / (DK/8) + 256 i / (DK/8), 16 bytes each) and the v
  // half of the right-hand side (rows r = tid % 64, columns 8 (wv + 4 i))
  constexpr int NKL = kCh * (DK / 8) / 256;
  constexpr int NVL = kCh * (DV / 8) / 256;
  static_assert(kCh * (DK / 8) % 256 == 0 && kCh * (DV / 8) % 256 == 0, "whole rounds of the workgroup");
  bf16x8 kl[NKL], vl[NVL];
#pragma unroll
  for (int i = 0; i < NKL; ++i) {
    const int idx = tid + 256 * i, r = idx / (DK / 8), cc = (idx % (DK / 8)) * 8;
    kl[i] = r < L ? load8(k + ((size_t)(t0 + r) * H + hk) * DK + cc) : zero8();
  }
#pragma unroll
  for (int i = 0; i < NVL; ++i) {
    const int idx = tid + 256 * i, r = idx % kCh, cg = 8 * (idx / kCh);
    vl[i] = r < L ? load8(v + ((size_t)(t0 + r) * Hv + hv) * DV + cg) : zero8();
  }
  if (wv == 0) {
    float gv = lane < L ? g[(size_t)(t0 + lane) * Hv + hv] : 0.0f;
    const float bv = lane < L ? beta[(size_t)(t0 + lane) * Hv + hv] : 0.0f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(gv, o);
      if (lane >= o) gv += y;
    }
    gcs[lane] = gv;
    bs[lane] = bv;
    gcw[((size_t)hv * nc + c) * kCh + lane] = gv;
    const float glast = __shfl(gv, 63);  // g is zero past L, so lane 63 holds gc of the last row
    dec[lane] = lane < L ? expf(glast - gv) : 0.0f;
    egs[lane] = lane < L ? expf(gv) : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < NKL; ++i) {
    const int idx = tid + 256 * i, r = idx / (DK / 8), cc = (idx % (DK / 8)) * 8;
    *reinterpret_cast<bf16x8*>(&ks[r][cc]) = kl[i];
  }
  __syncthreads();
  // M (rows m > n only are read): waves 0-2 form the lower 32x32 blocks of k k^T
  if (wv < 3) {
    const int mb = wv == 0 ? 0 : 1, nb = wv == 2 ? 1 : 0;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int a = 0; a < DK / 16; ++a)
      acc = mfma32x32x16(*reinterpret_cast<const bf16x8*>(&ks[32 * mb + lc][16 * a + 8 * lg]),
                         *reinterpret_cast<const bf16x8*>(&ks[32 * nb + lc][16 * a + 8 * lg]), acc);
    const int n = 32 * nb + lc;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = 32 * mb + 8 * (i >> 2) + 4 * lg + (i & 3);
      Ms[m][n] = n < m ? bs[m] * acc[i] * expf(gcs[m] - gcs[n]) : 0.0f;
    }
  }
  // kd^T = (k exp(gc_last - gc))^T, chunk-local, for the state pass
  {
    // 16 bytes per lane, eight lanes per 128-byte row of kd^T
    bf16* kto = kt + ((size_t)hv * nc + c) * DK * kCh;
#pragma unroll
    for (int it = 0; it < DK * (kCh / 8) / 256; ++it) {
      const int idx = tid + 256 * it, kk = idx / (kCh / 8), r0 = 8 * (idx % (kCh / 8));
      bf16x8 o8;
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = (bf16)((float)ks[r0 + e][kk] * dec[r0 + e]);
      *reinterpret_cast<bf16x8*>(kto + (size_t)kk * kCh + r0) = o8;
    }
  }
  // right-hand side, transposed: rt[col][row] = beta v (col < DV), beta k e^gc.
  // Lanes take consecutive rows, 8 columns each (16-byte loads along a row),
  // so each transposed LDS store covers 64 contiguous bytes.
#pragma unroll
  for (int i = 0; i < NVL; ++i) {
    const int idx = tid + 256 * i, r = idx % kCh, cg = 8 * (idx / kCh);
    const float sc = bs[r];
#pragma unroll
    for (int e = 0; e < 8; ++e) rt[cg + e][r] = (bf16)((float)vl[i][e] * sc);
  }
  for (int idx = tid + kCh * (DV / 8); idx < kCh * (NCOL / 8); idx += 256) {
    const int r = idx % kCh, cg = 8 * (idx / kCh);
    const bf16x8 x8 = *reinterpret_cast<const bf16x8*>(&ks[r][cg - DV]);
    const float sc = bs[r] * egs[r];
#pragma unroll
    for (int e = 0; e < 8; ++e) rt[cg + e][r] = (bf16)((float)x8[e] * sc);
  }
  __syncthreads();
  unit_lower_inverse([&](int r, int q) { return Ms[r][q]; }, ts, pscr, tid);
  // T^T for the backward (bf16, the precision its products read T in)
  {
    bf16* tto = tt + ((size_t)hv * nc + c) * kCh * kCh;
#pragma unroll 4
    for (int idx = tid; idx < kCh * kCh; idx += 256) tto[idx] = (bf16)ts[idx % kCh][idx / kCh];
  }
  // [u | w] = T rt^T: 32x32 output blocks (2 row blocks x NCOL/32 column
  // blocks), column blocks dealt to the waves in turn
  constexpr int NCB = NCOL / 32;
  for (int cb = wv; cb < NCB; cb += 4) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int a = 0; a < kCh / 16; ++a) {
        const f32x4 t0v = *reinterpret_cast<const f32x4*>(&ts[32 * mb + lc][16 * a + 8 * lg]);
        const f32x4 t1v = *reinterpret_cast<const f32x4*>(&ts[32 * mb + lc][16 * a + 8 * lg + 4]);
        bf16x8 A;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          A[e] = (bf16)t0v[e];
          A[4 + e] = (bf16)t1v[e];
        }
        acc = mfma32x32x16(A, *reinterpret_cast<const bf16x8*>(&rt[32 * cb + lc][16 * a + 8 * lg]), acc);
      }
      const int col = 32 * cb + lc;
      if (col < DV) {
        float* uo = u + ((size_t)hv * nc + c) * kCh * DV + col;
#pragma unroll
        for (int i = 0; i < 16; ++i) uo[(size_t)(32 * mb + 8 * (i >> 2) + 4 * lg + (i & 3)) * DV] = acc[i];
      } else {
        bf16* wo = wp + ((size_t)hv * nc + c) * kCh * DK + swap23(col - DV);
#pragma unroll
        for (int i = 0; i < 16; ++i) wo[(size_t)(32 * mb + 8 * (i >> 2) + 4 * lg + (i & 3)) * DK] = (bf16)acc[i];
      }
    }
  }
}

// Stage 2: one workgroup per (chain of this level, v-head); wave s owns state
// columns [32 s, 32 s + 32) of dv. The state h (dk x 32 per wave) lives in
// MFMA C registers: block b, register i <-> row 32b + 8(i/4) + 4(lane/32) + i%4.
// Per chunk the workgroup reads w (swizzled [64][dk]), kd^T (dk/64 swizzled
// [64][64] tiles) and u ([64][dv]) from LDS; the next chunk's copies are in
// flight meanwhile.
template <int DK, int DV>
struct StateBuf {
  bf16* w;
  bf16* k;
  float* u;
};

template <int DK, int DV>
__device__ __forceinline__ void gdn_state_chunk(const StateBuf<DK, DV>& sb, float gl, int lg, int lc, int n,
                                                f32x16 (&h)[DK / 32], bf16* __restrict__ vo, bf16* __restrict__ ho) {
  constexpr int NB = DK / 32;
  // store the start state (bf16, column-grouped: column n, rows of dk)
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (bf16)h[b][4 * j + e];
      *reinterpret_cast<bf16x4*>(ho + cr_off<DK>(n, 32 * b + 8 * j + 4 * lg)) = x;
    }
  // vn = u - w h0: B operand of k-step a = -h0 registers 8(a%2)..+7 of block a/2
  // (w's columns are stored in the matching swap23 order)
  bf16x8 hb[DK / 16];
#pragma unroll
  for (int a = 0; a < DK / 16; ++a)
#pragma unroll
    for (int s = 0; s < 8; ++s) hb[a][s] = (bf16)(-h[a >> 1][8 * (a & 1) + s]);
  f32x16 vn[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) vn[mb][i] = sb.u[(32 * mb + 8 * (i >> 2) + 4 * lg + (i & 3)) * DV + n];
#pragma unroll
    for (int a = 0; a < DK / 16; ++a)
      vn[mb] = mfma32x32x16(lds128(sb.w + toff<DK>(32 * mb + lc, 16 * a + 8 * lg)), hb[a], vn[mb]);
  }
  // vn^T (column-grouped: column n, the chunk's rows), for the output stage
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (bf16)vn[mb][4 * j + e];
      *reinterpret_cast<bf16x4*>(vo + cr_off<kCh>(n, 32 * mb + 8 * j + 4 * lg)) = x;
    }
  // h = exp(gc_last) h0 + kd^T vn. Contraction over the chunk rows in the
  // order whose k-step a, slot s is row 16a + 8(s/4) + 4(lane/32) + s%4 =
  // vn register 8(a%2)+s of block a/2; kd^T is read in the same row order.
  const float al = expf(gl);
#pragma unroll
  for (int b = 0; b < NB; ++b) h[b] *= al;
  bf16x8 vb[4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int s = 0; s < 8; ++s) vb[a][s] = (bf16)vn[a >> 1][8 * (a & 1) + s];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bf16* kt = sb.k + (b >> 1) * 64 * kCh;
    const int rr = 32 * (b & 1) + lc;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const bf16x8 A = cat(*reinterpret_cast<const bf16x4*>(kt + toff<kCh>(rr, 16 * a + 4 * lg)),
                           *reinterpret_cast<const bf16x4*>(kt + toff<kCh>(rr, 16 * a + 8 + 4 * lg)));
      h[b] = mfma32x32x16(A, vb[a], h[b]);
    }
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(64 * (DV / 32)) void gdn_state_kernel(
    const int* __restrict__ level_chains, int lvl0, const int* __restrict__ chain_begin,
    const int* __restrict__ cpar, int nc, int Hv, const float* __restrict__ gcw, const float* __restrict__ u,
    const bf16* __restrict__ wp, const bf16* __restrict__ kd, bf16* __restrict__ vnt, bf16* __restrict__ h0w) {
  constexpr int NW = DV / 32;
  constexpr int NB = DK / 32;
  __shared__ __attribute__((aligned(1024))) bf16 w0[kCh * DK];
  __shared__ __attribute__((aligned(1024))) bf16 w1[kCh * DK];
  __shared__ __attribute__((aligned(1024))) bf16 k0[DK * kCh];
  __shared__ __attribute__((aligned(1024))) bf16 k1[DK * kCh];
  __shared__ __attribute__((aligned(1024))) float u0[kCh * DV];
  __shared__ __attribute__((aligned(1024))) float u1[kCh * DV];
  const int ch = level_chains[lvl0 + blockIdx.x];
  const int hv = blockIdx.y;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lg = lane >> 5, lc = lane & 31;
  const int n = 32 * wv + lc;  // state column (dv index) of this lane
  const int cb = chain_begin[ch], ce = chain_begin[ch + 1];
  const int p = cpar[cb];
  TileDma<DK, false, NW> wdma;
  TileDma<kCh, false, NW> kdma;
  wdma.init(wv, lane);
  kdma.init(wv, lane);
  auto issue = [&](int c, bf16* wb, bf16* kb, float* ub) {
    const size_t hc = (size_t)hv * nc + c;
    wdma.issue(wp + hc * kCh * DK, wb, wv);
#pragma unroll
    for (int t = 0; t < DK / 64; ++t) kdma.issue(kd + (hc * DK + 64 * t) * kCh, kb + t * 64 * kCh, wv);
    const float* us = u + hc * kCh * DV;
#pragma unroll
    for (int j = wv; j < kCh * DV / 256; j += NW) dma16(us + 256 * j + 4 * lane, ub + 256 * j);
  };
  f32x16 h[NB];
  if (p < 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) h[b] = f32x16{};
  } else {
    // the start state of p's first child chunk p + 1 is p's end state
    const bf16* hp = h0w + ((size_t)(p + 1) * Hv + hv) * DV * DK;
    bf16x4 x[NB][4];  // every piece requested before any is converted
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) x[b][j] = *reinterpret_cast<const bf16x4*>(hp + cr_off<DK>(n, 32 * b + 8 * j + 4 * lg));
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) h[b][4 * j + e] = (float)x[b][j][e];
  }
  const StateBuf<DK, DV> sb0{w0, k0, u0}, sb1{w1, k1, u1};
  auto gl_of = [&](int c) { return gcw[((size_t)hv * nc + c) * kCh + kCh - 1]; };
  auto out_ptrs = [&](int c, bf16** vo, bf16** ho) {
    *vo = vnt + ((size_t)hv * nc + c) * DV * kCh;
    *ho = h0w + ((size_t)c * Hv + hv) * DV * DK;
  };
  issue(cb, w0, k0, u0);
  float gl0 = gl_of(cb), gl1 = 0.0f;
  for (int c = cb; c < ce; c += 2) {
    bf16 *vo, *ho;
    wait_dma();
    __syncthreads();
    if (c + 1 < ce) {
      issue(c + 1, w1, k1, u1);
      gl1 = gl_of(c + 1);
    }
    out_ptrs(c, &vo, &ho);
    gdn_state_chunk<DK, DV>(sb0, gl0, lg, lc, n, h, vo, ho);
    if (c + 1 < ce) {
      wait_dma();
      __syncthreads();
      if (c + 2 < ce) {
        issue(c + 2, w0, k0, u0);
        gl0 = gl_of(c + 2);
      }
      out_ptrs(c + 1, &vo, &ho);
      gdn_state_chunk<DK, DV>(sb1, gl1, lg, lc, n, h, vo, ho);
    }
  }
}

// Stage 3: per (chunk, v-head), 256 threads. Wave w: query rows 32(w%2) ..
// +31 (one per lane), dv blocks of 32 assigned by w/2. Works on O^T so that
// each lane owns one query: S^T = K Q^T, then O^T += vn^T P^T (P^T from the
// C registers; vn read in the matching row order) and O^T += h0^T (q e^gc)^T.
template <int DK, int DV, typename Tio>
__global__ __launch_bounds__(256) void gdn_out_kernel(const Tio* __restrict__ q, const Tio* __restrict__ k,
                                                      const int* __restrict__ cstart, const int* __restrict__ clen,
                                                      int nc, int H, int Hv, const float* __restrict__ gcw,
                                                      const bf16* __restrict__ vnt, const bf16* __restrict__ h0w,
                                                      Tio* __restrict__ o) {
  constexpr int NDW = DV / 64;  // 32-wide dv blocks per wave
  const int c = blockIdx.x, hv = blockIdx.y;
  const int hk = hv / (Hv / H);
  const int t0 = cstart[c], L = clen[c];
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, lg = lane >> 5, lc = lane & 31;
  const int qb = wv & 1;
  const int i = 32 * qb + lc;
  const bool qok = i < L;
  const size_t hc = (size_t)hv * nc + c;
  const float* gcc = gcw + hc * kCh;
  const float gi = gcc[i];
  bf16x8 qop[DK / 16];
  const Tio* qrow = q + ((size_t)(t0 + (qok ? i : 0)) * H + hk) * DK;
#pragma unroll
  for (int a = 0; a < DK / 16; ++a) qop[a] = qok ? load8(qrow + 16 * a + 8 * lg) : zero8();
  f32x16 acc[NDW];
#pragma unroll
  for (int bb = 0; bb < NDW; ++bb) acc[bb] = f32x16{};
  // inter-chunk term with the chunk's start state
  {
    const float eg = expf(gi);
    bf16x8 qs[DK / 16];
#pragma unroll
    for (int a = 0; a < DK / 16; ++a)
#pragma unroll
      for (int s = 0; s < 8; ++s) qs[a][s] = (bf16)((float)qop[a][s] * eg);
    // all of this wave's h0 operands are requested before the first product
    const bf16* hp = h0w + ((size_t)c * Hv + hv) * DV * DK;
    bf16x8 hA[NDW][DK / 16];
#pragma unroll
    for (int bb = 0; bb < NDW; ++bb)
#pragma unroll
      for (int a = 0; a < DK / 16; ++a)
        hA[bb][a] = load8(hp + cr_off<DK>(32 * (NDW * (wv >> 1) + bb) + lc, 16 * a + 8 * lg));
#pragma unroll
    for (int bb = 0; bb < NDW; ++bb)
#pragma unroll
      for (int a = 0; a < DK / 16; ++a) acc[bb] = mfma32x32x16(hA[bb][a], qs[a], acc[bb]);
  }
  // intra-chunk term; key blocks above the query block are fully masked
  for (int kb = 0; kb <= qb; ++kb) {
    const int j = 32 * kb + lc;
    const bool kok = j < L;
    const Tio* krow = k + ((size_t)(t0 + (kok ? j : 0)) * H + hk) * DK;
    // the block's k rows, vn^T pieces and decays are requested together
    bf16x8 kA[DK / 16];
#pragma unroll
    for (int a = 0; a < DK / 16; ++a) kA[a] = kok ? load8(krow + 16 * a + 8 * lg) : zero8();
    const bf16* vp = vnt + hc * DV * kCh;
    bf16x4 vA[2][NDW][2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int bb = 0; bb < NDW; ++bb) {
        const int d = 32 * (NDW * (wv >> 1) + bb) + lc, a2 = 2 * kb + h2;
        vA[h2][bb][0] = *reinterpret_cast<const bf16x4*>(vp + cr_off<kCh>(d, 16 * a2 + 4 * lg));
        vA[h2][bb][1] = *reinterpret_cast<const bf16x4*>(vp + cr_off<kCh>(d, 16 * a2 + 8 + 4 * lg));
      }
    float gj[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) gj[r] = gcc[32 * kb + 8 * (r >> 2) + 4 * lg + (r & 3)];
    f32x16 s = f32x16{};
#pragma unroll
    for (int a = 0; a < DK / 16; ++a) s = mfma32x32x16(kA[a], qop[a], s);
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jj = 32 * kb + 8 * (r >> 2) + 4 * lg + (r & 3);
      pb[r >> 3][r & 7] = (bf16)((jj <= i && qok) ? s[r] * expf(gi - gj[r]) : 0.0f);
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int bb = 0; bb < NDW; ++bb) acc[bb] = mfma32x32x16(cat(vA[h2][bb][0], vA[h2][bb][1]), pb[h2], acc[bb]);
  }
  if (qok) {
    Tio* orow = o + ((size_t)(t0 + i) * Hv + hv) * DV;
#pragma unroll
    for (int bb = 0; bb < NDW; ++bb)
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int d = 32 * (NDW * (wv >> 1) + bb) + 8 * j4 + 4 * lg;
#pragma unroll
        for (int e = 0; e < 4; ++e) orow[d + e] = from_f32<Tio>(acc[bb][4 * j4 + e]);
      }
  }
}

// ---------------------------------------------------------------- gated delta rule, backward
//
// Per chunk (L rows, local cumulative log decay gc, gl = gc of the last
// row), with P = (q k^T) exp(gc_i - gc_j) on j <= i, qg = q e^gc,
// kd = k e^(gl - gc), T = (I + M)^-1 and the forward's u, w, vn, h0:
//   o    = qg h0 + P vn,   h_end = e^gl h0 + kd^T vn,   vn = u - w h0,
//   u    = T (beta v),     w     = T (beta k e^gc).
// Given dO and the end-state gradient dh_end (the sum of the child chunks'
// start-state gradients):
//   dvn  = P^T dO + kd dh_end
//   dh0  = qg^T dO - w^T dvn + e^gl dh_end               (to the parent)
//   dq   = dS k + e^gc (dO h0^T),   dS = (dO vn^T) exp(gc_i - gc_j), j <= i
//   dk   = dS^T q + e^(gl-gc) (vn dh_end^T) + [WY part]
//   dw   = -dvn h0^T,  dbv = T^T dvn,  dbk = T^T dw,
//   dM   = -(dbv u^T + dbk w^T) on j < i,   M_ij = beta_i (k_i . k_j) exp(gc_i - gc_j)
//   dv   = beta dbv,   dbeta = v.dbv + e^gc k.dbk + sum_j dM_ij (k_i.k_j) exp(gc_i - gc_j)
//   dk  += beta e^gc dbk + (G + G^T) k,   G_ij = beta_i dM_ij exp(gc_i - gc_j)
// and dgc collects the derivative of every exp(gc ...) factor; dg is its
// reverse cumulative sum inside the chunk.
//   1. prep (all chunks): P^T dO, and the state pass's operands kd (rows,
//      swap23 columns), qg^T, w^T, dO^T;
//   2. state (levels deepest first, each chain from its last chunk back):
//      dh in MFMA accumulators as h in the forward; stores dh_end and dvn;
//   3. out (per chunk and q/k head, looping over its v-heads): dq, the
//      P / h0 / h_end parts of dk and dgc, and dw;
//   4. wy (per chunk and q/k head): T again, dbv, dbk, dM, dv, dbeta, the
//      rest of dk and dgc, dg.

__device__ __forceinline__ int crow(int i, int lg) { return 8 * (i >> 2) + 4 * lg + (i & 3); }

// Sum over the 32 lanes of each half-wave (lanes 0-31 and 32-63): quad
// exchanges and row rotations by DPP, then the two 16-lane rows swapped by a
// swizzle (no memory access).
template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum32(float x) {
  x += dppf<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dppf<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dppf<0x124>(x);  // row_ror 4
  x += dppf<0x128>(x);  // row_ror 8
  return x + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));  // lane ^ 16
}

// 8 elements along the contraction index k0..k0+7: of row r (contiguous) or
// of column c (stride ld)
__device__ __forceinline__ bf16x8 row8(const bf16* X, int ld, int r, int k0) {
  return *reinterpret_cast<const bf16x8*>(X + r * ld + k0);
}
__device__ __forceinline__ bf16x8 col8(const bf16* X, int ld, int c, int k0) {
  bf16x8 v;
#pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = X[(k0 + s) * ld + c];
  return v;
}

// A [R][C] row-major tile (global row stride gs, rows past rows_valid read
// as zero) bound for LDS rows of stride ls: issue() starts all of this
// thread's loads, commit() stores them, so a workgroup keeps every load of a
// tile (and of the tiles issued with it) in flight at once.
template <int R, int C, typename Tsrc, int NT = 256>
struct TileLoad {
  static_assert((R * (C / 8)) % NT == 0, "whole rounds of the workgroup's threads");
  static constexpr int N = R * (C / 8) / NT;
  bf16x8 x[N];
  __device__ __forceinline__ void issue(const Tsrc* __restrict__ g, size_t gs, int tid, int rows_valid) {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int idx = tid + NT * it, r = idx / (C / 8), c = 8 * (idx % (C / 8));
      x[it] = r < rows_valid ? load8(g + r * gs + c) : zero8();
    }
  }
  __device__ __forceinline__ void commit(bf16* l, int ls, int tid) const {
#pragma unroll
    for (int it = 0; it < N; ++it) {
      const int idx = tid + NT * it, r = idx / (C / 8), c = 8 * (idx % (C / 8));
      *reinterpret_cast<bf16x8*>(l + r * ls + c) = x[it];
    }
  }
};

// Stage B1, per (chunk, v-head), 256 threads: dvl^T[e][j] = sum_i dO[i][e]
// P[i][j] (wave: key block w % 2, dv blocks from w / 2), plus the state
// pass operands.
template <int DK, int DV, typename Tio>
__global__ __launch_bounds__(256) void gdn_bwd_prep_kernel(const Tio* __restrict__ q, const Tio* __restrict__ k,
                                                           const Tio* __restrict__ dout, const int* __restrict__ cstart,
                                                           const int* __restrict__ clen, int nc, int H, int Hv,
                                                           const float* __restrict__ gcw, const bf16* __restrict__ wp,
                                                           float* __restrict__ dvlt, bf16* __restrict__ kgl,
                                                           bf16* __restrict__ qgt, bf16* __restrict__ wt,
                                                           bf16* __restrict__ dot) {
  __shared__ __attribute__((aligned(16))) bf16 qs[kCh][DK + 8];
  __shared__ __attribute__((aligned(16))) bf16 ks[kCh][DK + 8];
  __shared__ __attribute__((aligned(16))) bf16 ws_[kCh][DK + 8];
  __shared__ __attribute__((aligned(16))) bf16 dT[DV][kCh + 8];
  __shared__ float gcs[kCh], egs[kCh], decs[kCh];
  const int c = blockIdx.x, hv = blockIdx.y;
  const int hk = hv / (Hv / H);
  const int t0 = cstart[c], L = clen[c];
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  const size_t hc = (size_t)hv * nc + c;
  {
    TileLoad<kCh, DK, Tio> lq, lk;
    TileLoad<kCh, DK, bf16> lw;
    lq.issue(q + ((size_t)t0 * H + hk) * DK, (size_t)H * DK, tid, L);
    lk.issue(k + ((size_t)t0 * H + hk) * DK, (size_t)H * DK, tid, L);
    lw.issue(wp + hc * kCh * DK, DK, tid, kCh);
    // dO rows (lanes over rows, 8 columns each), requested with the tiles
    constexpr int NDL = kCh * (DV / 8) / 256;
    bf16x8 dl[NDL];
#pragma unroll
    for (int it = 0; it < NDL; ++it) {
      const int idx = tid + 256 * it, i = idx % kCh, e0 = 8 * (idx / kCh);
      dl[it] = i < L ? load8(dout + ((size_t)(t0 + i) * Hv + hv) * DV + e0) : zero8();
    }
    if (tid < kCh) {
      const float gv = gcw[hc * kCh + tid], gl = gcw[hc * kCh + kCh - 1];
      gcs[tid] = gv;
      egs[tid] = tid < L ? expf(gv) : 0.0f;
      decs[tid] = tid < L ? expf(gl - gv) : 0.0f;
    }
    lq.commit(&qs[0][0], DK + 8, tid);
    lk.commit(&ks[0][0], DK + 8, tid);
    lw.commit(&ws_[0][0], DK + 8, tid);
    // dO^T into LDS (each transposed LDS store covers 64 contiguous bytes)
#pragma unroll
    for (int it = 0; it < NDL; ++it) {
      const int idx = tid + 256 * it, i = idx % kCh, e0 = 8 * (idx / kCh);
#pragma unroll
      for (int s = 0; s < 8; ++s) dT[e0 + s][i] = dl[it][s];
    }
  }
  __syncthreads();
  // transposed outputs, 16 bytes per lane, eight lanes per 128-byte row:
  // (q e^gc)^T and w^T (w's position p holds column swap23(p)), dO^T
#pragma unroll
  for (int it = 0; it < DK * (kCh / 8) / 256; ++it) {
    const int idx = tid + 256 * it, d = idx / (kCh / 8), i0 = 8 * (idx % (kCh / 8));
    bf16x8 qo, wo;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qo[s] = (bf16)((float)qs[i0 + s][d] * egs[i0 + s]);
      wo[s] = ws_[i0 + s][swap23(d)];
    }
    *reinterpret_cast<bf16x8*>(qgt + (hc * DK + d) * kCh + i0) = qo;
    *reinterpret_cast<bf16x8*>(wt + (hc * DK + d) * kCh + i0) = wo;
  }
  // dO^T in the column-grouped layout, written in its memory order
#pragma unroll
  for (int it = 0; it < DV * (kCh / 8) / 256; ++it) {
    const int idx = tid + 256 * it;
    const int e = 32 * (idx >> 8) + (idx & 31), i0 = 32 * ((idx >> 7) & 1) + 8 * ((idx >> 5) & 3);
    *reinterpret_cast<bf16x8*>(dot + hc * DV * kCh + (size_t)idx * 8) = *reinterpret_cast<const bf16x8*>(&dT[e][i0]);
  }
  // kd rows with swap23 columns (the A operand of dvn += kd dh)
#pragma unroll
  for (int it = 0; it < kCh * (DK / 8) / 256; ++it) {
    const int idx = tid + 256 * it, i = idx / (DK / 8), p0 = 8 * (idx % (DK / 8));
    bf16x8 o8;
#pragma unroll
    for (int s = 0; s < 8; ++s) o8[s] = (bf16)((float)ks[i][swap23(p0 + s)] * decs[i]);
    *reinterpret_cast<bf16x8*>(kgl + (hc * kCh + i) * DK + p0) = o8;
  }
  // P^T dO: S from q rows and k columns; P from the C registers is the B
  // operand of the contraction over i (swap23 row order, dO^T read to match)
  constexpr int NDW = DV / 64;
  const int kb = wv & 1, j = 32 * kb + lc;
  f32x16 acc[NDW];
#pragma unroll
  for (int m = 0; m < NDW; ++m) acc[m] = f32x16{};
  for (int qb = kb; qb < 2; ++qb) {
    f32x16 sv = f32x16{};
#pragma unroll
    for (int a = 0; a < DK / 16; ++a)
      sv = mfma32x32x16(row8(&qs[0][0], DK + 8, 32 * qb + lc, 16 * a + 8 * lg),
                        row8(&ks[0][0], DK + 8, j, 16 * a + 8 * lg), sv);
    bf16x8 pb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 32 * qb + crow(r, lg);
      pb[r >> 3][r & 7] = (bf16)((j <= i && i < L) ? sv[r] * expf(gcs[i] - gcs[j]) : 0.0f);
    }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int a2 = 2 * qb + h2;
#pragma unroll
      for (int m = 0; m < NDW; ++m) {
        const int e = 32 * ((wv >> 1) + 2 * m) + lc;
        const bf16x8 A = cat(*reinterpret_cast<const bf16x4*>(&dT[e][16 * a2 + 4 * lg]),
                             *reinterpret_cast<const bf16x4*>(&dT[e][16 * a2 + 8 + 4 * lg]));
        acc[m] = mfma32x32x16(A, pb[h2], acc[m]);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NDW; ++m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int e = 32 * ((wv >> 1) + 2 * m) + crow(r, lg);
      dvlt[hc * DV * kCh + cr_off<kCh>(e, j)] = acc[m][r];
    }
}

// Stage B2: one workgroup per (chain of this level, v-head), levels deepest
// first; wave s owns dv columns [32 s, 32 s + 32). dh (dk x 32 per wave) in
// MFMA C registers like the forward's h. Per chunk, from its end-state
// gradient: store it, dvn = dvl + kd dh (B from the C registers), store
// dvn^T, dh = e^gl dh + qg^T dO - w^T dvn. The next chunk back (kd, qg^T,
// w^T) streams into LDS meanwhile.
template <int DK>
struct BStateBuf {
  bf16* kg;
  bf16* qt;
  bf16* wt;
};

template <int DK, int DV>
__device__ __forceinline__ void gdn_bwd_state_chunk(const BStateBuf<DK>& sb, float gl, int lg, int lc, int n,
                                                    f32x16 (&dh)[DK / 32], const float* __restrict__ dvl_row,
                                                    const bf16* __restrict__ do_row, bf16* __restrict__ vo,
                                                    bf16* __restrict__ ho) {
  constexpr int NB = DK / 32;
  // dvl and dO of this lane's column, issued first
  f32x4 dl[2][4];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
      dl[mb][j4] = *reinterpret_cast<const f32x4*>(dvl_row + cr_off<kCh>(n, 32 * mb + 8 * j4 + 4 * lg));
  bf16x8 db[4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
    db[a] = cat(*reinterpret_cast<const bf16x4*>(do_row + cr_off<kCh>(n, 16 * a + 4 * lg)),
                *reinterpret_cast<const bf16x4*>(do_row + cr_off<kCh>(n, 16 * a + 8 + 4 * lg)));
  // the end-state gradient (bf16, column-grouped like the forward's start states)
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (bf16)dh[b][4 * j + e];
      *reinterpret_cast<bf16x4*>(ho + cr_off<DK>(n, 32 * b + 8 * j + 4 * lg)) = x;
    }
  bf16x8 hb[DK / 16];
#pragma unroll
  for (int a = 0; a < DK / 16; ++a)
#pragma unroll
    for (int s = 0; s < 8; ++s) hb[a][s] = (bf16)dh[a >> 1][8 * (a & 1) + s];
  f32x16 vn[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
      for (int e = 0; e < 4; ++e) vn[mb][4 * j4 + e] = dl[mb][j4][e];
#pragma unroll
    for (int a = 0; a < DK / 16; ++a)
      vn[mb] = mfma32x32x16(lds128(sb.kg + toff<DK>(32 * mb + lc, 16 * a + 8 * lg)), hb[a], vn[mb]);
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (bf16)vn[mb][4 * j + e];
      *reinterpret_cast<bf16x4*>(vo + cr_off<kCh>(n, 32 * mb + 8 * j + 4 * lg)) = x;
    }
  const float al = expf(gl);
#pragma unroll
  for (int b = 0; b < NB; ++b) dh[b] *= al;
  bf16x8 vb[4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int s = 0; s < 8; ++s) vb[a][s] = (bf16)(-vn[a >> 1][8 * (a & 1) + s]);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const bf16* qt = sb.qt + (b >> 1) * 64 * kCh;
    const bf16* wt = sb.wt + (b >> 1) * 64 * kCh;
    const int rr = 32 * (b & 1) + lc;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const bf16x8 Aq = cat(*reinterpret_cast<const bf16x4*>(qt + toff<kCh>(rr, 16 * a + 4 * lg)),
                            *reinterpret_cast<const bf16x4*>(qt + toff<kCh>(rr, 16 * a + 8 + 4 * lg)));
      dh[b] = mfma32x32x16(Aq, db[a], dh[b]);
      const bf16x8 Aw = cat(*reinterpret_cast<const bf16x4*>(wt + toff<kCh>(rr, 16 * a + 4 * lg)),
                            *reinterpret_cast<const bf16x4*>(wt + toff<kCh>(rr, 16 * a + 8 + 4 * lg)));
      dh[b] = mfma32x32x16(Aw, vb[a], dh[b]);
    }
  }
}

template <int DK, int DV>
__global__ __launch_bounds__(64 * (DV / 32)) void gdn_bwd_state_kernel(
    const int* __restrict__ level_chains, int lvl0, const int* __restrict__ chain_begin,
    const int* __restrict__ child_off, const int* __restrict__ child_chains, int nc, int Hv,
    const float* __restrict__ gcw, const float* __restrict__ dvlt, const bf16* __restrict__ kgl,
    const bf16* __restrict__ qgt, const bf16* __restrict__ wt, const bf16* __restrict__ dot, bf16* __restrict__ dvnt,
    bf16* __restrict__ dhe, float* __restrict__ dhead) {
  constexpr int NW = DV / 32;
  constexpr int NB = DK / 32;
  __shared__ __attribute__((aligned(1024))) bf16 g0[kCh * DK];
  __shared__ __attribute__((aligned(1024))) bf16 g1[kCh * DK];
  __shared__ __attribute__((aligned(1024))) bf16 q0[DK * kCh];
  __shared__ __attribute__((aligned(1024))) bf16 q1[DK * kCh];
  __shared__ __attribute__((aligned(1024))) bf16 x0[DK * kCh];
  __shared__ __attribute__((aligned(1024))) bf16 x1[DK * kCh];
  const int ch = level_chains[lvl0 + blockIdx.x];
  const int hv = blockIdx.y;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, lg = lane >> 5, lc = lane & 31;
  const int n = 32 * wv + lc;  // dv column of this lane
  const int cb = chain_begin[ch], ce = chain_begin[ch + 1];
  TileDma<DK, false, NW> gdma;
  TileDma<kCh, false, NW> tdma;
  gdma.init(wv, lane);
  tdma.init(wv, lane);
  auto issue = [&](int c, bf16* gb, bf16* qb, bf16* xb) {
    const size_t hc = (size_t)hv * nc + c;
    gdma.issue(kgl + hc * kCh * DK, gb, wv);
#pragma unroll
    for (int t = 0; t < DK / 64; ++t) {
      tdma.issue(qgt + (hc * DK + 64 * t) * kCh, qb + t * 64 * kCh, wv);
      tdma.issue(wt + (hc * DK + 64 * t) * kCh, xb + t * 64 * kCh, wv);
    }
  };
  f32x16 dh[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) dh[b] = f32x16{};
  // add the start-state gradients of the chains that begin under chunk c
  auto add_children = [&](int c) {
    for (int x = child_off[c]; x < child_off[c + 1]; ++x) {
      const float* hp = dhead + (((size_t)child_chains[x] * Hv + hv) * DV + n) * DK;
      // the child's whole gradient is requested before it is added
      f32x4 v[NB][4];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) v[b][j4] = *reinterpret_cast<const f32x4*>(hp + 32 * b + 8 * j4 + 4 * lg);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4)
#pragma unroll
          for (int e = 0; e < 4; ++e) dh[b][4 * j4 + e] += v[b][j4][e];
    }
  };
  const BStateBuf<DK> sb0{g0, q0, x0}, sb1{g1, q1, x1};
  auto gl_of = [&](int c) { return gcw[((size_t)hv * nc + c) * kCh + kCh - 1]; };
  auto run = [&](const BStateBuf<DK>& sb, int c, float gl) {
    const size_t hc = (size_t)hv * nc + c;
    gdn_bwd_state_chunk<DK, DV>(sb, gl, lg, lc, n, dh, dvlt + hc * DV * kCh, dot + hc * DV * kCh,
                                dvnt + hc * DV * kCh, dhe + ((size_t)c * Hv + hv) * DV * DK);
  };
  add_children(ce - 1);
  issue(ce - 1, g0, q0, x0);
  float gl0 = gl_of(ce - 1), gl1 = 0.0f;
  for (int c = ce - 1; c >= cb; c -= 2) {
    wait_dma();
    __syncthreads();
    if (c - 1 >= cb) {
      issue(c - 1, g1, q1, x1);
      gl1 = gl_of(c - 1);
    }
    run(sb0, c, gl0);
    if (c - 1 >= cb) {
      add_children(c - 1);
      wait_dma();
      __syncthreads();
      if (c - 2 >= cb) {
        issue(c - 2, g0, q0, x0);
        gl0 = gl_of(c - 2);
      }
      run(sb1, c - 1, gl1);
      if (c - 2 >= cb) add_children(c - 2);
    }
  }
  // dh is the start-state gradient of the chain's first chunk
  float* hp = dhead + (((size_t)ch * Hv + hv) * DV + n) * DK;
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j4 = 0; j4 < 4; ++j4) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = dh[b][4 * j4 + e];
      *reinterpret_cast<f32x4*>(hp + 32 * b + 8 * j4 + 4 * lg) = v;
    }
}

// The three lower 32 x 32 blocks of a 64 x 64 chunk matrix: (row block,
// column block) of block 0, 1, 2.
__device__ __forceinline__ int lower_mb(int b) { return b == 0 ? 0 : 1; }
__device__ __forceinline__ int lower_nb(int b) { return b == 2 ? 1 : 0; }

// Stage B3, per (chunk, q/k head), looping over the v-heads that read the
// head. Eight waves; wave w owns output block (row block w % 2, column block
// w / 2) of the 64 x dk results (dq, dk, dw); waves 0-2 own the lower blocks
// of the chunk matrices (S, dS), waves 4-6 form dP for them.
template <int DK, int DV>
struct BwdOutLds {
  bf16 q[kCh][DK + 8];
  bf16 k[kCh][DK + 8];
  bf16 dO[kCh][DV + 8];
  bf16 vnT[DV][kCh + 8];
  bf16 dvnT[DV][kCh + 8];
  bf16 hb[DV][DK + 8];  // h0, then dh_end, as [dv][dk]
  bf16 dS[kCh][kCh + 8];
  float dpx[3][16][64];  // dP of the lower blocks, C-register order
  float gc[kCh], eg[kCh], dec[kCh];
  float rs[4][kCh], rz[4][kCh];  // by column block
  float er[3][kCh], ec[3][kCh];  // row / column sums of dP * P, by lower block
  float red[8];
};

template <int DK, int DV, typename Tio>
__global__ __launch_bounds__(512) void gdn_bwd_out_kernel(const Tio* __restrict__ q, const Tio* __restrict__ k,
                                                          const Tio* __restrict__ dout, const int* __restrict__ cstart,
                                                          const int* __restrict__ clen, int nc, int H, int Hv,
                                                          const float* __restrict__ gcw, const bf16* __restrict__ vnt,
                                                          const bf16* __restrict__ h0w, const bf16* __restrict__ dvnt,
                                                          const bf16* __restrict__ dhe, Tio* __restrict__ dq,
                                                          float* __restrict__ dka, float* __restrict__ dgca,
                                                          bf16* __restrict__ dwt) {
  __shared__ __attribute__((aligned(16))) BwdOutLds<DK, DV> sm;
  const int c = blockIdx.x, hk = blockIdx.y, r = Hv / H;
  const int t0 = cstart[c], L = clen[c];
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  const int rb = wv & 1, cb = wv >> 1;
  const bool own = cb < DK / 32;
  const int col = 32 * cb + lc;  // dk column of this lane's output block
  {
    TileLoad<kCh, DK, Tio, 512> lq, lk;
    lq.issue(q + ((size_t)t0 * H + hk) * DK, (size_t)H * DK, tid, L);
    lk.issue(k + ((size_t)t0 * H + hk) * DK, (size_t)H * DK, tid, L);
    lq.commit(&sm.q[0][0], DK + 8, tid);
    lk.commit(&sm.k[0][0], DK + 8, tid);
  }
  f32x16 aq = f32x16{}, ak = f32x16{};
  for (int mv = 0; mv < r; ++mv) {
    const int hv = hk * r + mv;
    const size_t hc = (size_t)hv * nc + c;
    __syncthreads();
    if (tid < kCh) {
      const float gv = gcw[hc * kCh + tid], gl = gcw[hc * kCh + kCh - 1];
      sm.gc[tid] = gv;
      sm.eg[tid] = tid < L ? expf(gv) : 0.0f;
      sm.dec[tid] = tid < L ? expf(gl - gv) : 0.0f;
    }
    TileLoad<kCh, DV, Tio, 512> ldo;
    CrTileLoad<DV, kCh, 512> lvn, ldvn;
    CrTileLoad<DV, DK, 512> lh0, ldh;
    ldo.issue(dout + ((size_t)t0 * Hv + hv) * DV, (size_t)Hv * DV, tid, L);
    lvn.issue(vnt + hc * DV * kCh, tid);
    ldvn.issue(dvnt + hc * DV * kCh, tid);
    lh0.issue(h0w + ((size_t)c * Hv + hv) * DV * DK, tid);
    ldo.commit(&sm.dO[0][0], DV + 8, tid);
    lvn.commit(&sm.vnT[0][0], kCh + 8, tid);
    ldvn.commit(&sm.dvnT[0][0], kCh + 8, tid);
    lh0.commit(&sm.hb[0][0], DK + 8, tid);
    __syncthreads();
    // S = q k^T on the lower blocks (waves 0-2); dP = dO vn^T (waves 4-6)
    f32x16 sv = f32x16{};
    if (wv >= 4 && wv < 7) {
      const int bl = wv - 4;
      f32x16 dp = f32x16{};
#pragma unroll
      for (int a = 0; a < DV / 16; ++a)
        dp = mfma32x32x16(row8(&sm.dO[0][0], DV + 8, 32 * lower_mb(bl) + lc, 16 * a + 8 * lg),
                          col8(&sm.vnT[0][0], kCh + 8, 32 * lower_nb(bl) + lc, 16 * a + 8 * lg), dp);
#pragma unroll
      for (int x = 0; x < 16; ++x) sm.dpx[bl][x][lane] = dp[x];
    } else if (wv < 3) {
#pragma unroll
      for (int a = 0; a < DK / 16; ++a)
        sv = mfma32x32x16(row8(&sm.q[0][0], DK + 8, 32 * lower_mb(wv) + lc, 16 * a + 8 * lg),
                          row8(&sm.k[0][0], DK + 8, 32 * lower_nb(wv) + lc, 16 * a + 8 * lg), sv);
    } else if (wv == 3) {
      for (int idx = lane; idx < 32 * 32; idx += 64) sm.dS[idx >> 5][32 + (idx & 31)] = (bf16)0.0f;
    }
    __syncthreads();
    // dS = dP exp(gc_i - gc_j) on j <= i < L; E = dP * P summed by rows and columns
    if (wv < 3) {
      const int mb = lower_mb(wv), j = 32 * lower_nb(wv) + lc;
      float csum = 0.0f;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int i = 32 * mb + crow(x, lg);
        const bool ok = j <= i && i < L;
        const float gam = ok ? expf(sm.gc[i] - sm.gc[j]) : 0.0f;
        const float dp = sm.dpx[wv][x][lane];
        sm.dS[i][j] = (bf16)(dp * gam);
        const float e = dp * sv[x] * gam;
        const float rsum = sum32(e);
        if (lc == 0) sm.er[wv][i] = rsum;
        csum += e;
      }
      csum += __shfl_xor(csum, 32);
      if (lg == 0) sm.ec[wv][j] = csum;
    }
    __syncthreads();
    // dq += dS k + e^gc (dO h0^T); dk += dS^T q; dw = -dvn h0^T
    f32x16 y = f32x16{};
    if (own) {
      for (int a = 0; a < 2 * (rb + 1); ++a)
        aq = mfma32x32x16(row8(&sm.dS[0][0], kCh + 8, 32 * rb + lc, 16 * a + 8 * lg),
                          col8(&sm.k[0][0], DK + 8, col, 16 * a + 8 * lg), aq);
      for (int a = 2 * rb; a < 4; ++a)
        ak = mfma32x32x16(col8(&sm.dS[0][0], kCh + 8, 32 * rb + lc, 16 * a + 8 * lg),
                          col8(&sm.q[0][0], DK + 8, col, 16 * a + 8 * lg), ak);
      f32x16 x = f32x16{};
#pragma unroll 2
      for (int a = 0; a < DV / 16; ++a) {
        const bf16x8 hB = col8(&sm.hb[0][0], DK + 8, col, 16 * a + 8 * lg);
        x = mfma32x32x16(row8(&sm.dO[0][0], DV + 8, 32 * rb + lc, 16 * a + 8 * lg), hB, x);
        y = mfma32x32x16(col8(&sm.dvnT[0][0], kCh + 8, 32 * rb + lc, 16 * a + 8 * lg), hB, y);
      }
      float pq[16];
#pragma unroll
      for (int i4 = 0; i4 < 16; ++i4) {
        const int row = 32 * rb + crow(i4, lg);
        const float xv = x[i4] * sm.eg[row];
        aq[i4] += xv;
        pq[i4] = sum32(xv * (float)sm.q[row][col]);
      }
      if (lc == 0) {
#pragma unroll
        for (int i4 = 0; i4 < 16; ++i4) sm.rs[cb][32 * rb + crow(i4, lg)] = pq[i4];
      }
    }
    // dh_end loads first, then the dw stores (a load issued after a store
    // would wait for it)
    ldh.issue(dhe + ((size_t)c * Hv + hv) * DV * DK, tid);
    if (own) {
      bf16* wo = dwt + hc * DK * kCh;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (bf16)(-y[4 * j4 + e]);
        *reinterpret_cast<bf16x4*>(wo + cr_off<kCh>(col, 32 * rb + 8 * j4 + 4 * lg)) = o4;
      }
    }
    __syncthreads();
    // dh_end replaces h0 (each thread rewrites the elements it reads); s = <dh_end, h0>
    float sp = 0.0f;
#pragma unroll
    for (int it = 0; it < ldh.N; ++it) {
      const int idx = tid + 512 * it;
      const int e = 32 * ((idx >> 7) / (DK / 32)) + (idx & 31), d0 = 32 * ((idx >> 7) % (DK / 32)) + 8 * ((idx >> 5) & 3);
      const bf16x8 ov = *reinterpret_cast<const bf16x8*>(&sm.hb[e][d0]);
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) sp += (float)ldh.x[it][s2] * (float)ov[s2];
    }
    ldh.commit(&sm.hb[0][0], DK + 8, tid);
    sp = sum32(sp);
    sp += __shfl_xor(sp, 32);
    if (lane == 0) sm.red[wv] = sp;
    __syncthreads();
    // kd-part: x = e^(gl - gc) (vn dh_end^T); dk += x; z_i = sum_d x_id k_id
    if (own) {
      f32x16 x = f32x16{};
#pragma unroll 4
      for (int a = 0; a < DV / 16; ++a)
        x = mfma32x32x16(col8(&sm.vnT[0][0], kCh + 8, 32 * rb + lc, 16 * a + 8 * lg),
                         col8(&sm.hb[0][0], DK + 8, col, 16 * a + 8 * lg), x);
      float pz[16];
#pragma unroll
      for (int i4 = 0; i4 < 16; ++i4) {
        const int row = 32 * rb + crow(i4, lg);
        const float xv = x[i4] * sm.dec[row];
        ak[i4] += xv;
        pz[i4] = sum32(xv * (float)sm.k[row][col]);
      }
      if (lc == 0) {
#pragma unroll
        for (int i4 = 0; i4 < 16; ++i4) sm.rz[cb][32 * rb + crow(i4, lg)] = pz[i4];
      }
    }
    __syncthreads();
    if (tid < kCh) {
      const int i = tid;
      // rows < 32 lie in lower block 0, rows >= 32 in blocks 1 and 2;
      // columns < 32 in blocks 0 and 1, columns >= 32 in block 2
      const float r1 = i < 32 ? sm.er[0][i] : sm.er[1][i] + sm.er[2][i];
      const float c1 = i < 32 ? sm.ec[0][i] + sm.ec[1][i] : sm.ec[2][i];
      float rq = 0.0f, z = 0.0f;
#pragma unroll
      for (int q4 = 0; q4 < DK / 32; ++q4) {
        rq += sm.rs[q4][i];
        z += sm.rz[q4][i];
      }
      float d = r1 - c1 + rq - z;
      float zs = z;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) zs += __shfl_xor(zs, o);
      if (i == L - 1) {
        float sdot = 0.0f;
#pragma unroll
        for (int w8 = 0; w8 < 8; ++w8) sdot += sm.red[w8];
        d += zs + expf(sm.gc[kCh - 1]) * sdot;
      }
      dgca[hc * kCh + i] = d;
    }
  }
  if (own) {
#pragma unroll
    for (int i4 = 0; i4 < 16; ++i4) {
      const int row = 32 * rb + crow(i4, lg);
      if (row < L) dq[((size_t)(t0 + row) * H + hk) * DK + col] = from_f32<Tio>(aq[i4]);
      dka[(((size_t)hk * nc + c) * kCh + row) * DK + col] = ak[i4];
    }
  }
}

template <int DK, int DV, typename Tio>
struct BwdWyLds {
  bf16 k[kCh][DK + 8];
  bf16 vs[kCh][DV + 8];    // v rows of the v-head
  Tio dvs[kCh][DV + 8];    // dv rows, staged for row stores
  bf16 tt[kCh][kCh + 8];    // T^T
  bf16 gs[kCh][kCh + 8];    // G + G^T
  bf16 dbvT[DV][kCh + 8];
  bf16 dbkT[DK][kCh + 8];
  float dmw[3][16][64];     // the dbk w^T half of dM, per lower block, in C-register order
  float gc[kCh], bs[kCh], eg[kCh];
  float r1[4][kCh], r2[4][kCh];  // row sums v.dbv, k.dbk, by column block
  float ra[3][kCh], cs[3][kCh];  // row sums of a = dM Kg, column sums of beta a, by lower block
};

// Eight waves; wave w owns output block (row block w % 2, column block w / 2)
// of the 64 x D results (dbv, dbk, dk). Waves 0-2 own the lower blocks of the
// chunk matrices (Kg, dM); waves 4-6 form the w-half of dM for them.
template <int DK, int DV, typename Tio>
__global__ __launch_bounds__(512) void gdn_bwd_wy_kernel(
    const Tio* __restrict__ k, const Tio* __restrict__ v, const float* __restrict__ beta,
    const int* __restrict__ cstart, const int* __restrict__ clen, int nc, int H, int Hv,
    const float* __restrict__ gcw, const float* __restrict__ u, const bf16* __restrict__ wp,
    const bf16* __restrict__ ttw, const bf16* __restrict__ dvnt, const bf16* __restrict__ dwt,
    const float* __restrict__ dka, const float* __restrict__ dgca, Tio* __restrict__ dk, Tio* __restrict__ dv,
    float* __restrict__ dg, float* __restrict__ dbeta) {
  __shared__ __attribute__((aligned(16))) BwdWyLds<DK, DV, Tio> sm;
  const int c = blockIdx.x, hk = blockIdx.y, r = Hv / H;
  const int t0 = cstart[c], L = clen[c];
  const int tid = threadIdx.x, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lg = lane >> 5, lc = lane & 31;
  const int rb = wv & 1, cb = wv >> 1;
  const bool own_v = cb < DV / 32, own_k = cb < DK / 32;
  {
    TileLoad<kCh, DK, Tio, 512> lk;
    lk.issue(k + ((size_t)t0 * H + hk) * DK, (size_t)H * DK, tid, L);
    lk.commit(&sm.k[0][0], DK + 8, tid);
  }
  f32x16 ak = f32x16{};
  for (int mv = 0; mv < r; ++mv) {
    const int hv = hk * r + mv;
    const size_t hc = (size_t)hv * nc + c;
    __syncthreads();
    {
      TileLoad<kCh, kCh, bf16, 512> ltt;
      TileLoad<kCh, DV, Tio, 512> lv;
      ltt.issue(ttw + hc * kCh * kCh, kCh, tid, kCh);
      lv.issue(v + ((size_t)t0 * Hv + hv) * DV, (size_t)Hv * DV, tid, L);
      if (tid < kCh) {
        const float gv = gcw[hc * kCh + tid];
        sm.gc[tid] = gv;
        sm.bs[tid] = tid < L ? beta[(size_t)(t0 + tid) * Hv + hv] : 0.0f;
        sm.eg[tid] = tid < L ? expf(gv) : 0.0f;
      }
      ltt.commit(&sm.tt[0][0], kCh + 8, tid);
      lv.commit(&sm.vs[0][0], DV + 8, tid);
    }
    __syncthreads();
    // Kg = (k_i . k_j) exp(gc_i - gc_j) on j < i, kept in registers (waves 0-2)
    f32x16 kgr = f32x16{};
    if (wv < 3) {
      const int mb = lower_mb(wv), j = 32 * lower_nb(wv) + lc;
#pragma unroll 4
      for (int a = 0; a < DK / 16; ++a)
        kgr = mfma32x32x16(row8(&sm.k[0][0], DK + 8, 32 * mb + lc, 16 * a + 8 * lg),
                           row8(&sm.k[0][0], DK + 8, j, 16 * a + 8 * lg), kgr);
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int i = 32 * mb + crow(x, lg);
        kgr[x] = j < i ? kgr[x] * expf(sm.gc[i] - sm.gc[j]) : 0.0f;
      }
    }
    // dbv = T^T dvn (block rb, cb), dv = beta dbv; T[i][j] = 0 for i < j, so
    // rows j of block rb need i >= 32 rb. Right-hand sides are HBM / L2 rows.
    if (own_v) {
      const int e = 32 * cb + lc;
      const bf16* dvb = dvnt + hc * DV * kCh;
      // the block's right-hand sides are requested before the first product
      bf16x8 B[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (a >= 2 * rb) B[a] = load8(dvb + cr_off<kCh>(e, 16 * a + 8 * lg));
      f32x16 acc = f32x16{};
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (a >= 2 * rb) acc = mfma32x32x16(row8(&sm.tt[0][0], kCh + 8, 32 * rb + lc, 16 * a + 8 * lg), B[a], acc);
      float pv[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int j = 32 * rb + crow(x, lg);
        sm.dvs[j][e] = from_f32<Tio>(sm.bs[j] * acc[x]);
        pv[x] = sum32(acc[x] * (float)sm.vs[j][e]);
      }
      if (lc == 0) {
#pragma unroll
        for (int x = 0; x < 16; ++x) sm.r1[cb][32 * rb + crow(x, lg)] = pv[x];
      }
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        bf16x4 o4;
#pragma unroll
        for (int x = 0; x < 4; ++x) o4[x] = (bf16)acc[4 * j4 + x];
        *reinterpret_cast<bf16x4*>(&sm.dbvT[e][32 * rb + 8 * j4 + 4 * lg]) = o4;
      }
    }
    // dbk = T^T dw; dk += beta e^gc dbk
    if (own_k) {
      const int d = 32 * cb + lc;
      const bf16* dwb = dwt + hc * DK * kCh;
      bf16x8 B[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (a >= 2 * rb) B[a] = load8(dwb + cr_off<kCh>(d, 16 * a + 8 * lg));
      f32x16 acc = f32x16{};
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (a >= 2 * rb) acc = mfma32x32x16(row8(&sm.tt[0][0], kCh + 8, 32 * rb + lc, 16 * a + 8 * lg), B[a], acc);
      float pk[16];
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int j = 32 * rb + crow(x, lg);
        ak[x] += sm.bs[j] * sm.eg[j] * acc[x];
        pk[x] = sum32(acc[x] * (float)sm.k[j][d]);
      }
      if (lc == 0) {
#pragma unroll
        for (int x = 0; x < 16; ++x) sm.r2[cb][32 * rb + crow(x, lg)] = pk[x];
      }
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        bf16x4 o4;
#pragma unroll
        for (int x = 0; x < 4; ++x) o4[x] = (bf16)acc[4 * j4 + x];
        *reinterpret_cast<bf16x4*>(&sm.dbkT[d][32 * rb + 8 * j4 + 4 * lg]) = o4;
      }
    }
    __syncthreads();
    // dM = -(dbv u^T + dbk w^T) on the lower blocks: waves 4-6 form the w
    // half and hand it over through LDS; u, w rows come from HBM / L2
    f32x16 dmacc = f32x16{};
    if (wv >= 4 && wv < 7) {
      const int bl = wv - 4;
      const int i0 = 32 * lower_mb(bl) + lc, j0 = 32 * lower_nb(bl) + lc;
      const bf16* wrow = wp + (hc * kCh + j0) * DK;
#pragma unroll 4
      for (int a = 0; a < DK / 16; ++a) {
        bf16x8 A;
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) A[s2] = sm.dbkT[swap23(16 * a + 8 * lg + s2)][i0];
        dmacc = mfma32x32x16(A, load8(wrow + 16 * a + 8 * lg), dmacc);
      }
#pragma unroll
      for (int x = 0; x < 16; ++x) sm.dmw[bl][x][lane] = dmacc[x];
    } else if (wv < 3) {
      const int j0 = 32 * lower_nb(wv) + lc, i0 = 32 * lower_mb(wv) + lc;
      const float* urow = u + (hc * kCh + j0) * DV;
#pragma unroll 4
      for (int a = 0; a < DV / 16; ++a)
        dmacc = mfma32x32x16(col8(&sm.dbvT[0][0], kCh + 8, i0, 16 * a + 8 * lg), load8(urow + 16 * a + 8 * lg), dmacc);
    }
    __syncthreads();
    // a = dM Kg and G = beta_i dM exp(gc_i - gc_j) where j < i < L. G goes to
    // gs at (i, j) and (j, i) by the owner of (i, j); the diagonal is zero.
    if (wv < 3) {
      const int mb = lower_mb(wv), j0 = 32 * lower_nb(wv) + lc;
      float csum = 0.0f;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int i = 32 * mb + crow(x, lg);
        const bool ok = j0 < i && i < L;
        const float dm = -(dmacc[x] + sm.dmw[wv][x][lane]);
        const float av = ok ? dm * kgr[x] : 0.0f;
        const float gv = ok ? sm.bs[i] * dm * expf(sm.gc[i] - sm.gc[j0]) : 0.0f;
        if (j0 < i) {
          sm.gs[i][j0] = (bf16)gv;
          sm.gs[j0][i] = (bf16)gv;
        } else if (j0 == i) {
          sm.gs[i][i] = (bf16)0.0f;
        }
        const float rs = sum32(av);
        if (lc == 0) sm.ra[wv][i] = rs;
        csum += sm.bs[i] * av;
      }
      csum += __shfl_xor(csum, 32);
      if (lg == 0) sm.cs[wv][j0] = csum;
    }
    __syncthreads();
    // dv rows out (rows past the chunk are not written), after the dM phase's
    // row loads: a load issued after a store would wait for it
#pragma unroll
    for (int it = 0; it < kCh * (DV / 8) / 512; ++it) {
      const int idx = tid + 512 * it, j = idx / (DV / 8), e0 = 8 * (idx % (DV / 8));
      if (j < L) {
        Tio* o = dv + ((size_t)(t0 + j) * Hv + hv) * DV + e0;
        if constexpr (sizeof(Tio) == 2) {
          *reinterpret_cast<bf16x8*>(o) = *reinterpret_cast<const bf16x8*>(&sm.dvs[j][e0]);
        } else {
          reinterpret_cast<f32x4*>(o)[0] = reinterpret_cast<const f32x4*>(&sm.dvs[j][e0])[0];
          reinterpret_cast<f32x4*>(o)[1] = reinterpret_cast<const f32x4*>(&sm.dvs[j][e0])[1];
        }
      }
    }
    // dk += (G + G^T) k
    if (own_k) {
      const int d = 32 * cb + lc;
#pragma unroll
      for (int a = 0; a < 4; ++a)
        ak = mfma32x32x16(row8(&sm.gs[0][0], kCh + 8, 32 * rb + lc, 16 * a + 8 * lg),
                          col8(&sm.k[0][0], DK + 8, d, 16 * a + 8 * lg), ak);
    }
    if (tid < kCh) {
      const int i = tid;
      // row sums: rows < 32 lie in lower block 0, rows >= 32 in blocks 1 and
      // 2; columns < 32 in blocks 0 and 1, columns >= 32 in block 2
      const float ra = i < 32 ? sm.ra[0][i] : sm.ra[1][i] + sm.ra[2][i];
      const float cbs = i < 32 ? sm.cs[0][i] + sm.cs[1][i] : sm.cs[2][i];
      float zv = 0.0f, zk = 0.0f;
#pragma unroll
      for (int q = 0; q < DV / 32; ++q) zv += sm.r1[q][i];
#pragma unroll
      for (int q = 0; q < DK / 32; ++q) zk += sm.r2[q][i];
      const float db = zv + sm.eg[i] * zk + ra;
      float x = i < L ? dgca[hc * kCh + i] + sm.bs[i] * sm.eg[i] * zk + sm.bs[i] * ra - cbs : 0.0f;
      // dg_t = sum of dgc_i over i >= t in the chunk
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_down(x, o);
        if (i + o < 64) x += y;
      }
      if (i < L) {
        dg[(size_t)(t0 + i) * Hv + hv] = x;
        dbeta[(size_t)(t0 + i) * Hv + hv] = db;
      }
    }
  }
  if (own_k) {
    const int d = 32 * cb + lc;
    float pa[16];
#pragma unroll
    for (int x = 0; x < 16; ++x) pa[x] = dka[(((size_t)hk * nc + c) * kCh + 32 * rb + crow(x, lg)) * DK + d];
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int row = 32 * rb + crow(x, lg);
      if (row < L) dk[((size_t)(t0 + row) * H + hk) * DK + d] = from_f32<Tio>(ak[x] + pa[x]);
    }
  }
}

struct PlanView {
  int nc, nch, nl, chunk, T;
  int off_cstart, off_clen, off_cpar, off_chain, off_lchains, off_loff, off_coff, off_cch;
};

bool plan_view(const int32_t* ph, PlanView* v) {
  v->nc = ph[0];
  v->nch = ph[1];
  v->nl = ph[2];
  v->chunk = ph[3];
  v->T = ph[4];
  if (v->nc < 1 || v->nch < 1 || v->nch > v->nc || v->nl < 1 || v->nl > v->nch || v->chunk < 1 || v->chunk > kCh)
    return false;
  v->off_cstart = 8;
  v->off_clen = v->off_cstart + v->nc;
  v->off_cpar = v->off_clen + v->nc;
  v->off_chain = v->off_cpar + v->nc;
  v->off_lchains = v->off_chain + v->nch + 1;
  v->off_loff = v->off_lchains + v->nch;
  v->off_coff = v->off_loff + v->nl + 1;
  v->off_cch = v->off_coff + v->nc + 1;
  return true;
}

template <int DK, int DV, typename Tio>
void gdn_launch(const void* q, const void* k, const void* v, const float* g, const float* beta, int H, int Hv,
                const int32_t* plan, const int32_t* ph, const PlanView& pv, void* o, char* ws, const GdnLayout& L,
                hipStream_t st) {
  float* gcw = reinterpret_cast<float*>(ws + L.gc);
  float* u = reinterpret_cast<float*>(ws + L.u);
  bf16* wp = reinterpret_cast<bf16*>(ws + L.w);
  bf16* kt = reinterpret_cast<bf16*>(ws + L.kt);
  bf16* vnt = reinterpret_cast<bf16*>(ws + L.vnt);
  bf16* h0w = reinterpret_cast<bf16*>(ws + L.h0);
  bf16* tt = reinterpret_cast<bf16*>(ws + L.tt);
  const int* cstart = plan + pv.off_cstart;
  const int* clen = plan + pv.off_clen;
  {
    ProfScope ps("gdn_prep", st);
    hipLaunchKernelGGL((gdn_prep_kernel<DK, DV, Tio>), dim3(pv.nc, Hv), dim3(256), 0, st, static_cast<const Tio*>(k),
                       static_cast<const Tio*>(v), g, beta, cstart, clen, pv.nc, H, Hv, gcw, u, wp, kt, tt);
  }
  {
    ProfScope ps("gdn_state", st);
    const int32_t* loff = ph + pv.off_loff;
    for (int l = 0; l < pv.nl; ++l) {
      const int n = loff[l + 1] - loff[l];
      hipLaunchKernelGGL((gdn_state_kernel<DK, DV>), dim3(n, Hv), dim3(64 * (DV / 32)), 0, st,
                         plan + pv.off_lchains, loff[l], plan + pv.off_chain, plan + pv.off_cpar, pv.nc, Hv, gcw, u,
                         wp, kt, vnt, h0w);
    }
  }
  {
    ProfScope ps("gdn_out", st);
    hipLaunchKernelGGL((gdn_out_kernel<DK, DV, Tio>), dim3(pv.nc, Hv), dim3(256), 0, st, static_cast<const Tio*>(q),
                       static_cast<const Tio*>(k), cstart, clen, pv.nc, H, Hv, gcw, vnt, h0w, static_cast<Tio*>(o));
  }
}

template <typename Tio>
int gdn_dispatch(int dk, int dv, const void* q, const void* k, const void* v, const float* g, const float* beta,
                 int H, int Hv, const int32_t* plan, const int32_t* ph, const PlanView& pv, void* o, char* ws,
                 const GdnLayout& L, hipStream_t st) {
  if (dk == 128 && dv == 128)
    gdn_launch<128, 128, Tio>(q, k, v, g, beta, H, Hv, plan, ph, pv, o, ws, L, st);
  else if (dk == 128 && dv == 64)
    gdn_launch<128, 64, Tio>(q, k, v, g, beta, H, Hv, plan, ph, pv, o, ws, L, st);
  else if (dk == 64 && dv == 128)
    gdn_launch<64, 128, Tio>(q, k, v, g, beta, H, Hv, plan, ph, pv, o, ws, L, st);
  else
    gdn_launch<64, 64, Tio>(q, k, v, g, beta, H, Hv, plan, ph, pv, o, ws, L, st);
  return TA_OK;
}

template <int DK, int DV, typename Tio>
void gdn_bwd_launch(const void* q, const void* k, const void* v, const float* beta, const void* dout, int H, int Hv,
                    const int32_t* plan, const int32_t* ph, const PlanView& pv, void* dq, void* dk, void* dv,
                    float* dg, float* dbeta, char* ws, const GdnLayout& F, const GdnBwdLayout& B, hipStream_t st) {
  const float* gcw = reinterpret_cast<const float*>(ws + F.gc);
  const float* u = reinterpret_cast<const float*>(ws + F.u);
  const bf16* wp = reinterpret_cast<const bf16*>(ws + F.w);
  const bf16* vnt = reinterpret_cast<const bf16*>(ws + F.vnt);
  const bf16* h0w = reinterpret_cast<const bf16*>(ws + F.h0);
  float* dvlt = reinterpret_cast<float*>(ws + B.dvlt);
  bf16* kgl = reinterpret_cast<bf16*>(ws + B.kgl);
  bf16* qgt = reinterpret_cast<bf16*>(ws + B.qgt);
  bf16* wt = reinterpret_cast<bf16*>(ws + B.wt);
  bf16* dot = reinterpret_cast<bf16*>(ws + B.dot);
  bf16* dvnt = reinterpret_cast<bf16*>(ws + B.dvnt);
  bf16* dhe = reinterpret_cast<bf16*>(ws + B.dhe);
  bf16* dwt = reinterpret_cast<bf16*>(ws + B.dwt);
  float* dgca = reinterpret_cast<float*>(ws + B.dgca);
  float* dka = reinterpret_cast<float*>(ws + B.dka);
  const bf16* ttw = reinterpret_cast<const bf16*>(ws + F.tt);
  float* dhead = reinterpret_cast<float*>(ws + B.dhead);
  const int* cstart = plan + pv.off_cstart;
  const int* clen = plan + pv.off_clen;
  const Tio* qq = static_cast<const Tio*>(q);
  const Tio* kk = static_cast<const Tio*>(k);
  const Tio* dd = static_cast<const Tio*>(dout);
  {
    ProfScope ps("gdn_bwd_prep", st);
    hipLaunchKernelGGL((gdn_bwd_prep_kernel<DK, DV, Tio>), dim3(pv.nc, Hv), dim3(256), 0, st, qq, kk, dd, cstart, clen,
                       pv.nc, H, Hv, gcw, wp, dvlt, kgl, qgt, wt, dot);
  }
  {
    ProfScope ps("gdn_bwd_state", st);
    const int32_t* loff = ph + pv.off_loff;
    for (int l = pv.nl - 1; l >= 0; --l) {
      const int n = loff[l + 1] - loff[l];
      hipLaunchKernelGGL((gdn_bwd_state_kernel<DK, DV>), dim3(n, Hv), dim3(64 * (DV / 32)), 0, st,
                         plan + pv.off_lchains, loff[l], plan + pv.off_chain, plan + pv.off_coff, plan + pv.off_cch,
                         pv.nc, Hv, gcw, dvlt, kgl, qgt, wt, dot, dvnt, dhe, dhead);
    }
  }
  {
    ProfScope ps("gdn_bwd_out", st);
    hipLaunchKernelGGL((gdn_bwd_out_kernel<DK, DV, Tio>), dim3(pv.nc, H), dim3(512), 0, st, qq, kk, dd, cstart, clen,
                       pv.nc, H, Hv, gcw, vnt, h0w, dvnt, dhe, static_cast<Tio*>(dq), dka, dgca, dwt);
  }
  {
    ProfScope ps("gdn_bwd_wy", st);
    hipLaunchKernelGGL((gdn_bwd_wy_kernel<DK, DV, Tio>), dim3(pv.nc, H), dim3(512), 0, st, kk,
                       static_cast<const Tio*>(v), beta, cstart, clen, pv.nc, H, Hv, gcw, u, wp, ttw, dvnt, dwt, dka, dgca,
                       static_cast<Tio*>(dk), static_cast<Tio*>(dv), dg, dbeta);
  }
}

template <typename Tio>
void gdn_bwd_dispatch(int dk_, int dv_, const void* q, const void* k, const void* v, const float* beta,
                      const void* dout, int H, int Hv, const int32_t* plan, const int32_t* ph, const PlanView& pv,
                      void* dq, void* dk, void* dv, float* dg, float* dbeta, char* ws, const GdnLayout& F,
                      const GdnBwdLayout& B, hipStream_t st) {
  if (dk_ == 128 && dv_ == 128)
    gdn_bwd_launch<128, 128, Tio>(q, k, v, beta, dout, H, Hv, plan, ph, pv, dq, dk, dv, dg, dbeta, ws, F, B, st);
  else if (dk_ == 128 && dv_ == 64)
    gdn_bwd_launch<128, 64, Tio>(q, k, v, beta, dout, H, Hv, plan, ph, pv, dq, dk, dv, dg, dbeta, ws, F, B, st);
  else if (dk_ == 64 && dv_ == 128)
    gdn_bwd_launch<64, 128, Tio>(q, k, v, beta, dout, H, Hv, plan, ph, pv, dq, dk, dv, dg, dbeta, ws, F, B, st);
  else
    gdn_bwd_launch<64, 64, Tio>(q, k, v, beta, dout, H, Hv, plan, ph, pv, dq, dk, dv, dg, dbeta, ws, F, B, st);
}

bool al16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// kernels are instantiated for up to 4 taps (the common K) and up to 8
template <typename Tio>
void conv_fwd_launch(int K, dim3 grid, hipStream_t st, const Tio* x, const float* w, const float* b, const int* par,
                     int T, int C, int act, Tio* y) {
  if (K <= 4)
    hipLaunchKernelGGL((conv_fwd_kernel<Tio, 4>), grid, dim3(kConvThreads), 0, st, x, w, b, par, T, C, K, act, y);
  else
    hipLaunchKernelGGL((conv_fwd_kernel<Tio, kConvMaxK>), grid, dim3(kConvThreads), 0, st, x, w, b, par, T, C, K,
                       act, y);
}

template <typename Tio, int KM>
void conv_bwd_launch_k(int K, int nblk, int cy, hipStream_t st, const Tio* x, const Tio* dy, const float* w,
                       const float* b, const int* par, const int* pos, const int* se, int T, int C, int act,
                       Tio* gbuf, float* part, Tio* dx) {
  hipLaunchKernelGGL((conv_bwd_g_kernel<Tio, KM>), dim3(nblk, cy), dim3(kConvThreads), 0, st, x, dy, w, b, par, T, C,
                     K, act, gbuf, part);
  hipLaunchKernelGGL((conv_bwd_dx_kernel<Tio, KM>), dim3((T + kConvTB - 1) / kConvTB, cy), dim3(kConvThreads), 0, st,
                     gbuf, w, pos, se, T, C, K, dx);
}

template <typename Tio>
void conv_bwd_launch(int K, int nblk, int cy, hipStream_t st, const Tio* x, const Tio* dy, const float* w,
                     const float* b, const int* par, const int* pos, const int* se, int T, int C, int act, Tio* gbuf,
                     float* part, Tio* dx) {
  if (K <= 4)
    conv_bwd_launch_k<Tio, 4>(K, nblk, cy, st, x, dy, w, b, par, pos, se, T, C, act, gbuf, part, dx);
  else
    conv_bwd_launch_k<Tio, kConvMaxK>(K, nblk, cy, st, x, dy, w, b, par, pos, se, T, C, act, gbuf, part, dx);
}

}  // namespace
}  // namespace ta

using namespace ta;

// ---------------------------------------------------------------- C ABI: conv

extern "C" int tree_conv_fwd(const void* x, ta_dtype dt, int32_t T, int32_t C, int32_t K, const float* weight,
                             const float* bias, const int32_t* parent, int32_t activation, void* y, void* stream) {
  clear_error();
  if (!x || !weight || !parent || !y) return fail(TA_EINVAL, "tree_conv_fwd: NULL pointer argument");
  if (T < 1 || C < 8 || C % 8 != 0 || K < 1 || K > kConvMaxK)
    return fail(TA_EINVAL, "tree_conv_fwd: need T >= 1, C a positive multiple of 8, 1 <= K <= %d (T=%d C=%d K=%d)",
                kConvMaxK, T, C, K);
  if (dt != TA_BF16 && dt != TA_F32) return fail(TA_EINVAL, "tree_conv_fwd: bad dtype %d", (int)dt);
  if (activation != 0 && activation != 1) return fail(TA_EINVAL, "tree_conv_fwd: activation must be 0 or 1");
  if (!al16(x) || !al16(y)) return fail(TA_EINVAL, "tree_conv_fwd: x and y must be 16-byte aligned");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dim3 grid((T + kConvTB - 1) / kConvTB, (C / 8 + kConvThreads - 1) / kConvThreads);
  {
    ProfScope ps("conv_fwd", st);
    if (dt == TA_BF16)
      conv_fwd_launch<bf16>(K, grid, st, static_cast<const bf16*>(x), weight, bias, parent, T, C, activation,
                            static_cast<bf16*>(y));
    else
      conv_fwd_launch<float>(K, grid, st, static_cast<const float*>(x), weight, bias, parent, T, C, activation,
                             static_cast<float*>(y));
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TA_EHIP, "tree_conv_fwd: kernel launch failed: %s", hipGetErrorString(e));
  return TA_OK;
}

namespace {
size_t conv_ws_part_off(int32_t T, int32_t C) { return al256((size_t)T * C * 4); }
}  // namespace

extern "C" size_t tree_conv_workspace_bytes(int32_t T, int32_t C, int32_t K) {
  if (T < 1 || C < 1 || K < 1 || K > kConvMaxK) return 0;
  const size_t nblk = (T + kConvTokBlock - 1) / kConvTokBlock;
  return conv_ws_part_off(T, C) + al256(nblk * C * (K + 1) * 4);
}

extern "C" int tree_conv_bwd(const void* x, const void* dy, ta_dtype dt, int32_t T, int32_t C, int32_t K,
                             const float* weight, const float* bias, const int32_t* parent, const int32_t* pos,
                             const int32_t* subtree_end, int32_t activation, void* dx, float* dweight, float* dbias,
                             void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (!x || !dy || !weight || !parent || !pos || !subtree_end || !dx || !dweight || !workspace)
    return fail(TA_EINVAL, "tree_conv_bwd: NULL pointer argument");
  if (T < 1 || T >= (1 << 28) || C < 8 || C % 8 != 0 || K < 1 || K > kConvMaxK)
    return fail(TA_EINVAL,
                "tree_conv_bwd: need 1 <= T < 2^28, C a positive multiple of 8, 1 <= K <= %d (T=%d C=%d K=%d)",
                kConvMaxK, T, C, K);
  if (dt != TA_BF16 && dt != TA_F32) return fail(TA_EINVAL, "tree_conv_bwd: bad dtype %d", (int)dt);
  if (activation != 0 && activation != 1) return fail(TA_EINVAL, "tree_conv_bwd: activation must be 0 or 1");
  if (!al16(x) || !al16(dy) || !al16(dx)) return fail(TA_EINVAL, "tree_conv_bwd: x, dy, dx must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TA_EINVAL, "tree_conv_bwd: workspace must be 256-byte aligned");
  const size_t need = tree_conv_workspace_bytes(T, C, K);
  if (ws_bytes < need) return fail(TA_EINVAL, "tree_conv_bwd: workspace too small (%zu < %zu bytes)", ws_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + conv_ws_part_off(T, C));
  const int nblk = (T + kConvTokBlock - 1) / kConvTokBlock;
  const int cy = (C / 8 + kConvThreads - 1) / kConvThreads;
  {
    ProfScope ps("conv_bwd", st);
    if (dt == TA_BF16)
      conv_bwd_launch<bf16>(K, nblk, cy, st, static_cast<const bf16*>(x), static_cast<const bf16*>(dy), weight, bias,
                            parent, pos, subtree_end, T, C, activation, static_cast<bf16*>(workspace), part,
                            static_cast<bf16*>(dx));
    else
      conv_bwd_launch<float>(K, nblk, cy, st, static_cast<const float*>(x), static_cast<const float*>(dy), weight,
                             bias, parent, pos, subtree_end, T, C, activation, static_cast<float*>(workspace), part,
                             static_cast<float*>(dx));
    hipLaunchKernelGGL(conv_bwd_reduce_kernel, dim3((C * (K + 1) + 255) / 256), dim3(256), 0, st, part, nblk, C, K,
                       dweight, dbias);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TA_EHIP, "tree_conv_bwd: kernel launch failed: %s", hipGetErrorString(e));
  return TA_OK;
}

// ---------------------------------------------------------------- C ABI: gated delta rule

extern "C" size_t tree_gdn_workspace_bytes(int32_t H, int32_t Hv, int32_t dk, int32_t dv, int32_t n_chunks) {
  if (H < 1 || Hv < 1 || dk < 1 || dv < 1 || n_chunks < 1) return 0;
  return gdn_layout(H, Hv, dk, dv, n_chunks).total;
}

extern "C" int tree_gdn_fwd(const void* q, const void* k, const void* v, ta_dtype dt, const float* g,
                            const float* beta, int32_t T, int32_t H, int32_t Hv, int32_t dk, int32_t dv,
                            const int32_t* plan, const int32_t* plan_host, void* o, void* workspace, size_t ws_bytes,
                            void* stream) {
  clear_error();
  if (!q || !k || !v || !g || !beta || !plan || !plan_host || !o || !workspace)
    return fail(TA_EINVAL, "tree_gdn_fwd: NULL pointer argument");
  if (T < 1 || H < 1 || Hv < H || Hv % H != 0)
    return fail(TA_EINVAL, "tree_gdn_fwd: need T >= 1, H >= 1 and Hv a multiple of H (T=%d H=%d Hv=%d)", T, H, Hv);
  if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))
    return fail(TA_EUNSUPPORTED, "tree_gdn_fwd: dk and dv must be 64 or 128 (dk=%d dv=%d)", dk, dv);
  if (dt != TA_BF16 && dt != TA_F32) return fail(TA_EINVAL, "tree_gdn_fwd: bad dtype %d", (int)dt);
  if (!al16(q) || !al16(k) || !al16(v) || !al16(o))
    return fail(TA_EINVAL, "tree_gdn_fwd: q, k, v and o must be 16-byte aligned");
  PlanView pv;
  if (!plan_view(plan_host, &pv)) return fail(TA_EINVAL, "tree_gdn_fwd: plan header is not a tree_gdn_plan output");
  if (pv.T != T) return fail(TA_EINVAL, "tree_gdn_fwd: the plan covers %d tokens, T = %d", pv.T, T);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TA_EINVAL, "tree_gdn_fwd: workspace must be 256-byte aligned");
  const GdnLayout L = gdn_layout(H, Hv, dk, dv, pv.nc);
  if (ws_bytes < L.total) return fail(TA_EINVAL, "tree_gdn_fwd: workspace too small (%zu < %zu bytes)", ws_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (dt == TA_BF16)
    gdn_dispatch<bf16>(dk, dv, q, k, v, g, beta, H, Hv, plan, plan_host, pv, o, ws, L, st);
  else
    gdn_dispatch<float>(dk, dv, q, k, v, g, beta, H, Hv, plan, plan_host, pv, o, ws, L, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TA_EHIP, "tree_gdn_fwd: kernel launch failed: %s", hipGetErrorString(e));
  return TA_OK;
}

extern "C" size_t tree_gdn_bwd_workspace_bytes(int32_t H, int32_t Hv, int32_t dk, int32_t dv, int32_t n_chunks,
                                               int32_t n_chains) {
  if (H < 1 || Hv < 1 || dk < 1 || dv < 1 || n_chunks < 1 || n_chains < 1 || n_chains > n_chunks) return 0;
  return gdn_bwd_layout(H, Hv, dk, dv, n_chunks, n_chains).total;
}

extern "C" int tree_gdn_bwd(const void* q, const void* k, const void* v, ta_dtype dt, const float* g,
                            const float* beta, const void* dout, int32_t T, int32_t H, int32_t Hv, int32_t dk,
                            int32_t dv, const int32_t* plan, const int32_t* plan_host, void* dq, void* dk_out,
                            void* dv_out, float* dg, float* dbeta, void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (!q || !k || !v || !g || !beta || !dout || !plan || !plan_host || !dq || !dk_out || !dv_out || !dg || !dbeta ||
      !workspace)
    return fail(TA_EINVAL, "tree_gdn_bwd: NULL pointer argument");
  if (T < 1 || H < 1 || Hv < H || Hv % H != 0)
    return fail(TA_EINVAL, "tree_gdn_bwd: need T >= 1, H >= 1 and Hv a multiple of H (T=%d H=%d Hv=%d)", T, H, Hv);
  if ((dk != 64 && dk != 128) || (dv != 64 && dv != 128))
    return fail(TA_EUNSUPPORTED, "tree_gdn_bwd: dk and dv must be 64 or 128 (dk=%d dv=%d)", dk, dv);
  if (dt != TA_BF16 && dt != TA_F32) return fail(TA_EINVAL, "tree_gdn_bwd: bad dtype %d", (int)dt);
  if (!al16(q) || !al16(k) || !al16(v) || !al16(dout) || !al16(dq) || !al16(dk_out) || !al16(dv_out) || !al16(dg) ||
      !al16(dbeta))
    return fail(TA_EINVAL, "tree_gdn_bwd: tensors must be 16-byte aligned");
  PlanView pv;
  if (!plan_view(plan_host, &pv)) return fail(TA_EINVAL, "tree_gdn_bwd: plan header is not a tree_gdn_plan output");
  if (pv.T != T) return fail(TA_EINVAL, "tree_gdn_bwd: the plan covers %d tokens, T = %d", pv.T, T);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TA_EINVAL, "tree_gdn_bwd: workspace must be 256-byte aligned");
  const GdnLayout F = gdn_layout(H, Hv, dk, dv, pv.nc);
  const GdnBwdLayout B = gdn_bwd_layout(H, Hv, dk, dv, pv.nc, pv.nch);
  if (ws_bytes < B.total)
    return fail(TA_EINVAL, "tree_gdn_bwd: workspace too small (%zu < %zu bytes)", ws_bytes, B.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (dt == TA_BF16)
    gdn_bwd_dispatch<bf16>(dk, dv, q, k, v, beta, dout, H, Hv, plan, plan_host, pv, dq, dk_out, dv_out, dg, dbeta,
                           ws, F, B, st);
  else
    gdn_bwd_dispatch<float>(dk, dv, q, k, v, beta, dout, H, Hv, plan, plan_host, pv, dq, dk_out, dv_out, dg, dbeta,
                            ws, F, B, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TA_EHIP, "tree_gdn_bwd: kernel launch failed: %s", hipGetErrorString(e));
  return TA_OK;
}
