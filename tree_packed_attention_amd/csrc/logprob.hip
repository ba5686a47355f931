// tree_logprob for gfx950: per-occurrence log-probabilities on shared logit
// rows, weighted loss, and the gradient scatter-added into the shared rows.
//
// The "Trie packing" page ("Share logits, preserve every prediction",
// "Combine gradients at the shared logits"): a row predicts the token after
// its node, several occurrences can read one row, and their gradients
// (p - e_y) add on that row. "Tree Training" §3.1 Eq. 4 / §3.2 Loss Weights:
// each occurrence carries its weight (g_t / K for the branch-averaged loss).
//
// Pipeline (all on the caller's stream):
//   1. count entries per source row (invalid entries get logp = NaN here)
//   2. exclusive scan -> CSR row pointers
//   3. scatter entry ids into their row's CSR range
//   4. one workgroup per row: read the row once into registers, row max and
//      sum of exponentials, lse; rank-sort the row's entry ids so every sum
//      runs in entry order; logp for the row's entries; W_r = sum of weights;
//      dlogits = s * W_r * softmax(z_r), then the target columns get
//      s * (W_r p_t - sum of the weights aiming at t)
//   5. loss = -sum_m w_m logp_m in entry order (one workgroup)
// The row is read from HBM once and dlogits written once. Sums run in a
// fixed order, so results are bitwise reproducible.
//
// The clipped policy loss (tree_logprob_ppo) runs the same pipeline. Each
// entry keeps its own advantage, old log-probability, mask and weight (the
// "Trie packing" page, its PPO/GRPO paragraph); the row kernel, which holds
// the row and has just formed logp, turns every entry into its coefficient
// c_m = -dloss/dlogp_m (PPO clipped surrogate: w mask A r while the
// unclipped branch is the minimum, else 0) and writes
// dlogits = s * (sum c) * softmax - s * (sum of c aiming at each target),
// so the loss needs no second pass over the logits.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "ta_device.h"
#include "profile.h"
#include "ta_error.h"
#include "tree_attn.h"

namespace ta {
namespace {

constexpr int kRowThreads = 1024;

__global__ void lp_zero_kernel(int* __restrict__ a, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) a[i] = 0;
}

__device__ __forceinline__ bool entry_ok(int s, int t, int64_t R, int64_t V) {
  return s >= 0 && (int64_t)s < R && t >= 0 && (int64_t)t < V;
}

__global__ void lp_count_kernel(const int* __restrict__ src, const int* __restrict__ tgt, int64_t M, int64_t R,
                                int64_t V, int* __restrict__ cnt, float* __restrict__ logp) {
  const int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  const int s = src[m], t = tgt[m];
  if (entry_ok(s, t, R, V))
    atomicAdd(&cnt[s], 1);
  else
    logp[m] = __builtin_nanf("");
}

template <typename Tv, typename Op>
__device__ Tv block_reduce(Tv v, Op op, Tv* red) {
  // fixed-order reduction: lanes by xor tree, then waves in index order
  for (int o = 32; o >= 1; o >>= 1) v = op(v, __shfl_xor(v, o));
  const int wv = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  __syncthreads();
  Tv r = red[0];
  for (int i = 1; i < nw; ++i) r = op(r, red[i]);
  return r;
}

struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct SumOp {
  __device__ float operator()(float a, float b) const { return a + b; }
};
struct ISumOp {
  __device__ int operator()(int a, int b) const { return a + b; }
};

// Exclusive scan of cnt[0..R) into ptr[0..R], one workgroup.
__global__ __launch_bounds__(1024) void lp_scan_kernel(const int* __restrict__ cnt, int64_t R, int* __restrict__ ptr) {
  __shared__ int red[16];
  __shared__ int wave_off[16];
  const int tid = threadIdx.x;
  const int64_t per = (R + blockDim.x - 1) / blockDim.x;
  const int64_t b = tid * per;
  const int64_t e = b + per < R ? b + per : R;
  int local = 0;
  for (int64_t i = b; i < e; ++i) local += cnt[i];
  // inclusive scan of per-thread sums across the workgroup
  int x = local;
  const int lane = tid & 63, wv = tid >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[wv] = x;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
      wave_off[i] = acc;
      acc += red[i];
    }
  }
  __syncthreads();
  int run = wave_off[wv] + x - local;
  for (int64_t i = b; i < e; ++i) {
    ptr[i] = run;
    run += cnt[i];
  }
  if (tid == (int)blockDim.x - 1) ptr[R] = wave_off[wv] + x;
}

__global__ void lp_fill_kernel(const int* __restrict__ src, const int* __restrict__ tgt, int64_t M, int64_t R,
                               int64_t V, const int* __restrict__ ptr, int* __restrict__ fill, int* __restrict__ ids) {
  const int64_t m = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= M) return;
  const int s = src[m], t = tgt[m];
  if (!entry_ok(s, t, R, V)) return;
  const int slot = ptr[s] + atomicAdd(&fill[s], 1);
  ids[slot] = (int)m;
}

template <typename T>
struct Vec16;  // 16 bytes of logits
template <>
struct Vec16<bf16> {
  static constexpr int N = 8;
  typedef bf16x8 type;
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  typedef f32x4 type;
};

// How an entry's log-probability becomes its gradient coefficient
// c_m = -dloss/dlogp_m. Weighted log-likelihood (adv == nullptr): c = w.
// Clipped policy loss: r = exp(logp - old), c = w mask A r when r A <=
// clip(r, lo, hi) A (the unclipped branch is the minimum; ties inside the
// range have equal derivatives), else 0; written to coef[m].
struct EntryRule {
  const float* w;
  const float* adv;           // nullptr: weighted log-likelihood
  const float* old;
  const unsigned char* mask;  // nullptr: every entry on
  float lo, hi;               // clip range [1 - eps_low, 1 + eps_high]
  float* coef;                // per-entry coefficients (policy loss only)
  __device__ __forceinline__ const float* coefs() const { return adv ? coef : w; }
};

__device__ __forceinline__ float policy_ratio(float logp, float old) { return expf(logp - old); }

// -min(r A, clip(r) A) and whether the unclipped branch is the minimum. A NaN
// ratio (the logp of an invalid entry) stays NaN: fminf / fmaxf would drop it.
__device__ __forceinline__ float policy_term(float r, float A, float lo, float hi, bool* unclipped) {
  if (__builtin_isnan(r)) {
    *unclipped = false;
    return r;
  }
  const float a = r * A;
  const float b = fminf(fmaxf(r, lo), hi) * A;
  *unclipped = a <= b;
  return -fminf(a, b);
}

// Rows of the CSR range [beg, beg + n): rank-sort the ids (all distinct) into
// `sorted`, then logp, W_r and the per-target corrections in entry order.
template <typename T>
__device__ void row_entries(const T* __restrict__ row, int beg, int n, const int* __restrict__ ids,
                            int* __restrict__ sorted, const int* __restrict__ tgt, const EntryRule& er,
                            float lse, float* __restrict__ logp, float* red, float* W_out) {
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int id = ids[beg + e];
    int rank = 0;
    for (int f = 0; f < n; ++f) rank += ids[beg + f] < id;
    sorted[beg + rank] = id;
  }
  __syncthreads();
  float ws = 0.0f;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int m = sorted[beg + e];
    const float lp = to_f32(row[tgt[m]]) - lse;
    logp[m] = lp;
    float c = er.w[m];
    if (er.adv) {
      bool unclipped;
      const float r = policy_ratio(lp, er.old[m]);
      policy_term(r, er.adv[m], er.lo, er.hi, &unclipped);
      const bool on = er.mask == nullptr || er.mask[m] != 0;
      c = (unclipped && on) ? c * er.adv[m] * r : 0.0f;
      er.coef[m] = c;
    }
    ws += c;
  }
  *W_out = block_reduce(ws, SumOp(), red);
}

template <typename T>
__device__ void row_corrections(const T* __restrict__ row, int beg, int n, const int* __restrict__ sorted,
                                const int* __restrict__ tgt, const float* __restrict__ w, float lse, float W,
                                float gs, T* __restrict__ drow) {
  // w: the per-entry coefficients (weights, or the policy-loss coefficients)
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const int t = tgt[sorted[beg + e]];
    bool first = true;
    for (int f = 0; f < e; ++f) first = first && (tgt[sorted[beg + f]] != t);
    if (!first) continue;
    float tot = 0.0f;
    for (int f = e; f < n; ++f) {
      const int m = sorted[beg + f];
      if (tgt[m] == t) tot += w[m];
    }
    const float p = __builtin_amdgcn_exp2f((to_f32(row[t]) - lse) * kLog2e);
    drow[t] = from_f32<T>(gs * (W * p) - gs * tot);
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// Cache policy of the streamed row reads and gradient writes (nontemporal).
constexpr int kNt = 2;
// Raw buffer resource over [p, p + bytes): accesses past the end read zeros
// and drop stores.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// Between passes over the row: the compiler would otherwise keep each pass's
// float conversions of the packed row for the next pass, twice the registers
// of the row, and spill them.
template <typename V, int N>
__device__ __forceinline__ void keep_packed(V (&x)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) asm volatile("" : "+v"(x[k]));
}

// Workgroup barrier that orders LDS only: global loads still in flight stay
// in flight (__syncthreads waits for them too).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// block_reduce with LDS-only barriers (same order, same result).
template <typename Tv, typename Op>
__device__ Tv block_reduce_lds(Tv v, Op op, Tv* red) {
  for (int o = 32; o >= 1; o >>= 1) v = op(v, __shfl_xor(v, o));
  const int wv = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  lds_barrier();
  if ((threadIdx.x & 63) == 0) red[wv] = v;
  lds_barrier();
  Tv r = red[0];
  for (int i = 1; i < nw; ++i) r = op(r, red[i]);
  return r;
}

// Entries of one row that the register kernel keeps in LDS; a row with more
// takes the general path (ids rank-sorted through global memory).
constexpr int kEntCap = 256;

// Row kernel with the row held in registers: NV 16-byte vectors per thread.
// Vector vi of the row (EPV logits) sits in thread vi % TPB, slot vi / TPB.
// TPB threads per row: 1024 for long rows, 256 for rows of at most 4096
// vectors, so that several rows (and their reductions) are in flight per CU.
//
// Rows with at most kEntCap entries: the entry ids are requested before the
// row and rank-sorted in LDS while it is in flight; each entry's target,
// weight and logit are requested once the row is in and arrive during the
// reductions. The corrected gradient of a target column is stored by the
// thread that stored the column's vector, after it, so the row needs no
// second pass and the workgroup never waits for its own stores. Sums run in
// the same order as on the general path (sorted entry order), so both give
// the same bits.
template <typename T, int NV, int TPB>
__global__ __launch_bounds__(TPB) void lp_row_reg_kernel(
    const T* __restrict__ logits, int64_t V, const int* __restrict__ ptr, const int* __restrict__ ids,
    int* __restrict__ sorted, const int* __restrict__ tgt, EntryRule er, float* __restrict__ logp,
    float* __restrict__ row_lse, T* __restrict__ dlogits, float gs, int need_all_rows) {
  static_assert(TPB >= kEntCap && TPB <= 1024, "one thread per entry of a short row");
  typedef typename Vec16<T>::type vec;
  constexpr int EPV = Vec16<T>::N;
  constexpr int MAPW = (NV * TPB + 31) / 32;
  __shared__ float red[16];
  __shared__ unsigned int vmap[MAPW];  // bit vi: vector vi holds a target
  __shared__ int e_id[kEntCap];        // entry ids in CSR order
  __shared__ int e_t[kEntCap];         // the rest in sorted entry order: target column
  __shared__ float e_z[kEntCap];       // logit at the target
  __shared__ float e_c[kEntCap];       // coefficient c_m
  __shared__ float e_tot[kEntCap];     // sum of c over the entries aiming at the same target
  __shared__ unsigned char e_first[kEntCap];  // first entry (in sorted order) aiming at its target
  const int64_t r = blockIdx.x;
  const int beg = ptr[r], n = ptr[r + 1] - beg;
  if (n == 0 && !need_all_rows) return;
  const T* row = logits + r * V;
  const int64_t nvec = V / EPV;
  const int tid = threadIdx.x;
  vec x[NV];
  if (n > kEntCap) {
    // general path
    float mx = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t vi = tid + (int64_t)TPB * k;
      if (vi < nvec) {
        x[k] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(row) + vi);  // read once: streamed
#pragma unroll
        for (int s = 0; s < EPV; ++s) mx = fmaxf(mx, to_f32(x[k][s]));
      }
    }
    mx = block_reduce(mx, MaxOp(), red);
    float se = 0.0f;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t vi = tid + (int64_t)TPB * k;
      if (vi < nvec) {
#pragma unroll
        for (int s = 0; s < EPV; ++s) se += __builtin_amdgcn_exp2f((to_f32(x[k][s]) - mx) * kLog2e);
      }
    }
    se = block_reduce(se, SumOp(), red);
    const float lse = mx + logf(se);
    if (row_lse != nullptr && tid == 0) row_lse[r] = lse;
    float W = 0.0f;
    row_entries(row, beg, n, ids, sorted, tgt, er, lse, logp, red, &W);
    if (dlogits == nullptr) return;
    T* drow = dlogits + r * V;
    const float sw = gs * W;
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int64_t vi = tid + (int64_t)TPB * k;
      if (vi < nvec) {
        vec g;
#pragma unroll
        for (int s = 0; s < EPV; ++s)
          g[s] = from_f32<T>(sw * __builtin_amdgcn_exp2f((to_f32(x[k][s]) - lse) * kLog2e));
        __builtin_nontemporal_store(g, reinterpret_cast<vec*>(drow) + vi);  // written once: streamed
      }
    }
    __syncthreads();
    row_corrections(row, beg, n, sorted, tgt, er.coefs(), lse, W, gs, drow);
    return;
  }

  // the entry's id first, so that its load returns ahead of the row's
  // Buffer loads: a lane past the end reads zeros without a memory access,
  // so every thread issues the same loads, none behind a branch, and the
  // compiler's waits count exactly the loads issued before the awaited one.
  // The range check covers the per-lane offset, which therefore carries the
  // whole offset (the uniform operand stays 0).
  const bool ent = tid < n;
  const int id = (int)__builtin_amdgcn_raw_buffer_load_b32(buf_rsrc(ids + beg, 4 * n), 4 * tid, 0, 0);
  for (int i = tid; i < MAPW; i += TPB) vmap[i] = 0u;
  // this thread's vectors are tid + TPB k for k < nk (nvec < 2^31)
  const int nk = (int)((nvec - tid + TPB - 1) / TPB);
  const __amdgpu_buffer_rsrc_t rrow = buf_rsrc(row, (int)(16 * nvec));
  int off = 16 * tid;
#pragma unroll
  for (int k = 0; k < NV; ++k)  // read once: streamed
    x[k] = __builtin_bit_cast(vec, __builtin_amdgcn_raw_buffer_load_b128(rrow, off + 16 * TPB * k, 0, kNt));
  if (ent) e_id[tid] = id;
  lds_barrier();
  // rank among the row's ids (all distinct) = sorted position; the entry's
  // target, weight and policy inputs are requested behind the row
  int rank = 0, t = 0, mk = 1;
  float wv = 0.0f, av = 0.0f, ov = 0.0f;
  if (ent) {
    for (int f = 0; f < n; ++f) rank += e_id[f] < id;
    t = tgt[id];
    wv = er.w[id];
    if (er.adv) {
      av = er.adv[id];
      ov = er.old[id];
    }
  }
  float mx = -__builtin_inff();
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (k < nk) {
#pragma unroll
      for (int s = 0; s < EPV; ++s) mx = fmaxf(mx, to_f32(x[k][s]));
    }
  }
  mx = block_reduce_lds(mx, MaxOp(), red);
  // the logit at the target (just read, so served by the caches) and the
  // mask (tested where it is loaded) arrive during the exponentials
  float z = 0.0f;
  if (ent) {
    z = to_f32(row[t]);
    if (er.adv && er.mask != nullptr) mk = er.mask[id];
    e_t[rank] = t;
    const int tv = t / EPV;
    atomicOr(&vmap[tv >> 5], 1u << (tv & 31));
  }
  keep_packed(x);
  float se = 0.0f;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    if (k < nk) {
#pragma unroll
      for (int s = 0; s < EPV; ++s) se += __builtin_amdgcn_exp2f((to_f32(x[k][s]) - mx) * kLog2e);
    }
  }
  se = block_reduce_lds(se, SumOp(), red);  // its barriers also publish e_t and vmap
  const float lse = mx + logf(se);
  if (row_lse != nullptr && tid == 0) row_lse[r] = lse;
  // logp and the coefficient of each entry (weighted log-likelihood: c = w)
  if (ent) {
    const float lp = z - lse;
    logp[id] = lp;
    float c = wv;
    if (er.adv) {
      bool unclipped;
      const float ratio = policy_ratio(lp, ov);
      policy_term(ratio, av, er.lo, er.hi, &unclipped);
      c = (unclipped && mk != 0) ? c * av * ratio : 0.0f;
      er.coef[id] = c;
    }
    e_c[rank] = c;
    e_z[rank] = z;
  }
  lds_barrier();
  const float W = block_reduce_lds(tid < n ? e_c[tid] : 0.0f, SumOp(), red);  // sorted entry order
  if (dlogits == nullptr) return;
  if (tid < n) {
    const int te = e_t[tid];
    bool first = true;
    for (int f = 0; f < tid; ++f) first = first && (e_t[f] != te);
    float tot = 0.0f;
    if (first)
      for (int f = tid; f < n; ++f)
        if (e_t[f] == te) tot += e_c[f];
    e_tot[tid] = tot;
    e_first[tid] = first;
  }
  T* drow = dlogits + r * V;
  const __amdgpu_buffer_rsrc_t rd = buf_rsrc(drow, (int)(16 * nvec));
  const float sw = gs * W;
  keep_packed(x);
  asm volatile("" : "+v"(off));  // offsets recomputed here, not kept from the loads
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    vec g;
#pragma unroll
    for (int s = 0; s < EPV; ++s) g[s] = from_f32<T>(sw * __builtin_amdgcn_exp2f((to_f32(x[k][s]) - lse) * kLog2e));
    // written once: streamed; a store past the end is dropped
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, g), rd, off + 16 * TPB * k, 0, kNt);
  }
  lds_barrier();  // e_tot, e_first
  // target columns: s (W_r p_t - sum of the c aiming at t), written by the
  // thread that stored the column's vector above, so this store lands last
  for (int k = 0; k < nk; ++k) {
    const int vi = tid + TPB * k;
    if (!((vmap[vi >> 5] >> (vi & 31)) & 1u)) continue;
    for (int e = 0; e < n; ++e) {
      const int te = e_t[e];
      if (e_first[e] && te / EPV == vi) {
        const float p = __builtin_amdgcn_exp2f((e_z[e] - lse) * kLog2e);
        drow[te] = from_f32<T>(gs * (W * p) - gs * e_tot[e]);
      }
    }
  }
}

// Row kernel for any V and alignment: streams the row twice (the second
// read is served by the caches).
template <typename T>
__global__ __launch_bounds__(kRowThreads) void lp_row_stream_kernel(
    const T* __restrict__ logits, int64_t V, const int* __restrict__ ptr, const int* __restrict__ ids,
    int* __restrict__ sorted, const int* __restrict__ tgt, EntryRule er, float* __restrict__ logp,
    float* __restrict__ row_lse, T* __restrict__ dlogits, float gs, int need_all_rows) {
  __shared__ float red[16];
  const int64_t r = blockIdx.x;
  const int beg = ptr[r], n = ptr[r + 1] - beg;
  if (n == 0 && !need_all_rows) return;
  const T* row = logits + r * V;
  float m = -__builtin_inff(), s = 0.0f;
  for (int64_t c = threadIdx.x; c < V; c += blockDim.x) {
    const float x = to_f32(row[c]);
    if (x > m) {
      s = s * __builtin_amdgcn_exp2f((m - x) * kLog2e) + 1.0f;
      m = x;
    } else {
      s += __builtin_amdgcn_exp2f((x - m) * kLog2e);
    }
  }
  const float gm = block_reduce(m, MaxOp(), red);
  float sc = (m == -__builtin_inff()) ? 0.0f : s * __builtin_amdgcn_exp2f((m - gm) * kLog2e);
  sc = block_reduce(sc, SumOp(), red);
  const float lse = gm + logf(sc);
  if (row_lse != nullptr && threadIdx.x == 0) row_lse[r] = lse;
  float W = 0.0f;
  row_entries(row, beg, n, ids, sorted, tgt, er, lse, logp, red, &W);
  if (dlogits == nullptr) return;
  T* drow = dlogits + r * V;
  const float sw = gs * W;
  for (int64_t c = threadIdx.x; c < V; c += blockDim.x)
    drow[c] = from_f32<T>(sw * __builtin_amdgcn_exp2f((to_f32(row[c]) - lse) * kLog2e));
  __syncthreads();
  row_corrections(row, beg, n, sorted, tgt, er.coefs(), lse, W, gs, drow);
}

__global__ __launch_bounds__(1024) void lp_loss_kernel(const float* __restrict__ logp, const float* __restrict__ w,
                                                       int64_t M, float* __restrict__ loss) {
  __shared__ float red[16];
  float acc = 0.0f;
  for (int64_t m = threadIdx.x; m < M; m += blockDim.x) acc += w[m] * logp[m];
  acc = block_reduce(acc, SumOp(), red);
  if (threadIdx.x == 0) *loss = -acc;
}

// Clipped policy loss: sum_m w_m mask_m (-min(r A, clip(r) A)) in entry order,
// from the logp the row kernel wrote (NaN for an invalid entry, which then
// makes the loss NaN unless the entry is masked).
__global__ __launch_bounds__(1024) void lp_policy_loss_kernel(const float* __restrict__ logp, EntryRule er,
                                                              int64_t M, float* __restrict__ loss) {
  __shared__ float red[16];
  float acc = 0.0f;
  for (int64_t m = threadIdx.x; m < M; m += blockDim.x) {
    if (er.mask != nullptr && er.mask[m] == 0) continue;
    bool unclipped;
    const float l = policy_term(policy_ratio(logp[m], er.old[m]), er.adv[m], er.lo, er.hi, &unclipped);
    acc += er.w[m] * l;
  }
  acc = block_reduce(acc, SumOp(), red);
  if (threadIdx.x == 0) *loss = acc;
}

struct LpLayout {
  size_t off_cnt, off_ptr, off_fill, off_ids, off_sorted, off_coef, total;
};

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

LpLayout lp_layout(int64_t R, int64_t M) {
  LpLayout L{};
  size_t o = 0;
  L.off_cnt = o;
  o = al256(o + (size_t)R * 4);
  L.off_ptr = o;
  o = al256(o + (size_t)(R + 1) * 4);
  L.off_fill = o;
  o = al256(o + (size_t)R * 4);
  L.off_ids = o;
  o = al256(o + (size_t)(M > 0 ? M : 1) * 4);
  L.off_sorted = o;
  o = al256(o + (size_t)(M > 0 ? M : 1) * 4);
  L.off_coef = o;
  o = al256(o + (size_t)(M > 0 ? M : 1) * 4);
  L.total = o;
  return L;
}

template <typename T, int NV, int TPB = kRowThreads>
void launch_reg(int64_t R, const void* logits, int64_t V, char* ws, const LpLayout& L, const int* tgt, const EntryRule& w,
                float* logp, float* row_lse, void* dlogits, float gs, int need_all, hipStream_t st) {
  hipLaunchKernelGGL((lp_row_reg_kernel<T, NV, TPB>), dim3((unsigned)R), dim3(TPB), 0, st,
                     static_cast<const T*>(logits), V, reinterpret_cast<const int*>(ws + L.off_ptr),
                     reinterpret_cast<const int*>(ws + L.off_ids), reinterpret_cast<int*>(ws + L.off_sorted), tgt, w,
                     logp, row_lse, static_cast<T*>(dlogits), gs, need_all);
}

template <typename T>
void launch_rows(int64_t R, const void* logits, int64_t V, char* ws, const LpLayout& L, const int* tgt, const EntryRule& w,
                 float* logp, float* row_lse, void* dlogits, float gs, hipStream_t st) {
  constexpr int EPV = 16 / sizeof(T);
  const int need_all = (row_lse != nullptr || dlogits != nullptr) ? 1 : 0;
  const bool aligned = (V * (int64_t)sizeof(T)) % 16 == 0 && reinterpret_cast<uintptr_t>(logits) % 16 == 0 &&
                       (dlogits == nullptr || reinterpret_cast<uintptr_t>(dlogits) % 16 == 0);
  const int64_t nvec_per_thread = (V / EPV + kRowThreads - 1) / kRowThreads;
  const int64_t nv256 = (V / EPV + 255) / 256;  // vectors per thread at 256 threads per row
  if (aligned && nv256 <= 16) {
    if (nv256 <= 4) return launch_reg<T, 4, 256>(R, logits, V, ws, L, tgt, w, logp, row_lse, dlogits, gs, need_all, st);
    if (nv256 <= 8) return launch_reg<T, 8, 256>(R, logits, V, ws, L, tgt, w, logp, row_lse, dlogits, gs, need_all, st);
    return launch_reg<T, 16, 256>(R, logits, V, ws, L, tgt, w, logp, row_lse, dlogits, gs, need_all, st);
  }
  if (aligned && nvec_per_thread <= 20) {
    if (nvec_per_thread <= 8) return launch_reg<T, 8>(R, logits, V, ws, L, tgt, w, logp, row_lse, dlogits, gs, need_all, st);
    if (nvec_per_thread <= 12) return launch_reg<T, 12>(R, logits, V, ws, L, tgt, w, logp, row_lse, dlogits, gs, need_all, st);
    if (nvec_per_thread <= 16) return launch_reg<T, 16>(R, logits, V, ws, L, tgt, w, logp, row_lse, dlogits, gs, need_all, st);
    return launch_reg<T, 20>(R, logits, V, ws, L, tgt, w, logp, row_lse, dlogits, gs, need_all, st);
  }
  hipLaunchKernelGGL(lp_row_stream_kernel<T>, dim3((unsigned)R), dim3(kRowThreads), 0, st,
                     static_cast<const T*>(logits), V, reinterpret_cast<const int*>(ws + L.off_ptr),
                     reinterpret_cast<const int*>(ws + L.off_ids), reinterpret_cast<int*>(ws + L.off_sorted), tgt, w,
                     logp, row_lse, static_cast<T*>(dlogits), gs, need_all);
}

}  // namespace
}  // namespace ta

using namespace ta;

extern "C" size_t tree_logprob_workspace_bytes(int64_t R, int64_t M) {
  if (R < 1 || M < 0) return 0;
  return lp_layout(R, M).total;
}

namespace {

int logprob_impl(const char* fn, const void* logits, ta_dtype dt, int64_t R, int64_t V, const int32_t* src_row,
                 const int32_t* target, EntryRule er, int64_t M, float* logp, float* row_lse, float* loss,
                 void* dlogits, float grad_scale, void* workspace, size_t ws_bytes, void* stream) {
  if (R < 1 || R >= INT32_MAX || V < 1 || V >= INT32_MAX || M < 0 || M >= INT32_MAX - 1)
    return fail(TA_EINVAL, "%s: need 1 <= R, V < 2^31 and 0 <= M < 2^31-1 (R=%lld V=%lld M=%lld)", fn, (long long)R,
                (long long)V, (long long)M);
  if (!logits || !workspace || (M > 0 && (!src_row || !target || !er.w || !logp)))
    return fail(TA_EINVAL, "%s: NULL pointer argument", fn);
  if (dt != TA_BF16 && dt != TA_F32) return fail(TA_EINVAL, "%s: bad dtype %d", fn, (int)dt);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(TA_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  const LpLayout L = lp_layout(R, M);
  if (ws_bytes < L.total) return fail(TA_EINVAL, "%s: workspace too small (%zu < %zu bytes)", fn, ws_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int* cnt = reinterpret_cast<int*>(ws + L.off_cnt);
  int* fill = reinterpret_cast<int*>(ws + L.off_fill);
  er.coef = reinterpret_cast<float*>(ws + L.off_coef);
  {
  ProfScope ps("lp_csr", st);
  hipLaunchKernelGGL(lp_zero_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, st, cnt, R);
  hipLaunchKernelGGL(lp_zero_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, st, fill, R);
  if (M > 0)
    hipLaunchKernelGGL(lp_count_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, st, src_row, target, M, R, V,
                       cnt, logp);
  hipLaunchKernelGGL(lp_scan_kernel, dim3(1), dim3(1024), 0, st, cnt, R, reinterpret_cast<int*>(ws + L.off_ptr));
  if (M > 0)
    hipLaunchKernelGGL(lp_fill_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, st, src_row, target, M, R, V,
                       reinterpret_cast<const int*>(ws + L.off_ptr), fill, reinterpret_cast<int*>(ws + L.off_ids));
  }
  {
  ProfScope ps("lp_rows", st);
  if (dt == TA_BF16)
    launch_rows<bf16>(R, logits, V, ws, L, target, er, logp, row_lse, dlogits, grad_scale, st);
  else
    launch_rows<float>(R, logits, V, ws, L, target, er, logp, row_lse, dlogits, grad_scale, st);
  }
  if (loss != nullptr) {
    ProfScope ps("lp_loss", st);
    if (er.adv)
      hipLaunchKernelGGL(lp_policy_loss_kernel, dim3(1), dim3(1024), 0, st, logp, er, M, loss);
    else
      hipLaunchKernelGGL(lp_loss_kernel, dim3(1), dim3(1024), 0, st, logp, er.w, M, loss);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(TA_EHIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
  return TA_OK;
}

}  // namespace

extern "C" int tree_logprob(const void* logits, ta_dtype dt, int64_t R, int64_t V, const int32_t* src_row,
                            const int32_t* target, const float* weight, int64_t M, float* logp, float* row_lse,
                            float* loss, void* dlogits, float grad_scale, void* workspace, size_t ws_bytes,
                            void* stream) {
  clear_error();
  EntryRule er{weight, nullptr, nullptr, nullptr, 0.0f, 0.0f, nullptr};
  return logprob_impl("tree_logprob", logits, dt, R, V, src_row, target, er, M, logp, row_lse, loss, dlogits,
                      grad_scale, workspace, ws_bytes, stream);
}

extern "C" int tree_logprob_ppo(const void* logits, ta_dtype dt, int64_t R, int64_t V, const int32_t* src_row,
                                const int32_t* target, const float* weight, const float* advantage,
                                const float* old_logp, const uint8_t* mask, int64_t M, float eps_low, float eps_high,
                                float* logp, float* row_lse, float* loss, void* dlogits, float grad_scale,
                                void* workspace, size_t ws_bytes, void* stream) {
  clear_error();
  if (!(eps_low >= 0.0f) || !(eps_high >= 0.0f))
    return fail(TA_EINVAL, "tree_logprob_ppo: eps_low and eps_high must be >= 0 (got %g, %g)", (double)eps_low,
                (double)eps_high);
  if (M > 0 && (!advantage || !old_logp)) return fail(TA_EINVAL, "tree_logprob_ppo: NULL advantage or old_logp");
  EntryRule er{weight, advantage, old_logp, mask, 1.0f - eps_low, 1.0f + eps_high, nullptr};
  return logprob_impl("tree_logprob_ppo", logits, dt, R, V, src_row, target, er, M, logp, row_lse, loss, dlogits,
                      grad_scale, workspace, ws_bytes, stream);
}

// ------------------------------------------------------------------------
// tree_logprob without a workspace argument, for callers that cannot
// allocate. Its entry table (the workspace of tree_logprob) lives in this
// fixed array, one per device for the life of the process.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of the scratch array on the device `stream` belongs to
// (the current device for the null stream), resolved once per device with
// that device current. Host code never passes `scratch` itself: its name is
// a host-side stand-in, not a device address.
int scratch_on(hipStream_t stream, const char* fn, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TA_EHIP, "%s: no device for the stream: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TA_EUNSUPPORTED, "%s: device %d out of range", fn, dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return fail(TA_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(TA_EHIP, "%s: hipSetDevice(%d): %s", fn, dev, hipGetErrorString(e));
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess || p == nullptr)
      return fail(TA_EHIP, "%s: hipGetSymbolAddress of the scratch array: %s", fn, hipGetErrorString(e));
    if (back != hipSuccess)
      return fail(TA_EHIP, "%s: hipSetDevice(%d): %s", fn, cur, hipGetErrorString(back));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TA_OK;
}

}  // namespace

extern "C" int tree_logprob_noalloc(const void* logits, ta_dtype dt, int64_t R, int64_t V, const int32_t* src_row,
                                    const int32_t* target, const float* weight, int64_t M, float* logp,
                                    float* row_lse, float* loss, void* dlogits, float grad_scale, void* stream) {
  clear_error();
  const char* fn = "tree_logprob_noalloc";
  if (R >= 1 && M >= 0) {
    const size_t need = lp_layout(R, M).total;
    if (need > kNoAllocScratchBytes)
      return fail(TA_ECAPACITY, "%s: R=%lld rows and M=%lld entries need %zu bytes of scratch, more than the %zu "
                  "bytes this entry point has (use tree_logprob with a workspace)",
                  fn, (long long)R, (long long)M, need, kNoAllocScratchBytes);
  }
  // sizes out of range: logprob_impl rejects them before it looks at the
  // (then absent) scratch
  void* ws = nullptr;
  if (R >= 1 && R < INT32_MAX && V >= 1 && V < INT32_MAX && M >= 0 && M < INT32_MAX - 1) {
    if (int rc = scratch_on(static_cast<hipStream_t>(stream), fn, &ws)) return rc;
  }
  EntryRule er{weight, nullptr, nullptr, nullptr, 0.0f, 0.0f, nullptr};
  return logprob_impl(fn, logits, dt, R, V, src_row, target, er, M, logp, row_lse, loss, dlogits, grad_scale, ws,
                      kNoAllocScratchBytes, stream);
}
