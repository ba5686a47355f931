// tree_gdn_plan: host-side chunk schedule for the tree-routed gated delta
// rule.
//
// "Tree Training" §3.2 (SSM Layers, Eq. 10) makes every tree node's token
// segment the unit of state transfer: a node starts from the end state of its
// parent node, never from its DFS predecessor. Here a node is cut further
// into chunks of at most `chunk` tokens; a chunk's parent is the previous
// chunk of the same node, or the last chunk of the parent node (-1 at a
// root). A run of chunks in which every chunk's parent is the chunk just
// before it is a chain: a chain is computed sequentially, and chains whose
// parents lie in earlier levels run side by side. Level 0 holds the chains
// that start at a root; a chain starting under chunk p is one level above the
// chain that contains p.
//
// Blob (int32): header [n_chunks, n_chains, n_levels, chunk, T, 0, 0, 0],
// then chunk_start[n_chunks], chunk_len[n_chunks], chunk_parent[n_chunks],
// chain_begin[n_chains + 1], level_chains[n_chains], level_off[n_levels + 1],
// child_off[n_chunks + 1], child_chains[n_chains]: the chains that start
// under chunk c are child_chains[child_off[c] .. child_off[c + 1]), in
// increasing order (the backward sums their start-state gradients into c's
// end-state gradient in that order).
#include <cstdint>
#include <vector>

#include "ta_error.h"

using ta::fail;

extern "C" int tree_gdn_plan(const int32_t* node_start, const int32_t* node_end, const int32_t* node_parent,
                             int32_t n_nodes, int32_t chunk, int32_t* plan, int32_t cap,
                             ta_gdn_plan_sizes* sizes) {
  ta::clear_error();
  if (!node_start || !node_end || !node_parent || !sizes) return fail(TA_EINVAL, "tree_gdn_plan: NULL argument");
  if (n_nodes < 1) return fail(TA_EINVAL, "tree_gdn_plan: n_nodes must be >= 1 (got %d)", n_nodes);
  if (chunk < 1 || chunk > 64) return fail(TA_EINVAL, "tree_gdn_plan: chunk must be in [1, 64] (got %d)", chunk);
  std::vector<int32_t> cstart, clen, cpar, last(n_nodes, -1);
  int32_t expect = 0;
  for (int32_t n = 0; n < n_nodes; ++n) {
    const int32_t s = node_start[n], e = node_end[n], p = node_parent[n];
    if (s != expect || e <= s)
      return fail(TA_EINVAL, "tree_gdn_plan: node %d range [%d, %d) does not continue the layout at %d", n, s, e,
                  expect);
    if (p >= n || p < -1) return fail(TA_EINVAL, "tree_gdn_plan: node %d has parent %d (need -1 <= parent < node)", n, p);
    expect = e;
    int32_t prev = p >= 0 ? last[p] : -1;
    for (int32_t a = s; a < e; a += chunk) {
      const int32_t id = static_cast<int32_t>(cstart.size());
      cstart.push_back(a);
      clen.push_back(e - a < chunk ? e - a : chunk);
      cpar.push_back(prev);
      prev = id;
    }
    last[n] = prev;
  }
  const int32_t nc = static_cast<int32_t>(cstart.size());
  // chains: maximal runs with cpar[c] == c - 1
  std::vector<int32_t> chain_begin, chain_of(nc), level;
  for (int32_t c = 0; c < nc; ++c) {
    if (c == 0 || cpar[c] != c - 1) {
      chain_begin.push_back(c);
      level.push_back(cpar[c] < 0 ? 0 : level[chain_of[cpar[c]]] + 1);
    }
    chain_of[c] = static_cast<int32_t>(chain_begin.size()) - 1;
  }
  const int32_t nch = static_cast<int32_t>(chain_begin.size());
  chain_begin.push_back(nc);
  int32_t nl = 0;
  for (int32_t l : level) nl = l + 1 > nl ? l + 1 : nl;
  std::vector<int32_t> level_off(nl + 1, 0), level_chains(nch);
  for (int32_t l : level) ++level_off[l + 1];
  for (int32_t l = 0; l < nl; ++l) level_off[l + 1] += level_off[l];
  {
    std::vector<int32_t> fill(level_off.begin(), level_off.end() - 1);
    for (int32_t ch = 0; ch < nch; ++ch) level_chains[fill[level[ch]]++] = ch;
  }
  std::vector<int32_t> child_off(nc + 1, 0), child_chains;
  for (int32_t ch = 0; ch < nch; ++ch) {
    const int32_t p = cpar[chain_begin[ch]];
    if (p >= 0) ++child_off[p + 1];
  }
  for (int32_t c = 0; c < nc; ++c) child_off[c + 1] += child_off[c];
  child_chains.assign(nch, -1);
  {
    std::vector<int32_t> fill(child_off.begin(), child_off.end() - 1);
    for (int32_t ch = 0; ch < nch; ++ch) {
      const int32_t p = cpar[chain_begin[ch]];
      if (p >= 0) child_chains[fill[p]++] = ch;
    }
  }
  const int64_t need = 8 + 3ll * nc + (nch + 1) + nch + (nl + 1) + (nc + 1) + nch;
  sizes->n_chunks = nc;
  sizes->n_chains = nch;
  sizes->n_levels = nl;
  sizes->plan_ints = static_cast<int32_t>(need);
  if (plan == nullptr || cap < need)
    return fail(TA_ECAPACITY, "tree_gdn_plan: the plan needs %lld ints (capacity %d)", (long long)need, cap);
  int32_t* o = plan;
  const int32_t head[8] = {nc, nch, nl, chunk, expect, 0, 0, 0};
  for (int32_t v : head) *o++ = v;
  for (int32_t v : cstart) *o++ = v;
  for (int32_t v : clen) *o++ = v;
  for (int32_t v : cpar) *o++ = v;
  for (int32_t v : chain_begin) *o++ = v;
  for (int32_t v : level_chains) *o++ = v;
  for (int32_t v : level_off) *o++ = v;
  for (int32_t v : child_off) *o++ = v;
  for (int32_t v : child_chains) *o++ = v;
  return TA_OK;
}
