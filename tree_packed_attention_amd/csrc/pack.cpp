// tree_pack: host-side prefix-tree packer.
//
// Builds one trie per group of sequences, lays every trie out in preorder
// (children in first-insertion order) and emits O(T) metadata: depth
// positions, subtree ends, parents, path counts, g/K weights, the packed
// index of every input token, and the chunk (compressed node) table.
//
// Sources: the "Trie packing" page (a token is shared only when its whole
// preceding context is identical; position = depth on the original path);
// "Tree Training" §3.1 (Eq. 2-4 path counts and g/K; Eq. 8 DFS layout) and
// §3.2 (Eq. 9 positions); the Claw-R1 "Prefix Tree Merge" page, section 1
// (insert, compress single-child chains, preorder ranges).
#include <cstdint>
#include <cstring>
#include <unordered_map>
#include <vector>

#include "ta_error.h"

namespace {

// Open-addressing map (parent node, token) -> child node.
class ChildTable {
 public:
  explicit ChildTable(size_t expected) {
    size_t cap = 16;
    while (cap < 2 * expected + 16) cap <<= 1;
    keys_.assign(cap, kEmpty);
    vals_.assign(cap, -1);
    mask_ = cap - 1;
  }
  // Returns the child if present, else inserts `fresh` and returns -1.
  int32_t find_or_insert(int32_t parent, int32_t token, int32_t fresh) {
    const uint64_t key = (static_cast<uint64_t>(static_cast<uint32_t>(parent)) << 32) |
                         static_cast<uint32_t>(token);
    size_t h = mix(key) & mask_;
    while (true) {
      if (keys_[h] == kEmpty) {
        keys_[h] = key;
        vals_[h] = fresh;
        return -1;
      }
      if (keys_[h] == key) return vals_[h];
      h = (h + 1) & mask_;
    }
  }

 private:
  static constexpr uint64_t kEmpty = ~0ull;  // parent ids are < 2^31, never all ones
  static uint64_t mix(uint64_t x) {          // splitmix64 finalizer
    x ^= x >> 30;
    x *= 0xbf58476d1ce4e5b9ull;
    x ^= x >> 27;
    x *= 0x94d049bb133111ebull;
    x ^= x >> 31;
    return x;
  }
  std::vector<uint64_t> keys_;
  std::vector<int32_t> vals_;
  size_t mask_ = 0;
};

struct Trie {
  // node 0..n_groups-1 are the virtual roots of the groups
  std::vector<int32_t> token, parent, first_child, last_child, next_sibling;
  std::vector<int32_t> n_children, passes, ends;

  int32_t add(int32_t tok, int32_t par) {
    const int32_t id = static_cast<int32_t>(token.size());
    token.push_back(tok);
    parent.push_back(par);
    first_child.push_back(-1);
    last_child.push_back(-1);
    next_sibling.push_back(-1);
    n_children.push_back(0);
    passes.push_back(0);
    ends.push_back(0);
    if (par >= 0) {
      if (last_child[par] < 0)
        first_child[par] = id;
      else
        next_sibling[last_child[par]] = id;
      last_child[par] = id;
      n_children[par] += 1;
    }
    return id;
  }
};

}  // namespace

extern "C" int tree_pack(const int32_t* tokens, const int64_t* seq_offsets, int32_t n_seqs,
                         const int32_t* group_of_seq, int32_t cap_T, int32_t cap_nodes,
                         int32_t* packed_ids, int32_t* pos, int32_t* subtree_end, int32_t* parent,
                         int32_t* path_count, float* weight, int32_t* occ_map,
                         int32_t* node_start, int32_t* node_end, int32_t* node_parent,
                         int32_t* node_subtree_end, int32_t* tree_start, ta_pack_sizes* sizes) {
  ta::clear_error();
  if (seq_offsets == nullptr) return ta::fail(TA_EINVAL, "tree_pack: seq_offsets is NULL");
  if (n_seqs < 1) return ta::fail(TA_EINVAL, "tree_pack: n_seqs must be >= 1 (got %d)", n_seqs);
  if (seq_offsets[0] != 0) return ta::fail(TA_EINVAL, "tree_pack: seq_offsets[0] must be 0");
  for (int32_t s = 0; s < n_seqs; ++s) {
    if (seq_offsets[s + 1] <= seq_offsets[s])
      return ta::fail(TA_EINVAL, "tree_pack: sequence %d is empty or offsets decrease", s);
  }
  const int64_t total = seq_offsets[n_seqs];
  if (total > INT32_MAX - 1) return ta::fail(TA_EINVAL, "tree_pack: more than 2^31-2 tokens");
  if (tokens == nullptr) return ta::fail(TA_EINVAL, "tree_pack: tokens is NULL");
  if (cap_T < 0 || cap_nodes < 0) return ta::fail(TA_EINVAL, "tree_pack: negative capacity");

  try {
    // groups in order of first appearance
    std::vector<int32_t> group_index(n_seqs, 0);
    int32_t n_groups = 1;
    if (group_of_seq != nullptr) {
      std::unordered_map<int32_t, int32_t> seen;
      seen.reserve(static_cast<size_t>(n_seqs) * 2);
      n_groups = 0;
      for (int32_t s = 0; s < n_seqs; ++s) {
        auto it = seen.find(group_of_seq[s]);
        if (it == seen.end()) {
          seen.emplace(group_of_seq[s], n_groups);
          group_index[s] = n_groups++;
        } else {
          group_index[s] = it->second;
        }
      }
    }
    std::vector<int32_t> K(n_groups, 0);
    for (int32_t s = 0; s < n_seqs; ++s) K[group_index[s]] += 1;

    // trie insert; remember the trie node of every input token
    Trie trie;
    trie.token.reserve(static_cast<size_t>(total) + n_groups);
    for (int32_t gi = 0; gi < n_groups; ++gi) trie.add(0, -1);
    ChildTable table(static_cast<size_t>(total));
    std::vector<int32_t> tok_node(static_cast<size_t>(total));
    for (int32_t s = 0; s < n_seqs; ++s) {
      int32_t cur = group_index[s];
      for (int64_t a = seq_offsets[s]; a < seq_offsets[s + 1]; ++a) {
        const int32_t fresh = static_cast<int32_t>(trie.token.size());
        int32_t child = table.find_or_insert(cur, tokens[a], fresh);
        if (child < 0) child = trie.add(tokens[a], cur);
        trie.passes[child] += 1;
        tok_node[a] = child;
        cur = child;
      }
      trie.ends[cur] += 1;
    }
    const int64_t n_trie = static_cast<int64_t>(trie.token.size());
    const int32_t T = static_cast<int32_t>(n_trie - n_groups);

    // preorder DFS per group, children in insertion order
    std::vector<int32_t> index_of(n_trie, -1);
    std::vector<int32_t> t_ids(T), t_pos(T), t_par(T), t_g(T), t_se(T), t_node(T);
    std::vector<float> t_w(T);
    std::vector<int32_t> n_start, n_end, n_par, n_se;
    std::vector<int32_t> trees(n_groups + 1, 0);
    std::vector<int32_t> stack, kids, depth(n_trie, 0);
    int32_t next = 0;
    for (int32_t gi = 0; gi < n_groups; ++gi) {
      trees[gi] = next;
      stack.clear();
      kids.clear();
      for (int32_t c = trie.first_child[gi]; c >= 0; c = trie.next_sibling[c]) kids.push_back(c);
      for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back(*it);
      while (!stack.empty()) {
        const int32_t nd = stack.back();
        stack.pop_back();
        const int32_t i = next++;
        index_of[nd] = i;
        const int32_t p = trie.parent[nd];
        const bool at_root = (p == gi);
        depth[nd] = at_root ? 0 : depth[p] + 1;
        t_ids[i] = trie.token[nd];
        t_pos[i] = depth[nd];
        t_par[i] = at_root ? -1 : index_of[p];
        t_g[i] = trie.passes[nd];
        t_w[i] = static_cast<float>(trie.passes[nd]) / static_cast<float>(K[gi]);
        // chunk boundaries: tree root, below a fork, after a sequence end
        if (at_root || trie.n_children[p] >= 2 || trie.ends[p] > 0) {
          t_node[i] = static_cast<int32_t>(n_start.size());
          n_start.push_back(i);
          n_end.push_back(i + 1);
          n_par.push_back(at_root ? -1 : t_node[index_of[p]]);
        } else {
          t_node[i] = t_node[index_of[p]];
          n_end[t_node[i]] = i + 1;  // single child follows its parent in preorder
        }
        kids.clear();
        for (int32_t c = trie.first_child[nd]; c >= 0; c = trie.next_sibling[c]) kids.push_back(c);
        for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back(*it);
      }
      // subtree sizes by a reverse sweep (parents precede children)
      const int32_t base = trees[gi];
      for (int32_t i = base; i < next; ++i) t_se[i] = 1;
      for (int32_t i = next - 1; i > base; --i)
        if (t_par[i] >= 0) t_se[t_par[i]] += t_se[i];
      for (int32_t i = base; i < next; ++i) t_se[i] += i;
    }
    trees[n_groups] = next;
    const int32_t n_nodes = static_cast<int32_t>(n_start.size());
    n_se.resize(n_nodes);
    for (int32_t c = 0; c < n_nodes; ++c) n_se[c] = t_se[n_start[c]];

    if (sizes != nullptr) {
      sizes->T = T;
      sizes->n_nodes = n_nodes;
      sizes->n_trees = n_groups;
    }
    if (cap_T < T || cap_nodes < n_nodes)
      return ta::fail(TA_ECAPACITY, "tree_pack: need cap_T >= %d and cap_nodes >= %d (got %d, %d)",
                      T, n_nodes, cap_T, cap_nodes);

    auto put = [](int32_t* dst, const std::vector<int32_t>& src) {
      if (dst != nullptr && !src.empty()) std::memcpy(dst, src.data(), src.size() * sizeof(int32_t));
    };
    put(packed_ids, t_ids);
    put(pos, t_pos);
    put(subtree_end, t_se);
    put(parent, t_par);
    put(path_count, t_g);
    if (weight != nullptr) std::memcpy(weight, t_w.data(), t_w.size() * sizeof(float));
    if (occ_map != nullptr)
      for (int64_t a = 0; a < total; ++a) occ_map[a] = index_of[tok_node[a]];
    put(node_start, n_start);
    put(node_end, n_end);
    put(node_parent, n_par);
    put(node_subtree_end, n_se);
    put(tree_start, trees);
    return TA_OK;
  } catch (const std::bad_alloc&) {
    return ta::fail(TA_EINVAL, "tree_pack: out of host memory");
  } catch (...) {
    return ta::fail(TA_EINVAL, "tree_pack: internal error");
  }
}

extern "C" int tree_tile_stats(const int32_t* subtree_end, int32_t T, int32_t BQ, int32_t BK,
                               int64_t* full, int64_t* partial, int64_t* empty, int64_t* causal) {
  ta::clear_error();
  if (subtree_end == nullptr || full == nullptr || partial == nullptr || empty == nullptr ||
      causal == nullptr)
    return ta::fail(TA_EINVAL, "tree_tile_stats: NULL argument");
  if (T < 1 || BQ < 1 || BK < 1) return ta::fail(TA_EINVAL, "tree_tile_stats: T, BQ, BK must be >= 1");
  const int64_t nk = (static_cast<int64_t>(T) + BK - 1) / BK;
  const int64_t nq = (static_cast<int64_t>(T) + BQ - 1) / BQ;
  std::vector<int32_t> kmin(nk), kmax(nk);
  for (int64_t kt = 0; kt < nk; ++kt) {
    int32_t mn = INT32_MAX, mx = 0;
    for (int64_t j = kt * BK; j < (kt + 1) * BK; ++j) {
      const int32_t s = j < T ? subtree_end[j] : 0;  // padding keys: never visible
      mn = s < mn ? s : mn;
      mx = s > mx ? s : mx;
    }
    kmin[kt] = mn;
    kmax[kt] = mx;
  }
  int64_t f = 0, p = 0, e = 0, c = 0;
  for (int64_t qt = 0; qt < nq; ++qt) {
    const int64_t i0 = qt * BQ;
    const int64_t i1 = (i0 + BQ < T) ? i0 + BQ : T;
    for (int64_t kt = 0; kt < nk; ++kt) {
      const int64_t j0 = kt * BK, j1 = j0 + BK;
      if (j0 > i1 - 1) break;
      ++c;
      if (kmax[kt] <= i0)
        ++e;
      else if (j1 - 1 <= i0 && kmin[kt] >= i1)
        ++f;
      else
        ++p;
    }
  }
  *full = f;
  *partial = p;
  *empty = e;
  *causal = c;
  return TA_OK;
}
