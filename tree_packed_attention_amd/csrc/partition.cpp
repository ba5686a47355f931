// tree_partition: host-side partition planner for trees too large for one
// pass ("Tree Training" §3.3, Partitioning).
//
// Cuts fall on node boundaries, every partition keeps exactly one parent
// partition (so a backward pass holds one root-to-leaf chain of partition
// graphs), each holds at most C tokens, and the count is kept small:
//   1. cut: bottom-up, a node's residual is its length plus the residuals of
//      its children still attached; while it exceeds C, the attached child
//      with the largest residual (ties: the earlier child) is cut off and
//      becomes the root of its own piece. This gives the fewest connected
//      pieces of <= C tokens (the linear tree-partitioning greedy of Kundu
//      and Misra, 1977).
//   2. pack: pieces cut from the same node (or tree roots) share every
//      ancestor, so they may share a partition with one parent partition and
//      one gateway of cached ancestor rows; each such group is packed
//      first-fit decreasing (ties: preorder): tree roots first, then, for the
//      partitions in creation order, the groups of their nodes in preorder.
#include <algorithm>
#include <cstdint>
#include <deque>
#include <vector>

#include "ta_error.h"

using ta::fail;

extern "C" int tree_partition(const int32_t* node_start, const int32_t* node_end, const int32_t* node_parent,
                              int32_t n_nodes, int64_t capacity, int32_t* node_part, int32_t* part_tokens,
                              int32_t* part_parent, int32_t* part_cut, int32_t* n_parts) {
  ta::clear_error();
  if (!node_start || !node_end || !node_parent || !node_part || !part_tokens || !part_parent || !part_cut || !n_parts)
    return fail(TA_EINVAL, "tree_partition: NULL argument");
  if (n_nodes < 1) return fail(TA_EINVAL, "tree_partition: n_nodes must be >= 1 (got %d)", n_nodes);
  const int32_t n = n_nodes;
  std::vector<int64_t> len(n);
  std::vector<std::vector<int32_t>> children(n);
  for (int32_t v = 0; v < n; ++v) {
    len[v] = static_cast<int64_t>(node_end[v]) - node_start[v];
    const int32_t p = node_parent[v];
    if (len[v] < 1) return fail(TA_EINVAL, "tree_partition: node %d is empty", v);
    if (p < -1 || p >= v) return fail(TA_EINVAL, "tree_partition: node %d has parent %d (need -1 <= parent < node)", v, p);
    if (len[v] > capacity)
      return fail(TA_EINVAL, "tree_partition: node %d holds %lld tokens, more than the capacity %lld", v,
                  (long long)len[v], (long long)capacity);
    if (p >= 0) children[p].push_back(v);
  }
  // 1. cut
  std::vector<int64_t> resid(n);
  std::vector<char> is_cut(n, 0);
  for (int32_t v = n - 1; v >= 0; --v) {
    std::vector<int32_t> kids = children[v];
    int64_t total = len[v];
    for (int32_t c : kids) total += resid[c];
    std::sort(kids.begin(), kids.end(), [&](int32_t a, int32_t b) {
      return resid[a] != resid[b] ? resid[a] > resid[b] : a < b;
    });
    for (size_t i = 0; i < kids.size() && total > capacity; ++i) {
      is_cut[kids[i]] = 1;
      total -= resid[kids[i]];
    }
    resid[v] = total;
  }
  std::vector<int32_t> piece(n);
  std::vector<int64_t> ptok(n, 0);
  std::vector<std::vector<int32_t>> child_pieces(n);  // by piece root: pieces hanging from that piece
  std::vector<std::vector<int32_t>> hang(n);          // by node: pieces whose root's parent is that node
  std::vector<int32_t> root_pieces;
  for (int32_t v = 0; v < n; ++v) {
    const int32_t p = node_parent[v];
    piece[v] = (p < 0 || is_cut[v]) ? v : piece[p];
    ptok[piece[v]] += len[v];
    if (piece[v] == v) {
      if (p < 0) {
        root_pieces.push_back(v);
      } else {
        child_pieces[piece[p]].push_back(v);
        hang[p].push_back(v);
      }
    }
  }
  // 2. pack, one group per cut node (tree roots first)
  std::vector<int32_t> part_of(n, -1);  // by piece root
  std::vector<std::vector<int32_t>> pieces_of_part;
  std::vector<int64_t> tok;
  std::deque<int32_t> queue{-1};
  while (!queue.empty()) {
    const int32_t gp = queue.front();
    queue.pop_front();
    std::vector<int32_t> cuts;
    if (gp < 0) {
      cuts.push_back(-1);
    } else {
      for (int32_t pc : pieces_of_part[gp])
        for (int32_t r : child_pieces[pc]) cuts.push_back(node_parent[r]);
      std::sort(cuts.begin(), cuts.end());
      cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
    }
    for (int32_t u : cuts) {
      std::vector<int32_t> members = u < 0 ? root_pieces : hang[u];
      std::sort(members.begin(), members.end(), [&](int32_t a, int32_t b) {
        return ptok[a] != ptok[b] ? ptok[a] > ptok[b] : a < b;
      });
      std::vector<int32_t> mine;
      for (int32_t r : members) {
        int32_t dst = -1;
        for (int32_t b : mine)
          if (tok[b] + ptok[r] <= capacity) {
            dst = b;
            break;
          }
        if (dst < 0) {
          dst = static_cast<int32_t>(tok.size());
          tok.push_back(0);
          pieces_of_part.emplace_back();
          part_parent[dst] = gp;
          part_cut[dst] = u;
          mine.push_back(dst);
          queue.push_back(dst);
        }
        tok[dst] += ptok[r];
        part_of[r] = dst;
        pieces_of_part[dst].push_back(r);
      }
    }
  }
  for (int32_t v = 0; v < n; ++v) node_part[v] = part_of[piece[v]];
  for (size_t b = 0; b < tok.size(); ++b) part_tokens[b] = static_cast<int32_t>(tok[b]);
  *n_parts = static_cast<int32_t>(tok.size());
  return TA_OK;
}
