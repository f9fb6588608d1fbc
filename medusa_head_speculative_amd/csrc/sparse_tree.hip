// Sparse candidate tree: the N-node choice list of largest expected accept length (host code).
//
// Ultralytics "Medusa Heads", tree-attention section: a sparse tree built from the most
// accurate combinations of head candidates beats a dense tree several times its size; Wiblog
// "Medusa multi-head speculative decoding", heads section: per-head top-1 / top-5 accuracy.
// With head k's rank-r candidate right with probability acc[k][r], independently across heads,
// the accept length is at least d exactly when the right rank tuple of length d is a node, so
// the expected accept length is the sum over nodes of prod_k acc[k][r_k], and the best N-node
// tree is the N most likely nodes (ties: depth, then rank tuple); they form a tree because no
// node is more likely than its parent.
//
// Best-first search: the heap holds the children of the nodes taken so far; the next node taken
// is the heap's best, which is the next node in the global order, since every node ranks below
// its parent.  Probabilities are products in depth order (fp64), so equal products tie exactly.
// A checked host build (-DMEDUSA_CHECKED) turns on the standard library's bounds assertions on
// every container access below.
#ifdef MEDUSA_CHECKED
#define _GLIBCXX_ASSERTIONS 1
#endif
#include <algorithm>
#include <cstdint>
#include <queue>
#include <vector>

#include "kernels.h"

namespace medusa {

namespace {

struct TreeNode {
  double p;
  int depth;
  int8_t r[8];
};

// true if a ranks after b: lower probability, then deeper, then larger rank tuple
bool ranks_after(const TreeNode& a, const TreeNode& b) {
  if (a.p != b.p) return a.p < b.p;
  if (a.depth != b.depth) return a.depth > b.depth;
  for (int i = 0; i < a.depth; ++i)
    if (a.r[i] != b.r[i]) return a.r[i] > b.r[i];
  return false;
}

bool node_order(const TreeNode& a, const TreeNode& b) {   // depth, then rank tuple
  if (a.depth != b.depth) return a.depth < b.depth;
  for (int i = 0; i < a.depth; ++i)
    if (a.r[i] != b.r[i]) return a.r[i] < b.r[i];
  return false;
}

}  // namespace

double build_sparse_tree(const double* acc, int K, int topk, int N, int32_t* choices) {
  auto cmp = [](const TreeNode& a, const TreeNode& b) { return ranks_after(a, b); };
  std::priority_queue<TreeNode, std::vector<TreeNode>, decltype(cmp)> heap(cmp);
  for (int r = 0; r < topk; ++r) {
    TreeNode n{};
    n.p = acc[r];
    n.depth = 1;
    n.r[0] = static_cast<int8_t>(r);
    heap.push(n);
  }
  std::vector<TreeNode> taken;
  taken.reserve(N);
  while (static_cast<int>(taken.size()) < N) {
    const TreeNode n = heap.top();
    heap.pop();
    taken.push_back(n);
    if (n.depth < K) {
      for (int r = 0; r < topk; ++r) {
        TreeNode c = n;
        c.p = n.p * acc[static_cast<long>(n.depth) * topk + r];
        c.r[n.depth] = static_cast<int8_t>(r);
        c.depth = n.depth + 1;
        heap.push(c);
      }
    }
  }
  std::sort(taken.begin(), taken.end(), node_order);
  double expected = 0.0;
  for (int i = 0; i < N; ++i) {
    expected += taken[i].p;
    for (int k = 0; k < K; ++k) choices[static_cast<long>(i) * K + k] = k < taken[i].depth ? taken[i].r[k] : -1;
  }
  return expected;
}

}  // namespace medusa
