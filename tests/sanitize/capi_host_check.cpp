// Host-only exercise of libmedusa_hip's C ABI for the sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code, MEDUSA_CHECKED bounds assertions in the
// containers): the static-tree parser on valid, random and malformed choice lists, the
// sparse-tree search on random accuracy tables, and the argument checks of every entry point.
// Nothing here reaches a kernel launch, so it runs without a GPU.  Exit status 0: every call
// returned what it should.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "../../include/medusa.h"

static int failures = 0;
#define EXPECT(cond)                                                      \
  do {                                                                    \
    if (!(cond)) {                                                        \
      std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond);   \
      ++failures;                                                         \
    }                                                                     \
  } while (0)

// a choice list as [n][max_depth] with -1 padding
static std::vector<int32_t> flat(const std::vector<std::vector<int>>& ch, int md) {
  std::vector<int32_t> a(ch.size() * md, -1);
  for (size_t c = 0; c < ch.size(); ++c)
    for (size_t d = 0; d < ch[c].size(); ++d) a[c * md + d] = ch[c][d];
  return a;
}

static void cartesian(std::vector<std::vector<int>>& out, std::vector<int>& cur,
                      const std::vector<int>& ks, size_t depth) {
  if (depth == ks.size()) return;
  for (int r = 0; r < ks[depth]; ++r) {
    cur.push_back(r);
    out.push_back(cur);
    cartesian(out, cur, ks, depth + 1);
    cur.pop_back();
  }
}

static int dims(const std::vector<std::vector<int>>& ch, int md, int K, int topk, medusa_tree* t) {
  std::vector<int32_t> a = flat(ch, md);
  return medusa_tree_dims(a.data(), static_cast<int>(ch.size()), md, K, topk, t);
}

int main() {
  std::mt19937_64 rng(12345);
  // ---- valid trees: Cartesian products and random prefix-closed lists ----
  const std::vector<std::vector<int>> shapes = {{2, 3}, {10, 10, 10}, {1, 1, 1, 1, 1, 1, 1, 1},
                                                {64}, {3, 3, 3, 3}, {4, 4, 4, 4, 3}};
  for (const auto& ks : shapes) {
    std::vector<std::vector<int>> ch;
    std::vector<int> cur;
    cartesian(ch, cur, ks, 0);
    int topk = 0;
    for (int k : ks) topk = k > topk ? k : topk;
    medusa_tree t{};
    EXPECT(dims(ch, static_cast<int>(ks.size()), static_cast<int>(ks.size()), topk, &t) == MEDUSA_OK);
    EXPECT(t.T == static_cast<int>(ch.size()) + 1);
    EXPECT(t.dmax == static_cast<int>(ks.size()));
    EXPECT(t.W == (t.T + 63) / 64);
    EXPECT(t.n_internal + t.n_paths == t.T);
  }
  for (int trial = 0; trial < 400; ++trial) {
    const int topk = 1 + static_cast<int>(rng() % 64);
    const int K = 1 + static_cast<int>(rng() % 8);
    std::vector<std::vector<int>> nodes = {{}};
    std::vector<int> used = {0};
    const int target = 1 + static_cast<int>(rng() % 300);
    for (int it = 0; it < 4 * target && static_cast<int>(nodes.size()) <= target; ++it) {
      const size_t p = rng() % nodes.size();
      if (static_cast<int>(nodes[p].size()) >= K || used[p] >= topk) continue;
      std::vector<int> child = nodes[p];
      child.push_back(used[p]++);
      nodes.push_back(child);
      used.push_back(0);
    }
    if (nodes.size() < 2) continue;
    std::vector<std::vector<int>> ch(nodes.begin() + 1, nodes.end());
    std::shuffle(ch.begin(), ch.end(), rng);       // the list order does not matter
    medusa_tree t{};
    EXPECT(dims(ch, K, K, topk, &t) == MEDUSA_OK);
    EXPECT(t.T == static_cast<int>(ch.size()) + 1);
    EXPECT(t.max_rank < topk);
    // a list with one prefix removed is not prefix-closed (unless the removed node is a leaf)
    std::vector<std::vector<int>> broken = ch;
    broken.erase(broken.begin() + static_cast<long>(rng() % broken.size()));
    medusa_tree t2{};
    const int rc = broken.empty() ? MEDUSA_ERR_TREE : dims(broken, K, K, topk, &t2);
    EXPECT(rc == MEDUSA_OK || rc == MEDUSA_ERR_TREE);
  }
  // ---- malformed lists ----
  medusa_tree t{};
  EXPECT(dims({{0, 0}}, 2, 3, 3, &t) == MEDUSA_ERR_TREE);             // not prefix-closed
  EXPECT(dims({{0}, {3}}, 1, 3, 3, &t) == MEDUSA_ERR_TREE);           // rank >= topk
  EXPECT(dims({{0}, {0, 0}, {0, 0, 0}}, 3, 2, 3, &t) == MEDUSA_ERR_TREE);   // depth > K
  EXPECT(dims({{0}, {0}}, 1, 3, 3, &t) == MEDUSA_ERR_TREE);           // duplicate
  {
    std::vector<int32_t> gap = {0, -1, 1};                               // a value after -1
    EXPECT(medusa_tree_dims(gap.data(), 1, 3, 3, 3, &t) == MEDUSA_ERR_TREE);
    std::vector<int32_t> empty = {-1, -1};
    EXPECT(medusa_tree_dims(empty.data(), 1, 2, 3, 3, &t) == MEDUSA_ERR_TREE);
    EXPECT(medusa_tree_dims(gap.data(), 0, 3, 3, 3, &t) == MEDUSA_ERR_TREE);
    EXPECT(medusa_tree_dims(gap.data(), 1, 0, 3, 3, &t) == MEDUSA_ERR_TREE);
    EXPECT(medusa_tree_dims(gap.data(), 1, 9, 3, 3, &t) == MEDUSA_ERR_TREE);
    EXPECT(medusa_tree_dims(nullptr, 1, 3, 3, 3, &t) == MEDUSA_ERR_ARG);
    EXPECT(medusa_tree_dims(gap.data(), 1, 3, 3, 3, nullptr) == MEDUSA_ERR_ARG);
    EXPECT(medusa_tree_dims(gap.data(), 1, 3, 0, 3, &t) == MEDUSA_ERR_SHAPE);
    EXPECT(medusa_tree_dims(gap.data(), 1, 3, 3, 65, &t) == MEDUSA_ERR_SHAPE);
  }
  {
    std::vector<std::vector<int>> big;                                    // T over the limit
    std::vector<int> cur;
    cartesian(big, cur, {16, 16, 16}, 0);
    EXPECT(dims(big, 3, 3, 16, &t) == MEDUSA_ERR_TREE);
  }
  // ---- sparse trees from random accuracy tables ----
  for (int trial = 0; trial < 200; ++trial) {
    const int K = 1 + static_cast<int>(rng() % 8), topk = 1 + static_cast<int>(rng() % 64);
    std::vector<double> acc(static_cast<size_t>(K) * topk);
    std::uniform_real_distribution<double> u(0.0, 1.0);
    for (auto& x : acc) x = (rng() % 5 == 0) ? 0.5 : u(rng);    // some exact ties
    double full = 0.0, level = 1.0;
    for (int d = 0; d < K && full <= 4095.0; ++d) full += (level *= topk);
    const int nmax = full < 4095.0 ? static_cast<int>(full) : 4095;
    const int N = 1 + static_cast<int>(rng() % nmax);
    std::vector<int32_t> out(static_cast<size_t>(N) * K, -7);
    double e = -1.0;
    EXPECT(medusa_sparse_tree(acc.data(), K, topk, N, out.data(), &e) == MEDUSA_OK);
    EXPECT(e >= 0.0);
    medusa_tree ts{};
    EXPECT(medusa_tree_dims(out.data(), N, K, K, topk, &ts) == MEDUSA_OK);   // prefix-closed
    EXPECT(medusa_sparse_tree(acc.data(), K, topk, nmax + 1, out.data(), &e) == MEDUSA_ERR_SHAPE);
  }
  // ---- argument checks of the device entry points (rejected before any launch) ----
  void* p = reinterpret_cast<void*>(16);
  int32_t* ip = reinterpret_cast<int32_t*>(16);
  float* fp = reinterpret_cast<float*>(16);
  EXPECT(medusa_heads(p, p, p, p, 7, 1, 64, 100, 1, 1, nullptr, ip, nullptr, p, 1 << 20, nullptr) == MEDUSA_ERR_DTYPE);
  EXPECT(medusa_heads(p, p, p, p, 1, 9, 64, 100, 1, 1, nullptr, ip, nullptr, p, 1 << 20, nullptr) == MEDUSA_ERR_SHAPE);
  EXPECT(medusa_heads(p, p, p, p, 1, 1, 60, 100, 1, 1, nullptr, ip, nullptr, p, 1 << 20, nullptr) == MEDUSA_ERR_SHAPE);
  EXPECT(medusa_heads(p, p, p, p, 1, 1, 64, 100, 1, 1, nullptr, ip, nullptr, p, 16, nullptr) == MEDUSA_ERR_WORKSPACE);
  EXPECT(medusa_heads_packed(p, p, p, p, 1, 264, 100, 1, 1, nullptr, ip, nullptr, p, 1 << 20, nullptr) == MEDUSA_ERR_UNSUPPORTED);
  EXPECT(tree_attention(p, p, p, 1, ip, 10, 5, reinterpret_cast<uint64_t*>(p), 1, 4, 4, 9, 64, 0.f, p, p, 1 << 20, nullptr) == MEDUSA_ERR_SHAPE);
  EXPECT(tree_attention(p, p, p, 1, ip, 10, 100, reinterpret_cast<uint64_t*>(p), 1, 4, 4, 9, 96, 0.f, p, p, 1 << 20, nullptr) == MEDUSA_ERR_SHAPE);
  medusa_tree tf{};
  tf.T = 9; tf.W = 1; tf.n_paths = 6; tf.dmax = 2; tf.n_internal = 3; tf.max_rank = 2;
  tf.mask = reinterpret_cast<uint64_t*>(p);
  tf.parent = tf.depth = tf.rank = tf.paths = tf.path_len = tf.child_ptr = tf.child_idx = tf.internal = ip;
  EXPECT(typical_accept(p, 1, 1, 9, 100, ip, &tf, -1.f, 0.09f, 0.3f, ip, ip, ip, p, 1 << 20, nullptr) == MEDUSA_ERR_ARG);
  EXPECT(typical_accept(p, 1, 1, 8, 100, ip, &tf, 0.7f, 0.09f, 0.3f, ip, ip, ip, p, 1 << 20, nullptr) == MEDUSA_ERR_SHAPE);
  EXPECT(evaluate_posterior(p, 1, 1, 9, 100, ip, &tf, 0.7f, 0.09f, 0.3f, 0.9f, 2, 0, ip, ip, ip, p, 1 << 20, nullptr) == MEDUSA_ERR_ARG);
  EXPECT(typical_accept_noalloc(p, 1, 4000, 9, 1 << 20, ip, &tf, 0.7f, 0.09f, 0.3f, ip, ip, ip, nullptr) == MEDUSA_ERR_WORKSPACE);
  EXPECT(build_tree(nullptr, 0, 0, 1, 3, ip, ip, ip, 1, 1, &tf, ip, ip, nullptr) == MEDUSA_ERR_TREE);
  EXPECT(commit_accepted(&tf, 1, ip, ip, ip, ip, p, p, 1, 4, 5, 128, ip, ip, ip, ip, ip, nullptr, 0, nullptr, nullptr) == MEDUSA_ERR_SHAPE);
  EXPECT(medusa_stream_read(p, 24, reinterpret_cast<uint32_t*>(p), nullptr) == MEDUSA_ERR_SHAPE);
  (void)fp;
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("capi host checks ok\n");
  return 0;
}
