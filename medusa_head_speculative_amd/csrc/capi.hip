// C ABI of libmedusa_hip: argument validation, error reporting, workspace sizing, the host-side
// static tree, and dispatch to the kernel launchers.  Every check runs before any launch, so a
// rejected call writes nothing.  A checked host build (-DMEDUSA_CHECKED) turns on the standard
// library's bounds assertions on every container access of the host code (tree parsing).
#ifdef MEDUSA_CHECKED
#define _GLIBCXX_ASSERTIONS 1
#endif
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "../../include/medusa.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

// A fault of earlier asynchronous work (or a failed launch) is reported by the next call.
int check_pending() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MEDUSA_ERR_HIP, "HIP error from earlier work: %s", hipGetErrorString(e));
  return MEDUSA_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MEDUSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  g_err[0] = '\0';
  return MEDUSA_OK;
}

bool dtype_ok(int dt) { return dt == MEDUSA_F32 || dt == MEDUSA_BF16; }

// ---- static tree (host) -------------------------------------------------------------------
struct HostTree {
  int T = 0, W = 0, P = 0, dmax = 0, n_int = 0, max_rank = 0;
  std::vector<uint64_t> mask;
  std::vector<int32_t> parent, depth, rank, paths, path_len, child_ptr, child_idx, internal;
};

int parse_tree(const int32_t* choices, int n, int max_depth, int K, int topk, HostTree* out,
               bool want_arrays) {
  if (!choices) return fail(MEDUSA_ERR_ARG, "choices is NULL");
  if (n < 1 || n > 4095) return fail(MEDUSA_ERR_TREE, "n_choices = %d, need 1..4095", n);
  if (max_depth < 1 || max_depth > 8) return fail(MEDUSA_ERR_TREE, "max_depth = %d, need 1..8", max_depth);
  if (K < 1 || K > 8) return fail(MEDUSA_ERR_SHAPE, "K = %d, need 1..8", K);
  if (topk < 1 || topk > 64) return fail(MEDUSA_ERR_SHAPE, "topk = %d, need 1..64", topk);
  std::vector<std::vector<int32_t>> tup(n);
  for (int c = 0; c < n; ++c) {
    int d = 0;
    while (d < max_depth && choices[c * max_depth + d] >= 0) ++d;
    for (int e = d; e < max_depth; ++e)
      if (choices[c * max_depth + e] != -1)
        return fail(MEDUSA_ERR_TREE, "choice %d: entries after the first -1 must be -1", c);
    if (d == 0) return fail(MEDUSA_ERR_TREE, "choice %d is empty", c);
    if (d > K) return fail(MEDUSA_ERR_TREE, "choice %d has depth %d > K = %d", c, d, K);
    for (int e = 0; e < d; ++e)
      if (choices[c * max_depth + e] >= topk)
        return fail(MEDUSA_ERR_TREE, "choice %d: rank %d >= topk = %d", c, choices[c * max_depth + e], topk);
    tup[c].assign(choices + c * max_depth, choices + c * max_depth + d);
  }
  std::sort(tup.begin(), tup.end(), [](const std::vector<int32_t>& a, const std::vector<int32_t>& b) {
    return a.size() != b.size() ? a.size() < b.size() : a < b;
  });
  for (int c = 1; c < n; ++c)
    if (tup[c] == tup[c - 1]) return fail(MEDUSA_ERR_TREE, "duplicate choice");
  std::map<std::vector<int32_t>, int> index;
  index[{}] = 0;
  for (int c = 0; c < n; ++c) index[tup[c]] = c + 1;
  const int T = n + 1;
  std::vector<int32_t> parent(T, -1), depth(T, 0), rank(T, -1);
  for (int c = 0; c < n; ++c) {
    std::vector<int32_t> pre(tup[c].begin(), tup[c].end() - 1);
    auto it = index.find(pre);
    if (it == index.end()) return fail(MEDUSA_ERR_TREE, "choice list is not prefix-closed");
    parent[c + 1] = it->second;
    depth[c + 1] = static_cast<int32_t>(tup[c].size());
    rank[c + 1] = tup[c].back();
  }
  std::vector<int32_t> nchild(T, 0);
  for (int i = 1; i < T; ++i) ++nchild[parent[i]];
  HostTree& h = *out;
  h.T = T;
  h.W = (T + 63) / 64;
  h.dmax = *std::max_element(depth.begin(), depth.end());
  h.P = 0;
  h.n_int = 0;
  for (int i = 0; i < T; ++i) (nchild[i] == 0 ? h.P : h.n_int) += 1;
  h.max_rank = *std::max_element(rank.begin(), rank.end());
  if (!want_arrays) return MEDUSA_OK;
  h.parent = parent;
  h.depth = depth;
  h.rank = rank;
  h.mask.assign(static_cast<size_t>(T) * h.W, 0ull);
  for (int i = 0; i < T; ++i)
    for (int j = i; j >= 0; j = parent[j]) h.mask[static_cast<size_t>(i) * h.W + j / 64] |= 1ull << (j % 64);
  h.child_ptr.assign(T + 1, 0);
  for (int i = 0; i < T; ++i) h.child_ptr[i + 1] = h.child_ptr[i] + nchild[i];
  h.child_idx.assign(std::max(T - 1, 1), 0);
  std::vector<int32_t> fill(h.child_ptr.begin(), h.child_ptr.end() - 1);
  for (int i = 1; i < T; ++i) h.child_idx[fill[parent[i]]++] = i;   // ascending node order
  for (int i = 0; i < T; ++i)
    if (nchild[i]) h.internal.push_back(i);
  // leaves in rank-tuple order: node order is (depth, tuple); sort leaves by tuple
  std::vector<int> leaves;
  for (int i = 1; i < T; ++i)
    if (!nchild[i]) leaves.push_back(i);
  std::sort(leaves.begin(), leaves.end(), [&](int a, int b) { return tup[a - 1] < tup[b - 1]; });
  h.paths.assign(static_cast<size_t>(h.P) * (h.dmax + 1), -1);
  h.path_len.assign(h.P, 0);
  for (int p = 0; p < h.P; ++p) {
    int d = depth[leaves[p]];
    h.path_len[p] = d;
    for (int j = leaves[p]; j >= 0; j = parent[j]) h.paths[static_cast<size_t>(p) * (h.dmax + 1) + depth[j]] = j;
  }
  return MEDUSA_OK;
}

template <typename T>
int upload(T* dst, const std::vector<T>& src, const char* name) {
  if (!dst) return fail(MEDUSA_ERR_ARG, "tree->%s is NULL", name);
  hipError_t e = hipMemcpy(dst, src.data(), sizeof(T) * src.size(), hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(MEDUSA_ERR_HIP, "copy of tree->%s: %s", name, hipGetErrorString(e));
  return MEDUSA_OK;
}

}  // namespace

namespace medusa {
EventHook* event_hooks() {
  static thread_local EventHook hooks[kKernelCount];
  return hooks;
}
}  // namespace medusa

extern "C" {

const char* medusa_last_error(void) { return g_err; }

// ---- heads ----------------------------------------------------------------------------------
// packed: the weights come in the matrix-core operand order of medusa_pack_weights, which cuts
// the hidden dimension into whole 32-column blocks
static int heads_shape(int B, int hidden, long vocab, int K, int topk, bool packed = false) {
  if (B < 1 || B > 8) return fail(MEDUSA_ERR_SHAPE, "B = %d, need 1..8", B);
  if (hidden < 8 || hidden > 16384 || hidden % 8)
    return fail(MEDUSA_ERR_SHAPE, "hidden = %d, need a multiple of 8 in 8..16384", hidden);
  if (packed && hidden % 32)
    return fail(MEDUSA_ERR_UNSUPPORTED, "hidden = %d: packed weights need a multiple of 32", hidden);
  if (vocab < 1 || vocab >= (1l << 31)) return fail(MEDUSA_ERR_SHAPE, "vocab = %ld out of range", vocab);
  if (K < 1 || K > 8) return fail(MEDUSA_ERR_SHAPE, "K = %d, need 1..8", K);
  if (topk < 1 || topk > 64 || topk > vocab) return fail(MEDUSA_ERR_SHAPE, "topk = %d, need 1..min(64, vocab)", topk);
  return MEDUSA_OK;
}

size_t medusa_heads_workspace(int B, int hidden, long vocab, int K, int topk) {
  if (heads_shape(B, hidden, vocab, K, topk) != MEDUSA_OK) return 0;
  return medusa::heads_ws_layout(B, hidden, vocab, K, topk).total;
}

int medusa_heads(const void* h, const void* w1, const void* b1, const void* w2, int dtype, int B,
                 int hidden, long vocab, int K, int topk, float* logits, int32_t* topk_ids,
                 float* topk_logits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_DTYPE, "dtype = %d", dtype);
  if (!h || !w1 || !b1 || !w2 || !topk_ids) return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  int rc = heads_shape(B, hidden, vocab, K, topk);
  if (rc) return rc;
  const size_t need = medusa::heads_ws_layout(B, hidden, vocab, K, topk).total;
  if (!workspace || workspace_bytes < need)
    return fail(MEDUSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if ((rc = check_pending())) return rc;
  return launched(medusa::launch_heads(h, w1, b1, w2, dtype, 0, B, hidden, vocab, K, topk, logits,
                                       topk_ids, topk_logits, static_cast<char*>(workspace),
                                       static_cast<hipStream_t>(stream)),
                  "medusa_heads");
}

size_t medusa_heads_ex_workspace(int B, int hidden, long vocab, int K, int n_blocks, int layernorm,
                                 int topk) {
  if (heads_shape(B, hidden, vocab, K, topk) != MEDUSA_OK || n_blocks < 1 || n_blocks > 8) return 0;
  return medusa::heads_ws_layout(B, hidden, vocab, K, topk, n_blocks, layernorm ? 1 : 0).total;
}

int medusa_heads_ex(const void* h, const void* w1, const void* b1, const void* ln_gamma,
                    const void* ln_beta, float ln_eps, const void* w2, int dtype, int packed,
                    int B, int hidden, long vocab, int K, int n_blocks, int topk, float* logits,
                    int32_t* topk_ids, float* topk_logits, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_DTYPE, "dtype = %d", dtype);
  if (packed && dtype != MEDUSA_BF16) return fail(MEDUSA_ERR_DTYPE, "packed weights are bf16");
  if (!h || !w1 || !b1 || !w2 || !topk_ids) return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  if ((ln_gamma == nullptr) != (ln_beta == nullptr))
    return fail(MEDUSA_ERR_ARG, "give both ln_gamma and ln_beta or neither");
  if (ln_gamma && !(ln_eps > 0.f && std::isfinite(ln_eps))) return fail(MEDUSA_ERR_ARG, "ln_eps = %g, need > 0", ln_eps);
  int rc = heads_shape(B, hidden, vocab, K, topk, packed != 0);
  if (rc) return rc;
  if (n_blocks < 1 || n_blocks > 8) return fail(MEDUSA_ERR_SHAPE, "n_blocks = %d, need 1..8", n_blocks);
  const size_t need = medusa::heads_ws_layout(B, hidden, vocab, K, topk, n_blocks, ln_gamma ? 1 : 0).total;
  if (!workspace || workspace_bytes < need)
    return fail(MEDUSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if ((rc = check_pending())) return rc;
  return launched(medusa::launch_heads_ex(h, w1, b1, ln_gamma, ln_beta, ln_eps, w2, dtype, packed ? 1 : 0,
                                          n_blocks, B, hidden, vocab, K, topk, logits, topk_ids,
                                          topk_logits, static_cast<char*>(workspace),
                                          static_cast<hipStream_t>(stream)),
                  "medusa_heads_ex");
}

size_t medusa_packed_weight_bytes(int K, long rows, int hidden) {
  if (K < 1 || K > 64 || rows < 1 || rows >= (1l << 31) || hidden < 32 || hidden > 16384 || hidden % 32)
    return 0;
  return medusa::packed_weight_bytes(K, rows, hidden);
}

int medusa_pack_weights(const void* w, int K, long rows, int hidden, void* packed, void* stream) {
  if (!w || !packed) return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  if (medusa_packed_weight_bytes(K, rows, hidden) == 0)
    return fail(MEDUSA_ERR_SHAPE, "K = %d, rows = %ld, hidden = %d", K, rows, hidden);
  int rc;
  if ((rc = check_pending())) return rc;
  return launched(medusa::launch_pack_weights(w, K, rows, hidden, packed, static_cast<hipStream_t>(stream)),
                  "medusa_pack_weights");
}

int medusa_heads_packed(const void* h, const void* w1_packed, const void* b1,
                        const void* w2_packed, int B, int hidden, long vocab, int K, int topk,
                        float* logits, int32_t* topk_ids, float* topk_logits, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (!h || !w1_packed || !b1 || !w2_packed || !topk_ids) return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  int rc = heads_shape(B, hidden, vocab, K, topk, true);
  if (rc) return rc;
  const size_t need = medusa::heads_ws_layout(B, hidden, vocab, K, topk).total;
  if (!workspace || workspace_bytes < need)
    return fail(MEDUSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if ((rc = check_pending())) return rc;
  return launched(medusa::launch_heads(h, w1_packed, b1, w2_packed, MEDUSA_BF16, 1, B, hidden, vocab,
                                       K, topk, logits, topk_ids, topk_logits,
                                       static_cast<char*>(workspace), static_cast<hipStream_t>(stream)),
                  "medusa_heads_packed");
}

int medusa_heads_build_tree(const void* h, const void* w1, const void* b1, const void* w2,
                            int dtype, int packed, int B, int hidden, long vocab, int K, int topk,
                            const medusa_tree* tree, const int32_t* root_tokens,
                            const int32_t* prefix_len, float* logits, int32_t* topk_ids,
                            float* topk_logits, int32_t* tokens, int32_t* position_ids,
                            void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_DTYPE, "dtype = %d", dtype);
  if (packed != 0 && packed != 1) return fail(MEDUSA_ERR_ARG, "packed must be 0 or 1");
  if (packed && dtype != MEDUSA_BF16) return fail(MEDUSA_ERR_DTYPE, "packed weights are bf16");
  if (!h || !w1 || !b1 || !w2 || !topk_ids || !tree || !root_tokens || !prefix_len || !tokens ||
      !position_ids)
    return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  if (!tree->depth || !tree->rank) return fail(MEDUSA_ERR_ARG, "tree->depth / tree->rank is NULL");
  int rc = heads_shape(B, hidden, vocab, K, topk, packed != 0);
  if (rc) return rc;
  if (tree->T < 2 || tree->T > 4096) return fail(MEDUSA_ERR_TREE, "tree->T = %d", tree->T);
  // the merge of head d - 1 writes the nodes of depth d from its candidates of rank < topk
  if (tree->dmax < 1 || tree->dmax > K)
    return fail(MEDUSA_ERR_TREE, "tree->dmax = %d does not fit K = %d", tree->dmax, K);
  if (tree->max_rank < 0 || tree->max_rank >= topk)
    return fail(MEDUSA_ERR_TREE, "tree->max_rank = %d does not fit topk = %d", tree->max_rank, topk);
  const size_t need = medusa::heads_ws_layout(B, hidden, vocab, K, topk).total;
  if (!workspace || workspace_bytes < need)
    return fail(MEDUSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if ((rc = check_pending())) return rc;
  medusa::TreeGather g;
  g.depth = tree->depth;
  g.rank = tree->rank;
  g.root = root_tokens;
  g.prefix_len = prefix_len;
  g.tokens = tokens;
  g.pos = position_ids;
  g.T = tree->T;
  return launched(medusa::launch_heads(h, w1, b1, w2, dtype, packed, B, hidden, vocab, K, topk,
                                       logits, topk_ids, topk_logits, static_cast<char*>(workspace),
                                       static_cast<hipStream_t>(stream), &g),
                  "medusa_heads_build_tree");
}

// ---- tree -----------------------------------------------------------------------------------
int medusa_tree_dims(const int32_t* choices, int n_choices, int max_depth, int K, int topk,
                     medusa_tree* tree) {
  if (!tree) return fail(MEDUSA_ERR_ARG, "tree is NULL");
  HostTree h;
  int rc = parse_tree(choices, n_choices, max_depth, K, topk, &h, false);
  if (rc) return rc;
  tree->T = h.T;
  tree->W = h.W;
  tree->n_paths = h.P;
  tree->dmax = h.dmax;
  tree->n_internal = h.n_int;
  tree->max_rank = h.max_rank;
  g_err[0] = '\0';
  return MEDUSA_OK;
}

int build_tree(const int32_t* choices, int n_choices, int max_depth, int K, int topk,
               const int32_t* topk_ids, const int32_t* root_tokens, const int32_t* prefix_len,
               int B, int static_ready, const medusa_tree* tree, int32_t* tokens,
               int32_t* position_ids, void* stream) {
  if (!tree) return fail(MEDUSA_ERR_ARG, "tree is NULL");
  if (!topk_ids || !root_tokens || !prefix_len || !tokens || !position_ids)
    return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  if (B < 1 || B > 4096) return fail(MEDUSA_ERR_SHAPE, "B = %d", B);
  if (K < 1 || K > 8 || topk < 1 || topk > 64) return fail(MEDUSA_ERR_SHAPE, "K = %d, topk = %d", K, topk);
  if (static_ready != 0 && static_ready != 1) return fail(MEDUSA_ERR_ARG, "static_ready must be 0 or 1");
  if (!tree->depth || !tree->rank) return fail(MEDUSA_ERR_ARG, "tree->depth / tree->rank is NULL");
  int rc;
  if (static_ready == 0) {
    HostTree h;
    if ((rc = parse_tree(choices, n_choices, max_depth, K, topk, &h, true))) return rc;
    if (tree->T != h.T || tree->W != h.W || tree->n_paths != h.P || tree->dmax != h.dmax ||
        tree->n_internal != h.n_int || tree->max_rank != h.max_rank)
      return fail(MEDUSA_ERR_TREE, "tree dims do not match the choice list (call medusa_tree_dims)");
    if ((rc = check_pending())) return rc;
    if ((rc = upload(tree->mask, h.mask, "mask")) || (rc = upload(tree->parent, h.parent, "parent")) ||
        (rc = upload(tree->depth, h.depth, "depth")) || (rc = upload(tree->rank, h.rank, "rank")) ||
        (rc = upload(tree->paths, h.paths, "paths")) ||
        (rc = upload(tree->path_len, h.path_len, "path_len")) ||
        (rc = upload(tree->child_ptr, h.child_ptr, "child_ptr")) ||
        (rc = upload(tree->child_idx, h.child_idx, "child_idx")) ||
        (rc = upload(tree->internal, h.internal, "internal")))
      return rc;
  } else {
    if (tree->T < 2 || tree->T > 4096) return fail(MEDUSA_ERR_TREE, "tree->T = %d", tree->T);
    // the gather reads topk_ids[b][depth - 1][rank]: the tree must fit this K and topk
    if (tree->dmax < 1 || tree->dmax > K)
      return fail(MEDUSA_ERR_TREE, "tree->dmax = %d does not fit K = %d", tree->dmax, K);
    if (tree->max_rank < 0 || tree->max_rank >= topk)
      return fail(MEDUSA_ERR_TREE, "tree->max_rank = %d does not fit topk = %d", tree->max_rank, topk);
    if ((rc = check_pending())) return rc;
  }
  return launched(medusa::launch_tree_gather(topk_ids, K, topk, root_tokens, prefix_len, B, tree->T,
                                             tree->depth, tree->rank, tokens, position_ids,
                                             static_cast<hipStream_t>(stream)),
                  "build_tree");
}

// ---- tree attention -------------------------------------------------------------------------
static int attn_shape(int B, int Hq, int Hkv, int T, int D, int max_prefix_len) {
  if (B < 1 || B > 4096 || Hq < 1 || Hq > 256 || Hkv < 1 || Hq % Hkv)
    return fail(MEDUSA_ERR_SHAPE, "B = %d, Hq = %d, Hkv = %d (need B <= 4096, Hq %% Hkv == 0, Hq <= 256)", B, Hq, Hkv);
  if (D != 64 && D != 128) return fail(MEDUSA_ERR_SHAPE, "D = %d, need 64 or 128", D);
  if (T < 1 || T > 4096) return fail(MEDUSA_ERR_SHAPE, "T = %d, need 1..4096", T);
  if (max_prefix_len < 0 || max_prefix_len > (1 << 20)) return fail(MEDUSA_ERR_SHAPE, "max_prefix_len = %d", max_prefix_len);
  return MEDUSA_OK;
}

size_t tree_attention_workspace(int B, int Hq, int Hkv, int T, int D, int max_prefix_len) {
  if (attn_shape(B, Hq, Hkv, T, D, max_prefix_len) != MEDUSA_OK) return 0;
  // the larger of the two dtype plans, so one query serves both
  size_t a = medusa::attn_plan(1, B, Hq, Hkv, T, D, max_prefix_len).total;
  return a < 256 ? 256 : a;
}

int tree_attention(const void* q, const void* k_cache, const void* v_cache, int dtype,
                   const int32_t* prefix_len, int max_prefix_len, long lcap,
                   const uint64_t* mask, int B, int Hq, int Hkv, int T, int D, float scale,
                   void* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_DTYPE, "dtype = %d", dtype);
  if (!q || !k_cache || !v_cache || !prefix_len || !mask || !out)
    return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  int rc = attn_shape(B, Hq, Hkv, T, D, max_prefix_len);
  if (rc) return rc;
  if (lcap < static_cast<long>(max_prefix_len) + T) return fail(MEDUSA_ERR_SHAPE, "lcap = %ld < max_prefix_len + T", lcap);
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(static_cast<float>(D));
  if (!std::isfinite(scale)) return fail(MEDUSA_ERR_ARG, "scale is not finite");
  const size_t need = medusa::attn_plan(dtype, B, Hq, Hkv, T, D, max_prefix_len).total;
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MEDUSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if ((rc = check_pending())) return rc;
  return launched(medusa::launch_tree_attention(q, k_cache, v_cache, dtype, prefix_len, max_prefix_len,
                                                lcap, mask, B, Hq, Hkv, T, D, scale, out,
                                                static_cast<char*>(workspace),
                                                static_cast<hipStream_t>(stream)),
                  "tree_attention");
}

// ---- tree attention with rotary embedding at depth positions ---------------------------------
// The tree key rows are rotated in place by their own kernel, which also writes every node's
// cos/sin to a table [B*T][2][D/2] floats at the start of the workspace; the attention kernel
// rotates the queries with it as they are loaded.  The attention's own workspace follows.
static size_t rope_table_bytes(int B, int T, int D) {
  return (static_cast<size_t>(B) * T * D * sizeof(float) + 255) & ~static_cast<size_t>(255);
}

size_t tree_attention_rope_workspace(int B, int Hq, int Hkv, int T, int D, int max_prefix_len) {
  const size_t a = tree_attention_workspace(B, Hq, Hkv, T, D, max_prefix_len);
  return a ? rope_table_bytes(B, T, D) + a : 0;
}

int tree_attention_rope(const void* q, void* k_cache, const void* v_cache, int dtype,
                        const int32_t* prefix_len, int max_prefix_len, long lcap,
                        const uint64_t* mask, const int32_t* position_ids, float rope_base,
                        int B, int Hq, int Hkv, int T, int D, float scale, void* out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_DTYPE, "dtype = %d", dtype);
  if (!q || !k_cache || !v_cache || !prefix_len || !mask || !position_ids || !out)
    return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  int rc = attn_shape(B, Hq, Hkv, T, D, max_prefix_len);
  if (rc) return rc;
  if (lcap < static_cast<long>(max_prefix_len) + T) return fail(MEDUSA_ERR_SHAPE, "lcap = %ld < max_prefix_len + T", lcap);
  if (!(rope_base > 1.f) || !std::isfinite(rope_base)) return fail(MEDUSA_ERR_ARG, "rope_base = %g, need > 1", rope_base);
  if (!(scale > 0.f)) scale = 1.0f / std::sqrt(static_cast<float>(D));
  if (!std::isfinite(scale)) return fail(MEDUSA_ERR_ARG, "scale is not finite");
  const size_t tab = rope_table_bytes(B, T, D);
  const size_t need = tab + medusa::attn_plan(dtype, B, Hq, Hkv, T, D, max_prefix_len).total;
  if (!workspace || workspace_bytes < need)
    return fail(MEDUSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  if ((rc = check_pending())) return rc;
  char* ws = static_cast<char*>(workspace);
  float* cs = reinterpret_cast<float*>(ws);
  medusa::RopeArgs r{};
  r.kc = k_cache;
  r.cs_table = cs;
  r.prefix_len = prefix_len;
  r.pos = position_ids;
  r.base = rope_base;
  r.B = B;
  r.Hkv = Hkv;
  r.T = T;
  r.D = D;
  r.Lmax = max_prefix_len;
  r.lcap = lcap;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = launched(medusa::launch_rope_tree(r, dtype, st), "tree_attention_rope"))) return rc;
  return launched(medusa::launch_tree_attention(q, k_cache, v_cache, dtype, prefix_len,
                                                max_prefix_len, lcap, mask, B, Hq, Hkv, T, D,
                                                scale, out, ws + tab, st, cs),
                  "tree_attention_rope");
}

// ---- typical acceptance ---------------------------------------------------------------------
size_t typical_accept_workspace(int B, int T, long vocab, int n_internal) {
  if (B < 1 || T < 2 || T > 4096 || vocab < 1 || vocab >= (1l << 31) || n_internal < 1 || n_internal >= T) return 0;
  return medusa::accept_ws_layout(B, T, vocab, n_internal).total;
}

// Children per node at most: siblings carry distinct ranks below topk <= 64.  The nucleus mode
// keeps one mass per possible child of every chunk.
constexpr int kMaxChildren = 64;

// Checks of typical_accept's (evaluate_posterior's) arguments other than the workspace; *need
// receives the workspace bytes the call takes.
static int accept_args(const void* logits, int dtype, int B, int T, long vocab,
                       const int32_t* tokens, const medusa_tree* tree, float temperature,
                       float posterior_threshold, float posterior_alpha,
                       const int32_t* best_candidate, const int32_t* accept_length, size_t* need,
                       bool nucleus = false) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_DTYPE, "dtype = %d", dtype);
  if (!logits || !tokens || !tree || !best_candidate || !accept_length)
    return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  if (!tree->internal || !tree->child_ptr || !tree->child_idx || !tree->paths || !tree->path_len)
    return fail(MEDUSA_ERR_ARG, "a tree array is NULL");
  if (B < 1 || B > 65535) return fail(MEDUSA_ERR_SHAPE, "B = %d", B);
  if (T != tree->T || T < 2 || T > 4096) return fail(MEDUSA_ERR_SHAPE, "T = %d does not match tree->T = %d", T, tree->T);
  if (vocab < 1 || vocab >= (1l << 31)) return fail(MEDUSA_ERR_SHAPE, "vocab = %ld", vocab);
  if (tree->n_internal < 1 || tree->n_internal >= T || tree->n_paths < 1 || tree->dmax < 1)
    return fail(MEDUSA_ERR_TREE, "tree dims are inconsistent");
  if (!(temperature >= 0.f) || !std::isfinite(temperature)) return fail(MEDUSA_ERR_ARG, "temperature = %g, need >= 0", temperature);
  if (!(posterior_threshold > 0.f && posterior_threshold < 1.f))
    return fail(MEDUSA_ERR_ARG, "posterior_threshold = %g, need 0 < eps < 1", posterior_threshold);
  if (!(posterior_alpha > 0.f) || !std::isfinite(posterior_alpha))
    return fail(MEDUSA_ERR_ARG, "posterior_alpha = %g, need > 0", posterior_alpha);
  *need = medusa::accept_ws_layout(B, T, vocab, tree->n_internal, nucleus ? kMaxChildren : 0).total;
  return MEDUSA_OK;
}

static int accept_launch(const void* logits, int dtype, int B, int T, long vocab,
                         const int32_t* tokens, const medusa_tree* tree, float temperature,
                         float posterior_threshold, float posterior_alpha, int32_t* best_candidate,
                         int32_t* accept_length, int32_t* next_token, char* ws, void* stream,
                         const char* what, bool nucleus = false, float top_p = 1.f) {
  int rc;
  if ((rc = check_pending())) return rc;
  return launched(medusa::launch_typical_accept(logits, dtype, B, T, vocab, tokens, tree->n_internal,
                                                tree->internal, tree->child_ptr, tree->child_idx,
                                                tree->paths, tree->path_len, tree->n_paths, tree->dmax,
                                                temperature, posterior_threshold, posterior_alpha,
                                                nucleus ? 1 : 0, top_p, kMaxChildren,
                                                best_candidate, accept_length, next_token, ws,
                                                static_cast<hipStream_t>(stream)),
                  what);
}

// ---- the candidate-filtering call with its sampling modes ----------------------------------
static int posterior_mode(float top_p, int sampling, int fast) {
  if (sampling != MEDUSA_SAMPLING_TYPICAL && sampling != MEDUSA_SAMPLING_NUCLEUS)
    return fail(MEDUSA_ERR_ARG, "sampling = %d, need MEDUSA_SAMPLING_TYPICAL or _NUCLEUS", sampling);
  if (fast != 0 && fast != 1) return fail(MEDUSA_ERR_ARG, "fast = %d, need 0 or 1", fast);
  if (!(top_p > 0.f && top_p <= 1.f)) return fail(MEDUSA_ERR_ARG, "top_p = %g, need 0 < top_p <= 1", top_p);
  return MEDUSA_OK;
}

size_t evaluate_posterior_workspace(int B, long vocab, const medusa_tree* tree, int sampling) {
  if (!tree || (sampling != MEDUSA_SAMPLING_TYPICAL && sampling != MEDUSA_SAMPLING_NUCLEUS)) return 0;
  const int T = tree->T, n_int = tree->n_internal;
  if (B < 1 || B > 65535 || T < 2 || T > 4096 || vocab < 1 || vocab >= (1l << 31) || n_int < 1 || n_int >= T)
    return 0;
  return medusa::accept_ws_layout(B, T, vocab, n_int,
                                  sampling == MEDUSA_SAMPLING_NUCLEUS ? kMaxChildren : 0).total;
}

int evaluate_posterior(const void* logits, int dtype, int B, int T, long vocab,
                       const int32_t* tokens, const medusa_tree* tree, float temperature,
                       float posterior_threshold, float posterior_alpha, float top_p,
                       int sampling, int fast, int32_t* best_candidate, int32_t* accept_length,
                       int32_t* next_token, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc = posterior_mode(top_p, sampling, fast);
  if (rc) return rc;
  const bool nucleus = sampling == MEDUSA_SAMPLING_NUCLEUS;
  size_t need = 0;
  rc = accept_args(logits, dtype, B, T, vocab, tokens, tree, temperature, posterior_threshold,
                   posterior_alpha, best_candidate, accept_length, &need, nucleus);
  if (rc) return rc;
  if (!workspace || workspace_bytes < need)
    return fail(MEDUSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  return accept_launch(logits, dtype, B, T, vocab, tokens, tree, temperature, posterior_threshold,
                       posterior_alpha, best_candidate, accept_length, next_token,
                       static_cast<char*>(workspace), stream, "evaluate_posterior", nucleus, top_p);
}

int typical_accept(const void* logits, int dtype, int B, int T, long vocab,
                   const int32_t* tokens, const medusa_tree* tree, float temperature,
                   float posterior_threshold, float posterior_alpha, int32_t* best_candidate,
                   int32_t* accept_length, int32_t* next_token, void* workspace,
                   size_t workspace_bytes, void* stream) {
  size_t need = 0;
  int rc = accept_args(logits, dtype, B, T, vocab, tokens, tree, temperature, posterior_threshold,
                       posterior_alpha, best_candidate, accept_length, &need);
  if (rc) return rc;
  if (!workspace || workspace_bytes < need)
    return fail(MEDUSA_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  return accept_launch(logits, dtype, B, T, vocab, tokens, tree, temperature, posterior_threshold,
                       posterior_alpha, best_candidate, accept_length, next_token,
                       static_cast<char*>(workspace), stream, "typical_accept");
}

// ---- typical acceptance without a caller workspace --------------------------------------------
// Its intermediates live in `scratch`, a device array of the library (one copy per GPU, held
// until the process ends).  In host code the array's name is only a stand-in for the symbol: the
// device address of each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[MEDUSA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up on its first use.
int scratch_address(char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MEDUSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(MEDUSA_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MEDUSA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return MEDUSA_OK;
}
}  // namespace

int typical_accept_noalloc(const void* logits, int dtype, int B, int T, long vocab,
                           const int32_t* tokens, const medusa_tree* tree, float temperature,
                           float posterior_threshold, float posterior_alpha,
                           int32_t* best_candidate, int32_t* accept_length, int32_t* next_token,
                           void* stream) {
  size_t need = 0;
  int rc = accept_args(logits, dtype, B, T, vocab, tokens, tree, temperature, posterior_threshold,
                       posterior_alpha, best_candidate, accept_length, &need);
  if (rc) return rc;
  if (need > MEDUSA_NOALLOC_SCRATCH_BYTES)
    return fail(MEDUSA_ERR_WORKSPACE,
                "typical_accept_noalloc: these sizes need %zu bytes of scratch, more than the %d "
                "bytes the library holds per GPU (use typical_accept with a workspace)",
                need, MEDUSA_NOALLOC_SCRATCH_BYTES);
  char* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return accept_launch(logits, dtype, B, T, vocab, tokens, tree, temperature, posterior_threshold,
                       posterior_alpha, best_candidate, accept_length, next_token, ws, stream,
                       "typical_accept_noalloc");
}

// ---- commit of the accepted candidate --------------------------------------------------------
int commit_accepted(const medusa_tree* tree, int B, const int32_t* best_candidate,
                    const int32_t* accept_length, const int32_t* tokens,
                    const int32_t* next_token, void* k_cache, void* v_cache, int dtype, int Hkv,
                    long lcap, int D, const int32_t* prefix_len, int32_t* new_prefix_len,
                    int32_t* out_tokens, int32_t* out_count, int32_t* new_root,
                    const void* hidden, int hidden_size, void* next_hidden, void* stream) {
  if (!dtype_ok(dtype)) return fail(MEDUSA_ERR_DTYPE, "dtype = %d", dtype);
  if (!tree || !best_candidate || !accept_length || !tokens || !k_cache || !v_cache ||
      !prefix_len || !new_prefix_len || !out_tokens || !out_count)
    return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  if (new_root && !next_token) return fail(MEDUSA_ERR_ARG, "new_root needs next_token");
  if ((hidden == nullptr) != (next_hidden == nullptr))
    return fail(MEDUSA_ERR_ARG, "give both hidden and next_hidden or neither");
  if (!tree->paths || !tree->path_len) return fail(MEDUSA_ERR_ARG, "a tree array is NULL");
  if (tree->T < 1 || tree->T > 4096 || tree->n_paths < 1 || tree->dmax < 0 || tree->dmax >= tree->T)
    return fail(MEDUSA_ERR_TREE, "tree dims are inconsistent");
  if (B < 1 || B > 65535) return fail(MEDUSA_ERR_SHAPE, "B = %d", B);
  if (Hkv < 1 || Hkv > 256) return fail(MEDUSA_ERR_SHAPE, "Hkv = %d", Hkv);
  const int esz = dtype == MEDUSA_BF16 ? 2 : 4;
  if (D < 1 || (D * esz) % 16 != 0) return fail(MEDUSA_ERR_SHAPE, "D = %d: D * element size must be a multiple of 16", D);
  if (lcap < tree->T) return fail(MEDUSA_ERR_SHAPE, "lcap = %ld < T = %d", lcap, tree->T);
  if (hidden && (hidden_size < 1 || (static_cast<long>(hidden_size) * esz) % 16 != 0))
    return fail(MEDUSA_ERR_SHAPE, "hidden_size = %d: hidden_size * element size must be a multiple of 16", hidden_size);
  int rc;
  if ((rc = check_pending())) return rc;
  medusa::CommitArgs a{};
  a.paths = tree->paths;
  a.path_len = tree->path_len;
  a.n_paths = tree->n_paths;
  a.dmax = tree->dmax;
  a.T = tree->T;
  a.best = best_candidate;
  a.accept_len = accept_length;
  a.tokens = tokens;
  a.next_token = next_token;
  a.kc = static_cast<char*>(k_cache);
  a.vc = static_cast<char*>(v_cache);
  a.Hkv = Hkv;
  a.lcap = lcap;
  a.row_bytes = D * esz;
  a.prefix_len = prefix_len;
  a.new_prefix_len = new_prefix_len;
  a.out_tokens = out_tokens;
  a.out_count = out_count;
  a.new_root = new_root;
  a.hidden = static_cast<const char*>(hidden);
  a.hidden_bytes = hidden ? hidden_size * esz : 0;
  a.next_hidden = static_cast<char*>(next_hidden);
  return launched(medusa::launch_commit(a, B, static_cast<hipStream_t>(stream)), "commit_accepted");
}

// ---- sparse candidate tree (host) ------------------------------------------------------------
int medusa_sparse_tree(const double* accuracy, int K, int topk, int N, int32_t* choices,
                       double* expected_accept_length) {
  if (!accuracy || !choices) return fail(MEDUSA_ERR_ARG, "a required pointer is NULL");
  if (K < 1 || K > 8) return fail(MEDUSA_ERR_SHAPE, "K = %d, need 1..8", K);
  if (topk < 1 || topk > 64) return fail(MEDUSA_ERR_SHAPE, "topk = %d, need 1..64", topk);
  double total = 0.0, level = 1.0;                 // nodes of the full tree, capped
  for (int d = 0; d < K && total <= 4095.0; ++d) {
    level *= topk;
    total += level;
  }
  if (N < 1 || N > 4095 || N > total) return fail(MEDUSA_ERR_SHAPE, "N = %d, need 1..min(4095, nodes of the full tree)", N);
  for (long i = 0; i < static_cast<long>(K) * topk; ++i)
    if (!(accuracy[i] >= 0.0 && accuracy[i] <= 1.0))
      return fail(MEDUSA_ERR_ARG, "accuracy[%ld] = %g is not in [0, 1]", i, accuracy[i]);
  const double e = medusa::build_sparse_tree(accuracy, K, topk, N, choices);
  if (expected_accept_length) *expected_accept_length = e;
  g_err[0] = '\0';
  return MEDUSA_OK;
}

// ---- measurement hook ------------------------------------------------------------------------
int medusa_set_kernel_events(int which, void* before, void* after) {
  if (which < 0 || which >= medusa::kKernelCount) return fail(MEDUSA_ERR_ARG, "kernel id %d", which);
  if ((before == nullptr) != (after == nullptr)) return fail(MEDUSA_ERR_ARG, "give both events or neither");
  medusa::event_hooks()[which].before = static_cast<hipEvent_t>(before);
  medusa::event_hooks()[which].after = static_cast<hipEvent_t>(after);
  g_err[0] = '\0';
  return MEDUSA_OK;
}

int medusa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return fail(MEDUSA_ERR_ARG, "null pointer");
  if (bytes == 0 || bytes % 16 != 0) return fail(MEDUSA_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return fail(MEDUSA_ERR_ARG, "buf must be 16-byte aligned");
  if (int st = check_pending()) return st;
  return launched(medusa::launch_stream_read(buf, static_cast<long>(bytes / 16), sink,
                                             static_cast<hipStream_t>(stream)),
                  "medusa_stream_read");
}

}  // extern "C"
