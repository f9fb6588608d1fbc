// Per-step part of the candidate tree: token ids and depth-based position ids.
//
// Wiblog "Medusa multi-head speculative decoding", tree-attention section: the heads' top-k
// candidates combine into a tree (head d fills depth d) and every token gets the position index
// of its own path.  The static part (order, parents, mask, paths) is built once on the host.
#include "common.h"
#include "kernels.h"

namespace medusa {

__global__ __launch_bounds__(256) void tree_gather(const int32_t* __restrict__ topk_ids, int K,
                                                   int topk, const int32_t* __restrict__ root,
                                                   const int32_t* __restrict__ prefix_len, int B,
                                                   int T, const int32_t* __restrict__ depth,
                                                   const int32_t* __restrict__ rank,
                                                   int32_t* __restrict__ tokens,
                                                   int32_t* __restrict__ pos) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= static_cast<long>(B) * T) return;
  const int b = static_cast<int>(i / T), n = static_cast<int>(i - static_cast<long>(b) * T);
  // the four independent loads go out together, then the one that needs depth and rank; the
  // root (depth 0) reads head 0's first candidate, an always valid address, and keeps its own
  // token
  const int d = depth[n], r = rank[n], rt = root[b], pl = prefix_len[b];
  const int tk = topk_ids[(static_cast<long>(b) * K + (d > 0 ? d - 1 : 0)) * topk + (d > 0 ? r : 0)];
  tokens[i] = d == 0 ? rt : tk;
  pos[i] = pl + d;
}

hipError_t launch_tree_gather(const int32_t* topk_ids, int K, int topk, const int32_t* root_tokens,
                              const int32_t* prefix_len, int B, int T, const int32_t* depth,
                              const int32_t* rank, int32_t* tokens, int32_t* position_ids,
                              hipStream_t s) {
  const long n = static_cast<long>(B) * T;
  hook_before(K_TREE_GATHER, s);
  tree_gather<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
      topk_ids, K, topk, root_tokens, prefix_len, B, T, depth, rank, tokens, position_ids);
  hook_after(K_TREE_GATHER, s);
  return hipGetLastError();
}

}  // namespace medusa
