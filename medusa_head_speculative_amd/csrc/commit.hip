// Commit of one step's accepted candidate: the decode-loop glue after typical acceptance.
//
// Wiblog "Medusa multi-head speculative decoding", inference-flow section: acceptance walks from
// the root to the first rejection or a leaf; the accepted prefix is output and the next round
// starts from the last accepted token, whose distribution the verification logits already hold.
// So for sequence b, with best path p, accept length a, prefix length L and path[k] the node at
// depth k: the root and the a accepted nodes are emitted; the K/V of path[k] moves from tree
// row L + path[k] to row L + k (the root is already at L), so the cache holds the accepted
// sequence in order; the prefix grows by a + 1; next_token becomes the next root, and the last
// accepted node's hidden state is what the next step's heads read.
//
// One work-group of 1024 threads per sequence (one work-group, so the in-place update of
// prefix_len stays safe).  A thread owns some (kv head, K or V, 16-byte column) slots and walks
// them in increasing depth: node ids grow with depth (path[k] >= k), so no destination
// row L + k is the source of a later depth, and each store depends on the load just before it,
// which orders every read of a row before any later write to it.
#include "common.h"
#include "kernels.h"

namespace medusa {

constexpr int kCommitThreads = 1024;

__global__ __launch_bounds__(kCommitThreads) void commit_kernel(CommitArgs a) {
  const int b = blockIdx.x;
  const int p = a.best[b], acc = a.accept_len[b], L = a.prefix_len[b];
  const bool ok = p >= 0 && p < a.n_paths && acc >= 0 && acc <= a.path_len[p] && L >= 0 &&
                  static_cast<long>(L) + a.T <= a.lcap;
  const int32_t* path = a.paths + static_cast<long>(ok ? p : 0) * (a.dmax + 1);

  if (ok && acc > 0) {
    const int chunks = a.row_bytes / 16;
    const int cols = a.Hkv * 2 * chunks;
    for (int c = threadIdx.x; c < cols; c += kCommitThreads) {
      const int ch = c % chunks;
      const int rest = c / chunks;
      char* base = ((rest & 1) ? a.vc : a.kc) +
                   ((static_cast<long>(b) * a.Hkv + (rest >> 1)) * a.lcap + L) * a.row_bytes + ch * 16;
      for (int k = 1; k <= acc; ++k) {
        const uint4 v = *reinterpret_cast<const uint4*>(base + static_cast<long>(path[k]) * a.row_bytes);
        *reinterpret_cast<uint4*>(base + static_cast<long>(k) * a.row_bytes) = v;
      }
    }
  }
  for (int k = threadIdx.x; k <= a.dmax; k += kCommitThreads) {
    int32_t tok = -1;
    if (ok && k <= acc) tok = a.tokens[static_cast<long>(b) * a.T + path[k]];
    a.out_tokens[static_cast<long>(b) * (a.dmax + 1) + k] = tok;
  }
  if (ok && a.hidden && a.next_hidden) {
    const int last = path[acc];
    const char* src = a.hidden + (static_cast<long>(b) * a.T + last) * a.hidden_bytes;
    char* dst = a.next_hidden + static_cast<long>(b) * a.hidden_bytes;
    for (int i = threadIdx.x; i < a.hidden_bytes / 16; i += kCommitThreads)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  }
  __syncthreads();   // every thread has read prefix_len[b]; it may alias new_prefix_len
  if (threadIdx.x == 0) {
    a.out_count[b] = ok ? acc + 1 : 0;
    a.new_prefix_len[b] = ok ? L + acc + 1 : L;
    if (a.new_root) a.new_root[b] = a.next_token[b];
  }
}

hipError_t launch_commit(const CommitArgs& a, int B, hipStream_t s) {
  hook_before(K_COMMIT, s);
  commit_kernel<<<B, kCommitThreads, 0, s>>>(a);
  hook_after(K_COMMIT, s);
  return hipGetLastError();
}

}  // namespace medusa
