// Internal launchers of libmedusa_hip (host side).  Arguments are validated by the C ABI layer
// before any of these is called.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace medusa {

// ---- per-kernel timing hook (medusa_set_kernel_events) -----------------------------------
constexpr int kKernelCount = 9;
enum KernelId { K_HEADS_W1 = 0, K_HEADS_W2, K_TOPK, K_TREE_GATHER, K_ATTENTION, K_ATTN_COMBINE,
                K_ACCEPT, K_COMMIT, K_ROPE };
struct EventHook {
  hipEvent_t before = nullptr, after = nullptr;
};
EventHook* event_hooks();   // this thread's hooks, kKernelCount entries
inline void hook_before(int k, hipStream_t s) {
  if (event_hooks()[k].before) (void)hipEventRecord(event_hooks()[k].before, s);
}
inline void hook_after(int k, hipStream_t s) {
  if (event_hooks()[k].after) (void)hipEventRecord(event_hooks()[k].after, s);
}

// ---- heads -------------------------------------------------------------------------------
struct HeadsWs {
  size_t r, r2, xs, xs2, xn, logits, part, total;
  int chunks;
};
HeadsWs heads_ws_layout(int B, int hd, long V, int K, int topk, int nb = 1, int ln = 0);
// The tree gather done by the top-k merge (tokens == nullptr: none): tokens and position ids of
// every node from the merged candidates, as build_tree's gather computes them.
struct TreeGather {
  const int32_t* depth = nullptr;     // [T]
  const int32_t* rank = nullptr;      // [T]
  const int32_t* root = nullptr;      // [B]
  const int32_t* prefix_len = nullptr;  // [B]
  int32_t* tokens = nullptr;          // [B][T]
  int32_t* pos = nullptr;             // [B][T]
  int T = 0;
};
hipError_t launch_heads_ex(const void* h, const void* w1, const void* b1, const void* gamma,
                           const void* beta, float eps, const void* w2, int dtype, int packed, int nb,
                           int B, int hd, long V, int K, int topk, float* logits, int32_t* topk_ids,
                           float* topk_logits, char* ws, hipStream_t s,
                           const TreeGather* gather = nullptr);
hipError_t launch_heads(const void* h, const void* w1, const void* b1, const void* w2, int dtype,
                        int packed, int B, int hd, long V, int K, int topk, float* logits,
                        int32_t* topk_ids, float* topk_logits, char* ws, hipStream_t s,
                        const TreeGather* gather = nullptr);
size_t packed_weight_bytes(int K, long rows, int hd);
hipError_t launch_pack_weights(const void* w, int K, long rows, int hd, void* packed, hipStream_t s);

// ---- tree --------------------------------------------------------------------------------
hipError_t launch_tree_gather(const int32_t* topk_ids, int K, int topk, const int32_t* root_tokens,
                              const int32_t* prefix_len, int B, int T, const int32_t* depth,
                              const int32_t* rank, int32_t* tokens, int32_t* position_ids,
                              hipStream_t s);

// ---- tree attention ----------------------------------------------------------------------
struct AttnPlan {
  int G;          // q heads per kv head
  int M;          // query rows per (b, kv head) = G * T
  int rows;       // query rows per work-group (128, or 144 with nine one-block waves)
  int qtiles;     // work-group query tiles per (b, kv head)
  int splits;     // KV splits per (b, kv head, q tile)
  int nmb;        // 16-row blocks per wave of the bf16 kernel (1: 8 waves, 2: 4 waves)
  int xrem;       // query tiles that also own one row past the last full 128-row tile (0: none)
  int mpad;       // row stride of the split partials per (b, kv head)
  size_t ws_o, ws_ml, total;
};
AttnPlan attn_plan(int dtype, int B, int Hq, int Hkv, int T, int D, int max_prefix_len);
// rope_cs != nullptr: the queries are rotated in the kernel as they are loaded, with the cos/sin
// table [B*T][2][D/2] of launch_rope_tree; the tree key rows must already be rotated in the cache
hipError_t launch_tree_attention(const void* q, const void* kc, const void* vc, int dtype,
                                 const int32_t* prefix_len, int max_prefix_len, long lcap,
                                 const uint64_t* mask, int B, int Hq, int Hkv, int T, int D,
                                 float scale, void* out, char* ws, hipStream_t s,
                                 const float* rope_cs = nullptr);

// ---- typical acceptance ------------------------------------------------------------------
struct AcceptWs {
  size_t part, dec, mass, total;
  int chunks, unroll;
};
// maxc_nucleus > 0: the nucleus mode's per-child masses for nodes of at most that many children
AcceptWs accept_ws_layout(int B, int T, long V, int n_internal, int maxc_nucleus = 0);
hipError_t launch_typical_accept(const void* logits, int dtype, int B, int T, long V,
                                 const int32_t* tokens, int n_internal, const int32_t* internal,
                                 const int32_t* child_ptr, const int32_t* child_idx,
                                 const int32_t* paths, const int32_t* path_len, int n_paths,
                                 int dmax, float temperature, float eps, float delta,
                                 int nucleus, float top_p, int maxc,
                                 int32_t* best, int32_t* accept_len, int32_t* next_token,
                                 char* ws, hipStream_t s);

// ---- commit of the accepted candidate ----------------------------------------------------------
struct CommitArgs {
  const int32_t* paths;        // [n_paths][dmax + 1]
  const int32_t* path_len;     // [n_paths]
  int n_paths, dmax, T;
  const int32_t* best;
  const int32_t* accept_len;
  const int32_t* tokens;       // [B][T]
  const int32_t* next_token;   // [B]
  char* kc;                    // [B][Hkv][lcap][D]
  char* vc;
  int Hkv;
  long lcap;
  int row_bytes;               // D * element size, a multiple of 16
  const int32_t* prefix_len;
  int32_t* new_prefix_len;
  int32_t* out_tokens;         // [B][dmax + 1]
  int32_t* out_count;
  int32_t* new_root;           // nullable
  const char* hidden;          // [B][T][hd], nullable
  int hidden_bytes;            // hd * element size, a multiple of 16
  char* next_hidden;           // [B][hd], nullable
};
hipError_t launch_commit(const CommitArgs& a, int B, hipStream_t s);

// ---- rotary embedding of the tree tokens ----------------------------------------------------
struct RopeArgs {
  void* kc;                 // [B][Hkv][lcap][D], tree rows rotated in place
  const int32_t* prefix_len;
  const int32_t* pos;       // [B][T]
  float* cs_table;          // [B*T][2][D/2] cos then sin of every node, written (may be null)
  float base;
  int B, Hkv, T, D, Lmax;
  long lcap;
};
hipError_t launch_rope_tree(const RopeArgs& a, int dtype, hipStream_t s);

// ---- sparse candidate tree (host) ----------------------------------------------------------
double build_sparse_tree(const double* acc, int K, int topk, int N, int32_t* choices);

// ---- measurement --------------------------------------------------------------------------
hipError_t launch_stream_read(const void* buf, long n16, uint32_t* sink, hipStream_t s);

}  // namespace medusa
