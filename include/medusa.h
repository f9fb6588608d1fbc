/*
 * medusa.h -- C ABI of libmedusa_hip.so: one Medusa verification step on an AMD MI355X
 * (gfx950).
 *
 * The step, as the pages describe it:
 *   1. medusa_heads    K heads read the last hidden state h; head k computes
 *                      W2_k (h + SiLU(W1_k h + b1_k)) and keeps its top-k tokens.
 *                      (Ultralytics glossary "Medusa Heads", section on how the heads predict
 *                      the next tokens, and its code sample; Wiblog "Medusa multi-head
 *                      speculative decoding", heads section and inference-flow section.)
 *   2. build_tree      the heads' candidates are expanded into a fixed tree given by the
 *                      `medusa_choices` list; its ancestor mask, parents and root-to-leaf paths
 *                      are precomputed once, the per-step token ids and depth-based position
 *                      ids are gathered on the device.  (Wiblog page, tree-attention section;
 *                      Ultralytics page, tree-attention section; cnnetsun page, configuration
 *                      section.)
 *   3. tree_attention  every tree token attends to the prefix KV cache and to its own
 *                      ancestors in the tree, never across branches.  (Wiblog page,
 *                      tree-attention section; Ultralytics page, tree-attention section.)
 *   4. typical_accept  a candidate is accepted when p(x) > min(eps, delta * exp(-H(p)));
 *                      greedy (exact match) at temperature 0; the walk from the root stops at
 *                      the first rejection or a leaf; the result is the best path and its
 *                      accept length.  (Wiblog page, typical-acceptance and inference-flow
 *                      sections; Ultralytics page, tree-attention section; cnnetsun page,
 *                      architecture and candidate-filtering sections, which give the call
 *                      evaluate_posterior(logits, candidates, temperature, posterior_threshold,
 *                      posterior_alpha, ...) -> (best_candidate, accept_length) and the
 *                      defaults 0.09 / 0.3.)
 * Around the step:
 *   5. commit_accepted      emits the accepted tokens, moves their K/V rows into place in the
 *                           cache and hands over the next root and hidden state (Wiblog page,
 *                           inference-flow section).
 *   tree_attention_rope     tree_attention after the rotary embedding of the tree tokens at
 *                           their depth positions (Wiblog page, tree-attention section).
 *   medusa_sparse_tree      the N-node tree of largest expected accept length for given
 *                           per-head rank accuracies (Ultralytics page, tree-attention section).
 *   medusa_heads_ex         heads of several residual blocks, optionally opened by LayerNorm
 *                           (Wiblog page, heads section).
 * For measurement only: medusa_set_kernel_events (HIP events around each kernel family) and
 * medusa_stream_read (a plain HBM read, the bandwidth ceiling the heads are compared with).
 *
 * Tuning overrides, read from the environment once per process (unset: the measured defaults).
 * They change launch shapes and so the order of fp32 sums, never what is computed:
 *   MEDUSA_W1_VARIANT, MEDUSA_W2_VARIANT  0..13, the packed bf16 GEMV variant of each layer;
 *   MEDUSA_ATTN_WG_TARGET                 work-groups tree attention splits K/V to reach (256);
 *   MEDUSA_ACCEPT_UNROLL                  1, 2 or 4 rounds per acceptance chunk (workspace
 *                                         sizes follow it, so set it before the first query).
 *
 * Conventions for every entry point:
 *   - Pointers marked "device" are HIP device memory on the current device; "host" pointers are
 *     ordinary host memory.  Every tensor is dense, row-major, 16-byte aligned.  The caller owns
 *     every buffer, workspaces included; the library allocates no device memory and keeps no
 *     state between calls except a thread-local error string.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All device work is enqueued on it
 *     asynchronously; nothing synchronises the host except build_tree with static_ready == 0.
 *   - dtype: MEDUSA_F32 (float) or MEDUSA_BF16 (bfloat16 bit patterns, uint16 storage).  It is
 *     the element type of every floating-point tensor input of the call.
 *   - Return value: MEDUSA_OK or a negative medusa_status.  Arguments are checked before any
 *     launch: a call that fails validation writes nothing.  A fault of earlier asynchronous work
 *     is reported as MEDUSA_ERR_HIP by the next call.  medusa_last_error() gives the text.
 *   - Workspaces: size them with the matching *_workspace() query.  A workspace holds only
 *     intermediates that each call writes before it reads them, so its contents on entry do
 *     not matter and it needs no clearing.  Two calls in flight at the same time (on different
 *     streams) that share a workspace race.
 */
#ifndef MEDUSA_H
#define MEDUSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MEDUSA_F32 = 0, MEDUSA_BF16 = 1 } medusa_dtype;

typedef enum {
  MEDUSA_OK = 0,
  MEDUSA_ERR_ARG = -1,         /* null pointer, bad scalar (temperature, eps, ...) */
  MEDUSA_ERR_SHAPE = -2,       /* sizes out of the supported range */
  MEDUSA_ERR_DTYPE = -3,       /* unknown dtype */
  MEDUSA_ERR_TREE = -4,        /* malformed medusa_choices */
  MEDUSA_ERR_WORKSPACE = -5,   /* workspace missing or too small */
  MEDUSA_ERR_HIP = -6,         /* HIP runtime error (launch failure or earlier async fault) */
  MEDUSA_ERR_UNSUPPORTED = -7  /* valid request outside what this build implements */
} medusa_status;

/* Text describing the last failure on the calling thread ("" if none).  Never NULL. */
const char* medusa_last_error(void);

/* ---------------------------------------------------------------------------------------- *
 * 1. Medusa heads + per-head top-k
 * ---------------------------------------------------------------------------------------- */

/* Workspace bytes for medusa_heads with these sizes (0 on invalid sizes). */
size_t medusa_heads_workspace(int B, int hidden, long vocab, int K, int topk);

/*
 * For every sequence b < B and head k < K (Ultralytics "Medusa Heads", how-the-heads-predict
 * section: one fully connected layer with SiLU and a residual connection, then a vocab
 * projection; W1 has a bias, W2 has none; torch Linear [out, in] weight layout):
 *     r[b,k]      = h[b] + SiLU(W1[k] h[b] + b1[k]),     SiLU(u) = u / (1 + e^-u)
 *     logits[b,k] = W2[k] r[b,k]
 *     topk_ids[b,k,0..topk-1] = the topk largest logits[b,k,:], descending; equal values go to
 *                               the lower token id (Wiblog page, inference-flow section: each
 *                               head outputs its top-k candidates).
 * Arguments (all device):
 *   h        [B, hidden]            dtype
 *   w1       [K, hidden, hidden]    dtype  ([out, in])
 *   b1       [K, hidden]            dtype
 *   w2       [K, vocab, hidden]     dtype  ([out, in])
 *   logits   [B, K, vocab] float32, or NULL (then kept in the workspace only)
 *   topk_ids [B, K, topk] int32
 *   topk_logits [B, K, topk] float32, or NULL
 * Arithmetic: fp32 accumulation; r is kept in fp32.  For bf16 weights the fp32 r enters the
 * matrix cores as a bf16 hi + lo pair (relative error about 2^-17 per element).
 * Limits: 1 <= B <= 8, 8 <= hidden <= 16384 and hidden % 8 == 0, 1 <= vocab < 2^31,
 *         1 <= K <= 8, 1 <= topk <= min(64, vocab).
 */
int medusa_heads(const void* h, const void* w1, const void* b1, const void* w2, int dtype, int B,
                 int hidden, long vocab, int K, int topk, float* logits, int32_t* topk_ids,
                 float* topk_logits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same heads with bf16 weights pre-packed once by medusa_pack_weights (a device-side
 * reordering of the [out, in] matrices into the matrix-core operand order, so every weight is
 * read as part of one contiguous stream).  Semantics, arguments and limits are those of
 * medusa_heads with dtype = MEDUSA_BF16; only w1_packed / w2_packed differ:
 *   w1_packed  medusa_packed_weight_bytes(K, hidden, hidden) bytes from w1
 *   w2_packed  medusa_packed_weight_bytes(K, vocab, hidden) bytes from w2
 * The packed order cuts the hidden dimension into whole 32-column blocks, so a hidden size that
 * is a multiple of 8 but not of 32 gives MEDUSA_ERR_UNSUPPORTED (medusa_heads serves it).
 */
int medusa_heads_packed(const void* h, const void* w1_packed, const void* b1,
                        const void* w2_packed, int B, int hidden, long vocab, int K, int topk,
                        float* logits, int32_t* topk_ids, float* topk_logits, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Heads of n_blocks residual blocks each, optionally opened by LayerNorm (Wiblog page, heads
 * section: a head is one or more residual blocks, of LayerNorm and a feed-forward network,
 * followed by a linear layer; the block itself is Ultralytics' fully connected layer with SiLU
 * and a residual connection).  Per head k, starting from x = h:
 *     for j in 0 .. n_blocks-1:  x <- x + SiLU(W1[k][j] n(x) + b1[k][j])
 *     logits[b][k][:] = W2[k] x,   then the per-head top-k as medusa_heads,
 * with n(x) = x when ln_gamma and ln_beta are NULL, else the LayerNorm over the hidden
 * dimension, (x - mean) / sqrt(var + ln_eps) * ln_gamma[k][j] + ln_beta[k][j] (var the mean
 * squared deviation, statistics in fp32).  x is carried in fp32 between blocks.
 *   w1     [K][n_blocks][hidden][hidden] dtype, or with packed = 1 (bf16 only) the
 *          medusa_pack_weights form of that tensor taken as K * n_blocks matrices
 *   b1     [K][n_blocks][hidden] dtype;  ln_gamma, ln_beta [K][n_blocks][hidden] dtype or NULL
 *   w2     [K][vocab][hidden] dtype, or its packed form (packed = 1)
 * Everything else as medusa_heads; n_blocks = 1 without LayerNorm is exactly medusa_heads
 * (packed = 0) or medusa_heads_packed (packed = 1).  The workspace query takes layernorm = 0/1.
 * Limits: those of medusa_heads (packed = 1: those of medusa_heads_packed), 1 <= n_blocks <= 8,
 * ln_eps > 0.
 */
size_t medusa_heads_ex_workspace(int B, int hidden, long vocab, int K, int n_blocks, int layernorm,
                                 int topk);
int medusa_heads_ex(const void* h, const void* w1, const void* b1, const void* ln_gamma,
                    const void* ln_beta, float ln_eps, const void* w2, int dtype, int packed,
                    int B, int hidden, long vocab, int K, int n_blocks, int topk, float* logits,
                    int32_t* topk_ids, float* topk_logits, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Bytes of the packed form of K bf16 matrices of [rows, hidden] (0 on invalid sizes;
   limits as medusa_pack_weights). */
size_t medusa_packed_weight_bytes(int K, long rows, int hidden);

/*
 * Packs w (device, [K, rows, hidden] bf16, [out, in]) into `packed` (device,
 * medusa_packed_weight_bytes(K, rows, hidden) bytes).  The rows of all heads are cut into 16-row
 * tiles, numbered gt = k * ntiles + tile (G = K * ntiles, ntiles = ceil(rows / 16)).  The 64
 * lanes' 16-byte operands of tile gt for 32-column block kb form one 1 KB block, rows past
 * `rows` zero-filled:
 *   block(gt, kb)[lane][e] = w[k][16 tile + lane % 16][32 kb + 8 (lane / 16) + e],
 * kb < hidden / 32, lane < 64, e < 8.  The tiles are grouped gs at a time, with
 * rounds = ceil(G / 2048) and gs = 4 ceil(G / (4 rounds)) (the tiles one round of the heads
 * kernel's persistent grid reads); inside group g, of n tiles (gs, or what is left for the
 * last), the blocks are kb-major: block(g gs + w, kb) is 1 KB block number g nkb gs + kb n + w.
 * The heads kernels then read the weights in address order.  Done once per model, outside the
 * decode loop.
 * Limits: 1 <= K <= 64 (K heads, or K * n_blocks stacked block weights for medusa_heads_ex),
 *         1 <= rows < 2^31, hidden a multiple of 32 in 32..16384.
 */
int medusa_pack_weights(const void* w, int K, long rows, int hidden, void* packed, void* stream);

/* ---------------------------------------------------------------------------------------- *
 * 2. The candidate tree
 * ---------------------------------------------------------------------------------------- */

/*
 * A tree given as `medusa_choices` (cnnetsun page, configuration section): n_choices rank
 * tuples, choices[c*max_depth + d] for d < max_depth, padded with -1.  Tuple (r1..rd) is the
 * node made of head 1's rank-r1 candidate, ..., head d's rank-rd candidate, so head d fills
 * depth d; the root (depth 0) is the last accepted token.  The list must be prefix-closed
 * (every proper prefix present), without duplicates, with every rank < topk and depth <= K.
 *
 * Node order: root = 0, then by (depth, rank tuple) ascending, so parent < child.
 * Paths: one per leaf, leaves in ascending rank-tuple order.
 */
typedef struct {
  int T;           /* nodes including the root */
  int W;           /* 64-bit mask words per row: (T + 63) / 64 */
  int n_paths;     /* root-to-leaf paths (leaves) */
  int dmax;        /* tree depth */
  int n_internal;  /* nodes with at least one child (the root included) */
  int max_rank;    /* largest rank in the list: build_tree needs topk > max_rank */
  /* device arrays, filled by build_tree(static_ready = 0) */
  uint64_t* mask;      /* [T][W]: bit j%64 of word j/64 of row i is set iff node j is i or an
                          ancestor of i (Wiblog page, tree-attention section: each token sees
                          only its own prefix path) */
  int32_t* parent;     /* [T], -1 for the root */
  int32_t* depth;      /* [T] */
  int32_t* rank;       /* [T], the node's last rank, -1 for the root */
  int32_t* paths;      /* [n_paths][dmax + 1]: node per depth, -1 padded */
  int32_t* path_len;   /* [n_paths]: depth of the leaf */
  int32_t* child_ptr;  /* [T + 1]: children of i are child_idx[child_ptr[i] .. child_ptr[i+1]) */
  int32_t* child_idx;  /* [T - 1] */
  int32_t* internal;   /* [n_internal]: internal node ids, ascending */
} medusa_tree;

/*
 * Host only.  Validates a choice list and fills T, W, n_paths, dmax, n_internal and max_rank of
 * *tree (its pointers are left untouched).  Returns MEDUSA_ERR_TREE for a malformed list.
 * Limits: 1 <= n_choices, T <= 4096, 1 <= max_depth <= K <= 8, 1 <= topk <= 64.
 */
int medusa_tree_dims(const int32_t* choices, int n_choices, int max_depth, int K, int topk,
                     medusa_tree* tree);

/*
 * The per-step tree tokens and position ids (Wiblog page, tree-attention section: the
 * position encoding follows each token's path):
 *     tokens[b][0] = root_tokens[b]
 *     tokens[b][i] = topk_ids[b][depth(i) - 1][rank(i)]
 *     position_ids[b][i] = prefix_len[b] + depth(i)
 * static_ready == 0: the choice list (host) is validated, the static arrays of *tree are
 *   computed on the host and copied into its device arrays (sized from medusa_tree_dims); the
 *   host waits for that copy.  Do this once per tree; the pages precompute and cache the mask.
 * static_ready == 1: the device arrays are taken as already filled; choices may be NULL.  The
 *   dims in *tree must still fit this call: dmax <= K and max_rank < topk (else
 *   MEDUSA_ERR_TREE), since the gather reads topk_ids[b][depth - 1][rank].
 * Arguments: topk_ids device [B][K][topk]; root_tokens, prefix_len device [B];
 *            tokens, position_ids device [B][T] int32.
 */
int build_tree(const int32_t* choices, int n_choices, int max_depth, int K, int topk,
               const int32_t* topk_ids, const int32_t* root_tokens, const int32_t* prefix_len,
               int B, int static_ready, const medusa_tree* tree, int32_t* tokens,
               int32_t* position_ids, void* stream);

/*
 * medusa_heads (packed = 0) or medusa_heads_packed (packed = 1, bf16) followed by build_tree's
 * per-step gather, in the same launches: the merge that finishes head d - 1's top-k writes the
 * tokens and position ids of the tree's depth-d nodes, and head 0's merge writes the root.  The
 * step's chain heads -> build_tree with one launch fewer (Wiblog page, tree-attention section:
 * head d fills depth d).  Outputs are bit-identical to medusa_heads[_packed] followed by
 * build_tree(static_ready = 1).  The tree's static arrays must already be on the device (one
 * build_tree call with static_ready = 0).  Arguments: as medusa_heads / medusa_heads_packed and
 * build_tree; the workspace is medusa_heads_workspace's.  Errors: theirs, and MEDUSA_ERR_TREE
 * when tree->dmax > K or tree->max_rank >= topk.
 */
int medusa_heads_build_tree(const void* h, const void* w1, const void* b1, const void* w2,
                            int dtype, int packed, int B, int hidden, long vocab, int K, int topk,
                            const medusa_tree* tree, const int32_t* root_tokens,
                            const int32_t* prefix_len, float* logits, int32_t* topk_ids,
                            float* topk_logits, int32_t* tokens, int32_t* position_ids,
                            void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------- *
 * 3. Tree attention
 * ---------------------------------------------------------------------------------------- */

size_t tree_attention_workspace(int B, int Hq, int Hkv, int T, int D, int max_prefix_len);

/*
 * For every sequence b, query head hq and tree node i, with kv head g = hq / (Hq / Hkv):
 *     visible rows j: every prefix row j < prefix_len[b], and row prefix_len[b] + t for every
 *                     node t whose bit is set in mask row i (its ancestors and itself);
 *     out[b,hq,i] = sum_j softmax_j(scale * q[b,hq,i] . k[b,g,j]) v[b,g,j]
 * (Wiblog page, tree-attention section: one pass verifies all candidates; a token attends only
 * to its own prefix path.)  The tree tokens' K/V must already sit at cache rows
 * prefix_len[b] .. prefix_len[b] + T - 1, in node order.  No positional encoding is applied
 * here: q and k arrive as the caller produced them.
 * Arguments (device): q, out [B][Hq][T][D] dtype; k_cache, v_cache [B][Hkv][lcap][D] dtype;
 *   prefix_len [B] int32 with prefix_len[b] <= max_prefix_len and prefix_len[b] + T <= lcap;
 *   mask [T][W] uint64 as in medusa_tree.  scale <= 0 selects 1/sqrt(D).
 * Arithmetic: fp32 scores, softmax and accumulation; bf16 operands enter the matrix cores
 * directly; the output is rounded to dtype (nearest even).
 * Limits: D in {64, 128}, Hq % Hkv == 0, 1 <= T <= 4096, 0 <= max_prefix_len <= 1<<20,
 *         1 <= B <= 4096, Hq <= 256.
 */
int tree_attention(const void* q, const void* k_cache, const void* v_cache, int dtype,
                   const int32_t* prefix_len, int max_prefix_len, long lcap,
                   const uint64_t* mask, int B, int Hq, int Hkv, int T, int D, float scale,
                   void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * tree_attention with the rotary position embedding applied first (Wiblog page, tree-attention
 * section: the position encoding follows the tree so that each token gets its correct position
 * index; the pages do not name the encoding, this is the rotary one of LLaMA-family models).
 * position_ids [B][T] int32 (device; build_tree's, prefix_len + depth).  For every query row
 * (b, hq, i) and every tree key row prefix_len[b] + i of k_cache (all kv heads), dimension
 * j < D/2 and its partner j + D/2 turn by the angle position_ids[b][i] * rope_base^(-2j/D):
 *     (x_j, x_{j+D/2}) -> (x_j cos - x_{j+D/2} sin,  x_j sin + x_{j+D/2} cos),
 * in fp32 with the angle reduced in fp64, rounded to dtype (nearest even).  The rotated keys
 * are written back into k_cache (call once per step: the prefix rows are taken as already
 * rotated) by a first kernel; the queries are rotated inside the attention kernel as they are
 * loaded, and q is left unchanged.  The result is exactly tree_attention on the rotated queries
 * and keys.  Arguments, limits and errors as tree_attention, plus rope_base > 1 (10000 for
 * LLaMA-family models).  The workspace (size from tree_attention_rope_workspace, always > 0)
 * holds every node's cos/sin ([B*T][2][D/2] floats, rounded up to 256 bytes) followed by
 * tree_attention's own workspace.
 */
size_t tree_attention_rope_workspace(int B, int Hq, int Hkv, int T, int D, int max_prefix_len);
int tree_attention_rope(const void* q, void* k_cache, const void* v_cache, int dtype,
                        const int32_t* prefix_len, int max_prefix_len, long lcap,
                        const uint64_t* mask, const int32_t* position_ids, float rope_base,
                        int B, int Hq, int Hkv, int T, int D, float scale, void* out,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------- *
 * 4. Typical acceptance
 * ---------------------------------------------------------------------------------------- */

size_t typical_accept_workspace(int B, int T, long vocab, int n_internal);

/*
 * logits [B][T][vocab] dtype (device): row n is the model's next-token distribution after tree
 * node n, so child c of node n is judged by row n.  tokens [B][T] int32 (device) from
 * build_tree.  For temperature > 0, per internal row n:
 *     z = logits / temperature, p = softmax(z), H = -sum p ln p,
 *     thr = min(posterior_threshold, posterior_alpha * exp(-H)),
 *     child c accepted iff p(tokens[c]) > thr      (decided in fp32, in the log domain);
 * for temperature == 0: child c accepted iff tokens[c] is the row's argmax (lowest id on ties).
 * The root token is the greedy first token and is always kept.  Along each path the accept
 * count is the number of accepted nodes below the root before the first rejection;
 *     accept_length[b]  = the largest count,  best_candidate[b] = the lowest path index with it,
 *     next_token[b]     = argmax of the row of the last accepted node of that path (NULL skips
 *                         it), i.e. the greedy token that starts the next step.
 * Leaf rows are read only for next_token.  Outputs are device int32 [B].
 * Limits: temperature >= 0; 0 < posterior_threshold < 1; posterior_alpha > 0; vocab < 2^31.
 */
int typical_accept(const void* logits, int dtype, int B, int T, long vocab,
                   const int32_t* tokens, const medusa_tree* tree, float temperature,
                   float posterior_threshold, float posterior_alpha, int32_t* best_candidate,
                   int32_t* accept_length, int32_t* next_token, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * The candidate-filtering call as the cnnetsun page writes it (candidate-filtering section):
 *     evaluate_posterior(logits, candidates, temperature, posterior_threshold, posterior_alpha,
 *                        top_p, sampling, fast) -> (best_candidate, accept_length).
 * The page names top_p, sampling and fast and defines none of them; they are read as follows.
 *   sampling  which test a candidate passes at temperature > 0:
 *     MEDUSA_SAMPLING_TYPICAL  the typical-acceptance test of typical_accept (top_p unused);
 *                              with it this call is exactly typical_accept;
 *     MEDUSA_SAMPLING_NUCLEUS  child c of node n is accepted iff it lies in the top_p nucleus of
 *                              p = softmax(logits[b][n] / temperature): the probability mass of
 *                              the tokens whose logit is strictly larger than tokens[b][c]'s is
 *                              below top_p (tokens tied with it are not counted, so tied tokens
 *                              are in or out together).  Decided in fp32 from a single pass over
 *                              the row (sums of 2^(y - max) in a fixed order).
 *   At temperature 0 both modes are greedy (Wiblog page, typical-acceptance section).
 *   top_p     0 < top_p <= 1 (1: every candidate with a finite logit is in the nucleus).
 *   fast      0 or 1: a faster evaluation of the same rule.  This library has one evaluation,
 *             the single pass over each internal row, so the results do not depend on it.
 * Everything else (arguments, outputs, the path scan, next_token, errors) as typical_accept.
 * The workspace query takes the tree's dims (T, n_internal) and the mode; the nucleus mode
 * keeps 64 per-child partial sums for every chunk of every internal row on top of
 * typical_accept's workspace.  Errors: MEDUSA_ERR_ARG for a sampling, fast or top_p outside
 * the values above.
 */
typedef enum { MEDUSA_SAMPLING_TYPICAL = 0, MEDUSA_SAMPLING_NUCLEUS = 1 } medusa_sampling;
size_t evaluate_posterior_workspace(int B, long vocab, const medusa_tree* tree, int sampling);
int evaluate_posterior(const void* logits, int dtype, int B, int T, long vocab,
                       const int32_t* tokens, const medusa_tree* tree, float temperature,
                       float posterior_threshold, float posterior_alpha, float top_p,
                       int sampling, int fast, int32_t* best_candidate, int32_t* accept_length,
                       int32_t* next_token, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * typical_accept for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation, arguments and
 * results, without the workspace.  The intermediates go to a scratch array that the library
 * holds in device memory, one copy of MEDUSA_NOALLOC_SCRATCH_BYTES per GPU it runs on, kept
 * until the process ends.  The call allocates nothing and frees nothing; the first call on a
 * device looks up that device's copy (hipGetSymbolAddress).  Every call on one GPU shares its
 * copy: calls that overlap in time on one GPU (on different streams, or from different host
 * threads) race and must be serialised by the caller.  The scratch needs no clearing: each call
 * writes every intermediate before reading it.
 * Errors: those of typical_accept, and MEDUSA_ERR_WORKSPACE when typical_accept_workspace(B, T,
 * vocab, tree->n_internal) exceeds MEDUSA_NOALLOC_SCRATCH_BYTES (8 MiB holds, for example,
 * B = 64 sequences of a 1111-node tree with 111 internal rows at vocab 128256).
 */
#define MEDUSA_NOALLOC_SCRATCH_BYTES (8 << 20)
int typical_accept_noalloc(const void* logits, int dtype, int B, int T, long vocab,
                           const int32_t* tokens, const medusa_tree* tree, float temperature,
                           float posterior_threshold, float posterior_alpha,
                           int32_t* best_candidate, int32_t* accept_length, int32_t* next_token,
                           void* stream);

/* ---------------------------------------------------------------------------------------- *
 * 5. Commit of the accepted candidate (decode-loop glue)
 * ---------------------------------------------------------------------------------------- */

/*
 * After typical_accept: emits the accepted tokens, compacts their K/V in the cache and hands
 * over what the next step starts from (Wiblog page, inference-flow section: the accepted prefix
 * is output and the next round starts from the last accepted token; the verification logits
 * already give that round's first token).  For each sequence b, with p = best_candidate[b],
 * a = accept_length[b], L = prefix_len[b] and path = tree->paths[p] (node per depth):
 *   out_tokens[b][k]  = tokens[b][path[k]] for k <= a, -1 for a < k <= dmax    [B][dmax + 1]
 *   out_count[b]      = a + 1
 *   k_cache, v_cache  row L + k of every kv head <- row L + path[k], k = 1 .. a, in place (the
 *                     root already sits at row L); no other row changes
 *   new_prefix_len[b] = L + a + 1              (may be the same array as prefix_len)
 *   new_root[b]       = next_token[b]          (nullable: skipped)
 *   next_hidden[b][:] = hidden[b][path[a]][:]  (hidden [B][T][hidden_size] and next_hidden
 *                                               [B][hidden_size] in dtype; both NULL skips it)
 * A sequence whose p, a or L is out of range (p >= n_paths, a > path_len[p], L < 0 or
 * L + T > lcap) is left untouched and gets out_count[b] = 0, new_prefix_len[b] = L.
 * All pointers are device memory; tokens must not overlap out_tokens.
 * Limits: dtype F32 or BF16; D * element size and hidden_size * element size multiples of 16;
 *         1 <= B <= 65535, 1 <= Hkv <= 256.
 */
int commit_accepted(const medusa_tree* tree, int B, const int32_t* best_candidate,
                    const int32_t* accept_length, const int32_t* tokens,
                    const int32_t* next_token, void* k_cache, void* v_cache, int dtype, int Hkv,
                    long lcap, int D, const int32_t* prefix_len, int32_t* new_prefix_len,
                    int32_t* out_tokens, int32_t* out_count, int32_t* new_root,
                    const void* hidden, int hidden_size, void* next_hidden, void* stream);

/* ---------------------------------------------------------------------------------------- *
 * 6. Sparse candidate tree (host)
 * ---------------------------------------------------------------------------------------- */

/*
 * The N-node choice list of largest expected accept length (Ultralytics page, tree-attention
 * section: a sparse tree of the most accurate combinations beats a dense one several times its
 * size; Wiblog page, heads section: per-head top-1 / top-5 accuracy).  accuracy [K][topk] (host
 * fp64, each in [0, 1]): probability that head k's rank-r candidate is the right token, taken
 * independent across heads.  Then E[accept length] = sum over nodes of prod_k accuracy[k][r_k]
 * and the best tree is the N most likely nodes, ties broken by depth and then rank tuple
 * (node probabilities are products in depth order, fp64).  choices [N][K] (host int32) receives
 * the rank tuples in node order (depth, then rank tuple), -1 padded: a medusa_choices list for
 * build_tree with max_depth = K.  *expected_accept_length (nullable) receives the expectation,
 * summed in node order.  Host only; no device work.
 * Limits: 1 <= K <= 8, 1 <= topk <= 64, 1 <= N <= min(4095, nodes of the full tree).
 */
int medusa_sparse_tree(const double* accuracy, int K, int topk, int N, int32_t* choices,
                       double* expected_accept_length);

/* ---------------------------------------------------------------------------------------- *
 * Measurement hook (not part of the method)
 * ---------------------------------------------------------------------------------------- */

/* The kernels the entry points launch, for per-kernel timing. */
typedef enum {
  MEDUSA_KERNEL_HEADS_W1 = 0,      /* medusa_heads: first layer, r = h + SiLU(W1 h + b1)   */
  MEDUSA_KERNEL_HEADS_W2 = 1,      /* medusa_heads: vocab projection, logits = W2 r        */
  MEDUSA_KERNEL_TOPK = 2,          /* medusa_heads: per-head top-k                         */
  MEDUSA_KERNEL_TREE_GATHER = 3,   /* build_tree: tokens and position ids                  */
  MEDUSA_KERNEL_ATTENTION = 4,     /* tree_attention: main kernel                          */
  MEDUSA_KERNEL_ATTN_COMBINE = 5,  /* tree_attention: merge of K/V splits (when split)     */
  MEDUSA_KERNEL_ACCEPT = 6,        /* typical_accept: its three launches (row statistics,
                                      decisions, path scan and next token)                 */
  MEDUSA_KERNEL_COMMIT = 7,        /* commit_accepted                                      */
  MEDUSA_KERNEL_ROPE = 8,          /* tree_attention_rope: the rotation before attention   */
  MEDUSA_KERNEL_COUNT = 9
} medusa_kernel;

/*
 * While set, every launch of kernel `which` made by the calling thread records the HIP event
 * `before` (a hipEvent_t) on the call's stream just before the launch and `after` just after
 * it, so hipEventElapsedTime(before, after) is that launch's duration.  NULL for both clears
 * the hook.  The events are owned by the caller and must outlive their use.
 * Returns MEDUSA_ERR_ARG for an unknown kernel id or a single NULL event.
 */
int medusa_set_kernel_events(int which, void* before, void* after);

/*
 * Streaming-read ceiling (measurement only): reads `bytes` bytes at `buf` (device, 16-byte
 * aligned, bytes a positive multiple of 16) once, with 16-byte nontemporal loads in a grid-stride
 * sweep, and writes nothing except possibly sink[0] (device uint32, content unspecified).  Its
 * duration over a buffer much larger than the caches gives the read bandwidth that one plain
 * kernel reaches, the measured ceiling beside the published HBM peak.
 * Returns MEDUSA_ERR_ARG (null or misaligned pointer) or MEDUSA_ERR_SHAPE (bad size).
 */
int medusa_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MEDUSA_H */
