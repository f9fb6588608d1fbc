// Typical acceptance over the verification logits, then the longest accepted prefix.
//
// Wiblog "Medusa multi-head speculative decoding", typical-acceptance section: a candidate is
// accepted when its probability under the original model exceeds the minimum of a hard
// threshold and an entropy-dependent one; the first token is taken greedily; temperature 0 is
// greedy decoding.  Inference-flow section: walk from the root until the first rejection or a
// leaf.  cnnetsun page: posterior_threshold (eps) and posterior_alpha (delta), returning
// (best_candidate, accept_length).  Written out: p = softmax(l / T), H = -sum p ln p,
// accept iff p(x) > min(eps, delta * exp(-H)).
//
// Only internal rows are read (a leaf's row judges no child).  Three launches, none of whose
// work-groups waits for another (on this GPU a release fence per work-group serialises, so each
// handoff is a kernel boundary):
//   accept_chunks  one work-group per (sequence, internal row, chunk) computes in a single pass
//                  the chunk's max y, S = sum 2^(y - max) and A = sum (y - max) 2^(y - max) with
//                  y = l * log2(e) / T, plus the argmax (a chunk is 1, 2 or 4 rounds of 8
//                  elements per thread, see accept_unroll);
//   accept_rows    one work-group per (sequence, internal row) merges the row's partials in chunk
//                  order, so H = ln2 * (log2 S - A / S) and ln p(x) = ln2 * (y_x - max - log2 S),
//                  and decides the row's children in the log domain;
//   accept_paths   one work-group per sequence scans the paths for the longest accepted prefix
//                  and finds the next token.
#include <math.h>
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace medusa {

constexpr int kAccThreads = 256;
constexpr int kAccPerThread = 8;
constexpr int kAccVec = kAccThreads * kAccPerThread;    // elements per load round of a work-group
constexpr long kPathWideBytes = 32 << 10;   // leaf rows above this size get a 1024-thread block
constexpr int kMaxTreeTokens = 4096;
// Rounds of kAccVec elements per work-group of accept_chunks: the larger U of 4, 2 that still
// leaves at least 1024 work-groups (2048 when there are more than 256 rows), else 1; 8 rounds
// was never the fastest (70B-layer rows: 58.0 against 54.5 us for 4, three runs each).  Fitted to
// timings on MI355X once every round's loads were in flight together (event-timed acceptance,
// U = 1 / 2 / 4 / 8): 7B rows (32) 14.2 / 14.6 / 15.7 / 18.6 us; Llama-8B rows (37 of 128256)
// 18.5 / 17.0 / 17.6 / 19.7; 33B rows (352 of 32000) 30.2 / 27.4 / 28.5 / 29.3; 70B-layer rows
// (444 of 128256) 75 / 56.6 / 54.4 / 57.6.  MEDUSA_ACCEPT_UNROLL = 1, 2 or 4 overrides it.
static int accept_unroll(int B, long V, int n_int) {
  static const int forced = [] { const char* v = getenv("MEDUSA_ACCEPT_UNROLL"); return v ? atoi(v) : 0; }();
  if (forced == 1 || forced == 2 || forced == 4) return forced;
  const long rows = static_cast<long>(n_int) * B;
  const long target = rows <= 256 ? 1024 : 2048;
  for (int u = 4; u >= 2; u >>= 1) {
    const long C = (V + static_cast<long>(kAccVec) * u - 1) / (static_cast<long>(kAccVec) * u);
    if (C * rows >= target) return u;
  }
  return 1;
}

struct RowStat {   // partial softmax statistics of a set of elements (log2 units)
  float m, S, A, pad;
};

__device__ __forceinline__ RowStat stat_merge(RowStat a, RowStat b) {
  if (a.S == 0.f) return b;
  if (b.S == 0.f) return a;
  const float m = fmaxf(a.m, b.m);
  const float fa = exp2f(a.m - m), fb = exp2f(b.m - m);
  RowStat r;
  r.m = m;
  r.S = a.S * fa + b.S * fb;
  r.A = (a.A + (a.m - m) * a.S) * fa + (b.A + (b.m - m) * b.S) * fb;
  r.pad = 0.f;
  return r;
}

__device__ __forceinline__ RowStat shfl_down_stat(RowStat s, int off) {
  RowStat r;
  r.m = __shfl_down(s.m, off);
  r.S = __shfl_down(s.S, off);
  r.A = __shfl_down(s.A, off);
  r.pad = 0.f;
  return r;
}

__device__ __forceinline__ uint64_t shfl_down_u64(uint64_t v, int off) {
  uint32_t lo = __shfl_down(static_cast<uint32_t>(v), off);
  uint32_t hi = __shfl_down(static_cast<uint32_t>(v >> 32), off);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Loads 8 logits starting at element idx0 of a row (fp32 out); invalid -> valid[e] = false.
__device__ __forceinline__ void load8(const void* row, int dtype, long idx0, long V, float* x,
                                      bool* valid) {
  if (dtype == 1) {
    const uint16_t* p = static_cast<const uint16_t*>(row);
    if (idx0 + 8 <= V && (reinterpret_cast<uintptr_t>(p + idx0) & 15) == 0) {
      const uint4 v = *reinterpret_cast<const uint4*>(p + idx0);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] = bf16_to_f32(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1))));
        valid[e] = true;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        valid[e] = idx0 + e < V;
        x[e] = valid[e] ? bf16_to_f32(p[idx0 + e]) : 0.f;
      }
    }
  } else {
    const float* p = static_cast<const float*>(row);
    if (idx0 + 8 <= V && (reinterpret_cast<uintptr_t>(p + idx0) & 15) == 0) {
      const float4 a = *reinterpret_cast<const float4*>(p + idx0);
      const float4 b = *reinterpret_cast<const float4*>(p + idx0 + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
#pragma unroll
      for (int e = 0; e < 8; ++e) valid[e] = true;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        valid[e] = idx0 + e < V;
        x[e] = valid[e] ? p[idx0 + e] : 0.f;
      }
    }
  }
}

// Vector loads (used when V % 8 == 0 and the logits are 16-byte aligned, so the 8 elements a
// thread takes in a round are either all in the row or all past it).  A round past the row
// loads the row's first 8 elements instead, an address that is always valid, and is marked
// invalid, so no branch surrounds a load: all of a thread's rounds are in flight before the
// first is converted.  (The branchy load8 above makes each round wait for the previous one.)
// LOAD: 1 = bf16, 2 = fp32.
template <int LOAD>
__device__ __forceinline__ void load_vec8(const void* row, long idx0, long V, uint32_t (&w)[8],
                                          bool& in) {
  in = idx0 < V;
  const long i = in ? idx0 : 0;
  if constexpr (LOAD == 1) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row) + i);
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    w[4] = w[5] = w[6] = w[7] = 0u;
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const float*>(row) + i);
    const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const float*>(row) + i + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
}
template <int LOAD>
__device__ __forceinline__ void unpack_vec8(const uint32_t (&w)[8], bool in, float* x, bool* valid) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    valid[e] = in;
    x[e] = LOAD == 1 ? bf16_to_f32(static_cast<uint16_t>(w[e >> 1] >> (16 * (e & 1)))) : __uint_as_float(w[e]);
  }
}
// U rounds of 8 elements at idx0, idx0 + step, ...: LOAD 0 = the general per-round form
template <int LOAD, int U>
__device__ __forceinline__ void load_rounds(const void* row, int dtype, long idx0, long step, long V,
                                            float (&x)[U][8], bool (&valid)[U][8]) {
  if constexpr (LOAD == 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) load8(row, dtype, idx0 + u * step, V, x[u], valid[u]);
  } else {
    uint32_t w[U][8];
    bool in[U];
#pragma unroll
    for (int u = 0; u < U; ++u) load_vec8<LOAD>(row, idx0 + u * step, V, w[u], in[u]);
#pragma unroll
    for (int u = 0; u < U; ++u) unpack_vec8<LOAD>(w[u], in[u], x[u], valid[u]);
  }
}

struct AcceptArgs {
  const void* logits;
  int dtype, B, T;
  long V;
  const int32_t* tokens;
  int n_int;
  const int32_t* internal;
  const int32_t* child_ptr;
  const int32_t* child_idx;
  const int32_t* paths;
  const int32_t* path_len;
  int n_paths, dmax;
  int greedy;
  float y_scale;      // log2(e) / temperature
  float ln_eps, ln_delta;
  int C;
  int nucleus;            // nucleus test in place of the typical one (temperature > 0)
  float top_p;
  int maxc;               // children per node at most (nucleus mode)
  RowStat* part_stat;     // [B][n_int][C]
  uint64_t* part_arg;     // [B][n_int][C]
  float* part_mass;       // [B][n_int][C][maxc] masses above each child (nucleus mode)
  int32_t* dec;           // [B][T]
  int32_t* rowarg;        // [B][T]
  int32_t* best;
  int32_t* accept_len;
  int32_t* next_token;    // nullable
};

// Block-wide merge of (statistics, argmax key) in a fixed order: lanes toward lane 0 of each wave,
// then the waves in order.  The result is valid in thread 0.
__device__ __forceinline__ void block_merge(RowStat& st, uint64_t& arg, bool greedy, RowStat* s_stat,
                                            uint64_t* s_arg) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = shfl_down_u64(arg, off);
    arg = o > arg ? o : arg;
    if (!greedy) st = stat_merge(st, shfl_down_stat(st, off));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_stat[w] = st;
    s_arg[w] = arg;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kAccThreads / 64; ++i) {
      st = stat_merge(st, s_stat[i]);
      arg = s_arg[i] > arg ? s_arg[i] : arg;
    }
  }
}

// Kernel 1, grid (C, n_int, B): statistics and argmax of one chunk (U rounds of 2048 elements)
// of an internal row, written to the partial arrays.  All U rounds of loads are issued before
// any is used.
template <int U, int LOAD>
__global__ __launch_bounds__(kAccThreads) void accept_chunks(AcceptArgs a) {
  __shared__ RowStat s_stat[kAccThreads / 64];
  __shared__ uint64_t s_arg[kAccThreads / 64];
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int n = a.internal[r];
  const int esz = a.dtype == 1 ? 2 : 4;
  const char* row = static_cast<const char*>(a.logits) + (static_cast<long>(b) * a.T + n) * a.V * esz;
  const long base = static_cast<long>(c) * kAccVec * U + static_cast<long>(threadIdx.x) * kAccPerThread;
  float x[U][kAccPerThread];
  bool valid[U][kAccPerThread];
  load_rounds<LOAD, U>(row, a.dtype, base, kAccVec, a.V, x, valid);
  uint64_t arg = 0;
  RowStat st{-INFINITY, 0.f, 0.f, 0.f};
  if ((c + 1) * static_cast<long>(kAccVec) * U <= a.V) {
    // every element of the chunk is in the row (all chunks but a ragged last one): the argmax as
    // a float compare in index order (the first maximum wins; -0 == +0), the row statistics from
    // its value, with the hardware exp2.  A -inf logit contributes nothing: its exponent is
    // clamped to -256, where v_exp_f32 returns 0.
    float best = -INFINITY;
    int bpos = 0;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < kAccPerThread; ++e)
        if (x[u][e] > best) {
          best = x[u][e];
          bpos = u * kAccPerThread + e;
        }
    // (a thread whose elements are all -inf keeps its first one, like any tie)
    arg = sel_key(best, static_cast<uint32_t>(base + (bpos / kAccPerThread) * kAccVec + bpos % kAccPerThread));
    if (!a.greedy && best > -INFINITY) {
      const float m = best * a.y_scale;
      float S = 0.f, A = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kAccPerThread; ++e) {
          const float d = fmaxf(fmaf(x[u][e], a.y_scale, -m), -256.f);
          const float p = __builtin_amdgcn_exp2f(d);
          S += p;
          A = fmaf(d, p, A);
        }
      st = RowStat{m, S, A, 0.f};
    }
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < kAccPerThread; ++e)
        if (valid[u][e]) {
          const uint64_t k = sel_key(x[u][e], static_cast<uint32_t>(base + u * kAccVec + e));
          arg = k > arg ? k : arg;
        }
    if (!a.greedy) {
      float m = -INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < kAccPerThread; ++e)
          if (valid[u][e]) m = fmaxf(m, x[u][e] * a.y_scale);
      if (m > -INFINITY) {
        float S = 0.f, A = 0.f;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int e = 0; e < kAccPerThread; ++e) {
            if (!valid[u][e]) continue;
            const float d = fmaxf(fmaf(x[u][e], a.y_scale, -m), -256.f);
            const float p = __builtin_amdgcn_exp2f(d);
            S += p;
            A = fmaf(d, p, A);
          }
        st = RowStat{m, S, A, 0.f};
      }
    }
  }
  block_merge(st, arg, a.greedy, s_stat, s_arg);
  if (threadIdx.x == 0) {
    const long pidx = (static_cast<long>(b) * a.n_int + r) * a.C + c;
    a.part_stat[pidx] = st;
    a.part_arg[pidx] = arg;
  }
}

// Kernel 1 of the nucleus mode (temperature > 0), grid (C, n_int, B): the chunk's statistics and
// argmax as accept_chunks, and for every child j of the row the chunk's sum of 2^(y - m) over
// the elements whose logit is strictly larger than the child's own: the probability mass above
// the child, in the units of S.  Every thread takes the block's largest logit as m, so all the
// per-thread sums share one reference and add without rescaling.
constexpr int kNucGroup = 16;   // children summed per pass (a node has at most 64)
template <int U, int LOAD>
__global__ __launch_bounds__(kAccThreads) void accept_chunks_nucleus(AcceptArgs a) {
  __shared__ RowStat s_stat[kAccThreads / 64];
  __shared__ uint64_t s_arg[kAccThreads / 64];
  __shared__ float s_cl[64];
  __shared__ float s_max[kAccThreads / 64];
  __shared__ float s_mass[kAccThreads / 64][kNucGroup];
  const int c = blockIdx.x, r = blockIdx.y, b = blockIdx.z;
  const int n = a.internal[r];
  const int esz = a.dtype == 1 ? 2 : 4;
  const char* row = static_cast<const char*>(a.logits) + (static_cast<long>(b) * a.T + n) * a.V * esz;
  const long base = static_cast<long>(c) * kAccVec * U + static_cast<long>(threadIdx.x) * kAccPerThread;
  float x[U][kAccPerThread];
  bool valid[U][kAccPerThread];
  load_rounds<LOAD, U>(row, a.dtype, base, kAccVec, a.V, x, valid);
  // the children's own logits (+inf for a token outside the vocab: nothing lies above it, and
  // the decision rejects such a child anyway)
  // (siblings carry distinct ranks below topk <= 64, so a valid tree never reaches the clamp)
  const int c0 = a.child_ptr[n], nchild = min(min(a.child_ptr[n + 1] - c0, a.maxc), 64);
  if (static_cast<int>(threadIdx.x) < nchild) {
    const int tok = a.tokens[static_cast<long>(b) * a.T + a.child_idx[c0 + threadIdx.x]];
    s_cl[threadIdx.x] = tok < 0 || tok >= a.V ? INFINITY
                        : a.dtype == 1 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[tok])
                                       : reinterpret_cast<const float*>(row)[tok];
  }
  uint64_t arg = 0;
  float tmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int e = 0; e < kAccPerThread; ++e)
      if (valid[u][e]) {
        const uint64_t k = sel_key(x[u][e], static_cast<uint32_t>(base + u * kAccVec + e));
        arg = k > arg ? k : arg;
        tmax = fmaxf(tmax, x[u][e]);
      }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = tmax;
  __syncthreads();                                     // also publishes s_cl
  const float xb = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  RowStat st{-INFINITY, 0.f, 0.f, 0.f};
  float p[U][kAccPerThread];
  const float m = xb > -INFINITY ? xb * a.y_scale : 0.f;
  {
    float S = 0.f, A = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < kAccPerThread; ++e) {
        const float d = fmaxf(fmaf(x[u][e], a.y_scale, -m), -256.f);
        p[u][e] = valid[u][e] && xb > -INFINITY ? __builtin_amdgcn_exp2f(d) : 0.f;
        S += p[u][e];
        A = fmaf(d, p[u][e], A);
      }
    if (xb > -INFINITY) st = RowStat{m, S, A, 0.f};
  }
  const long pidx = (static_cast<long>(b) * a.n_int + r) * a.C + c;
  const int w = threadIdx.x >> 6;
  for (int g0 = 0; g0 < nchild; g0 += kNucGroup) {
    float cl[kNucGroup], acc[kNucGroup];
#pragma unroll
    for (int j = 0; j < kNucGroup; ++j) {
      cl[j] = g0 + j < nchild ? s_cl[g0 + j] : INFINITY;
      acc[j] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < kAccPerThread; ++e)
#pragma unroll
        for (int j = 0; j < kNucGroup; ++j) acc[j] += x[u][e] > cl[j] ? p[u][e] : 0.f;
#pragma unroll
    for (int j = 0; j < kNucGroup; ++j) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc[j] += __shfl_xor(acc[j], off);
    }
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int j = 0; j < kNucGroup; ++j) s_mass[w][j] = acc[j];
    }
    __syncthreads();
    const int j = threadIdx.x;
    if (j < kNucGroup && g0 + j < nchild)
      a.part_mass[pidx * a.maxc + g0 + j] = (s_mass[0][j] + s_mass[1][j]) + (s_mass[2][j] + s_mass[3][j]);
    __syncthreads();
  }
  block_merge(st, arg, false, s_stat, s_arg);
  if (threadIdx.x == 0) {
    a.part_stat[pidx] = st;
    a.part_arg[pidx] = arg;
  }
}

// argmax (lowest index on ties) of one row by a block of NT threads, UR rounds of 8 elements
// per thread in flight.  Each thread keeps its best value and index with float compares in
// increasing index order (the first maximum wins; -0 == +0) and keys them once at the end; a
// thread with no element of the row contributes key 0.
template <int NT, int UR, int LOAD>
__device__ __forceinline__ uint64_t block_row_argmax(const void* row, int dtype, long V,
                                                     uint64_t* scratch) {
  constexpr long kStep = static_cast<long>(NT) * kAccPerThread;
  float best = -INFINITY;
  long bidx = -1;
  for (long j0 = static_cast<long>(threadIdx.x) * kAccPerThread; j0 < V; j0 += UR * kStep) {
    float x[UR][kAccPerThread];
    bool valid[UR][kAccPerThread];
    load_rounds<LOAD, UR>(row, dtype, j0, kStep, V, x, valid);
    if (bidx < 0) {                                   // this thread's first element (j0 < V)
      best = x[0][0];
      bidx = j0;
    }
    int bpos = -1;                                    // best position in this sweep, if any
    if (j0 + (UR - 1) * kStep + kAccPerThread <= V) {
#pragma unroll
      for (int u = 0; u < UR; ++u)
#pragma unroll
        for (int e = 0; e < kAccPerThread; ++e)
          if (x[u][e] > best) {
            best = x[u][e];
            bpos = u * kAccPerThread + e;
          }
    } else {
#pragma unroll
      for (int u = 0; u < UR; ++u)
#pragma unroll
        for (int e = 0; e < kAccPerThread; ++e)
          if (valid[u][e] && x[u][e] > best) {
            best = x[u][e];
            bpos = u * kAccPerThread + e;
          }
    }
    if (bpos >= 0) bidx = j0 + (bpos / kAccPerThread) * kStep + bpos % kAccPerThread;
  }
  const uint64_t arg = bidx < 0 ? 0ull : sel_key(best, static_cast<uint32_t>(bidx));
  return block_max_u64<NT>(arg, scratch);
}

// Kernel 2, grid (n_int, B): merges one row's C partials in chunk order (fixed tree), then
// decides the row's children (at most 64).  The children's tokens and logits are fetched while
// the partials load.
__global__ __launch_bounds__(kAccThreads) void accept_rows(AcceptArgs a) {
  __shared__ RowStat s_stat[kAccThreads / 64];
  __shared__ uint64_t s_arg[kAccThreads / 64];
  __shared__ RowStat s_row;
  __shared__ uint64_t s_rowarg;
  const int r = blockIdx.x, b = blockIdx.y;
  const int n = a.internal[r];
  const int esz = a.dtype == 1 ? 2 : 4;
  const char* row = static_cast<const char*>(a.logits) + (static_cast<long>(b) * a.T + n) * a.V * esz;
  const int c0 = a.child_ptr[n], nchild = a.child_ptr[n + 1] - c0;
  int child = -1, tok = -1;
  float ltok = 0.f;
  if (threadIdx.x < nchild) {
    child = a.child_idx[c0 + threadIdx.x];
    tok = a.tokens[static_cast<long>(b) * a.T + child];
    if (tok >= 0 && tok < a.V)
      ltok = a.dtype == 1 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[tok])
                          : reinterpret_cast<const float*>(row)[tok];
  }
  const long prow = (static_cast<long>(b) * a.n_int + r) * a.C;
  RowStat st{-INFINITY, 0.f, 0.f, 0.f};
  uint64_t arg = 0;
  for (int i = threadIdx.x; i < a.C; i += kAccThreads) {   // thread t merges t, t+256, ...
    st = stat_merge(st, a.part_stat[prow + i]);
    const uint64_t g = a.part_arg[prow + i];
    arg = g > arg ? g : arg;
  }
  block_merge(st, arg, a.greedy, s_stat, s_arg);
  if (threadIdx.x == 0) {
    s_row = st;
    s_rowarg = arg;
    a.rowarg[static_cast<long>(b) * a.T + n] = static_cast<int32_t>(sel_key_index(arg));
  }
  __syncthreads();
  if (threadIdx.x < nchild) {
    int acc;
    if (tok < 0 || tok >= a.V) {
      acc = 0;                               // not a vocab id: never accepted, never read
    } else if (a.greedy) {
      acc = static_cast<uint32_t>(tok) == sel_key_index(s_rowarg);
    } else if (a.nucleus && static_cast<int>(threadIdx.x) >= a.maxc) {
      acc = 0;                               // more children than a valid tree has (see above)
    } else if (a.nucleus) {
      // the mass strictly above the child, merged over the chunks in chunk order, against
      // top_p of the row's total (both in the units of 2^(y - row max))
      float mass = 0.f;
      for (int i = 0; i < a.C; ++i) {
        const RowStat ps = a.part_stat[prow + i];
        if (ps.S > 0.f) mass += a.part_mass[(prow + i) * a.maxc + threadIdx.x] * exp2f(ps.m - s_row.m);
      }
      acc = mass < a.top_p * s_row.S;
    } else {
      const float log2S = log2f(s_row.S);
      const float ln2 = 0.69314718055994531f;
      const float lnp = ln2 * (ltok * a.y_scale - s_row.m - log2S);
      const float H = ln2 * (log2S - s_row.A / s_row.S);
      const float lnthr = fminf(a.ln_eps, a.ln_delta - H);
      acc = lnp > lnthr;
    }
    a.dec[static_cast<long>(b) * a.T + child] = acc;
  }
}

// Kernel 3, grid (B): the longest accepted prefix over the paths, and the next token.  When the
// last accepted node is a leaf, its row's argmax is read here by the whole block with 8 rounds
// of loads in flight per thread (NT = 1024 for rows above 32 KB: 128 KB at a time; else 256).
template <int NT, int LOAD>
__global__ __launch_bounds__(NT) void accept_paths(AcceptArgs a) {
  constexpr int kPathThreads = NT;
  constexpr int kPathRegs = 8;                        // path nodes held in registers
  __shared__ uint64_t s_scratch[kPathThreads / 64];
  __shared__ int32_t s_dec[kMaxTreeTokens];
  __shared__ uint8_t s_leaf[kMaxTreeTokens];
  __shared__ int32_t s_last;
  const int b = blockIdx.x;
  // every static load goes out before anything waits: this thread's path (nodes after the root,
  // the first kPathRegs of them; trees are at most 8 deep) and length, the decisions, and which
  // nodes are leaves
  int pn[kPathRegs];
  int plen = 0, loaded = -1;
  auto load_path = [&](int p) {
    const int32_t* path = a.paths + static_cast<long>(p) * (a.dmax + 1);
    plen = a.path_len[p];
#pragma unroll
    for (int j = 0; j < kPathRegs; ++j) pn[j] = path[min(j + 1, a.dmax)];
    loaded = p;
  };
  if (static_cast<int>(threadIdx.x) < a.n_paths) load_path(threadIdx.x);
  for (int i = threadIdx.x; i < a.T; i += kPathThreads) {
    s_dec[i] = i == 0 ? 1 : a.dec[static_cast<long>(b) * a.T + i];
    s_leaf[i] = a.child_ptr[i + 1] == a.child_ptr[i];
  }
  __syncthreads();
  uint64_t bestk = 0;
  for (int p = threadIdx.x; p < a.n_paths; p += kPathThreads) {
    if (p != loaded) load_path(p);
    int k = 0;
    bool go = true;
#pragma unroll
    for (int j = 0; j < kPathRegs; ++j) {
      if (go && j < plen && s_dec[pn[j]]) ++k;
      else go = false;
    }
    if (go && plen > kPathRegs) {                     // deeper than the registers hold
      const int32_t* path = a.paths + static_cast<long>(p) * (a.dmax + 1);
      while (k < plen && s_dec[path[k + 1]]) ++k;
    }
    const uint64_t key = (static_cast<uint64_t>(k) << 32) | (0xffffffffu - static_cast<uint32_t>(p));
    bestk = key > bestk ? key : bestk;
  }
  bestk = block_max_u64<kPathThreads>(bestk, s_scratch);
  const int p = static_cast<int>(0xffffffffu - static_cast<uint32_t>(bestk & 0xffffffffu));
  const int k = static_cast<int>(bestk >> 32);
  if (static_cast<int>(threadIdx.x) == p % kPathThreads) {   // the thread that walked path p
    int last = 0;                                            // the root when nothing is accepted
    if (k > 0) {
      if (loaded == p && k <= kPathRegs) {
#pragma unroll
        for (int j = 0; j < kPathRegs; ++j)
          if (j == k - 1) last = pn[j];
      } else {
        last = a.paths[static_cast<long>(p) * (a.dmax + 1) + k];
      }
    }
    s_last = last;
    a.best[b] = p;
    a.accept_len[b] = k;
  }
  if (!a.next_token) return;
  __syncthreads();
  const int last = s_last;
  // the greedy token after the last accepted node; its argmax is known if it has children
  if (!s_leaf[last]) {
    if (threadIdx.x == 0) a.next_token[b] = a.rowarg[static_cast<long>(b) * a.T + last];
  } else {
    const int esz = a.dtype == 1 ? 2 : 4;
    const char* lrow = static_cast<const char*>(a.logits) + (static_cast<long>(b) * a.T + last) * a.V * esz;
    const uint64_t g = block_row_argmax<kPathThreads, 8, LOAD>(lrow, a.dtype, a.V, s_scratch);
    if (threadIdx.x == 0) a.next_token[b] = static_cast<int32_t>(sel_key_index(g));
  }
}

AcceptWs accept_ws_layout(int B, int T, long V, int n_internal, int maxc_nucleus) {
  AcceptWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) & ~size_t(255); return o; };
  w.unroll = accept_unroll(B, V, n_internal);
  const long chunk = static_cast<long>(kAccVec) * w.unroll;
  const long C = (V + chunk - 1) / chunk;
  w.chunks = static_cast<int>(C);
  w.part = take((sizeof(RowStat) + sizeof(uint64_t)) * static_cast<size_t>(B) * n_internal * C);
  w.dec = take(sizeof(int32_t) * static_cast<size_t>(B) * T * 2);   // decisions + row argmax
  // nucleus mode: the mass above every child of every chunk
  w.mass = maxc_nucleus > 0 ? take(sizeof(float) * static_cast<size_t>(B) * n_internal * C * maxc_nucleus) : 0;
  w.total = off;
  return w;
}

hipError_t launch_typical_accept(const void* logits, int dtype, int B, int T, long V,
                                 const int32_t* tokens, int n_internal, const int32_t* internal,
                                 const int32_t* child_ptr, const int32_t* child_idx,
                                 const int32_t* paths, const int32_t* path_len, int n_paths,
                                 int dmax, float temperature, float eps, float delta,
                                 int nucleus, float top_p, int maxc,
                                 int32_t* best, int32_t* accept_len, int32_t* next_token,
                                 char* ws, hipStream_t s) {
  const AcceptWs L = accept_ws_layout(B, T, V, n_internal, nucleus ? maxc : 0);
  const size_t nstat = static_cast<size_t>(B) * n_internal * L.chunks;
  AcceptArgs a{};
  a.logits = logits;
  a.dtype = dtype;
  a.B = B;
  a.T = T;
  a.V = V;
  a.tokens = tokens;
  a.n_int = n_internal;
  a.internal = internal;
  a.child_ptr = child_ptr;
  a.child_idx = child_idx;
  a.paths = paths;
  a.path_len = path_len;
  a.n_paths = n_paths;
  a.dmax = dmax;
  a.greedy = temperature == 0.f;
  a.y_scale = a.greedy ? 0.f : static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
  a.ln_eps = logf(eps);
  a.ln_delta = logf(delta);
  a.C = L.chunks;
  a.nucleus = nucleus && !a.greedy;
  a.top_p = top_p;
  a.maxc = maxc;
  a.part_mass = nucleus ? reinterpret_cast<float*>(ws + L.mass) : nullptr;
  a.part_stat = reinterpret_cast<RowStat*>(ws + L.part);
  a.part_arg = reinterpret_cast<uint64_t*>(ws + L.part + sizeof(RowStat) * nstat);
  a.dec = reinterpret_cast<int32_t*>(ws + L.dec);
  a.rowarg = a.dec + static_cast<size_t>(B) * T;
  a.best = best;
  a.accept_len = accept_len;
  a.next_token = next_token;
  const dim3 grid(L.chunks, n_internal, B);
  hook_before(K_ACCEPT, s);
  // vector loads when every thread's 8-element group is wholly in or out of the row
  const bool vec = V % 8 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
  const int load = vec ? (dtype == 1 ? 1 : 2) : 0;
  const bool wide = V * (dtype == 1 ? 2 : 4) > kPathWideBytes;
#define MEDUSA_ACCEPT_LAUNCH(LD)                                                             \
  if (a.nucleus) {                                                                         \
    if (L.unroll == 4) accept_chunks_nucleus<4, LD><<<grid, kAccThreads, 0, s>>>(a);       \
    else if (L.unroll == 2) accept_chunks_nucleus<2, LD><<<grid, kAccThreads, 0, s>>>(a);  \
    else accept_chunks_nucleus<1, LD><<<grid, kAccThreads, 0, s>>>(a);                     \
  } else if (L.unroll == 4) accept_chunks<4, LD><<<grid, kAccThreads, 0, s>>>(a);          \
  else if (L.unroll == 2) accept_chunks<2, LD><<<grid, kAccThreads, 0, s>>>(a);            \
  else accept_chunks<1, LD><<<grid, kAccThreads, 0, s>>>(a);                               \
  accept_rows<<<dim3(n_internal, B), kAccThreads, 0, s>>>(a);                      \
  if (wide) accept_paths<1024, LD><<<B, 1024, 0, s>>>(a);                          \
  else accept_paths<256, LD><<<B, 256, 0, s>>>(a);
  if (load == 1) {
    MEDUSA_ACCEPT_LAUNCH(1)
  } else if (load == 2) {
    MEDUSA_ACCEPT_LAUNCH(2)
  } else {
    MEDUSA_ACCEPT_LAUNCH(0)
  }
#undef MEDUSA_ACCEPT_LAUNCH
  hook_after(K_ACCEPT, s);
  return hipGetLastError();
}

}  // namespace medusa
