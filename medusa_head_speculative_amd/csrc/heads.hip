// Medusa heads: r = h + SiLU(W1 h + b1), logits = W2 r, then per-head top-k.
//
// Ultralytics glossary "Medusa Heads", how-the-heads-predict section: every head reads the same
// last hidden state, applies one fully connected layer with SiLU and a residual connection and
// then its own vocab projection (W1 with bias, W2 without, [out, in] weights).  Wiblog "Medusa
// multi-head speculative decoding", inference-flow section: each head keeps its top-k tokens.
//
// At batch <= 8 both projections are matrix-vector products that stream every weight byte
// once, so they are HBM-bound.  The bf16 path runs them on the matrix cores anyway: the weights
// are the A operand exactly as stored, and the B operand packs the (at most 8) input vectors as
// 16 columns, hi and lo bf16 halves of the fp32 vector side by side, so r keeps ~17 bits of
// mantissa and each weight is loaded once with 16-byte loads.  The fp32 path (small models)
// uses plain FMAs.
#include "common.h"
#include "kernels.h"

namespace medusa {

// ------------------------------------------------------------------------------------------
// Epilogue shared by the two projections
// ------------------------------------------------------------------------------------------
struct HeadsEpi {
  int mode;               // 0: first layer (u -> r), 1: vocab projection (-> logits)
  int K;
  long rows;              // rows per head (hidden for mode 0, vocab for mode 1)
  int hd;
  int B;
  const void* b1;         // [K][hd] dtype            (mode 0)
  const void* h;          // [B][hd] dtype            (mode 0)
  int dtype;
  float* r_out;           // [B][K][hd] fp32          (mode 0)
  uint16_t* xfrag;        // [K][hd/32][64][8] bf16   (mode 0, bf16 path only)
  float* logits;          // [B][K][rows] fp32        (mode 1)
};

__device__ __forceinline__ float load_elem(const void* p, int dtype, long i) {
  return dtype == 0 ? static_cast<const float*>(p)[i] : bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// One finished output y = (W x_b)[row] of head k.
__device__ __forceinline__ void heads_epilogue(const HeadsEpi& ep, int k, long row, int b, float y) {
  if (ep.mode == 0) {
    const int i = static_cast<int>(row);
    const float u = y + load_elem(ep.b1, ep.dtype, static_cast<long>(k) * ep.hd + i);
    const float r = load_elem(ep.h, ep.dtype, static_cast<long>(b) * ep.hd + i) + u / (1.0f + expf(-u));
    ep.r_out[(static_cast<long>(b) * ep.K + k) * ep.hd + i] = r;
    if (ep.xfrag) {
      // B-operand fragment of the vocab projection: kblock i/32, lane group (i%32)/8, element i%8;
      // column b carries hi(r), column B+b carries lo(r) = r - hi(r); columns >= 2B are zero.
      const uint16_t hi = f32_to_bf16_rne(r);
      const uint16_t lo = f32_to_bf16_rne(r - bf16_to_f32(hi));
      const long kb = i >> 5;
      const int g = (i >> 3) & 3, e = i & 7;
      uint16_t* base = ep.xfrag + ((static_cast<long>(k) * (ep.hd >> 5) + kb) * 64) * 8;
      base[(g * 16 + b) * 8 + e] = hi;
      base[(g * 16 + ep.B + b) * 8 + e] = lo;
      if (b == 0)
        for (int n = 2 * ep.B; n < 16; ++n) base[(g * 16 + n) * 8 + e] = 0;
    }
  } else {
    ep.logits[(static_cast<long>(b) * ep.K + k) * ep.rows + row] = y;
  }
}

// ------------------------------------------------------------------------------------------
// bf16 weights on the matrix cores
// ------------------------------------------------------------------------------------------
// Work-group: 4 waves, 16*TPW consecutive rows of one head; wave w takes the w-th quarter of the
// hidden dim for all of them, so the 4 partial tiles are summed in LDS in a fixed order.
// MFMA v_mfma_f32_16x16x32_bf16, A = 16 weight rows x 32 columns (lane l: row l%16, columns
// 8*(l/16)..+7: one 16-byte load), B = 32 columns x 16 vectors, D lane l: rows 4*(l/16)+j of
// vector column l%16.
// XFROM_H: the B operand is built from h itself (bf16, so lo = 0); otherwise it is read from the
// fragment buffer written by the first layer's epilogue.
template <int TPW, bool XFROM_H>
__global__ __launch_bounds__(256) void heads_gemv_bf16(const uint16_t* __restrict__ W,
                                                        const uint16_t* __restrict__ xsrc,
                                                        HeadsEpi ep) {
  __shared__ float red[4][TPW][64][4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int k = blockIdx.y;
  const long row0 = static_cast<long>(blockIdx.x) * (16 * TPW);
  const int hd = ep.hd;
  const int nkb = hd >> 5;
  const int kb0 = (wave * nkb) >> 2, kb1 = ((wave + 1) * nkb) >> 2;
  const int g = lane >> 4, n = lane & 15;

  const uint16_t* wrow[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    long r = row0 + t * 16 + n;
    if (r > ep.rows - 1) r = ep.rows - 1;          // ragged tail: valid address, result dropped
    wrow[t] = W + (static_cast<long>(k) * ep.rows + r) * hd + g * 8;
  }
  const uint16_t* xf = XFROM_H ? (n < ep.B ? xsrc + static_cast<long>(n) * hd + g * 8 : nullptr)
                               : xsrc + (static_cast<long>(k) * nkb * 64 + lane) * 8;

  f32x4_t acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int kb = kb0;
  for (; kb + 4 <= kb1; kb += 4) {
    bf16x8_t a[4][TPW], x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) a[u][t] = load_bf16x8(wrow[t] + (kb + u) * 32);
      if (XFROM_H) x[u] = xf ? load_bf16x8(xf + (kb + u) * 32) : zero_bf16x8();
      else x[u] = load_bf16x8(xf + static_cast<long>(kb + u) * 512);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < TPW; ++t) acc[t] = mfma16x16x32(a[u][t], x[u], acc[t]);
  }
  for (; kb < kb1; ++kb) {
    bf16x8_t a[TPW], x;
#pragma unroll
    for (int t = 0; t < TPW; ++t) a[t] = load_bf16x8(wrow[t] + kb * 32);
    if (XFROM_H) x = xf ? load_bf16x8(xf + kb * 32) : zero_bf16x8();
    else x = load_bf16x8(xf + static_cast<long>(kb) * 512);
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = mfma16x16x32(a[t], x, acc[t]);
  }

#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[wave][t][lane][j] = acc[t][j];
  __syncthreads();

  // outputs of this work-group: 16*TPW rows x B vectors; y = sum over waves of (hi + lo) columns
  const int B = ep.B;
  for (int o = threadIdx.x; o < 16 * TPW * B; o += 256) {
    const int rr = o / B, b = o - rr * B;
    const int t = rr >> 4, m = rr & 15;
    const int lh = (m >> 2) * 16 + b, j = m & 3;
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) y += red[w][t][lh][j] + red[w][t][lh + B][j];
    const long row = row0 + rr;
    if (row < ep.rows) heads_epilogue(ep, k, row, b, y);
  }
}

// ------------------------------------------------------------------------------------------
// fp32 weights: one wave per row, lanes across the hidden dim, fixed-order butterfly sum
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void heads_gemv_f32(const float* __restrict__ W,
                                                       const float* __restrict__ x, long x_bstride,
                                                       long x_kstride, HeadsEpi ep) {
  const int lane = threadIdx.x & 63;
  const long row = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int k = blockIdx.y;
  if (row >= ep.rows) return;
  const int hd = ep.hd, B = ep.B;
  const float* w = W + (static_cast<long>(k) * ep.rows + row) * hd;
  const float* xk = x + static_cast<long>(k) * x_kstride;
  float acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = 0.f;
  for (int j = lane * 4; j < hd; j += 256) {
    const float4 wv = *reinterpret_cast<const float4*>(w + j);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      if (b < B) {
        const float4 xv = *reinterpret_cast<const float4*>(xk + b * x_bstride + j);
        acc[b] = fmaf(wv.x, xv.x, acc[b]);
        acc[b] = fmaf(wv.y, xv.y, acc[b]);
        acc[b] = fmaf(wv.z, xv.z, acc[b]);
        acc[b] = fmaf(wv.w, xv.w, acc[b]);
      }
    }
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    if (b < B) {
      float v = acc[b];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
      if (lane == b) heads_epilogue(ep, k, row, b, v);
    }
  }
}

// ------------------------------------------------------------------------------------------
// top-k over each row of the fp32 logits [R][V]
// ------------------------------------------------------------------------------------------
// Grid (C chunks, R rows).  Each work-group selects its chunk's k best keys by k rounds of a
// block-wide max (a round takes the best key below the previous winner; keys are unique), then
// the last work-group of the row to finish merges the C*k candidates the same way.
constexpr int kTopkThreads = 256;
constexpr int kTopkPerThread = 16;
constexpr int kTopkChunk = kTopkThreads * kTopkPerThread;

__global__ __launch_bounds__(kTopkThreads) void topk_rows(const float* __restrict__ logits, long V,
                                                          int k, int C, uint64_t* __restrict__ part,
                                                          unsigned* __restrict__ counters,
                                                          int32_t* __restrict__ ids,
                                                          float* __restrict__ vals) {
  __shared__ uint64_t scratch[kTopkThreads / 64];
  __shared__ int s_last;
  const int row = blockIdx.y, c = blockIdx.x;
  const float* x = logits + static_cast<long>(row) * V;
  uint64_t keys[kTopkPerThread];
#pragma unroll
  for (int e = 0; e < kTopkPerThread; ++e) {
    const long idx = static_cast<long>(c) * kTopkChunk + e * kTopkThreads + threadIdx.x;
    keys[e] = idx < V ? sel_key(x[idx], static_cast<uint32_t>(idx)) : 0ull;
  }
  uint64_t prev = ~0ull;
  for (int t = 0; t < k; ++t) {
    uint64_t best = 0;
#pragma unroll
    for (int e = 0; e < kTopkPerThread; ++e)
      if (keys[e] < prev && keys[e] > best) best = keys[e];
    best = block_max_u64<kTopkThreads>(best, scratch);
    if (threadIdx.x == 0) part[(static_cast<long>(row) * C + c) * k + t] = best;
    prev = best;
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&counters[row], 1u) == static_cast<unsigned>(C - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const uint64_t* pr = part + static_cast<long>(row) * C * k;
  const long n = static_cast<long>(C) * k;
  prev = ~0ull;
  for (int t = 0; t < k; ++t) {
    uint64_t best = 0;
    for (long i = threadIdx.x; i < n; i += kTopkThreads) {
      const uint64_t v = __builtin_nontemporal_load(pr + i);
      if (v < prev && v > best) best = v;
    }
    best = block_max_u64<kTopkThreads>(best, scratch);
    if (threadIdx.x == 0) {
      ids[static_cast<long>(row) * k + t] = static_cast<int32_t>(sel_key_index(best));
      if (vals) vals[static_cast<long>(row) * k + t] = sel_key_value(best);
    }
    prev = best;
  }
  if (threadIdx.x == 0) counters[row] = 0u;
}

// ------------------------------------------------------------------------------------------
// launcher
// ------------------------------------------------------------------------------------------
HeadsWs heads_ws_layout(int B, int hd, long V, int K, int topk) {
  HeadsWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) & ~size_t(255); return o; };
  w.r = take(sizeof(float) * B * K * hd);
  w.xfrag = take(sizeof(uint16_t) * static_cast<size_t>(K) * hd * 32);
  w.logits = take(sizeof(float) * static_cast<size_t>(B) * K * V);
  const long C = (V + kTopkChunk - 1) / kTopkChunk;
  w.part = take(sizeof(uint64_t) * static_cast<size_t>(B) * K * C * topk);
  w.counters = take(sizeof(unsigned) * B * K);
  w.total = off;
  w.chunks = static_cast<int>(C);
  return w;
}

hipError_t launch_heads(const void* h, const void* w1, const void* b1, const void* w2, int dtype,
                        int B, int hd, long V, int K, int topk, float* logits, int32_t* topk_ids,
                        float* topk_logits, char* ws, hipStream_t s) {
  const HeadsWs L = heads_ws_layout(B, hd, V, K, topk);
  float* r = reinterpret_cast<float*>(ws + L.r);
  uint16_t* xfrag = reinterpret_cast<uint16_t*>(ws + L.xfrag);
  float* lg = logits ? logits : reinterpret_cast<float*>(ws + L.logits);
  uint64_t* part = reinterpret_cast<uint64_t*>(ws + L.part);
  unsigned* counters = reinterpret_cast<unsigned*>(ws + L.counters);

  HeadsEpi e1{0, K, hd, hd, B, b1, h, dtype, r, dtype == 1 ? xfrag : nullptr, nullptr};
  HeadsEpi e2{1, K, V, hd, B, nullptr, nullptr, dtype, nullptr, nullptr, lg};
  if (dtype == 1) {
    constexpr int TPW1 = 2, TPW2 = 2;
    heads_gemv_bf16<TPW1, true><<<dim3((hd + 16 * TPW1 - 1) / (16 * TPW1), K), 256, 0, s>>>(
        static_cast<const uint16_t*>(w1), static_cast<const uint16_t*>(h), e1);
    heads_gemv_bf16<TPW2, false><<<dim3((V + 16 * TPW2 - 1) / (16 * TPW2), K), 256, 0, s>>>(
        static_cast<const uint16_t*>(w2), xfrag, e2);
  } else {
    heads_gemv_f32<<<dim3((hd + 3) / 4, K), 256, 0, s>>>(static_cast<const float*>(w1),
                                                         static_cast<const float*>(h), hd, 0, e1);
    heads_gemv_f32<<<dim3((V + 3) / 4, K), 256, 0, s>>>(static_cast<const float*>(w2), r,
                                                        static_cast<long>(K) * hd, hd, e2);
  }
  topk_rows<<<dim3(L.chunks, B * K), kTopkThreads, 0, s>>>(lg, V, topk, L.chunks, part, counters,
                                                           topk_ids, topk_logits);
  return hipGetLastError();
}

}  // namespace medusa
