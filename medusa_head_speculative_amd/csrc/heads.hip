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
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace medusa {

// ------------------------------------------------------------------------------------------
// Epilogue shared by the projections
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
  uint16_t* xs;           // [K][2B][hd] bf16         (mode 0, bf16 path): hi(r) rows, then lo(r)
  float* logits;          // [B][K][rows] fp32        (mode 1)
  // heads of several residual blocks (zero values: one block, residual from h, x shared)
  int nb;                 // blocks per head; the weights of head k, block blk are weight head
  int blk;                //   k * max(nb, 1) + blk of the [K * nb] stacked / packed tensors
  const float* r_res;     // [B][K][hd] fp32 residual input (mode 0), NULL: h
  int x_per_head;         // the vector operand is per head ([K][ncols][hd]) in mode 0 too
};

__device__ __forceinline__ int weight_head(const HeadsEpi& ep, int k) {
  return k * (ep.nb > 1 ? ep.nb : 1) + ep.blk;
}

__device__ __forceinline__ float load_elem(const void* p, int dtype, long i) {
  return dtype == 0 ? static_cast<const float*>(p)[i] : bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}

// The first layer's per-output inputs: bias b1[k][row] and residual x[b][row] (h or the previous
// block's r).
struct EpiIn {
  float bias, x;
};
__device__ __forceinline__ EpiIn epi_inputs(const HeadsEpi& ep, int k, long row, int b) {
  const int i = static_cast<int>(row);
  EpiIn in;
  in.bias = load_elem(ep.b1, ep.dtype, static_cast<long>(weight_head(ep, k)) * ep.hd + i);
  in.x = ep.r_res ? ep.r_res[(static_cast<long>(b) * ep.K + k) * ep.hd + i]
                  : load_elem(ep.h, ep.dtype, static_cast<long>(b) * ep.hd + i);
  return in;
}

// One finished output y = (W x_b)[row] of head k; `in` holds the first layer's inputs.
__device__ __forceinline__ void heads_epilogue_in(const HeadsEpi& ep, int k, long row, int b, float y,
                                                  EpiIn in) {
  if (ep.mode == 0) {
    const int i = static_cast<int>(row);
    const float u = y + in.bias;
    const float x = in.x;
    const float r = x + u / (1.0f + expf(-u));
    ep.r_out[(static_cast<long>(b) * ep.K + k) * ep.hd + i] = r;
    if (ep.xs) {
      // the vocab projection's vector operand: hi(r) and lo(r) = r - hi(r) as bf16 rows
      const uint16_t hi = f32_to_bf16_rne(r);
      const uint16_t lo = f32_to_bf16_rne(r - bf16_to_f32(hi));
      uint16_t* base = ep.xs + static_cast<long>(k) * 2 * ep.B * ep.hd + i;
      base[static_cast<long>(b) * ep.hd] = hi;
      base[static_cast<long>(ep.B + b) * ep.hd] = lo;
    }
  } else {
    ep.logits[(static_cast<long>(b) * ep.K + k) * ep.rows + row] = y;
  }
}

__device__ __forceinline__ void heads_epilogue(const HeadsEpi& ep, int k, long row, int b, float y) {
  heads_epilogue_in(ep, k, row, b, y, ep.mode == 0 ? epi_inputs(ep, k, row, b) : EpiIn{0.f, 0.f});
}

// The same inputs for bf16 heads, loaded early as raw 32-bit words and converted only when used,
// so that nothing waits for them before the weight stream starts: the aligned word holding the
// bf16 bias, and the fp32 residual (the previous block's r) or the aligned word holding the bf16
// h element.  (hd is a multiple of 32, so an element's aligned word lies inside its row.)
struct EpiRaw {
  uint32_t bias, x;
};
__device__ __forceinline__ EpiRaw epi_raw_bf16(const HeadsEpi& ep, int k, long row, int b) {
  const long i = row;
  const long bi = static_cast<long>(weight_head(ep, k)) * ep.hd + i;
  const uint32_t* xp = ep.r_res ? reinterpret_cast<const uint32_t*>(ep.r_res + (static_cast<long>(b) * ep.K + k) * ep.hd + i)
                                : reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(ep.h) + ((static_cast<long>(b) * ep.hd + i) & ~1l));
  EpiRaw in;
  in.bias = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(ep.b1) + (bi & ~1l));
  in.x = *xp;
  return in;
}
__device__ __forceinline__ EpiIn epi_from_raw_bf16(const HeadsEpi& ep, long row, EpiRaw r) {
  // the high half of a word holds the odd element (little endian); row parity is the element's
  // parity in both arrays since hd is even
  const int sh = (row & 1) ? 16 : 0;
  return EpiIn{bf16_to_f32(static_cast<uint16_t>(r.bias >> sh)),
               ep.r_res ? __uint_as_float(r.x) : bf16_to_f32(static_cast<uint16_t>(r.x >> sh))};
}

// B operand of v_mfma_f32_16x16x32_bf16 for contraction block kb: lane l holds column n = l%16,
// contraction indices 8*(l/16)..+7.  Columns n < ncols are rows of xs ([ncols][hd] bf16: the B
// vectors for the first layer, or hi then lo halves of r for the vocab projection); the others
// are zero.
__device__ __forceinline__ bf16x8_t x_operand(const uint16_t* xp, int kb) {
  return xp ? load_bf16x8(xp + kb * 32) : zero_bf16x8();
}

__device__ __forceinline__ bf16x8_t load_bf16x8_nt(const uint16_t* p) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return __builtin_bit_cast(bf16x8_t, v);
}

// ------------------------------------------------------------------------------------------
// bf16 weights in the [out, in] layout, on the matrix cores
// ------------------------------------------------------------------------------------------
// Work-group: 4 waves, 16*TPW consecutive rows of one head; wave w takes the w-th quarter of the
// hidden dim for all of them, so the 4 partial tiles are summed in LDS in a fixed order.
// A = 16 weight rows x 32 columns (lane l: row l%16, columns 8*(l/16)..+7: one 16-byte
// nontemporal load, the weights are read once), D lane l: rows 4*(l/16)+j of column l%16.
template <int TPW>
__global__ __launch_bounds__(256) void heads_gemv_bf16(const uint16_t* __restrict__ W,
                                                        const uint16_t* __restrict__ xsrc,
                                                        int ncols, HeadsEpi ep) {
  __shared__ float red[4][TPW][64][4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int k = blockIdx.y;
  const long row0 = static_cast<long>(blockIdx.x) * (16 * TPW);
  const int hd = ep.hd;
  // 32-column contraction blocks; when hd % 32 != 0 (hd is a multiple of 8) the last block is
  // partial and the wave that owns it loads zeros for its columns past hd
  const int nkb = (hd + 31) >> 5, nfull = hd >> 5;
  const int kb0 = (wave * nkb) >> 2, kb1 = ((wave + 1) * nkb) >> 2;
  const int kb1f = kb1 < nfull ? kb1 : nfull;
  const int g = lane >> 4, n = lane & 15;

  const uint16_t* wrow[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    long r = row0 + t * 16 + n;
    if (r > ep.rows - 1) r = ep.rows - 1;          // ragged tail: valid address, result dropped
    wrow[t] = W + (static_cast<long>(weight_head(ep, k)) * ep.rows + r) * hd + g * 8;
  }
  const int xph = ep.mode == 1 || ep.x_per_head;
  const uint16_t* xp = n < ncols ? xsrc + (static_cast<long>(k) * ncols * xph + n) * hd + g * 8
                                 : nullptr;

  f32x4_t acc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  int kb = kb0;
  for (; kb + 4 <= kb1f; kb += 4) {
    bf16x8_t a[4][TPW], x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int t = 0; t < TPW; ++t) a[u][t] = load_bf16x8_nt(wrow[t] + (kb + u) * 32);
      x[u] = x_operand(xp, kb + u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int t = 0; t < TPW; ++t) acc[t] = mfma16x16x32(a[u][t], x[u], acc[t]);
  }
  for (; kb < kb1f; ++kb) {
    bf16x8_t a[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) a[t] = load_bf16x8_nt(wrow[t] + kb * 32);
    const bf16x8_t x = x_operand(xp, kb);
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = mfma16x16x32(a[t], x, acc[t]);
  }
  if (kb1 > nfull) {
    // the partial last block: columns kb*32 + 8g .. +7 exist only when below hd (a multiple of
    // 8, so a lane's 8 columns are all in the row or all past it); the others contribute zeros
    // and are never loaded
    const bool in = nfull * 32 + g * 8 < hd;
    bf16x8_t a[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) a[t] = in ? load_bf16x8_nt(wrow[t] + nfull * 32) : zero_bf16x8();
    const bf16x8_t x = in ? x_operand(xp, nfull) : zero_bf16x8();
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
  const int lo_off = ncols > B ? B : 0;             // the first layer's vector has no lo part
  for (int o = threadIdx.x; o < 16 * TPW * B; o += 256) {
    const int rr = o / B, b = o - rr * B;
    const int t = rr >> 4, m = rr & 15;
    const int lh = (m >> 2) * 16 + b, j = m & 3;
    float y = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) y += lo_off ? red[w][t][lh][j] + red[w][t][lh + lo_off][j] : red[w][t][lh][j];
    const long row = row0 + rr;
    if (row < ep.rows) heads_epilogue(ep, k, row, b, y);
  }
}

// ------------------------------------------------------------------------------------------
// bf16 weights pre-packed in MFMA fragment order
// ------------------------------------------------------------------------------------------
// Packed layout (medusa_pack_weights).  The rows of all K heads are cut into 16-row tiles,
// numbered gt = k*ntiles + tile (G = K*ntiles tiles in all).  The 64 lanes' 16-byte A fragments
// of tile gt for 32-column block kb form one 1 KB block:
//   block(gt, kb)[lane][e] = W[k][16*tile + lane%16][32*kb + 8*(lane/16) + e]   (0 past the rows)
// The tiles are cut into groups of gs consecutive tiles, gs being the tiles that one round of
// the persistent grid reads (pack_group_tiles); inside group g (of size n, gs but for the last)
// the blocks are kb-major: block(g*gs + w, kb) is block number g*nkb*gs + kb*n + w.  One
// wave-wide 16-byte load reads 1 KB of contiguous memory; the waves of a round read neighbouring
// kilobytes at each contraction step, and each step's window follows the previous one, so the
// persistent grid sweeps the weights in address order, as a plain read does.
// Work item = TPW consecutive tiles of one head.  KSPLIT = 4: the 4 waves of a work-group split
// the contraction of one item and meet in LDS (short matrices: more bytes in flight).
// KSPLIT = 1: a wave owns an item and its whole contraction; with PERSIST the grid holds about
// two work-groups per CU and each wave takes items in grid-stride order, which keeps the window
// that the resident waves read narrow.
constexpr long kPersistWgs = 512;            // about two work-groups per CU

// Tiles per group of the packed layout: the waves one round of the persistent one-tile-per-wave
// grid holds (the fewest rounds of 4*kPersistWgs waves, then just enough work-groups for them).
__host__ __device__ __forceinline__ long pack_group_tiles(long G) {
  const long rounds = (G + 4 * kPersistWgs - 1) / (4 * kPersistWgs);
  return 4 * ((G + 4 * rounds - 1) / (4 * rounds));
}
// 1 KB block number of (tile gt, contraction block kb), and the distance in blocks from kb to
// kb + 1 for that tile (its group's size)
__host__ __device__ __forceinline__ long pack_block(long G, long gs, int nkb, long gt, long kb,
                                                    long& kbstride_blocks) {
  const long g = gt / gs, w = gt - g * gs;
  const long n = G - g * gs < gs ? G - g * gs : gs;
  kbstride_blocks = n;
  return g * nkb * gs + kb * n + w;
}

template <int TPW, int U, int KSPLIT, bool PERSIST>
__global__ __launch_bounds__(256) void heads_gemv_packed(const uint16_t* __restrict__ Wp,
                                                          const uint16_t* __restrict__ xsrc,
                                                          int ncols, HeadsEpi ep) {
  static_assert(KSPLIT == 1 || !PERSIST, "persistent variants own whole items");
  static_assert(KSPLIT == 1 || TPW <= 2, "the split epilogue gives each thread at most one output");
  __shared__ float red[KSPLIT == 4 ? 4 : 1][TPW][64][4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const long ntiles = (ep.rows + 15) >> 4;
  const long G = ntiles * ep.K * (ep.nb > 1 ? ep.nb : 1);   // tiles of all packed weight heads
  const long per_head = (ntiles + TPW - 1) / TPW;      // work items per head
  const int xph = ep.mode == 1 || ep.x_per_head;
  const int hd = ep.hd;
  const int nkb = hd >> 5;
  const long gs = pack_group_tiles(G);
  const int kb0 = KSPLIT == 4 ? (wave * nkb) >> 2 : 0;
  const int kb1 = KSPLIT == 4 ? ((wave + 1) * nkb) >> 2 : nkb;
  const int g = lane >> 4, n = lane & 15;
  const int B = ep.B;
  const int lo_off = ncols > B ? B : 0;                 // the first layer's vector has no lo part

  long item, step, end;
  if (PERSIST) {
    item = static_cast<long>(blockIdx.x) * 4 + wave;
    step = static_cast<long>(gridDim.x) * 4;
    end = per_head * ep.K;
  } else {
    const long i = KSPLIT == 4 ? static_cast<long>(blockIdx.x) : static_cast<long>(blockIdx.x) * 4 + wave;
    if (KSPLIT == 1 && i >= per_head) return;
    item = static_cast<long>(blockIdx.y) * per_head + i;
    step = 1;
    end = item + 1;
  }

  for (; item < end; item += step) {
    const int k = static_cast<int>(item / per_head);
    const long t0 = (item - static_cast<long>(k) * per_head) * TPW;
    const uint16_t* ap[TPW];
    long kbstride[TPW];                                 // elements from block kb to kb + 1
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      long tt = t0 + t;
      if (tt > ntiles - 1) tt = ntiles - 1;             // ragged: valid address, result dropped
      long sb;
      const long blk = pack_block(G, gs, nkb, static_cast<long>(weight_head(ep, k)) * ntiles + tt, kb0, sb);
      ap[t] = Wp + blk * 512 + lane * 8;
      kbstride[t] = sb * 512;
    }
    const uint16_t* xp = n < ncols ? xsrc + (static_cast<long>(k) * ncols * xph + n) * hd + g * 8
                                   : nullptr;

    f32x4_t acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // split epilogue: thread o < 16*TPW*B finishes output (row t0*16 + o/B, sequence o%B); its
    // first-layer inputs (bf16: this kernel serves only bf16 heads) are loaded now, so their
    // latency hides behind the weight stream
    EpiRaw pre{0u, 0u};
    if (KSPLIT == 4 && ep.mode == 0 && static_cast<int>(threadIdx.x) < 16 * TPW * B) {
      const int rr = static_cast<int>(threadIdx.x) / B;
      const long row = t0 * 16 + rr;
      if (row < ep.rows) pre = epi_raw_bf16(ep, k, row, static_cast<int>(threadIdx.x) - rr * B);
    }

    int kb = kb0;
    for (; kb + U <= kb1; kb += U) {
      bf16x8_t a[U][TPW], x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int t = 0; t < TPW; ++t) a[u][t] = load_bf16x8_nt(ap[t] + u * kbstride[t]);
        x[u] = x_operand(xp, kb + u);
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) ap[t] += U * kbstride[t];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < TPW; ++t) acc[t] = mfma16x16x32(a[u][t], x[u], acc[t]);
    }
    for (; kb < kb1; ++kb) {
      bf16x8_t a[TPW];
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        a[t] = load_bf16x8_nt(ap[t]);
        ap[t] += kbstride[t];
      }
      const bf16x8_t x = x_operand(xp, kb);
#pragma unroll
      for (int t = 0; t < TPW; ++t) acc[t] = mfma16x16x32(a[t], x, acc[t]);
    }

    if (KSPLIT == 4) {
#pragma unroll
      for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[wave][t][lane][j] = acc[t][j];
      __syncthreads();
      const int o = threadIdx.x;
      if (o < 16 * TPW * B) {
        const int rr = o / B, b = o - rr * B;
        const int t = rr >> 4, m = rr & 15;
        const int lh = (m >> 2) * 16 + b, j = m & 3;
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) y += lo_off ? red[w][t][lh][j] + red[w][t][lh + lo_off][j] : red[w][t][lh][j];
        const long row = t0 * 16 + rr;
        // the opaque step keeps the conversions (and so the wait for the loads) here, after the
        // weight stream, instead of hoisted next to the loads
        asm volatile("" : "+v"(pre.bias), "+v"(pre.x));
        if (row < ep.rows) heads_epilogue_in(ep, k, row, b, y, epi_from_raw_bf16(ep, row, pre));
      }
    } else {
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float y = acc[t][j];
          const float ylo = __shfl_down(y, lo_off > 0 ? lo_off : 1);
          if (lo_off) y += ylo;
          const long row = (t0 + t) * 16 + 4 * g + j;
          if (n < B && row < ep.rows) heads_epilogue(ep, k, row, n, y);
        }
      }
    }
  }
}

// Repack [K][rows][hd] bf16 weights into the fragment order above; one thread per 16 bytes of
// the packed tensor (block index = i / 64).
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ W, long rows,
                                                           int hd, int K, long total16,
                                                           uint16_t* __restrict__ P) {
  const long i = static_cast<long>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total16) return;
  const long ntiles = (rows + 15) >> 4;
  const long G = ntiles * K;
  const int nkb = hd >> 5;
  const long gs = pack_group_tiles(G);
  const int lane = static_cast<int>(i & 63);
  const long blk = i >> 6;
  // invert the block number: group, then kb-major inside the group
  const long g = blk / (static_cast<long>(nkb) * gs);
  const long off = blk - g * nkb * gs;
  const long n = G - g * gs < gs ? G - g * gs : gs;
  const long kb = off / n;
  const long gt = g * gs + (off - kb * n);
  const long k = gt / ntiles, tile = gt - k * ntiles;
  const long row = tile * 16 + (lane & 15);
  uint4 v = make_uint4(0, 0, 0, 0);
  if (row < rows) v = *reinterpret_cast<const uint4*>(W + (k * rows + row) * hd + kb * 32 + 8 * (lane >> 4));
  *reinterpret_cast<uint4*>(P + i * 8) = v;
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
  const float* w = W + (static_cast<long>(weight_head(ep, k)) * ep.rows + row) * hd;
  const float* xk = x + static_cast<long>(k) * x_kstride;
  // lane b < B finishes sequence b's output; its first-layer inputs are loaded up front
  EpiIn pre{0.f, 0.f};
  if (ep.mode == 0 && lane < B) pre = epi_inputs(ep, k, row, lane);
  float acc[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) acc[b] = 0.f;
  for (int j = lane * 4; j < hd; j += 256) {
    // the weight and all 8 vector loads go out together (sequences past B read sequence 0's
    // vector and are ignored)
    const float4 wv = *reinterpret_cast<const float4*>(w + j);
    float4 xv[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) xv[b] = *reinterpret_cast<const float4*>(xk + (b < B ? b : 0) * x_bstride + j);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      acc[b] = fmaf(wv.x, xv[b].x, acc[b]);
      acc[b] = fmaf(wv.y, xv[b].y, acc[b]);
      acc[b] = fmaf(wv.z, xv[b].z, acc[b]);
      acc[b] = fmaf(wv.w, xv[b].w, acc[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    if (b < B) {
      float v = acc[b];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
      if (lane == b) heads_epilogue_in(ep, k, row, b, v, pre);
    }
  }
}

// ------------------------------------------------------------------------------------------
// top-k over each row of the fp32 logits [R][V]
// ------------------------------------------------------------------------------------------
// Selection keys are unique (value, then lower id), so "the k best" is a well defined set and
// the rounds below need no tie handling.  One round picks the best key below the previous
// winner with a wave-wide max (DPP, no LDS).
//
// Two launches, no cross-work-group handoff: topk_chunks (grid C x R) reduces each 2048-element
// chunk to its k best (each wave its 512 elements, then wave 0 merges the 4 lists);
// topk_merge (grid R, one wave) merges the C*k candidates of a row, 512 at a time together with
// the running list.
constexpr int kTopkThreads = 256;
constexpr int kTopkPerLane = 8;
constexpr int kTopkChunk = kTopkThreads * kTopkPerLane;   // 2048

// k rounds over NK keys per lane plus a running list (lane t < k holds entry t).  Returns the
// new list in lanes 0..k-1 (lane t: t-th best); other lanes get 0.
template <int NK>
__device__ __forceinline__ uint64_t wave_select(const uint64_t (&keys)[NK], uint64_t running, int k) {
  const int lane = threadIdx.x & 63;
  uint64_t prev = ~0ull, mine = 0;
  for (int t = 0; t < k; ++t) {
    uint64_t best = running < prev ? running : 0ull;
#pragma unroll
    for (int e = 0; e < NK; ++e)
      if (keys[e] < prev && keys[e] > best) best = keys[e];
    best = wave_max_u64_dpp(best);
    if (lane == t) mine = best;
    prev = best;
  }
  return mine;
}

__global__ __launch_bounds__(kTopkThreads) void topk_chunks(const float* __restrict__ logits, long V,
                                                            int k, int C,
                                                            uint64_t* __restrict__ part) {
  __shared__ uint64_t s_cand[4][64];
  const int row = blockIdx.y, c = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* x = logits + static_cast<long>(row) * V;
  uint64_t keys[kTopkPerLane];
  const long base = static_cast<long>(c) * kTopkChunk + wave * (kTopkChunk / 4);
  // every load goes out before any is used: an element past the row loads element 0 instead
  // (always valid) and is dropped, so no branch surrounds a load
  float v[kTopkPerLane];
#pragma unroll
  for (int e = 0; e < kTopkPerLane; ++e) {
    const long idx = base + e * 64 + lane;
    v[e] = x[idx < V ? idx : 0];
  }
#pragma unroll
  for (int e = 0; e < kTopkPerLane; ++e) {
    const long idx = base + e * 64 + lane;
    keys[e] = idx < V ? sel_key(v[e], static_cast<uint32_t>(idx)) : 0ull;
  }
  s_cand[wave][lane] = wave_select(keys, 0ull, k);
  __syncthreads();
  if (wave != 0) return;
  uint64_t k4[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) k4[w] = lane < k ? s_cand[w][lane] : 0ull;
  const uint64_t mine = wave_select(k4, 0ull, k);
  if (lane < k) part[(static_cast<long>(row) * C + c) * k + lane] = mine;
}

// With g.tokens set, the merge wave of (sequence b, head kh) also writes the tree tokens and
// position ids of depth kh + 1, which head kh fills (Wiblog, tree-attention section): node i of
// that depth takes the candidate of rank rank[i], which lane rank[i] holds; the (b, 0) wave also
// writes the root.  The same values as build_tree's gather, without its launch.
__global__ __launch_bounds__(64) void topk_merge(const uint64_t* __restrict__ part, int k, int C,
                                                 int32_t* __restrict__ ids, float* __restrict__ vals,
                                                 int K, TreeGather g) {
  const int row = blockIdx.x, lane = threadIdx.x;
  const uint64_t* pr = part + static_cast<long>(row) * C * k;
  const long n = static_cast<long>(C) * k;
  uint64_t running = 0;
  for (long b0 = 0; b0 < n; b0 += 64 * kTopkPerLane) {
    uint64_t keys[kTopkPerLane];
#pragma unroll
    for (int e = 0; e < kTopkPerLane; ++e) {
      const long i = b0 + e * 64 + lane;
      keys[e] = i < n ? pr[i] : 0ull;
    }
    running = wave_select(keys, running, k);
  }
  const int32_t id = static_cast<int32_t>(sel_key_index(running));
  if (lane < k) {
    ids[static_cast<long>(row) * k + lane] = id;
    if (vals) vals[static_cast<long>(row) * k + lane] = sel_key_value(running);
  }
  if (g.tokens) {
    const int b = row / K, kh = row - b * K;
    const int pl = g.prefix_len[b];
    const int rt = g.root[b];
    int32_t* tk = g.tokens + static_cast<long>(b) * g.T;
    int32_t* ps = g.pos + static_cast<long>(b) * g.T;
    // Eight 64-node slices per pass: all their depth / rank loads are issued before the first
    // store (the stores could alias the static arrays as far as the compiler knows, so a
    // one-slice loop would wait out a full load latency per slice).  Lanes past the end read the
    // last node and are masked by depth -1.
    constexpr int kSlices = 8;
    for (int i0 = 0; i0 < g.T; i0 += 64 * kSlices) {
      int d[kSlices], r[kSlices];
#pragma unroll
      for (int u = 0; u < kSlices; ++u) {
        const int i = i0 + u * 64 + lane;
        const int ic = i < g.T ? i : g.T - 1;
        d[u] = g.depth[ic];
        r[u] = g.rank[ic];
        if (i >= g.T) d[u] = -1;
      }
#pragma unroll
      for (int u = 0; u < kSlices; ++u) {
        const int i = i0 + u * 64 + lane;
        const int32_t cand = __shfl(id, r[u] > 0 ? r[u] : 0);   // every lane takes part
        if (d[u] == kh + 1) {
          tk[i] = cand;
          ps[i] = pl + d[u];
        } else if (d[u] == 0 && kh == 0) {
          tk[i] = rt;
          ps[i] = pl;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
// LayerNorm of a block's input (heads whose residual blocks start with LayerNorm)
// ------------------------------------------------------------------------------------------
// One work-group per (sequence, head): mean and mean squared deviation over the hidden dimension
// in fp32 (two passes over the row, which stays in cache, fixed-order sums), then
// (x - mean) / sqrt(var + eps) * gamma + beta as the next layer's vector operand: hi/lo bf16
// rows of xs (matrix-core path) or fp32 rows of xn (fp32 path).
__device__ __forceinline__ float block_sum256(float v, float* s_red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float t = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
  __syncthreads();
  return t;
}

// 8 elements i0, i0 + 256, ... of a row, every load issued before any is converted (a slot past
// hd reads element 0, always valid, and is ignored by the caller)
template <bool BF16>
__device__ __forceinline__ void ln_load8(const void* p, int i0, int hd, float (&v)[8]) {
  uint32_t raw[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int i = i0 + e * 256;
    const int ii = i < hd ? i : 0;
    raw[e] = BF16 ? static_cast<uint32_t>(static_cast<const uint16_t*>(p)[ii])
                  : __float_as_uint(static_cast<const float*>(p)[ii]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = BF16 ? bf16_to_f32(static_cast<uint16_t>(raw[e])) : __uint_as_float(raw[e]);
}

// XBF16: the input row is bf16 (h of a bf16 head), else fp32 (h of an fp32 head, or the previous
// block's r); WBF16: gamma and beta are bf16.
template <bool XBF16, bool WBF16>
__device__ __forceinline__ void layernorm_row(const void* x, const void* gamma, const void* beta,
                                              float eps, int B, int K, int hd, int b, int k,
                                              long wb, uint16_t* xs, float* xn, float* s_red) {
  float sum = 0.f;
  for (int i0 = threadIdx.x; i0 < hd; i0 += 8 * 256) {
    float v[8];
    ln_load8<XBF16>(x, i0, hd, v);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (i0 + e * 256 < hd) sum += v[e];
  }
  const float mean = block_sum256(sum, s_red) / static_cast<float>(hd);
  float sq = 0.f;
  for (int i0 = threadIdx.x; i0 < hd; i0 += 8 * 256) {
    float v[8];
    ln_load8<XBF16>(x, i0, hd, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = v[e] - mean;
      if (i0 + e * 256 < hd) sq = fmaf(d, d, sq);
    }
  }
  const float var = block_sum256(sq, s_red) / static_cast<float>(hd);
  const float rstd = 1.0f / sqrtf(var + eps);
  const char* g = static_cast<const char*>(gamma) + wb * (WBF16 ? 2 : 4);
  const char* be = static_cast<const char*>(beta) + wb * (WBF16 ? 2 : 4);
  for (int i0 = threadIdx.x; i0 < hd; i0 += 8 * 256) {
    float v[8], gv[8], bv[8];
    ln_load8<XBF16>(x, i0, hd, v);
    ln_load8<WBF16>(g, i0, hd, gv);
    ln_load8<WBF16>(be, i0, hd, bv);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = i0 + e * 256;
      if (i >= hd) continue;
      const float y = (v[e] - mean) * rstd * gv[e] + bv[e];
      if (xs) {
        const uint16_t hi = f32_to_bf16_rne(y);
        const uint16_t lo = f32_to_bf16_rne(y - bf16_to_f32(hi));
        uint16_t* base = xs + static_cast<long>(k) * 2 * B * hd + i;
        base[static_cast<long>(b) * hd] = hi;
        base[static_cast<long>(B + b) * hd] = lo;
      } else {
        xn[(static_cast<long>(b) * K + k) * hd + i] = y;
      }
    }
  }
}

__global__ __launch_bounds__(256) void heads_layernorm(const void* h, const float* r_in, int dtype,
                                                       const void* gamma, const void* beta, float eps,
                                                       int B, int K, int hd, int wh_mul, int blk,
                                                       uint16_t* xs, float* xn) {
  __shared__ float s_red[4];
  const int b = blockIdx.x, k = blockIdx.y;
  const long wb = static_cast<long>(k * wh_mul + blk) * hd;
  if (r_in) {
    const float* x = r_in + (static_cast<long>(b) * K + k) * hd;
    if (dtype == 1) layernorm_row<false, true>(x, gamma, beta, eps, B, K, hd, b, k, wb, xs, xn, s_red);
    else layernorm_row<false, false>(x, gamma, beta, eps, B, K, hd, b, k, wb, xs, xn, s_red);
  } else if (dtype == 1) {
    const uint16_t* x = static_cast<const uint16_t*>(h) + static_cast<long>(b) * hd;
    layernorm_row<true, true>(x, gamma, beta, eps, B, K, hd, b, k, wb, xs, xn, s_red);
  } else {
    const float* x = static_cast<const float*>(h) + static_cast<long>(b) * hd;
    layernorm_row<false, false>(x, gamma, beta, eps, B, K, hd, b, k, wb, xs, xn, s_red);
  }
}

// ------------------------------------------------------------------------------------------
// launcher
// ------------------------------------------------------------------------------------------
HeadsWs heads_ws_layout(int B, int hd, long V, int K, int topk, int nb, int ln) {
  HeadsWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) & ~size_t(255); return o; };
  const size_t rbytes = sizeof(float) * B * K * hd;
  const size_t xbytes = sizeof(uint16_t) * static_cast<size_t>(K) * 2 * B * hd;
  w.r = take(rbytes);
  w.r2 = nb > 1 ? take(rbytes) : w.r;            // block inputs and outputs alternate
  w.xs = take(xbytes);
  w.xs2 = nb > 1 || ln ? take(xbytes) : w.xs;
  w.xn = ln ? take(rbytes) : 0;                   // LayerNorm output of the fp32 path
  w.logits = take(sizeof(float) * static_cast<size_t>(B) * K * V);
  const long C = (V + kTopkChunk - 1) / kTopkChunk;
  w.part = take(sizeof(uint64_t) * static_cast<size_t>(B) * K * C * topk);
  w.total = off;
  w.chunks = static_cast<int>(C);
  return w;
}

size_t packed_weight_bytes(int K, long rows, int hd) {
  return static_cast<size_t>(K) * ((rows + 15) / 16) * 16 * hd * sizeof(uint16_t);
}

hipError_t launch_pack_weights(const void* w, int K, long rows, int hd, void* packed, hipStream_t s) {
  const long total16 = static_cast<long>(packed_weight_bytes(K, rows, hd) / 16);
  pack_weights_kernel<<<static_cast<unsigned>((total16 + 255) / 256), 256, 0, s>>>(
      static_cast<const uint16_t*>(w), rows, hd, K, total16, static_cast<uint16_t*>(packed));
  return hipGetLastError();
}

// Packed-layout kernel variants (tiles per wave, unroll, contraction split, persistent grid);
// selectable for tuning through MEDUSA_W1_VARIANT / MEDUSA_W2_VARIANT.
struct PackedVariant {
  int tpw, u, ksplit, persist;
};
static const PackedVariant kPackedVariants[] = {
    {1, 8, 4, 0}, {2, 8, 4, 0}, {1, 8, 1, 0}, {2, 4, 1, 0}, {2, 8, 1, 0}, {4, 4, 1, 0},
    {1, 8, 1, 1}, {1, 16, 1, 1}, {2, 8, 1, 1}, {2, 4, 1, 1}, {1, 4, 1, 1}, {1, 16, 4, 0},
    {1, 4, 4, 0}, {8, 1, 1, 0}};
// Defaults from timing each variant on MI355X at the workload shapes (hidden 4096-8192, vocab
// 32000-128256): B <= 2 persistent with one tile per wave, B <= 4 persistent with two tiles per
// wave, B > 4 (16 vector columns, so the x loads cost as much as the weight loads) one grid of
// non-persistent waves with eight tiles sharing each x load, one block in flight per tile (on
// the 33B shape at B = 8: 186.5 us, against 202 us with two tiles per wave and 8 blocks).
constexpr int kDefaultW1Variant = 0;
static int default_w2_variant(int B) { return B <= 2 ? 10 : (B <= 4 ? 8 : 13); }

static int variant_from_env(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  const int i = atoi(v);
  return (i >= 0 && i < static_cast<int>(sizeof(kPackedVariants) / sizeof(kPackedVariants[0]))) ? i : dflt;
}

static void launch_packed(int variant, const uint16_t* Wp, const uint16_t* x, int ncols,
                          const HeadsEpi& ep, hipStream_t s) {
  const PackedVariant v = kPackedVariants[variant];
  const long ntiles = (ep.rows + 15) / 16;
  const long per_head = (ntiles + v.tpw - 1) / v.tpw;
  dim3 grid;
  if (v.persist) {
    // the fewest rounds of 4*kPersistWgs waves, then just enough work-groups for that many
    // rounds, so every wave gets the same number of items (give or take one)
    const long items = per_head * ep.K;
    const long rounds = (items + 4 * kPersistWgs - 1) / (4 * kPersistWgs);
    grid = dim3(static_cast<unsigned>((items + 4 * rounds - 1) / (4 * rounds)));
  } else {
    const long per_block = v.ksplit == 4 ? 1 : 4;
    grid = dim3(static_cast<unsigned>((per_head + per_block - 1) / per_block), ep.K);
  }
#define MEDUSA_PACKED_CASE(I, T, U_, S_, P_) \
  case I: heads_gemv_packed<T, U_, S_, P_><<<grid, 256, 0, s>>>(Wp, x, ncols, ep); break;
  switch (variant) {
    MEDUSA_PACKED_CASE(0, 1, 8, 4, false)
    MEDUSA_PACKED_CASE(1, 2, 8, 4, false)
    MEDUSA_PACKED_CASE(2, 1, 8, 1, false)
    MEDUSA_PACKED_CASE(3, 2, 4, 1, false)
    MEDUSA_PACKED_CASE(4, 2, 8, 1, false)
    MEDUSA_PACKED_CASE(5, 4, 4, 1, false)
    MEDUSA_PACKED_CASE(6, 1, 8, 1, true)
    MEDUSA_PACKED_CASE(7, 1, 16, 1, true)
    MEDUSA_PACKED_CASE(8, 2, 8, 1, true)
    MEDUSA_PACKED_CASE(9, 2, 4, 1, true)
    MEDUSA_PACKED_CASE(10, 1, 4, 1, true)
    MEDUSA_PACKED_CASE(11, 1, 16, 4, false)
    MEDUSA_PACKED_CASE(13, 8, 1, 1, false)
    default: MEDUSA_PACKED_CASE(12, 1, 4, 4, false)
  }
#undef MEDUSA_PACKED_CASE
}

hipError_t launch_heads_ex(const void* h, const void* w1, const void* b1, const void* gamma,
                           const void* beta, float eps, const void* w2, int dtype, int packed, int nb,
                           int B, int hd, long V, int K, int topk, float* logits, int32_t* topk_ids,
                           float* topk_logits, char* ws, hipStream_t s, const TreeGather* gather) {
  const bool ln = gamma != nullptr;
  const HeadsWs L = heads_ws_layout(B, hd, V, K, topk, nb, ln);
  float* rb[2] = {reinterpret_cast<float*>(ws + L.r), reinterpret_cast<float*>(ws + L.r2)};
  uint16_t* xb[2] = {reinterpret_cast<uint16_t*>(ws + L.xs), reinterpret_cast<uint16_t*>(ws + L.xs2)};
  float* xn = ln ? reinterpret_cast<float*>(ws + L.xn) : nullptr;
  float* lg = logits ? logits : reinterpret_cast<float*>(ws + L.logits);
  uint64_t* part = reinterpret_cast<uint64_t*>(ws + L.part);
  const uint16_t* hb = static_cast<const uint16_t*>(h);
  static const int v1 = variant_from_env("MEDUSA_W1_VARIANT", kDefaultW1Variant);
  static const int v2_env = variant_from_env("MEDUSA_W2_VARIANT", -1);

  // block j reads its input from h (j = 0) or r buffer `cur`, writes r buffer `cur ^ 1` (0 for
  // j = 0) and the next layer's hi/lo operand into the xs buffer it does not read
  int cur = -1, xcur = -1;
  for (int j = 0; j < nb; ++j) {
    const int out = cur < 0 ? 0 : cur ^ 1;
    HeadsEpi e1{0, K, hd, hd, B, b1, h, dtype, rb[out], nullptr, nullptr, nb, j,
                cur < 0 ? nullptr : rb[cur], 0};
    const uint16_t* xop = hb;          // the layer's vector operand (bf16 paths)
    int ncols = B;
    const float* xf = static_cast<const float*>(h);   // (fp32 path)
    long xf_b = hd, xf_k = 0;
    if (ln) {
      const int xl = xcur == 0 ? 1 : 0;
      heads_layernorm<<<dim3(B, K), 256, 0, s>>>(h, cur < 0 ? nullptr : rb[cur], dtype, gamma, beta,
                                                 eps, B, K, hd, nb, j, dtype == 1 ? xb[xl] : nullptr, xn);
      xop = xb[xl];
      ncols = 2 * B;
      e1.x_per_head = 1;
      xcur = xl;
      xf = xn;
      xf_b = static_cast<long>(K) * hd;
      xf_k = hd;
    } else if (j > 0) {
      xop = xb[xcur];
      ncols = 2 * B;
      e1.x_per_head = 1;
      xf = rb[cur];
      xf_b = static_cast<long>(K) * hd;
      xf_k = hd;
    }
    const int xo = xcur == 0 ? 1 : 0;  // the operand written for the next layer
    if (dtype == 1) e1.xs = xb[xo];
    hook_before(K_HEADS_W1, s);
    if (dtype == 1 && packed) {
      launch_packed(v1, static_cast<const uint16_t*>(w1), xop, ncols, e1, s);
    } else if (dtype == 1) {
      constexpr int TPW1 = 2;
      heads_gemv_bf16<TPW1><<<dim3((hd + 16 * TPW1 - 1) / (16 * TPW1), K), 256, 0, s>>>(
          static_cast<const uint16_t*>(w1), xop, ncols, e1);
    } else {
      heads_gemv_f32<<<dim3((hd + 3) / 4, K), 256, 0, s>>>(static_cast<const float*>(w1), xf, xf_b,
                                                           xf_k, e1);
    }
    hook_after(K_HEADS_W1, s);
    cur = out;
    xcur = xo;
  }

  HeadsEpi e2{1, K, V, hd, B, nullptr, nullptr, dtype, nullptr, nullptr, lg, 0, 0, nullptr, 1};
  hook_before(K_HEADS_W2, s);
  if (dtype == 1 && packed) {
    const int v2 = v2_env >= 0 ? v2_env : default_w2_variant(B);
    launch_packed(v2, static_cast<const uint16_t*>(w2), xb[xcur], 2 * B, e2, s);
  } else if (dtype == 1) {
    constexpr int TPW2 = 2;
    heads_gemv_bf16<TPW2><<<dim3((V + 16 * TPW2 - 1) / (16 * TPW2), K), 256, 0, s>>>(
        static_cast<const uint16_t*>(w2), xb[xcur], 2 * B, e2);
  } else {
    heads_gemv_f32<<<dim3((V + 3) / 4, K), 256, 0, s>>>(static_cast<const float*>(w2), rb[cur],
                                                        static_cast<long>(K) * hd, hd, e2);
  }
  hook_after(K_HEADS_W2, s);
  hook_before(K_TOPK, s);
  topk_chunks<<<dim3(L.chunks, B * K), kTopkThreads, 0, s>>>(lg, V, topk, L.chunks, part);
  topk_merge<<<B * K, 64, 0, s>>>(part, topk, L.chunks, topk_ids, topk_logits, K,
                                  gather ? *gather : TreeGather{});
  hook_after(K_TOPK, s);
  return hipGetLastError();
}

hipError_t launch_heads(const void* h, const void* w1, const void* b1, const void* w2, int dtype,
                        int packed, int B, int hd, long V, int K, int topk, float* logits,
                        int32_t* topk_ids, float* topk_logits, char* ws, hipStream_t s,
                        const TreeGather* gather) {
  return launch_heads_ex(h, w1, b1, nullptr, nullptr, 0.f, w2, dtype, packed, 1, B, hd, V, K, topk,
                         logits, topk_ids, topk_logits, ws, s, gather);
}

}  // namespace medusa
