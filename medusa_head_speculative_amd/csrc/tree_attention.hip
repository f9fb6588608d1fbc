// Tree-masked attention of the candidate tokens over the prefix KV cache and their ancestors.
//
// Wiblog "Medusa multi-head speculative decoding", tree-attention section: all candidates are
// verified in one forward pass; a token attends only to the tokens on its own prefix path,
// never across branches; the fixed tree's mask is precomputed.  Ultralytics "Medusa Heads",
// tree-attention section: each token sees only its ancestors in the tree.
//
// bf16 path (matrix cores).  A work-group owns 128 query rows of one (sequence, kv head), 32 or
// 16 per wave: the rows are (node, q head of the group) pairs, node-major, so grouped query heads
// share every K/V tile.  It walks 64-row K/V tiles (the prefix, then the tree rows), staged in LDS row-major:
//   S^T = K Q^T   v_mfma_f32_16x16x32_bf16, A = K rows from LDS, B = Q rows held in registers;
//                 a lane ends up with 4 columns of one query row per 16-column block, so the
//                 online softmax runs per lane plus two cross-lane steps;
//   O^T = V^T P^T the exponentiated scores are already laid out as the B operand; the A operand
//                 V^T comes from LDS with ds_read_b64_tr_b16 (16-lane transposed reads), so V is
//                 never transposed in memory.
// Tree tiles that no row of the work-group can see are skipped; inside a tile each row's mask
// word selects its ancestors.  A row or two past the last full 128-row tile ride along as extra
// rows on the vector units (bf16 pair dot products) instead of taking a query tile of their own.
// When there are too few (sequence, kv head, query tile) units to fill the chip, the K/V range
// is split and a second kernel merges the partial results in a fixed order.  fp32 path (small
// models): one wave per output row, plain FMAs.
#include <math.h>
#include <stdlib.h>

#include "common.h"
#include "kernels.h"

namespace medusa {

constexpr int kAttnRows = 128;   // query rows per work-group (4 waves x 32, or 8 x 16) ...
constexpr int kAttnRowsWide = 144;   // ... or 9 waves x 16 when that takes fewer query tiles
constexpr int kKvTile = 64;
constexpr int kMaxSplits = 16;
// Work-groups at or above which the bf16 kernel keeps two row blocks per wave (4 waves of 32
// rows, 198 VGPRs, two waves per SIMD) instead of one (8 waves of 16 rows, 120 VGPRs, four per
// SIMD).  Measured on MI355X: the 8-wave form is faster on grids up to a few rounds of the 512
// work-groups that fit at two per CU (7B shape 16.2 -> 15.1 us, Llama-8B shape 21.5 -> 20.0,
// 33B shape 159 -> 155 at 832 work-groups), and no faster on the 70B-layer grid of 2240
// (1277-1307 against 1293 us; its rotary variant 1264-1283 against 1326-1329), where each wave
// reading K for only 16 rows doubles the LDS traffic per row.
constexpr long kAttnTwoBlockUnits = 1536;

typedef __attribute__((ext_vector_type(4))) short s16x4_t;

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* prefix_len;
  const uint64_t* mask;
  uint16_t* out;
  float* o_part;     // [splits][B][Hkv][Mpad][D]
  float2* ml_part;   // [splits][B][Hkv][Mpad]
  long lcap;
  int B, Hq, Hkv, T, W, G, M, Mpad, qtiles, splits, nwork, Lmax;
  int xrem, xbase;   // query tiles qt < xrem also own row xbase + qt (the extra-row kernel)
  float sl2;         // scale * log2(e)
  const float* rope_cs;  // [B*T][2][D/2] cos, sin of every node; queries are rotated when ROPE is set
};

// Rotary embedding of one pair (x_i, x_{i+D/2}) with the cos/sin of its angle, in fp32 as the
// rotation of the key rows does
__device__ __forceinline__ void rope_rotate(float cs, float sn, float& x, float& y) {
  const float xr = fmaf(x, cs, -(y * sn));
  const float yr = fmaf(x, sn, y * cs);
  x = xr;
  y = yr;
}

__device__ __forceinline__ bf16x8_t lds_read16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ s16x4_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4_t*)(p));
}

// A lane's value after a DPP move (quad permutation or a rotation inside the 16-lane row)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// c + a.lo * b.lo + a.hi * b.hi over two bf16 pairs (v_dot2c_f32_bf16)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// LDS tile layout: 64 K (or V) rows of D bf16, rows back to back; the 16-byte chunks of a row are
// permuted by an XOR with a row-dependent slot key.  The direct global->LDS loads write 64
// consecutive 16-byte slots per wave instruction, so the permutation is applied on the global
// side: the lane that fills slot s of row r loads chunk s ^ key(r).
// For D = 128 the key is 2 * (r mod 8).  With it the bank-conflict counter reads zero for both
// operand reads below, which then run at the rate of linear reads: 4 LDS cycles per 16-byte K read
// (16 rows, one chunk each; the earlier key cost 8) and 2 per transposed V read (8 rows of a
// half-wave, 2 chunks each; the earlier key cost 4).  The transposed reads see 64 four-byte banks
// per half-wave, so the 8 rows of a half-wave must use 8 different chunk pairs; the 16-byte reads
// group lanes in a way that rows 0-7 against rows 8-15 of one chunk do not disturb.
template <int D>
__device__ __forceinline__ int slot_key(int r) {
  if constexpr (D == 128) {
    return (r & 7) << 1;
  } else {
    return (r >> 1) & 7;
  }
}

template <int D>
__device__ __forceinline__ int tile_elem(int r, int c) {   // element offset of (row r, chunk c)
  return r * D + ((c ^ slot_key<D>(r)) << 3);
}

// The operand reads below touch rows whose slot key depends on the lane only (the row bits that
// vary from read to read are above bit 3; the key reads bits 0-2 for D = 128, 1-3 for D = 64),
// so every address is one per-lane base XOR a compile-time block index: no per-read address
// registers.
//   K fragment (cb, kb): row cb*16 + mm, chunk kb*4 + lg  ->  (kbase ^ (kb << 5)) + cb*16*D
//   V fragment (db, ks, hi): row ks*32 + hi*16 + 4*lg + mm/4, chunk db*2 + (mm&3)/2, +4 if mm odd
//                        ->  (vbase ^ (db << 4)) + (ks*32 + hi*16)*D
template <int D>
__device__ __forceinline__ int k_frag_base(int lg, int mm) {
  const int key = slot_key<D>(mm);
  return mm * D + (((lg ^ key) & 3) << 3) + ((key >> 2) << 5);
}
template <int D>
__device__ __forceinline__ int v_frag_base(int lg, int mm) {
  const int r = 4 * lg + (mm >> 2);
  const int key = slot_key<D>(r);
  return r * D + ((((mm & 3) >> 1) ^ key) & 1) * 8 + (mm & 1) * 4 + ((key >> 1) << 4);
}

// Async loads of one 64-row K/V tile straight into LDS (no registers), as buffer loads: the
// buffer descriptors (scalar) start at the tile's first row and cover its nvalid valid rows, so
// rows past them read as zeros (finite data whose scores the mask removes; no clamp), and each
// lane's byte offset inside the tile is the same for every tile (tile_voffsets, computed once).
// No vector instruction per tile besides the loads.
template <int D, int NW>
struct TileLoad {
  static constexpr int SLOTS = D / 8;                 // 16-byte chunks per row
  static constexpr int RPI = 64 / SLOTS;              // rows per wave instruction
  static constexpr int NWL = NW < 8 ? NW : 8;         // loading waves (a ninth wave loads nothing)
  static constexpr int INST = kKvTile / RPI / NWL;    // instructions per wave per matrix
};

template <int D, int NW>
__device__ __forceinline__ void tile_voffsets(int wave, int lane, int (&voff)[TileLoad<D, NW>::INST]) {
  using TL = TileLoad<D, NW>;
#pragma unroll
  for (int u = 0; u < TL::INST; ++u) {
    const int r = (wave * TL::INST + u) * TL::RPI + lane / TL::SLOTS;
    const int c = (lane % TL::SLOTS) ^ slot_key<D>(r);
    voff[u] = (r * D + c * 8) * 2;
  }
}

// stream: nontemporal loads (each K/V row is read by this work-group only)
template <int D, int NW>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ kc,
                                           const uint16_t* __restrict__ vc, long rowbase,
                                           int nvalid, uint16_t* Kd, uint16_t* Vd, int wave,
                                           const int* voff, bool stream = false) {
  using TL = TileLoad<D, NW>;
  if (NW > TL::NWL && wave >= TL::NWL) return;
  const int bytes = nvalid * D * 2;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kc + rowbase * D), 0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(vc + rowbase * D), 0, bytes, 0x00020000);
  if (stream) {
#pragma unroll
    for (int u = 0; u < TL::INST; ++u) {
      const int rbase = (wave * TL::INST + u) * TL::RPI;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(Kd + rbase * D), 16, voff[u], 0, 0, 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(Vd + rbase * D), 16, voff[u], 0, 0, 2);
    }
  } else {
#pragma unroll
    for (int u = 0; u < TL::INST; ++u) {
      const int rbase = (wave * TL::INST + u) * TL::RPI;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(Kd + rbase * D), 16, voff[u], 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(Vd + rbase * D), 16, voff[u], 0, 0, 0);
    }
  }
}

// Async load of the mask words of one tree tile for this wave's RPW query rows straight into
// LDS (4 bytes per lane: lane l < 2*RPW fills half l%2 of row l/2's word).  Invalid rows read
// node 0's word.
template <int RPW>
__device__ __forceinline__ void issue_mask(const uint64_t* __restrict__ mask, int W, int tt,
                                           int row_node, uint64_t* Md, int wave, int lane) {
  if (RPW == 32 || lane < 2 * RPW) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(mask + static_cast<long>(row_node) * W + tt) + (lane & 1);
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(Md + wave * RPW), 4, 0, 0);
  }
}

// The extra row's mask word of one tree tile, into LDS by two lanes of wave 0
__device__ __forceinline__ void issue_xmask(const uint64_t* __restrict__ mask, int W, int tt, int node,
                                            uint64_t* Md, int wave, int lane) {
  if (wave == 0 && lane < 2) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(mask + static_cast<long>(node) * W + tt) + lane;
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)Md, 4, 0, 0);
  }
}

// NMB 16-row blocks per wave and NW waves, so a work-group owns ROWS = NW * 16 * NMB query rows:
// 128 with NW = 8 / NMB (NMB = 2 keeps more rows per wave, NMB = 1 twice the waves with half the
// registers each, so four waves share a SIMD), or 144 with nine waves of one block, when a
// (sequence, kv head) has a few rows past a multiple of 128 that would otherwise take a query
// tile of their own and stream the whole K/V range once more.
// XR (4 waves of 32 rows): query tiles qt < xrem also own row xbase + qt, one row past the full
// 128-row tiles, on the vector units.  In every K/V tile wave w takes keys 16w..16w+15 of that
// row: a lane holds one key and a quarter of the head dim for the scores (bf16 pair dot products,
// summed over the four quarters with row rotations that leave every copy with the same bits), and
// for P V the transposed V reads of the matrix-core path give it four keys of one output column.
// Each wave keeps its own online softmax state of the row; the four are merged at the end, in
// wave order.  A lone row thus costs a few dozen vector instructions per tile and wave instead of
// a sixteen-row block of matrix products, and the 4-wave form keeps two work-groups per CU.
template <int D, bool ROPE, int NMB, int NW, bool XR = false>
__global__ __launch_bounds__(NW * 64, 2) void tree_attn_bf16(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int RPW = NMB * 16;          // query rows per wave
  constexpr int ROWS = NW * RPW;         // query rows per work-group
  static_assert(ROWS == kAttnRows || ROWS == kAttnRowsWide, "a work-group owns 128 or 144 rows");
  static_assert(!XR || (NMB == 2 && NW == 4), "the extra row is split over four waves of 16 keys");
  constexpr int NKB = D / 32;            // 32-wide contraction blocks over the head dim
  constexpr int NDB = D / 16;            // 16-wide output blocks over the head dim
  constexpr int TILE = kKvTile * D;      // elements per K (or V) tile
  __shared__ __align__(16) uint16_t K0[TILE];
  __shared__ __align__(16) uint16_t V0[TILE];
  __shared__ __align__(16) uint16_t K1[TILE];
  __shared__ __align__(16) uint16_t V1[TILE];
  __shared__ int s_active[64];
  // mask words of the tree tile in flight (the extra row's last)
  __shared__ __align__(16) uint64_t s_mask[2][ROWS + (XR ? 1 : 0)];
  __shared__ float s_xo[XR ? NW : 1][XR ? D : 1];   // per-wave extra-row states for the merge
  __shared__ float2 s_xml[XR ? NW : 1];

  // ---- work item; consecutive logical items (query tiles of one K/V range) share an XCD ----
  const int per_xcd = gridDim.x >> 3;
  const int logical = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (logical >= a.nwork) return;
  const int qt = logical % a.qtiles;
  int rest = logical / a.qtiles;
  const int split = rest % a.splits;
  rest /= a.splits;
  const int kvh = rest % a.Hkv;
  const int b = rest / a.Hkv;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases stay scalar
  const int lg = lane >> 4, mm = lane & 15;
  const int L = min(max(a.prefix_len[b], 0), a.Lmax);   // callers promise prefix_len <= Lmax
  const int np = (L + kKvTile - 1) / kKvTile;
  const int ntt = (a.T + kKvTile - 1) / kKvTile;
  const int ntiles = np + ntt;
  // split s covers tiles [ceil(s n / S), ceil((s + 1) n / S)): the longer splits come first and
  // the last one, which holds the tree tiles (masked, with the mask scan before them), is the
  // shortest
  const int t_begin = static_cast<int>((static_cast<long>(split) * ntiles + a.splits - 1) / a.splits);
  const int t_end = static_cast<int>((static_cast<long>(split + 1) * ntiles + a.splits - 1) / a.splits);
  const long kvbase = (static_cast<long>(b) * a.Hkv + kvh) * a.lcap;
  // the extra row of this query tile (XR), if it has one
  const bool has_x = XR && qt < a.xrem;
  const int xrow_m = has_x ? a.xbase + qt : 0;
  const int xnode = xrow_m / a.G;

  // ---- tree tiles that some row of this work-group can see (only needed if the K/V range of
  //      this work-group reaches the tree rows) ----
  const bool has_tree = t_end > np;
  if (has_tree) {
    for (int t = tid; t < 64; t += NT) s_active[t] = 0;
    __syncthreads();
    // four mask words per thread in flight at once (a slot past the rows reads word 0, always
    // valid, and is ignored)
    for (int p0 = tid; p0 < ROWS * ntt; p0 += 4 * NT) {
      uint64_t w[4];
      int tt[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + u * NT;
        const int r = p / ntt;
        tt[u] = p - r * ntt;
        const int m = qt * ROWS + r;
        ok[u] = p < ROWS * ntt && m < a.M;
        w[u] = a.mask[ok[u] ? static_cast<long>(m / a.G) * a.W + tt[u] : 0];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (ok[u] && w[u] != 0ull) s_active[tt[u]] = 1;
    }
    if (has_x)
      for (int p = tid; p < ntt; p += NT)
        if (a.mask[static_cast<long>(xnode) * a.W + p] != 0ull) s_active[p] = 1;
    __syncthreads();
  }
  auto next_active = [&](int t) {   // (uniform: every thread reads the same flags)
    while (t < t_end && t >= np && !s_active[t - np]) ++t;
    return __builtin_amdgcn_readfirstlane(t);
  };
  auto tile_rows = [&](int t, long& row0, int& nvalid) {   // first cache row, valid rows
    if (t < np) {
      row0 = static_cast<long>(t) * kKvTile;
      nvalid = min(kKvTile, L - t * kKvTile);
    } else {
      row0 = L + static_cast<long>(t - np) * kKvTile;
      nvalid = min(kKvTile, a.T - (t - np) * kKvTile);
    }
  };

  // node whose mask word this lane stages: row wave*RPW + lane/2 of the work-group
  const int mrow_m = qt * ROWS + wave * RPW + (lane >> 1);
  // a wave whose rows are all past M only helps stage tiles and meets the barriers (the
  // extra-row kernel runs only full 128-row tiles)
  const bool wave_active = XR || qt * ROWS + wave * RPW < a.M;
  const int mrow_node = mrow_m < a.M ? mrow_m / a.G : 0;

  int voff[TileLoad<D, NW>::INST];   // this lane's byte offsets inside a tile
  tile_voffsets<D, NW>(wave, lane, voff);
  // With one query tile per (sequence, kv head) no other work-group reads these K/V rows: the
  // extra-row kernel then streams them with nontemporal loads (on the 33B shape attention went
  // from 106 to 101.5 us; the split grids of the other forms measured no gain or a loss).
  const bool stream = XR && a.qtiles == 1;
  int t = next_active(t_begin);
  int buf = 0;
  if (t < t_end) {
    long row0;
    int nvalid;
    tile_rows(t, row0, nvalid);
    issue_tile<D, NW>(a.kc, a.vc, kvbase + row0, nvalid, K0, V0, wave, voff, stream);
    if (t >= np) {
      issue_mask<RPW>(a.mask, a.W, t - np, mrow_node, s_mask[0], wave, lane);
      if (has_x) issue_xmask(a.mask, a.W, t - np, xnode, &s_mask[0][ROWS], wave, lane);
    }
  }

  // ---- this lane's query rows (one per row block mb) ----
  int node[NMB];
  bool rvalid[NMB];
  bf16x8_t qf[NMB][NKB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const int m = qt * ROWS + wave * RPW + mb * 16 + mm;
    rvalid[mb] = m < a.M;
    node[mb] = rvalid[mb] ? m / a.G : 0;
    const int hq = kvh * a.G + (rvalid[mb] ? m % a.G : 0);
    const uint16_t* qrow = a.q + ((static_cast<long>(b) * a.Hq + hq) * a.T + node[mb]) * D;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
      qf[mb][kb] = rvalid[mb] ? load_bf16x8(qrow + kb * 32 + 8 * lg) : zero_bf16x8();
  }
  if constexpr (ROPE) {
    // rotary embedding of the queries in registers: fragment kb holds elements
    // kb*32 + 8*lg + e, so the partner i + D/2 of element i (kb < NKB/2) sits at the same (lg, e)
    // of fragment kb + NKB/2; the result is rounded to bf16 as a stored rotated query would be
    constexpr int HKB = NKB / 2;
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      if (!rvalid[mb]) continue;
      const float* cs = a.rope_cs + (static_cast<long>(b) * a.T + node[mb]) * D;
#pragma unroll
      for (int kb = 0; kb < HKB; ++kb) {
        const float4* cp = reinterpret_cast<const float4*>(cs + kb * 32 + 8 * lg);
        const float4* sp = reinterpret_cast<const float4*>(cs + D / 2 + kb * 32 + 8 * lg);
        const float4 c0 = cp[0], c1 = cp[1], s0 = sp[0], s1 = sp[1];
        const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        uint4 lo = __builtin_bit_cast(uint4, qf[mb][kb]);
        uint4 hi = __builtin_bit_cast(uint4, qf[mb][kb + HKB]);
        uint32_t* lw = reinterpret_cast<uint32_t*>(&lo);
        uint32_t* hw = reinterpret_cast<uint32_t*>(&hi);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int sh = 16 * (e & 1);
          float x = bf16_to_f32(static_cast<uint16_t>(lw[e >> 1] >> sh));
          float y = bf16_to_f32(static_cast<uint16_t>(hw[e >> 1] >> sh));
          rope_rotate(cv[e], sv[e], x, y);
          lw[e >> 1] = (lw[e >> 1] & (0xffff0000u >> sh)) | (static_cast<uint32_t>(f32_to_bf16_rne(x)) << sh);
          hw[e >> 1] = (hw[e >> 1] & (0xffff0000u >> sh)) | (static_cast<uint32_t>(f32_to_bf16_rne(y)) << sh);
        }
        qf[mb][kb] = __builtin_bit_cast(bf16x8_t, lo);
        qf[mb][kb + HKB] = __builtin_bit_cast(bf16x8_t, hi);
      }
    }
  }

  // ---- the extra row: this lane's key of every tile and quarter of the head dim ----
  constexpr int XCH = D / 32;                   // 16-byte chunks per lane
  const int xkey = 16 * wave + 4 * lg + (mm & 3);
  int xoff[XR ? XCH : 1];                       // element offsets of those chunks inside a tile
  uint32_t qx[XR ? D / 8 : 1];                  // the query's bf16 pairs of the same chunks
  float xo[XR ? NDB : 1];                       // P V partial of output column db*16 + mm
  float xref = -INFINITY, xl = 0.f;             // reference (log2 domain) and row sum, per wave
  int xva[XR ? NDB : 1];                        // byte offsets of its transposed V reads
  if constexpr (XR) {
    // this wave's 16 keys: rows 16*wave.. of the tile, the block the matrix-core path reads as
    // (ks, hi) = (wave / 2, wave % 2)
    const int xv = v_frag_base<D>(lg, mm) + (wave >> 1) * 32 * D + (wave & 1) * 16 * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) xva[db] = (xv ^ (db << 4)) * 2;
    const int hqx = kvh * a.G + xrow_m % a.G;
    const uint16_t* qrow = a.q + ((static_cast<long>(b) * a.Hq + hqx) * a.T + xnode) * D;
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      // lanes of odd 16-lane rows take the chunks in pair-swapped order: the lanes that one LDS
      // cycle serves then hit distinct bank groups (a probe of the bank-conflict counter read
      // zero this way, and two-way conflicts for orders set by the key)
      const int c = XCH * (mm >> 2) + (i ^ (lg & 1 & (XCH - 1)));
      xoff[i] = tile_elem<D>(xkey, c);
      uint4 v = has_x ? *reinterpret_cast<const uint4*>(qrow + c * 8) : make_uint4(0, 0, 0, 0);
      if constexpr (ROPE) {
        if (has_x) {
          // rotate against the partner half of the head dim, as the other rows are rotated
          constexpr int HC = D / 16;   // chunks per half
          const uint4 pv = *reinterpret_cast<const uint4*>(qrow + (c ^ HC) * 8);
          const float* cs = a.rope_cs + (static_cast<long>(b) * a.T + xnode) * D + (c & (HC - 1)) * 8;
          uint32_t* ow = reinterpret_cast<uint32_t*>(&v);
          const uint32_t* pw = reinterpret_cast<const uint32_t*>(&pv);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int sh = 16 * (e & 1);
            const float own = bf16_to_f32(static_cast<uint16_t>(ow[e >> 1] >> sh));
            const float par = bf16_to_f32(static_cast<uint16_t>(pw[e >> 1] >> sh));
            float x = c < HC ? own : par, y = c < HC ? par : own;
            rope_rotate(cs[e], cs[D / 2 + e], x, y);
            const float r = c < HC ? x : y;
            ow[e >> 1] = (ow[e >> 1] & (0xffff0000u >> sh)) | (static_cast<uint32_t>(f32_to_bf16_rne(r)) << sh);
          }
        }
      }
      qx[4 * i] = v.x;
      qx[4 * i + 1] = v.y;
      qx[4 * i + 2] = v.z;
      qx[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) xo[db] = 0.f;
  }

  float mrow[NMB];
  float mthr[NMB];   // mrow + 8: the reference is raised past this
  float mneg[NMB];   // -mrow, or 0 before the first visible column: the exponent's offset
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    mrow[mb] = -INFINITY;
    mthr[mb] = -INFINITY;
    mneg[mb] = 0.f;
  }
  // Per-lane LDS offsets of the K and V fragment reads, fixed for every tile (the XOR of the
  // swizzle cannot go into the instructions' offset field), and the row blocks' threshold and
  // exponent offset kept beside the reference: 18 fewer vector instructions per tile and wave
  // in the 4-wave form (70B layer 1.19-1.23 -> 1.17 ms, Llama-8B shape 19.4-20.8 -> 18.7-19.4
  // us).  The extra-row kernel, near the register limit, recomputes them per tile instead:
  // holding them measured 102-103 -> 106-107 us on the 33B shape.
  int kaddr[XR ? 1 : NKB], vaddr[XR ? 1 : NDB];
  if constexpr (!XR) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) kaddr[kb] = (k_frag_base<D>(lg, mm) ^ (kb << 5)) * 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db) vaddr[db] = (v_frag_base<D>(lg, mm) ^ (db << 4)) * 2;
  }
  // row sums of the (bf16) probabilities, accumulated on the matrix cores: P^T times a block of
  // ones gives every lane the sum of its own query row in all four entries
  f32x4_t lacc[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) lacc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  f32x4_t oacc[NMB][NDB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[mb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // One pipeline step: wait for tile t in (Kc, Vc), start tile tn into (Kn, Vn), compute tile t.
  auto step = [&](const uint16_t* Kc, const uint16_t* Vc, uint16_t* Kn, uint16_t* Vn) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part of tile t has landed
    __syncthreads();                                    // everyone's part; the other buffer is free
    const bool is_tree = t >= np;
    long row0;
    int nvalid;
    tile_rows(t, row0, nvalid);
    const bool full = !is_tree && nvalid == kKvTile;
    // visible columns of this lane's two rows: the staged mask word (tree tiles) and the valid
    // rows of the tile; read from LDS, so nothing here waits for the next tile's loads
    const uint64_t vmask = nvalid >= 64 ? ~0ull : ((1ull << nvalid) - 1ull);
    uint64_t mw[NMB];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) mw[mb] = vmask;
    if (is_tree) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) mw[mb] &= s_mask[buf][wave * RPW + mb * 16 + mm];
    }
    // the extra row's visible keys: those below xlim that its mask word (tree tiles) selects
    uint64_t xw = 0ull;
    int xlim = 0;
    if constexpr (XR) {
      xw = is_tree ? s_mask[buf][ROWS] : ~0ull;
      xlim = has_x ? nvalid : 0;
    }
    const int tn = next_active(t + 1);
    if (tn < t_end) {
      long nrow0;
      int nnvalid;
      tile_rows(tn, nrow0, nnvalid);
      issue_tile<D, NW>(a.kc, a.vc, kvbase + nrow0, nnvalid, Kn, Vn, wave, voff, stream);
      if (tn >= np) {
        issue_mask<RPW>(a.mask, a.W, tn - np, mrow_node, s_mask[buf ^ 1], wave, lane);
        if (has_x) issue_xmask(a.mask, a.W, tn - np, xnode, &s_mask[buf ^ 1][ROWS], wave, lane);
      }
    }
    if (!wave_active) {
      t = tn;
      buf ^= 1;
      return;
    }

    // ---- scores S^T = K Q^T ----
    f32x4_t sacc[NMB][4];
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) sacc[mb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int kb_base = k_frag_base<D>(lg, mm);
    if constexpr (XR) asm volatile("" : "+v"(kb_base));   // opaque: addresses rebuilt per read
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int ko = XR ? ((kb_base ^ (kb << 5)) + cb * 16 * D) * 2 : kaddr[XR ? 0 : kb] + cb * 32 * D;
        const bf16x8_t kf = lds_read16(reinterpret_cast<const uint16_t*>(
            reinterpret_cast<const char*>(Kc) + ko));
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) sacc[mb][cb] = mfma16x16x32(kf, qf[mb][kb], sacc[mb][cb]);
      }
    }
    // the extra row's score of this lane's key, summed over the four quarters of the head dim
    // by rotations of 8 and then 4 inside the 16-lane row (commutative pairs: equal bits)
    float xs = 0.f;
    if constexpr (XR) {
      float s0 = 0.f, s1 = 0.f;
#pragma unroll
      for (int i = 0; i < XCH; ++i) {
        const uint4 kv = *reinterpret_cast<const uint4*>(Kc + xoff[i]);
        s0 = dot2_bf16(kv.x, qx[4 * i], s0);
        s1 = dot2_bf16(kv.y, qx[4 * i + 1], s1);
        s0 = dot2_bf16(kv.z, qx[4 * i + 2], s0);
        s1 = dot2_bf16(kv.w, qx[4 * i + 3], s1);
      }
      xs = s0 + s1;
      xs += dpp_f32<0x128>(xs);
      xs += dpp_f32<0x124>(xs);
    }

    // ---- mask, online softmax (log2 domain), P as the B operand of the second product.
    //      The running max is raised lazily: p = 2^(s*scale - m) with s*scale <= m + 8, so the
    //      rescale of O and l (exact either way) runs only when the max grows by more than 8. ----
    uint32_t pb[NMB][2][4];   // [mb][ks][dword] packed bf16 pairs
#pragma unroll
    for (int mb = 0; mb < NMB; ++mb) {
      float sv[4][4];
      if (full) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int j = 0; j < 4; ++j) sv[cb][j] = sacc[mb][cb][j];
      } else {
        // bits of columns cb*16 + 4*lg + j, j = 0..3, at bit 4*cb + j
        const uint64_t sh = mw[mb] >> (4 * lg);
        const uint32_t bits = static_cast<uint32_t>((sh & 0xFull) | ((sh >> 12) & 0xF0ull) |
                                                    ((sh >> 24) & 0xF00ull) | ((sh >> 36) & 0xF000ull));
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            sv[cb][j] = ((bits >> (4 * cb + j)) & 1u) ? sacc[mb][cb][j] : -INFINITY;
      }
      float mx = sv[0][0];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sv[cb][j]);
      // A row's maximum exceeds its reference + 8 only if the maximum of one of its four lanes
      // does (scaling is monotonic), so the cross-lane maximum is taken only when some lane of
      // the wave sees such a column: rare after the first tiles.
      const float thr = XR ? mrow[mb] + 8.f : mthr[mb];
      if (__builtin_amdgcn_ballot_w64(mx * a.sl2 > thr) != 0ull) {
        mx = xor32_max(xor16_max(mx));
        const float mxs = mx * a.sl2;
        if (mxs > thr) {                              // raise the reference
          const float alpha = exp2f(mrow[mb] - mxs);
          mrow[mb] = mxs;
          mthr[mb] = mxs + 8.f;
          mneg[mb] = -mxs;
#pragma unroll
          for (int j = 0; j < 4; ++j) lacc[mb][j] *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int j = 0; j < 4; ++j) oacc[mb][db][j] *= alpha;
        }
      }
      const float nm = XR ? (mrow[mb] == -INFINITY ? 0.f : -mrow[mb]) : mneg[mb];
      float pr[4][4];
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // the hardware exp2 (v_exp_f32): results below 2^-126 flush to zero, which cannot
          // matter next to the row's largest term (>= 1 against the running reference)
          pr[cb][j] = __builtin_amdgcn_exp2f(fmaf(sv[cb][j], a.sl2, nm));
        }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        pb[mb][ks][0] = pack_bf16x2(pr[2 * ks][0], pr[2 * ks][1]);
        pb[mb][ks][1] = pack_bf16x2(pr[2 * ks][2], pr[2 * ks][3]);
        pb[mb][ks][2] = pack_bf16x2(pr[2 * ks + 1][0], pr[2 * ks + 1][1]);
        pb[mb][ks][3] = pack_bf16x2(pr[2 * ks + 1][2], pr[2 * ks + 1][3]);
      }
    }

    // ---- the extra row's online softmax over this wave's 16 keys ----
    uint32_t xp01 = 0u, xp23 = 0u;   // P of keys 4*lg + 0..3 of the wave's 16, as bf16 pairs
    if constexpr (XR) {
      xs = (xkey < xlim && ((xw >> xkey) & 1ull)) ? xs : -INFINITY;
      // the reference (one per wave) is raised when some key of the wave's 16 passes it by 8
      if (__builtin_amdgcn_ballot_w64(xs * a.sl2 > xref + 8.f) != 0ull) {
        float mx = fmaxf(xs, dpp_f32<0xB1>(xs));   // quad_perm [1,0,3,2]
        mx = fmaxf(mx, dpp_f32<0x4E>(mx));         // quad_perm [2,3,0,1]
        mx = xor32_max(xor16_max(mx));
        const float mxs = mx * a.sl2;
        const float alpha = exp2f(xref - mxs);
        xref = mxs;
        xl *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) xo[db] *= alpha;
      }
      const float nm = xref == -INFINITY ? 0.f : -xref;
      const float p = __builtin_amdgcn_exp2f(fmaf(xs, a.sl2, nm));
      xp01 = pack_bf16x2(dpp_f32<0x00>(p), dpp_f32<0x55>(p));
      xp23 = pack_bf16x2(dpp_f32<0xAA>(p), dpp_f32<0xFF>(p));
      // row sum of the same bf16 values that weight V
      xl = dot2_bf16(xp23, 0x3F803F80u, dot2_bf16(xp01, 0x3F803F80u, xl));
    }

    // ---- O^T += V^T P^T; contraction index 8*lg+e <-> tile column
    //      ks*32 + (e < 4 ? 4*lg + e : 16 + 4*lg + e - 4), matching the score layout ----
    int vb_base = v_frag_base<D>(lg, mm);
    if constexpr (XR) asm volatile("" : "+v"(vb_base));
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int vo = XR ? ((vb_base ^ (db << 4)) + ks * 32 * D) * 2 : vaddr[XR ? 0 : db] + ks * 64 * D;
        const uint16_t* vp = reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(Vc) + vo);
        const s16x4_t v0 = lds_read_tr(vp);
        const s16x4_t v1 = lds_read_tr(vp + 16 * D);
        typedef __attribute__((ext_vector_type(8))) short s16x8_t;
        const s16x8_t vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, vv);
#pragma unroll
        for (int mb = 0; mb < NMB; ++mb) {
          const uint4 bv = make_uint4(pb[mb][ks][0], pb[mb][ks][1], pb[mb][ks][2], pb[mb][ks][3]);
          oacc[mb][db] = mfma16x16x32(va, __builtin_bit_cast(bf16x8_t, bv), oacc[mb][db]);
        }
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int mb = 0; mb < NMB; ++mb) {
        const uint4 bv = make_uint4(pb[mb][ks][0], pb[mb][ks][1], pb[mb][ks][2], pb[mb][ks][3]);
        lacc[mb] = mfma16x16x32(ones, __builtin_bit_cast(bf16x8_t, bv), lacc[mb]);
      }
    }
    if constexpr (XR) {
      // the transposed V read of this wave's 16 keys: columns 4*lg + 0..3 of output column
      // db*16 + mm, the same layout as the matrix-core operand
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint2 w = __builtin_bit_cast(uint2, lds_read_tr(reinterpret_cast<const uint16_t*>(
                                                      reinterpret_cast<const char*>(Vc) + xva[db])));
        xo[db] = dot2_bf16(w.y, xp23, dot2_bf16(w.x, xp01, xo[db]));
      }
    }
    t = tn;
    buf ^= 1;
  };

  // two copies of the step, one per buffer pair: with the buffers fixed per copy every LDS
  // offset is a constant (a single body with a runtime buffer index measured 10-14 % slower)
  while (t < t_end) {
    step(K0, V0, K1, V1);
    if (t >= t_end) break;
    step(K1, V1, K0, V0);
  }

  if constexpr (XR) {
    // ---- the extra row: each wave's 16-key state, then the merge in wave order ----
    const float lw = xor32_sum(xor16_sum(xl));
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const float v = xor32_sum(xor16_sum(xo[db]));
      if (lg == 0) s_xo[wave][db * 16 + mm] = v;
    }
    if (lane == 0) s_xml[wave] = make_float2(xref, lw);
    __syncthreads();
    if (has_x && tid < D) {
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) mx = fmaxf(mx, s_xml[w].x);
      const float mu = mx == -INFINITY ? 0.f : mx;
      float o = 0.f, l = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = exp2f(s_xml[w].x - mu);
        o += s_xo[w][tid] * f;
        l += s_xml[w].y * f;
      }
      if (a.splits == 1) {
        const int hq = kvh * a.G + xrow_m % a.G;
        a.out[((static_cast<long>(b) * a.Hq + hq) * a.T + xnode) * D + tid] = f32_to_bf16_rne(o * (1.f / l));
      } else {
        const long pr = ((static_cast<long>(split) * a.B + b) * a.Hkv + kvh) * a.Mpad + xrow_m;
        a.o_part[pr * D + tid] = o;
        if (tid == 0) a.ml_part[pr] = make_float2(mx, l);
      }
    }
  }

  // ---- finish: full row sums, then the output or this split's partial ----
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const float l = lacc[mb][0];
    const int m = qt * ROWS + wave * RPW + mb * 16 + mm;
    if (!rvalid[mb]) continue;
    if (a.splits == 1) {
      const float inv = 1.f / l;
      const int hq = kvh * a.G + m % a.G;
      uint16_t* orow = a.out + ((static_cast<long>(b) * a.Hq + hq) * a.T + node[mb]) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        uint2 w;
        w.x = pack_bf16x2(oacc[mb][db][0] * inv, oacc[mb][db][1] * inv);
        w.y = pack_bf16x2(oacc[mb][db][2] * inv, oacc[mb][db][3] * inv);
        *reinterpret_cast<uint2*>(orow + db * 16 + 4 * lg) = w;
      }
    } else {
      const long pr = ((static_cast<long>(split) * a.B + b) * a.Hkv + kvh) * a.Mpad + m;
      float* op = a.o_part + pr * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<float4*>(op + db * 16 + 4 * lg) =
            make_float4(oacc[mb][db][0], oacc[mb][db][1], oacc[mb][db][2], oacc[mb][db][3]);
      if (lg == 0) a.ml_part[pr] = make_float2(mrow[mb], l);
    }
  }
}

// Merge of the K/V splits, in split order.  One wave per query row; every load is issued before
// any is used (at most kMaxSplits splits).
template <int D>
__global__ __launch_bounds__(256) void tree_attn_combine(const float* __restrict__ o_part,
                                                         const float2* __restrict__ ml,
                                                         uint16_t* __restrict__ out, int B, int Hq,
                                                         int Hkv, int T, int G, int M, int Mpad,
                                                         int splits) {
  constexpr int PER = D / 64;   // values per lane
  const long rowid = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);   // over B*Hkv*M
  if (rowid >= static_cast<long>(B) * Hkv * M) return;
  const int lane = threadIdx.x & 63;
  const int m = static_cast<int>(rowid % M);
  const long bk = rowid / M;       // b * Hkv + kvh
  const long stride = static_cast<long>(B) * Hkv * Mpad;
  float2 v[kMaxSplits];
  float o[kMaxSplits][PER];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (s < splits) {
      const long pr = s * stride + bk * Mpad + m;
      v[s] = ml[pr];
#pragma unroll
      for (int e = 0; e < PER; ++e) o[s][e] = o_part[pr * D + e * 64 + lane];
    } else {
      v[s] = make_float2(-INFINITY, 0.f);
#pragma unroll
      for (int e = 0; e < PER; ++e) o[s][e] = 0.f;
    }
  }
  float mx = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) mx = fmaxf(mx, v[s].x);
  float l = 0.f, acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) {
    if (v[s].y == 0.f) continue;
    const float f = exp2f(v[s].x - mx);
    l += v[s].y * f;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] += o[s][e] * f;
  }
  const int b = static_cast<int>(bk / Hkv), kvh = static_cast<int>(bk % Hkv);
  const int node = m / G, hq = kvh * G + m % G;
  uint16_t* orow = out + ((static_cast<long>(b) * Hq + hq) * T + node) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[e * 64 + lane] = f32_to_bf16_rne(acc[e] / l);
}

// fp32 path: one wave per (b, q head, node).  Columns go 64 at a time: lanes compute one score
// each (the lane's K row), the wave updates the online softmax, then lanes switch to the head
// dim and accumulate the chunk's p-weighted V rows (coalesced V loads).
__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_down(v, off);
  return __shfl(v, 0);
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// D is a template parameter so that a lane's whole K row (D/4 16-byte loads) and every V load
// of a batch are issued before any is used
template <int D>
__global__ __launch_bounds__(64) void tree_attn_f32(const float* __restrict__ q,
                                                    const float* __restrict__ kc,
                                                    const float* __restrict__ vc,
                                                    const int32_t* __restrict__ prefix_len,
                                                    const uint64_t* __restrict__ mask, float* out,
                                                    long lcap, int Hq, int Hkv, int T, int W,
                                                    float sl2, int Lmax,
                                                    const float* __restrict__ rope_cs) {
  __shared__ float s_q[128];
  __shared__ float s_p[64];
  const long u = blockIdx.x;
  const int i = static_cast<int>(u % T);
  const int hq = static_cast<int>((u / T) % Hq);
  const int b = static_cast<int>(u / (static_cast<long>(T) * Hq));
  const int g = hq / (Hq / Hkv);
  const int lane = threadIdx.x;
  const int L = min(max(prefix_len[b], 0), Lmax);
  const long base = (static_cast<long>(b) * Hkv + g) * lcap;
  const float* qr = q + u * D;
  for (int d = lane; d < D; d += 64) s_q[d] = qr[d];
  __syncthreads();
  if (rope_cs) {                           // rotary embedding of the query at its position
    const int half = D / 2;
    if (lane < half) {
      const float* cs = rope_cs + (static_cast<long>(b) * T + i) * D;
      float x = s_q[lane], y = s_q[lane + half];
      rope_rotate(cs[lane], cs[half + lane], x, y);
      s_q[lane] = x;
      s_q[lane + half] = y;
    }
    __syncthreads();
  }
  float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
  const long ncols = static_cast<long>(L) + T;
  for (long c0 = 0; c0 < ncols; c0 += 64) {
    const long j = c0 + lane;
    const bool inr = j < ncols;
    // the mask word and the key row go out together (a column past the range reads the first
    // word and the first row, always valid); a masked-out tree column is computed and dropped
    const int t = inr && j >= L ? static_cast<int>(j - L) : 0;
    const uint64_t mw = mask[static_cast<long>(i) * W + t / 64];
    float s = -INFINITY;
    const float4* kr = reinterpret_cast<const float4*>(kc + (base + (inr ? j : 0)) * D);
    float4 kv[D / 4];
#pragma unroll
    for (int d4 = 0; d4 < D / 4; ++d4) kv[d4] = kr[d4];
    const bool vis = inr && (j < L || ((mw >> (t % 64)) & 1ull));
    {
      float acc = 0.f;
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4) {
        acc = fmaf(s_q[4 * d4], kv[d4].x, acc);
        acc = fmaf(s_q[4 * d4 + 1], kv[d4].y, acc);
        acc = fmaf(s_q[4 * d4 + 2], kv[d4].z, acc);
        acc = fmaf(s_q[4 * d4 + 3], kv[d4].w, acc);
      }
      if (vis) s = acc * sl2;
    }
    const float mnew = fmaxf(m, wave_max_f32(s));
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    const float p = vis ? exp2f(s - muse) : 0.f;
    const float alpha = exp2f(m - muse);
    l = l * alpha + wave_sum_f32(p);
    m = mnew;
    s_p[lane] = p;
    __syncthreads();
    o0 *= alpha;
    o1 *= alpha;
    // p-weighted V rows, 8 rows' loads in flight before their FMAs (same order of summation;
    // an invisible column has p = 0 and a finite V row, so it adds nothing)
    const int nc = static_cast<int>(min(static_cast<long>(64), ncols - c0));
    int cc = 0;
    for (; cc + 8 <= nc; cc += 8) {
      float v0[8], v1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* vr = vc + (base + c0 + cc + u) * D;
        v0[u] = lane < D ? vr[lane] : 0.f;
        v1[u] = lane + 64 < D ? vr[lane + 64] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float pc = s_p[cc + u];
        o0 = fmaf(pc, v0[u], o0);
        o1 = fmaf(pc, v1[u], o1);
      }
    }
    for (; cc < nc; ++cc) {
      const float pc = s_p[cc];
      const float* vr = vc + (base + c0 + cc) * D;
      if (lane < D) o0 = fmaf(pc, vr[lane], o0);
      if (lane + 64 < D) o1 = fmaf(pc, vr[lane + 64], o1);
    }
    __syncthreads();
  }
  float* orow = out + u * D;
  if (lane < D) orow[lane] = o0 / l;
  if (lane + 64 < D) orow[lane + 64] = o1 / l;
}

static long wg_target_from_env() {
  const char* v = getenv("MEDUSA_ATTN_WG_TARGET");
  const long t = v ? atol(v) : 256;
  return t >= 1 && t <= 4096 ? t : 256;
}

AttnPlan attn_plan(int dtype, int B, int Hq, int Hkv, int T, int D, int max_prefix_len) {
  AttnPlan p{};
  p.G = Hq / Hkv;
  p.M = p.G * T;
  p.rows = kAttnRows;
  p.qtiles = (p.M + kAttnRows - 1) / kAttnRows;
  p.splits = 1;
  if (dtype == 1) {
    // 144-row work-groups (nine waves of one row block) when they take fewer query tiles than
    // 128-row ones, leave enough work-groups that the K/V range needs no split, and keep the grid
    // in the one-block-per-wave range (and the extra rows below do not apply).  At 118-120
    // VGPRs only one nine-wave work-group fits on a CU; still, on the 33B shape (129 rows per kv
    // head: a 128-row tile and a 1-row tile that streams the whole K/V range again) attention
    // went from 157.5 to 137.8 us.  Forcing two per CU
    // (five waves per SIMD: 96 VGPRs, 3 spilled, with the buffer-load tiles) took 138-140 us
    // against 135.5-136.2 on the same GPU.  On the Llama-8B shape (260 rows, split grid) the
    // attention kernel gained 1 us and the merge of 16 splits instead of 10 lost 2.  Setting
    // MEDUSA_ATTN_ROWS to 128 or 144 forces the choice where it is possible.
    static const int forced_rows = [] { const char* v = getenv("MEDUSA_ATTN_ROWS"); return v ? atoi(v) : 0; }();
    // extra rows on the vector units: -1 (unset) one or two where the grid needs no split, 0
    // never, 1 wherever the rows fit
    static const int xrow_mode = [] { const char* v = getenv("MEDUSA_ATTN_XROW"); return v ? atoi(v) : -1; }();
    static const long target = wg_target_from_env();
    // rows past the full 128-row tiles, one per tile at most: the 4-wave kernel takes them as
    // extra rows instead of a query tile of their own.  An extra row costs its work-group about a
    // fifth of its time (70B-layer shape: 56 extra rows per kv head took 1.46-1.52 ms against
    // 1.24-1.29 ms with a 56-row query tile), so by default only one or two rows are taken
    // (33B shape: one row, 135 -> 103 us against the nine-wave 144-row form).
    const int q128 = p.M / kAttnRows, rem = p.M - q128 * kAttnRows;
    const bool x_fits = q128 >= 1 && rem >= 1 && rem <= q128;
    const bool x_use = x_fits && (xrow_mode == 1 || (xrow_mode != 0 && forced_rows == 0 && rem <= 2 &&
                                                     static_cast<long>(B) * Hkv * q128 >= target));
    if (x_use) {
      p.qtiles = q128;
      p.xrem = rem;
    } else {
      const int q144 = (p.M + kAttnRowsWide - 1) / kAttnRowsWide;
      const bool small_grid = static_cast<long>(B) * Hkv * p.qtiles < kAttnTwoBlockUnits;
      const bool unsplit = static_cast<long>(B) * Hkv * q144 >= target;
      const bool wide = forced_rows == kAttnRowsWide ? small_grid
                      : forced_rows == kAttnRows ? false : small_grid && unsplit && q144 < p.qtiles;
      if (wide) {
        p.rows = kAttnRowsWide;
        p.qtiles = q144;
      }
    }
    const long units = static_cast<long>(B) * Hkv * p.qtiles;
    const int ntiles = (max_prefix_len + kKvTile - 1) / kKvTile + (T + kKvTile - 1) / kKvTile;
    // too few units to cover the CUs: split the K/V range until the grid reaches the target
    // (256 work-groups, one per CU, unless MEDUSA_ATTN_WG_TARGET says otherwise), keeping at
    // least two tiles per split
    if (units < target) {
      long s = target / units;
      s = s < ntiles / 2 ? s : ntiles / 2;
      s = s < kMaxSplits ? s : kMaxSplits;
      p.splits = s < 1 ? 1 : static_cast<int>(s);
    }
  }
  p.nmb = p.xrem > 0 || (p.rows == kAttnRows &&
                         static_cast<long>(B) * Hkv * p.qtiles * p.splits >= kAttnTwoBlockUnits) ? 2 : 1;
  p.mpad = p.xrem > 0 ? p.M : p.qtiles * p.rows;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) & ~size_t(255); return o; };
  const size_t rows = static_cast<size_t>(p.splits) * B * Hkv * p.mpad;
  p.ws_o = take(p.splits > 1 ? rows * D * sizeof(float) : 0);
  p.ws_ml = take(p.splits > 1 ? rows * sizeof(float2) : 0);
  p.total = off;
  return p;
}

hipError_t launch_tree_attention(const void* q, const void* kc, const void* vc, int dtype,
                                 const int32_t* prefix_len, int max_prefix_len, long lcap,
                                 const uint64_t* mask, int B, int Hq, int Hkv, int T, int D,
                                 float scale, void* out, char* ws, hipStream_t s,
                                 const float* rope_cs) {
  const AttnPlan P = attn_plan(dtype, B, Hq, Hkv, T, D, max_prefix_len);
  const int W = (T + 63) / 64;
  const float sl2 = scale * 1.4426950408889634f;
  if (dtype == 0) {
    hook_before(K_ATTENTION, s);
    const unsigned g = static_cast<unsigned>(static_cast<long>(B) * Hq * T);
    if (D == 128)
      tree_attn_f32<128><<<g, 64, 0, s>>>(
          static_cast<const float*>(q), static_cast<const float*>(kc), static_cast<const float*>(vc),
          prefix_len, mask, static_cast<float*>(out), lcap, Hq, Hkv, T, W, sl2, max_prefix_len, rope_cs);
    else
      tree_attn_f32<64><<<g, 64, 0, s>>>(
          static_cast<const float*>(q), static_cast<const float*>(kc), static_cast<const float*>(vc),
          prefix_len, mask, static_cast<float*>(out), lcap, Hq, Hkv, T, W, sl2, max_prefix_len, rope_cs);
    hook_after(K_ATTENTION, s);
    return hipGetLastError();
  }
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(kc);
  a.vc = static_cast<const uint16_t*>(vc);
  a.prefix_len = prefix_len;
  a.mask = mask;
  a.out = static_cast<uint16_t*>(out);
  a.o_part = reinterpret_cast<float*>(ws + P.ws_o);
  a.ml_part = reinterpret_cast<float2*>(ws + P.ws_ml);
  a.lcap = lcap;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.T = T;
  a.W = W;
  a.G = P.G;
  a.M = P.M;
  a.Mpad = P.mpad;
  a.xrem = P.xrem;
  a.xbase = P.qtiles * kAttnRows;
  a.qtiles = P.qtiles;
  a.splits = P.splits;
  a.nwork = B * Hkv * P.qtiles * P.splits;
  a.sl2 = sl2;
  a.Lmax = max_prefix_len;
  a.rope_cs = rope_cs;
  const unsigned grid = static_cast<unsigned>(((a.nwork + 7) / 8) * 8);
  hook_before(K_ATTENTION, s);
#define MEDUSA_ATTN_LAUNCH(NMB_, NW_, XR_)                                                   \
  if (rope_cs) {                                                                          \
    if (D == 128) tree_attn_bf16<128, true, NMB_, NW_, XR_><<<grid, NW_ * 64, 0, s>>>(a);  \
    else tree_attn_bf16<64, true, NMB_, NW_, XR_><<<grid, NW_ * 64, 0, s>>>(a);            \
  } else {                                                                                \
    if (D == 128) tree_attn_bf16<128, false, NMB_, NW_, XR_><<<grid, NW_ * 64, 0, s>>>(a); \
    else tree_attn_bf16<64, false, NMB_, NW_, XR_><<<grid, NW_ * 64, 0, s>>>(a);           \
  }
  if (P.xrem > 0) {
    MEDUSA_ATTN_LAUNCH(2, 4, true)
  } else if (P.rows == kAttnRowsWide) {
    MEDUSA_ATTN_LAUNCH(1, 9, false)
  } else if (P.nmb == 1) {
    MEDUSA_ATTN_LAUNCH(1, 8, false)
  } else {
    MEDUSA_ATTN_LAUNCH(2, 4, false)
  }
#undef MEDUSA_ATTN_LAUNCH
  hook_after(K_ATTENTION, s);
  if (P.splits > 1) {
    hook_before(K_ATTN_COMBINE, s);
    const unsigned cgrid = static_cast<unsigned>((static_cast<long>(B) * Hkv * P.M + 3) / 4);
    if (D == 128)
      tree_attn_combine<128><<<cgrid, 256, 0, s>>>(a.o_part, a.ml_part, a.out, B, Hq, Hkv, T, P.G,
                                                   P.M, a.Mpad, P.splits);
    else
      tree_attn_combine<64><<<cgrid, 256, 0, s>>>(a.o_part, a.ml_part, a.out, B, Hq, Hkv, T, P.G,
                                                  P.M, a.Mpad, P.splits);
    hook_after(K_ATTN_COMBINE, s);
  }
  return hipGetLastError();
}

}  // namespace medusa
