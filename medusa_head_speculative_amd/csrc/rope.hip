// Rotary embedding of the tree tokens at their position ids, for tree attention.
//
// Wiblog "Medusa multi-head speculative decoding", tree-attention section: besides the mask, the
// position encoding must give every tree token its correct position index: prefix_len + depth,
// the position it has when its own path is decoded one token at a time (build_tree's
// position_ids).  The encoding is the rotary one of the LLaMA-family models: dimension i < D/2
// turns with i + D/2 by the angle pos * base^(-2i/D).  The prefix keys in the cache were rotated
// when they were written; this kernel rotates the tree tokens' key rows in the cache (in place),
// rounding to the storage type (nearest even for bf16), and writes every tree node's cos/sin to
// a table from which the attention kernel rotates the queries as it loads them.
//
// One wave per (sequence, node, chunk of kv heads): the rows of one node share the angles.  A lane
// owns 4 consecutive pairs (i, i + D/2) of one row, so a wave instruction covers 64 / (D/8) rows
// with 8-byte (bf16) or 16-byte (fp32) accesses, and a chunk is kRopeGroups such row groups, all
// loaded before the angles are formed.  Each lane forms the 4 angles it owns (no LDS, no
// barrier); the wave of the first chunk also writes the node's cos/sin.  An angle is formed and reduced to
// [-pi, pi] in fp64 (at position 8192 an fp32 angle would already be off by ~5e-4 rad), from
// inverse frequencies base^(-2i/D) computed once on the host in fp64; sin/cos and the rotation
// run in fp32.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace medusa {

constexpr int kRopeThreads = 256;
constexpr unsigned kRopeMaxGrid = 65535;
constexpr int kRopeGroups = 2;                // row groups of one wave, in flight at once

struct RopeKArgs {
  RopeArgs a;
  double inv[64];                             // base^(-2i/D), i < D/2
};

// 4 consecutive elements at element offset i (a multiple of 4), as raw bits (bf16: the low two
// words) so that every load of a thread is issued before any is converted
template <bool BF16>
__device__ __forceinline__ uint4 rope_load4(const void* p, long i) {
  if (BF16) {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    return make_uint4(v.x, v.y, 0u, 0u);
  }
  return *reinterpret_cast<const uint4*>(static_cast<const float*>(p) + i);
}
template <bool BF16>
__device__ __forceinline__ float4 rope_unpack4(uint4 v) {
  if (BF16)
    return make_float4(bf16_to_f32(static_cast<uint16_t>(v.x)), bf16_to_f32(static_cast<uint16_t>(v.x >> 16)),
                       bf16_to_f32(static_cast<uint16_t>(v.y)), bf16_to_f32(static_cast<uint16_t>(v.y >> 16)));
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
template <bool BF16>
__device__ __forceinline__ void rope_store4(void* p, long i, float4 v) {
  if (BF16) {
    uint2 w;
    w.x = static_cast<uint32_t>(f32_to_bf16_rne(v.x)) | (static_cast<uint32_t>(f32_to_bf16_rne(v.y)) << 16);
    w.y = static_cast<uint32_t>(f32_to_bf16_rne(v.z)) | (static_cast<uint32_t>(f32_to_bf16_rne(v.w)) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p) + i) = w;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p) + i) = v;
  }
}

__device__ __forceinline__ void rope_cs(double p, double inv, float& cs, float& sn) {
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  const double ang = p * inv;
  const float red = static_cast<float>(fma(-two_pi, rint(ang * inv_two_pi), ang));
  sincosf(red, &sn, &cs);
}

template <bool BF16>
__global__ __launch_bounds__(kRopeThreads) void rope_tree_kernel(RopeKArgs k) {
  const RopeArgs& a = k.a;
  const int half = a.D / 2;
  const int lpr = half / 4;                                  // lanes per row
  const int rpi = 64 / lpr;                                  // rows per wave instruction
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q4 = (lane % lpr) * 4;                           // this lane's first pair index
  const int rsub = lane / lpr;
  const int chunk = kRopeGroups * rpi;                      // kv heads per wave
  const int nch = (a.Hkv + chunk - 1) / chunk;
  const long units = static_cast<long>(a.B) * a.T * nch;
  for (long u = static_cast<long>(blockIdx.x) * 4 + wave; u < units; u += static_cast<long>(gridDim.x) * 4) {
    const long bn = u / nch;
    const int j0 = static_cast<int>(u % nch) * chunk;
    const int b = static_cast<int>(bn / a.T), n = static_cast<int>(bn % a.T);
    const int L = min(max(a.prefix_len[b], 0), a.Lmax);    // as tree attention reads it
    auto row_base = [&](int j) {                            // kv head j's tree row of this node
      return ((static_cast<long>(b) * a.Hkv + j) * a.lcap + L + n) * a.D;
    };
    {
      // every row group's loads go out before any is used; a lane past the last kv head loads
      // head 0's row (always valid) and stores nothing
      uint4 xr[kRopeGroups], yr[kRopeGroups];
      long base[kRopeGroups];
#pragma unroll
      for (int g = 0; g < kRopeGroups; ++g) {
        const int j = j0 + g * rpi + rsub;
        base[g] = row_base(j < a.Hkv ? j : 0);
        xr[g] = rope_load4<BF16>(a.kc, base[g] + q4);
        yr[g] = rope_load4<BF16>(a.kc, base[g] + q4 + half);
        if (j >= a.Hkv) base[g] = -1;
      }
      float c[4], s[4];
      const double p = static_cast<double>(a.pos[bn]);
#pragma unroll
      for (int e = 0; e < 4; ++e) rope_cs(p, k.inv[q4 + e], c[e], s[e]);
      if (j0 == 0 && rsub == 0 && a.cs_table) {               // cos/sin of this node for the queries
        float* t = a.cs_table + bn * 2 * half;
        *reinterpret_cast<float4*>(t + q4) = make_float4(c[0], c[1], c[2], c[3]);
        *reinterpret_cast<float4*>(t + half + q4) = make_float4(s[0], s[1], s[2], s[3]);
      }
#pragma unroll
      for (int g = 0; g < kRopeGroups; ++g) {
        if (base[g] < 0) continue;
        const float4 xv = rope_unpack4<BF16>(xr[g]), yv = rope_unpack4<BF16>(yr[g]);
        rope_store4<BF16>(a.kc, base[g] + q4,
                          make_float4(fmaf(xv.x, c[0], -(yv.x * s[0])), fmaf(xv.y, c[1], -(yv.y * s[1])),
                                      fmaf(xv.z, c[2], -(yv.z * s[2])), fmaf(xv.w, c[3], -(yv.w * s[3]))));
        rope_store4<BF16>(a.kc, base[g] + q4 + half,
                          make_float4(fmaf(xv.x, s[0], yv.x * c[0]), fmaf(xv.y, s[1], yv.y * c[1]),
                                      fmaf(xv.z, s[2], yv.z * c[2]), fmaf(xv.w, s[3], yv.w * c[3])));
      }
    }
  }
}

hipError_t launch_rope_tree(const RopeArgs& a, int dtype, hipStream_t s) {
  RopeKArgs k{};
  k.a = a;
  for (int i = 0; i < a.D / 2 && i < 64; ++i)
    k.inv[i] = pow(static_cast<double>(a.base), -2.0 * i / a.D);
  const int chunk = kRopeGroups * (64 / (a.D / 8));
  const long units = static_cast<long>(a.B) * a.T * ((a.Hkv + chunk - 1) / chunk);
  const long wgs = (units + 3) / 4;
  const unsigned grid = static_cast<unsigned>(wgs < kRopeMaxGrid ? wgs : kRopeMaxGrid);
  hook_before(K_ROPE, s);
  if (dtype == 1) rope_tree_kernel<true><<<grid, kRopeThreads, 0, s>>>(k);
  else rope_tree_kernel<false><<<grid, kRopeThreads, 0, s>>>(k);
  hook_after(K_ROPE, s);
  return hipGetLastError();
}

}  // namespace medusa
