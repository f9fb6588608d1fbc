// Rotary embedding of the tree tokens at their position ids, ahead of tree attention.
//
// Wiblog "Medusa multi-head speculative decoding", tree-attention section: besides the mask, the
// position encoding must give every tree token its correct position index: prefix_len + depth,
// the position it has when its own path is decoded one token at a time (build_tree's
// position_ids).  The encoding is the rotary one of the LLaMA-family models: dimension i < D/2
// turns with i + D/2 by the angle pos * base^(-2i/D).  The prefix keys in the cache were rotated
// when they were written; this kernel rotates the tree tokens' queries (into a buffer) and their
// key rows in the cache (in place), rounding to the storage type (nearest even for bf16).
//
// The rows of one tree node share their angles, so a work-group takes one (sequence, node) and a
// chunk of up to 32 of its rows (q heads, then kv heads), 8 per wave.  A lane owns 4 consecutive
// pairs (i, i + D/2) of one row, so a wave instruction covers 64 / (D/8) rows with 8-byte (bf16)
// or 16-byte (fp32) accesses.  Every wave issues its rows' loads first; meanwhile wave 0 forms
// the node's D/2 angles and their cos/sin into LDS.  An angle is formed and reduced to [-pi, pi]
// in fp64 (at position 8192 an fp32 angle would already be off by ~5e-4 rad), from inverse
// frequencies base^(-2i/D) computed once on the host in fp64; sin/cos and the rotation run in
// fp32.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace medusa {

constexpr int kRopeThreads = 256;
constexpr int kRopeRowsPerWg = 32;            // 8 rows per wave
constexpr unsigned kRopeMaxGrid = 65535;

struct RopeKArgs {
  RopeArgs a;
  double inv[64];                             // base^(-2i/D), i < D/2
};

// 4 consecutive elements at element offset i (a multiple of 4)
template <bool BF16>
__device__ __forceinline__ float4 rope_load4(const void* p, long i) {
  if (BF16) {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    return make_float4(bf16_to_f32(static_cast<uint16_t>(v.x)), bf16_to_f32(static_cast<uint16_t>(v.x >> 16)),
                       bf16_to_f32(static_cast<uint16_t>(v.y)), bf16_to_f32(static_cast<uint16_t>(v.y >> 16)));
  }
  return *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
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

template <bool BF16>
__global__ __launch_bounds__(kRopeThreads) void rope_tree_kernel(RopeKArgs k) {
  const RopeArgs& a = k.a;
  __shared__ __align__(16) float s_cs[64];
  __shared__ __align__(16) float s_sn[64];
  const int half = a.D / 2;
  const int lpr = half / 4;                                  // lanes per row
  const int rpi = 64 / lpr;                                  // rows per wave instruction
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q4 = (lane % lpr) * 4;                           // this lane's first pair index
  const int R = a.Hq + a.Hkv;                                // rows of one node
  const int chunks = (R + kRopeRowsPerWg - 1) / kRopeRowsPerWg;
  const long items = static_cast<long>(a.B) * a.T * chunks;
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  for (long it = blockIdx.x; it < items; it += gridDim.x) {
    const int ch = static_cast<int>(it % chunks);
    const long bn = it / chunks;
    const int b = static_cast<int>(bn / a.T), n = static_cast<int>(bn % a.T);
    const int L = min(max(a.prefix_len[b], 0), a.Lmax);    // as tree attention reads it
    // this wave's 8 rows: rows ch*32 + wave*8 + g*rpi + lane/lpr, g < 8/rpi
    constexpr int kMaxG = 2;                               // 8 rows / rpi: 2 for D = 128, 1 for D = 64
    float4 x[kMaxG], y[kMaxG];
    long base[kMaxG];
    void* dst[kMaxG];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
      base[g] = -1;
      const int j = ch * kRopeRowsPerWg + wave * 8 + g * rpi + lane / lpr;
      if (g * rpi < 8 && j < R) {
        const void* src;
        if (j < a.Hq) {
          src = a.q;
          dst[g] = a.q_rot;
          base[g] = ((static_cast<long>(b) * a.Hq + j) * a.T + n) * a.D;
        } else {
          src = a.kc;
          dst[g] = a.kc;
          base[g] = ((static_cast<long>(b) * a.Hkv + (j - a.Hq)) * a.lcap + L + n) * a.D;
        }
        x[g] = rope_load4<BF16>(src, base[g] + q4);
        y[g] = rope_load4<BF16>(src, base[g] + q4 + half);
      }
    }
    __syncthreads();                                        // the last item's readers are done
    if (wave == 0 && lane < half) {
      const double ang = static_cast<double>(a.pos[bn]) * k.inv[lane];
      const float red = static_cast<float>(fma(-two_pi, rint(ang * inv_two_pi), ang));
      float sn, cs;
      sincosf(red, &sn, &cs);
      s_cs[lane] = cs;
      s_sn[lane] = sn;
    }
    __syncthreads();
    const float4 cs = *reinterpret_cast<const float4*>(s_cs + q4);
    const float4 sn = *reinterpret_cast<const float4*>(s_sn + q4);
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
      if (base[g] < 0) continue;
      const float4 xv = x[g], yv = y[g];
      rope_store4<BF16>(dst[g], base[g] + q4,
                        make_float4(fmaf(xv.x, cs.x, -(yv.x * sn.x)), fmaf(xv.y, cs.y, -(yv.y * sn.y)),
                                    fmaf(xv.z, cs.z, -(yv.z * sn.z)), fmaf(xv.w, cs.w, -(yv.w * sn.w))));
      rope_store4<BF16>(dst[g], base[g] + q4 + half,
                        make_float4(fmaf(xv.x, sn.x, yv.x * cs.x), fmaf(xv.y, sn.y, yv.y * cs.y),
                                    fmaf(xv.z, sn.z, yv.z * cs.z), fmaf(xv.w, sn.w, yv.w * cs.w)));
    }
  }
}

hipError_t launch_rope_tree(const RopeArgs& a, int dtype, hipStream_t s) {
  RopeKArgs k{};
  k.a = a;
  for (int i = 0; i < a.D / 2 && i < 64; ++i)
    k.inv[i] = pow(static_cast<double>(a.base), -2.0 * i / a.D);
  const int R = a.Hq + a.Hkv;
  const long items = static_cast<long>(a.B) * a.T * ((R + kRopeRowsPerWg - 1) / kRopeRowsPerWg);
  const unsigned grid = static_cast<unsigned>(items < kRopeMaxGrid ? items : kRopeMaxGrid);
  hook_before(K_ROPE, s);
  if (dtype == 1) rope_tree_kernel<true><<<grid, kRopeThreads, 0, s>>>(k);
  else rope_tree_kernel<false><<<grid, kRopeThreads, 0, s>>>(k);
  hook_after(K_ROPE, s);
  return hipGetLastError();
}

}  // namespace medusa
