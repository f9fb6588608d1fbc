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
// One wave per row (query row or cache key row), lane i < D/2 owns the pair (i, i + D/2).  The
// angle is formed and reduced to [-pi, pi] in fp64 (at position 8192 an fp32 angle would already
// be off by ~5e-4 rad), then sin/cos and the rotation run in fp32.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace medusa {

constexpr int kRopeThreads = 256;
constexpr unsigned kRopeMaxGrid = 2048;

template <bool BF16>
__device__ __forceinline__ float rope_load(const void* p, long i) {
  return BF16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}
template <bool BF16>
__device__ __forceinline__ void rope_store(void* p, long i, float v) {
  if (BF16) static_cast<uint16_t*>(p)[i] = f32_to_bf16_rne(v);
  else static_cast<float*>(p)[i] = v;
}

template <bool BF16>
__global__ __launch_bounds__(kRopeThreads) void rope_tree_kernel(RopeArgs a) {
  __shared__ double s_inv[64];
  const int half = a.D / 2;
  for (int i = threadIdx.x; i < half; i += kRopeThreads)
    s_inv[i] = pow(static_cast<double>(a.base), -2.0 * i / a.D);
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long qrows = static_cast<long>(a.B) * a.Hq * a.T;
  const long rows = qrows + static_cast<long>(a.B) * a.Hkv * a.T;
  const double two_pi = 6.283185307179586476925286766559;
  const double inv_two_pi = 0.15915494309189533576888376337251;
  for (long r = static_cast<long>(blockIdx.x) * 4 + wave; r < rows; r += static_cast<long>(gridDim.x) * 4) {
    const void* src;
    void* dst;
    long base;
    int b, n;
    if (r < qrows) {
      b = static_cast<int>(r / (static_cast<long>(a.Hq) * a.T));
      n = static_cast<int>(r % a.T);
      src = a.q;
      dst = a.q_rot;
      base = r * a.D;
    } else {
      const long r2 = r - qrows;
      b = static_cast<int>(r2 / (static_cast<long>(a.Hkv) * a.T));
      const int g = static_cast<int>((r2 / a.T) % a.Hkv);
      n = static_cast<int>(r2 % a.T);
      const int L = min(max(a.prefix_len[b], 0), a.Lmax);   // as tree attention reads it
      src = a.kc;
      dst = a.kc;
      base = ((static_cast<long>(b) * a.Hkv + g) * a.lcap + L + n) * a.D;
    }
    if (lane < half) {
      const double ang = static_cast<double>(a.pos[static_cast<long>(b) * a.T + n]) * s_inv[lane];
      const float red = static_cast<float>(fma(-two_pi, rint(ang * inv_two_pi), ang));
      float sn, cs;
      sincosf(red, &sn, &cs);
      const float x = rope_load<BF16>(src, base + lane);
      const float y = rope_load<BF16>(src, base + lane + half);
      rope_store<BF16>(dst, base + lane, fmaf(x, cs, -(y * sn)));
      rope_store<BF16>(dst, base + lane + half, fmaf(x, sn, y * cs));
    }
  }
}

hipError_t launch_rope_tree(const RopeArgs& a, int dtype, hipStream_t s) {
  const long rows = static_cast<long>(a.B) * (a.Hq + a.Hkv) * a.T;
  long blocks = (rows + 3) / 4;
  const unsigned grid = static_cast<unsigned>(blocks < kRopeMaxGrid ? blocks : kRopeMaxGrid);
  hook_before(K_ROPE, s);
  if (dtype == 1) rope_tree_kernel<true><<<grid, kRopeThreads, 0, s>>>(a);
  else rope_tree_kernel<false><<<grid, kRopeThreads, 0, s>>>(a);
  hook_after(K_ROPE, s);
  return hipGetLastError();
}

}  // namespace medusa
