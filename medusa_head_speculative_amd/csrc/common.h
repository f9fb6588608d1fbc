// Internal helpers shared by the HIP kernels of libmedusa_hip (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace medusa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// two floats -> packed bf16 pair (lo in bits 0..15), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Order-preserving map of a float to uint32 (larger float -> larger key; -0 < +0 is fine here).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// 64-bit selection key: larger value wins, equal values -> lower index wins.  -0 is keyed as +0
// (v + 0 turns -0 into +0), so the two zeros count as equal, as in a numeric comparison.  Key 0
// is below every real key (a real key has a float_key >= 0x007fffff in its high word).
__device__ __forceinline__ uint64_t sel_key(float v, uint32_t idx) {
  return (static_cast<uint64_t>(float_key(v + 0.0f)) << 32) | static_cast<uint64_t>(0xffffffffu - idx);
}
__device__ __forceinline__ uint32_t sel_key_index(uint64_t k) {
  return 0xffffffffu - static_cast<uint32_t>(k & 0xffffffffu);
}
__device__ __forceinline__ float sel_key_value(uint64_t k) {
  return key_float(static_cast<uint32_t>(k >> 32));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m);
  uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

// Wave-wide max of 64-bit keys with DPP row steps (xor 1, xor 2, rotate 4, rotate 8 inside each
// 16-lane row) and a 4-way scalar combine of the rows; every lane gets the result.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v)), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(static_cast<uint32_t>(v >> 32)), CTRL, 0xF, 0xF, false));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), l));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
  v = umax64(v, dpp_u64<0xB1>(v));    // quad_perm [1,0,3,2]
  v = umax64(v, dpp_u64<0x4E>(v));    // quad_perm [2,3,0,1]
  v = umax64(v, dpp_u64<0x124>(v));   // row_ror:4
  v = umax64(v, dpp_u64<0x128>(v));   // row_ror:8
  return umax64(umax64(readlane_u64(v, 0), readlane_u64(v, 16)),
                umax64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

// Max over a block of NT threads (NT a multiple of 64, <= 1024); every thread gets the result.
// `scratch` holds NT/64 entries.  Contains __syncthreads().
template <int NT>
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* scratch) {
  v = wave_max_u64(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) scratch[w] = v;
  __syncthreads();
  uint64_t r = scratch[0];
#pragma unroll
  for (int i = 1; i < NT / kWave; ++i) r = scratch[i] > r ? scratch[i] : r;
  __syncthreads();
  return r;
}

// Combine a value with the one in lane i ^ 16 (i ^ 32) without LDS: v_permlane16_swap /
// v_permlane32_swap with the value as both operands give, lane by lane, the own value and the
// partner's (in one order or the other; the order was checked on the GPU and does not matter
// for a max or a two-term sum).
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte global load of 8 bf16 as an MFMA operand
__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t* p) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t zero_bf16x8() { return __builtin_bit_cast(bf16x8_t, make_uint4(0, 0, 0, 0)); }

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace medusa
