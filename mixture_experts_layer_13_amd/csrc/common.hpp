// Shared device helpers for the gfx950 MoE kernels: vector types, bf16
// conversion, MFMA wrappers, wave-level reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxE = 256;
constexpr int kMaxK = 8;
constexpr int kInt4Group = 128;

// element types the kernels are instantiated for
struct F32 {};
struct BF16 {};
struct INT4 {};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

// 16-byte global load / store
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l supplies row (l % 16) of A and column (l % 16) of B, eight K values
// each; any K order works as long as A and B use the same one.  Output:
// lane l holds D[4 * (l / 16) + i][l % 16], i = 0..3.
__device__ __forceinline__ f32x4 mma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// D(16x16, f32) += A(16x4, f32) * B(4x16, f32); one K value per lane.
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint64_t w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// Monotone map float -> uint32 (total order; -0 is canonicalised to +0 first).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t b = __float_as_uint(f + 0.0f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// lanes sharing value `v` (v < 2^nbits) among the active lanes in `active`
__device__ __forceinline__ uint64_t match_peers(uint32_t v, uint64_t active, int nbits) {
  uint64_t m = active;
  for (int b = 0; b < nbits; ++b) {
    uint64_t bal = __ballot((v >> b) & 1u);
    m &= ((v >> b) & 1u) ? bal : ~bal;
  }
  return m;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
