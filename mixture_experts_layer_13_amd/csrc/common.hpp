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
struct FP8 {  // one OCP E4M3 byte per weight, one fp32 scale per output channel
  uint8_t bits;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

// 16-byte global load / store
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// 16-byte load at a block-uniform base plus a per-lane unsigned 32-bit byte
// offset (lets the compiler use the scalar-base addressing form)
__device__ __forceinline__ u32x4 ld16_at(const void* base, uint32_t byte_off) {
  return *reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + byte_off);
}

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
// Whole-wave reductions (all 64 lanes active) in low-latency form: four DPP
// steps combine each lane with a partner inside its row of 16 (swap neighbours,
// swap pairs, mirror halves of 8, mirror the row of 16), leaving every row
// uniform; the four row values are then read into scalars and combined in a
// fixed order, so every lane gets the same, deterministic result.  The _n forms
// reduce N independent values at once (N tokens per wave), so the N
// dependency chains interleave and hide each other's latency.
__device__ __forceinline__ int lane_id() { return __lane_id(); }

constexpr int kDppSwap1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppSwap2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror
constexpr int kDppMirror = 0x140;      // row_mirror

template <int CTRL> __device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Inclusive prefix sum over the 64 lanes: Hillis-Steele steps inside each
// 16-lane row (row_shr 1, 2, 4, 8), then each row adds the running total of
// the rows before it (row_bcast 15 into rows 1 and 3, row_bcast 31 into rows
// 2 and 3).  Lanes without a source add 0.
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return v;
}
__device__ __forceinline__ float readlane_f32(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
template <int N> __device__ __forceinline__ void wave_max_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f32<kDppSwap1>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f32<kDppSwap2>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f32<kDppHalfMirror>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = fmaxf(v[i], dpp_f32<kDppMirror>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = fmaxf(fmaxf(readlane_f32(v[i], 0), readlane_f32(v[i], 16)),
                 fmaxf(readlane_f32(v[i], 32), readlane_f32(v[i], 48)));
}
template <int N> __device__ __forceinline__ void wave_sum_n(float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<kDppSwap1>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<kDppSwap2>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<kDppHalfMirror>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] += dpp_f32<kDppMirror>(v[i]);
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = (readlane_f32(v[i], 0) + readlane_f32(v[i], 16)) + (readlane_f32(v[i], 32) + readlane_f32(v[i], 48));
}
template <int N> __device__ __forceinline__ void wave_max_u32_n(uint32_t (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = max(v[i], dpp_u32<kDppSwap1>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = max(v[i], dpp_u32<kDppSwap2>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = max(v[i], dpp_u32<kDppHalfMirror>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = max(v[i], dpp_u32<kDppMirror>(v[i]));
#pragma unroll
  for (int i = 0; i < N; ++i)
    v[i] = max(max((uint32_t)__builtin_amdgcn_readlane((int)v[i], 0), (uint32_t)__builtin_amdgcn_readlane((int)v[i], 16)),
               max((uint32_t)__builtin_amdgcn_readlane((int)v[i], 32), (uint32_t)__builtin_amdgcn_readlane((int)v[i], 48)));
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
