// Device helpers shared by the expert FFN kernels (streaming, tiled bf16,
// tiled INT4): bf16 packing, INT4 nibble decoding, SiLU, weight-matrix
// addressing and the tile list of the tiled kernels.
#pragma once
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(bf16)lo, (bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Eight nibbles q (two's complement, element i at bits 4i..4i+3) to eight
// bf16 values 136 + q, exactly: with u = q + 8 in 0..15, bf16 bits 0x4300 | u
// are 128 + u (exponent 2^7, mantissa step 1).  Per pair one byte permute
// puts byte p of the nibbles (low nibble) and of the nibbles >> 4 (high
// nibble) into the two halves, one and-or keeps the nibbles and sets 0x43.
// A product with x then carries 136 x extra, taken off as 136 sum(x).
__device__ __forceinline__ u32x4 int4x8_to_bf16_off136(uint32_t w) {
  const uint32_t x = w ^ 0x88888888u, xs = x >> 4;
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t sel = (uint32_t)p | (0x0Cu << 8) | ((uint32_t)(4 + p) << 16) | (0x0Cu << 24);
    r[p] = (__builtin_amdgcn_perm(xs, x, sel) & 0x000F000Fu) | 0x43004300u;
  }
  return r;
}

// Eight two's-complement nibbles (element i in bits 4i..4i+3) times the group
// scale, rounded once to bf16 (operand of the tiled kernels).  sc16 is 16
// times the scale: v_cvt_off_f32_i4 turns the low 4 bits of its operand into
// q / 16 exactly, and (q / 16) * (16 s) = q s exactly in fp32 (a 4-bit by
// 8-bit product), so the only rounding is the final one to bf16.
__device__ __forceinline__ u32x4 int4x8_to_bf16_scaled(uint32_t w, float sc16) {
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float lo = __builtin_amdgcn_cvt_off_f32_i4(w >> (8 * p)) * sc16;
    const float hi = __builtin_amdgcn_cvt_off_f32_i4(w >> (8 * p + 4)) * sc16;
    r[p] = pack_bf16x2(lo, hi);
  }
  return r;
}

// silu(z) = z sigma(z) with the hardware exponential and reciprocal (a few ulp in
// fp32, far below the bf16 rounding of h; measured -5.5 us on the OLMoE T=4096
// gate/up epilogue against expf and IEEE division)
__device__ __forceinline__ float silu(float z) { return z * __frcp_rn(1.0f + __expf(-z)); }

// bytes of one K-contiguous weight row
template <typename TW> __device__ __forceinline__ constexpr int row_bytes(int K) { return K * (int)sizeof(TW); }
template <> __device__ __forceinline__ constexpr int row_bytes<INT4>(int K) { return K / 2; }

// bytes (or elements) of one expert's [N][K] matrix, to step between experts
template <typename TW> __device__ __forceinline__ const void* expert_mat(const void* base, int e, int N, int K);
template <> __device__ __forceinline__ const void* expert_mat<float>(const void* b, int e, int N, int K) {
  return (const float*)b + (size_t)e * N * K;
}
template <> __device__ __forceinline__ const void* expert_mat<bf16>(const void* b, int e, int N, int K) {
  return (const bf16*)b + (size_t)e * N * K;
}
template <> __device__ __forceinline__ const void* expert_mat<INT4>(const void* b, int e, int N, int K) {
  return (const uint8_t*)b + (size_t)e * N * (K / 2);
}
template <> __device__ __forceinline__ const void* expert_mat<FP8>(const void* b, int e, int N, int K) {
  return (const uint8_t*)b + (size_t)e * N * K;
}
__device__ __forceinline__ const void* expert_scales(const void* b, int e, int N, int K) {
  return b ? (const void*)((const uint16_t*)b + (size_t)e * N * (K / kInt4Group)) : nullptr;
}
// scales of expert e by weight type: INT4 one bf16 per (channel, 128-K group), FP8 one fp32 per channel
template <typename TW> __device__ __forceinline__ const void* expert_scales_of(const void* b, int e, int N, int K) {
  if constexpr (std::is_same<TW, FP8>::value) return b ? (const void*)((const float*)b + (size_t)e * N) : nullptr;
  else return expert_scales(b, e, N, K);
}

__device__ __forceinline__ f32x16 mma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

constexpr int TBM = 128;

// The tile a block of a tiled kernel owns.  Tile list: routed items
// (expert-major, so one expert's tiles are adjacent) times N blocks of NT
// output channels, then the shared-expert tiles.  Blocks are dispatched
// round-robin over the 8 XCDs, so XCD x = blockIdx % 8 takes the x-th of 8
// contiguous chunks of the list: the tiles of an expert then run together on
// one XCD and share their weight and activation K slabs in its L2.  The chunks
// hold equal work, a tile weighing its K length: a shared down tile runs over
// the S shared experts' concatenated K, S FS against F for a routed one.
// tile_work() gives the two weights; the grid (tiled_blocks_per_xcd) covers
// the largest chunk any routing can produce.
__host__ __device__ inline void tile_work(bool gateup, int F, int S, int FS, int64_t& wr, int64_t& ws) {
  wr = gateup ? 1 : F;
  ws = gateup ? 1 : (int64_t)S * FS;
}
// Tiles per chunk are at most (chunk work + 1) / (lightest tile) + 1; with at
// most Wmax work in all, one more block per XCD of slack.
__host__ __device__ inline int tiled_blocks_per_xcd(int64_t routed_tiles_max, int64_t shared_tiles, int64_t wr,
                                                    int64_t ws) {
  const int64_t wmin = shared_tiles > 0 && ws < wr ? ws : wr;
  const int64_t wmax = routed_tiles_max * wr + shared_tiles * ws;
  return (int)((wmax / 8 + 1 + wmin - 1) / wmin + 2);
}
// Routed items of the tile map as the expert kernels read them, clamped so
// that a corrupted map (a race on the workspace, a stray write into it) gives
// wrong rows, never an access outside the weights or the row buffers: the item
// count into [0, items_max], the expert into [0, E), the first row into
// [0, R), the rows into [1, min(bm, R - first row)]; false for an empty item.
__device__ __forceinline__ int routed_items(const FfnArgs& a) { return min(max(*a.n_items, 0), a.items_max); }
__device__ __forceinline__ bool load_item(const FfnArgs& a, int slot, int& e, int& row0, int& mrows) {
  if (a.R <= 0) return false;
  const int4 it = a.items[slot];
  e = min(max(it.x, 0), a.E - 1);
  row0 = min(max(it.y, 0), a.R - 1);
  mrows = min(min(it.z, a.bm), a.R - row0);
  return mrows > 0;
}

struct TileInfo {
  int e, row0, mrows, n0;
  bool shared;
};
__device__ __forceinline__ bool tile_of(const FfnArgs& a, int NT, TileInfo& t) {
  const bool gu = NT == 128;  // gate/up blocks cover 128 channels, down blocks 256 columns
  const int Nr = gu ? a.F : a.d, Ns = gu ? a.S * a.FS : a.d;
  const int nbr = (Nr + NT - 1) / NT, nbs = (Ns + NT - 1) / NT;
  const int routed_tiles = routed_items(a) * nbr;
  const int shared_tiles = a.S > 0 ? a.sh_items * nbs : 0;
  int64_t wr, ws;
  tile_work(gu, a.F, a.S, a.FS, wr, ws);
  const int64_t W = routed_tiles * wr + shared_tiles * ws;
  // first tile whose starting work is at least W x / 8
  auto first_tile = [&](int x) -> int {
    const int64_t target = W * x / 8;
    if (target <= routed_tiles * wr) return (int)((target + wr - 1) / wr);
    return routed_tiles + (int)((target - routed_tiles * wr + ws - 1) / ws);
  };
  const int xcd = blockIdx.x & 7;
  const int lo = first_tile(xcd), hi = first_tile(xcd + 1);
  // Dispatch order inside the chunk.  With many N blocks per item (>= 11: the
  // DeepSeek-V3 layers, DeepSeek-V2-Lite gate/up) blocks take groups of 8
  // consecutive items N-block major, so the tiles that share a weight slab
  // start together and find it in L2 (measured: DeepSeek-V3 T=16384 gate/up
  // 11.36 -> 9.59 ms, down 5.66 -> 4.69 ms); with fewer, item-major order keeps
  // an item's activation rows in L2 and was 1-2% faster.
  const int j = (int)(blockIdx.x >> 3);
  int tile = lo + j;
  if (nbr >= 11) {
    const int gsz = 8 * nbr, full = (hi - lo) / gsz * gsz;
    if (j < full) tile = lo + (j / gsz) * gsz + (j % 8) * nbr + (j % gsz) / 8;
  }
  if (tile >= hi) return false;
  int nb;
  t.shared = tile >= routed_tiles;
  if (!t.shared) {
    const int slot = tile / nbr;
    nb = tile - slot * nbr;
    if (!load_item(a, slot, t.e, t.row0, t.mrows)) return false;
  } else {
    const int sb = tile - routed_tiles;
    const int slot = sb / nbs;
    nb = sb - slot * nbs;
    t.e = 0;
    t.row0 = slot * a.bm;
    t.mrows = min(a.bm, a.T - t.row0);
  }
  t.n0 = nb * NT;
  return true;
}

}  // namespace moe
