// Grouped expert SwiGLU GEMMs and the weighted combine for gfx950.
//
// "MoE: dynamism the compiler cannot remove", grouped-GEMM section: one
// launch over a fixed grid sized for the worst case; each block reads a small
// device-side descriptor (here a tile-map item {expert, first row, rows}) to
// find its group, so the grid never depends on how the rows split between
// experts, nothing is padded on the host and nothing is dropped.  Shared
// (always-on) experts ("MoE Research" section 2) are extra groups over all T
// tokens behind the routed ones in the same launch.
//
// Two tilings of the same computation, chosen by the host from T alone:
//  - streaming kernels (small M, decode; ffn_stream.hip): a block owns one
//    item (<= 64 rows of one expert) and a few output channels and reads its
//    weight slice once, straight from memory into MFMA operands;
//  - tiled kernels (large M, prefill; ffn_tiled.hip for bf16,
//    ffn_tiled_int4.hip for INT4 weights): 128-row x 256-weight-row blocks,
//    activations through double-buffered LDS.
// The gate/up kernels fuse the SwiGLU epilogue silu(x Wg) * (x Wu) and write
// the bf16 (fp32 for fp32 layers) intermediate h; the down kernels write
// y_rows.  INT4 weights (two's-complement nibbles, bf16 scale per 128-K group)
// are dequantised in-kernel.  This file holds the launch dispatch, the
// weight packing kernel and the weighted combine.
#include "ffn_common.hpp"

namespace moe {

// ------------------------------------------------------------------ weight packing
// Tiled layout from the row layout (a byte permutation): output 16-byte unit
// u = 64 * fragment + 16 * g + c of fragment (row group r16, chunk j) takes
// bytes 64j + 16g .. +15 of row 16 * r16 + c.  Writes are consecutive; reads
// gather 16 rows.  Grid-stride over all units.
__global__ __launch_bounds__(256) void pack_tiled_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t units, int64_t chunks_per_row) {
  for (int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (int64_t)gridDim.x * 256) {
    const int64_t frag = u >> 6;
    const int lane = (int)(u & 63), g = lane >> 4, c = lane & 15;
    const int64_t r16 = frag / chunks_per_row, j = frag - r16 * chunks_per_row;
    dst[u] = src[((16 * r16 + c) * chunks_per_row + j) * 4 + g];
  }
}

hipError_t launch_pack_tiled(const void* src, void* dst, int64_t rows, int64_t row_bytes, hipStream_t s) {
  const int64_t units = rows * row_bytes / 16;
  if (units == 0) return hipSuccess;
  const int64_t want = (units + 255) / 256;
  const int grid = (int)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(pack_tiled_kernel, dim3(grid), dim3(256), 0, s, (const u32x4*)src, (u32x4*)dst, units,
                     row_bytes / 64);
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// out[t] = sum_j gate[t,j] * y_rows[slot_row[t,j]] (+ y_shared[t]), fp32, j in order.
template <typename TA>
__global__ __launch_bounds__(256) void combine_kernel(const TA* __restrict__ y, const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ gw, const TA* __restrict__ ysh,
                                                      TA* __restrict__ out, int T, int d, int k, int R) {
  constexpr int V = 16 / sizeof(TA);
  const int t = blockIdx.x;
  const int c0 = (blockIdx.y * 256 + threadIdx.x) * V;
  if (c0 >= d) return;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int r = slot_row[(size_t)t * k + j];
    if ((unsigned)r >= (unsigned)R) continue;
    const float gj = gw[(size_t)t * k + j];
    const u32x4 v = ld16(y + (size_t)r * d + c0);
    if constexpr (sizeof(TA) == 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = fmaf(gj, bf16_bits_to_f32((v[i / 2] >> (16 * (i & 1))) & 0xFFFFu), acc[i]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(gj, __uint_as_float(v[i]), acc[i]);
    }
  }
  if (ysh) {
    const u32x4 v = ld16(ysh + (size_t)t * d + c0);
    if constexpr (sizeof(TA) == 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += bf16_bits_to_f32((v[i / 2] >> (16 * (i & 1))) & 0xFFFFu);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += __uint_as_float(v[i]);
    }
  }
  u32x4 o;
  if constexpr (sizeof(TA) == 2) {
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = pack_bf16x2(acc[2 * p], acc[2 * p + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[i]);
  }
  st16(out + (size_t)t * d + c0, o);
}

// ------------------------------------------------------------------ host launchers
static int ffn_grid(const FfnArgs& a, int nt_routed, int nt_shared) {
  return a.items_max * nt_routed + (a.S > 0 ? a.sh_items * nt_shared : 0);
}
// tiled kernels: 8 XCD chunks of equal work, each given enough blocks for its
// largest possible tile count (blocks past a chunk's end return at once)
static int ffn_grid_xcd(const FfnArgs& a, bool gateup, int nt_routed, int nt_shared) {
  if (ffn_grid(a, nt_routed, nt_shared) == 0) return 0;
  int64_t wr, ws;
  tile_work(gateup, a.F, a.S, a.FS, wr, ws);
  return 8 * tiled_blocks_per_xcd((int64_t)a.items_max * nt_routed, a.S > 0 ? (int64_t)a.sh_items * nt_shared : 0,
                                  wr, ws);
}

hipError_t launch_ffn_gateup(int mode, int act, int wdt, const FfnArgs& a, hipStream_t s) {
  if (mode == 0) {
    const int cpb = stream_channels_per_block(true, wdt);
    const int grid = ffn_grid(a, a.F / cpb, a.S * a.FS / cpb);
    if (grid == 0) return hipSuccess;
    launch_stream_ffn(true, wdt, a, grid, s);
  } else {
    const int grid = ffn_grid_xcd(a, true, a.F / 128, a.S * a.FS / 128);
    if (grid == 0) return hipSuccess;
    if (wdt == kBF16) launch_tiled_bf16(true, a, grid, s);
    else launch_tiled_int4(true, a, grid, s);
  }
  (void)act;
  return hipGetLastError();
}

hipError_t launch_ffn_down(int mode, int act, int wdt, const FfnArgs& a, hipStream_t s) {
  if (mode == 0) {
    const int cpb = stream_channels_per_block(false, wdt);
    const int grid = ffn_grid(a, a.d / cpb, a.d / cpb);
    if (grid == 0) return hipSuccess;
    launch_stream_ffn(false, wdt, a, grid, s);
  } else {
    const int grid = ffn_grid_xcd(a, false, (a.d + 255) / 256, (a.d + 255) / 256);
    if (grid == 0) return hipSuccess;
    if (wdt == kBF16) launch_tiled_bf16(false, a, grid, s);
    else launch_tiled_int4(false, a, grid, s);
  }
  (void)act;
  return hipGetLastError();
}

hipError_t launch_combine(int act, const void* y, const int32_t* slot_row, const float* w, const void* ysh, void* out,
                          int T, int d, int k, int R, hipStream_t s) {
  const int V = act == kF32 ? 4 : 8;
  dim3 grid(T, (d + 256 * V - 1) / (256 * V));
  if (T == 0) return hipSuccess;
  if (act == kF32)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, (const float*)y, slot_row, w, (const float*)ysh,
                       (float*)out, T, d, k, R);
  else
    hipLaunchKernelGGL(combine_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)y, slot_row, w, (const bf16*)ysh,
                       (bf16*)out, T, d, k, R);
  return hipGetLastError();
}

}  // namespace moe
