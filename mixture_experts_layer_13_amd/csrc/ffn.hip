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
//    ffn_tiled_int4.hip for INT4 and ffn_tiled_fp8.hip for FP8 weights,
//    ffn_tiled_f8f8.hip for FP8 weights with FP8 activations on the FP8 MFMA):
//    128-row x 256-weight-row blocks, activations through double-buffered LDS;
//    for the bf16 gate/up GEMM of long-K layers (d >= 4096, at least 128 rows
//    per expert) 256-row x 256-weight-row blocks of eight waves fed through an
//    LDS ring by direct loads (ffn_tiled256.hip), the down GEMM then reading a
//    tile map of its own with 128-row items.
// The gate/up kernels fuse the SwiGLU epilogue silu(x Wg) * (x Wu) and write
// the bf16 (fp32 for fp32 layers) intermediate h; the down kernels write
// y_rows.  INT4 weights (two's-complement nibbles, bf16 scale per 128-K group)
// are dequantised in-kernel.  This file holds the launch dispatch, the
// weight packing kernel and the weighted combine.
#include "ffn_common.hpp"
#include "kernels_f8f8.hpp"

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
// Every y row is read once and out written once, so both go through non-temporal
// loads and stores (measured, one GPU: DeepSeek-V3-shaped T=16384 441-449 -> 385-386 us,
// DeepSeek-V2-Lite-shaped T=8192 50 -> 45 us, OLMoE-shaped T=4096 29.1 -> 27.5-28.0 us;
// the decode layers unchanged).
template <typename TA, bool PRE>
__global__ __launch_bounds__(1024) void combine_kernel(const TA* __restrict__ y, const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ gw, const TA* __restrict__ ysh,
                                                      TA* __restrict__ out, int T, int d, int k, int R) {
  constexpr int V = 16 / sizeof(TA);
  const int t = blockIdx.x;
  const int c0 = (blockIdx.y * blockDim.x + threadIdx.x) * V;
  if (c0 >= d) return;
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  auto load = [&](const TA* row) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + c0)); };
  // acc += g * row (g = 1: the shared experts' row, added, not multiplied)
  auto add = [&](float g, u32x4 v, bool scaled) {
    if constexpr (sizeof(TA) == 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = bf16_bits_to_f32((v[i / 2] >> (16 * (i & 1))) & 0xFFFFu);
        acc[i] = scaled ? fmaf(g, x, acc[i]) : acc[i] + x;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = scaled ? fmaf(g, __uint_as_float(v[i]), acc[i]) : acc[i] + __uint_as_float(v[i]);
    }
  };
  if constexpr (PRE) {
    // every load first (slot rows and gates, then the up to k + 1 rows), then the sums in order
    int rr[kMaxK];
    float gg[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      rr[j] = j < k ? slot_row[(size_t)t * k + j] : -1;
      gg[j] = j < k ? gw[(size_t)t * k + j] : 0.f;
    }
    u32x4 vv[kMaxK], vs = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if ((unsigned)rr[j] < (unsigned)R) vv[j] = load(y + (size_t)rr[j] * d);
    if (ysh) vs = load(ysh + (size_t)t * d);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j)
      if ((unsigned)rr[j] < (unsigned)R) add(gg[j], vv[j], true);
    if (ysh) add(1.f, vs, false);
  } else {
    for (int j = 0; j < k; ++j) {
      const int r = slot_row[(size_t)t * k + j];
      if ((unsigned)r >= (unsigned)R) continue;
      add(gw[(size_t)t * k + j], load(y + (size_t)r * d), true);
    }
    if (ysh) add(1.f, load(ysh + (size_t)t * d), false);
  }
  u32x4 o;
  if constexpr (sizeof(TA) == 2) {
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = pack_bf16x2(acc[2 * p], acc[2 * p + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[i]);
  }
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + (size_t)t * d + c0));
}

// tokens up to which the combine issues every load of a thread at once (the decode sizes)
constexpr int kCombinePrefetchMaxT = 64;

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
    if (wdt == kBF16 && a.bm == 256) launch_tiled256_bf16(true, a, grid, s);
    else if (wdt == kBF16) launch_tiled_bf16(true, a, grid, s);
    else if (wdt == kFP8) launch_tiled_fp8(true, a, grid, s);
    else launch_tiled_int4(true, a, grid, s);
  }
  (void)act;
  return hipGetLastError();
}

hipError_t launch_ffn_down(int mode, int act, int wdt, const FfnArgs& a, hipStream_t s) {
  if (mode == 0) {
    const int cpb = stream_channels_per_block(false, wdt) / stream_down_split(wdt, a.T);
    const int grid = ffn_grid(a, a.d / cpb, a.d / cpb);
    if (grid == 0) return hipSuccess;
    launch_stream_ffn(false, wdt, a, grid, s);
  } else {
    const int grid = ffn_grid_xcd(a, false, (a.d + 255) / 256, (a.d + 255) / 256);
    if (grid == 0) return hipSuccess;
    if (wdt == kBF16 && a.bm == 256) launch_tiled256_bf16(false, a, grid, s);
    else if (wdt == kBF16) launch_tiled_bf16(false, a, grid, s);
    else if (wdt == kFP8) launch_tiled_fp8(false, a, grid, s);
    else launch_tiled_int4(false, a, grid, s);
  }
  (void)act;
  return hipGetLastError();
}

hipError_t launch_ffn_a8(bool gateup, const FfnArgs& a, const A8Args& q, hipStream_t s) {
  const int grid = gateup ? ffn_grid_xcd(a, true, a.F / 128, a.S * a.FS / 128)
                          : ffn_grid_xcd(a, false, (a.d + 255) / 256, (a.d + 255) / 256);
  if (grid == 0) return hipSuccess;
  launch_tiled_f8f8(gateup, a, q, grid, s);
  return hipGetLastError();
}

hipError_t launch_ffn_a8_stream(bool gateup, const FfnArgs& a, const A8Args& q, hipStream_t s) {
  const int cpb = gateup ? stream_channels_per_block(true, kFP8)
                         : stream_channels_per_block(false, kFP8) / stream_down_split(kFP8, a.T);
  const int grid = gateup ? ffn_grid(a, a.F / cpb, a.S * a.FS / cpb) : ffn_grid(a, a.d / cpb, a.d / cpb);
  if (grid == 0) return hipSuccess;
  launch_stream_ffn_a8(gateup, a, q, grid, s);
  return hipGetLastError();
}

hipError_t launch_combine(int act, const void* y, const int32_t* slot_row, const float* w, const void* ysh, void* out,
                          int T, int d, int k, int R, hipStream_t s) {
  const int V = act == kF32 ? 4 : 8;
  // one block per token, of up to 1024 threads (V channels each), when that covers the row:
  // no idle threads in a last partial block (measured: DeepSeek-V3-shaped d = 7168 at
  // T=16384, 896 threads per token instead of 4 blocks of 256, 480 -> 448 us)
  const int per = (d / V + 63) / 64 * 64;
  const int tpb = per <= 1024 ? per : 256;
  dim3 grid(T, (d + tpb * V - 1) / (tpb * V));
  if (T == 0) return hipSuccess;
  // few tokens: every load of a thread issued at once (latency-bound); many: one row at a time,
  // which keeps more blocks in flight (measured, graph replays with several layers per graph /
  // eager, two GPUs: OLMoE-shaped T=8 87.1 -> 84.0 and 87.3 -> 85.4 us per layer, T=32 129.8 ->
  // 128.1 and 131.0 -> 130.0, T=64 148.9 -> 147.2 and 149.7 -> 148.9, Qwen3 INT4-shaped T=32
  // 82.8 -> 81.0; DeepSeek-V3-shaped T=16384 combine 385 -> 417 us with it)
  const bool pre = T <= kCombinePrefetchMaxT;
  if (act == kF32) {
    if (pre)
      hipLaunchKernelGGL((combine_kernel<float, true>), grid, dim3(tpb), 0, s, (const float*)y, slot_row, w,
                         (const float*)ysh, (float*)out, T, d, k, R);
    else
      hipLaunchKernelGGL((combine_kernel<float, false>), grid, dim3(tpb), 0, s, (const float*)y, slot_row, w,
                         (const float*)ysh, (float*)out, T, d, k, R);
  } else {
    if (pre)
      hipLaunchKernelGGL((combine_kernel<bf16, true>), grid, dim3(tpb), 0, s, (const bf16*)y, slot_row, w,
                         (const bf16*)ysh, (bf16*)out, T, d, k, R);
    else
      hipLaunchKernelGGL((combine_kernel<bf16, false>), grid, dim3(tpb), 0, s, (const bf16*)y, slot_row, w,
                         (const bf16*)ysh, (bf16*)out, T, d, k, R);
  }
  return hipGetLastError();
}

}  // namespace moe
