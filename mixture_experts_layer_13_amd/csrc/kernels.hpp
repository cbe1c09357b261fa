// Internal interface between the C ABI (api.hip) and the kernels
// (route.hip, ffn.hip).  Not part of the public header.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

enum { kF32 = 0, kBF16 = 1, kINT4 = 2, kFP8 = 3 };
enum { kScoreSoftmax = 0, kScoreSigmoid = 1 };

constexpr int kSmallMaxPairs = 2048;    // T*k handled by the many-block route and its one-block permutation
constexpr int kOneWaveMaxPairs = 32;    // up to here the small route's permutation runs on one wave
// tokens per block of the small-T route launch: one block for a single token
// (no hand-off), else a block per token up to 32 tokens, then 4 per block
inline int route_small_tpb(int T) { return T <= 32 ? 1 : 4; }
// partial logits one small-T route block sums (K chunks x experts x its tokens)
constexpr int kSmallPartials = 8192;
constexpr int kPrefillRows = 128;       // rows per item in the tiled (large-M) expert kernels
constexpr int kMaxRouteBlocks = 512;    // large T: router / permute blocks at most (each over several tiles)

struct RouteArgs {
  int T, d, E, k;
  int score;         // kScoreSoftmax | kScoreSigmoid
  int renorm;
  float gate_scale;
  const float* logit_bias;   // [E] or null
  const float* select_bias;  // [E] or null
  int32_t* idx;              // [T][k]
  float* gates;              // [T][k]
  float* scores;             // [T][E] or null
  int tiles_per_block;       // large-T router: consecutive 16/64-token tiles per block (>= 1)
  int n_groups, topk_groups; // group-limited selection (topk_groups < n_groups), else 0 / 0
};

struct PermArgs {
  int T, k, E;
  int cap;                   // < 0: dropless
  int32_t* counts;           // [E]
  int32_t* offsets;          // [E+1]
  int32_t* row_token;        // [R]
  int32_t* slot_row;         // [T][k]
  uint8_t* drop;             // [T][k]
  int4* items;               // tile map {expert, first row, rows, 0} (null: not built)
  int32_t* n_items;
  int bm;                    // rows per tile-map item
  int4* items_dn;            // many-token permutation: the down GEMM's own tile map of bm_dn-row
  int32_t* n_items_dn;       // items (null: the down GEMM reads `items`)
  int bm_dn;
  int rt;                    // tokens per router block / tile-histogram row (large T)
};

struct FfnArgs {
  int T, d, E, F, S, FS;     // tokens, hidden, experts, ffn, shared experts, shared ffn
  int R;                     // row bound of the routed row buffers
  const void* x;             // [T][d]
  const int32_t* row_token;  // [R]
  const int4* items;         // routed tile map
  const int32_t* n_items;
  int items_max;             // static routed item slots of the grid
  int sh_items;              // static shared items (ceil(T / bm)) when S > 0
  int bm;
  int wtiled;                // expert weights in the tiled layout (else one K-contiguous row per channel)
  int wstream;               // tiled kernels: non-temporal weight loads (each expert's weights read by one row tile)
  int rowskip_gu, rowskip_dn;  // tiled gate/up, down: skip the idle 32-row tiles of partly filled items
  const void *wg, *wu, *wd, *sg, *su, *sd;         // routed weights / INT4 scales
  const void *shg, *shu, *shd, *shsg, *shsu, *shsd;  // shared weights / INT4 scales
  void* h;                   // [R][F]     act dtype
  void* hsh;                 // [T][S*FS]  act dtype
  void* y;                   // [R][d]     act dtype
  void* ysh;                 // [T][d]     act dtype
};

hipError_t launch_router_partial(int act, const void* x, const void* wr, int T, int d, int E, int kchunk, int KS,
                                 float* part, int32_t* zero, hipStream_t s);
hipError_t launch_route_small(const float* part, int KS, const RouteArgs& ra, const int32_t* idx_in,
                              const PermArgs& pa, int do_route, int do_perm, int32_t* arrived, hipStream_t s);
hipError_t launch_router_fused(int act, const void* x, const void* wr, const RouteArgs& ra, int rt, int32_t* hist,
                               hipStream_t s);
hipError_t launch_tile_hist(const int32_t* idx, int T, int k, int E, int rt, int32_t* hist, hipStream_t s);
hipError_t launch_permute_multi(const int32_t* idx, const int32_t* hist, const PermArgs& pa, hipStream_t s);
hipError_t launch_tile_map(const int32_t* offsets, int E, int R, int bm, int4* items, int32_t* n_items,
                           hipStream_t s);

// per-family launchers of the expert FFN kernels (grid from launch_ffn_*)
void launch_stream_ffn(bool gateup, int wdt, const FfnArgs& a, int grid, hipStream_t s);
int stream_channels_per_block(bool gateup, int wdt);
int stream_down_split(int wdt, int T);
hipError_t launch_down_combine_one(int wdt, const FfnArgs& a, const int32_t* topk_idx, const int32_t* slot_row,
                                   const float* gw, void* out, int k, hipStream_t s);
void launch_tiled_bf16(bool gateup, const FfnArgs& a, int grid, hipStream_t s);
void launch_tiled256_bf16(bool gateup, const FfnArgs& a, int grid, hipStream_t s);
void launch_tiled_int4(bool gateup, const FfnArgs& a, int grid, hipStream_t s);
void launch_tiled_fp8(bool gateup, const FfnArgs& a, int grid, hipStream_t s);

// expert FFN: mode 0 = streaming small-M kernels, 1 = LDS-tiled MFMA kernels
hipError_t launch_ffn_gateup(int mode, int act, int wdt, const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn_down(int mode, int act, int wdt, const FfnArgs& a, hipStream_t s);
// row layout -> tiled layout of `rows` weight rows of `row_bytes` bytes each
hipError_t launch_pack_tiled(const void* src, void* dst, int64_t rows, int64_t row_bytes, hipStream_t s);
hipError_t launch_combine(int act, const void* y, const int32_t* slot_row, const float* w, const void* ysh,
                          void* out, int T, int d, int k, int R, hipStream_t s);

}  // namespace moe
