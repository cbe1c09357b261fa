// Routing and permutation kernels for gfx950.
//
// Router ("MoE: dynamism the compiler cannot remove", natural implementation:
// logits = router(x), then top-k): an MFMA product of the token tile with the
// router rows, FP32 scoring (max-subtract-expsum softmax, as in the launch-bound
// study's FusedSoftmax description, or sigmoid plus a selection-only bias, as
// in "MoE Research" section 2), then a wave-level top-k over the E scores held
// in registers (E <= 256: at most 4 per lane), ties to the lower expert index.
//
// Permutation (same page, capacity section and batch-1 recipe: fixed-shape
// scatter into preallocated buffers): an atomic-free expert histogram built
// from wave ballots, an exclusive scan, and a stable token-major ranking that
// applies the capacity rule and fills the expert-major row map.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ------------------------------------------------------------------ helpers
// One 16-byte chunk per lane per step: bf16 -> 8 K values (one MFMA),
// f32 -> 4 K values (four MFMAs, one K value each).
template <typename T> struct Chunk;
template <> struct Chunk<bf16> {
  static constexpr int EPC = 8;
  __device__ static f32x4 mma(u32x4 a, u32x4 b, f32x4 c) { return mma_bf16(a, b, c); }
};
template <> struct Chunk<float> {
  static constexpr int EPC = 4;
  __device__ static f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c = mma_f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c);
    return c;
  }
};

// Routes NT tokens at once with one full wave (their reductions interleave).
// logit[i][j] holds expert e = lane + 64 j (j < EPL, E <= 64 EPL) of token
// t0 + i.  Scores: softmax (max-subtract-expsum, fp32) or sigmoid; selection
// key: the score, plus the selection-only bias for sigmoid scoring.  Top-k:
// k rounds; each takes the wave-wide maximum of the fp32 keys in a monotone
// 32-bit encoding, then, among the entries holding that maximum, the lowest
// expert index (ballots over the lanes' best entries), so equal keys select
// the lower index and slots come out in descending key order.  Group-limited
// selection first zeroes the keys outside the token's topk_groups best groups
// (group score: its largest key; equal scores keep the lower group).  Gates: the
// selected unbiased scores (renormalised over the k picks when asked), times
// gate_scale.  Tokens i >= nvalid are computed but not written.
// GRP: the group-limited step is compiled in (kernels without it keep their registers).
template <int NT, int EPL, bool GRP = false>
__device__ __forceinline__ void route_tokens(float (&logit)[NT][EPL], const RouteArgs& a, int t0, int nvalid,
                                             uint16_t* sel) {
  const int lane = lane_id();
  const int E = a.E, k = a.k;
  float score[NT][EPL];
  uint32_t key[NT][EPL];
  if (a.score == kScoreSoftmax) {
    float m[NT], sum[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      m[i] = -INFINITY;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (lane + 64 * j < E) m[i] = fmaxf(m[i], logit[i][j]);
    }
    wave_max_n<NT>(m);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      sum[i] = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        score[i][j] = (lane + 64 * j < E) ? expf(logit[i][j] - m[i]) : 0.f;
        sum[i] += score[i][j];
      }
    }
    wave_sum_n<NT>(sum);
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        score[i][j] = score[i][j] / sum[i];
        key[i][j] = float_order_key(score[i][j]);
      }
  } else {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      const float b = (a.select_bias && e < E) ? a.select_bias[e] : 0.f;
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        score[i][j] = 1.0f / (1.0f + expf(-logit[i][j]));
        key[i][j] = float_order_key(score[i][j] + b);
      }
    }
  }
  if (a.scores) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
      if (i < nvalid)
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (lane + 64 * j < E) a.scores[(size_t)(t0 + i) * E + lane + 64 * j] = score[i][j];
  }
  // 0 marks an absent or already selected entry: every finite or infinite key encodes above 0
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (lane + 64 * j >= E)
#pragma unroll
      for (int i = 0; i < NT; ++i) key[i][j] = 0u;
  if (GRP) {
    const int G = a.n_groups, gsz = E / G;
    int grp[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) grp[j] = (lane + 64 * j) / gsz;  // >= G past E (keys 0 there)
    uint32_t gk[NT];  // lane g < G: the score of group g
#pragma unroll
    for (int i = 0; i < NT; ++i) gk[i] = 0u;
    for (int gi = 0; gi < G; ++gi) {
      uint32_t m[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        m[i] = 0u;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
          if (grp[j] == gi) m[i] = max(m[i], key[i][j]);
      }
      wave_max_u32_n<NT>(m);
#pragma unroll
      for (int i = 0; i < NT; ++i)
        if (lane == gi) gk[i] = m[i];
    }
    uint64_t keep[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) keep[i] = 0ull;
    for (int r = 0; r < a.topk_groups; ++r) {
      uint32_t b[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) b[i] = (lane < G && !((keep[i] >> lane) & 1ull)) ? gk[i] : 0u;
      uint32_t top[NT];
#pragma unroll
      for (int i = 0; i < NT; ++i) top[i] = b[i];
      wave_max_u32_n<NT>(top);
#pragma unroll
      for (int i = 0; i < NT; ++i) {
        // lowest group among the not yet kept ones holding the maximum
        const uint64_t bl = __ballot(lane < G && !((keep[i] >> lane) & 1ull) && b[i] == top[i]);
        keep[i] |= 1ull << (__ffsll((unsigned long long)bl) - 1);
      }
    }
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (grp[j] >= G || !((keep[i] >> grp[j]) & 1ull)) key[i][j] = 0u;
  }
  float gsum[NT], sel_s[NT];
  int sel_e[NT];
#pragma unroll
  for (int i = 0; i < NT; ++i) {
    gsum[i] = 0.f;
    sel_s[i] = 0.f;
    sel_e[i] = 0;
  }
  for (int r = 0; r < k; ++r) {
    uint32_t best[NT], lbest[NT];
    int lj[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {  // the lane's best entry (lowest j among equals)
      lbest[i] = key[i][0];
      lj[i] = 0;
#pragma unroll
      for (int j = 1; j < EPL; ++j)
        if (key[i][j] > lbest[i]) {
          lbest[i] = key[i][j];
          lj[i] = j;
        }
      best[i] = lbest[i];
    }
    wave_max_u32_n<NT>(best);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      // lowest expert index holding the maximum: smallest j first, then the lowest lane
      int e = 0;
#pragma unroll
      for (int j = EPL - 1; j >= 0; --j) {
        const uint64_t b = __ballot(lbest[i] == best[i] && lj[i] == j);
        if (b) e = __ffsll((unsigned long long)b) - 1 + 64 * j;
      }
      const int owner = e & 63, jj = e >> 6;
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        if (j == jj && lane == owner) {
          key[i][j] = 0u;
          s = score[i][j];
        }
      }
      s = readlane_f32(s, owner);
      gsum[i] += s;
      if (lane == r) {
        sel_e[i] = e;
        sel_s[i] = s;
      }
    }
  }
  if (lane < k) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (i >= nvalid) break;
      float gt = a.renorm ? sel_s[i] / gsum[i] : sel_s[i];
      gt *= a.gate_scale;
      a.idx[(size_t)(t0 + i) * k + lane] = sel_e[i];
      a.gates[(size_t)(t0 + i) * k + lane] = gt;
      if (sel) sel[i * k + lane] = (uint16_t)sel_e[i];
    }
  }
}

// Loads the logits of NT tokens (rows of `src`, row stride ld) for route_tokens.
template <int NT, int EPL>
__device__ __forceinline__ void load_logits(float (&logit)[NT][EPL], const float* src, int ld, int E,
                                            const float* bias) {
  const int lane = lane_id();
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    const float b = (e < E && bias) ? bias[e] : 0.f;
#pragma unroll
    for (int i = 0; i < NT; ++i) logit[i][j] = e < E ? src[i * ld + e] + b : 0.f;
  }
}

// Routes tokens [0, nt) whose logits sit in LDS rows (wave w takes groups of 4).
template <int EPL, bool GRP>
__device__ void route_rows(const float* slog, int ld, int nt, int t0, const RouteArgs& ra, const float* bias,
                           uint16_t* sel, int w, int nw) {
  const int k = ra.k;
  for (int t4 = 4 * w; t4 < nt; t4 += 4 * nw) {
    if (nt - t4 >= 4) {
      float logit[4][EPL];
      load_logits<4, EPL>(logit, slog + t4 * ld, ld, ra.E, bias);
      route_tokens<4, EPL, GRP>(logit, ra, t0 + t4, 4, sel + t4 * k);
    } else {
      for (int i = t4; i < nt; ++i) {
        float logit[1][EPL];
        load_logits<1, EPL>(logit, slog + i * ld, ld, ra.E, bias);
        route_tokens<1, EPL, GRP>(logit, ra, t0 + i, 1, sel + i * k);
      }
    }
  }
}

// Exclusive scan of n <= 256 ints in LDS by one wave; returns the total.
__device__ __forceinline__ int wave_exclusive_scan256(const int* in, int* out, int n) {
  const int lane = lane_id();
  int v[4], run = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 4 * lane + i;
    v[i] = p < n ? in[p] : 0;
  }
  const int local = v[0] + v[1] + v[2] + v[3];
  const int incl = wave_incl_scan_i32(local);
  run = incl - local;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 4 * lane + i;
    if (p < n) out[p] = run;
    run += v[i];
  }
  return __builtin_amdgcn_readlane(incl, 63);
}

// Item i of the n = ceil(kept / bm) items of an expert with `kept` rows from row `first`.
// For the tiled kernels (bm = 128 or 256) the expert's 32-row tiles are spread evenly over its items
// (their sizes differ by at most 32 rows), so the items that read the same weight slabs run
// for about as long, instead of n - 1 full items and one short one that runs ahead of them
// (measured: Qwen3 INT4 T=4096 0.495 -> 0.483 ms, DeepSeek-V2-Lite T=8192 1.324 -> 1.302 ms).
// Otherwise consecutive bm-row slices.
__device__ __forceinline__ int4 item_of(int e, int first, int kept, int n, int i, int bm) {
  if (bm < kPrefillRows) return make_int4(e, first + i * bm, min(bm, kept - i * bm), 0);
  const int tiles = (kept + 31) / 32, base = tiles / n, extra = tiles % n;
  const int s = 32 * (i * base + min(i, extra));
  return make_int4(e, first + s, min(32 * (base + (i < extra ? 1 : 0)), kept - s), 0);
}

// Tile map for the grouped expert GEMMs: ceil(kept / bm) items {expert, first row, rows}
// per expert (item_of).  Called by a whole block
// after kept[] and off[] (LDS) are final; tmp is LDS scratch of >= 257 ints.
__device__ void write_tile_map(const int* kept, const int* off, int E, int bm, int4* items, int32_t* n_items,
                               int* tmp) {
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) tmp[e] = (kept[e] + bm - 1) / bm;
  __syncthreads();
  if (tid < 64) {
    int total = wave_exclusive_scan256(tmp, tmp + 256, E);
    if (tid == 0) *n_items = total;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    const int n = tmp[e], start = tmp[256 + e];
    for (int i = 0; i < n; ++i)
      items[start + i] = item_of(e, off[e], kept[e], n, i, bm);
  }
}

// ------------------------------------------------------------------ router GEMM
// Partial logits part[z][t][e] = sum over the z-th K chunk of x[t,:] . w_router[e,:].
// grid (ceil(T/16), ceil(E/64), KS), block 256: wave w owns experts
// blockIdx.y*64 + 16w .. +16 for a 16-token tile.  `zero` (if set) is the
// arrival counter of the route launch that follows; the first block clears it.
template <typename TIN>
__global__ __launch_bounds__(256) void router_partial_kernel(const TIN* __restrict__ x,
                                                             const TIN* __restrict__ wr, int T, int d, int E,
                                                             int kchunk, float* __restrict__ part, int32_t* zero) {
  constexpr int EPC = Chunk<TIN>::EPC;
  if (zero && threadIdx.x == 0 && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) *zero = 0;
  constexpr int KSTEP = 4 * EPC;
  const int lane = lane_id(), w = threadIdx.x / 64;
  const int e0 = blockIdx.y * 64 + w * 16;
  if (e0 >= E) return;
  const int t0 = blockIdx.x * 16;
  const int k0 = blockIdx.z * kchunk, k1 = min(d, k0 + kchunk);
  const int ta = min(t0 + (lane & 15), T - 1);
  const int eb = min(e0 + (lane & 15), E - 1);
  const int g = lane >> 4;
  const TIN* pa = x + (size_t)ta * d + g * EPC;
  const TIN* pb = wr + (size_t)eb * d + g * EPC;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int kk = k0;
  for (; kk + 8 * KSTEP <= k1; kk += 8 * KSTEP) {  // 8 loads per operand in flight
    u32x4 a[8], b[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      a[u] = ld16(pa + kk + u * KSTEP);
      b[u] = ld16(pb + kk + u * KSTEP);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = Chunk<TIN>::mma(a[u], b[u], acc);
  }
  for (; kk < k1; kk += KSTEP) acc = Chunk<TIN>::mma(ld16(pa + kk), ld16(pb + kk), acc);
  const int e = e0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 4 * g + i;
    if (t < T && e < E) part[((size_t)blockIdx.z * T + t) * E + e] = acc[i];
  }
}

// ------------------------------------------------------------------ ranking core
// Ranks one pass of up to blockDim.x pairs (one per thread, token-major order).
// wcnt: LDS [nwaves][256]; base: LDS [256] running per-expert count (updated).
// Returns this pair's rank within its expert (undefined when !valid).
__device__ __forceinline__ int rank_pass(int e, bool valid, int* wcnt, int* base, int E) {
  const int tid = threadIdx.x, lane = lane_id(), w = tid / 64, nw = blockDim.x / 64;
  __syncthreads();  // the previous pass's readers of wcnt are done
  for (int i = tid; i < nw * 256; i += blockDim.x) wcnt[i] = 0;
  __syncthreads();
  const uint64_t active = __ballot(valid);
  const uint64_t peers = match_peers(valid ? (uint32_t)e : 0u, active, 8);
  if (valid && lane == __ffsll((unsigned long long)peers) - 1) wcnt[w * 256 + e] = __popcll(peers);
  __syncthreads();
  for (int x = tid; x < E; x += blockDim.x) {
    int acc = base[x];
    for (int ww = 0; ww < nw; ++ww) {
      const int c = wcnt[ww * 256 + x];
      wcnt[ww * 256 + x] = acc;
      acc += c;
    }
    base[x] = acc;
  }
  __syncthreads();
  return valid ? wcnt[w * 256 + e] + __popcll(peers & lanemask_lt()) : 0;
}

// Applies a rank: writes slot_row / drop / row_token for pair i = t*k + j.
__device__ __forceinline__ void place_pair(const PermArgs& p, int i, int e, bool valid, int rank, const int* off) {
  const bool kept = valid && (p.cap < 0 || rank < p.cap);
  if (kept) {
    const int row = off[e] + rank;
    p.slot_row[i] = row;
    p.drop[i] = 0;
    p.row_token[row] = i / p.k;
  } else {
    p.slot_row[i] = -1;
    p.drop[i] = 1;
  }
}

// The permutation of one token's top-k picks (one wave, no barriers): the k
// experts are distinct, so every count is 0 or 1 and the rows go to the picked
// experts in expert order.  A pick's row is the number of kept picks with a
// lower expert index (ballots over the lanes, lane = expert mod 64), each kept
// expert gets one single-row item, and capacity only matters as cap = 0.
__device__ void permute_single_token(const PermArgs& p, const uint16_t* sel, int* off) {
  const int lane = lane_id(), E = p.E, k = p.k;
  const bool keep = p.cap != 0;
  int run = 0;
  for (int j = 0; j * 64 < E; ++j) {
    const int e = 64 * j + lane;
    bool picked = false;
    for (int i = 0; i < k; ++i) picked |= (int)sel[i] == e;
    const uint64_t m = __ballot(picked && e < E);
    const int o = run + (keep ? __popcll(m & lanemask_lt()) : 0);
    if (e < E) {
      p.counts[e] = picked ? 1 : 0;
      p.offsets[e] = o;
      off[e] = o;
      if (p.items && keep && picked) p.items[o] = make_int4(e, o, 1, 0);
    }
    run += keep ? __popcll(m) : 0;
  }
  if (lane == 0) {
    p.offsets[E] = run;
    if (p.items) *p.n_items = run;
  }
  if (lane < k) {
    const int e = sel[lane];
    if (keep) {
      const int row = off[e];
      p.slot_row[lane] = row;
      p.drop[lane] = 0;
      p.row_token[row] = 0;
    } else {
      p.slot_row[lane] = -1;
      p.drop[lane] = 1;
    }
  }
}

// ------------------------------------------------------------------ small-T route + permute
// Ranks every pair with one wave (no barriers): pair i = 64 j + lane.  One
// pass in token-major order gives each pair its stable rank inside its expert
// (lanes holding the same expert found with ballots; a running per-expert
// count in LDS, bumped by the lowest such lane) and leaves the expert counts;
// then the capacity rule, the exclusive scan, the tile map and the placement.
// The picks are loaded first (all at once); the per-pair loops are kept
// rolled and run over the occupied 64-pair chunks only, so the code a launch
// executes once stays short.  LDS: base [256], off [257], tmp [512],
// pr [kSmallMaxPairs] (rank * 256 + expert, or -1).
__device__ void permute_one_wave(const PermArgs& p, const int32_t* idx, const uint16_t* sel, int* base, int* off,
                                 int* tmp, int* pr) {
  constexpr int PPL = kSmallMaxPairs / 64;
  const int lane = lane_id(), n = p.T * p.k, E = p.E, nch = (n + 63) / 64;
  const int nbits = E <= 1 ? 0 : 32 - __clz(E - 1);
  int raw[PPL];
#pragma unroll
  for (int j = 0; j < PPL; ++j) {
    const int i = 64 * j + lane;
    raw[j] = i >= n ? -1 : (idx ? idx[i] : (int)sel[i]);
  }
#pragma unroll
  for (int j = 0; j < PPL; ++j)
    if (64 * j + lane < n) pr[64 * j + lane] = raw[j];
  for (int x = lane; x < 256; x += 64) base[x] = 0;
#pragma unroll 1
  for (int j = 0; j < nch; ++j) {
    const int i = 64 * j + lane;
    const int r = i < n ? pr[i] : -1;
    const bool valid = r >= 0 && r < E;
    const int e = valid ? r : 0;
    const uint64_t peers = match_peers((uint32_t)e, __ballot(valid), nbits);
    const int before = __popcll(peers & lanemask_lt());
    const int b = valid ? base[e] : 0;
    if (valid && before == 0) base[e] = b + __popcll(peers);
    if (i < n) pr[i] = valid ? (b + before) * 256 + e : -1;
  }
  for (int x = lane; x < E; x += 64) {
    p.counts[x] = base[x];
    tmp[x] = p.cap < 0 ? base[x] : min(base[x], p.cap);
  }
  const int total = wave_exclusive_scan256(tmp, off, E);
  if (lane == 0) off[E] = total;
  for (int x = lane; x <= E; x += 64) p.offsets[x] = off[x];
  if (p.items) {
    for (int x = lane; x < E; x += 64) tmp[256 + x] = (tmp[x] + p.bm - 1) / p.bm;
    const int nit = wave_exclusive_scan256(tmp + 256, tmp, E);  // tmp[e] = first item of expert e
    if (lane == 0) *p.n_items = nit;
#pragma unroll 1
    for (int x = lane; x < E; x += 64) {
      const int kept = off[x + 1] - off[x], start = tmp[x];
      const int n = (kept + p.bm - 1) / p.bm;
#pragma unroll 1
      for (int i = 0; i < n; ++i) p.items[start + i] = item_of(x, off[x], kept, n, i, p.bm);
    }
  }
#pragma unroll 1
  for (int j = 0; j < nch; ++j) {
    const int i = 64 * j + lane;
    if (i < n) {
      const int v = pr[i];
      place_pair(p, i, v & 255, v >= 0, v >> 8, off);
    }
  }
}

// The same permutation by a whole block, for many pairs: passes of blockDim.x
// pairs in token-major order through rank_pass (which keeps each expert's
// running count in base[], so ranks stay stable in t across passes), then the
// capacity rule, the scan, the tile map (write_tile_map) and the placement, with
// barriers between the phases.  Every thread of the block must call it.
// LDS: base [256], off [257], tmp [512], wcnt [nwaves][256], pr [kSmallMaxPairs].
__device__ void permute_block(const PermArgs& p, const int32_t* idx, const uint16_t* sel, int* base, int* off,
                              int* tmp, int* wcnt, int* pr) {
  const int tid = threadIdx.x, n = p.T * p.k, E = p.E;
  for (int x = tid; x < 256; x += blockDim.x) base[x] = 0;  // ordered by the barriers inside rank_pass
  for (int p0 = 0; p0 < n; p0 += blockDim.x) {
    const int i = p0 + tid;
    const int raw = i < n ? (idx ? idx[i] : (int)sel[i]) : -1;
    const bool valid = raw >= 0 && raw < E;
    const int e = valid ? raw : 0;
    const int r = rank_pass(e, valid, wcnt, base, E);
    if (i < n) pr[i] = valid ? r * 256 + e : -1;
  }
  __syncthreads();
  for (int x = tid; x < E; x += blockDim.x) {
    p.counts[x] = base[x];
    tmp[x] = p.cap < 0 ? base[x] : min(base[x], p.cap);
  }
  __syncthreads();
  if (tid < 64) {
    const int total = wave_exclusive_scan256(tmp, off, E);
    if (tid == 0) off[E] = total;
  }
  __syncthreads();
  for (int x = tid; x <= E; x += blockDim.x) p.offsets[x] = off[x];
  if (p.items) {
    for (int x = tid; x < E; x += blockDim.x) base[x] = tmp[x];  // kept per expert
    write_tile_map(base, off, E, p.bm, p.items, p.n_items, tmp);
  }
  for (int i = tid; i < n; i += blockDim.x) {
    const int v = pr[i];
    place_pair(p, i, v & 255, v >= 0, v >> 8, off);
  }
}

// For T*k <= kSmallMaxPairs (T <= 256), E <= 64 EPL: block b takes tokens tpb*b .. +tpb-1.
// Its threads add the KS K-chunk partial logits of those tokens (each output's
// chunks in order by one lane, or split over KG lanes and added in a fixed
// butterfly); the biases are fetched at entry, so the selection does not wait
// for them.  Wave w scores and selects token tpb*b + w.  One block (T = 1):
// the picks stay in LDS and wave 0 ranks them.  Several blocks: each block
// publishes its topk_idx rows (release fence, then one device-scope increment
// of `arrived`, which the router launch zeroed), and the block that arrives
// last ranks all pairs after an acquire fence: with one wave up to
// kOneWaveMaxPairs pairs, else with the whole block.  do_route = 0: one block
// permutes idx_in the same way.
template <int EPL, bool GRP>
__global__ __launch_bounds__(256) void route_small_kernel(const float* __restrict__ part, int KS, int tpb,
                                                          RouteArgs ra, const int32_t* idx_in, PermArgs pa,
                                                          int do_route, int do_perm, int32_t* arrived) {
  __shared__ float slog[4 * 256];
  __shared__ float sbias[256], ssel[256];
  __shared__ uint16_t sel[kSmallMaxPairs];
  __shared__ int base[256], off[257], tmp[512], pr[kSmallMaxPairs];
  __shared__ int wcnt[4 * 256];
  __shared__ int last;
  const int tid = threadIdx.x, w = tid >> 6;
  const int T = ra.T, E = ra.E;
  const int32_t* pidx = idx_in;  // where the permutation reads the picks
  const uint16_t* psel = nullptr;
  if (do_route) {
    const float lb = (ra.logit_bias && tid < E) ? ra.logit_bias[tid] : 0.f;
    const float sb = (ra.select_bias && tid < E) ? ra.select_bias[tid] : 0.f;
    const int t0 = blockIdx.x * tpb, nt = min(tpb, T - t0), nout = nt * E;
    int KG = 1;
    while (KG < 64 && 2 * KG * nout <= (int)blockDim.x && 2 * KG <= KS) KG *= 2;
    const int g = tid % KG, per = (int)blockDim.x / KG;
    const size_t zs = (size_t)T * E;
    for (int i = tid / KG; i < ((nout + per - 1) / per) * per; i += per) {
      const bool ok = i < nout;
      const size_t src = ok ? (size_t)(t0 + i / E) * E + i % E : 0;
      float acc = 0.f;
      for (int z0 = g; z0 < KS; z0 += 32 * KG) {  // up to 32 loads in flight per lane
        float v[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const int z = z0 + u * KG;
          v[u] = (ok && z < KS) ? part[(size_t)z * zs + src] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 32; ++u)
          if (z0 + u * KG < KS) acc += v[u];
      }
      for (int o = 1; o < KG; o <<= 1) acc += __shfl_xor(acc, o);
      if (ok && g == 0) slog[i] = acc;
    }
    if (tid < E) {
      sbias[tid] = lb;
      ssel[tid] = sb;
    }
    __syncthreads();
    RouteArgs rl = ra;
    if (ra.select_bias) rl.select_bias = ssel;
    const float* bias = ra.logit_bias ? sbias : nullptr;
    const bool one = nt == T;  // a single block (T = 1): the picks stay in LDS, no hand-off
    if (w < nt) {
      float lg[1][EPL];
      load_logits<1, EPL>(lg, slog + w * E, E, E, bias);
      route_tokens<1, EPL, GRP>(lg, rl, t0 + w, 1, one ? sel + w * ra.k : nullptr);
    }
    if (!do_perm) return;
    if (one) {
      __syncthreads();
      pidx = nullptr;
      psel = sel;
    } else {
      __threadfence();  // release this block's topk_idx rows
      __syncthreads();
      if (tid == 0)
        last = __hip_atomic_fetch_add(arrived, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == (int)gridDim.x - 1;
      __syncthreads();
      if (!last) return;
      __threadfence();  // acquire every block's rows
      pidx = ra.idx;
    }
  }
  if (psel && pa.T == 1) {  // the picks of one token, from this kernel's own top-k
    if (w == 0) permute_single_token(pa, psel, off);
  } else if (pa.T * pa.k > kOneWaveMaxPairs) permute_block(pa, pidx, psel, base, off, tmp, wcnt, pr);
  else if (w == 0) permute_one_wave(pa, pidx, psel, base, off, tmp, pr);
}

// ------------------------------------------------------------------ fused router (large T)
// A block takes ra.tiles_per_block consecutive tiles of 16 * MT tokens.  For
// each tile it computes all E logits with MFMA (the four waves split K into
// quarters, and their partial sums are added in LDS in fixed wave order), then
// scores and selects each token (a wave per token) and adds the tile's picks to
// the block's expert histogram, which it writes once at the end.  NB = experts / 16 held
// per wave (compile-time bound, E <= 16 * NB).
template <typename TIN, int MT, int NB, bool GRP>
__global__ __launch_bounds__(256) void router_fused_kernel(const TIN* __restrict__ x, const TIN* __restrict__ wr,
                                                           RouteArgs ra, int32_t* __restrict__ hist) {
  constexpr int EPC = Chunk<TIN>::EPC;
  constexpr int KSTEP = 4 * EPC;
  constexpr int TM = 16 * MT;
  constexpr int LD = 16 * NB + 4;
  constexpr int U = 2;  // steps whose loads are issued together (deeper costs occupancy)
  __shared__ float slog[TM * LD];
  __shared__ uint16_t sel[TM * kMaxK];
  __shared__ int wcnt[4 * 256];
  __shared__ int base[256];
  const int tid = threadIdx.x, lane = lane_id(), w = tid / 64, g = lane >> 4, c = lane & 15;
  const int T = ra.T, E = ra.E, d = ra.d, k = ra.k;
  const int nblk = (E + 15) / 16;
  for (int xx = tid; xx < 256; xx += blockDim.x) base[xx] = 0;  // ordered before use by the barriers below
  for (int tt = 0; tt < ra.tiles_per_block; ++tt) {
    const int t0 = (blockIdx.x * ra.tiles_per_block + tt) * TM;
    if (t0 >= T) break;  // block-uniform
    f32x4 acc[MT][NB];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[m][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const TIN* pa[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) pa[m] = x + (size_t)min(t0 + 16 * m + c, T - 1) * d + g * EPC;
    const TIN* pb = wr + (size_t)min(c, E - 1) * d + g * EPC;   // expert block b adds 16 * b rows
    const int nsteps = d / KSTEP;
    const int s0 = w * nsteps / 4, s1 = (w + 1) * nsteps / 4;
    for (int st = s0; st < s1; st += U) {
      u32x4 av[U][MT], bv[U][NB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (st + u < s1) {
          const int kk = (st + u) * KSTEP;
#pragma unroll
          for (int m = 0; m < MT; ++m) av[u][m] = ld16(pa[m] + kk);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const int row = min(16 * b + c, E - 1) - min(c, E - 1);
            if (b < nblk) bv[u][b] = ld16(pb + (size_t)row * d + kk);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (st + u < s1)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            if (b < nblk)
#pragma unroll
              for (int m = 0; m < MT; ++m) acc[m][b] = Chunk<TIN>::mma(av[u][m], bv[u][b], acc[m][b]);
    }
    // sum the four K quarters in wave order
    for (int ww = 0; ww < 4; ++ww) {
      if (w == ww) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if (b >= nblk) continue;
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float* p = &slog[(16 * m + 4 * g + i) * LD + 16 * b + c];
              *p = ww == 0 ? acc[m][b][i] : *p + acc[m][b][i];
            }
        }
      }
      __syncthreads();
    }
    const int nt = min(TM, T - t0);
    route_rows<(16 * NB + 63) / 64, GRP>(slog, LD, nt, t0, ra, ra.logit_bias, sel, w, 4);
    // the tile's pairs into the block histogram (sel[] is complete only after this barrier; the
    // next tile overwrites slog and sel only after the barriers inside the rank passes)
    __syncthreads();
    const int np = nt * k;
    for (int p0 = 0; p0 < np; p0 += blockDim.x) {
      const int i = p0 + tid;
      const int e = i < np ? (int)sel[i] : 0xFFFF;
      rank_pass(e, e < E, wcnt, base, E);
    }
  }
  __syncthreads();
  for (int xx = tid; xx < E; xx += blockDim.x) hist[(size_t)blockIdx.x * E + xx] = base[xx];
}

// Wide router for large E (bf16, 128 < E <= 256): a block takes 64-token tiles
// (ra.tiles_per_block of them) and its four waves split the experts, wave w
// computing experts 64 w .. 64 w + 63 over the whole K, so the router weight
// (3.7 MB at DeepSeek-V3 size) is read once per 64 tokens instead of once per
// 16.  The tile's token rows go through double-buffered LDS (64 K at a time,
// shared by the four waves); each wave's router rows go straight from memory
// into MFMA operands one stage ahead.  The logits then take the staging
// space, and scoring, top-k and the block histogram follow as in
// router_fused_kernel.
template <bool GRP>
__global__ __launch_bounds__(256, 2) void router_wide_kernel(const bf16* __restrict__ x, const bf16* __restrict__ wr,
                                                             RouteArgs ra, int32_t* __restrict__ hist) {
  constexpr int TM = 64, KS = 128, LDX = KS + 8, LDL = 256 + 4;
  constexpr int XCH = TM * KS / 8 / 256;  // 16-byte token-row chunks a thread stages per step
  constexpr int SMEM = TM * LDL > TM * LDX ? TM * LDL : TM * LDX;  // floats: logits, or two bf16 staging buffers
  __shared__ float smem[SMEM];
  __shared__ uint16_t sel[TM * kMaxK];
  __shared__ int wcnt[4 * 256];
  __shared__ int base[256];
  bf16* const xs = reinterpret_cast<bf16*>(smem);  // [2][TM][LDX] during the K loop
  float* const slog = smem;                        // [TM][LDL] afterwards
  const int tid = threadIdx.x, lane = lane_id(), w = tid / 64, g = lane >> 4, c = lane & 15;
  const int T = ra.T, E = ra.E, d = ra.d, k = ra.k;
  const int nst = d / KS;
  // this lane's router rows (B operand): experts 64 w + 16 nb + c, K offset 8 g of each 32-K slice
  const bf16* pb[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) pb[nb] = wr + (size_t)min(64 * w + 16 * nb + c, E - 1) * d + 8 * g;
  for (int xx = tid; xx < 256; xx += blockDim.x) base[xx] = 0;  // ordered before use by the barriers below
  for (int tt = 0; tt < ra.tiles_per_block; ++tt) {
    const int t0 = (blockIdx.x * ra.tiles_per_block + tt) * TM;
    if (t0 >= T) break;  // block-uniform
    // token-row chunks this thread stages: rows (tid + 256 q) / 16, 16-byte chunk tid % 16
    const bf16* px[XCH];
#pragma unroll
    for (int q = 0; q < XCH; ++q) px[q] = x + (size_t)min(t0 + (tid + 256 * q) / 16, T - 1) * d + 8 * (tid % 16);
    f32x4 acc[4][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) acc[mt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 xr[XCH], b0[4][4], b1[4][4];
    auto load_x = [&](int st) {
#pragma unroll
      for (int q = 0; q < XCH; ++q) xr[q] = ld16(px[q] + st * KS);
    };
    auto store_x = [&](int buf) {
#pragma unroll
      for (int q = 0; q < XCH; ++q)
        *reinterpret_cast<u32x4*>(&xs[(buf * TM + (tid + 256 * q) / 16) * LDX + 8 * (tid % 16)]) = xr[q];
    };
    auto load_w = [&](u32x4 (&bq)[4][4], int st) {
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) bq[sl][nb] = ld16(pb[nb] + st * KS + 32 * sl);
    };
    auto compute = [&](int buf, const u32x4 (&bq)[4][4]) {
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        u32x4 af[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          af[mt] = *reinterpret_cast<const u32x4*>(&xs[(buf * TM + 16 * mt + c) * LDX + 32 * sl + 8 * g]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb) acc[mt][nb] = mma_bf16(af[mt], bq[sl][nb], acc[mt][nb]);
      }
    };
    // two-step ping-pong, one step (128 K) ahead
    load_w(b0, 0);
    load_x(0);
    store_x(0);
    __syncthreads();
    int st = 0;
    for (; st + 2 <= nst; st += 2) {
      load_x(min(st + 1, nst - 1));
      load_w(b1, min(st + 1, nst - 1));
      compute(0, b0);
      store_x(1);
      __syncthreads();
      load_x(min(st + 2, nst - 1));
      load_w(b0, min(st + 2, nst - 1));
      compute(1, b1);
      store_x(0);
      __syncthreads();
    }
    if (st < nst) compute(0, b0);
    __syncthreads();  // every wave is past its last read of the staging space
    // logits into LDS
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) slog[(16 * mt + 4 * g + i) * LDL + 64 * w + 16 * nb + c] = acc[mt][nb][i];
    __syncthreads();
    const int nt = min(TM, T - t0);
    route_rows<4, GRP>(slog, LDL, nt, t0, ra, ra.logit_bias, sel, w, 4);
    __syncthreads();  // sel[] complete; slog free for the next tile after the rank passes' barriers
    const int np = nt * k;
    for (int p0 = 0; p0 < np; p0 += blockDim.x) {
      const int i = p0 + tid;
      const int e = i < np ? (int)sel[i] : 0xFFFF;
      rank_pass(e, e < E, wcnt, base, E);
    }
  }
  __syncthreads();
  for (int xx = tid; xx < E; xx += blockDim.x) hist[(size_t)blockIdx.x * E + xx] = base[xx];
}

// Tile histogram of given indices (for the standalone permute on large T).
__global__ __launch_bounds__(512) void tile_hist_kernel(const int32_t* __restrict__ idx, int T, int k, int E, int rt,
                                                        int32_t* __restrict__ hist) {
  __shared__ int wcnt[8 * 256];
  __shared__ int base[256];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * rt, nt = min(rt, T - t0), np = nt * k;
  for (int x = tid; x < 256; x += blockDim.x) base[x] = 0;
  __syncthreads();
  for (int p0 = 0; p0 < np; p0 += blockDim.x) {
    const int i = p0 + tid;
    int e = 0xFFFF;
    if (i < np) {
      const int v = idx[(size_t)t0 * k + i];
      e = (v >= 0 && v < E) ? v : 0xFFFF;
    }
    rank_pass(e, e < E, wcnt, base, E);
  }
  __syncthreads();
  for (int x = tid; x < E; x += blockDim.x) hist[(size_t)blockIdx.x * E + x] = base[x];
}

// ------------------------------------------------------------------ multi-block permute (large T)
// One block per 64-token tile: expert bases from the tile histograms of the
// tiles before it, totals from all of them, then the tile's pairs are ranked
// and placed.  Block 0 also writes counts, offsets and the tile map.
__global__ __launch_bounds__(512) void permute_multi_kernel(const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ hist, int n_tiles,
                                                            PermArgs pa) {
  __shared__ int wcnt[8 * 256];
  __shared__ int red_b[512], red_t[512];
  __shared__ int base[256], tot[256], kept[256], off[257], tmp[512];
  const int tid = threadIdx.x;
  const int E = pa.E, k = pa.k, T = pa.T, tile = blockIdx.x;
  // partial sums over tiles: thread -> (expert, part)
  const int P = max(1, (int)blockDim.x / E);
  {
    int sb = 0, st = 0;
    const int e = tid % E, part = tid / E;
    if (part < P) {
      // 32 tile rows per batch: the loads are issued together (one batch covers 256 tiles of
      // 64 experts; measured against 8: DeepSeek-V3 T=16384 permute 34 -> 30 us)
      for (int r0 = part; r0 < n_tiles; r0 += 32 * P) {
        int v[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const int r = r0 + u * P;
          v[u] = r < n_tiles ? hist[(size_t)r * E + e] : 0;
        }
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          st += v[u];
          if (r0 + u * P < tile) sb += v[u];
        }
      }
    }
    red_b[tid] = sb;
    red_t[tid] = st;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    int sb = 0, st = 0;
    for (int part = 0; part < P; ++part) {
      sb += red_b[part * E + e];
      st += red_t[part * E + e];
    }
    base[e] = sb;
    tot[e] = st;
    kept[e] = pa.cap < 0 ? st : min(st, pa.cap);
  }
  __syncthreads();
  if (tid < 64) {
    const int s = wave_exclusive_scan256(kept, off, E);
    if (tid == 0) off[E] = s;
  }
  __syncthreads();
  if (tile == 0) {
    for (int x = tid; x < E; x += blockDim.x) pa.counts[x] = tot[x];
    for (int x = tid; x <= E; x += blockDim.x) pa.offsets[x] = off[x];
    if (pa.items) write_tile_map(kept, off, E, pa.bm, pa.items, pa.n_items, tmp);
    if (pa.items_dn) {
      __syncthreads();  // tmp is reused
      write_tile_map(kept, off, E, pa.bm_dn, pa.items_dn, pa.n_items_dn, tmp);
    }
  }
  const int t0 = tile * pa.rt, nt = min(pa.rt, T - t0), np = nt * k;
  for (int p0 = 0; p0 < np; p0 += blockDim.x) {
    const int i = p0 + tid;
    int e = 0xFFFF;
    if (i < np) {
      const int v = idx[(size_t)t0 * k + i];
      e = (v >= 0 && v < E) ? v : 0xFFFF;
    }
    const bool valid = e < E;
    const int r = rank_pass(e, valid, wcnt, base, E);
    if (i < np) place_pair(pa, t0 * k + i, e, valid, r, off);
  }
}

// ------------------------------------------------------------------ tile map from offsets
// For moe_expert_ffn called with caller-provided offsets: clamps them into
// [0, R] (non-decreasing) and writes the tile map.
__global__ __launch_bounds__(256) void tile_map_kernel(const int32_t* __restrict__ offsets, int E, int R, int bm,
                                                       int4* items, int32_t* n_items) {
  __shared__ int off[257], kept[256], tmp[512];
  const int tid = threadIdx.x;
  if (tid == 0) {
    int prev = 0;
    for (int e = 0; e <= E; ++e) {
      int v = e == 0 ? 0 : offsets[e];
      v = min(max(v, prev), R);
      off[e] = v;
      prev = v;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) kept[e] = off[e + 1] - off[e];
  __syncthreads();
  write_tile_map(kept, off, E, bm, items, n_items, tmp);
}

// ------------------------------------------------------------------ host launchers
hipError_t launch_router_partial(int act, const void* x, const void* wr, int T, int d, int E, int kchunk, int KS,
                                 float* part, int32_t* zero, hipStream_t s) {
  dim3 grid((T + 15) / 16, (E + 63) / 64, KS);
  if (act == kF32)
    hipLaunchKernelGGL(router_partial_kernel<float>, grid, dim3(256), 0, s, (const float*)x, (const float*)wr, T, d,
                       E, kchunk, part, zero);
  else
    hipLaunchKernelGGL(router_partial_kernel<bf16>, grid, dim3(256), 0, s, (const bf16*)x, (const bf16*)wr, T, d, E,
                       kchunk, part, zero);
  return hipGetLastError();
}

// the group-limited step is needed (fewer groups kept than there are)
static bool route_groups(const RouteArgs& ra) { return ra.topk_groups > 0 && ra.topk_groups < ra.n_groups; }

hipError_t launch_route_small(const float* part, int KS, const RouteArgs& ra, const int32_t* idx_in,
                              const PermArgs& pa, int do_route, int do_perm, int32_t* arrived, hipStream_t s) {
  const int tpb = route_small_tpb(ra.T);
  const int grid = do_route ? (ra.T + tpb - 1) / tpb : 1;
  auto kern = route_groups(ra)
                  ? (ra.E <= 64 ? route_small_kernel<1, true>
                                : (ra.E <= 128 ? route_small_kernel<2, true> : route_small_kernel<4, true>))
                  : (ra.E <= 64 ? route_small_kernel<1, false>
                                : (ra.E <= 128 ? route_small_kernel<2, false> : route_small_kernel<4, false>));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, s, part, KS, tpb, ra, idx_in, pa, do_route, do_perm, arrived);
  return hipGetLastError();
}

template <bool GRP>
void launch_router_fused_t(int act, const void* x, const void* wr, const RouteArgs& ra, int rt, int32_t* hist,
                           hipStream_t s) {
  const int span = rt * ra.tiles_per_block;
  dim3 grid((ra.T + span - 1) / span);
  const int nb = (ra.E + 15) / 16;
  const bf16 *xb = (const bf16*)x, *wb = (const bf16*)wr;
  if (act == kF32) {
    hipLaunchKernelGGL((router_fused_kernel<float, 1, 16, GRP>), grid, dim3(256), 0, s, (const float*)x,
                       (const float*)wr, ra, hist);
  } else if (rt == 64) {
    hipLaunchKernelGGL(router_wide_kernel<GRP>, grid, dim3(256), 0, s, xb, wb, ra, hist);
  } else if (nb <= 4) {
    hipLaunchKernelGGL((router_fused_kernel<bf16, 1, 4, GRP>), grid, dim3(256), 0, s, xb, wb, ra, hist);
  } else if (nb <= 8) {
    hipLaunchKernelGGL((router_fused_kernel<bf16, 1, 8, GRP>), grid, dim3(256), 0, s, xb, wb, ra, hist);
  } else {
    hipLaunchKernelGGL((router_fused_kernel<bf16, 1, 16, GRP>), grid, dim3(256), 0, s, xb, wb, ra, hist);
  }
}

hipError_t launch_router_fused(int act, const void* x, const void* wr, const RouteArgs& ra, int rt, int32_t* hist,
                               hipStream_t s) {
  if (route_groups(ra)) launch_router_fused_t<true>(act, x, wr, ra, rt, hist, s);
  else launch_router_fused_t<false>(act, x, wr, ra, rt, hist, s);
  return hipGetLastError();
}

hipError_t launch_tile_hist(const int32_t* idx, int T, int k, int E, int rt, int32_t* hist, hipStream_t s) {
  hipLaunchKernelGGL(tile_hist_kernel, dim3((T + rt - 1) / rt), dim3(512), 0, s, idx, T, k, E, rt, hist);
  return hipGetLastError();
}

hipError_t launch_permute_multi(const int32_t* idx, const int32_t* hist, const PermArgs& pa, hipStream_t s) {
  const int n_tiles = (pa.T + pa.rt - 1) / pa.rt;
  hipLaunchKernelGGL(permute_multi_kernel, dim3(n_tiles), dim3(512), 0, s, idx, hist, n_tiles, pa);
  return hipGetLastError();
}

hipError_t launch_tile_map(const int32_t* offsets, int E, int R, int bm, int4* items, int32_t* n_items,
                           hipStream_t s) {
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(256), 0, s, offsets, E, R, bm, items, n_items);
  return hipGetLastError();
}

}  // namespace moe
