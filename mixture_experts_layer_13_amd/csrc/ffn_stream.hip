// Streaming (small-M, decode) expert FFN kernels for gfx950: a block owns one
// tile-map item (<= 64 rows of one expert) and 16 (gate/up) or 64 (down)
// output channels; its waves read their weight slice once, straight from
// memory into MFMA operands, so the weight stream is the whole cost.
#include "ffn_common.hpp"
#include "kernels_f8f8.hpp"

namespace moe {

// Per weight type: K covered by one 16-byte weight load per lane (KSTEP),
// 16-byte activation loads per m-tile per step (AL), steps unrolled (U).
template <typename TW> struct Dec;
template <> struct Dec<float> {
  using TA = float;
  static constexpr int KSTEP = 16, AL = 1, U = 4;
};
template <> struct Dec<bf16> {
  using TA = bf16;
  static constexpr int KSTEP = 32, AL = 1, U = 4;
};
template <> struct Dec<INT4> {
  using TA = bf16;
  static constexpr int KSTEP = 128, AL = 4, U = 2;
};
template <> struct Dec<FP8> {
  using TA = bf16;
  static constexpr int KSTEP = 64, AL = 2, U = 8;
};

// Weight bytes of one output channel n (row n of an [N][K] matrix, Kb bytes
// per row) as one lane sees them: the row is read in 64-byte chunks, the lane
// taking bytes 16g..16g+15 of each (g = lane / 16; lane % 16 = n % 16).
//  - row layout: chunk j of row n at n*Kb + 64j;
//  - tiled layout: the 16-row x 64-byte fragment (n/16, j) is one contiguous
//    KB at ((n/16)*(Kb/64) + j)*1024, lane-major: bytes 16*(16g + c).. hold
//    row 16*(n/16) + c, bytes 16g.. of the chunk, so one wave-wide 16-byte load
//    of a fragment reads 1 KB of consecutive addresses.
// Weight bytes are read exactly once per forward: non-temporal 16-byte loads
// (a plain streaming read of 4 GiB, csrc/probe.hip: 6.5-7.0 TB/s against
// 5.8-6.2 TB/s with ordinary loads, GPU to GPU).
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

struct WRow {
  const uint8_t* p;  // chunk 0 of this lane
  int shift;         // log2 of the bytes from chunk j to chunk j + 1
  __device__ WRow() {}
  __device__ WRow(const void* m, int n, int Kb, int g, int tiled) {
    const int c = n & 15;
    p = (const uint8_t*)m + (tiled ? (size_t)(n - c) * Kb + 256 * g + 16 * c : (size_t)n * Kb + 16 * g);
    shift = tiled ? 10 : 6;
  }
  __device__ u32x4 chunk(int j) const { return ld16_stream(p + ((uint32_t)j << shift)); }
};

// One weight row of a [N][K] matrix as seen by one lane; a step of KSTEP K
// values is one 64-byte chunk of the row.  Lane K order inside a step:
// bf16 k = kb + 8g + i; f32 k = kb + 4g + i; INT4 k = kb + 32g + 8s + i
// (s = dword of the 16-byte load); FP8 k = kb + 16g + i (byte i of the load).
template <typename TW> struct BRow {
  WRow w;
  const uint16_t* s;  // INT4 scales of the row (bf16, one per 128-K group)
  float cs;           // FP8: the channel's scale
  __device__ BRow() {}
  __device__ BRow(const void* m, int n, int K, int g, const void* sc, int tiled)
      : w(m, n, row_bytes<TW>(K), g, tiled),
        s(std::is_same<TW, INT4>::value ? (const uint16_t*)sc + (size_t)n * (K / kInt4Group) : nullptr),
        cs(std::is_same<TW, FP8>::value ? ((const float*)sc)[n] : 1.f) {}
  __device__ u32x4 load(int kb) const { return w.chunk(kb / Dec<TW>::KSTEP); }
  __device__ float scale(int kb) const {
    if constexpr (std::is_same<TW, INT4>::value) return bf16_bits_to_f32(s[kb / kInt4Group]);
    else if constexpr (std::is_same<TW, FP8>::value) return cs;
    else return 1.f;
  }
};

template <typename TW>
__device__ __forceinline__ f32x4 dstep(const u32x4 (&av)[Dec<TW>::AL], u32x4 b, float sc, f32x4 acc);
template <> __device__ __forceinline__ f32x4 dstep<float>(const u32x4 (&av)[1], u32x4 b, float, f32x4 acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = mma_f32(__uint_as_float(av[0][i]), __uint_as_float(b[i]), acc);
  return acc;
}
template <> __device__ __forceinline__ f32x4 dstep<bf16>(const u32x4 (&av)[1], u32x4 b, float, f32x4 acc) {
  return mma_bf16(av[0], b, acc);
}
// INT4: one 128-K scale group.  The MFMAs take the nibbles as 136 + q (see
// int4x8_to_bf16_off136) on an accumulator that starts at -136 sum(x) over the
// group (xn), so they leave sum(q x); the group scale is applied once.
__device__ __forceinline__ f32x4 dstep_int4(const u32x4 (&av)[4], u32x4 b, float sc, f32x4 xn, f32x4 acc) {
  f32x4 t = xn;
#pragma unroll
  for (int s = 0; s < 4; ++s) t = mma_bf16(av[s], int4x8_to_bf16_off136(b[s]), t);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, t[i], acc[i]);
  return acc;
}
// FP8: sixteen E4M3 bytes (K = 16g + i) become two bf16 operands (bytes 0-7 and
// 8-15; every E4M3 value is exact in bf16) by the chip's conversion, two bytes
// per instruction; the products of one step are summed from zero and the
// channel scale is applied once per step.
template <bool HI> __device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ f32x4 dstep_fp8(const u32x4 (&av)[2], u32x4 b, float sc, f32x4 acc) {
  f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 bb = {fp8x2_to_bf16x2<false>(b[2 * h]), fp8x2_to_bf16x2<true>(b[2 * h]),
                      fp8x2_to_bf16x2<false>(b[2 * h + 1]), fp8x2_to_bf16x2<true>(b[2 * h + 1])};
    t = mma_bf16(av[h], bb, t);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, t[i], acc[i]);
  return acc;
}

// -136 times the sum over the group of each activation row, in the MFMA
// output layout (an all-ones weight operand: every column holds the row sum).
__device__ __forceinline__ f32x4 int4_group_offset(const u32x4 (&av)[4]) {
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) x = mma_bf16(av[s], ones, x);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] *= -136.f;
  return x;
}

// 16-channel tiles per wave of the streaming kernels (channels per block:
// gate/up 16 NT, down 64 NT; the host grid uses the same numbers)
template <typename TW> constexpr int stream_tiles() { return std::is_same<TW, INT4>::value ? 2 : 1; }
static_assert(Dec<FP8>::AL == 2 && Dec<FP8>::KSTEP == 64, "FP8 steps: 16 bytes per lane, two bf16 operands");
int stream_channels_per_block(bool gateup, int wdt) { return (gateup ? 16 : 64) * (wdt == kINT4 ? 2 : 1); }
// waves sharing one channel tile of the streaming down GEMM (each a contiguous part of K):
// bf16 and FP8 weights from two tokens on; one token keeps whole-K waves, the order of the
// single-token down + combine launch
int stream_down_split(int wdt, int T) { return (T > 1 && (wdt == kBF16 || wdt == kFP8)) ? 2 : 1; }

// GATEUP: h[row][n] = silu(A Wg^T) * (A Wu^T); else y[row][n] = A Wd^T.
// A block owns one item (<= 16 * MT rows of one expert).  A wave covers NT
// tiles of 16 channels (INT4: two, so one set of activation registers feeds
// twice the weight bytes in flight; else one).  Gate/up (K = d, large): the
// four waves split K into quarters for the same channels and add their
// partial sums in LDS in wave order.  Down (K = ffn): DKS waves share a
// channel tile, each over a contiguous part of K, added in LDS in wave order, so
// a block covers 4 / DKS times NT tiles (DKS = 2 for bf16 and FP8 weights from two
// tokens on, measured on graph replays of one GPU: FP8 OLMoE-shaped T=64 99.9 ->
// 97.8 us, T=8 63.0 -> 62.3 us, bf16 within noise; else 1, the whole K per wave,
// which one token keeps: the order of the single-token down + combine).  Steps are unrolled
// U deep so each lane keeps U weight loads per matrix and tile in flight.
// grid: items_max * (N / channels per block) routed blocks, then the shared blocks.
// PIPE (bf16, one row tile): two register buffers of PU steps, the loads of the next PU steps
// in flight while the current ones are multiplied; the same steps in the same order, so the
// same sums.  Measured (graph replays, one GPU): it pays for single-row items, where a wave has
// little to multiply between its loads (layers with the single-token down + combine: OLMoE-shaped
// T=1 39.8 -> 38.7 us, DeepSeek-V3-shaped T=1 151.8 -> 147.6 us, DeepSeek-V2-Lite-shaped 49.8 ->
// 48.7 us), and costs from 32 rows per expert on (OLMoE T=32 136.7 -> 138.5 us, T=64 154.4 ->
// 157.1 us), so the host takes it for T = 1 only.  The same buffers in the single-token down +
// combine launch were slower (DeepSeek-V3-shaped T=1 147.6 -> 148.3 / 150.3 us with 8 / 4 steps
// per buffer).
// A8 (FP8 weights, FP8 activations at decode sizes): the activation rows hold the E4M3 codes of x
// (gate/up) or h (down) as exact bf16 values, and the epilogue multiplies each row's sums by its
// fp32 row scale (qa.xs by token for gate/up, qa.hs / qa.hshs by row for down) before SwiGLU
// or the store.
template <typename TW, bool GATEUP, int MT, bool PIPE = false, int DKS = 1, bool A8 = false>
__global__ __launch_bounds__(256) void ffn_stream_kernel(FfnArgs a, A8Args qa) {
  using D = Dec<TW>;
  using TA = typename D::TA;
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int NT = stream_tiles<TW>();
  constexpr int KSPLIT = GATEUP ? 4 : DKS;       // waves sharing one channel tile (K parts)
  constexpr int CPB = 16 * NT * (4 / KSPLIT);     // channels per block
  constexpr int NRED = KSPLIT > 1 ? (4 / KSPLIT) * (KSPLIT - 1) : 1;  // partial-sum slots
  // steps whose loads go out together (per step: weights, scales, then activations, so a step's
  // MFMAs can start while later steps land).  Measured on decode layers: INT4 gate/up 1 (its
  // small register footprint keeps 5 blocks per CU), INT4 down 2, bf16 16 / 8 / 4 for items of
  // 16 / 32 / 64 rows
  constexpr int U = std::is_same<TW, INT4>::value  ? (GATEUP ? 1 : 2)
                    : std::is_same<TW, FP8>::value ? (MT == 1 ? 4 : (MT == 2 ? 2 : 1))
                                                   : (MT == 1 ? 16 : (MT == 2 ? 8 : 4));
  constexpr int AL = D::AL, KSTEP = D::KSTEP;
  constexpr int PU = 4;  // PIPE: steps per register buffer
  static_assert(!PIPE || (std::is_same<TW, bf16>::value && MT == 1), "PIPE: bf16, one row tile");
  __shared__ f32x4 red[NRED][NM][NT][MT][64];
  const int lane = lane_id(), w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;

  const int Nr = GATEUP ? a.F : a.d;
  const int Ns = GATEUP ? a.S * a.FS : a.d;
  const int nbr = Nr / CPB, nbs = Ns / CPB;
  const int routed_blocks = a.items_max * nbr;
  int bid = blockIdx.x, e = 0, row0, mrows, nb;
  const bool shared = bid >= routed_blocks;
  if (!shared) {
    const int slot = bid / nbr;
    nb = bid - slot * nbr;
    if (slot >= routed_items(a) || !load_item(a, slot, e, row0, mrows)) return;
  } else {
    bid -= routed_blocks;
    const int slot = bid / nbs;
    nb = bid - slot * nbs;
    row0 = slot * a.bm;
    mrows = min(a.bm, a.T - row0);
  }
  const int nmt = (mrows + 15) / 16;
  const int kpart = w % KSPLIT, tgrp = w / KSPLIT;  // K part, channel tile group of this wave
  const int n0 = nb * CPB + 16 * NT * tgrp + c;     // channel of tile j: n0 + 16 j

  const int K = GATEUP ? a.d : (shared ? a.FS : a.F);  // K of one segment
  const int nseg = (!GATEUP && shared) ? a.S : 1;
  // weight rows first: their loads do not wait for the activation row lookup
  const void* m0 = GATEUP ? (shared ? a.shg : expert_mat<TW>(a.wg, e, a.F, a.d))
                          : (shared ? a.shd : expert_mat<TW>(a.wd, e, a.d, K));
  const void* s0 = GATEUP ? (shared ? a.shsg : expert_scales_of<TW>(a.sg, e, a.F, a.d))
                          : (shared ? a.shsd : expert_scales_of<TW>(a.sd, e, a.d, K));
  const void* m1 = GATEUP ? (shared ? a.shu : expert_mat<TW>(a.wu, e, a.F, a.d)) : m0;
  const void* s1p = GATEUP ? (shared ? a.shsu : expert_scales_of<TW>(a.su, e, a.F, a.d)) : s0;
  BRow<TW> b0[NT], b1[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    b0[j] = BRow<TW>(m0, n0 + 16 * j, K, g, s0, a.wtiled);
    b1[j] = BRow<TW>(m1, n0 + 16 * j, K, g, s1p, a.wtiled);
  }

  // activation rows (clamped into the item so every load is in bounds)
  const TA* arow[MT];
  const int Kfull = GATEUP ? a.d : (shared ? a.S * a.FS : a.F);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(16 * mt + c, mrows - 1);
    if (GATEUP) {
      int tok = shared ? row0 + r : a.row_token[row0 + r];
      tok = min(max(tok, 0), a.T - 1);
      arow[mt] = (const TA*)a.x + (size_t)tok * a.d;
    } else {
      arow[mt] = (const TA*)(shared ? a.hsh : a.h) + (size_t)(row0 + r) * Kfull;
    }
  }

  f32x4 acc[NM][NT][MT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[m][j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int seg = 0; seg < nseg; ++seg) {
    if (seg > 0) {  // next slab of the shared down projection: [S][d][FS]
#pragma unroll
      for (int j = 0; j < NT; ++j)
        b0[j] = b1[j] = BRow<TW>(expert_mat<TW>(a.shd, seg, a.d, K), n0 + 16 * j, K, g,
                                 expert_scales_of<TW>(a.shsd, seg, a.d, K), a.wtiled);
    }
    const int aoff = seg * K;
    const int nsteps = K / KSTEP;
    const int s0 = kpart * nsteps / KSPLIT, s1 = (kpart + 1) * nsteps / KSPLIT;
    if constexpr (PIPE) {
      struct Buf {
        u32x4 bq[NM][NT][PU];
        u32x4 av[MT][PU][AL];
      };
      auto issue = [&](int st, Buf& b) {
#pragma unroll
        for (int u = 0; u < PU; ++u)
          if (st + u < s1) {
            const int kb = (st + u) * KSTEP;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
              b.bq[0][j][u] = b0[j].load(kb);
              if (NM > 1) b.bq[NM - 1][j][u] = b1[j].load(kb);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int q = 0; q < AL; ++q) b.av[mt][u][q] = ld16(arow[mt] + aoff + kb + (KSTEP / 4) * g + 8 * q);
          }
      };
      auto consume = [&](int st, const Buf& b) {
#pragma unroll
        for (int u = 0; u < PU; ++u)
          if (st + u < s1)
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                  acc[m][j][mt] = dstep<TW>(b.av[mt][u], b.bq[m][j][u], 1.f, acc[m][j][mt]);
      };
      Buf A, B;
      if (s0 < s1) issue(s0, A);
#pragma unroll 1
      for (int st = s0; st < s1; st += 2 * PU) {
        if (st + PU < s1) issue(st + PU, B);
        consume(st, A);
        if (st + 2 * PU < s1) issue(st + 2 * PU, A);
        if (st + PU < s1) consume(st + PU, B);
      }
      continue;
    }
#pragma unroll 1  // U-deep unroll inside already; a further unroll only costs occupancy
    for (int st = s0; st < s1; st += U) {
      u32x4 bq[NM][NT][U];
      float sc[NM][NT][U];
      u32x4 av[MT][U][AL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (st + u < s1) {
          const int kb = (st + u) * KSTEP;
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            bq[0][j][u] = b0[j].load(kb);
            sc[0][j][u] = b0[j].scale(kb);
            if (NM > 1) {
              bq[NM - 1][j][u] = b1[j].load(kb);
              sc[NM - 1][j][u] = b1[j].scale(kb);
            }
          }
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (mt < nmt)
#pragma unroll
              for (int q = 0; q < AL; ++q)
                av[mt][u][q] = ld16(arow[mt] + aoff + kb + (KSTEP / 4) * g + 8 * q);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (st + u < s1) {
          if constexpr (std::is_same<TW, INT4>::value) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              if (mt < nmt) {
                const f32x4 xn = int4_group_offset(av[mt][u]);  // shared by gate and up
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                  for (int j = 0; j < NT; ++j)
                    acc[m][j][mt] = dstep_int4(av[mt][u], bq[m][j][u], sc[m][j][u], xn, acc[m][j][mt]);
              }
          } else if constexpr (std::is_same<TW, FP8>::value) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                  if (mt < nmt) acc[m][j][mt] = dstep_fp8(av[mt][u], bq[m][j][u], sc[m][j][u], acc[m][j][mt]);
          } else {
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                  if (mt < nmt) acc[m][j][mt] = dstep<TW>(av[mt][u], bq[m][j][u], sc[m][j][u], acc[m][j][mt]);
          }
        }
      }
    }
  }

  if (KSPLIT > 1) {
    // add the K parts of each channel tile (fixed order) in its part-0 wave
    if (kpart > 0) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (mt < nmt) red[tgrp * (KSPLIT - 1) + kpart - 1][m][j][mt][lane] = acc[m][j][mt];
    }
    __syncthreads();
    if (kpart != 0) return;
#pragma unroll
    for (int p = 1; p < KSPLIT; ++p)
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (mt < nmt) acc[m][j][mt] = acc[m][j][mt] + red[tgrp * (KSPLIT - 1) + p - 1][m][j][mt][lane];
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt >= nmt) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mt + 4 * g + i;
      if (r >= mrows) continue;
      float rs = 1.f;
      if constexpr (A8) {
        if (GATEUP) {
          int tok = shared ? row0 + r : a.row_token[row0 + r];
          tok = min(max(tok, 0), a.T - 1);
          rs = qa.xs[tok];
        } else {
          rs = (shared ? qa.hshs : qa.hs)[row0 + r];
        }
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int n = n0 + 16 * j;
        if (GATEUP) {
          float gv = acc[0][j][mt][i], uv = acc[NM - 1][j][mt][i];
          if constexpr (A8) {
            gv *= rs;
            uv *= rs;
          }
          const float hv = silu(gv) * uv;
          TA* hout = (TA*)(shared ? a.hsh : a.h);
          hout[(size_t)(row0 + r) * (shared ? Ns : Nr) + n] = from_f32<TA>(hv);
        } else {
          float yv = acc[0][j][mt][i];
          if constexpr (A8) yv *= rs;
          TA* yout = (TA*)(shared ? a.ysh : a.y);
          yout[(size_t)(row0 + r) * a.d + n] = from_f32<TA>(yv);
        }
      }
    }
  }
}


// ------------------------------------------------------------------ one token: down + combine
// For a single token (T = 1) the down projection and the weighted combine are one launch:
// block b covers output channels 16 NT b .. +16 NT - 1; wave j < k runs pick j's h row
// through its expert's down rows (what one wave of the down kernel above computes for
// those channels: the same steps in the same K order, so the same fp32 sums) and wave k,
// when there are shared experts, the shared slab (all S segments in order).  Each wave
// rounds its row to the activation type, as the down kernel's store does; wave 0 then adds
// the rows as the combine kernel does: fp32, gate-weighted fma in pick order, picks without
// a row (dropped) skipped, the shared row added last.  No y rows, no combine launch.
template <typename TW>
__global__ __launch_bounds__(64 * (kMaxK + 1)) void down_combine_one_kernel(
    FfnArgs a, const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ slot_row,
    const float* __restrict__ gw, void* __restrict__ out, int k) {
  using D = Dec<TW>;
  using TA = typename D::TA;
  constexpr int NT = stream_tiles<TW>();
  constexpr int CPW = 16 * NT;  // channels per block (one wave's channel tiles)
  // steps whose loads go out together; measured for this launch (graph replays, one GPU): bf16
  // 16 / 8 / 4 took OLMoE-shaped T=1 to 45.8 / 40.5 / 39.5 us and DeepSeek-V3-shaped T=1 to
  // 174 / 151.7 / 151.1 us (five launches: 41.4 and 153.8), DeepSeek-V2-Lite-shaped T=1 to
  // 56.1 / 50.5 / 53.1 us (five launches: 52.3)
  constexpr int U = std::is_same<TW, INT4>::value ? 2 : (std::is_same<TW, FP8>::value ? 4 : 8);
  constexpr int AL = D::AL, KSTEP = D::KSTEP;
  __shared__ float ys[kMaxK + 1][CPW];
  __shared__ int has[kMaxK + 1];
  const int lane = lane_id(), w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const bool sh = w == k;  // the shared experts' wave (launched only when S > 0)
  const int r = sh ? 0 : slot_row[w];
  const bool ok = sh || (unsigned)r < (unsigned)a.R;
  if (ok) {
    const int e = sh ? 0 : min(max(topk_idx[w], 0), a.E - 1);
    const int K = sh ? a.FS : a.F, nseg = sh ? a.S : 1;
    const TA* arow = sh ? (const TA*)a.hsh : (const TA*)a.h + (size_t)r * a.F;
    const int n0 = blockIdx.x * CPW + c;
    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int seg = 0; seg < nseg; ++seg) {
      const void* m = sh ? expert_mat<TW>(a.shd, seg, a.d, K) : expert_mat<TW>(a.wd, e, a.d, K);
      const void* sc0 = sh ? expert_scales_of<TW>(a.shsd, seg, a.d, K) : expert_scales_of<TW>(a.sd, e, a.d, K);
      BRow<TW> b[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) b[j] = BRow<TW>(m, n0 + 16 * j, K, g, sc0, a.wtiled);
      const int aoff = seg * K, nsteps = K / KSTEP;
#pragma unroll 1
      for (int st = 0; st < nsteps; st += U) {
        u32x4 bq[NT][U];
        float sc[NT][U];
        u32x4 av[U][AL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (st + u < nsteps) {
            const int kb = (st + u) * KSTEP;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
              bq[j][u] = b[j].load(kb);
              sc[j][u] = b[j].scale(kb);
            }
#pragma unroll
            for (int q = 0; q < AL; ++q) av[u][q] = ld16(arow + aoff + kb + (KSTEP / 4) * g + 8 * q);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (st + u < nsteps) {
            if constexpr (std::is_same<TW, INT4>::value) {
              const f32x4 xn = int4_group_offset(av[u]);
#pragma unroll
              for (int j = 0; j < NT; ++j) acc[j] = dstep_int4(av[u], bq[j][u], sc[j][u], xn, acc[j]);
            } else if constexpr (std::is_same<TW, FP8>::value) {
#pragma unroll
              for (int j = 0; j < NT; ++j) acc[j] = dstep_fp8(av[u], bq[j][u], sc[j][u], acc[j]);
            } else {
#pragma unroll
              for (int j = 0; j < NT; ++j) acc[j] = dstep<TW>(av[u], bq[j][u], sc[j][u], acc[j]);
            }
          }
        }
      }
    }
    // row 0 of the MFMA output (every A row is the token's row): lanes 0..15, element 0
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < NT; ++j) ys[w][16 * j + c] = (float)from_f32<TA>(acc[j][0]);
    }
  }
  if (lane == 0) has[w] = ok;
  __syncthreads();
  if (w == 0 && lane < CPW) {
    float o = 0.f;
    for (int j = 0; j < k; ++j)
      if (has[j]) o = fmaf(gw[j], ys[j][lane], o);
    if (a.S > 0) o += ys[k][lane];
    ((TA*)out)[blockIdx.x * CPW + lane] = from_f32<TA>(o);
  }
}

hipError_t launch_down_combine_one(int wdt, const FfnArgs& a, const int32_t* topk_idx, const int32_t* slot_row,
                                   const float* gw, void* out, int k, hipStream_t s) {
  const int cpw = stream_channels_per_block(false, wdt) / 4;  // one wave's channels
  const dim3 grid(a.d / cpw), block(64 * (k + (a.S > 0 ? 1 : 0)));
  if (wdt == kF32)
    hipLaunchKernelGGL(down_combine_one_kernel<float>, grid, block, 0, s, a, topk_idx, slot_row, gw, out, k);
  else if (wdt == kBF16)
    hipLaunchKernelGGL(down_combine_one_kernel<bf16>, grid, block, 0, s, a, topk_idx, slot_row, gw, out, k);
  else if (wdt == kFP8)
    hipLaunchKernelGGL(down_combine_one_kernel<FP8>, grid, block, 0, s, a, topk_idx, slot_row, gw, out, k);
  else
    hipLaunchKernelGGL(down_combine_one_kernel<INT4>, grid, block, 0, s, a, topk_idx, slot_row, gw, out, k);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launch
template <bool GATEUP, int MT>
static void launch_stream(int wdt, const FfnArgs& a, int grid, hipStream_t s) {
  if (MT == 1 && wdt == kBF16 && a.T == 1)
    hipLaunchKernelGGL((ffn_stream_kernel<bf16, GATEUP, 1, true>), dim3(grid), dim3(256), 0, s, a, A8Args{});
  else if (wdt == kF32)
    hipLaunchKernelGGL((ffn_stream_kernel<float, GATEUP, MT>), dim3(grid), dim3(256), 0, s, a, A8Args{});
  else if (wdt == kBF16 && !GATEUP && stream_down_split(wdt, a.T) == 2)
    hipLaunchKernelGGL((ffn_stream_kernel<bf16, GATEUP, MT, false, 2>), dim3(grid), dim3(256), 0, s, a, A8Args{});
  else if (wdt == kBF16)
    hipLaunchKernelGGL((ffn_stream_kernel<bf16, GATEUP, MT>), dim3(grid), dim3(256), 0, s, a, A8Args{});
  else if (wdt == kFP8 && !GATEUP && stream_down_split(wdt, a.T) == 2)
    hipLaunchKernelGGL((ffn_stream_kernel<FP8, GATEUP, MT, false, 2>), dim3(grid), dim3(256), 0, s, a, A8Args{});
  else if (wdt == kFP8)
    hipLaunchKernelGGL((ffn_stream_kernel<FP8, GATEUP, MT>), dim3(grid), dim3(256), 0, s, a, A8Args{});
  else
    hipLaunchKernelGGL((ffn_stream_kernel<INT4, GATEUP, MT>), dim3(grid), dim3(256), 0, s, a, A8Args{});
}

// FP8 weights with FP8 activations at decode sizes (the down GEMM split as for FP8 weights)
template <bool GATEUP, int MT>
static void launch_stream_a8(const FfnArgs& a, const A8Args& q, int grid, hipStream_t s) {
  if (!GATEUP && stream_down_split(kFP8, a.T) == 2)
    hipLaunchKernelGGL((ffn_stream_kernel<FP8, GATEUP, MT, false, 2, true>), dim3(grid), dim3(256), 0, s, a, q);
  else
    hipLaunchKernelGGL((ffn_stream_kernel<FP8, GATEUP, MT, false, 1, true>), dim3(grid), dim3(256), 0, s, a, q);
}

void launch_stream_ffn_a8(bool gateup, const FfnArgs& a, const A8Args& q, int grid, hipStream_t s) {
  const int mt = a.bm <= 16 ? 1 : (a.bm <= 32 ? 2 : 4);
  if (gateup) {
    if (mt == 1) launch_stream_a8<true, 1>(a, q, grid, s);
    else if (mt == 2) launch_stream_a8<true, 2>(a, q, grid, s);
    else launch_stream_a8<true, 4>(a, q, grid, s);
  } else {
    if (mt == 1) launch_stream_a8<false, 1>(a, q, grid, s);
    else if (mt == 2) launch_stream_a8<false, 2>(a, q, grid, s);
    else launch_stream_a8<false, 4>(a, q, grid, s);
  }
}

// items of <= 16, 32 or 64 rows take 1, 2 or 4 row tiles of 16
void launch_stream_ffn(bool gateup, int wdt, const FfnArgs& a, int grid, hipStream_t s) {
  const int mt = a.bm <= 16 ? 1 : (a.bm <= 32 ? 2 : 4);
  if (gateup) {
    if (mt == 1) launch_stream<true, 1>(wdt, a, grid, s);
    else if (mt == 2) launch_stream<true, 2>(wdt, a, grid, s);
    else launch_stream<true, 4>(wdt, a, grid, s);
  } else {
    if (mt == 1) launch_stream<false, 1>(wdt, a, grid, s);
    else if (mt == 2) launch_stream<false, 2>(wdt, a, grid, s);
    else launch_stream<false, 4>(wdt, a, grid, s);
  }
}

}  // namespace moe
