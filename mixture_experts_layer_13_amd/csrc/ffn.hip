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
//  - streaming kernels (small M, decode): a block owns one item (<= 64 rows of
//    one expert) and 16 output channels; its four waves split K, read their
//    weight slice once straight from HBM into MFMA operands and reduce
//    through LDS.  The weight stream is the whole cost here.
//  - tiled kernels (large M, prefill): 128 x 128 MFMA tiles with A and B
//    staged through double-buffered LDS, K tiles of 64.
// The gate/up kernel fuses the SwiGLU epilogue silu(x Wg) * (x Wu) and writes
// the bf16 (fp32 for fp32 layers) intermediate h; the down kernel writes
// y_rows.  INT4 weights (two's-complement nibbles, bf16 scale per 128-K group)
// are dequantised in-kernel.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(bf16)lo, (bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Eight two's-complement nibbles (element i in bits 4i..4i+3) -> eight exact
// bf16 values.  Flipping bit 3 of each nibble gives q + 8; OR-ing that into
// the mantissa of 2^23 and subtracting 2^23 + 8 yields q exactly in fp32.
__device__ __forceinline__ u32x4 int4x8_to_bf16(uint32_t w) {
  const uint32_t x = w ^ 0x88888888u;
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float lo = __uint_as_float(0x4B000000u | ((x >> (8 * p)) & 0xFu)) - 8388616.0f;
    const float hi = __uint_as_float(0x4B000000u | ((x >> (8 * p + 4)) & 0xFu)) - 8388616.0f;
    r[p] = pack_bf16x2(lo, hi);
  }
  return r;
}

// Same, times the group scale, rounded once to bf16 (operand of the tiled kernels).
__device__ __forceinline__ u32x4 int4x8_to_bf16_scaled(uint32_t w, float sc) {
  const uint32_t x = w ^ 0x88888888u;
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float lo = (__uint_as_float(0x4B000000u | ((x >> (8 * p)) & 0xFu)) - 8388616.0f) * sc;
    const float hi = (__uint_as_float(0x4B000000u | ((x >> (8 * p + 4)) & 0xFu)) - 8388616.0f) * sc;
    r[p] = pack_bf16x2(lo, hi);
  }
  return r;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// ------------------------------------------------------------------ streaming (small-M) kernels
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

// Weight bytes of one output channel n (row n of an [N][K] matrix, Kb bytes
// per row) as one lane sees them: the row is read in 64-byte chunks, the lane
// taking bytes 16g..16g+15 of each (g = lane / 16; lane % 16 = n % 16).
//  - row layout: chunk j of row n at n*Kb + 64j;
//  - tiled layout: the 16-row x 64-byte fragment (n/16, j) is one contiguous
//    KB at ((n/16)*(Kb/64) + j)*1024, lane-major: bytes 16*(16g + c).. hold
//    row 16*(n/16) + c, bytes 16g.. of the chunk, so one wave-wide 16-byte load
//    of a fragment reads 1 KB of consecutive addresses.
struct WRow {
  const uint8_t* p;  // chunk 0 of this lane
  int shift;         // log2 of the bytes from chunk j to chunk j + 1
  __device__ WRow(const void* m, int n, int Kb, int g, int tiled) {
    const int c = n & 15;
    p = (const uint8_t*)m + (tiled ? (size_t)(n - c) * Kb + 256 * g + 16 * c : (size_t)n * Kb + 16 * g);
    shift = tiled ? 10 : 6;
  }
  __device__ u32x4 chunk(int j) const { return ld16(p + ((uint32_t)j << shift)); }
};

// bytes of one K-contiguous weight row
template <typename TW> __device__ constexpr int row_bytes(int K) { return K * (int)sizeof(TW); }
template <> __device__ constexpr int row_bytes<INT4>(int K) { return K / 2; }

// One weight row of a [N][K] matrix as seen by one lane; a step of KSTEP K
// values is one 64-byte chunk of the row.  Lane K order inside a step:
// bf16 k = kb + 8g + i; f32 k = kb + 4g + i; INT4 k = kb + 32g + 8s + i
// (s = dword of the 16-byte load).
template <typename TW> struct BRow {
  WRow w;
  const uint16_t* s;  // INT4 scales of the row (bf16, one per 128-K group)
  __device__ BRow(const void* m, int n, int K, int g, const void* sc, int tiled)
      : w(m, n, row_bytes<TW>(K), g, tiled),
        s(std::is_same<TW, INT4>::value ? (const uint16_t*)sc + (size_t)n * (K / kInt4Group) : nullptr) {}
  __device__ u32x4 load(int kb) const { return w.chunk(kb / Dec<TW>::KSTEP); }
  __device__ float scale(int kb) const {
    if constexpr (std::is_same<TW, INT4>::value) return bf16_bits_to_f32(s[kb / kInt4Group]);
    else return 1.f;
  }
};

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
__device__ __forceinline__ const void* expert_scales(const void* b, int e, int N, int K) {
  return b ? (const void*)((const uint16_t*)b + (size_t)e * N * (K / kInt4Group)) : nullptr;
}

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
template <> __device__ __forceinline__ f32x4 dstep<INT4>(const u32x4 (&av)[4], u32x4 b, float sc, f32x4 acc) {
  f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) t = mma_bf16(av[s], int4x8_to_bf16(b[s]), t);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc, t[i], acc[i]);
  return acc;
}

// GATEUP: h[row][n] = silu(A Wg^T) * (A Wu^T); else y[row][n] = A Wd^T.
// A block owns one item (<= 16 * MT rows of one expert).  Gate/up (K = d,
// large): the four waves split K into quarters for the same 16 channels and
// add their partial sums in LDS in wave order.  Down (K = ffn): each wave owns
// 16 channels over the whole K, so a block covers 64.  Steps are unrolled U
// deep so each lane keeps U weight loads per matrix in flight.
// grid: items_max * (N / channels per block) routed blocks, then the shared blocks.
template <typename TW, bool GATEUP, int MT>
__global__ __launch_bounds__(256) void ffn_stream_kernel(FfnArgs a) {
  using D = Dec<TW>;
  using TA = typename D::TA;
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int KSPLIT = GATEUP ? 4 : 1;         // waves sharing one channel block
  constexpr int CPB = 16 * (4 / KSPLIT);          // channels per block
  constexpr int U = (std::is_same<TW, INT4>::value || MT == 4) ? 4 : 8;
  constexpr int AL = D::AL, KSTEP = D::KSTEP;
  __shared__ f32x4 red[KSPLIT > 1 ? 3 : 1][NM][MT][64];
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
    if (slot >= *a.n_items) return;
    const int4 it = a.items[slot];
    e = it.x;
    row0 = it.y;
    mrows = it.z;
  } else {
    bid -= routed_blocks;
    const int slot = bid / nbs;
    nb = bid - slot * nbs;
    row0 = slot * a.bm;
    mrows = min(a.bm, a.T - row0);
  }
  const int nmt = (mrows + 15) / 16;
  const int kpart = KSPLIT > 1 ? w : 0;
  const int n = nb * CPB + (KSPLIT > 1 ? 0 : 16 * w) + c;

  const int K = GATEUP ? a.d : (shared ? a.FS : a.F);  // K of one segment
  const int nseg = (!GATEUP && shared) ? a.S : 1;
  // weight rows first: their loads do not wait for the activation row lookup
  BRow<TW> b0 = GATEUP ? BRow<TW>(shared ? a.shg : expert_mat<TW>(a.wg, e, a.F, a.d), n, K, g,
                                  shared ? a.shsg : expert_scales(a.sg, e, a.F, a.d), a.wtiled)
                       : BRow<TW>(shared ? a.shd : expert_mat<TW>(a.wd, e, a.d, K), n, K, g,
                                  shared ? a.shsd : expert_scales(a.sd, e, a.d, K), a.wtiled);
  BRow<TW> b1 = GATEUP ? BRow<TW>(shared ? a.shu : expert_mat<TW>(a.wu, e, a.F, a.d), n, K, g,
                                  shared ? a.shsu : expert_scales(a.su, e, a.F, a.d), a.wtiled)
                       : b0;

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

  f32x4 acc[NM][MT];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[m][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int seg = 0; seg < nseg; ++seg) {
    if (seg > 0) {  // next slab of the shared down projection: [S][d][FS]
      b0 = BRow<TW>(expert_mat<TW>(a.shd, seg, a.d, K), n, K, g, expert_scales(a.shsd, seg, a.d, K), a.wtiled);
      b1 = b0;
    }
    const int aoff = seg * K;
    const int nsteps = K / KSTEP;
    const int s0 = kpart * nsteps / KSPLIT, s1 = (kpart + 1) * nsteps / KSPLIT;
#pragma unroll 1  // U-deep unroll inside already; a further unroll only costs occupancy
    for (int st = s0; st < s1; st += U) {
      u32x4 bq[NM][U];
      float sc[NM][U];
      u32x4 av[MT][U][AL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (st + u < s1) {
          const int kb = (st + u) * KSTEP;
          bq[0][u] = b0.load(kb);
          sc[0][u] = b0.scale(kb);
          if (NM > 1) {
            bq[NM - 1][u] = b1.load(kb);
            sc[NM - 1][u] = b1.scale(kb);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (st + u < s1) {
          const int kb = (st + u) * KSTEP;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            if (mt < nmt)
#pragma unroll
              for (int q = 0; q < AL; ++q)
                av[mt][u][q] = ld16(arow[mt] + aoff + kb + (AL == 1 ? (KSTEP / 4) * g : 32 * g + 8 * q));
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (st + u < s1) {
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              if (mt < nmt) acc[m][mt] = dstep<TW>(av[mt][u], bq[m][u], sc[m][u], acc[m][mt]);
        }
      }
    }
  }

  if (KSPLIT > 1) {
    // add the K slices (fixed order) in wave 0
    if (w > 0) {
#pragma unroll
      for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          if (mt < nmt) red[w - 1][m][mt][lane] = acc[m][mt];
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (mt < nmt) acc[m][mt] = ((acc[m][mt] + red[0][m][mt][lane]) + red[1][m][mt][lane]) + red[2][m][mt][lane];
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt >= nmt) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mt + 4 * g + i;
      if (r >= mrows) continue;
      if (GATEUP) {
        const float hv = silu(acc[0][mt][i]) * acc[NM - 1][mt][i];
        TA* hout = (TA*)(shared ? a.hsh : a.h);
        hout[(size_t)(row0 + r) * (shared ? Ns : Nr) + n] = from_f32<TA>(hv);
      } else {
        TA* yout = (TA*)(shared ? a.ysh : a.y);
        yout[(size_t)(row0 + r) * a.d + n] = from_f32<TA>(acc[0][mt][i]);
      }
    }
  }
}

// ------------------------------------------------------------------ tiled (large-M) kernels
// Block: 128 rows of one item x 256 weight rows, four waves.  The gathered
// activation tile goes through double-buffered LDS (every wave needs all 128
// rows); each wave owns 64 weight rows (four 16-row MFMA fragments) that no
// other wave reads, so they travel from global memory straight into MFMA
// operand registers, prefetched one K step ahead.  Per K step a wave issues
// 8 x 4 MFMA 16x16x32 per 32-wide K slice against 8 LDS fragment reads, half
// the LDS traffic per MFMA of a 64 x 64 wave tile.
// Gate/up: wave w's fragments are gate rows n0+32w .. +32 and the up rows of
// the same channels, so the SwiGLU epilogue stays in registers.
// Lane K order inside a step: bf16 (64-wide steps) k = kb + 32 s + 8 g + i;
// INT4 (128-wide steps, one scale group) k = kb + 32 g + 8 s + i, so a lane's
// 16-byte weight load covers 32 nibbles of one group.
// K step per weight type and projection (measured: the gate/up kernel, with
// two weight matrices, runs best with 64-wide steps; the down kernel with
// 32-wide steps, whose smaller register footprint avoids spills).
template <typename TW, bool GATEUP> struct Til;
template <> struct Til<bf16, true> {
  static constexpr int KSTEP = 64, SUB = 2, BL = 2;   // BL: 16-byte weight loads per fragment per step
};
template <> struct Til<bf16, false> {
  static constexpr int KSTEP = 32, SUB = 1, BL = 1;
};
template <bool G> struct Til<INT4, G> {
  static constexpr int KSTEP = 128, SUB = 4, BL = 1;
};
constexpr int TBM = 128;

// The tile a block of a tiled kernel owns.  Tile list: routed items
// (expert-major, so one expert's tiles are adjacent) times N blocks of NT
// output channels, then the shared-expert tiles.  Blocks are dispatched
// round-robin over the 8 XCDs, so XCD x = blockIdx % 8 takes the x-th of 8
// contiguous, equal chunks of the list: the tiles of an expert then run
// together on one XCD and share their weight and activation K slabs in its L2.
struct TileInfo {
  int e, row0, mrows, n0;
  bool shared;
};
__device__ __forceinline__ bool tile_of(const FfnArgs& a, int NT, TileInfo& t) {
  const bool gu = NT == 128;  // gate/up blocks cover 128 channels, down blocks 256 columns
  const int Nr = gu ? a.F : a.d, Ns = gu ? a.S * a.FS : a.d;
  const int nbr = (Nr + NT - 1) / NT, nbs = (Ns + NT - 1) / NT;
  const int routed_tiles = *a.n_items * nbr;
  const int total = routed_tiles + (a.S > 0 ? a.sh_items * nbs : 0);
  const int xcd = blockIdx.x & 7;
  const int lo = (int)((int64_t)total * xcd / 8), hi = (int)((int64_t)total * (xcd + 1) / 8);
  const int tile = lo + (int)(blockIdx.x >> 3);
  if (tile >= hi) return false;
  int nb;
  t.shared = tile >= routed_tiles;
  if (!t.shared) {
    const int slot = tile / nbr;
    nb = tile - slot * nbr;
    const int4 it = a.items[slot];
    t.e = it.x;
    t.row0 = it.y;
    t.mrows = it.z;
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

template <typename TW, bool GATEUP, bool TILED>
__global__ __launch_bounds__(256, (std::is_same<TW, INT4>::value ? 1 : 2)) void ffn_tiled_kernel(FfnArgs a) {
  using TT = Til<TW, GATEUP>;
  constexpr int KSTEP = TT::KSTEP, SUB = TT::SUB, BL = TT::BL;
  constexpr bool I4 = std::is_same<TW, INT4>::value;
  constexpr int LDA = KSTEP + 16;         // padded LDS row (bf16 elements)
  constexpr int CPR = KSTEP / 8;          // 16-byte chunks per A row per step
  constexpr int CPT = TBM * CPR / 256;    // A chunks per thread per step
  constexpr int RPT = 256 / CPR;          // row stride between a thread's chunks
  constexpr int NT = GATEUP ? 128 : 256;  // output channels per block (F, S*FS multiples of 128)
  __shared__ bf16 As[2][TBM * LDA];
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6, g = lane >> 4, c = lane & 15;
  const int Nr = GATEUP ? a.F : a.d;
  const int Ns = GATEUP ? a.S * a.FS : a.d;
  TileInfo ti;
  if (!tile_of(a, NT, ti)) return;
  const int e = ti.e, row0 = ti.row0, mrows = ti.mrows, n0 = ti.n0;
  const bool shared = ti.shared;
  const int Kfull = GATEUP ? a.d : (shared ? a.S * a.FS : a.F);
  const int Kseg = GATEUP ? a.d : (shared ? a.FS : a.F);

  // activation chunk sources: rows (tid / CPR) + RPT q, 16-byte chunk tid % CPR
  // (64-bit addresses: x and h may exceed 4 GiB)
  const int ch = tid % CPR;
  const char* aptr[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int r = min(tid / CPR + RPT * q, mrows - 1);
    if (GATEUP) {
      int tok = shared ? row0 + r : a.row_token[row0 + r];
      tok = min(max(tok, 0), a.T - 1);
      aptr[q] = (const char*)a.x + ((size_t)tok * a.d + ch * 8) * 2;
    } else {
      aptr[q] = (const char*)(shared ? a.hsh : a.h) + ((size_t)(row0 + r) * Kfull + ch * 8) * 2;
    }
  }
  // weight fragment f of this wave: byte offset of its lane's bytes inside one
  // of two block-uniform matrices (gate / up, or down; the shared down
  // projection adds a block-uniform slab offset per K step), in the row or the
  // tiled weight layout (16-row x 64-byte fragments stored lane-major)
  const char* bmat[2];
  const uint16_t* smat[2];
  uint32_t boff[4], soff[4];
  if (GATEUP) {
    bmat[0] = (const char*)(shared ? a.shg : expert_mat<TW>(a.wg, e, a.F, a.d));
    bmat[1] = (const char*)(shared ? a.shu : expert_mat<TW>(a.wu, e, a.F, a.d));
    smat[0] = (const uint16_t*)(shared ? a.shsg : expert_scales(a.sg, e, a.F, a.d));
    smat[1] = (const uint16_t*)(shared ? a.shsu : expert_scales(a.su, e, a.F, a.d));
  } else {
    bmat[0] = bmat[1] = (const char*)(shared ? a.shd : expert_mat<TW>(a.wd, e, a.d, Kseg));
    smat[0] = smat[1] = (const uint16_t*)(shared ? a.shsd : expert_scales(a.sd, e, a.d, Kseg));
  }
  const int Kb = row_bytes<TW>(Kseg);
  constexpr uint32_t cstride = TILED ? 1024u : 64u;  // bytes between the 64-byte chunks of a row
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    // first row of the fragment's 16-row group (a last down block may be half
    // past d: its surplus fragments re-read the last group, results unused)
    const int row16 = GATEUP ? n0 + 32 * w + 16 * (f & 1) : min(n0 + 64 * w + 16 * f, a.d - 16);
    boff[f] = TILED ? (uint32_t)row16 * Kb + 256 * g + 16 * c : (uint32_t)(row16 + c) * Kb + 16 * g;
    soff[f] = I4 ? (uint32_t)(row16 + c) * (Kseg / kInt4Group) * 2u : 0u;
  }
  // byte offset of K step kt inside the weight matrix (slab plus row chunk), and scale index
  auto woff = [&](int kt, int* so) -> size_t {
    const int k0 = kt * KSTEP;
    const int slab = (!GATEUP && shared) ? k0 / Kseg : 0;
    const int kk = k0 - slab * Kseg;
    *so = I4 ? slab * a.d * (Kseg / kInt4Group) + kk / kInt4Group : 0;
    return (size_t)slab * a.d * Kb + (size_t)(row_bytes<TW>(kk) / 64) * cstride;
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[m][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 ar[CPT];
  u32x4 bcur[4][BL], bnext[4][BL];
  float scur[4], snext[4];
  const int nkt = Kfull / KSTEP;

  auto load_a = [&](int kt) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) ar[q] = ld16(aptr[q] + kt * KSTEP * 2);
  };
  auto store_a = [&](bf16* dst) {
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      *reinterpret_cast<u32x4*>(&dst[(tid / CPR + RPT * q) * LDA + ch * 8]) = ar[q];
  };
  auto load_b = [&](u32x4 (&bq)[4][BL], float (&bs)[4], int kt) {
    int so;
    const size_t o = woff(kt, &so);
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const char* m = bmat[GATEUP ? (f >> 1) : 0] + o;
      if constexpr (I4) {
        bq[f][0] = ld16_at(m, boff[f]);
        const char* sm = (const char*)(smat[GATEUP ? (f >> 1) : 0] + so);
        bs[f] = bf16_bits_to_f32(*(const uint16_t*)(sm + soff[f]));
      } else {
#pragma unroll
        for (int s = 0; s < BL; ++s) bq[f][s] = ld16_at(m + cstride * s, boff[f]);
        bs[f] = 1.f;
      }
    }
  };

  // one K step: SUB slices of 32; the activation fragment of the next m is
  // read from LDS before the four MFMAs of the current one are issued
  auto compute = [&](const bf16* A, const u32x4 (&bq)[4][BL], const float (&bs)[4]) {
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      u32x4 bf[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        if constexpr (I4) bf[f] = int4x8_to_bf16_scaled(bq[f][0][s], bs[f]);
        else bf[f] = bq[f][s];
      }
      const int col = I4 ? (32 * g + 8 * s) : (32 * s + 8 * g);
      u32x4 af = *reinterpret_cast<const u32x4*>(&A[c * LDA + col]);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        u32x4 an = af;
        if (m + 1 < 8) an = *reinterpret_cast<const u32x4*>(&A[(16 * (m + 1) + c) * LDA + col]);
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[m][f] = mma_bf16(af, bf[f], acc[m][f]);
        af = an;
      }
    }
  };

  // two-step ping-pong without branches: step kt computes from (As[kt & 1],
  // register set kt & 1) while step kt + 1 loads into the other pair; past the
  // last step the prefetch repeats step nkt - 1 (harmless, never used)
  u32x4 b1q[4][BL];
  float s1q[4];
  load_a(0);
  load_b(bcur, scur, 0);
  store_a(As[0]);
  __syncthreads();
  int kt = 0;
  // the scheduling barriers keep the next step's loads ahead of this step's
  // MFMAs (left alone, the scheduler sinks them next to their first use)
  for (; kt + 2 <= nkt; kt += 2) {
    load_a(min(kt + 1, nkt - 1));
    load_b(b1q, s1q, min(kt + 1, nkt - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(As[0], bcur, scur);
    __builtin_amdgcn_sched_barrier(0);
    store_a(As[1]);
    __syncthreads();
    load_a(min(kt + 2, nkt - 1));
    load_b(bcur, scur, min(kt + 2, nkt - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(As[1], b1q, s1q);
    __builtin_amdgcn_sched_barrier(0);
    store_a(As[0]);
    __syncthreads();
  }
  if (kt < nkt) compute(As[0], bcur, scur);
  (void)bnext;
  (void)snext;

#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * g + i;
      if (r >= mrows) continue;
      if (GATEUP) {
        bf16* hout = (bf16*)(shared ? a.hsh : a.h);
        const int ld = shared ? Ns : Nr;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const float hv = silu(acc[m][f][i]) * acc[m][f + 2][i];
          hout[(size_t)(row0 + r) * ld + n0 + 32 * w + 16 * f + c] = (bf16)hv;
        }
      } else {
        bf16* yout = (bf16*)(shared ? a.ysh : a.y);
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + 64 * w + 16 * f + c;
          if (col < a.d) yout[(size_t)(row0 + r) * a.d + col] = (bf16)acc[m][f][i];
        }
      }
    }
  }
}

// ------------------------------------------------------------------ tiled bf16 kernels, 32x32x16 MFMA
// The bf16 expert GEMMs on v_mfma_f32_32x32x16_bf16, which on gfx950 retires
// twice the flops per cycle of the 16x16x32 form (measured: ~2.4 vs ~1.3
// PFLOP/s over the chip).  Same block tile and pipeline as the kernel above
// (128 rows x 256 weight rows, four waves, activations through double-buffered
// LDS, weights straight from memory into operand registers one K step ahead);
// wave w owns 128 rows x 64 weight rows as 4 x 2 tiles of 32 x 32.
// Operand lane l holds row (weight row) l % 32 and K values 8 (l / 32) .. +7
// of a 16-wide K slice; slice s of a 64-byte weight-row chunk is its bytes
// 32 (s % 2) .. +31, so a lane's 16-byte weight load for slice s reads chunk
// bytes 16 (2 (s % 2) + l / 32).  Output: lane l holds column l % 32 of a
// 32 x 32 tile, rows 8 (i / 4) + 4 (l / 32) + i % 4, i = 0..15.
// Gate/up: wave w's two tiles are gate rows n0 + 32w .. +31 and the up rows of
// the same channels, so the SwiGLU epilogue stays in registers.
template <bool GATEUP> struct Til32 {
  static constexpr int KSTEP = GATEUP ? 64 : 32;
};

__device__ __forceinline__ f32x16 mma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

template <bool GATEUP, bool TILED>
__global__ __launch_bounds__(256, 2) void ffn_tiled32_kernel(FfnArgs a) {
  constexpr int KSTEP = Til32<GATEUP>::KSTEP, SUB = KSTEP / 16;
  constexpr int LDA = KSTEP + 8;          // padded LDS row (bf16 elements)
  constexpr int CPR = KSTEP / 8;          // 16-byte chunks per A row per step
  constexpr int CPT = TBM * CPR / 256;    // A chunks per thread per step
  constexpr int RPT = 256 / CPR;          // row stride between a thread's chunks
  constexpr int NT = GATEUP ? 128 : 256;  // output channels per block
  constexpr uint32_t cstride = TILED ? 1024u : 64u;  // bytes between the 64-byte chunks of a weight row
  constexpr uint32_t hstride = TILED ? 512u : 32u;   // bytes between the two halves of a chunk
  constexpr int NC = GATEUP ? 128 : 256;  // output columns of a block
  constexpr int LDH = NC + 8;             // padded row of the output staging tile
  constexpr int SMEM = 2 * TBM * LDA > TBM * LDH ? 2 * TBM * LDA : TBM * LDH;
  __shared__ bf16 smem[SMEM];
  bf16* const As[2] = {smem, smem + TBM * LDA};
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6, h = lane >> 5, c = lane & 31;
  TileInfo ti;
  if (!tile_of(a, NT, ti)) return;
  const int e = ti.e, row0 = ti.row0, mrows = ti.mrows, n0 = ti.n0;
  const bool shared = ti.shared;
  const int Kfull = GATEUP ? a.d : (shared ? a.S * a.FS : a.F);
  const int Kseg = GATEUP ? a.d : (shared ? a.FS : a.F);
  const int Kb = Kseg * 2;

  // weight tile nt of this wave: 32 rows from rb; byte offset of this lane's bytes
  const char* bmat[2];
  if (GATEUP) {
    bmat[0] = (const char*)(shared ? a.shg : expert_mat<bf16>(a.wg, e, a.F, a.d));
    bmat[1] = (const char*)(shared ? a.shu : expert_mat<bf16>(a.wu, e, a.F, a.d));
  } else {
    bmat[0] = bmat[1] = (const char*)(shared ? a.shd : expert_mat<bf16>(a.wd, e, a.d, Kseg));
  }
  uint32_t boff[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    // a last down block may be half past d: its surplus tiles re-read the last 32 rows, results unused
    const int rb = GATEUP ? n0 + 32 * w : min(n0 + 64 * w + 32 * nt, a.d - 32);
    const int row = rb + c;
    boff[nt] = TILED ? (uint32_t)(row & ~15) * Kb + 256 * h + 16 * (row & 15) : (uint32_t)row * Kb + 16 * h;
  }
  // activation chunk sources: rows (tid / CPR) + RPT q, 16-byte chunk tid % CPR
  const int ch = tid % CPR;
  const char* aptr[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int r = min(tid / CPR + RPT * q, mrows - 1);
    if (GATEUP) {
      int tok = shared ? row0 + r : a.row_token[row0 + r];
      tok = min(max(tok, 0), a.T - 1);
      aptr[q] = (const char*)a.x + ((size_t)tok * a.d + ch * 8) * 2;
    } else {
      aptr[q] = (const char*)(shared ? a.hsh : a.h) + ((size_t)(row0 + r) * Kfull + ch * 8) * 2;
    }
  }
  // byte offset of K step kt inside the weight matrix: shared down slab plus row chunk
  auto woff = [&](int kt) -> size_t {
    const int k0 = kt * KSTEP;
    const int slab = (!GATEUP && shared) ? k0 / Kseg : 0;
    const int kk = k0 - slab * Kseg;
    return (size_t)slab * a.d * Kb + (size_t)(kk / 32) * cstride;
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16{};

  u32x4 ar[CPT];
  u32x4 b0q[2][SUB], b1q[2][SUB];
  const int nkt = Kfull / KSTEP;

  auto load_a = [&](int kt) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) ar[q] = ld16(aptr[q] + kt * KSTEP * 2);
  };
  auto store_a = [&](bf16* dst) {
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      *reinterpret_cast<u32x4*>(&dst[(tid / CPR + RPT * q) * LDA + ch * 8]) = ar[q];
  };
  auto load_b = [&](u32x4 (&bq)[2][SUB], int kt) {
    const size_t o = woff(kt);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s = 0; s < SUB; ++s)
        bq[nt][s] = ld16_at(bmat[nt] + o + (s >> 1) * cstride + (s & 1) * hstride, boff[nt]);
  };
  // one K step: SUB slices of 16.  The four activation fragments of slice s + 1
  // are read from LDS while the eight MFMAs of slice s issue: the group
  // barriers at the end pin that order (left alone, the scheduler places each
  // read right before its first use and the LDS latency shows every time).
  auto compute = [&](const bf16* A, const u32x4 (&bq)[2][SUB]) {
    u32x4 af[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) af[mt] = *reinterpret_cast<const u32x4*>(&A[(32 * mt + c) * LDA + 8 * h]);
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      u32x4 an[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        an[mt] = s + 1 < SUB ? *reinterpret_cast<const u32x4*>(&A[(32 * mt + c) * LDA + 16 * (s + 1) + 8 * h])
                             : af[mt];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mma32_bf16(af[mt], bq[nt][s], acc[mt][nt]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) af[mt] = an[mt];
    }
    // order: 4 reads (slice 0); per slice but the last: (1 MFMA, 1 read) x 4, 4 MFMAs; last slice: 8 MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int s = 0; s + 1 < SUB; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  };

  // two-step ping-pong without branches (as in the kernel above)
  load_b(b0q, 0);  // weights first: they do not wait for the row -> token lookup
  load_a(0);
  store_a(As[0]);
  __syncthreads();
  int kt = 0;
  for (; kt + 2 <= nkt; kt += 2) {
    load_a(min(kt + 1, nkt - 1));
    load_b(b1q, min(kt + 1, nkt - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(As[0], b0q);
    __builtin_amdgcn_sched_barrier(0);
    store_a(As[1]);
    __syncthreads();
    load_a(min(kt + 2, nkt - 1));
    load_b(b0q, min(kt + 2, nkt - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(As[1], b1q);
    __builtin_amdgcn_sched_barrier(0);
    store_a(As[0]);
    __syncthreads();
  }
  if (kt < nkt) compute(As[0], b0q);

  // epilogue through LDS: each wave writes its 32 x 32 tiles (SwiGLU applied)
  // into a 128 x NC staging tile, then the block stores 16-byte row chunks
  __syncthreads();  // every wave is done reading the activation tiles
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
      if (GATEUP) {
        smem[r * LDH + 32 * w + c] = (bf16)(silu(acc[mt][0][i]) * acc[mt][1][i]);
      } else {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) smem[r * LDH + 64 * w + 32 * nt + c] = (bf16)acc[mt][nt][i];
      }
    }
  }
  __syncthreads();
  bf16* const out = (bf16*)(GATEUP ? (shared ? a.hsh : a.h) : (shared ? a.ysh : a.y));
  const int ld = GATEUP ? (shared ? a.S * a.FS : a.F) : a.d;
  const int ncols = GATEUP ? ld : a.d;  // a last down block may be half past d
  constexpr int CK = NC / 8;              // 16-byte chunks per staged row
#pragma unroll
  for (int q = 0; q < TBM * CK / 256; ++q) {
    const int idx = tid + 256 * q, r = idx / CK, ck = idx % CK, col = n0 + 8 * ck;
    if (r < mrows && col < ncols)
      st16(out + (size_t)(row0 + r) * ld + col, *reinterpret_cast<const u32x4*>(&smem[r * LDH + 8 * ck]));
  }
}

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
// tiled kernels: one block per tile slot, rounded up to whole rounds of the 8 XCDs
static int ffn_grid_xcd(const FfnArgs& a, int nt_routed, int nt_shared) {
  return (ffn_grid(a, nt_routed, nt_shared) + 7) / 8 * 8;
}

template <bool GATEUP, int MT>
static void launch_stream(int wdt, const FfnArgs& a, int grid, hipStream_t s) {
  if (wdt == kF32)
    hipLaunchKernelGGL((ffn_stream_kernel<float, GATEUP, MT>), dim3(grid), dim3(256), 0, s, a);
  else if (wdt == kBF16)
    hipLaunchKernelGGL((ffn_stream_kernel<bf16, GATEUP, MT>), dim3(grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((ffn_stream_kernel<INT4, GATEUP, MT>), dim3(grid), dim3(256), 0, s, a);
}

template <bool GATEUP>
static void launch_stream_mt(int wdt, const FfnArgs& a, int grid, hipStream_t s) {
  if (a.bm <= 16)
    launch_stream<GATEUP, 1>(wdt, a, grid, s);
  else if (a.bm <= 32)
    launch_stream<GATEUP, 2>(wdt, a, grid, s);
  else
    launch_stream<GATEUP, 4>(wdt, a, grid, s);
}

template <bool GATEUP> void launch_tiled(int wdt, const FfnArgs& a, int grid, hipStream_t s) {
  if (wdt == kBF16) {
    if (a.wtiled) hipLaunchKernelGGL((ffn_tiled32_kernel<GATEUP, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((ffn_tiled32_kernel<GATEUP, false>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (a.wtiled) hipLaunchKernelGGL((ffn_tiled_kernel<INT4, GATEUP, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((ffn_tiled_kernel<INT4, GATEUP, false>), dim3(grid), dim3(256), 0, s, a);
  }
}

hipError_t launch_ffn_gateup(int mode, int act, int wdt, const FfnArgs& a, hipStream_t s) {
  if (mode == 0) {
    const int grid = ffn_grid(a, a.F / 16, a.S * a.FS / 16);
    if (grid == 0) return hipSuccess;
    launch_stream_mt<true>(wdt, a, grid, s);
  } else {
    const int grid = ffn_grid_xcd(a, a.F / 128, a.S * a.FS / 128);
    if (grid == 0) return hipSuccess;
    launch_tiled<true>(wdt, a, grid, s);
  }
  (void)act;
  return hipGetLastError();
}

hipError_t launch_ffn_down(int mode, int act, int wdt, const FfnArgs& a, hipStream_t s) {
  if (mode == 0) {
    const int grid = ffn_grid(a, a.d / 64, a.d / 64);
    if (grid == 0) return hipSuccess;
    launch_stream_mt<false>(wdt, a, grid, s);
  } else {
    const int grid = ffn_grid_xcd(a, (a.d + 255) / 256, (a.d + 255) / 256);
    if (grid == 0) return hipSuccess;
    launch_tiled<false>(wdt, a, grid, s);
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
