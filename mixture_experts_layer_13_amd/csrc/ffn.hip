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

// One weight row of a [N][K] matrix as seen by one lane (lane group g = lane/16).
// Lane K order inside a step: bf16 k = kb + 8g + i; f32 k = kb + 4g + i;
// INT4 k = kb + 32g + 8s + i (s = dword of the 16-byte load).
template <typename TW> struct BRow;
template <> struct BRow<float> {
  const float* p;
  __device__ BRow(const void* m, int n, int K, int g, const void*) : p((const float*)m + (size_t)n * K + 4 * g) {}
  __device__ u32x4 load(int kb) const { return ld16(p + kb); }
  __device__ float scale(int) const { return 1.f; }
};
template <> struct BRow<bf16> {
  const bf16* p;
  __device__ BRow(const void* m, int n, int K, int g, const void*) : p((const bf16*)m + (size_t)n * K + 8 * g) {}
  __device__ u32x4 load(int kb) const { return ld16(p + kb); }
  __device__ float scale(int) const { return 1.f; }
};
template <> struct BRow<INT4> {
  const uint8_t* p;
  const uint16_t* s;
  __device__ BRow(const void* m, int n, int K, int g, const void* sc)
      : p((const uint8_t*)m + (size_t)n * (K / 2) + 16 * g), s((const uint16_t*)sc + (size_t)n * (K / kInt4Group)) {}
  __device__ u32x4 load(int kb) const { return ld16(p + kb / 2); }
  __device__ float scale(int kb) const { return bf16_bits_to_f32(s[kb / kInt4Group]); }
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
// grid: items_max * (N / 16) routed blocks, then sh_items * (Ns / 16) shared blocks.
template <typename TW, bool GATEUP>
__global__ __launch_bounds__(256) void ffn_stream_kernel(FfnArgs a) {
  using D = Dec<TW>;
  using TA = typename D::TA;
  constexpr int NM = GATEUP ? 2 : 1;
  constexpr int MT = kDecodeRows / 16;
  constexpr int U = D::U, AL = D::AL, KSTEP = D::KSTEP;
  __shared__ f32x4 red[3][NM][MT][64];
  const int lane = lane_id(), w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;

  const int Nr = GATEUP ? a.F : a.d;
  const int Ns = GATEUP ? a.S * a.FS : a.d;
  const int nbr = Nr / 16, nbs = Ns / 16;
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
  const int n = nb * 16 + c;

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

  const int K = GATEUP ? a.d : (shared ? a.FS : a.F);  // K of one segment
  const int nseg = (!GATEUP && shared) ? a.S : 1;
  for (int seg = 0; seg < nseg; ++seg) {
    BRow<TW> b0 = GATEUP ? BRow<TW>(shared ? a.shg : expert_mat<TW>(a.wg, e, a.F, a.d), n, K, g,
                                    shared ? a.shsg : expert_scales(a.sg, e, a.F, a.d))
                         : BRow<TW>(shared ? expert_mat<TW>(a.shd, seg, a.d, K) : expert_mat<TW>(a.wd, e, a.d, K), n,
                                    K, g, shared ? expert_scales(a.shsd, seg, a.d, K) : expert_scales(a.sd, e, a.d, K));
    BRow<TW> b1 = GATEUP ? BRow<TW>(shared ? a.shu : expert_mat<TW>(a.wu, e, a.F, a.d), n, K, g,
                                    shared ? a.shsu : expert_scales(a.su, e, a.F, a.d))
                         : b0;
    const int aoff = seg * K;
    const int nsteps = K / KSTEP;
    const int s0 = w * nsteps / 4, s1 = (w + 1) * nsteps / 4;
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

  // reduce the four K slices (fixed order) and write
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
// Block tile 128 rows x 128 weight rows x 64 K, 4 waves as 2 x 2, each wave
// 64 rows x 64 weight rows as 4 x 4 MFMA 16x16x32 tiles.  Gate/up: weight rows
// 0..63 are gate rows n0..n0+63, rows 64..127 the up rows of the same
// channels, and each wave holds the gate and up tiles of the same 32 channels
// so the SwiGLU epilogue stays in registers.
constexpr int PBM = 128, PBN = 128, PBK = 64, PLD = PBK + 8;

template <typename TW> struct PLoad;
template <> struct PLoad<bf16> {
  u32x4 v[4];
};
template <> struct PLoad<INT4> {
  u32x4 v;
  float s;
};

template <typename TW, bool GATEUP>
__global__ __launch_bounds__(256) void ffn_tiled_kernel(FfnArgs a) {
  __shared__ bf16 As[2][PBM * PLD];
  __shared__ bf16 Bs[2][PBN * PLD];
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6, g = lane >> 4, c = lane & 15;
  const int wm = w >> 1, wn = w & 1;
  constexpr int NT = GATEUP ? 64 : 128;  // output channels per block
  const int Nr = GATEUP ? a.F : a.d;
  const int Ns = GATEUP ? a.S * a.FS : a.d;
  const int nbr = Nr / NT, nbs = Ns / NT;
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
  const int n0 = nb * NT;
  const int Kfull = GATEUP ? a.d : (shared ? a.S * a.FS : a.F);
  const int Kseg = GATEUP ? a.d : (shared ? a.FS : a.F);

  // A sources: rows (tid >> 3) + 32 i, 16-byte chunk (tid & 7)
  const int ch = tid & 7;
  const bf16* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min((tid >> 3) + 32 * i, mrows - 1);
    if (GATEUP) {
      int tok = shared ? row0 + r : a.row_token[row0 + r];
      tok = min(max(tok, 0), a.T - 1);
      asrc[i] = (const bf16*)a.x + (size_t)tok * a.d + ch * 8;
    } else {
      asrc[i] = (const bf16*)(shared ? a.hsh : a.h) + (size_t)(row0 + r) * Kfull + ch * 8;
    }
  }
  // B source row for weight-tile row rb, K offset k0 (returns element / byte pointer)
  auto brow_ptr = [&](int rb, int k0, const void** sptr) -> const void* {
    const void* mat;
    const void* sc;
    int n;
    int kk = k0;
    if (GATEUP) {
      const bool up = rb >= 64;
      n = n0 + (rb & 63);
      mat = shared ? (up ? a.shu : a.shg) : expert_mat<TW>(up ? a.wu : a.wg, e, a.F, a.d);
      sc = shared ? (up ? a.shsu : a.shsg) : expert_scales(up ? a.su : a.sg, e, a.F, a.d);
    } else {
      n = n0 + rb;
      const int slab = shared ? k0 / Kseg : 0;
      kk = k0 - slab * Kseg;
      mat = shared ? expert_mat<TW>(a.shd, slab, a.d, Kseg) : expert_mat<TW>(a.wd, e, a.d, Kseg);
      sc = shared ? expert_scales(a.shsd, slab, a.d, Kseg) : expert_scales(a.sd, e, a.d, Kseg);
    }
    if constexpr (std::is_same<TW, INT4>::value) {
      *sptr = (const uint16_t*)sc + (size_t)n * (Kseg / kInt4Group) + kk / kInt4Group;
      return (const uint8_t*)mat + (size_t)n * (Kseg / 2) + kk / 2;
    } else {
      *sptr = nullptr;
      return (const bf16*)mat + (size_t)n * Kseg + kk;
    }
  };

  PLoad<TW> pl;
  u32x4 ar[4];
  auto gload = [&](int kt) {
    const int k0 = kt * PBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = ld16(asrc[i] + k0);
    if constexpr (std::is_same<TW, INT4>::value) {
      const void* sp;
      const uint8_t* p = (const uint8_t*)brow_ptr(tid >> 1, k0, &sp);
      pl.v = ld16(p + 16 * (tid & 1));
      pl.s = bf16_bits_to_f32(*(const uint16_t*)sp);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const void* sp;
        const bf16* p = (const bf16*)brow_ptr((tid >> 3) + 32 * i, k0, &sp);
        pl.v[i] = ld16(p + ch * 8);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4*>(&As[buf][((tid >> 3) + 32 * i) * PLD + ch * 8]) = ar[i];
    if constexpr (std::is_same<TW, INT4>::value) {
      const int rb = tid >> 1, half = tid & 1;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 d8 = int4x8_to_bf16(pl.v[q]);
        // apply the group scale and round once to bf16
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const float lo = bf16_bits_to_f32(d8[p] & 0xFFFFu) * pl.s;
          const float hi = bf16_bits_to_f32(d8[p] >> 16) * pl.s;
          o[p] = pack_bf16x2(lo, hi);
        }
        *reinterpret_cast<u32x4*>(&Bs[buf][rb * PLD + 32 * half + 8 * q]) = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4*>(&Bs[buf][((tid >> 3) + 32 * i) * PLD + ch * 8]) = pl.v[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  int brow[4];
#pragma unroll
  for (int nf = 0; nf < 4; ++nf)
    brow[nf] = GATEUP ? (nf < 2 ? 32 * wn + 16 * nf : 64 + 32 * wn + 16 * (nf - 2)) : 64 * wn + 16 * nf;

  const int nkt = Kfull / PBK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      u32x4 af[4], bfr[4];
#pragma unroll
      for (int mf = 0; mf < 4; ++mf)
        af[mf] = *reinterpret_cast<const u32x4*>(&As[buf][(64 * wm + 16 * mf + c) * PLD + sub * 32 + 8 * g]);
#pragma unroll
      for (int nf = 0; nf < 4; ++nf)
        bfr[nf] = *reinterpret_cast<const u32x4*>(&Bs[buf][(brow[nf] + c) * PLD + sub * 32 + 8 * g]);
#pragma unroll
      for (int mf = 0; mf < 4; ++mf)
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) acc[mf][nf] = mma_bf16(af[mf], bfr[nf], acc[mf][nf]);
    }
    if (kt + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int mf = 0; mf < 4; ++mf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 64 * wm + 16 * mf + 4 * g + i;
      if (r >= mrows) continue;
      if (GATEUP) {
        bf16* hout = (bf16*)(shared ? a.hsh : a.h);
        const int ld = shared ? Ns : Nr;
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          const float hv = silu(acc[mf][nf][i]) * acc[mf][nf + 2][i];
          hout[(size_t)(row0 + r) * ld + n0 + 32 * wn + 16 * nf + c] = (bf16)hv;
        }
      } else {
        bf16* yout = (bf16*)(shared ? a.ysh : a.y);
#pragma unroll
        for (int nf = 0; nf < 4; ++nf) yout[(size_t)(row0 + r) * a.d + n0 + 64 * wn + 16 * nf + c] = (bf16)acc[mf][nf][i];
      }
    }
  }
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

hipError_t launch_ffn_gateup(int mode, int act, int wdt, const FfnArgs& a, hipStream_t s) {
  if (mode == 0) {
    const int grid = ffn_grid(a, a.F / 16, a.S * a.FS / 16);
    if (grid == 0) return hipSuccess;
    if (wdt == kF32)
      hipLaunchKernelGGL((ffn_stream_kernel<float, true>), dim3(grid), dim3(256), 0, s, a);
    else if (wdt == kBF16)
      hipLaunchKernelGGL((ffn_stream_kernel<bf16, true>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((ffn_stream_kernel<INT4, true>), dim3(grid), dim3(256), 0, s, a);
  } else {
    const int grid = ffn_grid(a, a.F / 64, a.S * a.FS / 64);
    if (grid == 0) return hipSuccess;
    if (wdt == kBF16)
      hipLaunchKernelGGL((ffn_tiled_kernel<bf16, true>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((ffn_tiled_kernel<INT4, true>), dim3(grid), dim3(256), 0, s, a);
  }
  (void)act;
  return hipGetLastError();
}

hipError_t launch_ffn_down(int mode, int act, int wdt, const FfnArgs& a, hipStream_t s) {
  if (mode == 0) {
    const int grid = ffn_grid(a, a.d / 16, a.d / 16);
    if (grid == 0) return hipSuccess;
    if (wdt == kF32)
      hipLaunchKernelGGL((ffn_stream_kernel<float, false>), dim3(grid), dim3(256), 0, s, a);
    else if (wdt == kBF16)
      hipLaunchKernelGGL((ffn_stream_kernel<bf16, false>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((ffn_stream_kernel<INT4, false>), dim3(grid), dim3(256), 0, s, a);
  } else {
    const int grid = ffn_grid(a, a.d / 128, a.d / 128);
    if (grid == 0) return hipSuccess;
    if (wdt == kBF16)
      hipLaunchKernelGGL((ffn_tiled_kernel<bf16, false>), dim3(grid), dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((ffn_tiled_kernel<INT4, false>), dim3(grid), dim3(256), 0, s, a);
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
