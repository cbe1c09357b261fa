// Tiled (large-M, prefill) expert FFN kernels with INT4 weights for gfx950:
// nibbles dequantised in registers to bf16 MFMA operands (16x16x32).
#include "ffn_common.hpp"

namespace moe {

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
template <bool G> struct Til<INT4, G> {
  static constexpr int KSTEP = 128, SUB = 4, BL = 1;   // BL: 16-byte weight loads per fragment per step
};
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

// ------------------------------------------------------------------ launch
void launch_tiled_int4(bool gateup, const FfnArgs& a, int grid, hipStream_t s) {
  if (gateup) {
    if (a.wtiled) hipLaunchKernelGGL((ffn_tiled_kernel<INT4, true, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((ffn_tiled_kernel<INT4, true, false>), dim3(grid), dim3(256), 0, s, a);
  } else {
    if (a.wtiled) hipLaunchKernelGGL((ffn_tiled_kernel<INT4, false, true>), dim3(grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((ffn_tiled_kernel<INT4, false, false>), dim3(grid), dim3(256), 0, s, a);
  }
}

}  // namespace moe
