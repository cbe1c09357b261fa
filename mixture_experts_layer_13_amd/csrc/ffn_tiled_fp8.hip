// Tiled (large-M, prefill) expert FFN kernels with FP8 (OCP E4M3) weights for
// gfx950, on the 32x32x16 bf16 MFMA: each weight byte is widened to fp32, times
// its output channel's scale, rounded once to bf16, right before the MFMAs
// that use it ("MoE at the inference level", workarounds: fp8 expert weights
// halve the weight bytes; the activations stay bf16).
//
// Why not the FP8 MFMA: it needs both operands in FP8, i.e. the activations
// quantised as well, which is a different layer from the one with bf16
// activations and fp8 weights (that layer is ffn_tiled_f8f8.hip).  Why not
// the chip's scaled FP8 conversion: it applies only the exponent of its fp32
// scale (measured: bf16(fp8 * s) for power-of-two s only), and the channel
// scales here are arbitrary.
#include "ffn_common.hpp"

namespace moe {

// Eight E4M3 bytes (two dwords, K order byte 0..7) times the channel scale,
// each rounded once from fp32 to bf16.  The fp32 product is exact when it has
// at most 24 significant bits (3 + 1 from the code, 24 from the scale: it may
// round once there too, far below the bf16 rounding that follows).
__device__ __forceinline__ u32x4 fp8x8_to_bf16_scaled(uint32_t w0, uint32_t w1, float s) {
  const auto f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false), f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
  const auto f2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false), f3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
  u32x4 r;
  r[0] = pack_bf16x2(f0[0] * s, f0[1] * s);
  r[1] = pack_bf16x2(f1[0] * s, f1[1] * s);
  r[2] = pack_bf16x2(f2[0] * s, f2[1] * s);
  r[3] = pack_bf16x2(f3[0] * s, f3[1] * s);
  return r;
}

// Block: 128 rows of one item x 256 weight rows, four waves, each owning 128
// rows x 64 weight rows as 4 x 2 tiles of 32 x 32 (the bf16 tiled kernel's
// structure).  A K step is 64 wide, i.e. one 64-byte chunk of each weight row:
// the activation tile (128 rows x 64 bf16) goes through double-buffered LDS;
// each wave's weight rows arrive as two 16-byte loads per lane plus one scale
// per row, one step ahead.  Lane l (row l % 32 of a tile, h = l / 32) reads
// 16-byte units 2p + h (p = 0, 1) of the row's chunk; slice s (16 K) of the
// step takes bytes 8 (s % 2) .. +7 of load s / 2, i.e. K = 32 (s / 2) + 16 h +
// 8 (s % 2) + i, and the activation fragments are read from LDS in the same
// order.  Each converted 8-value operand feeds four MFMAs (the four 32-row tiles).
// STREAMW: weights loaded non-temporally (each expert's weights read by one row tile).
template <bool GATEUP, bool TILED, bool STREAMW>
__global__ __launch_bounds__(256, 2) void ffn_tiled_fp8_kernel(FfnArgs a) {
  constexpr int KSTEP = 64, SUB = KSTEP / 16;
  constexpr int LDA = KSTEP + 8;          // padded LDS row (bf16 elements), conflict-free operand reads
  constexpr int CPR = KSTEP / 8;          // 16-byte chunks per A row per step
  constexpr int CPT = TBM * CPR / 256;    // A chunks per thread per step
  constexpr int RPT = 256 / CPR;          // row stride between a thread's chunks
  constexpr int NT = GATEUP ? 128 : 256;  // output channels per block
  constexpr uint32_t cstride = TILED ? 1024u : 64u;  // bytes between the 64-byte chunks of a weight row
  constexpr uint32_t pstride = TILED ? 512u : 32u;   // bytes from unit h to unit 2 + h
  constexpr int NC = GATEUP ? 128 : 256;
  constexpr int LDH = NC + 8;
  constexpr int SMEM = 2 * TBM * LDA > TBM * LDH ? 2 * TBM * LDA : TBM * LDH;
  static_assert(CPT == 4 && RPT == 32, "a thread's activation chunk q must lie in row tile q");
  __shared__ bf16 smem[SMEM];
  bf16* const As[2] = {smem, smem + TBM * LDA};
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6, h = lane >> 5, c = lane & 31;
  TileInfo ti;
  if (!tile_of(a, NT, ti)) return;
  const int e = ti.e, row0 = ti.row0, mrows = ti.mrows, n0 = ti.n0;
  const bool shared = ti.shared;
  const int Kfull = GATEUP ? a.d : (shared ? a.S * a.FS : a.F);
  const int Kseg = GATEUP ? a.d : (shared ? a.FS : a.F);
  const int Kb = Kseg;  // bytes per weight row

  // weight tile nt of this wave: 32 rows from rb; byte offset of this lane's unit h, and its scale
  const char* bmat[2];
  const float* smat[2];
  if (GATEUP) {
    bmat[0] = (const char*)(shared ? a.shg : expert_mat<FP8>(a.wg, e, a.F, a.d));
    bmat[1] = (const char*)(shared ? a.shu : expert_mat<FP8>(a.wu, e, a.F, a.d));
    smat[0] = (const float*)(shared ? a.shsg : expert_scales_of<FP8>(a.sg, e, a.F, a.d));
    smat[1] = (const float*)(shared ? a.shsu : expert_scales_of<FP8>(a.su, e, a.F, a.d));
  } else {
    bmat[0] = bmat[1] = (const char*)(shared ? a.shd : expert_mat<FP8>(a.wd, e, a.d, Kseg));
    smat[0] = smat[1] = (const float*)(shared ? a.shsd : expert_scales_of<FP8>(a.sd, e, a.d, Kseg));
  }
  uint32_t boff[2];
  int srow[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    // a last down block may be half past d: its surplus tiles re-read the last 32 rows, results unused
    const int rb = GATEUP ? n0 + 32 * w : min(n0 + 64 * w + 32 * nt, a.d - 32);
    const int row = rb + c;
    boff[nt] = TILED ? (uint32_t)(row & ~15) * Kb + 256 * h + 16 * (row & 15) : (uint32_t)row * Kb + 16 * h;
    srow[nt] = row;
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
  // byte offset of K step kt inside the weight matrix (shared down: slab plus chunk) and the
  // scale index of the slab (the shared down's slabs are separate experts, each with its scales)
  auto woff = [&](int kt, int* so) -> size_t {
    const int k0 = kt * KSTEP;
    const int slab = (!GATEUP && shared) ? k0 / Kseg : 0;
    const int kc = (k0 - slab * Kseg) / KSTEP;
    *so = slab * a.d;
    return (size_t)slab * a.d * Kb + (size_t)kc * cstride;
  };

  u32x4 b0q[2][2], b1q[2][2];
  float s0q[2], s1q[2];
  const int nkt = Kfull / KSTEP;
  auto load_b = [&](u32x4 (&bq)[2][2], float (&bs)[2], int kt) {
    int so;
    const size_t o = woff(kt, &so);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const char* src = bmat[nt] + o + p * pstride;
        if constexpr (STREAMW) bq[nt][p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + boff[nt]));
        else bq[nt][p] = ld16_at(src, boff[nt]);
      }
      bs[nt] = smat[nt][so + srow[nt]];
    }
  };

  // Main loop and epilogue for MTA active 32-row tiles (1..4), as in the bf16
  // tiled kernel: the idle row tiles of a partly filled item cost nothing.
  auto body = [&](auto mta_tag) {
    constexpr int MTA = decltype(mta_tag)::value;
    f32x16 acc[MTA][2];
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16{};
    u32x4 ar[MTA];
    auto load_a = [&](int kt) {
#pragma unroll
      for (int q = 0; q < MTA; ++q) ar[q] = ld16(aptr[q] + kt * KSTEP * 2);
    };
    auto store_a = [&](bf16* dst) {
#pragma unroll
      for (int q = 0; q < MTA; ++q)
        *reinterpret_cast<u32x4*>(&dst[(tid / CPR + RPT * q) * LDA + ch * 8]) = ar[q];
    };
    auto compute = [&](const bf16* A, const u32x4 (&bq)[2][2], const float (&bs)[2]) {
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        const int col = 32 * (s >> 1) + 16 * h + 8 * (s & 1);
        u32x4 af[MTA], bf[2];
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt) af[mt] = *reinterpret_cast<const u32x4*>(&A[(32 * mt + c) * LDA + col]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          bf[nt] = fp8x8_to_bf16_scaled(bq[nt][s >> 1][2 * (s & 1)], bq[nt][s >> 1][2 * (s & 1) + 1], bs[nt]);
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mma32_bf16(af[mt], bf[nt], acc[mt][nt]);
      }
    };

    // two-step ping-pong without branches (as in the bf16 tiled kernel)
    load_b(b0q, s0q, 0);  // weights first: they do not wait for the row -> token lookup
    load_a(0);
    store_a(As[0]);
    __syncthreads();
    int kt = 0;
    for (; kt + 2 <= nkt; kt += 2) {
      load_a(min(kt + 1, nkt - 1));
      load_b(b1q, s1q, min(kt + 1, nkt - 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(As[0], b0q, s0q);
      __builtin_amdgcn_sched_barrier(0);
      store_a(As[1]);
      __syncthreads();
      load_a(min(kt + 2, nkt - 1));
      load_b(b0q, s0q, min(kt + 2, nkt - 1));
      __builtin_amdgcn_sched_barrier(0);
      compute(As[1], b1q, s1q);
      __builtin_amdgcn_sched_barrier(0);
      store_a(As[0]);
      __syncthreads();
    }
    if (kt < nkt) compute(As[0], b0q, s0q);

    // epilogue through LDS (as in the bf16 tiled kernel)
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt) {
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
    const int ncols = GATEUP ? ld : a.d;
    constexpr int CK = NC / 8;
#pragma unroll
    for (int q = 0; q < 32 * MTA * CK / 256; ++q) {
      const int idx = tid + 256 * q, r = idx / CK, ck = idx % CK, col = n0 + 8 * ck;
      if (r < mrows && col < ncols)
        st16(out + (size_t)(row0 + r) * ld + col, *reinterpret_cast<const u32x4*>(&smem[r * LDH + 8 * ck]));
    }
  };
  const int mta = (GATEUP ? a.rowskip_gu : a.rowskip_dn) ? (mrows + 31) >> 5 : 4;
  if (mta >= 4) body(std::integral_constant<int, 4>{});
  else if (mta == 3) body(std::integral_constant<int, 3>{});
  else if (mta == 2) body(std::integral_constant<int, 2>{});
  else body(std::integral_constant<int, 1>{});
}

// ------------------------------------------------------------------ launch
template <bool GATEUP, bool TILED>
static void launch_fp8(const FfnArgs& a, int grid, hipStream_t s) {
  if (a.wstream) hipLaunchKernelGGL((ffn_tiled_fp8_kernel<GATEUP, TILED, true>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((ffn_tiled_fp8_kernel<GATEUP, TILED, false>), dim3(grid), dim3(256), 0, s, a);
}

void launch_tiled_fp8(bool gateup, const FfnArgs& a, int grid, hipStream_t s) {
  if (gateup) {
    if (a.wtiled) launch_fp8<true, true>(a, grid, s);
    else launch_fp8<true, false>(a, grid, s);
  } else {
    if (a.wtiled) launch_fp8<false, true>(a, grid, s);
    else launch_fp8<false, false>(a, grid, s);
  }
}

}  // namespace moe
