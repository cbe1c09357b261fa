// Tiled (large-M, prefill) bf16 expert FFN kernels for gfx950 on the
// 32x32x16 MFMA.
#include "ffn_common.hpp"

namespace moe {

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
  static constexpr int KSTEP = 64;
};

// STREAMW: weights loaded non-temporally (when an expert's weights are read by a
// single row tile, nothing is lost by not keeping them in L2).
template <bool GATEUP, bool TILED, bool STREAMW>
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

  u32x4 b0q[2][SUB], b1q[2][SUB];
  const int nkt = Kfull / KSTEP;
  auto load_b = [&](u32x4 (&bq)[2][SUB], int kt) {
    const size_t o = woff(kt);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        const char* src = bmat[nt] + o + (s >> 1) * cstride + (s & 1) * hstride;
        if constexpr (STREAMW) bq[nt][s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + boff[nt]));
        else bq[nt][s] = ld16_at(src, boff[nt]);
      }
  };

  // Main loop and epilogue for MTA active 32-row tiles (1..4): the last item of
  // an expert usually holds fewer than 128 rows, and its idle row tiles then
  // cost no MFMAs, LDS traffic or activation loads.
  auto body = [&](auto mta_tag) {
    constexpr int MTA = decltype(mta_tag)::value;
    f32x16 acc[MTA][2];
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16{};
    u32x4 ar[CPT];
    // a thread's chunk q lies in row tile q (RPT = 32): only q < MTA is needed
    auto load_a = [&](int kt) {
#pragma unroll
      for (int q = 0; q < MTA; ++q) ar[q] = ld16(aptr[q] + kt * KSTEP * 2);
    };
    auto store_a = [&](bf16* dst) {
#pragma unroll
      for (int q = 0; q < MTA; ++q)
        *reinterpret_cast<u32x4*>(&dst[(tid / CPR + RPT * q) * LDA + ch * 8]) = ar[q];
    };
    // one K step: SUB slices of 16.  The MTA activation fragments of slice s + 1
    // are read from LDS while the MFMAs of slice s issue: the group barriers at
    // the end pin that order (left alone, the scheduler places each read right
    // before its first use and the LDS latency shows every time).
    auto compute = [&](const bf16* A, const u32x4 (&bq)[2][SUB]) {
      u32x4 af[MTA];
#pragma unroll
      for (int mt = 0; mt < MTA; ++mt) af[mt] = *reinterpret_cast<const u32x4*>(&A[(32 * mt + c) * LDA + 8 * h]);
#pragma unroll
      for (int s = 0; s < SUB; ++s) {
        u32x4 an[MTA];
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt)
          an[mt] = s + 1 < SUB ? *reinterpret_cast<const u32x4*>(&A[(32 * mt + c) * LDA + 16 * (s + 1) + 8 * h])
                               : af[mt];
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mma32_bf16(af[mt], bq[nt][s], acc[mt][nt]);
#pragma unroll
        for (int mt = 0; mt < MTA; ++mt) af[mt] = an[mt];
      }
      // order: MTA reads (slice 0); per slice but the last: (1 MFMA, 1 read) x MTA,
      // MTA MFMAs; last slice: 2 MTA MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, MTA, 0);
#pragma unroll
      for (int s = 0; s + 1 < SUB; ++s) {
#pragma unroll
        for (int i = 0; i < MTA; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, MTA, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * MTA, 0);
    };

    // two-step ping-pong without branches
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
    // into a 32 MTA x NC staging tile, then the block stores 16-byte row chunks
    __syncthreads();  // every wave is done reading the activation tiles
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
    const int ncols = GATEUP ? ld : a.d;  // a last down block may be half past d
    constexpr int CK = NC / 8;              // 16-byte chunks per staged row
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
static void launch_tiled32(const FfnArgs& a, int grid, hipStream_t s) {
  if (a.wstream) hipLaunchKernelGGL((ffn_tiled32_kernel<GATEUP, TILED, true>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((ffn_tiled32_kernel<GATEUP, TILED, false>), dim3(grid), dim3(256), 0, s, a);
}

void launch_tiled_bf16(bool gateup, const FfnArgs& a, int grid, hipStream_t s) {
  if (gateup) {
    if (a.wtiled) launch_tiled32<true, true>(a, grid, s);
    else launch_tiled32<true, false>(a, grid, s);
  } else {
    if (a.wtiled) launch_tiled32<false, true>(a, grid, s);
    else launch_tiled32<false, false>(a, grid, s);
  }
}

}  // namespace moe
