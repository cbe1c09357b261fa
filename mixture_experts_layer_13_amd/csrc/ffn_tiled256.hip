// Tiled (large-M, prefill) bf16 expert FFN kernels for gfx950 with 256-row x
// 256-weight-row blocks fed through an LDS ring by direct global -> LDS loads.
//
// The 128-row kernel (ffn_tiled.hip) keeps one K step of operands in flight per
// wave in registers.  Here a block of eight waves (two per SIMD) owns 256 rows x
// 256 weight rows, which halves the operand bytes per flop, and stages both
// operands in a ring of P = 4 LDS slots of one 32-wide K step each (128 KB, one
// block per CU), filled by global_load_lds_dwordx4 (each lane's 16 bytes go
// straight to LDS, no registers held): three K steps stay in flight while one
// is computed.  With two waves per SIMD one wave's LDS fragment reads and waits
// overlap the other's MFMAs (a four-wave form, one wave per SIMD and 4 x 4
// tiles each, lost that time: DeepSeek-V3-shaped gate/up at T=16384 9.42 ms
// against 9.12, down 5.33 against 4.88); a fifth slot (the whole 160 KB)
// measured slower (9.35 ms).
//
// LDS image of one slot: A (activation rows) then B (weight rows), each 16
// groups of 16 rows x 64 bytes (32 bf16 of K), 1 KB per group, written by one
// DMA instruction (lane l's 16 bytes land at byte 16 l of the group).  Weights
// in the tiled layout keep its unit-major order (16-byte unit 16 q + n holds
// bytes 16 q .. +15 of row n), so a B group is one contiguous KB of memory.
// Gathered activation rows use a row-major order (unit 4 n + v holds row n),
// so each group of four lanes reads one contiguous 64-byte run, with the four
// units of a row XOR-permuted by f(n) = ((n / 2) xor (n / 8)) % 4.  In both
// images the MFMA fragment reads (lane l: row l % 32, K half l / 32 of a
// 16-wide slice) hit distinct banks within every group of sixteen lanes (and
// so of eight): a 128-bit LDS read of gfx950 serves sixteen lanes, 256 bytes,
// per cycle.  The four rows n = r, r + 4, r + 8, r + 12 share a 256-byte bank
// window there and f gives them four different units; the earlier f = (n / 2)
// % 4, distinct only over eight lanes, cost 2.6 bank-conflict cycles per LDS
// instruction (SQ_LDS_BANK_CONFLICT).
//
// Waits.  The compiler tracks LDS written by DMA only coarsely (it drains every
// outstanding load before the first LDS read of a loop iteration, and a
// workgroup fence drains them at every barrier), so the DMA instructions are
// written as inline assembly the compiler does not model, and the kernel waits
// on the vector-memory counter itself: before the barrier that publishes K step
// t + 1 each wave waits until only the 4 loads per step it issued for later
// steps are outstanding; the barrier then also tells every wave that all waves
// have finished reading the slot that the next DMA overwrites.  The main loop
// issues no other vector-memory instruction, so those counts are exact.
//
// Waves: wave w = 4 i + j owns rows 128 i .. +127 and weight rows of column
// quarter j (gate/up: gate channels n0 + 32 j .. +31 and the up rows of the
// same channels; down: output columns n0 + 64 j .. +63) as 4 x 2 tiles of 32 x
// 32 (v_mfma_f32_32x32x16_bf16, 128 fp32 accumulators per lane).  Every output
// element sums the same products in the same K order as the 128-row kernel, so
// the two give identical results, bit for bit.  The main loop is instantiated
// for 0-4 of a wave's 32-row tiles holding rows of the item: the idle tiles of
// a partly filled item cost no MFMAs and no LDS fragment reads (their rows are
// still fetched, as copies of the item's last row, so that every wave issues
// the same loads per K step and the waits keep their exact counts).  The host
// turns this off where an expert's items share weight slabs: a skipping item
// runs ahead of the others over the same slab and their L2 hits turn to misses.
#include "ffn_common.hpp"

namespace moe {

namespace {

constexpr int kWaves = 8;                // waves per block
constexpr int kRingP = 4;                // LDS slots
constexpr int kStepK = 32;               // K elements per slot
constexpr int kSlotB = 16384;            // bytes of one operand in a slot (16 groups x 1 KB)
constexpr int kSlot = 2 * kSlotB;        // A then B

// 16 bytes per lane from global memory into LDS at lds + 16 * lane.  M0 carries
// the wave-uniform LDS address; it is restored afterwards, so the compiler's own
// view of M0 stays valid.  One wait state after writing M0 (the LDS-DMA hazard).
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  uint32_t keep;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(keep)
      : "v"(g), "s"(lds)
      : "memory");
}

// s_waitcnt with only the vector-memory count set (gfx9 encoding: vmcnt bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N> __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// waits until at most n K steps of D loads each are outstanding (n wave-uniform, 0..4)
template <int D> __device__ __forceinline__ void wait_steps(int n) {
  if (n >= 4) wait_vm<4 * D>();
  else if (n == 3) wait_vm<3 * D>();
  else if (n == 2) wait_vm<2 * D>();
  else if (n == 1) wait_vm<D>();
  else wait_vm<0>();
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// keeps the compiler from moving memory accesses across this point (emits nothing)
__device__ __forceinline__ void mem_fence_compiler() { asm volatile("" ::: "memory"); }
// s_barrier with compiler-level ordering on both sides: LDS reads stay on their side of it
__device__ __forceinline__ void block_barrier() {
  mem_fence_compiler();
  __builtin_amdgcn_s_barrier();
  mem_fence_compiler();
}

}  // namespace

// SKIP: skip the idle 32-row tiles (else a wave computes all four of its tiles or none)
template <bool GATEUP, bool TILED, bool SKIP>
__global__ __launch_bounds__(64 * kWaves, 1) void ffn_tiled256_kernel(FfnArgs a) {
  constexpr int NW = kWaves;
  constexpr int NT = GATEUP ? 128 : 256;  // output channels (gate/up) or columns (down) per block
  constexpr int NTH = 64 * NW;            // threads
  constexpr int GPW = 16 / NW;            // A groups and B groups each wave loads per K step
  constexpr int kDma = 2 * GPW;           // DMA instructions per wave and K step
  constexpr int NCW = NW / 2;             // waves over the weight rows (two over the rows)
  constexpr int NB = 8 / NCW;             // 32-row weight tiles per wave
  constexpr int GT = NB / 2;              // gate/up: gate tiles per wave (and as many up tiles)
  __shared__ __attribute__((aligned(1024))) char smem[kRingP * kSlot];
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
  const int tid = threadIdx.x, lane = lane_id();
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = w / NCW, wj = w % NCW;
  TileInfo ti;
  if (!tile_of(a, NT, ti)) return;
  const int e = ti.e, row0 = ti.row0, mrows = ti.mrows, n0 = ti.n0;
  const bool shared = ti.shared;
  const int Kfull = GATEUP ? a.d : (shared ? a.S * a.FS : a.F);
  const int Kseg = GATEUP ? a.d : (shared ? a.FS : a.F);
  const int Kb = Kseg * 2;  // bytes per weight row of one K segment
  const int nkt = Kfull / kStepK;

  // ---- DMA sources: this wave fills A groups and B groups GPW w .. GPW w + GPW - 1.
  // Row-major image (activations, and weights in the row layout): lane l loads row l / 4 of the
  // group, so every group of four lanes reads one contiguous 64-byte run (rows spread over the
  // lanes of a quad cost the address and tag units one lookup per lane), and it stores K unit
  // v = l % 4 of that row's slot, holding logical unit u = v ^ f(row): the XOR keeps the
  // fragment reads below (sixteen lanes, sixteen rows, one unit) on distinct banks.
  const int rn = lane >> 2, ru = (lane & 3) ^ (((rn >> 1) ^ (rn >> 3)) & 3);  // row in group, logical 16-byte unit
  const char* asrc[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int r = min(16 * (GPW * w + gi) + rn, mrows - 1);
    if (GATEUP) {
      int tok = shared ? row0 + r : a.row_token[row0 + r];
      tok = min(max(tok, 0), a.T - 1);
      asrc[gi] = (const char*)a.x + ((size_t)tok * a.d + 8 * ru) * 2;
    } else {
      asrc[gi] = (const char*)(shared ? a.hsh : a.h) + ((size_t)(row0 + r) * Kfull + 8 * ru) * 2;
    }
  }
  const char* bmat[2];
  if (GATEUP) {
    bmat[0] = (const char*)(shared ? a.shg : expert_mat<bf16>(a.wg, e, a.F, a.d));
    bmat[1] = (const char*)(shared ? a.shu : expert_mat<bf16>(a.wu, e, a.F, a.d));
  } else {
    bmat[0] = bmat[1] = (const char*)(shared ? a.shd : expert_mat<bf16>(a.wd, e, a.d, Kseg));
  }
  uint32_t boff[GPW];
  const char* bsrc[GPW];
#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int g = GPW * w + gi;  // B group of the block: gate/up 0..7 gate, 8..15 up
    int row;
    if (GATEUP) row = n0 + 16 * (g & 7) + rn;
    else row = min(n0 + 16 * g, a.d - 16) + rn;  // a last block may run past d: re-read, never stored
    // tiled layout: the group's KB of this K chunk is contiguous and lane l takes its bytes 16 l
    // (unit-major image); row layout: the row-major image as for the activations
    boff[gi] = TILED ? (uint32_t)(row & ~15) * Kb + 16 * lane : (uint32_t)row * Kb + 16 * ru;
    bsrc[gi] = bmat[GATEUP ? (g >> 3) : 0];
  }
  constexpr uint32_t cstride = TILED ? 1024u : 64u;  // bytes between consecutive 32-K chunks of a row
  // byte offset of K step kt inside the weight matrix (shared down: slab kt*32 / Kseg)
  auto woff = [&](int kt) -> size_t {
    const int k0 = kt * kStepK;
    const int slab = (!GATEUP && shared) ? k0 / Kseg : 0;
    const int kk = k0 - slab * Kseg;
    return (size_t)slab * a.d * Kb + (size_t)(kk / kStepK) * cstride;
  };
  auto issue = [&](int kt) {
    const uint32_t slot = lds0 + (uint32_t)(kt % kRingP) * kSlot;
    const size_t wo = woff(kt);
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) dma16(asrc[gi] + (size_t)kt * (kStepK * 2), slot + (GPW * w + gi) * 1024);
#pragma unroll
    for (int gi = 0; gi < GPW; ++gi) dma16(bsrc[gi] + wo + boff[gi], slot + kSlotB + (GPW * w + gi) * 1024);
  };

  // ---- fragment reads: lane l takes row n = l % 16 of group 2 m + (l % 32) / 16 of a 32-row tile
  // and logical unit u = 2 s + l / 32 of slice s: at byte 64 n + 16 (u ^ f(n)) of the row-major
  // image, at 256 u + 16 n of the unit-major one.  Slice 1 of the row-major image is slice 0's
  // offset with bit 5 flipped.
  const int fn = lane & 15, fh = lane >> 5, fx = ((fn >> 1) ^ (fn >> 3)) & 3;
  const int rofs = ((lane >> 4) & 1) * 1024 + 64 * fn + 16 * ((fx & 2) | (fh ^ (fx & 1)));
  const int uofs = ((lane >> 4) & 1) * 1024 + 256 * fh + 16 * fn;
  const int aofs[2] = {rofs, rofs ^ 32};
  const int bofs[2] = {TILED ? uofs : rofs, TILED ? uofs + 512 : (rofs ^ 32)};
  int ga[4], gb[NB];
#pragma unroll
  for (int m = 0; m < 4; ++m) ga[m] = 8 * wi + 2 * m;
#pragma unroll
  for (int n = 0; n < NB; ++n) gb[n] = GATEUP ? ((n / GT) * 8 + 2 * GT * wj + 2 * (n % GT)) : (2 * NB * wj + 2 * n);
  // 32-row tiles of this wave that it computes: those holding rows of the item, or without
  // SKIP all four unless none does (0: the wave only moves data)
  const int ma = SKIP ? min(max((mrows - 128 * wi + 31) / 32, 0), 4) : (128 * wi < mrows ? 4 : 0);
  const bool active = ma > 0;

  f32x16 acc[4][NB];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < NB; ++n) acc[m][n] = f32x16{};
  u32x4 fa[2][4], fb[2][NB];
  // MA: the wave's row tiles that hold rows (compile-time), the first MA of its four
  auto rd = [&](auto ma_tag, int kt, int s, u32x4 (&A)[4], u32x4 (&B)[NB]) {
    constexpr int MA = decltype(ma_tag)::value;
    const char* slot = smem + (kt % kRingP) * kSlot;
#pragma unroll
    for (int m = 0; m < MA; ++m) A[m] = *reinterpret_cast<const u32x4*>(slot + aofs[s] + ga[m] * 1024);
#pragma unroll
    for (int n = 0; n < NB; ++n) B[n] = *reinterpret_cast<const u32x4*>(slot + kSlotB + bofs[s] + gb[n] * 1024);
  };
  auto mma = [&](auto ma_tag, const u32x4 (&A)[4], const u32x4 (&B)[NB]) {
    constexpr int MA = decltype(ma_tag)::value;
#pragma unroll
    for (int m = 0; m < MA; ++m)
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[m][n] = mma32_bf16(A[m], B[n], acc[m][n]);
  };
  // the MA + NB LDS reads of one slice go out between the first MFMAs of the other
  // (pinned: left alone, the scheduler bunches them)
  auto pin_slice = [&](auto ma_tag) {
    constexpr int MA = decltype(ma_tag)::value;
    constexpr int R = MA + NB, M = MA * NB, P = R < M ? R : M;
#pragma unroll
    for (int i = 0; i < P; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (M > P) __builtin_amdgcn_sched_group_barrier(0x008, M - P, 0);
    if constexpr (R > P) __builtin_amdgcn_sched_group_barrier(0x100, R - P, 0);
  };

  // Main loop.  MA = 0: the wave only moves data and meets the barriers.
  auto run = [&](auto ma_tag) {
    constexpr bool ACT = decltype(ma_tag)::value > 0;
    const int pro = min(kRingP, nkt);
    for (int kt = 0; kt < pro; ++kt) issue(kt);
    wait_steps<kDma>(pro - 1);  // K step 0 landed; the others stay in flight
    block_barrier();
    if (ACT) rd(ma_tag, 0, 0, fa[0], fb[0]);
    int kt = 0;
    // steady state: K step kt + 1 must have landed at the barrier, kt + 2 .. kt + P - 1 stay in
    // flight, and K step kt + P goes into the slot of kt (every wave has read it by then)
    for (; kt + kRingP < nkt; ++kt) {
      if (ACT) {
        rd(ma_tag, kt, 1, fa[1], fb[1]);
        mma(ma_tag, fa[0], fb[0]);
        pin_slice(ma_tag);
        mem_fence_compiler();
        wait_lgkm0();
      }
      wait_steps<kDma>(kRingP - 2);
      block_barrier();
      issue(kt + kRingP);
      if (ACT) {
        rd(ma_tag, kt + 1, 0, fa[0], fb[0]);
        mma(ma_tag, fa[1], fb[1]);
        pin_slice(ma_tag);
      }
    }
    // the last (at most P) K steps: everything is issued, the waits shrink
    for (; kt < nkt; ++kt) {
      if (ACT) {
        rd(ma_tag, kt, 1, fa[1], fb[1]);
        mma(ma_tag, fa[0], fb[0]);
        mem_fence_compiler();
        wait_lgkm0();
      }
      if (kt + 1 < nkt) {
        const int later = nkt - 2 - kt;  // K steps issued after kt + 1
        wait_steps<kDma>(min(later, kRingP - 2));
        block_barrier();
        if (ACT) rd(ma_tag, kt + 1, 0, fa[0], fb[0]);
      }
      if (ACT) mma(ma_tag, fa[1], fb[1]);
    }
  };
  // (the instantiations for 1-3 tiles exist only with SKIP: beside them the compiler schedules
  // the four-tile loop less well, DeepSeek-V3-shaped gate/up at T=16384 1.5% slower)
  if (ma == 4) run(std::integral_constant<int, 4>{});
  else if (SKIP && ma == 3) run(std::integral_constant<int, SKIP ? 3 : 4>{});
  else if (SKIP && ma == 2) run(std::integral_constant<int, SKIP ? 2 : 4>{});
  else if (SKIP && ma == 1) run(std::integral_constant<int, SKIP ? 1 : 4>{});
  else run(std::integral_constant<int, 0>{});

  // ---- epilogue through LDS: staged 16-byte row chunks
  wait_vm<0>();
  __syncthreads();  // every wave is done with the ring
  bf16* const stage = reinterpret_cast<bf16*>(smem);
  bf16* const out = (bf16*)(GATEUP ? (shared ? a.hsh : a.h) : (shared ? a.ysh : a.y));
  const int ld = GATEUP ? (shared ? a.S * a.FS : a.F) : a.d;
  const int h = lane >> 5, c = lane & 31;
  if (GATEUP) {
    // 256 rows x 128 channels: wave (i, j) writes rows 128 i.., channels 32 GT j..
    constexpr int LDH = 128 + 8;
    if (active) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int n = 0; n < GT; ++n)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = 128 * wi + 32 * m + 8 * (i >> 2) + 4 * h + (i & 3);
            stage[r * LDH + 32 * GT * wj + 32 * n + c] = (bf16)(silu(acc[m][n][i]) * acc[m][n + GT][i]);
          }
        mem_fence_compiler();
      }
    }
    __syncthreads();
    constexpr int CK = 128 / 8;
#pragma unroll 4
    for (int q = 0; q < 256 * CK / NTH; ++q) {
      const int idx = tid + NTH * q, r = idx / CK, ck = idx % CK;
      if (r < mrows) st16(out + (size_t)(row0 + r) * ld + n0 + 8 * ck, *reinterpret_cast<const u32x4*>(&stage[r * LDH + 8 * ck]));
    }
  } else {
    // 256 rows x 256 columns, in two passes of 128 rows (the staging tile would not fit at once)
    constexpr int LDH = 256 + 8;
    constexpr int CK = 256 / 8;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      if (wi == pass && active) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
#pragma unroll
          for (int n = 0; n < NB; ++n)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int r = 32 * m + 8 * (i >> 2) + 4 * h + (i & 3);
              stage[r * LDH + 32 * NB * wj + 32 * n + c] = (bf16)acc[m][n][i];
            }
          mem_fence_compiler();  // one row tile at a time keeps the accumulator reads short-lived
        }
      }
      __syncthreads();
#pragma unroll 4
      for (int q = 0; q < 128 * CK / NTH; ++q) {
        const int idx = tid + NTH * q, r = idx / CK, ck = idx % CK, col = n0 + 8 * ck;
        const int row = 128 * pass + r;
        if (row < mrows && col < a.d)
          st16(out + (size_t)(row0 + row) * ld + col, *reinterpret_cast<const u32x4*>(&stage[r * LDH + 8 * ck]));
      }
      __syncthreads();
    }
  }
}

template <bool GATEUP, bool TILED>
static void launch256(const FfnArgs& a, int grid, hipStream_t s) {
  const dim3 blk(64 * kWaves);
  if (GATEUP ? a.rowskip_gu : a.rowskip_dn) hipLaunchKernelGGL((ffn_tiled256_kernel<GATEUP, TILED, true>), dim3(grid), blk, 0, s, a);
  else hipLaunchKernelGGL((ffn_tiled256_kernel<GATEUP, TILED, false>), dim3(grid), blk, 0, s, a);
}

void launch_tiled256_bf16(bool gateup, const FfnArgs& a, int grid, hipStream_t s) {
  if (gateup) {
    if (a.wtiled) launch256<true, true>(a, grid, s);
    else launch256<true, false>(a, grid, s);
  } else {
    if (a.wtiled) launch256<false, true>(a, grid, s);
    else launch256<false, false>(a, grid, s);
  }
}

}  // namespace moe
