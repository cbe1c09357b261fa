// Expert FFN with FP8 (OCP E4M3) weights AND FP8 activations on gfx950's FP8
// matrix unit (v_mfma_scale_f32_32x32x64_f8f6f4, both operands E4M3, block
// scales fixed at 2^0).  "MoE at the inference level", workarounds and Fields:
// fp8 expert weights (weight_dtype) halve the bytes; run on the FP8 matrix unit
// they also double the matrix rate, which takes the activations in FP8 too.
//
// Quantisation of an activation row (x_t for the gate/up GEMM, the bf16 SwiGLU
// output h for the down GEMM): amax = max |v|, inv = 448 / amax and scale =
// amax / 448 in IEEE fp32, code_i = E4M3(v_i * inv) rounded to nearest even;
// an all-zero row has codes 0 and scale 0.  quant_rows_e4m3_kernel writes the
// codes and the row scales ahead of each GEMM.  A GEMM then accumulates code
// products in fp32 and its epilogue multiplies by the row's scale and the
// output channel's weight scale.
//
// The tiled GEMM keeps the bf16 tiled kernel's structure and byte traffic per
// K step: 128 rows x 256 weight rows per block, four waves of 4 x 2 tiles of
// 32 x 32, the activation tile through double-buffered LDS, weights straight
// into operand registers one K step ahead.  A K step is 128 wide (128 bytes of
// a row, two 64-byte chunks), i.e. two FP8 MFMAs per tile.  Operand layout: an
// FP8 MFMA lane l supplies 32 bytes of row (weight row) l % 32; the same byte
// positions of the A and B operands must hold the same K, whatever K order the
// unit assigns to them.  Lane half h = l / 32 takes, of 64-byte chunk j, the
// 16-byte units h and 2 + h (bytes 16h.. and 32 + 16h..) of both operands.
#include "ffn_common.hpp"
#include "kernels_f8f8.hpp"

namespace moe {

typedef int i32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x16 mma32_fp8(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1, f32x16 c) {
  const i32x8 a = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
  const i32x8 b = __builtin_bit_cast(i32x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
  // formats 0 / 0: both operands E4M3; E8M0 block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ------------------------------------------------------------------ activation quantisation
// One wave per row.  Two segments in one launch (the routed h rows and the
// shared experts' h rows); blocks [0, nb0) take segment 0.
struct QuantSeg {
  const bf16* src;  // [rows][cols]
  uint8_t* q;       // [rows][cols] codes, or with bf16 set [rows][cols] bf16 values of the codes
  float* scale;     // [rows]
  int rows, cols;
  int bf16;         // store each code as its (exact) bf16 value: the streaming kernels' operand
};

__global__ __launch_bounds__(256) void quant_rows_e4m3_kernel(QuantSeg s0, QuantSeg s1, int nb0) {
  const bool first = (int)blockIdx.x < nb0;
  const QuantSeg& sg = first ? s0 : s1;
  const int r = (first ? (int)blockIdx.x : (int)blockIdx.x - nb0) * 4 + (int)(threadIdx.x >> 6);
  if (r >= sg.rows) return;
  const int lane = lane_id(), nch = sg.cols / 8;
  const char* row = reinterpret_cast<const char*>(sg.src) + (size_t)r * sg.cols * 2;
  float m = 0.f;
  for (int c = lane; c < nch; c += kWave) {
    const u32x4 v = ld16(row + 16 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m = fmaxf(m, fmaxf(fabsf(bf16_bits_to_f32(v[i] & 0xFFFFu)), fabsf(bf16_bits_to_f32(v[i] >> 16))));
  }
  float mv[1] = {m};
  wave_max_n<1>(mv);
  m = mv[0];
  const float inv = m > 0.f ? __fdiv_rn(448.f, m) : 0.f;
  uint8_t* qrow = sg.q + (size_t)r * sg.cols * (sg.bf16 ? 2 : 1);
  for (int c = lane; c < nch; c += kWave) {
    const u32x4 v = ld16(row + 16 * c);
    uint32_t w[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      // element 2i of the pair goes to the lower byte
      int o = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_bits_to_f32(v[2 * p] & 0xFFFFu) * inv,
                                              bf16_bits_to_f32(v[2 * p] >> 16) * inv, 0, false);
      o = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_bits_to_f32(v[2 * p + 1] & 0xFFFFu) * inv,
                                          bf16_bits_to_f32(v[2 * p + 1] >> 16) * inv, o, true);
      w[p] = (uint32_t)o;
    }
    if (sg.bf16) {
      // codes 4p .. 4p + 3 of the chunk back to fp32 (exact) and to bf16 (exact: 4 significant bits)
      u32x4 b;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[p], false);
        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[p], true);
        b[2 * p] = pack_bf16x2(lo[0], lo[1]);
        b[2 * p + 1] = pack_bf16x2(hi[0], hi[1]);
      }
      st16(qrow + 16 * c, b);
    } else {
      *reinterpret_cast<uint2*>(qrow + 8 * c) = make_uint2(w[0], w[1]);
    }
  }
  if (lane == 0) sg.scale[r] = m > 0.f ? __fdiv_rn(m, 448.f) : 0.f;
}

hipError_t launch_quant_rows(const void* src0, void* q0, float* sc0, int rows0, int cols0, const void* src1, void* q1,
                             float* sc1, int rows1, int cols1, bool bf16_codes, hipStream_t s) {
  QuantSeg a{(const bf16*)src0, (uint8_t*)q0, sc0, rows0, cols0, bf16_codes ? 1 : 0};
  QuantSeg b{(const bf16*)src1, (uint8_t*)q1, sc1, src1 ? rows1 : 0, cols1, bf16_codes ? 1 : 0};
  const int nb0 = (a.rows + 3) / 4, nb1 = (b.rows + 3) / 4;
  if (nb0 + nb1 == 0) return hipSuccess;
  hipLaunchKernelGGL(quant_rows_e4m3_kernel, dim3(nb0 + nb1), dim3(256), 0, s, a, b, nb0);
  return hipGetLastError();
}

// ------------------------------------------------------------------ tiled FP8 x FP8 GEMMs
// A operand: the quantised activations (x codes gathered through row_token for
// gate/up; h codes for down); B operand: the fp8 weight rows.  The shared
// experts' down GEMM runs over their S concatenated K slabs, each with its own
// channel scales, as S passes of the K loop: with s'_j = s_j (or 1 where a
// channel's scale is 0, whose codes are then all 0), the sums are multiplied by
// s'_j / s'_(j+1) between slab j and slab j + 1 and by the last slab's s' in the
// epilogue, which gives the sum over j of s'_j times slab j's products.
// STREAMW: weights loaded non-temporally (each expert's weights read by one row tile).
template <bool GATEUP, bool TILED, bool STREAMW>
__global__ __launch_bounds__(256, 2) void ffn_tiled_f8f8_kernel(FfnArgs a, A8Args qa) {
  constexpr int KSTEP = 128, SUB = KSTEP / 64;  // bytes (= K) per step; FP8 MFMAs per tile per step
  constexpr int LDA = KSTEP + 16;               // padded LDS row in bytes (the bf16 kernel's 144)
  constexpr int CPR = KSTEP / 16;               // 16-byte chunks per A row per step
  constexpr int CPT = TBM * CPR / 256;          // A chunks per thread per step
  constexpr int RPT = 256 / CPR;                // row stride between a thread's chunks
  constexpr int NT = GATEUP ? 128 : 256;        // output channels per block
  constexpr uint32_t cstride = TILED ? 1024u : 64u;  // bytes between the 64-byte chunks of a weight row
  constexpr uint32_t hstride = TILED ? 512u : 32u;   // bytes from unit h to unit 2 + h
  constexpr int NC = NT;
  constexpr int LDH = NC + 8;  // padded row (bf16 elements) of the output staging tile
  constexpr int SMEM = 2 * TBM * LDA > TBM * LDH * 2 ? 2 * TBM * LDA : TBM * LDH * 2;
  static_assert(CPT == 4 && RPT == 32, "a thread's activation chunk q must lie in row tile q");
  __shared__ __align__(16) unsigned char smem[SMEM];
  __shared__ float rscale[TBM];
  unsigned char* const As[2] = {smem, smem + TBM * LDA};
  const int tid = threadIdx.x, lane = lane_id(), w = tid >> 6, h = lane >> 5, c = lane & 31;
  TileInfo ti;
  if (!tile_of(a, NT, ti)) return;
  const int e = ti.e, row0 = ti.row0, mrows = ti.mrows, n0 = ti.n0;
  const bool shared = ti.shared;
  const int Kfull = GATEUP ? a.d : (shared ? a.S * a.FS : a.F);  // K of the activation rows
  const int Kseg = GATEUP ? a.d : (shared ? a.FS : a.F);          // K of one weight matrix
  const int nslab = Kfull / Kseg;                                  // weight slabs (shared down: S)
  const uint32_t Kb = (uint32_t)Kseg;                              // bytes per weight row

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
  float wsc[2];  // the lane's output-channel weight scales (gate, up; or its two down columns)
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    // a last down block may be half past d: its surplus tiles re-read the last 32 rows, results unused
    const int rb = GATEUP ? n0 + 32 * w : min(n0 + 64 * w + 32 * nt, a.d - 32);
    const int row = rb + c;
    boff[nt] = TILED ? (uint32_t)(row & ~15) * Kb + 256 * h + 16 * (row & 15) : (uint32_t)row * Kb + 16 * h;
    const float sv = smat[nt][row];
    wsc[nt] = sv == 0.f ? 1.f : sv;
  }
  // activation chunk sources: rows (tid / CPR) + RPT q, 16-byte chunk tid % CPR; row scales
  const int ch = tid % CPR;
  const unsigned char* aptr[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int r = min(tid / CPR + RPT * q, mrows - 1);
    if (GATEUP) {
      int tok = shared ? row0 + r : a.row_token[row0 + r];
      tok = min(max(tok, 0), a.T - 1);
      aptr[q] = qa.xq + (size_t)tok * a.d + ch * 16;
    } else {
      aptr[q] = (shared ? qa.hshq : qa.hq) + (size_t)(row0 + r) * Kfull + ch * 16;
    }
  }
  if (tid < TBM) {
    const int r = min(tid, mrows - 1);
    float sv;
    if (GATEUP) {
      int tok = shared ? row0 + r : a.row_token[row0 + r];
      tok = min(max(tok, 0), a.T - 1);
      sv = qa.xs[tok];
    } else {
      sv = (shared ? qa.hshs : qa.hs)[row0 + r];
    }
    rscale[tid] = sv;
  }

  u32x4 b0q[2][2 * SUB], b1q[2][2 * SUB];
  const int nkt = Kseg / KSTEP;  // K steps of one slab
  size_t slab_off = 0;           // byte offset of the current slab's weight matrix
  int slab_k = 0;                // first K step of the current slab in the activation rows
  auto load_b = [&](u32x4 (&bq)[2][2 * SUB], int kt) {
    const size_t o = slab_off + (size_t)(kt * KSTEP / 64) * cstride;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int u = 0; u < 2 * SUB; ++u) {
        const char* src = bmat[nt] + o + (u >> 1) * cstride + (u & 1) * hstride;
        if constexpr (STREAMW) bq[nt][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + boff[nt]));
        else bq[nt][u] = ld16_at(src, boff[nt]);
      }
  };

  auto body = [&](auto mta_tag) {
    constexpr int MTA = decltype(mta_tag)::value;
    constexpr int NF = SUB * MTA;  // A fragments (slice, row tile) per step
    f32x16 acc[MTA][2];
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16{};
    u32x4 ar[CPT];
    auto load_a = [&](int kt) {
#pragma unroll
      for (int q = 0; q < MTA; ++q) ar[q] = ld16(aptr[q] + (slab_k + kt) * KSTEP);
    };
    auto store_a = [&](unsigned char* dst) {
#pragma unroll
      for (int q = 0; q < MTA; ++q) *reinterpret_cast<u32x4*>(&dst[(tid / CPR + RPT * q) * LDA + ch * 16]) = ar[q];
    };
    // fragment f = (slice s = f / MTA, row tile mt = f % MTA): bytes 64 s + 16 h and 64 s + 32 + 16 h
    // of the tile's row c; the next fragment's two LDS reads issue while this one's two MFMAs run
    auto compute = [&](const unsigned char* A, const u32x4 (&bq)[2][2 * SUB]) {
      auto rd = [&](int f, u32x4& x0, u32x4& x1) {
        const unsigned char* p = &A[(32 * (f % MTA) + c) * LDA + 64 * (f / MTA) + 16 * h];
        x0 = *reinterpret_cast<const u32x4*>(p);
        x1 = *reinterpret_cast<const u32x4*>(p + 32);
      };
      u32x4 a0, a1;
      rd(0, a0, a1);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        u32x4 n0v = a0, n1v = a1;
        if (f + 1 < NF) rd(f + 1, n0v, n1v);
        const int s = f / MTA, mt = f % MTA;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = mma32_fp8(a0, a1, bq[nt][2 * s], bq[nt][2 * s + 1], acc[mt][nt]);
        a0 = n0v;
        a1 = n1v;
      }
      // order: 2 reads; per fragment but the last: 1 MFMA, 2 reads, 1 MFMA; last: 2 MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int f = 0; f + 1 < NF; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    };

    for (int slab = 0; slab < nslab; ++slab) {
      if (slab > 0) {
        // the next shared slab: its weights and scales, the sums rescaled to them; every wave is
        // done reading the activation buffers before they are refilled
        slab_off = (size_t)slab * a.d * Kb;
        slab_k = slab * nkt;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int row = min(n0 + 64 * w + 32 * nt, a.d - 32) + c;
          float cur = smat[nt][(size_t)slab * a.d + row];
          cur = cur == 0.f ? 1.f : cur;
          const float ratio = wsc[nt] / cur;
#pragma unroll
          for (int mt = 0; mt < MTA; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] *= ratio;
          wsc[nt] = cur;
        }
        __syncthreads();
      }
      // two-step ping-pong without branches (as in the bf16 tiled kernel)
      load_b(b0q, 0);
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
    }

    // epilogue through LDS: row scale x channel scale, SwiGLU (gate/up), one bf16 rounding
    __syncthreads();
    bf16* const stage = reinterpret_cast<bf16*>(smem);
#pragma unroll
    for (int mt = 0; mt < MTA; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
        const float rs = rscale[r];
        if (GATEUP) {
          const float g = acc[mt][0][i] * (rs * wsc[0]), u = acc[mt][1][i] * (rs * wsc[1]);
          stage[r * LDH + 32 * w + c] = (bf16)(silu(g) * u);
        } else {
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) stage[r * LDH + 64 * w + 32 * nt + c] = (bf16)(acc[mt][nt][i] * (rs * wsc[nt]));
        }
      }
    }
    __syncthreads();
    bf16* const out = (bf16*)(GATEUP ? (shared ? a.hsh : a.h) : (shared ? a.ysh : a.y));
    const int ld = GATEUP ? (shared ? a.S * a.FS : a.F) : a.d;
    const int ncols = ld;
    constexpr int CK = NC / 8;
#pragma unroll
    for (int q = 0; q < 32 * MTA * CK / 256; ++q) {
      const int idx = tid + 256 * q, r = idx / CK, ck = idx % CK, col = n0 + 8 * ck;
      if (r < mrows && col < ncols)
        st16(out + (size_t)(row0 + r) * ld + col, *reinterpret_cast<const u32x4*>(&stage[r * LDH + 8 * ck]));
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
static void launch_f8f8(const FfnArgs& a, const A8Args& q, int grid, hipStream_t s) {
  if (a.wstream) hipLaunchKernelGGL((ffn_tiled_f8f8_kernel<GATEUP, TILED, true>), dim3(grid), dim3(256), 0, s, a, q);
  else hipLaunchKernelGGL((ffn_tiled_f8f8_kernel<GATEUP, TILED, false>), dim3(grid), dim3(256), 0, s, a, q);
}

void launch_tiled_f8f8(bool gateup, const FfnArgs& a, const A8Args& q, int grid, hipStream_t s) {
  if (gateup) {
    if (a.wtiled) launch_f8f8<true, true>(a, q, grid, s);
    else launch_f8f8<true, false>(a, q, grid, s);
  } else {
    if (a.wtiled) launch_f8f8<false, true>(a, q, grid, s);
    else launch_f8f8<false, false>(a, q, grid, s);
  }
}

}  // namespace moe
