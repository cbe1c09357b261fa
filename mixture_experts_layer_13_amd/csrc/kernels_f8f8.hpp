// Internal interface of the FP8-activation expert FFN (ffn_tiled_f8f8.hip):
// FP8 weights with FP8 activations on the FP8 matrix unit.  Not part of the
// public header.
#pragma once
#include "kernels.hpp"

namespace moe {

// E4M3 codes and fp32 row scales of the GEMMs' activation operands (written by the row
// quantisation, read by the GEMMs)
struct A8Args {
  uint8_t* xq;    // [T][d]
  float* xs;      // [T]
  uint8_t* hq;    // [R][F]
  float* hs;      // [R]
  uint8_t* hshq;  // [T][S * FS] (null without shared experts)
  float* hshs;    // [T]
};

void launch_tiled_f8f8(bool gateup, const FfnArgs& a, const A8Args& q, int grid, hipStream_t s);
// decode sizes: the streaming FP8 kernels on activation rows of E4M3 codes held as bf16, the
// row scales applied in their epilogues (a.x: the x codes for gate/up; a.h / a.hsh: the h codes
// for down)
void launch_stream_ffn_a8(bool gateup, const FfnArgs& a, const A8Args& q, int grid, hipStream_t s);
// the gate/up (gateup) or down GEMM over the tiled kernels' grid
hipError_t launch_ffn_a8(bool gateup, const FfnArgs& a, const A8Args& q, hipStream_t s);
hipError_t launch_ffn_a8_stream(bool gateup, const FfnArgs& a, const A8Args& q, hipStream_t s);
// per-row E4M3 quantisation of bf16 rows (codes and fp32 scales), two segments in one launch
// (src1 null: one segment); bf16_codes: each code stored as its exact bf16 value (2 bytes)
hipError_t launch_quant_rows(const void* src0, void* q0, float* sc0, int rows0, int cols0, const void* src1, void* q1,
                             float* sc1, int rows1, int cols1, bool bf16_codes, hipStream_t s);

}  // namespace moe
