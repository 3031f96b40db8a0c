// Sustained dense bf16 matrix-core rate of the device: a measurement aid
// beside the attention kernels, so that their throughput can be stated as a
// share of what this device's matrix cores sustain under their own clock and
// power limit, not only of the rate quoted at 2.4 GHz.
//
// One workgroup of 8 waves per CU (two per SIMD, the occupancy of the
// attention main pass).  Every wave holds kProbeSets operand pairs (A, B) of
// v_mfma_f32_16x16x32_bf16 in registers, read once from `operands`, and runs
// `iters` rounds of kProbeAcc independent MFMAs: accumulator a adds
// A_{a % kProbeSets} x B_{a % kProbeSets} every round.  The accumulators'
// dependency chains are kProbeAcc MFMAs long, so each MFMA issues as soon as
// the matrix core is free.  With entries in {-1, 0, 1} every product and
// partial sum is a small integer, so after the loop accumulator a holds exactly
// iters * (A_s B_s) as long as iters * 32 < 2^24: the output proves that every
// MFMA ran.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_kernel.h"

namespace chunkattn {

constexpr int kProbeSets = 4;   // operand pairs per wave
constexpr int kProbeAcc = 8;    // independent accumulators per wave
constexpr int kProbeWaves = 8;  // waves per workgroup (one workgroup per CU)
// operand words per lane: kProbeSets x (A fragment, B fragment) x 4 words
constexpr int kProbeWordsPerLane = kProbeSets * 2 * 4;
// output floats per wave: kProbeAcc accumulators x 64 lanes x 4
constexpr int kProbeOutPerWave = kProbeAcc * 64 * 4;

// operands: [lane 0..63][kProbeWordsPerLane] 32-bit words (pairs of bf16), set
// s at words 8s .. 8s+3 (A) and 8s+4 .. 8s+7 (B); the same for every wave.
// out: [workgroup][wave][accumulator][lane][4] floats.
__global__ __launch_bounds__(kProbeWaves * 64, 1) void mfma_peak_probe(const uint32_t* operands,
                                                                       long long iters,
                                                                       float* out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  u32x4_t a[kProbeSets], b[kProbeSets];
#pragma unroll
  for (int s = 0; s < kProbeSets; ++s) {
    const uint32_t* w = operands + lane * kProbeWordsPerLane + 8 * s;
    a[s] = u32x4_t{w[0], w[1], w[2], w[3]};
    b[s] = u32x4_t{w[4], w[5], w[6], w[7]};
  }
  f32x4_t acc[kProbeAcc];
#pragma unroll
  for (int i = 0; i < kProbeAcc; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (long long it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kProbeAcc; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8_t, a[i % kProbeSets]),
          __builtin_bit_cast(bf16x8_t, b[i % kProbeSets]), acc[i], 0, 0, 0);
  }
  float* o = out + ((size_t)blockIdx.x * kProbeWaves + wave) * kProbeOutPerWave;
#pragma unroll
  for (int i = 0; i < kProbeAcc; ++i)
    *reinterpret_cast<f32x4_t*>(o + (i * 64 + lane) * 4) = acc[i];
}

}  // namespace chunkattn
