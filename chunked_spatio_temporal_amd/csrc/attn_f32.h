// gfx950 chunk-attention forward kernel for fp32 storage, computed in fp32.
//
// The attention of one chunk over [predecessor ; own] K/V (DualParal
// write-up, section 三) with fp32 inputs keeps fp32 throughout: both products
// run on the fp32 matrix cores (v_mfma_f32_16x16x4_f32, fp32 operands and
// accumulation), the softmax keeps a running maximum in fp32, and the output
// is stored as fp32.  No operand is rounded to bf16, so the result agrees with
// exact attention to fp32 rounding, and no recheck pass is needed.  Meant for
// the small fp32 configurations (the fp32 matrix-core peak is a sixteenth of
// the bf16 one).
//
// Work item: 64 query rows of one (chunk, head), 4 waves of 16 rows, one
// workgroup per item (the plan's die-aware slot order).  Key/value tiles of 64
// rows pass through LDS: K row-major, V transposed (dims x keys), both with
// rows padded by 16 bytes so that the 16 rows one read instruction spans fall
// in distinct banks.
//
// Per tile and wave, lane (j, g) = (lane & 15, lane >> 4):
//   S^T = K . Q^T    A = K (16 keys x 4 dims), B = Q^T (4 dims x 16 queries).
//                    The contraction runs over the dims in the order
//                    16s + 4g + i (step 4s + i, lane group g), so a lane takes
//                    four consecutive dims of K with one 16-byte read and
//                    holds four consecutive dims of its query per s.
//                    Lane (j, g) gets query j's scores for keys 16kb + 4g + r.
//   softmax          running maximum m per query row (over the four lane
//                    groups of the row), P = 2^(S*scale*log2 e - m), O and l
//                    rescaled when m rises.
//   O^T += V^T . P^T  A = V^T (16 dims x 4 keys), B = P^T (4 keys x 16
//                    queries); the contraction over the keys runs in the order
//                    16kb + 4g + r (step (kb, r), lane group g), so B is the
//                    lane's own P value and A four consecutive keys of V^T.
//                    Lane (j, g) accumulates query j's dims 16db + 4g + rr.
#pragma once

#include "attn_kernel.h"

namespace chunkattn {

typedef float f32x4f_t __attribute__((ext_vector_type(4)));

template <int D>
struct GeoF32 {
  static constexpr int kKStride = D + 4;    // floats per K row in LDS
  static constexpr int kVStride = kBN + 4;  // floats per V^T row (one dim) in LDS
  static constexpr uint32_t kKBytes = kBN * kKStride * 4;
  static constexpr uint32_t kVBytes = D * kVStride * 4;
  static constexpr uint32_t kLdsBytes = kKBytes + kVBytes;
};

template <int D>
constexpr uint32_t kF32LdsBytes = GeoF32<D>::kLdsBytes;

constexpr int kF32BlockRows = 64;  // query rows per work item (4 waves x 16)

template <int D>
__global__ __launch_bounds__(256) void chunk_attn_fwd_f32(KernelArgs a) {
  using G = GeoF32<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* ks = reinterpret_cast<float*>(smem);
  float* vt = reinterpret_cast<float*>(smem + G::kKBytes);

  const Item it = decode(a.plan, plan_slot_work(a.plan, blockIdx.x));
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 15;
  const int g = lane >> 4;

  const int pred = it.pred_rows;
  const int total = pred + it.own_rows;
  const int n_tiles = (total + kBN - 1) / kBN;
  const int64_t rs = a.row_stride;
  const int64_t e = a.entry(it.b);
  const float* qb = static_cast<const float*>(a.q) + e * a.q_bstride + (int64_t)it.h * D;
  const float* kown = static_cast<const float*>(a.k) + e * a.kv_bstride + (int64_t)it.h * D;
  const float* vown = static_cast<const float*>(a.v) + e * a.kv_bstride + (int64_t)it.h * D;
  const float* kpre = kown;
  const float* vpre = vown;
  if (pred > 0) {
    const int64_t pi = a.entry(it.b - a.pred_shift) * a.p_bstride + (int64_t)it.h * D;
    kpre = static_cast<const float*>(a.pk) + pi;
    vpre = static_cast<const float*>(a.pv) + pi;
  }

  // Q of this lane's query row: dims 16s + 4g .. +3 for every s
  const int qr = wave * 16 + j;  // row within the item
  const bool qvalid = qr < it.q_rows;
  f32x4f_t qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = qvalid ? *reinterpret_cast<const f32x4f_t*>(qb + (int64_t)(it.q0 + qr) * rs +
                                                        16 * s + 4 * g)
                   : f32x4f_t{0.f, 0.f, 0.f, 0.f};

  f32x4f_t oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4f_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_part = 0.f;  // this lane's keys only; summed over the row's lanes at the end
  const float s2 = a.scale_log2;

  constexpr int kVec = kBN * D / 4;  // float4s per K (or V) tile
  for (int t = 0; t < n_tiles; ++t) {
    // ---- tile t into LDS: K row-major, V transposed; rows past the key set
    // are zero (their scores are masked below)
    __syncthreads();  // the previous tile's reads are done
#pragma unroll
    for (int i = tid; i < kVec; i += 256) {
      const int row = i / (D / 4);
      const int c4 = i % (D / 4);
      const int kr = t * kBN + row;
      f32x4f_t kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
      if (kr < total) {
        const bool in_pred = kr < pred;
        const int64_t off = (int64_t)(in_pred ? kr : kr - pred) * rs + 4 * c4;
        kv = *reinterpret_cast<const f32x4f_t*>((in_pred ? kpre : kown) + off);
        vv = *reinterpret_cast<const f32x4f_t*>((in_pred ? vpre : vown) + off);
      }
      *reinterpret_cast<f32x4f_t*>(ks + row * G::kKStride + 4 * c4) = kv;
#pragma unroll
      for (int c = 0; c < 4; ++c) vt[(4 * c4 + c) * G::kVStride + row] = vv[c];
    }
    __syncthreads();

    // ---- S^T for the 4 key blocks of the tile
    f32x4f_t sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4f_t acc = {0.f, 0.f, 0.f, 0.f};
      const float* krow = ks + (16 * kb + j) * G::kKStride + 4 * g;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const f32x4f_t kf = *reinterpret_cast<const f32x4f_t*>(krow + 16 * s);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[i], qf[s][i], acc, 0, 0, 0);
      }
      sacc[kb] = acc;
    }

    // ---- softmax: scores of keys 16kb + 4g + r for query j, scaled to log2
    // units; keys past the set take no weight
    float tmax = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = t * kBN + 16 * kb + 4 * g + r;
        const float x = key < total ? sacc[kb][r] * s2 : -__builtin_inff();
        sacc[kb][r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);  // finite: every tile holds a valid key
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(sacc[kb][r] - m_new);
        sacc[kb][r] = p;
        psum += p;
      }
    l_part = l_part * alpha + psum;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;

    // ---- O^T += V^T . P^T
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const float* vrow = vt + (16 * db + j) * G::kVStride + 4 * g;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const f32x4f_t vf = *reinterpret_cast<const f32x4f_t*>(vrow + 16 * kb);
#pragma unroll
        for (int r = 0; r < 4; ++r)
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[r], sacc[kb][r], oacc[db], 0, 0, 0);
      }
    }
  }

  // ---- normalise and store: lane (j, g) holds dims 16db + 4g .. +3 of query j
  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot = l_tot + __shfl_xor(l_tot, 32);
  if (qvalid) {
    const float inv = 1.0f / l_tot;
    float* orow = static_cast<float*>(a.o) + e * a.o_bstride + (int64_t)(it.q0 + qr) * rs +
                  (int64_t)it.h * D + 4 * g;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<f32x4f_t*>(orow + 16 * db) = oacc[db] * inv;
  }
}

}  // namespace chunkattn
