// gfx950 chunk-attention forward kernel.
//
// One workgroup (4 waves, 256 lanes) computes BM = 128 query rows of one
// (chunk, head): each wave owns 32 query rows.  Key/value rows are walked in
// tiles of BN = 64 logical rows; a tile may straddle the predecessor/own
// boundary, each row picking its source as it is loaded (no concatenation).
//
// Per tile and wave, on bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulate):
//   S^T = K . Q^T      keys on the M side, queries on N; each lane ends up
//                      holding 32 scores of ONE query row (its column), so the
//                      softmax statistics of a row live in one lane pair.
//   online softmax     running max m and sum l per query row, exp2 with
//                      scale*log2(e) folded in; P rounded to bf16 once.
//   O^T += V^T . P^T   P^T comes straight out of the S^T accumulators as the
//                      B operand; V^T is read from an LDS copy stored
//                      transposed.  O^T is again one query row per lane column,
//                      so the rescale by exp(m_old - m_new) is a per-lane scalar.
//
// Data movement.  K and V tiles go global -> registers (128-bit loads, issued
// one tile ahead) -> LDS (double buffered, one barrier per tile).  K is kept
// row-major with a 16-byte-block XOR swizzle; V is transposed in registers
// (4 keys x 8 dims per lane) and stored as V^T rows of 64 keys with a key
// order matching the lanes' score layout, also XOR-swizzled.  Q stays in
// registers for the whole walk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace chunkattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // key/value rows per tile

struct KernelArgs {
  Plan plan;
  const void* q;
  const void* k;      // own K: entry b at k + b*kv_bstride
  const void* v;
  const void* pk;     // predecessor K: entry b at pk + (b - pred_shift)*p_bstride
  const void* pv;
  void* o;
  int64_t q_bstride;  // elements between batch entries of q and out
  int64_t kv_bstride;
  int64_t p_bstride;
  int pred_shift;
  int row_stride;     // heads * head_dim
  float scale_log2;   // scale * log2(e)
};

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t p = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32, nearest-even
  return __builtin_bit_cast(uint32_t, p);
}

template <typename T>
struct Io;

template <>
struct Io<__bf16> {
  static __device__ __forceinline__ u32x4_t load8(const __bf16* p) {
    return *reinterpret_cast<const u32x4_t*>(p);
  }
  static __device__ __forceinline__ void store4(__bf16* p, float a, float b, float c, float d) {
    u32x2_t w = {pack_bf16(a, b), pack_bf16(c, d)};
    *reinterpret_cast<u32x2_t*>(p) = w;
  }
};

template <>
struct Io<float> {
  static __device__ __forceinline__ u32x4_t load8(const float* p) {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(p)[0];
    const f32x4_t b = reinterpret_cast<const f32x4_t*>(p)[1];
    u32x4_t r = {pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]), pack_bf16(b[0], b[1]),
                 pack_bf16(b[2], b[3])};
    return r;
  }
  static __device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    f32x4_t w = {a, b, c, d};
    *reinterpret_cast<f32x4_t*>(p) = w;
  }
};

// ---- LDS addressing -------------------------------------------------------
// K tile: kBN rows of D bf16 (D/8 blocks of 16 bytes), block index XOR (row & 7).
template <int D>
__device__ __forceinline__ uint32_t k_lds_off(int row, int blk) {
  return (uint32_t)(row * (D * 2) + ((blk ^ (row & 7)) << 4));
}
// V^T tile: D rows of kBN = 64 keys (8 blocks of 16 bytes).  Within each group
// of 16 keys the stored order is [0-3, 8-11, 4-7, 12-15] so that a lane half
// finds the 8 keys it multiplies in one block; blocks XOR-swizzled by row.
__device__ __forceinline__ int vt_swz(int d) { return (d + (d >> 3)) & 7; }
__device__ __forceinline__ uint32_t vt_lds_off(int d, int blk) {
  return (uint32_t)(d * (kBN * 2) + ((blk ^ vt_swz(d)) << 4));
}

template <int D>
struct Tile {
  static constexpr int kDch = D / 8;                    // 16-byte chunks per row
  static constexpr int kKRowsPerPass = kThreads / kDch;  // rows one pass loads
  static constexpr int kKPasses = kBN / kKRowsPerPass;
  static constexpr int kVBlocks = (kBN / 4) * kDch;      // 4 keys x 8 dims each
  static constexpr uint32_t kKBytes = kBN * D * 2;
  static constexpr uint32_t kVBytes = D * kBN * 2;
  static constexpr uint32_t kBufBytes = kKBytes + kVBytes;
  static_assert(kKRowsPerPass * kKPasses == kBN, "K tile split");
  static_assert(kVBlocks <= kThreads, "V tile split");
};

template <int D, typename T>
__global__ __launch_bounds__(kThreads, 2) void chunk_attn_fwd(KernelArgs a) {
  using TL = Tile<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;  // lane half

  const int64_t w = slot_to_work(blockIdx.x, a.plan.n_items, a.plan.n_xcd);
  const Item it = decode(a.plan, w);
  const int total = it.pred_rows + it.own_rows;
  const int n_tiles = (total + kBN - 1) / kBN;

  const T* qb = static_cast<const T*>(a.q) + it.b * a.q_bstride + (int64_t)it.h * D;
  const T* kown = static_cast<const T*>(a.k) + it.b * a.kv_bstride + (int64_t)it.h * D;
  const T* vown = static_cast<const T*>(a.v) + it.b * a.kv_bstride + (int64_t)it.h * D;
  const T* kpre = kown;
  const T* vpre = vown;
  if (it.pred_rows > 0) {
    const int64_t pi = (int64_t)(it.b - a.pred_shift) * a.p_bstride + (int64_t)it.h * D;
    kpre = static_cast<const T*>(a.pk) + pi;
    vpre = static_cast<const T*>(a.pv) + pi;
  }
  const int64_t rs = a.row_stride;

  // ---- Q fragment: B operand of S^T = K.Q^T, one query row per lane column
  const int qrow = it.q0 + wave * 32 + l32;
  const bool qvalid = qrow < a.plan.lq;
  u32x4_t qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (qvalid)
      qf[ks] = Io<T>::load8(qb + qrow * rs + ks * 16 + hh * 8);
    else
      qf[ks] = u32x4_t{0u, 0u, 0u, 0u};
  }

  // ---- per-thread load assignment for one K/V tile
  const int k_row0 = tid / TL::kDch;
  const int k_blk = tid % TL::kDch;
  int v_dc = 0, v_kg = 0;
  const bool v_loader = tid < TL::kVBlocks;
  {
    const int l16 = tid & 15, grp = tid >> 4;
    int bi;
    if (TL::kDch == 16) {
      v_dc = (l16 & 7) + 8 * (grp & 1);
      bi = grp >> 1;
    } else {
      v_dc = l16 & 7;
      bi = grp;
    }
    v_kg = ((bi >> 1) << 2) + (bi & 1) + 2 * (l16 >> 3);
  }

  u32x4_t kreg[TL::kKPasses];
  u32x4_t vreg[4];

  auto row_ptr = [&](const T* pre, const T* own, int j) -> const T* {
    return j < it.pred_rows ? pre + j * rs : own + (j - it.pred_rows) * rs;
  };

  auto load_tile = [&](int t) {
    const int base = t * kBN;
#pragma unroll
    for (int i = 0; i < TL::kKPasses; ++i) {
      const int j = base + k_row0 + i * TL::kKRowsPerPass;
      if (j < total)
        kreg[i] = Io<T>::load8(row_ptr(kpre, kown, j) + k_blk * 8);
      else
        kreg[i] = u32x4_t{0u, 0u, 0u, 0u};
    }
    if (v_loader) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = base + v_kg * 4 + i;
        if (j < total)
          vreg[i] = Io<T>::load8(row_ptr(vpre, vown, j) + v_dc * 8);
        else
          vreg[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  };

  auto store_tile = [&](int buf) {
    unsigned char* kb = smem + buf * TL::kBufBytes;
    unsigned char* vb = kb + TL::kKBytes;
#pragma unroll
    for (int i = 0; i < TL::kKPasses; ++i) {
      const int r = k_row0 + i * TL::kKRowsPerPass;
      *reinterpret_cast<u32x4_t*>(kb + k_lds_off<D>(r, k_blk)) = kreg[i];
    }
    if (v_loader) {
      // 4 keys x 8 dims -> for each dim, the 4 keys as two packed pairs
      const int blk = 2 * (v_kg >> 2) + (v_kg & 1);
      const int half = (v_kg & 3) >> 1;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t e0 = vreg[0][m], e1 = vreg[1][m], e2 = vreg[2][m], e3 = vreg[3][m];
        const u32x2_t even = {(e0 & 0xffffu) | (e1 << 16), (e2 & 0xffffu) | (e3 << 16)};
        const u32x2_t odd = {(e0 >> 16) | (e1 & 0xffff0000u), (e2 >> 16) | (e3 & 0xffff0000u)};
        const int d0 = v_dc * 8 + 2 * m;
        *reinterpret_cast<u32x2_t*>(vb + vt_lds_off(d0, blk) + half * 8) = even;
        *reinterpret_cast<u32x2_t*>(vb + vt_lds_off(d0 + 1, blk) + half * 8) = odd;
      }
    }
  };

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -__builtin_inff();
  float l_run = 0.f;
  const float s2 = a.scale_log2;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const bool has_next = t + 1 < n_tiles;
    if (has_next) load_tile(t + 1);

    const unsigned char* kb = smem + (t & 1) * TL::kBufBytes;
    const unsigned char* vb = kb + TL::kKBytes;

    // S^T = K . Q^T for two blocks of 32 keys
    f32x16_t sacc[kBN / 32];
#pragma unroll
    for (int kb2 = 0; kb2 < kBN / 32; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb2][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int kb2 = 0; kb2 < kBN / 32; ++kb2) {
        const u32x4_t kv =
            *reinterpret_cast<const u32x4_t*>(kb + k_lds_off<D>(kb2 * 32 + l32, 2 * ks + hh));
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, kv), __builtin_bit_cast(bf16x8_t, qf[ks]), sacc[kb2],
            0, 0, 0);
      }
    }

    // keys past the end of R_c (last tile only) take no part
    const bool ragged = (t + 1) * kBN > total;
    if (ragged) {
#pragma unroll
      for (int kb2 = 0; kb2 < kBN / 32; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t * kBN + kb2 * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= total) sacc[kb2][i] = -__builtin_inff();
        }
    }

    // online softmax for this lane's query row
    float mx = sacc[0][0];
#pragma unroll
    for (int kb2 = 0; kb2 < kBN / 32; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb2][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    // first tile: nothing to rescale (also keeps scale = 0 free of inf*0)
    const float alpha =
        m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * s2);
    m_run = m_new;
    const float msc = m_new * s2;

    uint32_t pk[kBN / 32][8];
    float psum = 0.f;
#pragma unroll
    for (int kb2 = 0; kb2 < kBN / 32; ++kb2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][2 * i], s2, -msc));
        float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][2 * i + 1], s2, -msc));
        if (ragged) {
          const int key0 = t * kBN + kb2 * 32 + 8 * ((2 * i) >> 2) + 4 * hh + ((2 * i) & 3);
          if (key0 >= total) p0 = 0.f;
          if (key0 + 1 >= total) p1 = 0.f;
        }
        pk[kb2][i] = pack_bf16(p0, p1);
        psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[kb2][i]),
                                               bf16x2_t{(__bf16)1.0f, (__bf16)1.0f}, psum,
                                               false);
      }
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // O^T += V^T . P^T, 16 keys per step
#pragma unroll
    for (int s = 0; s < kBN / 16; ++s) {
      const u32x4_t pb = {pk[s >> 1][(s & 1) * 4 + 0], pk[s >> 1][(s & 1) * 4 + 1],
                          pk[s >> 1][(s & 1) * 4 + 2], pk[s >> 1][(s & 1) * 4 + 3]};
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x4_t vv =
            *reinterpret_cast<const u32x4_t*>(vb + vt_lds_off(db * 32 + l32, 2 * s + hh));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv),
                                                           __builtin_bit_cast(bf16x8_t, pb),
                                                           oacc[db], 0, 0, 0);
      }
    }

    if (has_next) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: normalise and store this lane's query row
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    T* ob = static_cast<T*>(a.o) + it.b * a.q_bstride + (int64_t)qrow * rs + (int64_t)it.h * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hh;
        Io<T>::store4(ob + d0, oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                      oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      }
  }
}

// Writes the decoded work item of every workgroup slot (7 ints each), using
// the same slot_to_work/decode as the attention kernel.
__global__ void plan_dump(Plan p, int* out, int64_t cap) {
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= p.n_items || slot >= cap) return;
  const Item it = decode(p, slot_to_work(slot, p.n_items, p.n_xcd));
  int* r = out + slot * 7;
  r[0] = it.b;
  r[1] = it.h;
  r[2] = it.q0;
  r[3] = it.q_rows;
  r[4] = it.pred_rows > 0 ? it.b - 1 : -1;
  r[5] = it.pred_rows;
  r[6] = it.own_rows;
}

}  // namespace chunkattn
