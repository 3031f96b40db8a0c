// gfx950 chunk-attention forward kernel with 48 query rows per wave (384-row
// work items, 8 waves, two per SIMD), bf16 storage, head_dim 128.
//
// Same schedule as attn_pingpong.h (the two waves of a SIMD take turns between
// a matrix phase and a softmax phase, one workgroup barrier per phase, K/V
// tiles of 64 keys in four-slot LDS rings filled by LDS DMA, softmax without a
// maximum, a recheck pass for items that leave fp32's range), with the matrix
// work done as 16x16x32 bf16 MFMAs (v_mfma_f32_16x16x32_bf16) on three 16-row
// query blocks per wave.  Every K or V fragment a wave reads from LDS feeds
// three MFMAs instead of one, so a 64-key tile costs the CU the same LDS reads
// (256 KB: each of the 8 waves reads the whole K and V tile) for 384 query rows
// instead of 256, and the matrix phase (96 MFMAs, 1536 matrix-core cycles)
// outgrows the softmax phase, so the matrix core is the bound.
//
// Per tile and wave:
//   S^T = K . Q^T    A = K fragment (16 keys x 32 dims, one ds_read_b128),
//                    B = Q^T of one query block (32 dims x 16 queries, in
//                    registers for the whole item, pre-scaled by scale*log2 e);
//                    lane (j, g) = (lane & 15, lane >> 4) gets the scores of
//                    query j of the block for keys 16*kb + 4g + e, e = 0..3.
//   softmax          P = 2^S, rounded to bf16; l summed from the rounded P.
//   O^T += V^T . P^T  B = P^T for 32 keys: the lane's four keys of key block
//                    2s and its four of block 2s+1, packed as they come out of
//                    S^T (the contraction order of the keys is free, so the
//                    A operand uses the same order); A = V^T for 16 dims x those
//                    32 keys: two transposing reads (ds_read_b64_tr_b16) of
//                    four keys each.
// Both products accumulate in fp32.
//
// LDS layout of a tile: 64 rows x 256 bytes, row r at r*256.
//   K: 16-byte block b of row r stored at block b ^ (r & 15): the 16 lanes
//      that read one block of 16 consecutive keys hit 16 distinct blocks.
//   V: 32-byte unit u of row r stored at unit u ^ (r & 7): a transposing read
//      of 32 lanes covers 8 consecutive rows x 32 bytes of one unit, which then
//      lie in 8 distinct units.
#pragma once

#include <type_traits>

#include "attn_kernel.h"
#include "attn_pingpong.h"

namespace chunkattn {

constexpr int kWideRows = 48;            // query rows per wave
constexpr int kWideWaves = 8;
constexpr int kWideBlockRows = kWideRows * kWideWaves;  // 384 rows per work item

__device__ __forceinline__ int wide_kswz(int r) { return r & 15; }        // 16-byte blocks
__device__ __forceinline__ int wide_vswz(int r) { return 2 * (r & 7); }   // 16-byte blocks

__device__ __forceinline__ void pin(f32x4_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(u32x4_t& x) { asm volatile("" : "+v"(x)); }

// One work item of up to 384 rows (head_dim 128, bf16), with kQB 16-row query
// blocks per wave: wave w takes rows [16*kQB*w, 16*kQB*(w+1)) of the item.
// kQB = 3 covers 384 rows; an item with at most 256 (128) rows, the last
// query tile of a chunk, runs with kQB = 2 (1): its matrix phases shrink to
// 64 (32) MFMAs instead of padding the missing rows.  after_prologue() runs
// once in every thread, after the prologue's barrier.  A wave whose rows left
// fp32's range sets *range_flag (LDS); the caller marks the item.
template <int kQB, typename AfterPrologue>
__device__ __forceinline__ void attn_item_wide(const KernelArgs& a, const Item& it,
                                               unsigned char* smem, int* range_flag,
                                               AfterPrologue&& after_prologue) {
  using T = __bf16;
  constexpr int D = 128;
  using G = Geo<D>;
  constexpr int W = kWideWaves;
  constexpr int kCpw = G::kChunks / W;  // 1 KB load chunks per wave per tile (2)
  static_assert(kCpw == 2, "two 1 KB chunks per wave");
  static_assert(kQB >= 1 && kQB * 16 <= kWideRows, "query blocks per wave");
  constexpr int kRowsW = 16 * kQB;      // query rows per wave
  constexpr int kKS = D / 32;           // 32-dim steps of S (4)
  constexpr int kKB = kBN / 16;         // 16-key blocks of S (4)
  constexpr int kDB = D / 16;           // 16-dim blocks of O (8)
  constexpr int kPS = kBN / 32;         // 32-key steps of P.V (2)
  constexpr int kStepsPV = kPS * kDB;   // 16 V fragments
  constexpr int kStepsQK = kKB * kKS;   // 16 K fragments

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 15;
  const int g = lane >> 4;
  const bool group_b = wave >= 4;

  const int pred = it.pred_rows;
  const int total = pred + it.own_rows;
  const int n_tiles = (total + kBN - 1) / kBN;
  const int64_t rs = a.row_stride;

  const int64_t e = a.entry(it.b);
  const T* qb = static_cast<const T*>(a.q) + e * a.q_bstride + (int64_t)it.h * D;
  const T* kown = static_cast<const T*>(a.k) + e * a.kv_bstride + (int64_t)it.h * D;
  const T* vown = static_cast<const T*>(a.v) + e * a.kv_bstride + (int64_t)it.h * D;
  const T* kpre = kown;
  const T* vpre = vown;
  if (pred > 0) {
    const int64_t pi = a.entry(it.b - a.pred_shift) * a.p_bstride + (int64_t)it.h * D;
    kpre = static_cast<const T*>(a.pk) + pi;
    vpre = static_cast<const T*>(a.pv) + pi;
  }
  auto uniform_ptr = [](const T* p) __attribute__((always_inline)) {
    const uint64_t b = (uint64_t)(uintptr_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    return (const T*)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
  };
  kpre = uniform_ptr(kpre);
  vpre = uniform_ptr(vpre);
  kown = uniform_ptr(kown);
  vown = uniform_ptr(vown);
  // Tiles wholly inside one segment: [0, np) in the predecessor, [no, nf) in
  // the own chunk (tile t's first row at byte address base + t * tstride);
  // the straddling tile and a ragged last tile take the per-row path.
  const int np = pred / kBN;
  const int no = (pred + kBN - 1) / kBN;
  const int nf = total / kBN;
  const uint64_t tstride = (uint64_t)kBN * (uint64_t)rs * sizeof(T);
  const uint64_t pshift = (uint64_t)pred * (uint64_t)rs * sizeof(T);
  const uint64_t kpre_b = (uint64_t)(uintptr_t)kpre, vpre_b = (uint64_t)(uintptr_t)vpre;
  const uint64_t kown_s = (uint64_t)(uintptr_t)kown - pshift, vown_s = (uint64_t)(uintptr_t)vown - pshift;

  // ---- Q^T fragments: B operand of S^T = K.Q^T; lane (j, g) holds dims
  // 32*ks + 8g .. +7 of query row 16*qb + j of this wave's rows (loaded in
  // the prologue, after the first key/value loads are on their way)
  u32x4_t qf[kQB][kKS];
  auto load_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3) {
      const int r = wave * kRowsW + q3 * 16 + j;
      const bool valid = r < it.q_rows;
      const T* qrow = qb + (int64_t)(it.q0 + r) * rs + g * 8;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        qf[q3][ks] = valid ? Io<T>::load8(qrow + ks * 32) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  // scaled by scale * log2 e (nearest-even): S^T comes out in the log2 domain
  auto scale_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3)
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t x = qf[q3][ks][w];
          qf[q3][ks][w] = pack_bf16(__uint_as_float(x << 16) * a.scale_log2,
                                    __uint_as_float(x & 0xffff0000u) * a.scale_log2);
        }
  };

  // ---- per-lane DMA map: LDS chunk c = wave*2 + i of a tile receives tile
  // row 4c + g at physical block j (logical block j ^ swizzle(row))
  auto lrow = [&](int i) __attribute__((always_inline)) { return (wave * kCpw + i) * 4 + g; };
  uint32_t koffs[kCpw], voffs[kCpw];
#pragma unroll
  for (int i = 0; i < kCpw; ++i) {
    const int r = lrow(i);
    koffs[i] = (uint32_t)((r * rs + ((j ^ wide_kswz(r)) * 8)) * sizeof(T));
    voffs[i] = (uint32_t)((r * rs + ((j ^ wide_vswz(r)) * 8)) * sizeof(T));
  }
  auto load_one = [&](int t, unsigned char* dst, auto v_tag) __attribute__((always_inline)) {
    constexpr bool kV = decltype(v_tag)::value;
    const T* pre = kV ? vpre : kpre;
    const T* own = kV ? vown : kown;
    const int r0 = t * kBN;
    if (t < np || (t >= no && t < nf)) {
      const uint64_t b = (t < np ? (kV ? vpre_b : kpre_b) : (kV ? vown_s : kown_s)) +
                         (uint64_t)(uint32_t)t * tstride;
      const char* base = reinterpret_cast<const char*>((uintptr_t)b);
      load_lds16x2_async(base, kV ? voffs[0] : koffs[0], kV ? voffs[1] : koffs[1],
                         dst + wave * kCpw * 1024);
    } else {
      // straddling or ragged tile: rows past the end re-read the last row
#pragma unroll
      for (int i = 0; i < kCpw; ++i) {
        const int r = lrow(i);
        int jj = r0 + r;
        jj = jj < total ? jj : total - 1;
        const int blk = j ^ (kV ? wide_vswz(r) : wide_kswz(r));
        const T* src = jj < pred ? pre + (int64_t)jj * rs : own + (int64_t)(jj - pred) * rs;
        load_lds16_async(src + blk * 8, dst + (wave * kCpw + i) * 1024);
      }
    }
  };
  auto kslot = [&](int t) __attribute__((always_inline)) { return (uint32_t)(t & 3) * G::kTileBytes; };
  auto vslot = [&](int t) __attribute__((always_inline)) {
    return (uint32_t)(4 + (t & 3)) * G::kTileBytes;
  };
  // group t of loads: K(t) and V(t-1), whichever exist
  auto issue = [&](int t) __attribute__((always_inline)) {
    if (t < n_tiles) load_one(t, smem + kslot(t), std::false_type{});
    if (t >= 1 && t <= n_tiles) load_one(t - 1, smem + vslot(t - 1), std::true_type{});
  };
  auto group_loads = [&](int t) __attribute__((always_inline)) {
    return kCpw * ((t < n_tiles ? 1 : 0) + (t >= 1 && t <= n_tiles ? 1 : 0));
  };
  auto wait_left = [&](int left) __attribute__((always_inline)) {
    if (left <= 0)
      wait_vmem();
    else if (left <= kCpw)
      wait_vmem_le<kCpw>();
    else
      wait_vmem_le<2 * kCpw>();
  };

  // ---- per-lane LDS read offsets.  K fragment (kb, ks): row 16kb + j,
  // logical block 4ks + g (kb by immediate: the swizzle repeats every 16
  // rows).  V^T fragment (s, db): rows 32s + 4g + (j >> 2) and 16 further,
  // dims 16db + 4(j & 3) .. +3 (s and the second read by immediates).
  uint32_t koff_lds[kKS];
#pragma unroll
  for (int ks = 0; ks < kKS; ++ks)
    koff_lds[ks] = (uint32_t)(j * G::kRowBytes + (((4 * ks + g) ^ wide_kswz(j)) << 4));
  uint32_t voff_lds[kDB];
  {
    const int r = 4 * g + (j >> 2);
#pragma unroll
    for (int db = 0; db < kDB; ++db)
      voff_lds[db] = (uint32_t)(r * G::kRowBytes + ((db ^ (r & 7)) << 5) + 8 * (j & 3));
  }

  f32x4_t oacc[kQB][kDB];
#pragma unroll
  for (int q3 = 0; q3 < kQB; ++q3)
#pragma unroll
    for (int db = 0; db < kDB; ++db) oacc[q3][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t sacc[kQB][kKB];  // S^T of the current tile
  u32x4_t pk[kQB][kPS];    // P^T of the previous tile, B operands of P.V
  // l per query block: this lane's keys, two partial sums each, from the
  // rounded numerators (one dot2 against (1, 1) per pair)
  float lsum[kQB][2];
#pragma unroll
  for (int q3 = 0; q3 < kQB; ++q3) lsum[q3][0] = lsum[q3][1] = 0.f;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  auto rk = [&](uint32_t k_at, int i) __attribute__((always_inline)) {
    // QK step i: key block i / kKS, dim step i % kKS
    const CA_LDS unsigned char* kl = (const CA_LDS unsigned char*)smem + k_at;
    return *(CA_LDS const u32x4_t*)(kl + koff_lds[i % kKS] + (i / kKS) * 16 * G::kRowBytes);
  };
  auto rv = [&](uint32_t v_at, int i) __attribute__((always_inline)) {
    // PV step i: key step i / kDB, dim block i % kDB
    const CA_LDS unsigned char* vl = (const CA_LDS unsigned char*)smem + v_at;
    const uint32_t base = voff_lds[i % kDB] + (uint32_t)((i / kDB) * 32 * G::kRowBytes);
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CA_LDS i16x4_t*)(vl + base));
    const i16x4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((CA_LDS i16x4_t*)(vl + base + 16 * G::kRowBytes));
    const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
    const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
  };

  // Matrix phase: P.V of the previous tile (kPV; V at v_at), then S of the
  // current one (kQK; K at k_at), as one stream of fragment steps (V steps
  // first, so the P^T registers are free before the S^T accumulators fill).
  // LDS reads run two steps ahead; with kPf the first two fragments are
  // already in fr (read in the softmax phase before).
  u32x4_t fr[3];
  auto matrix_phase = [&](uint32_t k_at, uint32_t v_at, auto pv_tag, auto qk_tag, auto pf_tag)
      __attribute__((always_inline)) {
    constexpr bool kPV = decltype(pv_tag)::value;
    constexpr bool kQK = decltype(qk_tag)::value;
    constexpr bool kPf = decltype(pf_tag)::value;
    constexpr int i0 = kPV ? 0 : kStepsPV;
    constexpr int i1 = kQK ? kStepsPV + kStepsQK : kStepsPV;
    auto read = [&](int i) __attribute__((always_inline)) {
      return i < kStepsPV ? rv(v_at, i) : rk(k_at, i - kStepsPV);
    };
    if constexpr (!kPf) {
      fr[0] = read(i0);
      fr[1] = read(i0 + 1);
    }
#pragma unroll
    for (int i = i0; i < i1; ++i) {
      if (i + 2 < i1) fr[(i - i0 + 2) % 3] = read(i + 2);
      const u32x4_t f = fr[(i - i0) % 3];
      if (i < kStepsPV) {
        const int s = i / kDB, db = i % kDB;
#pragma unroll
        for (int q3 = 0; q3 < kQB; ++q3)
          oacc[q3][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, f), __builtin_bit_cast(bf16x8_t, pk[q3][s]),
              oacc[q3][db], 0, 0, 0);
      } else {
        const int kb = (i - kStepsPV) / kKS, ks = (i - kStepsPV) % kKS;
#pragma unroll
        for (int q3 = 0; q3 < kQB; ++q3)
          sacc[q3][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, f), __builtin_bit_cast(bf16x8_t, qf[q3][ks]),
              ks == 0 ? f32x4_t{0.f, 0.f, 0.f, 0.f} : sacc[q3][kb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax phase of tile t: numerators 2^S into pk and l (with a mask, keys
  // >= total get P = 0; they re-read the last key row, so their scores are
  // finite).
  auto softmax_phase = [&](int t, auto mask_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float p0 = __builtin_amdgcn_exp2f(sacc[q3][kb][2 * h2]);
          float p1 = __builtin_amdgcn_exp2f(sacc[q3][kb][2 * h2 + 1]);
          if constexpr (decltype(mask_tag)::value) {
            const int key0 = t * kBN + kb * 16 + 4 * g + 2 * h2;
            if (key0 >= total) p0 = 0.f;
            if (key0 + 1 >= total) p1 = 0.f;
          }
          const uint32_t w = pack_bf16(p0, p1);
          pk[q3][kb >> 1][(kb & 1) * 2 + h2] = w;
          lsum[q3][h2] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one2,
                                                         lsum[q3][h2], false);
        }
  };

  auto end_matrix = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) pin(sacc[q3][kb]);
    wg_barrier();
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) pin(sacc[q3][kb]);
  };
  auto end_softmax = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3) {
      pin(pk[q3][0]);
      pin(pk[q3][1]);
      asm volatile("" : "+v"(lsum[q3][0]), "+v"(lsum[q3][1]));
    }
    wg_barrier();
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3) {
      pin(pk[q3][0]);
      pin(pk[q3][1]);
    }
  };

  auto step = [&](int t, auto first_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_tag)::value;
    __builtin_amdgcn_s_setprio(3);
    matrix_phase(kslot(t), vslot(t - 1), std::integral_constant<bool, !kFirst>{}, std::true_type{},
                 std::integral_constant<bool, !kFirst>{});
    __builtin_amdgcn_s_setprio(0);
    wait_left(group_loads(t + 2));
    end_matrix();
    softmax_phase(t, mask_tag);
    issue(t + 3);
    // The next matrix phase's first two fragments: rows 0-31 of V(t), which
    // waves 0-3 load; they waited for them at the end of their matrix phase
    // of tile t, and the barrier after it made them visible.
    fr[0] = rv(vslot(t), 0);
    fr[1] = rv(vslot(t), 1);
    end_softmax();
  };

  // ---- prologue: the first three groups of key/value loads and the Q
  // loads go out together (one memory latency for all), then Q is scaled
  load_one(0, smem + kslot(0), std::false_type{});
  issue(1);
  issue(2);
  load_q();
  wait_vmem();
  scale_q();
  wg_barrier();
  after_prologue();
  if (group_b) wg_barrier();  // group B runs one phase behind group A

  if (n_tiles == 1) {
    step(0, std::true_type{}, Mask{});
  } else {
    step(0, std::true_type{}, NoMask{});
    for (int t = 1; t + 1 < n_tiles; ++t) step(t, std::false_type{}, NoMask{});
    step(n_tiles - 1, std::false_type{}, Mask{});
  }
  matrix_phase(0u, vslot(n_tiles - 1), std::true_type{}, std::false_type{}, std::true_type{});
  if (!group_b) wg_barrier();  // matches group B's first barrier

  // ---- epilogue: l over the four lane groups (keys 4g + e), range check over
  // the workgroup, normalise and store
  float l_tot[kQB];
  float acc = 0.f;
#pragma unroll
  for (int q3 = 0; q3 < kQB; ++q3) {
    float x = lsum[q3][0] + lsum[q3][1];
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    l_tot[q3] = x;
    acc += x;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
      acc += (oacc[q3][db][0] + oacc[q3][db][1]) + (oacc[q3][db][2] + oacc[q3][db][3]);
  }
  bool bad = !__builtin_isfinite(acc);
#pragma unroll
  for (int q3 = 0; q3 < kQB; ++q3) bad = bad || !(l_tot[q3] >= 0x1p-64f);
  // the range check folds into the workgroup's flag; after the barrier that
  // ends the item, thread 0 marks the item for the recheck pass if it is set
  if (__ballot(bad) != 0 && lane == 0) *range_flag = 1;
  T* ob = static_cast<T*>(a.o) + e * a.o_bstride + (int64_t)it.h * D;
#pragma unroll
  for (int q3 = 0; q3 < kQB; ++q3) {
    const int r = wave * kRowsW + q3 * 16 + j;
    if (r < it.q_rows) {
      const float inv = 1.0f / l_tot[q3];
      T* orow = ob + (int64_t)(it.q0 + r) * rs + 4 * g;
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        Io<T>::store4(orow + 16 * db, oacc[q3][db][0] * inv, oacc[q3][db][1] * inv,
                      oacc[q3][db][2] * inv, oacc[q3][db][3] * inv);
    }
  }
}

// Main pass with 384-row work items, persistent over the die work queues
// exactly as chunk_attn_fwd_pingpong (the claim words a.queue[0 .. n_xcd) are
// zero at launch).
__global__ __launch_bounds__(512, 1) void chunk_attn_fwd_wide(KernelArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ long long next_item;  // >= 0 item, -1 none left, -2 claim again
  __shared__ int used_up;          // thread 0: dies (from our own on) found empty
  __shared__ int range_flag;       // some row of the current item left fp32's range
  const int nx = a.plan.n_xcd;
  const int die = (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) % (unsigned)nx);
  auto die_at = [&](int k) __attribute__((always_inline)) {
    return die + k < nx ? die + k : die + k - nx;
  };
  auto claim_sync = [&]() __attribute__((always_inline)) {
    int k = used_up;
    long long w = -1;
    for (; k < nx; ++k) {
      const unsigned long long old = atomicAdd(&a.queue[die_at(k)], 1ull);
      w = claim_word_item(a.plan, die_at(k), old);
      if (w >= 0) break;
    }
    used_up = k;
    next_item = w;
  };
  if (threadIdx.x == 0) {
    used_up = 0;
    range_flag = 0;
    claim_sync();
  }
  __syncthreads();
  long long w = next_item;
  while (w >= 0) {
    unsigned long long ticket = 0;
    int k = nx;
    if (threadIdx.x == 0) {
      k = used_up;
      if (k < nx) ticket = atomicAdd(&a.queue[die_at(k)], 1ull);
    }
    auto after_prologue = [&]() __attribute__((always_inline)) {
      if (threadIdx.x == 0) {
        long long nw = -1;
        if (k < nx) {
          nw = claim_word_item(a.plan, die_at(k), ticket);
          if (nw < 0) nw = -2;
        }
        next_item = nw;
      }
    };
    const Item it = decode(a.plan, w);
    if (it.q_rows > 2 * 16 * kWideWaves)
      attn_item_wide<3>(a, it, smem, &range_flag, after_prologue);
    else if (it.q_rows > 16 * kWideWaves)
      attn_item_wide<2>(a, it, smem, &range_flag, after_prologue);
    else
      attn_item_wide<1>(a, it, smem, &range_flag, after_prologue);
    wg_barrier();
    if (threadIdx.x == 0 && range_flag != 0) {
      // the marker follows thread 0's own store of that element
      static_cast<__bf16*>(a.o)[a.entry(it.b) * a.o_bstride + (int64_t)it.q0 * a.row_stride +
                                (int64_t)it.h * 128] = overflow_marker<__bf16>();
      range_flag = 0;
    }
    w = next_item;
    if (w == -2) {
      wg_barrier();  // every wave has read next_item before thread 0 rewrites it
      if (threadIdx.x == 0) {
        used_up = used_up + 1;
        claim_sync();
      }
      wg_barrier();
      w = next_item;
    }
  }
}

// Recheck of 384-row items: the item's first output element carries the
// overflow marker if the main pass left fp32's range; the item is then
// recomputed as three 128-row items on the running-maximum schedule.
template <int W>
__global__ __launch_bounds__(W * 64, 8 / W) void chunk_attn_recheck_wide(KernelArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const Item it = decode(a.plan, plan_slot_work(a.plan, blockIdx.x));
  const __bf16 first = static_cast<const __bf16*>(a.o)[a.entry(it.b) * a.o_bstride +
                                                      (int64_t)it.q0 * a.row_stride +
                                                      (int64_t)it.h * 128];
  if (!__builtin_isnan((float)first)) return;
  for (int sub = 0; sub * 32 * W < it.q_rows; ++sub) {
    Item s = it;
    s.q0 = it.q0 + sub * 32 * W;
    const int left = it.q_rows - sub * 32 * W;
    s.q_rows = left < 32 * W ? left : 32 * W;
    attn_item_sync<128, __bf16, W, false>(a, s, smem);
    __syncthreads();
  }
}

}  // namespace chunkattn
