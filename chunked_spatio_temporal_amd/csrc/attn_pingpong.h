// gfx950 chunk-attention forward kernel, ping-pong schedule (256-row work
// items, 8 waves of 32 query rows, two waves per SIMD).
//
// A SIMD issues matrix instructions from one wave while it issues vector-ALU
// instructions from another, but inside one wave the in-order issue lets a
// softmax dependency chain hold up the next MFMA.  So the two waves that share
// a SIMD take turns: in every phase one of them does only matrix work (P.V of
// the previous key tile and S = K.Q^T of the current one) and the other only
// the softmax of the tile whose scores it just computed.  Waves 0-3 (group A)
// and waves 4-7 (group B) sit on SIMDs 0-3 once each, so group A runs matrix
// phases while group B runs softmax phases and the other way round; one
// workgroup barrier ends every phase.
//
//   phase:     0      1      2      3      4   ...  2n     2n+1
//   group A:  S(0)   sm(0)  PV(0)  sm(1)  PV(1) ... PV(n-1)  -
//                           S(1)          S(2)
//   group B:   -     S(0)   sm(0)  PV(0)  sm(1) ...  sm(n-1) PV(n-1)
//                                  S(1)
//
// The wave in its matrix phase runs at the higher wave priority (s_setprio):
// the two waves of a SIMD compete for instruction issue, and without it the
// older wave's softmax slows the younger wave's matrix phase by a fifth.
//
// Softmax without a maximum: Q is multiplied by scale * log2 e and rounded to
// bf16 once per work item, so the matrix core returns the scores in the log2
// domain and P = 2^S needs no subtraction.  softmax(S) is unchanged by leaving
// the maximum out; only the range of fp32 is at stake, and a work item whose
// l or O is not finite, or whose l is below 2^-64, writes the overflow marker
// and is redone exactly by chunk_attn_recheck (running maximum).  A score pair
// costs the softmax wave two exponentials, one pack and one dot2 into l, which
// sums the rounded numerators: the weights of a row sum to one exactly, so a
// row with one dominant key returns its value.  (l summed by the matrix core
// instead, with an all-ones operand, takes four more MFMAs per tile from the
// matrix phase; fp32 adds of the unrounded numerators leave a dominant key's
// weight off by its bf16 rounding.)
//
// The K/V tiles go global -> LDS by LDS DMA written as inline asm
// (load_lds16_async): each wave waits for its own loads with vmcnt.
//
// LDS: rings of four K slots and four V slots (tile t in slot t mod 4).  The
// loads of "group" g = {K(g), V(g-1)} (the tiles the matrix phase of tile g
// reads for the first time) start in the softmax phase of tile g-3, three
// phases or more before any wave reads them; each wave waits for its own
// loads of group t+1 at the end of its matrix phase of tile t, and the
// barrier that ends global phase 2t+1 publishes them.  A slot is reloaded
// only after both groups have finished reading it (K(g) replaces K(g-4),
// V(g-1) replaces V(g-5)).  Both groups run the same code: group B starts one
// phase later (an extra barrier first) and group A ends with one.
#pragma once

#include <type_traits>

#include "attn_kernel.h"

namespace chunkattn {

// Two 1 KB LDS DMA chunks into consecutive LDS kilobytes, from one
// wave-uniform base in scalar registers plus per-lane byte offsets: one M0
// save and restore for both.  The first load waits as load_lds16_async does
// (the base may have been written by a vector instruction just before); the
// second needs only the one wait state an M0 write takes before an LDS DMA.
__device__ __forceinline__ void load_lds16x2_async(const void* sbase, uint32_t voff0,
                                                   uint32_t voff1, void* lds_chunk) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = (uint32_t)(uintptr_t)(CA_LDS void*)lds_chunk;
  const uint64_t sb = (uint64_t)(uintptr_t)sbase;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "s_add_i32 m0, m0, 0x400\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff0), "v"(voff1), "s"(sb), "s"(m0)
      : "memory");
#endif
}


// Eight 64-row tiles: K slots 0..3, then V slots 0..3.
template <int D>
constexpr uint32_t kPingPongLdsBytes = 8 * Geo<D>::kTileBytes;

// Empty asm statements that "modify" a value: they are ordered with the
// workgroup barrier (both have side effects), so a value pinned on both sides
// of a barrier is computed before it and only used after it.  The optimiser
// would otherwise move the arithmetic of a phase across the barrier into the
// other phase.
__device__ __forceinline__ void pin(f32x16_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(uint32_t (&p)[8]) {
  asm volatile("" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]));
  asm volatile("" : "+v"(p[4]), "+v"(p[5]), "+v"(p[6]), "+v"(p[7]));
}
__device__ __forceinline__ void pin(float (&l)[4]) {
  asm volatile("" : "+v"(l[0]), "+v"(l[1]), "+v"(l[2]), "+v"(l[3]));
}

// after_prologue() runs once in every thread, after the prologue's barrier
// (every wave has started the item by then).
template <int D, typename T, typename AfterPrologue>
__device__ __forceinline__ void attn_item_pingpong(const KernelArgs& a, const Item& it,
                                                   unsigned char* smem,
                                                   AfterPrologue&& after_prologue) {
  using G = Geo<D>;
  constexpr int W = 8;
  constexpr int kCpw = G::kChunks / W;  // 1 KB load chunks per wave per matrix
  static_assert(kCpw >= 1 && kCpw * W == G::kChunks, "tile split across waves");
  static_assert(sizeof(T) == 2, "bf16 storage (fp32 calls run attn_f32.h)");
  constexpr int kKs = D / 16;
  constexpr int kDb = D / 32;
  constexpr int kStepsQK = 2 * kKs;              // 2 key blocks x k-steps
  constexpr int kStepsPV = (kBN / 16) * kDb;     // 16-key steps x d-blocks
  constexpr int kSteps = kStepsQK > kStepsPV ? kStepsQK : kStepsPV;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
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
  // the four segment bases are wave-uniform: keep them in scalar registers
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
  // the own chunk; the straddling tile and a ragged last tile take the
  // per-row path.  Tile t's first row is at byte address base + t * tstride,
  // with base the predecessor's start or, for own-chunk tiles, the own
  // chunk's start minus pred rows (an integer, only ever offset forward into
  // the own chunk).  Precomputed here, the per-tile address is one select and
  // one multiply-add in scalar registers.
  const int np = pred / kBN;
  const int no = (pred + kBN - 1) / kBN;
  const int nf = total / kBN;
  const uint64_t tstride = (uint64_t)kBN * (uint64_t)rs * sizeof(T);
  const uint64_t pshift = (uint64_t)pred * (uint64_t)rs * sizeof(T);
  const uint64_t kpre_b = (uint64_t)(uintptr_t)kpre, vpre_b = (uint64_t)(uintptr_t)vpre;
  const uint64_t kown_s = (uint64_t)(uintptr_t)kown - pshift, vown_s = (uint64_t)(uintptr_t)vown - pshift;

  // ---- Q fragment: B operand of S^T = K.Q^T, one query row per lane column
  const int qrow = it.q0 + wave * 32 + l32;
  const bool qvalid = wave * 32 + l32 < it.q_rows;
  u32x4_t qf[kKs];
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks)
    qf[ks] = qvalid ? Io<T>::load8(qb + (int64_t)qrow * rs + ks * 16 + hh * 8)
                    : u32x4_t{0u, 0u, 0u, 0u};
  // scaled by scale * log2 e (nearest-even), so S^T comes out in the log2
  // domain
#pragma unroll
  for (int ks = 0; ks < kKs; ++ks)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = qf[ks][w];
      qf[ks][w] = pack_bf16(__uint_as_float(x << 16) * a.scale_log2,
                            __uint_as_float(x & 0xffff0000u) * a.scale_log2);
    }

  // ---- per-lane global load map: LDS chunk c = wave*kCpw + i of a tile
  // receives tile row c*kRowsPerKB + lane/kBlk, physical block lane%kBlk
  auto lrow = [&](int i) __attribute__((always_inline)) {
    return (wave * kCpw + i) * G::kRowsPerKB + lane / G::kBlk;
  };
  uint32_t koffs[kCpw], voffs[kCpw];
#pragma unroll
  for (int i = 0; i < kCpw; ++i) {
    const int r = lrow(i);
    const int pb = lane % G::kBlk;
    koffs[i] = (uint32_t)((r * rs + ((pb ^ k_swz<D>(r)) * 8)) * sizeof(T));
    voffs[i] = (uint32_t)((r * rs + ((pb ^ v_swz<D>(r)) * 8)) * sizeof(T));
  }
  // This wave's share of rows [t*kBN, (t+1)*kBN) of K (kV false) or V into
  // the LDS tile at dst.
  auto load_one = [&](int t, unsigned char* dst, auto v_tag) __attribute__((always_inline)) {
    constexpr bool kV = decltype(v_tag)::value;
    const T* pre = kV ? vpre : kpre;
    const T* own = kV ? vown : kown;
    const int r0 = t * kBN;
    if (t < np || (t >= no && t < nf)) {
      const uint64_t b = (t < np ? (kV ? vpre_b : kpre_b) : (kV ? vown_s : kown_s)) +
                         (uint64_t)(uint32_t)t * tstride;
      const char* base = reinterpret_cast<const char*>((uintptr_t)b);
      if constexpr (kCpw == 2) {
        load_lds16x2_async(base, kV ? voffs[0] : koffs[0], kV ? voffs[1] : koffs[1],
                           dst + wave * kCpw * 1024);
      } else {
#pragma unroll
        for (int i = 0; i < kCpw; ++i)
          load_lds16_async(base, kV ? voffs[i] : koffs[i], dst + (wave * kCpw + i) * 1024);
      }
    } else {
      // straddling or ragged tile: rows past the end re-read the last row
#pragma unroll
      for (int i = 0; i < kCpw; ++i) {
        const int r = lrow(i);
        int j = r0 + r;
        j = j < total ? j : total - 1;
        const int blk = (lane % G::kBlk) ^ (kV ? v_swz<D>(r) : k_swz<D>(r));
        const T* src = j < pred ? pre + (int64_t)j * rs : own + (int64_t)(j - pred) * rs;
        load_lds16_async(src + blk * 8, dst + (wave * kCpw + i) * 1024);
      }
    }
  };
  // ring slot byte offsets; tile g of K in slot g & 3, of V in slot 4 + (g & 3)
  auto kslot = [&](int g) __attribute__((always_inline)) { return (uint32_t)(g & 3) * G::kTileBytes; };
  auto vslot = [&](int g) __attribute__((always_inline)) {
    return (uint32_t)(4 + (g & 3)) * G::kTileBytes;
  };
  // group g of loads: K(g) and V(g-1), whichever exist
  auto issue = [&](int g) __attribute__((always_inline)) {
    if (g < n_tiles) load_one(g, smem + kslot(g), std::false_type{});
    if (g >= 1 && g <= n_tiles) load_one(g - 1, smem + vslot(g - 1), std::true_type{});
  };
  auto group_loads = [&](int g) __attribute__((always_inline)) {
    return kCpw * ((g < n_tiles ? 1 : 0) + (g >= 1 && g <= n_tiles ? 1 : 0));
  };
  // waits until at most `left` of this wave's loads are in flight
  auto wait_left = [&](int left) __attribute__((always_inline)) {
    if (left <= 0)
      wait_vmem();
    else if (left <= kCpw)
      wait_vmem_le<kCpw>();
    else
      wait_vmem_le<2 * kCpw>();
  };

  // ---- per-lane LDS read offsets (per-lane base + immediates, as in
  // attn_kernel.h): K read of k-step ks for key row l32 of a 32-key block; V
  // transposing reads of d-block db, lo/hi half w2
  uint32_t koff_lds[kKs];
  {
    const int x = l32 & (G::kBlk - 1);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks)
      koff_lds[ks] = (uint32_t)(l32 * G::kRowBytes +
                                ((2 * (ks ^ (x >> 1)) + (hh ^ (x & 1))) << 4));
  }
  uint32_t voff_lds[kDb][2];
  {
    const int g1 = (lane >> 4) & 1;
    const int j16 = lane & 15;
#pragma unroll
    for (int db = 0; db < kDb; ++db)
#pragma unroll
      for (int w2 = 0; w2 < 2; ++w2) {
        const int r = 4 * hh + (j16 >> 2) + 8 * w2;
        const int col = 32 * db + 16 * g1 + 4 * (j16 & 3);
        voff_lds[db][w2] = v_off<D>(r, col >> 3) + ((col >> 2) & 1) * 8;
      }
  }

  f32x16_t oacc[kDb];
#pragma unroll
  for (int db = 0; db < kDb; ++db) oacc[db] = f32x16_t{};
  f32x16_t sacc[2];       // S^T of the current tile, two 32-key blocks
  uint32_t pk[2][8];      // P^T of the previous tile as bf16 pairs
  // The softmax denominator l: this lane's part (its 16 keys of each 32-key
  // block), summed in the softmax phase from the same bf16-rounded numerators
  // the P.V product uses (one dot2 against (1, 1) per pair), so the weights sum
  // to one exactly; the two half-waves' parts are added in the epilogue.  Eight
  // partial sums keep each dot2's accumulator chain two deep (with two, the
  // chains' latency held up the softmax phase: 1.6% slower overall).
  float lsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  // Matrix phase of tile t: P.V of tile t-1 (kPV) and S of tile t (kQK), with
  // K(t) at LDS byte offset k_at and V(t-1) at v_at.  The two MFMA streams
  // are interleaved step by step; the LDS reads run two steps ahead.  With
  // kPf the first two steps' fragments are already in kf/vf (read at the end
  // of the softmax phase before).
  // LDS fragment reads.  QK step i: key block i / kKs, k-step i % kKs (key
  // block 0 first, so the first two steps read only key rows 0-31); PV step
  // i: 16-key step i / kDb, d-block i % kDb.
  auto rk = [&](uint32_t k_at, int i) __attribute__((always_inline)) {
    const CA_LDS unsigned char* kl = (const CA_LDS unsigned char*)smem + k_at;
    return *(CA_LDS const u32x4_t*)(kl + koff_lds[i % kKs] + (i / kKs) * 32 * G::kRowBytes);
  };
  auto rv = [&](uint32_t v_at, int i) __attribute__((always_inline)) {
    const CA_LDS unsigned char* vl = (const CA_LDS unsigned char*)smem + v_at;
    const int db = i % kDb;
    const uint32_t imm = 16 * (i / kDb) * G::kRowBytes;
    const i16x4_t lo =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((CA_LDS i16x4_t*)(vl + voff_lds[db][0] + imm));
    const i16x4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((CA_LDS i16x4_t*)(vl + voff_lds[db][1] + imm));
    const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
    const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4_t{lo2[0], lo2[1], hi2[0], hi2[1]};
  };
  u32x4_t kf[3], vf[3];  // K and V fragments in flight (ring of three steps)
  auto matrix_phase = [&](uint32_t k_at, uint32_t v_at, auto pv_tag, auto qk_tag, auto pf_tag)
      __attribute__((always_inline)) {
    constexpr bool kPV = decltype(pv_tag)::value;
    constexpr bool kQK = decltype(qk_tag)::value;
    constexpr bool kPf = decltype(pf_tag)::value;
    auto read_k = [&](int i) __attribute__((always_inline)) { return rk(k_at, i); };
    auto read_v = [&](int i) __attribute__((always_inline)) { return rv(v_at, i); };
    if constexpr (!kPf) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (kQK) kf[i] = read_k(i);
        if constexpr (kPV) vf[i] = read_v(i);
      }
    }
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
      if constexpr (kQK) {
        if (i + 2 < kStepsQK) kf[(i + 2) % 3] = read_k(i + 2);
      }
      if constexpr (kPV) {
        if (i + 2 < kStepsPV) vf[(i + 2) % 3] = read_v(i + 2);
      }
      if constexpr (kQK) {
        if (i < kStepsQK) {
          const int kb2 = i / kKs, ks = i % kKs;
          sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, kf[i % 3]), __builtin_bit_cast(bf16x8_t, qf[ks]),
              ks == 0 ? f32x16_t{} : sacc[kb2], 0, 0, 0);
        }
      }
      if constexpr (kPV) {
        if (i < kStepsPV) {
          const int s = i / kDb, db = i % kDb;
          const u32x4_t pb = {pk[s >> 1][(s & 1) * 4 + 0], pk[s >> 1][(s & 1) * 4 + 1],
                              pk[s >> 1][(s & 1) * 4 + 2], pk[s >> 1][(s & 1) * 4 + 3]};
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, vf[i % 3]), __builtin_bit_cast(bf16x8_t, pb), oacc[db],
              0, 0, 0);
        }
      }
      // one step at a time: the scheduler would otherwise start most of the
      // phase's LDS reads at once and run out of registers
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Softmax phase of tile t: numerators 2^S of the scores in sacc into pk and
  // l (with a mask, keys >= total get P = 0; they re-read the last key row,
  // so their scores are finite).
  auto softmax_phase = [&](int t, auto mask_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float p0 = __builtin_amdgcn_exp2f(sacc[kb2][2 * i]);
        float p1 = __builtin_amdgcn_exp2f(sacc[kb2][2 * i + 1]);
        if constexpr (decltype(mask_tag)::value) {
          const int key0 = t * kBN + kb2 * 32 + 8 * ((2 * i) >> 2) + 4 * hh + ((2 * i) & 3);
          if (key0 >= total) p0 = 0.f;
          if (key0 + 1 >= total) p1 = 0.f;
        }
        const uint32_t w = pack_bf16(p0, p1);
        pk[kb2][i] = w;
        const bf16x2_t pw = __builtin_bit_cast(bf16x2_t, w);
        const int li = (i & 3) + 4 * kb2;
        lsum[li] = __builtin_amdgcn_fdot2_f32_bf16(pw, one2, lsum[li], false);
      }
  };

  // Barrier at the end of a matrix phase (the scores cross it) and at the end
  // of a softmax phase (the numerators cross it).
  auto end_matrix = [&]() __attribute__((always_inline)) {
    pin(sacc[0]);
    pin(sacc[1]);
    wg_barrier();
    pin(sacc[0]);
    pin(sacc[1]);
  };
  auto end_softmax = [&]() __attribute__((always_inline)) {
    pin(pk[0]);
    pin(pk[1]);
    asm volatile("" : "+v"(lsum[0]), "+v"(lsum[1]), "+v"(lsum[2]), "+v"(lsum[3]));
    asm volatile("" : "+v"(lsum[4]), "+v"(lsum[5]), "+v"(lsum[6]), "+v"(lsum[7]));
    wg_barrier();
    pin(pk[0]);
    pin(pk[1]);
  };

  // One tile: matrix phase (P.V of tile t-1 unless kFirst, S of tile t), then
  // the softmax phase, with the loads of group t+3 started in it.
  auto step = [&](int t, auto first_tag, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_tag)::value;
    // the matrix phase issues at the higher wave priority, so the SIMD picks
    // this wave's MFMAs and LDS reads over the other wave's softmax
    __builtin_amdgcn_s_setprio(3);
    matrix_phase(kslot(t), vslot(t - 1), std::integral_constant<bool, !kFirst>{}, std::true_type{},
                 std::integral_constant<bool, !kFirst>{});
    __builtin_amdgcn_s_setprio(0);
    wait_left(group_loads(t + 2));
    end_matrix();
    softmax_phase(t, mask_tag);
    issue(t + 3);
    // The next matrix phase's first two steps: key rows 0-31 of K(t+1) and
    // rows 0-15 of V(t).  Waves 0-3 load rows 0-31 of every tile; they waited
    // for these loads at the end of their matrix phase of tile t, and the
    // barrier after it made them visible, before either group gets here.  The
    // read latency moves into the softmax phase.
    if (t + 1 < n_tiles) {
      kf[0] = rk(kslot(t + 1), 0);
      kf[1] = rk(kslot(t + 1), 1);
    }
    vf[0] = rv(vslot(t), 0);
    vf[1] = rv(vslot(t), 1);
    end_softmax();
  };

  // ---- prologue: K(0) lands, groups 1 and 2 start
  load_one(0, smem + kslot(0), std::false_type{});
  wait_vmem();
  wg_barrier();
  after_prologue();
  issue(1);
  issue(2);
  if (group_b) wg_barrier();  // group B runs one phase behind group A

  // ---- tiles 0 .. n-1 (the last one masked), then P.V of tile n-1
  if (n_tiles == 1) {
    step(0, std::true_type{}, Mask{});
  } else {
    step(0, std::true_type{}, NoMask{});
    for (int t = 1; t + 1 < n_tiles; ++t) step(t, std::false_type{}, NoMask{});
    step(n_tiles - 1, std::false_type{}, Mask{});
  }
  matrix_phase(0u, vslot(n_tiles - 1), std::true_type{}, std::false_type{}, std::true_type{});
  if (!group_b) wg_barrier();  // matches group B's first barrier

  // ---- epilogue: range check over the workgroup (this barrier also joins the
  // two groups), then normalise and store this lane's query row
  const float lh = ((lsum[0] + lsum[1]) + (lsum[2] + lsum[3])) + ((lsum[4] + lsum[5]) + (lsum[6] + lsum[7]));
  const float l_tot = lh + other_half(lh);
  float acc = l_tot;
#pragma unroll
  for (int db = 0; db < kDb; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += oacc[db][i];
  T* ob = static_cast<T*>(a.o) + e * a.o_bstride + (int64_t)it.h * D;
  if (__syncthreads_or(!__builtin_isfinite(acc) || !(l_tot >= 0x1p-64f))) {
    if (tid == 0) ob[(int64_t)it.q0 * rs] = overflow_marker<T>();
    return;
  }
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    T* orow = ob + (int64_t)qrow * rs;
#pragma unroll
    for (int db = 0; db < kDb; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hh;
        Io<T>::store4(orow + d0, oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv,
                      oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      }
  }
}

// Main pass, 256-row work items on the ping-pong schedule, as a persistent
// launch: one workgroup per CU takes work items from its die's queue (the
// die's launch-slot share of plan_slot_work, longest items first) until it is
// empty, then from the other dies' queues, so a die that runs at a lower clock
// ends up with less work and a new item needs no workgroup launch.  Thread 0
// starts the claim of the next item before the current one; the atomic's
// latency overlaps the first tile's load, whose wait (vmcnt 0) also covers it,
// and the result goes to LDS after the prologue's barrier.  The claim words
// (a.queue[0 .. n_xcd)) are zero at launch (queue_clear runs just before).
template <int D, typename T>
__global__ __launch_bounds__(512, 1) void chunk_attn_fwd_pingpong(KernelArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ long long next_item;  // >= 0 item, -1 none left, -2 claim again
  __shared__ int used_up;          // thread 0: dies (from our own on) found empty
  const int nx = a.plan.n_xcd;
  // the die this workgroup runs on (hardware register XCC_ID, bits 3:0)
  const int die = (int)(__builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) % (unsigned)nx);
  auto die_at = [&](int k) __attribute__((always_inline)) {
    return die + k < nx ? die + k : die + k - nx;
  };
  // thread 0: claim with one atomic per die until one has work left
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
    attn_item_pingpong<D, T>(a, decode(a.plan, w), smem, [&]() __attribute__((always_inline)) {
      if (threadIdx.x == 0) {
        long long nw = -1;
        if (k < nx) {
          nw = claim_word_item(a.plan, die_at(k), ticket);
          if (nw < 0) nw = -2;
        }
        next_item = nw;
      }
    });
    wg_barrier();
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

}  // namespace chunkattn
