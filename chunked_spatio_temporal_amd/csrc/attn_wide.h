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
// Workspace slot of one part of a key-split item: the partial O of 8 waves x
// 3 query blocks x 8 dim blocks x 64 lanes x 4 floats, in register order, then
// the partial l of 8 waves x 3 query blocks x 64 lanes.
constexpr int kSplitOFloats = kWideWaves * 3 * 8 * 64 * 4;
constexpr int kSplitSlotFloats = kSplitOFloats + kWideWaves * 3 * 64;

__device__ __forceinline__ int wide_kswz(int r) { return r & 15; }        // 16-byte blocks
__device__ __forceinline__ int wide_vswz(int r) { return 2 * (r & 7); }   // 16-byte blocks

// Two 1 KB LDS DMA chunks 4 KB apart (chunks c and c + 4 of a tile), each
// from its own wave-uniform base in scalar registers plus the same per-lane
// byte offset: one M0 save and restore for both.  Wait states as in
// load_lds16x2_async.
__device__ __forceinline__ void load_lds16x2_split(const void* sbase0, const void* sbase1,
                                                   uint32_t voff, void* lds_chunk) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = (uint32_t)(uintptr_t)(CA_LDS void*)lds_chunk;
  const uint64_t sb0 = (uint64_t)(uintptr_t)sbase0;
  const uint64_t sb1 = (uint64_t)(uintptr_t)sbase1;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_add_i32 m0, m0, 0x1000\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sb0), "s"(sb1), "s"(m0)
      : "memory");
#endif
}

// Device-scope (sc1) store and loads of key-split partials: written through to
// the memory every die sees and read from it, so neither side needs a fence
// that writes back or invalidates a whole L2 (other CUs keep their K/V tiles
// cached).  The loads wait for their data inside the same asm block.
__device__ __forceinline__ void store_device16(float* p, const f32x4_t& x) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(x) : "memory");
}
__device__ __forceinline__ void store_device4(float* p, float x) {
  asm volatile("global_store_dword %0, %1, off sc1" : : "v"(p), "v"(x) : "memory");
}
// eight 16-byte loads at p, p + 1 KB, ... p + 7 KB and one 4-byte load at
// pl, all in flight together (one memory latency); two base addresses with
// immediate offsets keep the address registers few
__device__ __forceinline__ void load_device16x8_4(const float* p, f32x4_t (&x)[8],
                                                  const float* pl, float& l) {
  const float* p4 = p + 1024;  // + 4 KB
  asm volatile(
      "global_load_dwordx4 %0, %9, off sc1\n\t"
      "global_load_dwordx4 %1, %9, off offset:1024 sc1\n\t"
      "global_load_dwordx4 %2, %9, off offset:2048 sc1\n\t"
      "global_load_dwordx4 %3, %9, off offset:3072 sc1\n\t"
      "global_load_dwordx4 %4, %10, off sc1\n\t"
      "global_load_dwordx4 %5, %10, off offset:1024 sc1\n\t"
      "global_load_dwordx4 %6, %10, off offset:2048 sc1\n\t"
      "global_load_dwordx4 %7, %10, off offset:3072 sc1\n\t"
      "global_load_dword %8, %11, off sc1\n\t"
      "s_waitcnt vmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
        "=&v"(x[6]), "=&v"(x[7]), "=&v"(l)
      : "v"(p), "v"(p4), "v"(pl)
      : "memory");
}

__device__ __forceinline__ void pin(f32x4_t& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(u32x4_t& x) { asm volatile("" : "+v"(x)); }

// One work item (head_dim 128, bf16) with kQB 16-row query blocks per wave:
// wave w takes rows [16*kQB*w, 16*kQB*(w+1)) of each 384-row block of the
// item.  kQB = 3 covers 384 rows; an item with at most 256 (128) rows, the last
// query tile of a chunk, runs with kQB = 2 (1): its matrix phases shrink to
// 64 (32) MFMAs instead of padding the missing rows.
//
// With kQB = 3 an item may hold several consecutive 384-row blocks of one
// (chunk, head) (the caller sees to at least two key tiles then): the blocks
// walk the same key/value tiles one after the other as one stream, so the
// load pipeline and the two-group schedule run on across block boundaries
// instead of draining and refilling per block.  Block j+1's Q is loaded in
// the softmax phase of block j's last tile (Q's registers are free once that
// tile's S is computed), and block j's normalise-and-store runs in the softmax
// phase of block j+1's first tile (its O is complete once that tile's matrix
// phase has added P.V of block j's last tile).
//
// kExact: Q stays as stored and each key block's scores are multiplied by
// scale * log2 e in fp32 inside the matrix phase (while the matrix core works
// on the next key block), instead of rounding scale * log2 e * Q to bf16 once
// per block: the scores then carry no extra rounding, at the cost of 48
// multiplies per wave and tile.
//
// after_prologue() runs once in every thread, after the prologue's barrier.
// A wave whose rows of block j left fp32's range sets range_flags[j & 1]
// (LDS).  Thread 0 marks block j for the recheck in the opening step of block
// j+2, when every wave is a full phase past block j's stores; the caller
// marks the item's last two blocks.
template <int kQB, bool kStream, bool kExact, typename AfterPrologue>
__device__ __forceinline__ void attn_item_wide(const KernelArgs& a, const Item& it,
                                               unsigned char* smem, int* range_flags,
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
  // Lane values (lane & 15, lane >> 4) and the per-lane offsets derived from
  // them come from lane_now().  Items of one block keep them in registers; in
  // the stream form every use derives them afresh from the thread id, so that
  // none holds a register across the tile loops (the block boundaries leave
  // no register to spare).
  const bool group_b = wave >= 4;

  const int pred = it.pred_rows;
  const int total = pred + it.own_rows;
  const int n_tiles = (total + kBN - 1) / kBN;  // key/value tiles per block
  static_assert(!kStream || kQB == 3, "multi-block items run with three query blocks per wave");
  const int nblk = kStream ? (it.q_rows + kWideBlockRows - 1) / kWideBlockRows : 1;
  // the walk: key tiles [t0, t0 + nt) (a part of a key-split item walks its
  // share of the tiles), or nblk times all of them in the stream form
  const int t0 = kStream ? 0 : it.t_lo;
  const int nt = kStream ? n_tiles : it.t_hi - it.t_lo;
  const int n_stream = kStream ? nblk * n_tiles : nt;  // tiles of the whole stream
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
  // Lane-dependent addresses of the Q loads and O stores are computed where
  // they are used (the empty asm keeps the compiler from hoisting them out of
  // the tile loops, where they would hold registers for the whole stream).
  const int lane_fixed = tid & 63;
  auto lane_now = [&]() __attribute__((always_inline)) {
    if constexpr (kStream) {
      int x = tid;
      asm volatile("" : "+v"(x));
      return x & 63;
    } else {
      // one item walk per block: the lane values stay in registers
      return lane_fixed;
    }
  };
  auto opaque_lane_row = [&]() __attribute__((always_inline)) {
    return wave * kRowsW + (lane_now() & 15);
  };
  auto load_q = [&](int jb) __attribute__((always_inline)) {
    const int r_lane = opaque_lane_row();
    const int g8 = (lane_now() >> 4) * 8;
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3) {
      const int r = jb * kWideBlockRows + r_lane + q3 * 16;
      const bool valid = r < it.q_rows;
      const T* qrow = qb + (int64_t)(it.q0 + r) * rs + g8;
#pragma unroll
      for (int ks = 0; ks < kKS; ++ks)
        qf[q3][ks] = valid ? Io<T>::load8(qrow + ks * 32) : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  // scaled by scale * log2 e (nearest-even): S^T comes out in the log2 domain
  // (exact-scale items leave Q as stored and scale S instead)
  auto scale_q = [&]() __attribute__((always_inline)) {
    if constexpr (kExact) return;
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

  // ---- per-lane DMA map: wave w fills LDS chunks c0 and c0 + 4 of a tile
  // (c0 = w for w < 4, w + 4 otherwise: rows 0-31 come from waves 0-3); chunk
  // c receives tile row 4c + g at physical block j (logical block j ^
  // swizzle(row)).  The two rows of a lane are 16 apart, so they share the
  // swizzle and one per-lane offset; the second chunk's 16-row shift goes into
  // the scalar base.
  const int c0 = wave < 4 ? wave : wave + 4;
  auto dma_off = [&](auto v_tag) __attribute__((always_inline)) {
    const int l = lane_now();
    const int r = c0 * 4 + (l >> 4);
    const int sw = decltype(v_tag)::value ? wide_vswz(r) : wide_kswz(r);
    return (uint32_t)(((uint32_t)r * (uint32_t)rs + (uint32_t)(((l & 15) ^ sw) * 8)) *
                      (uint32_t)sizeof(T));
  };
  const uint64_t shift16 = (uint64_t)16 * (uint64_t)rs * sizeof(T);
  auto load_one = [&](int t, unsigned char* dst, auto v_tag) __attribute__((always_inline)) {
    constexpr bool kV = decltype(v_tag)::value;
    const T* pre = kV ? vpre : kpre;
    const T* own = kV ? vown : kown;
    const int r0 = t * kBN;
    if (t < np || (t >= no && t < nf)) {
      const uint64_t b = (t < np ? (kV ? vpre_b : kpre_b) : (kV ? vown_s : kown_s)) +
                         (uint64_t)(uint32_t)t * tstride;
      load_lds16x2_split(reinterpret_cast<const char*>((uintptr_t)b),
                         reinterpret_cast<const char*>((uintptr_t)(b + shift16)),
                         dma_off(v_tag), dst + c0 * 1024);
    } else {
      // straddling or ragged tile: rows past the end re-read the last row
      const int l = lane_now();
#pragma unroll
      for (int i = 0; i < kCpw; ++i) {
        const int r = (c0 + 4 * i) * 4 + (l >> 4);
        int jj = r0 + r;
        jj = jj < total ? jj : total - 1;
        const int blk = (l & 15) ^ (kV ? wide_vswz(r) : wide_kswz(r));
        const T* src = jj < pred ? pre + (int64_t)jj * rs : own + (int64_t)(jj - pred) * rs;
        load_lds16_async(src + blk * 8, dst + (c0 + 4 * i) * 1024);
      }
    }
  };
  // Ring slots by stream position u (block u / n_tiles, tile u % n_tiles).
  auto kslot = [&](int u) __attribute__((always_inline)) { return (uint32_t)(u & 3) * G::kTileBytes; };
  auto vslot = [&](int u) __attribute__((always_inline)) {
    return (uint32_t)(4 + (u & 3)) * G::kTileBytes;
  };
  // group u of loads: K of stream position u and V of position u-1, whichever
  // exist; t = u % n_tiles
  auto issue = [&](int u, int t) __attribute__((always_inline)) {
    if (u < n_stream) load_one(t, smem + kslot(u), std::false_type{});
    if (u >= 1 && u <= n_stream)
      load_one(kStream && t == 0 ? n_tiles - 1 : t - 1, smem + vslot(u - 1), std::true_type{});
  };
  auto group_loads = [&](int u) __attribute__((always_inline)) {
    return kCpw * ((u < n_stream ? 1 : 0) + (u >= 1 && u <= n_stream ? 1 : 0));
  };
  // tile index of stream position u + d (0 <= d <= 3) given t = u % n_tiles
  auto tile_ahead = [&](int t, int d) __attribute__((always_inline)) {
    int x = t + d;
    if constexpr (!kStream) return x;  // positions past the item are not loaded
#pragma unroll
    for (int k = 0; k < 3; ++k) x = x >= n_tiles ? x - n_tiles : x;
    return x;
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
  // logical block 4ks + g, at kbase ^ (ks << 6) (kb by immediate: the swizzle
  // repeats every 16 rows).  V^T fragment (s, db): rows 32s + 4g + (j >> 2)
  // and 16 further, dims 16db + 4(j & 3) .. +3, at vbase ^ (db << 5) (s and
  // the second read by immediates).  The XOR touches only bits 5-7, so it
  // commutes with adding the 1 KB-aligned tile address; one register per
  // operand instead of one per fragment column.
  auto kbase_now = [&]() __attribute__((always_inline)) {
    const int l = lane_now();
    const int jj = l & 15, gg = l >> 4;
    return (uint32_t)(jj * G::kRowBytes + ((jj & 12) << 4) + (((gg ^ jj) & 3) << 4));
  };
  auto vbase_now = [&]() __attribute__((always_inline)) {
    const int l = lane_now();
    const int r = 4 * (l >> 4) + ((l & 15) >> 2);
    return (uint32_t)(r * G::kRowBytes + ((r & 7) << 5) + 8 * (l & 3));
  };

  f32x4_t oacc[kQB][kDB];
#pragma unroll
  for (int q3 = 0; q3 < kQB; ++q3)
#pragma unroll
    for (int db = 0; db < kDB; ++db) oacc[q3][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t sacc[kQB][kKB];  // S^T of the current tile
  u32x4_t pk[kQB][kPS];    // P^T of the previous tile, B operands of P.V
  // l per query block: this lane's keys, kLs partial sums each (short
  // dependency chains in the softmax phase), from the rounded numerators (one
  // dot2 against (1, 1) per pair)
  constexpr int kLs = 4;
  float lsum[kQB][kLs];
#pragma unroll
  for (int q3 = 0; q3 < kQB; ++q3)
#pragma unroll
    for (int c = 0; c < kLs; ++c) lsum[q3][c] = 0.f;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  // k_at, v_at: LDS byte offsets of the tiles within smem
  auto rk = [&](uint32_t k_at, uint32_t kbase, int i) __attribute__((always_inline)) {
    // QK step i: key block i / kKS, dim step i % kKS
    const uint32_t at = ((uint32_t)(uintptr_t)(CA_LDS void*)smem + k_at + kbase) ^
                        (uint32_t)((i % kKS) << 6);
    return *(CA_LDS const u32x4_t*)((CA_LDS unsigned char*)(uintptr_t)at +
                                    (i / kKS) * 16 * G::kRowBytes);
  };
  auto rv = [&](uint32_t v_at, uint32_t vbase, int i) __attribute__((always_inline)) {
    // PV step i: key step i / kDB, dim block i % kDB
    const uint32_t at = ((uint32_t)(uintptr_t)(CA_LDS void*)smem + v_at + vbase) ^
                        (uint32_t)((i % kDB) << 5);
    const CA_LDS unsigned char* vl =
        (CA_LDS unsigned char*)(uintptr_t)at + (i / kDB) * 32 * G::kRowBytes;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CA_LDS i16x4_t*)vl);
    const i16x4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((CA_LDS i16x4_t*)(vl + 16 * G::kRowBytes));
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
  auto no_mid = []() __attribute__((always_inline)) {};
  auto matrix_phase = [&](uint32_t k_at, uint32_t v_at, auto pv_tag, auto qk_tag, auto pf_tag,
                          auto&& mid) __attribute__((always_inline)) {
    constexpr bool kPV = decltype(pv_tag)::value;
    constexpr bool kQK = decltype(qk_tag)::value;
    constexpr bool kPf = decltype(pf_tag)::value;
    constexpr int i0 = kPV ? 0 : kStepsPV;
    constexpr int i1 = kQK ? kStepsPV + kStepsQK : kStepsPV;
    const uint32_t kb = kbase_now(), vb = vbase_now();
    auto read = [&](int i) __attribute__((always_inline)) {
      return i < kStepsPV ? rv(v_at, vb, i) : rk(k_at, kb, i - kStepsPV);
    };
    if constexpr (!kPf) {
      fr[0] = read(i0);
      fr[1] = read(i0 + 1);
    }
    auto scale_s = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
      for (int q3 = 0; q3 < kQB; ++q3)
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[q3][kb][e] *= a.scale_log2;
    };
    auto one_step = [&](int i) __attribute__((always_inline)) {
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
        // exact scale: S of key block kb-1 is complete; into the log2 domain
        // while the matrix core works on block kb
        if (kExact && ks == 2 && kb >= 1) scale_s(kb - 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
#pragma unroll
    for (int i = i0; i < kStepsPV; ++i) one_step(i);
    // between the P.V and the S steps (a new block's Q is made ready here)
    mid();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = kStepsPV > i0 ? kStepsPV : i0; i < i1; ++i) one_step(i);
    if constexpr (kExact && kQK) scale_s(kKB - 1);
  };

  // Softmax phase of tile t: numerators 2^S into pk and l (with a mask, keys
  // >= total get P = 0; they re-read the last key row, so their scores are
  // finite).
  auto softmax_phase = [&](int t, auto mask_tag) __attribute__((always_inline)) {
    const int key_lane = decltype(mask_tag)::value ? t * kBN + 4 * (lane_now() >> 4) : 0;
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3)
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          float p0 = __builtin_amdgcn_exp2f(sacc[q3][kb][2 * h2]);
          float p1 = __builtin_amdgcn_exp2f(sacc[q3][kb][2 * h2 + 1]);
          if constexpr (decltype(mask_tag)::value) {
            const int key0 = key_lane + kb * 16 + 2 * h2;
            if (key0 >= total) p0 = 0.f;
            if (key0 + 1 >= total) p1 = 0.f;
          }
          const uint32_t w = pack_bf16(p0, p1);
          pk[q3][kb >> 1][(kb & 1) * 2 + h2] = w;
          float& ls = lsum[q3][(kb * 2 + h2) % kLs];
          ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one2, ls, false);
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
#pragma unroll
      for (int c = 0; c < kLs; ++c) asm volatile("" : "+v"(lsum[q3][c]));
    }
    wg_barrier();
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3) {
      pin(pk[q3][0]);
      pin(pk[q3][1]);
    }
  };

  // Row sums of the block just completed: l over the four lane groups (keys
  // 4g + e); lsum restarts for the next block.
  auto take_l = [&](float (&l_tot)[kQB]) __attribute__((always_inline)) {
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3) {
      float x = lsum[q3][0];
#pragma unroll
      for (int c = 1; c < kLs; ++c) x += lsum[q3][c];
      l_tot[q3] = sum_xor32(sum_xor16(x));
#pragma unroll
      for (int c = 0; c < kLs; ++c) lsum[q3][c] = 0.f;
    }
  };
  // Normalise and store block jb (its O complete, its row sums l_tot), folding
  // its range check into range_flags[jb & 1].
  T* const ob = static_cast<T*>(a.o) + e * a.o_bstride + (int64_t)it.h * D;
  auto finish_block = [&](int jb, const float (&l_tot)[kQB]) __attribute__((always_inline)) {
    float acc = 0.f;
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3) {
      acc += l_tot[q3];
#pragma unroll
      for (int db = 0; db < kDB; ++db)
        acc += (oacc[q3][db][0] + oacc[q3][db][1]) + (oacc[q3][db][2] + oacc[q3][db][3]);
    }
    bool bad = !__builtin_isfinite(acc);
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3) bad = bad || !(l_tot[q3] >= 0x1p-64f);
    const int l = lane_now();
    if (__ballot(bad) != 0 && l == 0) range_flags[jb & 1] = 1;
    const int r_lane = wave * kRowsW + (l & 15);
    // Lane (j, g) holds dims 16db + 4g .. +3 of its row for every db.  Lanes g
    // and g ^ 1 (16 apart, same row) trade halves so that each writes 8
    // consecutive dims (16 bytes) per pair of db: even g the dims 32m + 4g ..
    // +7 (its own db = 2m values and its partner's), odd g the dims
    // 32m + 16 + 4(g-1) .. +7 (its partner's db = 2m+1 values and its own):
    // half as many store instructions as 8-byte stores.  The trade is one
    // 16-lane row swap per word pair (x from db 2m, y from db 2m+1): x of the
    // odd row (g odd) goes to the even row's y, which leaves even g with
    // {own x, partner's x} and odd g with {partner's y, own y}, each in dim
    // order.
    const bool odd = (l >> 4) & 1;
    const int col = 8 * (l >> 5) + (odd ? 16 : 0);
#pragma unroll
    for (int q3 = 0; q3 < kQB; ++q3) {
      const int r = jb * kWideBlockRows + r_lane + q3 * 16;
      const float inv = 1.0f / l_tot[q3];
      T* orow = ob + (int64_t)(it.q0 + r) * rs + col;
#pragma unroll
      for (int m = 0; m < kDB / 2; ++m) {
        const f32x4_t& oa = oacc[q3][2 * m];
        const f32x4_t& ob2 = oacc[q3][2 * m + 1];
        const uint32_t a0 = pack_bf16(oa[0] * inv, oa[1] * inv);
        const uint32_t a1 = pack_bf16(oa[2] * inv, oa[3] * inv);
        const uint32_t b0 = pack_bf16(ob2[0] * inv, ob2[1] * inv);
        const uint32_t b1 = pack_bf16(ob2[2] * inv, ob2[3] * inv);
        uint32_t x0 = a0, y0 = b0, x1 = a1, y1 = b1;
        swap_rows16(x0, y0);
        swap_rows16(x1, y1);
        const u32x4_t v4 = {x0, x1, y0, y1};
        if (r < it.q_rows) *reinterpret_cast<u32x4_t*>(orow + 32 * m) = v4;
      }
    }
  };

  // One tile of the stream: matrix phase (P.V of position u-1, S of position
  // u), then the softmax phase of tile t = u % n_tiles of block jb.
  //   kFirst: the stream's first tile (no P.V yet, fragments not prefetched);
  //   kOpen:  the first tile of block jb >= 1: between the P.V and the S
  //           steps it waits for block jb's Q (and the key/value group due at
  //           the end of this phase anyway), scales it and issues load group
  //           u+2; after the softmax, block jb-1 is stored and block jb-2
  //           marked if it left fp32's range;
  //   kLast:  block jb's last tile (masked).  If block jb+1 follows, its Q
  //           loads go out at the start of the softmax phase (Q's registers
  //           are free once this tile's S is computed) and load group u+3
  //           waits for the next phase: the compiler, which sees the Q loads
  //           but not the key/value DMA, waits for every load before Q's
  //           first use, so no DMA is issued after Q until then.
  // The boundary work sits where the S accumulators are dead (after the
  // softmax) or not yet live (before the S steps), so the register peak stays
  // that of an ordinary tile.
  auto step = [&](int u, int t, int jb, auto first_tag, auto open_tag, auto last_tag)
      __attribute__((always_inline)) {
    constexpr bool kFirst = decltype(first_tag)::value;
    constexpr bool kOpen = decltype(open_tag)::value;
    constexpr bool kLast = decltype(last_tag)::value;
    __builtin_amdgcn_s_setprio(3);
    if constexpr (kOpen) {
      matrix_phase(kslot(u), vslot(u - 1), std::true_type{}, std::true_type{}, std::true_type{},
                   [&]() __attribute__((always_inline)) {
                     wait_vmem();
                     scale_q();
                     issue(u + 2, tile_ahead(t, 2));
                   });
    } else {
      matrix_phase(kslot(u), vslot(u - 1), std::integral_constant<bool, !kFirst>{},
                   std::true_type{}, std::integral_constant<bool, !kFirst>{}, no_mid);
    }
    __builtin_amdgcn_s_setprio(0);
    wait_left(group_loads(u + 2));
    end_matrix();
    const bool next_q = kLast && jb + 1 < nblk;
    if (next_q) load_q(jb + 1);
    float l_prev[kQB];
    if constexpr (kOpen) take_l(l_prev);
    softmax_phase(t, std::integral_constant<bool, kLast>{});
    if constexpr (kOpen) {
      if (jb >= 2 && tid == 0 && range_flags[jb & 1] != 0) {
        // block jb-2 (flag parity jb & 1): every wave stored it at least a
        // phase ago; the marker follows thread 0's own store of that element
        ob[(int64_t)(it.q0 + (jb - 2) * kWideBlockRows) * rs] = overflow_marker<T>();
        range_flags[jb & 1] = 0;
      }
      finish_block(jb - 1, l_prev);
#pragma unroll
      for (int q3 = 0; q3 < kQB; ++q3)
#pragma unroll
        for (int db = 0; db < kDB; ++db) oacc[q3][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    if (!next_q) issue(u + 3, tile_ahead(t, 3));
    // The next matrix phase's first two fragments: rows 0-31 of V(u), which
    // waves 0-3 load; they waited for them at the end of their matrix phase
    // of position u, and the barrier after it made them visible.
    {
      const uint32_t vb = vbase_now();
      fr[0] = rv(vslot(u), vb, 0);
      fr[1] = rv(vslot(u), vb, 1);
    }
    end_softmax();
  };

  // ---- prologue: the first three groups of key/value loads and the Q
  // loads go out together (one memory latency for all), then Q is scaled
  issue(0, t0);
  issue(1, tile_ahead(t0, 1));
  issue(2, tile_ahead(t0, 2));
  load_q(0);
  wait_vmem();
  scale_q();
  wg_barrier();
  after_prologue();
  if (group_b) wg_barrier();  // group B runs one phase behind group A

  using F = std::false_type;
  using Tr = std::true_type;
  if (nt == 1) {
    // one tile per block: every step opens and closes a block
    step(0, t0, 0, Tr{}, F{}, Tr{});
    for (int jb = 1; jb < nblk; ++jb) step(jb, 0, jb, F{}, Tr{}, Tr{});
  } else {
    step(0, t0, 0, Tr{}, F{}, F{});
    for (int u = 1; u + 1 < nt; ++u) step(u, t0 + u, 0, F{}, F{}, F{});
    step(nt - 1, t0 + nt - 1, 0, F{}, F{}, Tr{});
    for (int jb = 1; jb < nblk; ++jb) {
      const int u0 = jb * n_tiles;
      step(u0, 0, jb, F{}, Tr{}, F{});
      for (int t = 1; t + 1 < n_tiles; ++t) step(u0 + t, t, jb, F{}, F{}, F{});
      step(u0 + n_tiles - 1, n_tiles - 1, jb, F{}, F{}, Tr{});
    }
  }
  matrix_phase(0u, vslot(n_stream - 1), std::true_type{}, std::false_type{}, std::true_type{},
               no_mid);
  if (!group_b) wg_barrier();  // matches group B's first barrier

  // ---- epilogue: the last block
  float l_last[kQB];
  take_l(l_last);
  if constexpr (!kStream) {
    if (it.part >= 0) {
      // A part of a key-split item.  Without a maximum the parts' sums add:
      // O = (O_1 + ... + O_S) / (l_1 + ... + l_S).  Each part stores its
      // unnormalised O and l; the part that arrives last adds all of them in
      // part order and finishes the block.
      const int parts = a.plan.split_parts;
      const int l6 = lane_now();
      auto slot_of = [&](int part) __attribute__((always_inline)) {
        return a.split_ws + ((size_t)it.split_idx * parts + part) * kSplitSlotFloats;
      };
      {
        float* ws = slot_of(it.part);
#pragma unroll
        for (int q3 = 0; q3 < kQB; ++q3) {
#pragma unroll
          for (int db = 0; db < kDB; ++db)
            store_device16(ws + (((wave * 3 + q3) * kDB + db) * 64 + l6) * 4, oacc[q3][db]);
          store_device4(ws + kSplitOFloats + (wave * 3 + q3) * 64 + l6, l_last[q3]);
        }
      }
      // the partial has reached device scope before this workgroup arrives
      asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
      wg_barrier();
      if (tid == 0)
        range_flags[2] = atomicAdd(&a.split_cnt[it.split_idx], 1u) == (unsigned)(parts - 1);
      wg_barrier();
      if (range_flags[2] == 0) return;
      // all parts, the own one read back too, added in part order: the sum
      // does not depend on which part arrived last.  A block's O and l of one
      // part come in one batch of loads (8 dim blocks of 64 * 4 floats, 1 KB
      // apart, and l): one memory latency per part and block.
      for (int p = 0; p < parts; ++p) {
        const float* ws = slot_of(p);
#pragma unroll
        for (int q3 = 0; q3 < kQB; ++q3) {
          f32x4_t x[kDB];
          float lp;
          load_device16x8_4(ws + ((wave * 3 + q3) * kDB * 64 + l6) * 4, x,
                            ws + kSplitOFloats + (wave * 3 + q3) * 64 + l6, lp);
#pragma unroll
          for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              oacc[q3][db][e] = p == 0 ? x[db][e] : oacc[q3][db][e] + x[db][e];
          l_last[q3] = p == 0 ? lp : l_last[q3] + lp;
        }
      }
    }
  }
  finish_block(nblk - 1, l_last);
}

// Persistent main pass over the die work queues, exactly as
// chunk_attn_fwd_pingpong (the claim words a.queue[0 .. n_xcd) are zero at
// launch).  kStream = false: work items of up to 384 rows (plan.bm = 384),
// three, two or one query blocks per wave by the item's rows; kStream = true:
// work items of several 384-row blocks of one (chunk, head) (plan.bm a
// multiple of 384), every block with three query blocks per wave.
template <bool kStream, bool kExact>
__device__ __forceinline__ void wide_persistent(const KernelArgs& a, unsigned char* smem) {
  __shared__ long long next_item;  // >= 0 item, -1 none left, -2 claim again
  __shared__ int used_up;          // thread 0: dies (from our own on) found empty
  // [0], [1]: some row of a block (by block parity) left fp32's range; [2]:
  // this workgroup finishes a key-split item
  __shared__ int range_flags[3];
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
      // (items of several blocks are never split)
      w = kStream ? claim_word_item(a.plan, die_at(k), old)
                  : claim_word_unit(a.plan, die_at(k), old);
      if (w >= 0) break;
    }
    used_up = k;
    next_item = w;
  };
  auto uniform_ll = [](long long x) __attribute__((always_inline)) {
    const uint64_t b = (uint64_t)x;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
    return (long long)(((uint64_t)hi << 32) | (uint64_t)lo);
  };
  if (threadIdx.x == 0) {
    used_up = 0;
    range_flags[0] = range_flags[1] = 0;
    claim_sync();
  }
  __syncthreads();
  long long w = uniform_ll(next_item);
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
          nw = kStream ? claim_word_item(a.plan, die_at(k), ticket)
                       : claim_word_unit(a.plan, die_at(k), ticket);
          if (nw < 0) nw = -2;
        }
        next_item = nw;
      }
    };
    const Item it = kStream ? decode(a.plan, w) : decode_unit(a.plan, w);
    if (kStream || it.q_rows > 2 * 16 * kWideWaves)
      attn_item_wide<3, kStream, kExact>(a, it, smem, range_flags, after_prologue);
    else if (it.q_rows > 16 * kWideWaves)
      attn_item_wide<2, false, kExact>(a, it, smem, range_flags, after_prologue);
    else
      attn_item_wide<1, false, kExact>(a, it, smem, range_flags, after_prologue);
    wg_barrier();
    if (threadIdx.x == 0) {
      // the item's last two blocks (the item marked the ones before); each
      // marker follows thread 0's own store of that element
      const int nblk = (it.q_rows + kWideBlockRows - 1) / kWideBlockRows;
      for (int jb = nblk >= 2 ? nblk - 2 : 0; jb < nblk; ++jb) {
        if (range_flags[jb & 1] != 0) {
          static_cast<__bf16*>(a.o)[a.entry(it.b) * a.o_bstride +
                                    (int64_t)(it.q0 + jb * kWideBlockRows) * a.row_stride +
                                    (int64_t)it.h * 128] = overflow_marker<__bf16>();
          range_flags[jb & 1] = 0;
        }
      }
    }
    w = uniform_ll(next_item);
    if (w == -2) {
      wg_barrier();  // every wave has read next_item before thread 0 rewrites it
      if (threadIdx.x == 0) {
        used_up = used_up + 1;
        claim_sync();
      }
      wg_barrier();
      w = uniform_ll(next_item);
    }
  }
}

__global__ __launch_bounds__(512, 1) void chunk_attn_fwd_wide(KernelArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  wide_persistent<false, false>(a, smem);
}

__global__ __launch_bounds__(512, 1) void chunk_attn_fwd_wide_stream(KernelArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  wide_persistent<true, false>(a, smem);
}

// The same two passes with the scale applied to S in fp32 (exact-scale
// contexts).
__global__ __launch_bounds__(512, 1) void chunk_attn_fwd_wide_exact(KernelArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  wide_persistent<false, true>(a, smem);
}

__global__ __launch_bounds__(512, 1) void chunk_attn_fwd_wide_stream_exact(KernelArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  wide_persistent<true, true>(a, smem);
}

// Recheck of 384-row blocks, planned one block per item, organised as
// chunk_attn_recheck: each workgroup tests its share of the blocks (one per
// thread) and recomputes the marked ones, each as three 128-row items on the
// running-maximum schedule.
template <int W>
__global__ __launch_bounds__(W * 64, 8 / W) void chunk_attn_recheck_wide(KernelArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  __shared__ int marked[W * 64];
  __shared__ int n_marked;
  const int64_t n = a.plan.n_items;
  const int64_t per = (n + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n ? lo + per : n;
  for (int64_t base = lo; base < hi; base += blockDim.x) {
    if (threadIdx.x == 0) n_marked = 0;
    __syncthreads();
    if (base + threadIdx.x < hi) {
      const Item it = decode(a.plan, base + threadIdx.x);
      const __bf16 first = static_cast<const __bf16*>(a.o)[a.entry(it.b) * a.o_bstride +
                                                          (int64_t)it.q0 * a.row_stride +
                                                          (int64_t)it.h * 128];
      if (__builtin_isnan((float)first)) marked[atomicAdd(&n_marked, 1)] = (int)threadIdx.x;
    }
    __syncthreads();
    const int m = n_marked;
    for (int i = 0; i < m; ++i) {
      const Item it = decode(a.plan, base + marked[i]);
      for (int sub = 0; sub * 32 * W < it.q_rows; ++sub) {
        Item s = it;
        s.q0 = it.q0 + sub * 32 * W;
        const int left = it.q_rows - sub * 32 * W;
        s.q_rows = left < 32 * W ? left : 32 * W;
        attn_item_sync<128, __bf16, W, false>(a, s, smem);
        __syncthreads();
      }
    }
  }
}

}  // namespace chunkattn
