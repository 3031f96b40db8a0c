// gfx950 chunk-attention forward kernel.
//
// One workgroup (W = 4 or 8 waves) computes BM = 32*W query rows of one
// (chunk, head): each wave owns 32 query rows.  Key/value rows are walked in
// tiles of BN = 64 logical rows; a tile may straddle the predecessor/own
// boundary, each row then picking its source as it is loaded, so the
// predecessor's cached K/V is never concatenated with the chunk's own K/V
// (feature cache, DualParal write-up section 三).
//
// Per tile and wave, on bf16 matrix cores (v_mfma_f32_32x32x16_bf16, fp32
// accumulate):
//   S^T = K . Q^T      keys on the M side, queries on N: each lane ends up
//                      holding 32 scores of ONE query row (its column), so the
//                      softmax statistics of a row live in one lane pair.
//   softmax            sum l per query row in the log2 domain (scale*log2(e)
//                      folded into one FMA before exp2), with a reference
//                      maximum m shared by O and l, so any m gives the exact
//                      result as long as nothing overflows.  Two schedules:
//                      fixed m   m is the row maximum of the first tile and
//                                never changes (no max, rescale or branch per
//                                tile); a work item whose l or O comes out
//                                non-finite marks its output and is redone by
//                                chunk_attn_recheck with the running m.
//                      running m m is raised only when a tile's maximum
//                                exceeds it by more than 2^8, skipping almost
//                                every rescale of O.
//                      P is rounded to bf16 once and l is summed from the
//                      rounded P.
//   O^T += V^T . P^T   P^T comes straight out of the S^T accumulators as the
//                      B operand; V^T is read from row-major V in LDS with the
//                      transposing LDS read (ds_read_b64_tr_b16).  O^T again
//                      has one query row per lane column, so any rescale is a
//                      per-lane scalar.
//
// Data movement.  K and V tiles are stored row-major in LDS, double
// buffered, one barrier per tile.  bf16 tiles go straight from global memory
// to LDS (global_load_lds_dwordx4, 16 bytes per lane, no VGPR staging): each
// wave instruction fills 1 KB of LDS in lane order, and the lane -> global
// address map realises a 16-byte-block XOR swizzle.  Tiles inside one segment
// use a wave-uniform base address plus a fixed per-lane 32-bit offset; only
// the tile that straddles the predecessor/own boundary and the ragged last
// tile compute per-lane row addresses.  Q stays in registers throughout.
// (fp32 storage runs its own kernel, attn_f32.h.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "plan.h"

namespace chunkattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

#define CA_LDS __attribute__((address_space(3)))

constexpr int kBN = 64;               // key/value rows per tile
constexpr float kRescaleLog2 = 8.0f;  // raise m when the tile max exceeds it by > 2^8

struct KernelArgs {
  Plan plan;
  const void* q;
  const void* k;      // own K: entry b at k + b*kv_bstride
  const void* v;
  const void* pk;     // predecessor K: entry b at pk + (b - pred_shift)*p_bstride
  const void* pv;
  void* o;
  int64_t q_bstride;  // elements between batch entries of q
  int64_t o_bstride;  // elements between batch entries of out
  int64_t kv_bstride;
  int64_t p_bstride;
  int pred_shift;
  int row_stride;     // heads * head_dim (elements between consecutive tokens)
  float scale_log2;   // scale * log2(e)
  // Ring of chunk slots (streaming queue): with ring_slots > 0, batch index b
  // (processing order, 0 = the newest chunk) lives in slot
  // (ring_tail - b) mod ring_slots of q, k, v and out, and reads its
  // predecessor in place from the slot of b - 1.  0: batch b is entry b.
  int ring_slots;
  int ring_tail;
  // Work queue of the persistent 256-row main pass (chunk_attn_fwd_pingpong;
  // the other kernels take item plan_slot_work(blockIdx.x)).  Word x <
  // n_xcd counts the claims on die x's share (claim_word_item); queue_clear
  // zeroes the words on the same stream just before the launch.
  unsigned long long* queue;
  // Key-axis split (plan.split_parts > 1, 384-row items only): per split item
  // and part, a slot of kSplitSlotFloats floats for the partial O and l, and
  // per split item an arrival counter, zero at launch.
  float* split_ws;
  unsigned* split_cnt;

  // Physical entry of batch index b (b > -ring_slots).
  __host__ __device__ __forceinline__ int64_t entry(int b) const {
    if (ring_slots == 0) return b;
    const int p = ring_tail - b;
    return p < 0 ? p + ring_slots : p;
  }
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

// ---- tile geometry and LDS swizzles ----------------------------------------
template <int D>
struct Geo {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBlk = D / 8;                       // 16-byte blocks per row
  static constexpr uint32_t kTileBytes = kBN * kRowBytes;  // one K or V tile
  static constexpr uint32_t kBufBytes = 2 * kTileBytes;    // K + V
  static constexpr int kRowsPerKB = 1024 / kRowBytes;      // rows per wave load (1 KB)
  static constexpr int kChunks = kTileBytes / 1024;        // 1 KB chunks per tile
};

// K tile: block b of row r is stored at block b ^ (r mod kBlk), so the lanes
// that read one block of consecutive rows hit distinct banks.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  return r & (Geo<D>::kBlk - 1);
}
// V tile: the transposing read takes 4 consecutive rows x 2 adjacent blocks per
// 16 lanes (4 blocks per 32 lanes); placing consecutive rows 4 blocks apart
// keeps those (row, block) pairs on distinct banks.
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  return (4 * (r & 3) + ((r >> 2) & 3)) & (Geo<D>::kBlk - 1);
}
template <int D>
__device__ __forceinline__ uint32_t k_off(int r, int blk) {
  return (uint32_t)(r * Geo<D>::kRowBytes + ((blk ^ k_swz<D>(r)) << 4));
}
template <int D>
__device__ __forceinline__ uint32_t v_off(int r, int blk) {
  return (uint32_t)(r * Geo<D>::kRowBytes + ((blk ^ v_swz<D>(r)) << 4));
}

// 16 bytes per lane from global memory straight into LDS: the wave writes 1 KB
// at `lds_chunk` (a wave-uniform address) in lane order.  The builtin exists
// only in the device compilation pass.
__device__ __forceinline__ void load_lds16(const void* g, void* lds_chunk) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (CA_LDS void*)lds_chunk, 16, 0, 0);
#endif
}

// The same load written as inline assembly.  After the builtin the compiler
// makes every later LDS read wait for the load (it cannot tell the target
// apart from what is read); it does not count these, so a kernel that uses
// them waits itself (wait_vmem, wait_vmem_le) before it reads the tile.  The
// block saves and restores M0, inserts the five wait states an M0 write (or a
// base SGPR written by a vector instruction just before) needs ahead of an
// LDS DMA, and clobbers memory so that no memory access moves across it.
// Device pass only.
__device__ __forceinline__ void load_lds16_async(const void* g, void* lds_chunk) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = (uint32_t)(uintptr_t)(CA_LDS void*)lds_chunk;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(m0)
      : "memory");
#endif
}
// With a wave-uniform base address (SGPRs) plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void load_lds16_async(const void* sbase, uint32_t voff,
                                                 void* lds_chunk) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t m0 = (uint32_t)(uintptr_t)(CA_LDS void*)lds_chunk;
  // The base is wave-uniform; make that explicit so it lives in SGPRs.  The
  // builtin works on int: both halves are zero-extended back explicitly.
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sb), "s"(m0)
      : "memory");
#endif
}

// The value held by lane (l ^ 32): the other half of the wave, which holds the
// other 32 keys of the same query row.  (ds_bpermute; the compiler used here
// folds the two results of a same-operand v_permlane32_swap into one, which
// would drop the other half.)
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32); }

// Lane exchanges on the vector ALU.  v_permlane16_swap trades the odd 16-lane
// rows of its first operand with the even rows of its second (in each pair of
// rows); v_permlane32_swap the upper half of the first with the lower half of
// the second.  Unlike a ds_bpermute they do not go through the LDS pipe, whose
// queue the other waves' LDS traffic keeps long.  Written as asm with both
// operands read and written (the compiler used here returns the first result
// of the corresponding builtin in place of the second); the nops cover the
// wait states after a VALU write of an operand and before a VALU read of a
// result.
__device__ __forceinline__ void swap_rows16(uint32_t& a, uint32_t& b) {
  asm("s_nop 4\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 2" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_halves32(uint32_t& a, uint32_t& b) {
  asm("s_nop 4\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 2" : "+v"(a), "+v"(b));
}

// x + (x of lane l ^ 16) and x + (x of lane l ^ 32): after a swap of x with a
// copy of itself each lane holds its own x and its partner's, in an order that
// does not change an fp32 sum.
__device__ __forceinline__ float sum_xor16(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_rows16(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float sum_xor32(float x) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  swap_halves32(a, b);
  return __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b);
}

// s_waitcnt vmcnt(0): every global load of this wave (including the ones that
// write LDS directly) has completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): at most N of this wave's global loads are still in
// flight.  A wave's loads complete in the order they were issued.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier that leaves in-flight global->LDS loads alone (unlike
// __syncthreads, whose release fence waits for every outstanding global load).
// LDS operations of this wave complete first (lgkmcnt(0)); loads whose data the
// barrier must publish are waited for explicitly with wait_vmem().  The signal
// fences keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

struct NoMask {
  static constexpr bool value = false;
};
template <int B>
struct Buf {
  static constexpr int value = B;
};
struct Mask {
  static constexpr bool value = true;
};

// Marks a work item whose main pass left fp32's range (either kernel's): a
// quiet NaN in the first element of its first query row (the output of finite
// inputs is finite).
template <typename T>
__device__ __forceinline__ T overflow_marker() {
  return __builtin_bit_cast(T, std::conditional_t<sizeof(T) == 2, uint16_t, uint32_t>(
                                   sizeof(T) == 2 ? 0x7FC0u : 0x7FC00000u));
}

// LDS bytes of the synchronous schedule: two K/V tile buffers.
template <int D>
constexpr uint32_t kSyncLdsBytes = 2 * Geo<D>::kBufBytes;

// One work item with the synchronous schedule: every wave of the workgroup
// computes S, the softmax and P.V of the same tile, one barrier per tile.
// K/V tiles are double buffered in LDS.  kFixed selects the fixed-maximum softmax (see the file header);
// without it the running maximum is used and the result is always final.
template <int D, typename T, int W, bool kFixed>
__device__ __forceinline__ void attn_item_sync(const KernelArgs& a, const Item& it,
                                               unsigned char* smem) {
  using G = Geo<D>;
  constexpr int kCpw = G::kChunks / W;  // 1 KB load chunks per wave per matrix
  static_assert(sizeof(T) == 2, "bf16 storage (fp32 calls run attn_f32.h)");
  static_assert(kCpw * W == G::kChunks, "tile split across waves");

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;  // lane half

  const int pred = it.pred_rows;
  const int total = pred + it.own_rows;
  const int n_tiles = (total + kBN - 1) / kBN;
  const int64_t rs = a.row_stride;

  const int64_t e = a.entry(it.b);  // physical entry (slot) of this chunk
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

  // ---- Q fragment: B operand of S^T = K.Q^T, one query row per lane column
  const int qrow = it.q0 + wave * 32 + l32;
  const bool qvalid = wave * 32 + l32 < it.q_rows;
  u32x4_t qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (qvalid)
      qf[ks] = Io<T>::load8(qb + qrow * rs + ks * 16 + hh * 8);
    else
      qf[ks] = u32x4_t{0u, 0u, 0u, 0u};
  }

  // ---- per-lane load map: LDS chunk c = wave*kCpw + i receives, at byte
  // c*1024 + lane*16, tile row r = c*kRowsPerKB + lane/kBlk and physical block
  // lane%kBlk, i.e. logical block (lane%kBlk) ^ swizzle(r).
  auto lrow = [&](int i) __attribute__((always_inline)) { return (wave * kCpw + i) * G::kRowsPerKB + lane / G::kBlk; };
  uint32_t koffs[kCpw], voffs[kCpw];  // byte offsets within a one-segment tile
#pragma unroll
  for (int i = 0; i < kCpw; ++i) {
    const int r = lrow(i);
    const int pb = lane % G::kBlk;
    koffs[i] = (uint32_t)((r * rs + ((pb ^ k_swz<D>(r)) * 8)) * sizeof(T));
    voffs[i] = (uint32_t)((r * rs + ((pb ^ v_swz<D>(r)) * 8)) * sizeof(T));
  }

  // Issues the loads of tile t into LDS buffer `buf`.
  auto load_tile = [&](int t, unsigned char* kb) __attribute__((always_inline)) {
    unsigned char* vb = kb + G::kTileBytes;
    const int r0 = t * kBN;
    if (r0 + kBN <= pred || (r0 >= pred && r0 + kBN <= total)) {
      // whole tile in one segment: uniform base + fixed per-lane offsets
      const bool in_pred = r0 + kBN <= pred;
      const int64_t row = in_pred ? r0 : r0 - pred;
      const char* kbase = reinterpret_cast<const char*>((in_pred ? kpre : kown) + row * rs);
      const char* vbase = reinterpret_cast<const char*>((in_pred ? vpre : vown) + row * rs);
#pragma unroll
      for (int i = 0; i < kCpw; ++i) {
        const int c = wave * kCpw + i;
        load_lds16(kbase + koffs[i], kb + c * 1024);
        load_lds16(vbase + voffs[i], vb + c * 1024);
      }
    } else {
      // straddling or ragged tile: per-lane row select; rows past the end
      // re-read the last row (their scores are masked, their P is zero)
#pragma unroll
      for (int i = 0; i < kCpw; ++i) {
        const int c = wave * kCpw + i;
        const int r = lrow(i);
        int j = r0 + r;
        j = j < total ? j : total - 1;
        const int pb = lane % G::kBlk;
        const int kblk = pb ^ k_swz<D>(r);
        const int vblk = pb ^ v_swz<D>(r);
        const T* kr = j < pred ? kpre + j * rs : kown + (j - pred) * rs;
        const T* vr = j < pred ? vpre + j * rs : vown + (j - pred) * rs;
        load_lds16(kr + kblk * 8, kb + c * 1024);
        load_lds16(vr + vblk * 8, vb + c * 1024);
      }
    }
  };

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -__builtin_inff();  // running max, log2 domain (score * scale * log2 e)
  float l4[4] = {0.f, 0.f, 0.f, 0.f};  // this lane half's share of the denominator
  const float s2 = a.scale_log2;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Per-lane LDS byte offsets; everything else in an address is an immediate.
  // K read for k-step ks and key block kb2: row 32*kb2 + l32, logical block
  // 2*ks + hh.  With x = l32 & (kBlk-1) the swizzled block is
  // 2*(ks ^ (x>>1)) + (hh ^ (x&1)), so only ks ^ (x>>1) varies per lane.
  constexpr int kKs = D / 16;
  uint32_t koff_lds[kKs];
  {
    const int x = l32 & (G::kBlk - 1);
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks)
      koff_lds[ks] = (uint32_t)(l32 * G::kRowBytes +
                                ((2 * (ks ^ (x >> 1)) + (hh ^ (x & 1))) << 4));
  }
  // V transposing reads for d-block db and lo/hi half w: row 16s + 4hh + j/4 + 8w
  // (s only shifts the row by 16, which leaves the swizzle unchanged), column
  // block 4db + 2g1 + (j&3)/2, 8-byte half j&1.
  constexpr int kDb = D / 32;
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

  // One tile: S^T, online softmax, O^T update.  kBuf: LDS buffer (compile-time
  // so that it folds into the immediate offsets).  Mask: keys >= total are out.
  auto compute = [&](int t, const unsigned char* buf, auto mask_tag) __attribute__((always_inline)) {
    constexpr bool kMask = decltype(mask_tag)::value;
    constexpr uint32_t kKBase = 0;
    constexpr uint32_t kVBase = G::kTileBytes;
    const CA_LDS unsigned char* lds = (const CA_LDS unsigned char*)buf;

    f32x16_t sacc[kBN / 32];
#pragma unroll
    for (int kb2 = 0; kb2 < kBN / 32; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb2][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kKs; ++ks) {
#pragma unroll
      for (int kb2 = 0; kb2 < kBN / 32; ++kb2) {
        const u32x4_t kv = *(CA_LDS const u32x4_t*)(lds + koff_lds[ks] +
                                                   (kKBase + kb2 * 32 * G::kRowBytes));
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, kv), __builtin_bit_cast(bf16x8_t, qf[ks]), sacc[kb2],
            0, 0, 0);
      }
    }

    if constexpr (kMask) {
#pragma unroll
      for (int kb2 = 0; kb2 < kBN / 32; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t * kBN + kb2 * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= total) sacc[kb2][i] = -__builtin_inff();
        }
    }

    // tile max over this lane's 32 scores (a balanced tree).  The two lane
    // halves hold the other 32 keys of the same rows and exchange their maxima
    // whenever m is set.
    auto tile_max = [&]() __attribute__((always_inline)) {
      float t8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kb2 = i >> 2, j = (i & 3) * 4;
        t8[i] = fmaxf(fmaxf(sacc[kb2][j], sacc[kb2][j + 1]),
                      fmaxf(sacc[kb2][j + 2], sacc[kb2][j + 3]));
      }
      return fmaxf(fmaxf(fmaxf(t8[0], t8[1]), fmaxf(t8[2], t8[3])),
                   fmaxf(fmaxf(t8[4], t8[5]), fmaxf(t8[6], t8[7])));
    };
    if constexpr (kFixed) {
      // m from the first tile (which always holds valid keys); O and l are
      // still zero there, so nothing is rescaled.
      if (t == 0) {
        const float mx = tile_max();
        m_run = fmaxf(mx, other_half(mx)) * s2;
      }
    } else {
      // each lane tests its own half against the running max; only when some
      // lane exceeds it by 2^8 do the halves agree on a new m together
      const float mx = tile_max();
      if (__builtin_amdgcn_ballot_w64(mx * s2 > m_run + kRescaleLog2) != 0) {
        const float m_new = fmaxf(m_run, fmaxf(mx, other_half(mx)) * s2);
        const float alpha =
            m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) l4[i] *= alpha;
#pragma unroll
        for (int db = 0; db < kDb; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
    }

    uint32_t pk[kBN / 32][8];
#pragma unroll
    for (int kb2 = 0; kb2 < kBN / 32; ++kb2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][2 * i], s2, -m_run));
        float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb2][2 * i + 1], s2, -m_run));
        if constexpr (kMask) {
          const int key0 = t * kBN + kb2 * 32 + 8 * ((2 * i) >> 2) + 4 * hh + ((2 * i) & 3);
          if (key0 >= total) p0 = 0.f;
          if (key0 + 1 >= total) p1 = 0.f;
        }
        pk[kb2][i] = pack_bf16(p0, p1);
        const int acc = (kb2 * 8 + i) & 3;  // four independent partial sums
        l4[acc] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[kb2][i]), ones,
                                                  l4[acc], false);
      }
    }

    // O^T += V^T . P^T, 16 keys per step.  Lane (group g = lane/16, j = lane%16)
    // addresses row 16s + 4hh + j/4 (and +8), columns 32db + 16(g&1) + 4(j&3)..+3;
    // the transposing read hands lane j those 4 rows at its own column
    // 32db + 16(g&1) + j, which are the keys its P^T operand holds.
#pragma unroll
    for (int s = 0; s < kBN / 16; ++s) {
      const u32x4_t pb = {pk[s >> 1][(s & 1) * 4 + 0], pk[s >> 1][(s & 1) * 4 + 1],
                          pk[s >> 1][(s & 1) * 4 + 2], pk[s >> 1][(s & 1) * 4 + 3]};
#pragma unroll
      for (int db = 0; db < kDb; ++db) {
        const uint32_t imm = kVBase + 16 * s * G::kRowBytes;
        const i16x4_t lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((CA_LDS i16x4_t*)(lds + voff_lds[db][0] + imm));
        const i16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((CA_LDS i16x4_t*)(lds + voff_lds[db][1] + imm));
        const u32x2_t lo2 = __builtin_bit_cast(u32x2_t, lo);
        const u32x2_t hi2 = __builtin_bit_cast(u32x2_t, hi);
        const u32x4_t va = {lo2[0], lo2[1], hi2[0], hi2[1]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                           __builtin_bit_cast(bf16x8_t, pb),
                                                           oacc[db], 0, 0, 0);
      }
    }
  };

  // One pipeline step: start loading tile t+1 into the other buffer, compute
  // tile t, then wait for the loads and synchronise the workgroup.  The two
  // buffers are restrict pointers: the compiler then knows that the LDS reads
  // of tile t do not touch the buffer being filled, and does not make them
  // wait for those loads.
  auto step = [&](int t, unsigned char* __restrict__ cur, unsigned char* __restrict__ nxt,
                  auto mask_tag) __attribute__((always_inline)) {
    if (t + 1 < n_tiles) load_tile(t + 1, nxt);
    compute(t, cur, mask_tag);
    wait_vmem();
    wg_barrier();
  };
  unsigned char* const buf0 = smem;
  unsigned char* const buf1 = smem + G::kBufBytes;

  load_tile(0, buf0);
  wait_vmem();
  wg_barrier();
  // full tiles in pairs (buffer 0, buffer 1), so every buffer address is a
  // constant
  const int n_full = total / kBN;
  int t = 0;
  for (; t + 2 <= n_full; t += 2) {
    step(t, buf0, buf1, NoMask{});
    step(t + 1, buf1, buf0, NoMask{});
  }
  if (t < n_full) {
    step(t, buf0, buf1, NoMask{});
    ++t;
  }
  // the ragged last tile, if any
  if (t < n_tiles) {
    if (t & 1)
      step(t, buf1, buf0, Mask{});
    else
      step(t, buf0, buf1, Mask{});
  }

  // ---- epilogue: (fixed m) overflow check over the workgroup, then
  // normalise and store this lane's query row
  const float l_half = (l4[0] + l4[1]) + (l4[2] + l4[3]);
  if constexpr (kFixed) {
    float acc = l_half;
#pragma unroll
    for (int db = 0; db < kDb; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc += oacc[db][i];
    if (__syncthreads_or(!__builtin_isfinite(acc))) {
      if (tid == 0)
        static_cast<T*>(a.o)[e * a.o_bstride + (int64_t)it.q0 * rs + (int64_t)it.h * D] =
            overflow_marker<T>();
      return;
    }
  }
  const float l_tot = l_half + other_half(l_half);
  const float inv = 1.0f / l_tot;
  if (qvalid) {
    T* ob = static_cast<T*>(a.o) + e * a.o_bstride + (int64_t)qrow * rs + (int64_t)it.h * D;
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

// Main pass: one work item per workgroup, fixed-maximum softmax.
template <int D, typename T, int W>
__global__ __launch_bounds__(W * 64, 8 / W) void chunk_attn_fwd(KernelArgs a) {
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const Item it = decode(a.plan, plan_slot_work(a.plan, blockIdx.x));
  attn_item_sync<D, T, W, true>(a, it, smem);
}

// Range recheck after the main pass.  Workgroup g takes a contiguous share of
// the work items (ceil(n_items / gridDim.x) of them), tests their overflow
// markers (the first output element of each item) one item per thread, and
// recomputes the items it found marked, one after the other, with the running
// maximum.  With two workgroups per CU the test costs one load per item,
// spread over the chip, and a launch whose items all overflowed still
// recomputes them on every CU.
template <int D, typename T, int W>
__global__ __launch_bounds__(W * 64, 8 / W) void chunk_attn_recheck(KernelArgs a) {
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
      const T first = static_cast<const T*>(a.o)[a.entry(it.b) * a.o_bstride +
                                                  (int64_t)it.q0 * a.row_stride +
                                                  (int64_t)it.h * D];
      if (__builtin_isnan((float)first)) marked[atomicAdd(&n_marked, 1)] = (int)threadIdx.x;
    }
    __syncthreads();
    const int m = n_marked;
    for (int i = 0; i < m; ++i) {
      attn_item_sync<D, T, W, false>(a, decode(a.plan, base + marked[i]), smem);
      __syncthreads();
    }
  }
}

// Zeroes the n claim words of a work queue (one thread per word), launched on
// the stream of the persistent main pass just before it.  A kernel rather than
// a memset, so that it can sit in a captured graph and repeats on every
// replay; and because every launch starts from cleared words, no earlier
// launch has to leave them clean.
__global__ void queue_clear(unsigned long long* words, int n) {
  if ((int)threadIdx.x < n) words[threadIdx.x] = 0ull;
}

// Writes the decoded work item of every workgroup slot (7 ints each), using
// the same plan_slot_work/decode as the attention kernel.
__global__ void plan_dump(Plan p, int* out, int64_t cap) {
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= p.n_items || slot >= cap) return;
  const Item it = decode(p, plan_slot_work(p, slot));
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
