// C-ABI entry points of the chunk-attention library (declared in
// include/chunkattn.h): argument validation, the integer launch plan and the
// kernel launch.  No allocation happens on the hot calls.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "attn_f32.h"
#include "attn_kernel.h"
#include "attn_pingpong.h"
#include "attn_wide.h"
#include "chunkattn.h"
#include "fifo.h"
#include "mfma_probe.h"
#include "noise.h"

// Work-queue slots of a context.  A slot is kQueueWords 64-bit words (one
// claim word per die), cleared by a kernel on the call's stream right before
// the persistent main pass (256- or 384-row items) that uses it.  Eager calls
// take the next of kQueueSlots slots in turn, so up to kQueueSlots of them may
// be in flight on different streams at once.  A call made while its stream is
// being captured into a graph takes a slot of its own from the next
// kCaptureSlots, never used again by another call of the context: the graph
// keeps that slot for all its replays, and eager calls or other graphs cannot
// land on it.
constexpr int kQueueSlots = 64;
constexpr int kCaptureSlots = 448;
constexpr int kQueueWords = 16;

// Scratch of chunkattn_queue_step_noalloc: one work-queue slot (16 claim words,
// 128 bytes) in a static device array, so that entry point needs no memory
// from the context.  Each device the library runs on holds its own copy until
// the process ends.  In host code `scratch` only stands in for the symbol and
// is never passed to a kernel: chunkattn_create looks up the array's device
// address with hipGetSymbolAddress (the device current) and the context keeps
// it; kernels and the clearing kernel get that address.  Every noalloc call on
// a device shares the array, so such calls must not overlap on one device.
constexpr int kStaticScratchWords = 16;
static __device__ __align__(256) unsigned long long scratch[kStaticScratchWords];

struct chunkattn_ctx {
  int device = 0;
  int n_cu = 0;
  int n_xcd = 1;
  // query rows per work item: 128, 256 or 384 (fixed by the flags), or 0 for
  // the default (call_block_rows)
  int block_rows = 0;
  // 384-row query blocks per work item: 0 = chosen per call (item_blocks)
  int item_blocks = 0;
  // scores scaled in fp32 (CHUNKATTN_FLAG_EXACT_SCALE)
  bool exact_scale = false;
  // key-axis split of the last items: items -1 = chosen per call, 0 = off,
  // > 0 = that many items into `split_parts` parts
  int split_items = -1;
  int split_parts = 0;
  // stream-ordered pool of the split workspaces (created on first use)
  hipMemPool_t split_pool = nullptr;
  std::mutex split_pool_mu;
  // device, (kQueueSlots + kCaptureSlots) * kQueueWords words
  unsigned long long* queue = nullptr;
  // device address of this device's `scratch` array (noalloc entry point)
  unsigned long long* static_scratch = nullptr;
  std::atomic<unsigned> next_slot{0};
  std::atomic<unsigned> next_capture{0};
  std::string arch;
  std::string err;
};

namespace {

using chunkattn::KernelArgs;
using chunkattn::Plan;

constexpr int kMinBlockRows = 128;  // smallest bf16 work item (4 waves); bounds the grid

// Smallest work item of a call of this dtype (fp32 calls: 64 rows).
int min_block_rows(int dtype) {
  return dtype == CHUNKATTN_F32 ? chunkattn::kF32BlockRows : kMinBlockRows;
}

// The 384-row kernel exists for bf16 storage and head_dim 128 only.
bool wide_supported(int head_dim, int dtype) { return head_dim == 128 && dtype == CHUNKATTN_BF16; }

// Query rows per work item of one call.  fp32 calls always run the fp32
// kernel (64-row items).  For bf16 calls, contexts of 128 or 256 rows use that
// size; the default context (and a 384-row one) uses 384-row items where the
// 384-row kernel exists (head_dim 128) and 256-row items otherwise.
int call_block_rows(const chunkattn_ctx* ctx, int head_dim, int dtype) {
  if (dtype == CHUNKATTN_F32) return chunkattn::kF32BlockRows;
  if (ctx->block_rows == 128 || ctx->block_rows == 256) return ctx->block_rows;
  // exact-scale contexts: the 256-row pass rounds the scaled Q to bf16
  return wide_supported(head_dim, dtype) ? 384 : ctx->exact_scale ? 128 : 256;
}

thread_local std::string g_thread_err;

constexpr int kMaxSplitParts = 8;

// Key-axis split of the last items of a launch with one 384-row block per
// item: {items, parts}, {0, 0} for none.  When a launch has few items per CU
// (fewer than 8), the last wave of items decides when it ends: the last long
// items (plan_with_split) are cut along their keys, so the end of the launch is
// made of part items.  Below 3 items per CU, 2/3 n_cu items into 2 parts; from
// 3 to 7, n_cu items into 4 parts (measured best of 1/2..2.7 n_cu items and 2,
// 3, 4 and 8 parts on the 5-head and 12-head 480p queues).  Every part walks
// at least one key tile.
struct SplitChoice {
  int64_t items;
  int parts;
};
SplitChoice split_choice(const chunkattn_ctx* ctx, const Plan& p) {
  if (ctx->split_items == 0 || p.n_items == 0) return {0, 0};
  int min_keys = 0x7fffffff;
  for (int b = 0; b < p.n_batch; ++b) {
    const int keys =
        (b >= p.first_pred ? p.lpred : 0) + (b == p.n_batch - 1 ? p.lown_last : p.lown);
    min_keys = keys < min_keys ? keys : min_keys;
  }
  const int min_tiles = (min_keys + chunkattn::kBN - 1) / chunkattn::kBN;
  int64_t items;
  int parts;
  if (ctx->split_items > 0) {
    items = ctx->split_items;
    parts = ctx->split_parts;
  } else {
    const int64_t per_cu = p.n_items / (ctx->n_cu > 0 ? ctx->n_cu : 1);
    if (per_cu >= 8) return {0, 0};
    items = per_cu < 3 ? ctx->n_cu * 2 / 3 : ctx->n_cu;
    parts = per_cu < 3 ? 2 : 4;
  }
  if (parts > min_tiles) parts = min_tiles;
  if (parts < 2) return {0, 0};
  return {items < p.n_items ? items : p.n_items, parts};
}

constexpr int kMaxItemBlocks = 8;

// 384-row query blocks per work item of a call with 384-row blocks.  A short
// key walk (cross-attention over a few hundred text tokens: 8 tiles) costs
// per item about as much as its tiles (claim, Q load, pipeline fill and
// drain, final stores); an item of several blocks of one (chunk, head) pays
// that once.  Chosen: enough blocks for about 48 key tiles per item, while the
// launch keeps at least 4 items per CU, and one block where an item walks a
// single key tile.  A context's fixed setting (1..8) overrides the choice.
int item_blocks(const chunkattn_ctx* ctx, const Plan& p) {
  if (ctx->item_blocks > 0) return ctx->item_blocks;
  int min_keys = 0x7fffffff, max_keys = 0;
  for (int b = 0; b < p.n_batch; ++b) {
    const int keys =
        (b >= p.first_pred ? p.lpred : 0) + (b == p.n_batch - 1 ? p.lown_last : p.lown);
    min_keys = keys < min_keys ? keys : min_keys;
    max_keys = keys > max_keys ? keys : max_keys;
  }
  if (p.n_batch == 0 || min_keys <= chunkattn::kBN) return 1;
  const int t_max = (max_keys + chunkattn::kBN - 1) / chunkattn::kBN;
  int g = (48 + t_max - 1) / t_max;
  g = g < kMaxItemBlocks ? g : kMaxItemBlocks;
  for (; g > 1; --g) {
    const Plan q = chunkattn::make_plan(p.n_batch, p.first_pred, p.heads, p.lq, p.lown, p.lpred,
                                        g * p.bm, p.n_xcd, p.lq_last, p.lown_last);
    if (q.n_items >= 4 * (int64_t)ctx->n_cu) break;
  }
  return g;
}

int set_err(std::string* sink, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (sink) *sink = buf;
  return code;
}

size_t elem_size(int dtype) { return dtype == CHUNKATTN_F32 ? 4 : 2; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

int check_common(std::string* err, int heads, int head_dim, float scale, int dtype) {
  if (dtype != CHUNKATTN_BF16 && dtype != CHUNKATTN_F32)
    return set_err(err, CHUNKATTN_EUNSUPPORTED, "dtype %d is not CHUNKATTN_BF16 or CHUNKATTN_F32",
                   dtype);
  if (head_dim != 64 && head_dim != 128)
    return set_err(err, CHUNKATTN_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (heads < 1) return set_err(err, CHUNKATTN_EINVAL, "heads must be >= 1 (got %d)", heads);
  if (!std::isfinite(scale) || scale < 0.f)
    return set_err(err, CHUNKATTN_EINVAL, "scale must be finite and >= 0 (got %g)",
                   (double)scale);
  return CHUNKATTN_OK;
}

// Largest element count accepted for one tensor: keeps every byte offset well
// inside int64 and every row index of the kernel inside int32.
constexpr long double kMaxElems = 4.0e18L;

// The kernels address the rows of one 64-row key/value tile by 32-bit
// per-lane byte offsets from the tile's first row (up to 63 rows of
// heads * head_dim elements, plus the row itself): they must stay below 2^32.
bool tile_offsets_fit(int heads, int head_dim, int dtype) {
  const long double span = 64.0L * heads * head_dim * elem_size(dtype);
  return span < 4294967296.0L;
}

// Queue step (window = false) and window step (window = true: out holds two
// chunks' rows per window, a work item walks up to 3 * chunk_len key rows).
int validate_queue(std::string* err, const void* q, const void* k, const void* v,
                   const void* kv_cache, const void* out, int L, int n, int heads, int head_dim,
                   float scale, int dtype, bool window = false) {
  int rc = check_common(err, heads, head_dim, scale, dtype);
  if (rc) return rc;
  if (L < 0 || n < 0)
    return set_err(err, CHUNKATTN_EINVAL, "chunk_len (%d) and n_chunks (%d) must be >= 0", L, n);
  if (L == 0 || n == 0) return CHUNKATTN_OK;
  const int max_log2 = window ? 29 : 30;
  if (L > (1 << max_log2))
    return set_err(err, CHUNKATTN_EUNSUPPORTED, "chunk_len %d too large (max 2^%d)", L, max_log2);
  const long double elems = (long double)n * L * heads * head_dim;
  if (elems * 2 > kMaxElems)
    return set_err(err, CHUNKATTN_EINVAL, "tensor size overflows 64-bit offsets");
  if ((long double)heads * head_dim > 2147483647.0L)
    return set_err(err, CHUNKATTN_EINVAL, "heads * head_dim overflows int32");
  if (!tile_offsets_fit(heads, head_dim, dtype))
    return set_err(err, CHUNKATTN_EUNSUPPORTED,
                   "heads * head_dim too large: a 64-row key/value tile must span under 4 GiB");
  if (!q || !k || !v || !out)
    return set_err(err, CHUNKATTN_EINVAL, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (kv_cache && !aligned16(kv_cache)))
    return set_err(err, CHUNKATTN_EINVAL, "tensor pointers must be 16-byte aligned");
  const size_t bytes = (size_t)elems * elem_size(dtype);
  const size_t obytes = window ? 2 * bytes : bytes;
  if (overlaps(out, obytes, q, bytes) || overlaps(out, obytes, k, bytes) ||
      overlaps(out, obytes, v, bytes) || (kv_cache && overlaps(out, obytes, kv_cache, 2 * bytes)))
    return set_err(err, CHUNKATTN_EINVAL, "out overlaps an input tensor");
  const long double q_rows = window ? 2.0L * L : (long double)L;
  const long double items =
      (long double)n * heads *
      ((long long)((q_rows + min_block_rows(dtype) - 1) / min_block_rows(dtype)));
  if (items > 2147483647.0L)
    return set_err(err, CHUNKATTN_EUNSUPPORTED, "too many work items for one launch");
  return CHUNKATTN_OK;
}

int validate_ring(std::string* err, const void* q, const void* k, const void* v,
                  const void* out, int slots, int tail_slot, int n_live, int L, int heads,
                  int head_dim, float scale, int dtype) {
  if (slots < 1) return set_err(err, CHUNKATTN_EINVAL, "slots must be >= 1 (got %d)", slots);
  if (n_live < 0 || n_live > slots)
    return set_err(err, CHUNKATTN_EINVAL, "n_live must be in [0, slots] (got %d of %d)", n_live,
                   slots);
  if (tail_slot < 0 || tail_slot >= slots)
    return set_err(err, CHUNKATTN_EINVAL, "tail_slot must be in [0, slots) (got %d of %d)",
                   tail_slot, slots);
  // the ring buffers hold `slots` chunks each
  return validate_queue(err, q, k, v, nullptr, out, L, n_live == 0 ? 0 : slots, heads,
                        head_dim, scale, dtype);
}

int validate_full(std::string* err, const void* q, const void* k, const void* v,
                  const void* out, int batch, int lq, int lkv, long long kv_stride, int heads,
                  int head_dim, float scale, int dtype) {
  int rc = check_common(err, heads, head_dim, scale, dtype);
  if (rc) return rc;
  if (batch < 0 || lq < 0)
    return set_err(err, CHUNKATTN_EINVAL, "batch (%d) and lq (%d) must be >= 0", batch, lq);
  if (kv_stride < 0)
    return set_err(err, CHUNKATTN_EINVAL, "kv_batch_stride must be >= 0 (got %lld)", kv_stride);
  if (batch == 0 || lq == 0) return CHUNKATTN_OK;
  if (lkv < 1)
    return set_err(err, CHUNKATTN_EINVAL, "lkv must be >= 1: attention over no keys (got %d)",
                   lkv);
  if (lq > (1 << 30) || lkv > (1 << 30))
    return set_err(err, CHUNKATTN_EUNSUPPORTED, "lq/lkv too large (max 2^30)");
  const long double row = (long double)heads * head_dim;
  const long double qel = (long double)batch * lq * row;
  const long double kvel = (long double)(batch - 1) * kv_stride + (long double)lkv * row;
  if (qel > kMaxElems || kvel > kMaxElems)
    return set_err(err, CHUNKATTN_EINVAL, "tensor size overflows 64-bit offsets");
  if (row > 2147483647.0L)
    return set_err(err, CHUNKATTN_EINVAL, "heads * head_dim overflows int32");
  if (!tile_offsets_fit(heads, head_dim, dtype))
    return set_err(err, CHUNKATTN_EUNSUPPORTED,
                   "heads * head_dim too large: a 64-row key/value tile must span under 4 GiB");
  if (!q || !k || !v || !out)
    return set_err(err, CHUNKATTN_EINVAL, "q, k, v and out must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      ((kv_stride * (long long)elem_size(dtype)) & 15))
    return set_err(err, CHUNKATTN_EINVAL,
                   "tensor pointers and the K/V batch stride must be 16-byte aligned");
  const size_t es = elem_size(dtype);
  const size_t qb = (size_t)qel * es, kb = (size_t)kvel * es;
  if (overlaps(out, qb, q, qb) || overlaps(out, qb, k, kb) || overlaps(out, qb, v, kb))
    return set_err(err, CHUNKATTN_EINVAL, "out overlaps an input tensor");
  const long double items =
      (long double)batch * heads * ((lq + min_block_rows(dtype) - 1) / min_block_rows(dtype));
  if (items > 2147483647.0L)
    return set_err(err, CHUNKATTN_EUNSUPPORTED, "too many work items for one launch");
  return CHUNKATTN_OK;
}

}  // namespace

// Every kernel configuration the host can launch, instantiated explicitly.
namespace chunkattn {
template __global__ void chunk_attn_fwd_pingpong<128, __bf16>(KernelArgs);
template __global__ void chunk_attn_fwd_pingpong<64, __bf16>(KernelArgs);
template __global__ void chunk_attn_fwd<128, __bf16, 4>(KernelArgs);
template __global__ void chunk_attn_recheck<128, __bf16, 4>(KernelArgs);
template __global__ void chunk_attn_fwd<64, __bf16, 4>(KernelArgs);
template __global__ void chunk_attn_recheck<64, __bf16, 4>(KernelArgs);
template __global__ void chunk_attn_recheck<128, __bf16, 8>(KernelArgs);
template __global__ void chunk_attn_recheck<64, __bf16, 8>(KernelArgs);
template __global__ void chunk_attn_fwd_f32<128>(KernelArgs);
template __global__ void chunk_attn_fwd_f32<64>(KernelArgs);

// The clears before a key-split launch in one kernel: the nq claim words of
// the work-queue slot and the ncnt arrival counters of the split items (one
// launch rather than two; a short launch pays a few microseconds per extra
// kernel).
__global__ void split_launch_clear(unsigned long long* queue, int nq, unsigned* cnt,
                                   int64_t ncnt) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nq) queue[i] = 0ull;
  for (int64_t j = i; j < ncnt; j += (int64_t)gridDim.x * blockDim.x) cnt[j] = 0u;
}
}  // namespace chunkattn

namespace {

// The ping-pong kernel uses more than the default 64 KB of dynamic LDS; the
// limit is raised once per device (bit d of `done` for device d).
template <int D, typename T>
hipError_t allow_pingpong_lds() {
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&chunkattn::chunk_attn_fwd_pingpong<D, T>),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)chunkattn::kPingPongLdsBytes<D>);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// The main pass (W = 8: 256-row work items on the ping-pong schedule, softmax
// without a maximum; W = 4: 128-row items on the synchronous one, fixed
// maximum), then the range recheck (synchronous schedule, running maximum) on
// the same stream.
// W = 8: the main pass is persistent, n_persist workgroups (one per CU) share
// the work items through the work queue a.queue.
// Recheck grid: two workgroups per CU, each testing a contiguous share of the
// work items (fewer if there are fewer items).
dim3 recheck_grid(int64_t n_items, int n_cu) {
  const int64_t g = 2 * (int64_t)(n_cu > 0 ? n_cu : 1);
  return dim3((unsigned)(n_items < g ? (n_items > 0 ? n_items : 1) : g));
}

template <int D, typename T, int W>
hipError_t launch_t(const KernelArgs& a, int n_persist, int n_cu, hipStream_t stream) {
  const dim3 grid((unsigned)a.plan.n_items);
  constexpr uint32_t kLds = chunkattn::kSyncLdsBytes<D>;
  if constexpr (W == 8) {
    if (!a.queue || n_persist < 1 || a.plan.n_xcd > kQueueWords) return hipErrorInvalidValue;
    const hipError_t el = allow_pingpong_lds<D, T>();
    if (el != hipSuccess) return el;
    hipLaunchKernelGGL(chunkattn::queue_clear, dim3(1), dim3(64), 0, stream, a.queue,
                       a.plan.n_xcd);
    const hipError_t ec = hipGetLastError();
    if (ec != hipSuccess) return ec;
    hipLaunchKernelGGL((chunkattn::chunk_attn_fwd_pingpong<D, T>), dim3((unsigned)n_persist),
                       dim3(512),
                       chunkattn::kPingPongLdsBytes<D>, stream, a);
  } else {
    hipLaunchKernelGGL((chunkattn::chunk_attn_fwd<D, T, W>), grid, dim3(64 * W), kLds, stream,
                       a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 check_grid = recheck_grid(a.plan.n_items, n_cu);
  hipLaunchKernelGGL((chunkattn::chunk_attn_recheck<D, T, W>), check_grid, dim3(64 * W), kLds,
                     stream, a);
  return hipGetLastError();
}

template <int W>
hipError_t launch_w(const KernelArgs& a, int n_persist, int n_cu, int head_dim, int dtype,
                    hipStream_t stream) {
  (void)dtype;  // bf16 only: fp32 calls run launch_f32
  if (head_dim == 128) return launch_t<128, __bf16, W>(a, n_persist, n_cu, stream);
  return launch_t<64, __bf16, W>(a, n_persist, n_cu, stream);
}

// fp32 calls: one workgroup of 4 waves per 64-row item, fp32 throughout (no
// work queue, no recheck: the softmax keeps a running maximum).
hipError_t launch_f32(const KernelArgs& a, int head_dim, hipStream_t stream) {
  if (a.plan.n_items < 1) return hipSuccess;
  const dim3 grid((unsigned)a.plan.n_items);
  if (head_dim == 128)
    hipLaunchKernelGGL(chunkattn::chunk_attn_fwd_f32<128>, grid, dim3(256),
                       chunkattn::kF32LdsBytes<128>, stream, a);
  else
    hipLaunchKernelGGL(chunkattn::chunk_attn_fwd_f32<64>, grid, dim3(256),
                       chunkattn::kF32LdsBytes<64>, stream, a);
  return hipGetLastError();
}

// The 384-row main pass (48 rows per wave, persistent like the 256-row one):
// chunk_attn_fwd_wide for items of one block, chunk_attn_fwd_wide_stream for
// items of several; then the recheck (three 128-row items per marked block).
// a: the main pass (work items of one or more 384-row blocks); blocks: the same
// call planned with one block per item, for the recheck.
hipError_t launch_wide(const KernelArgs& a, const KernelArgs& blocks, int n_persist, int n_cu,
                       bool exact, hipStream_t stream) {
  if (!a.queue || n_persist < 1 || a.plan.n_xcd > kQueueWords) return hipErrorInvalidValue;
  if (a.plan.split_parts > 1) {
    const int64_t n = a.plan.split_count;
    hipLaunchKernelGGL(chunkattn::split_launch_clear, dim3((unsigned)((n + 255) / 256)),
                       dim3(256), 0, stream, a.queue, a.plan.n_xcd, a.split_cnt, n);
  } else {
    hipLaunchKernelGGL(chunkattn::queue_clear, dim3(1), dim3(64), 0, stream, a.queue,
                       a.plan.n_xcd);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool multi = a.plan.bm > chunkattn::kWideBlockRows;
  auto kernel = multi ? (exact ? chunkattn::chunk_attn_fwd_wide_stream_exact
                               : chunkattn::chunk_attn_fwd_wide_stream)
                      : (exact ? chunkattn::chunk_attn_fwd_wide_exact : chunkattn::chunk_attn_fwd_wide);
  hipLaunchKernelGGL(kernel, dim3((unsigned)n_persist), dim3(512),
                     chunkattn::kPingPongLdsBytes<128>, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunkattn::chunk_attn_recheck_wide<4>, recheck_grid(blocks.plan.n_items, n_cu),
                     dim3(256), chunkattn::kSyncLdsBytes<128>, stream, blocks);
  return hipGetLastError();
}

hipError_t launch(const KernelArgs& a, const KernelArgs& blocks, int block_rows, int n_persist,
                  int n_cu, int head_dim, int dtype, bool exact, hipStream_t stream) {
  if (block_rows == chunkattn::kF32BlockRows) return launch_f32(a, head_dim, stream);
  if (block_rows == 384) return launch_wide(a, blocks, n_persist, n_cu, exact, stream);
  return block_rows == 128 ? launch_w<4>(a, n_persist, n_cu, head_dim, dtype, stream)
                           : launch_w<8>(a, n_persist, n_cu, head_dim, dtype, stream);
}

hipError_t allow_wide_lds() {
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  for (const void* f : {reinterpret_cast<const void*>(&chunkattn::chunk_attn_fwd_wide),
                        reinterpret_cast<const void*>(&chunkattn::chunk_attn_fwd_wide_stream),
                        reinterpret_cast<const void*>(&chunkattn::chunk_attn_fwd_wide_exact),
                        reinterpret_cast<const void*>(&chunkattn::chunk_attn_fwd_wide_stream_exact)}) {
    e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)chunkattn::kPingPongLdsBytes<128>);
    if (e != hipSuccess) return e;
  }
  done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Makes the context's device current for the duration of a call.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

// The context's pool for split workspaces: device memory, kept by the pool
// between calls (no release threshold), created on first use.
hipError_t split_pool(chunkattn_ctx* ctx) {
  std::lock_guard<std::mutex> lock(ctx->split_pool_mu);
  if (ctx->split_pool) return hipSuccess;
  hipMemPoolProps props = {};
  props.allocType = hipMemAllocationTypePinned;
  props.handleTypes = hipMemHandleTypeNone;
  props.location.type = hipMemLocationTypeDevice;
  props.location.id = ctx->device;
  hipMemPool_t pool = nullptr;
  hipError_t e = hipMemPoolCreate(&pool, &props);
  if (e != hipSuccess) return e;
  uint64_t keep = ~0ull;
  e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
  if (e != hipSuccess) {
    (void)hipMemPoolDestroy(pool);
    return e;
  }
  ctx->split_pool = pool;
  return hipSuccess;
}

// Launches the main pass (and the recheck) of a prepared argument block.
// fixed_queue: NULL = the work-queue slot comes from the context's buffer;
// otherwise the persistent pass uses these kStaticScratchWords words (the
// noalloc entry point's static scratch).
int run(chunkattn_ctx* ctx, const KernelArgs& args, int head_dim, int dtype, void* stream,
        unsigned long long* fixed_queue = nullptr) {
  DeviceGuard g(ctx->device);
  if (!g.ok) return set_err(&ctx->err, CHUNKATTN_EDEVICE, "cannot make device %d current",
                            ctx->device);
  KernelArgs a = args;
  a.queue = nullptr;
  const int bm = a.plan.bm;
  if (bm == 384 && !wide_supported(head_dim, dtype))
    return set_err(&ctx->err, CHUNKATTN_ELAUNCH,
                   "internal: 384-row work items planned for a call without that kernel");
  if (bm >= 256 && fixed_queue) {
    // one claim word per die must fit in the static scratch
    if (a.plan.n_xcd > kStaticScratchWords)
      return set_err(&ctx->err, CHUNKATTN_EUNSUPPORTED,
                     "device has %d dies; the static work queue holds %d claim words",
                     a.plan.n_xcd, kStaticScratchWords);
    a.queue = fixed_queue;
  }
  bool capturing = false;
  if (bm >= 256 && !fixed_queue) {
    // one claim word per die must fit in a slot
    if (a.plan.n_xcd > kQueueWords) a.plan.n_xcd = 1;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cap) != hipSuccess)
      return set_err(&ctx->err, CHUNKATTN_ELAUNCH, "cannot query the stream's capture state");
    capturing = cap == hipStreamCaptureStatusActive;
    unsigned slot;
    if (capturing) {
      const unsigned c = ctx->next_capture.fetch_add(1, std::memory_order_relaxed);
      if (c >= (unsigned)kCaptureSlots) {
        ctx->next_capture.store(kCaptureSlots, std::memory_order_relaxed);
        return set_err(&ctx->err, CHUNKATTN_EUNSUPPORTED,
                       "more than %d calls captured into graphs on one context", kCaptureSlots);
      }
      slot = kQueueSlots + c;
    } else {
      slot = ctx->next_slot.fetch_add(1, std::memory_order_relaxed) % kQueueSlots;
    }
    a.queue = ctx->queue + (size_t)slot * kQueueWords;
  }
  // 384-row blocks: the main pass may take several blocks per work item
  KernelArgs main = a;
  if (bm == 384) {
    const int nb = item_blocks(ctx, a.plan);
    if (nb > 1) {
      const Plan& p = a.plan;
      main.plan = chunkattn::make_plan(p.n_batch, p.first_pred, p.heads, p.lq, p.lown, p.lpred,
                                       nb * bm, p.n_xcd, p.lq_last, p.lown_last);
      if (p.head_major) main.plan = chunkattn::plan_head_major(main.plan);
    }
  }
  // One block per item, few items per CU: cut the last items along the keys.
  // The workspace comes from the context's stream-ordered pool and returns to
  // it after the launch, so calls on other streams get their own.  Not under
  // graph capture and not for the no-allocation entry point.
  void* ws = nullptr;
  if (bm == 384 && main.plan.bm == 384 && !fixed_queue && !capturing) {
    const SplitChoice sc = split_choice(ctx, a.plan);
    if (sc.items > 0) {
      const size_t ws_bytes =
          (size_t)sc.items * sc.parts * chunkattn::kSplitSlotFloats * sizeof(float);
      const size_t cnt_bytes = ((size_t)sc.items * sizeof(unsigned) + 255) & ~(size_t)255;
      if (split_pool(ctx) == hipSuccess &&
          hipMallocFromPoolAsync(&ws, ws_bytes + cnt_bytes, ctx->split_pool,
                                 static_cast<hipStream_t>(stream)) == hipSuccess) {
        main.plan = chunkattn::plan_with_split(main.plan, sc.items, sc.parts);
        main.split_ws = static_cast<float*>(ws);
        main.split_cnt = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + ws_bytes);
      } else {
        ws = nullptr;  // no workspace: run unsplit
        (void)hipGetLastError();
      }
    }
  }
  const int n_persist = (int)(main.plan.n_units < ctx->n_cu ? main.plan.n_units : ctx->n_cu);
  const hipError_t e =
      launch(main, a, bm, n_persist, ctx->n_cu, head_dim, dtype, ctx->exact_scale,
             static_cast<hipStream_t>(stream));
  if (ws) (void)hipFreeAsync(ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return set_err(&ctx->err, CHUNKATTN_ELAUNCH, "kernel launch failed: %s",
                   hipGetErrorString(e));
  ctx->err.clear();
  return CHUNKATTN_OK;
}

// Plan of the window step: entry c = window c, queries = 2L rows starting at
// chunk c (L for the last window), own rows = chunks c and c+1 (L for the
// last), predecessor = chunk c-1 for c >= 1.
Plan window_plan(int L, int n, int heads, int bm, int n_xcd) {
  return chunkattn::make_plan(n, 1, heads, 2 * L, 2 * L, L, bm, n_xcd, L, L);
}

}  // namespace

extern "C" {

int chunkattn_block_rows(void) { return 384; }

int chunkattn_ctx_block_rows(const chunkattn_ctx* ctx) {
  return ctx ? call_block_rows(ctx, 128, CHUNKATTN_BF16) : 0;
}

int chunkattn_ctx_call_block_rows(const chunkattn_ctx* ctx, int head_dim, int dtype) {
  return ctx ? call_block_rows(ctx, head_dim, dtype) : 0;
}

int chunkattn_ctx_set_tail_split(chunkattn_ctx* ctx, int items, int parts) {
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "ctx must be non-NULL");
  if (items < -1 || (items > 0 && (parts < 2 || parts > kMaxSplitParts)))
    return set_err(&ctx->err, CHUNKATTN_EINVAL,
                   "tail split: items %d (-1, 0 or > 0), parts %d (2..%d)", items, parts,
                   kMaxSplitParts);
  ctx->split_items = items;
  ctx->split_parts = items > 0 ? parts : 0;
  ctx->err.clear();
  return CHUNKATTN_OK;
}

int chunkattn_ctx_set_item_blocks(chunkattn_ctx* ctx, int blocks) {
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "ctx must be non-NULL");
  if (blocks < 0 || blocks > kMaxItemBlocks)
    return set_err(&ctx->err, CHUNKATTN_EINVAL, "item blocks %d outside [0, %d]", blocks,
                   kMaxItemBlocks);
  ctx->item_blocks = blocks;
  ctx->err.clear();
  return CHUNKATTN_OK;
}

int chunkattn_create(chunkattn_ctx** out, int device_ordinal, unsigned flags) {
  if (!out) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "out must be non-NULL");
  *out = nullptr;
  const unsigned sizes = CHUNKATTN_FLAG_BLOCK128 | CHUNKATTN_FLAG_BLOCK256 | CHUNKATTN_FLAG_BLOCK384;
  const unsigned size = flags & sizes;
  const bool exact = (flags & CHUNKATTN_FLAG_EXACT_SCALE) != 0;
  if ((flags & ~(sizes | CHUNKATTN_FLAG_EXACT_SCALE)) != 0 || (size & (size - 1)) != 0 ||
      (exact && size == CHUNKATTN_FLAG_BLOCK256))
    return set_err(&g_thread_err, CHUNKATTN_EINVAL, "unknown or conflicting flags 0x%x", flags);
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device_ordinal < 0 || device_ordinal >= count)
    return set_err(&g_thread_err, CHUNKATTN_EDEVICE, "no HIP device %d (found %d)",
                   device_ordinal, count);
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device_ordinal) != hipSuccess)
    return set_err(&g_thread_err, CHUNKATTN_EDEVICE, "cannot query device %d", device_ordinal);
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return set_err(&g_thread_err, CHUNKATTN_EUNSUPPORTED,
                   "device %d is %s; this library is built for gfx950 only", device_ordinal,
                   prop.gcnArchName);
  chunkattn_ctx* ctx = new (std::nothrow) chunkattn_ctx();
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_ENOMEM, "context allocation failed");
  ctx->device = device_ordinal;
  ctx->block_rows = size == CHUNKATTN_FLAG_BLOCK128   ? 128
                    : size == CHUNKATTN_FLAG_BLOCK256 ? 256
                    : size == CHUNKATTN_FLAG_BLOCK384 ? 384
                                                      : 0;
  ctx->exact_scale = exact;
  ctx->n_cu = prop.multiProcessorCount;
  ctx->arch = prop.gcnArchName;
  int xcc = 0;
  if (hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, device_ordinal) ==
          hipSuccess &&
      xcc > 0)
    ctx->n_xcd = xcc;
  if (ctx->block_rows != 128) {
    // the work queues of the persistent main pass (each launch clears its own)
    DeviceGuard g(device_ordinal);
    const size_t bytes =
        sizeof(unsigned long long) * (kQueueSlots + kCaptureSlots) * kQueueWords;
    void* q = nullptr;
    if (!g.ok || hipMalloc(&q, bytes) != hipSuccess) {
      delete ctx;
      return set_err(&g_thread_err, CHUNKATTN_EDEVICE, "device %d: work-queue allocation failed",
                     device_ordinal);
    }
    if (hipMemset(q, 0, bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
      (void)hipFree(q);
      delete ctx;
      return set_err(&g_thread_err, CHUNKATTN_EDEVICE, "device %d: work-queue setup failed",
                     device_ordinal);
    }
    ctx->queue = static_cast<unsigned long long*>(q);
  }
  {
    // the noalloc entry point's static scratch on this device, and the LDS
    // limit of the main kernels, set up once here so that hot calls do
    // neither
    DeviceGuard g(device_ordinal);
    void* p = nullptr;
    const hipError_t es = g.ok ? hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) : hipErrorInvalidDevice;
    if (es != hipSuccess || !p) {
      if (ctx->queue) (void)hipFree(ctx->queue);
      delete ctx;
      return set_err(&g_thread_err, CHUNKATTN_EDEVICE,
                     "device %d: cannot locate the static scratch buffer (%s)", device_ordinal,
                     hipGetErrorString(es));
    }
    ctx->static_scratch = static_cast<unsigned long long*>(p);
    if (allow_wide_lds() != hipSuccess || allow_pingpong_lds<128, __bf16>() != hipSuccess ||
        allow_pingpong_lds<64, __bf16>() != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&chunkattn::chunk_attn_fwd_f32<128>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)chunkattn::kF32LdsBytes<128>) != hipSuccess) {
      if (ctx->queue) (void)hipFree(ctx->queue);
      delete ctx;
      return set_err(&g_thread_err, CHUNKATTN_EDEVICE,
                     "device %d: cannot raise the LDS limit of the main kernels",
                     device_ordinal);
    }
  }
  *out = ctx;
  return CHUNKATTN_OK;
}

int chunkattn_destroy(chunkattn_ctx* ctx) {
  if (ctx && (ctx->queue || ctx->split_pool)) {
    DeviceGuard g(ctx->device);
    if (ctx->queue) (void)hipFree(ctx->queue);
    // released once the last stream-ordered free has run
    if (ctx->split_pool) (void)hipMemPoolDestroy(ctx->split_pool);
  }
  delete ctx;
  return CHUNKATTN_OK;
}

int chunkattn_ctx_xcd_count(const chunkattn_ctx* ctx) { return ctx ? ctx->n_xcd : 0; }

int chunkattn_validate_queue_step(const void* q, const void* k, const void* v,
                                  const void* kv_cache, const void* out, int chunk_len,
                                  int n_chunks, int heads, int head_dim, float scale,
                                  int dtype) {
  g_thread_err.clear();
  return validate_queue(&g_thread_err, q, k, v, kv_cache, out, chunk_len, n_chunks, heads,
                        head_dim, scale, dtype);
}

int chunkattn_validate_full(const void* q, const void* k, const void* v, const void* out,
                            int batch, int lq, int lkv, long long kv_batch_stride, int heads,
                            int head_dim, float scale, int dtype) {
  g_thread_err.clear();
  return validate_full(&g_thread_err, q, k, v, out, batch, lq, lkv, kv_batch_stride, heads,
                       head_dim, scale, dtype);
}

}  // extern "C"

namespace {

// Body of chunkattn_queue_step and chunkattn_queue_step_noalloc
// (fixed_queue: see run()).
int queue_step_impl(chunkattn_ctx* ctx, const void* q, const void* k, const void* v,
                    const void* kv_cache, void* out, int chunk_len, int n_chunks, int heads,
                    int head_dim, float scale, int dtype, void* hip_stream,
                    unsigned long long* fixed_queue) {
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "ctx must be non-NULL");
  int rc = validate_queue(&ctx->err, q, k, v, kv_cache, out, chunk_len, n_chunks, heads,
                          head_dim, scale, dtype);
  if (rc) return rc;
  if (chunk_len == 0 || n_chunks == 0) {
    ctx->err.clear();
    return CHUNKATTN_OK;
  }
  const int64_t per_chunk = (int64_t)chunk_len * heads * head_dim;
  const size_t es = elem_size(dtype);
  KernelArgs a{};  // zero: linear batch entries unless set below
  a.plan = chunkattn::make_plan(n_chunks, 1, heads, chunk_len, chunk_len, chunk_len,
                                call_block_rows(ctx, head_dim, dtype), ctx->n_xcd);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.q_bstride = per_chunk;
  a.o_bstride = per_chunk;
  a.kv_bstride = per_chunk;
  if (kv_cache) {
    a.pk = kv_cache;
    a.pv = static_cast<const unsigned char*>(kv_cache) + (size_t)per_chunk * es;
    a.p_bstride = 2 * per_chunk;
    a.pred_shift = 0;
  } else {
    a.pk = k;
    a.pv = v;
    a.p_bstride = per_chunk;
    a.pred_shift = 1;
  }
  a.row_stride = heads * head_dim;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  return run(ctx, a, head_dim, dtype, hip_stream, fixed_queue);
}

}  // namespace

extern "C" {

int chunkattn_queue_step(chunkattn_ctx* ctx, const void* q, const void* k, const void* v,
                         const void* kv_cache, void* out, int chunk_len, int n_chunks,
                         int heads, int head_dim, float scale, int dtype, void* hip_stream) {
  return queue_step_impl(ctx, q, k, v, kv_cache, out, chunk_len, n_chunks, heads, head_dim,
                         scale, dtype, hip_stream, nullptr);
}

int chunkattn_queue_step_noalloc(chunkattn_ctx* ctx, const void* q, const void* k,
                                 const void* v, const void* kv_cache, void* out, int chunk_len,
                                 int n_chunks, int heads, int head_dim, float scale, int dtype,
                                 void* hip_stream) {
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "ctx must be non-NULL");
  if (!ctx->static_scratch)
    return set_err(&ctx->err, CHUNKATTN_EDEVICE, "no static scratch buffer on device %d",
                   ctx->device);
  return queue_step_impl(ctx, q, k, v, kv_cache, out, chunk_len, n_chunks, heads, head_dim,
                         scale, dtype, hip_stream, ctx->static_scratch);
}

int chunkattn_full(chunkattn_ctx* ctx, const void* q, const void* k, const void* v, void* out,
                   int batch, int lq, int lkv, long long kv_batch_stride, int heads,
                   int head_dim, float scale, int dtype, void* hip_stream) {
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "ctx must be non-NULL");
  int rc = validate_full(&ctx->err, q, k, v, out, batch, lq, lkv, kv_batch_stride, heads,
                         head_dim, scale, dtype);
  if (rc) return rc;
  if (batch == 0 || lq == 0) {
    ctx->err.clear();
    return CHUNKATTN_OK;
  }
  KernelArgs a{};  // zero: linear batch entries unless set below
  a.plan = chunkattn::make_plan(batch, batch, heads, lq, lkv, 0,
                                call_block_rows(ctx, head_dim, dtype), ctx->n_xcd);
  a.q = q;
  a.k = k;
  a.v = v;
  a.pk = nullptr;
  a.pv = nullptr;
  a.o = out;
  a.q_bstride = (int64_t)lq * heads * head_dim;
  a.o_bstride = a.q_bstride;
  a.kv_bstride = kv_batch_stride;
  // every entry reads one K/V: run the items of one head together
  if (kv_batch_stride == 0) a.plan = chunkattn::plan_head_major(a.plan);
  a.p_bstride = 0;
  a.pred_shift = 0;
  a.row_stride = heads * head_dim;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  return run(ctx, a, head_dim, dtype, hip_stream);
}

int chunkattn_validate_window_step(const void* q, const void* k, const void* v,
                                   const void* kv_cache, const void* out, int chunk_len,
                                   int n_chunks, int heads, int head_dim, float scale,
                                   int dtype) {
  g_thread_err.clear();
  return validate_queue(&g_thread_err, q, k, v, kv_cache, out, chunk_len, n_chunks, heads,
                        head_dim, scale, dtype, true);
}

int chunkattn_window_step(chunkattn_ctx* ctx, const void* q, const void* k, const void* v,
                          const void* kv_cache, void* out, int chunk_len, int n_chunks,
                          int heads, int head_dim, float scale, int dtype, void* hip_stream) {
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "ctx must be non-NULL");
  int rc = validate_queue(&ctx->err, q, k, v, kv_cache, out, chunk_len, n_chunks, heads,
                          head_dim, scale, dtype, true);
  if (rc) return rc;
  if (chunk_len == 0 || n_chunks == 0) {
    ctx->err.clear();
    return CHUNKATTN_OK;
  }
  const int64_t per_chunk = (int64_t)chunk_len * heads * head_dim;
  const size_t es = elem_size(dtype);
  KernelArgs a{};  // zero: linear batch entries unless set below
  a.plan = window_plan(chunk_len, n_chunks, heads, call_block_rows(ctx, head_dim, dtype),
                       ctx->n_xcd);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.q_bstride = per_chunk;      // window c's queries start at chunk c
  a.o_bstride = 2 * per_chunk;  // out[c] = [2][L][H][D]
  a.kv_bstride = per_chunk;     // own rows start at chunk c
  if (kv_cache) {
    a.pk = kv_cache;
    a.pv = static_cast<const unsigned char*>(kv_cache) + (size_t)per_chunk * es;
    a.p_bstride = 2 * per_chunk;
    a.pred_shift = 0;
  } else {
    a.pk = k;
    a.pv = v;
    a.p_bstride = per_chunk;
    a.pred_shift = 1;
  }
  a.row_stride = heads * head_dim;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  return run(ctx, a, head_dim, dtype, hip_stream);
}

int chunkattn_window_plan_debug(int chunk_len, int n_chunks, int heads, int n_xcd,
                                int block_rows, int* items, long long cap, long long* n_items) {
  g_thread_err.clear();
  if (!n_items) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "n_items must be non-NULL");
  if (block_rows == 0) block_rows = 384;
  if (chunk_len < 0 || n_chunks < 0 || heads < 1 || cap < 0 || (cap > 0 && !items) ||
      (block_rows != 128 && block_rows != 256 && block_rows != 384))
    return set_err(&g_thread_err, CHUNKATTN_EINVAL, "bad window_plan_debug arguments");
  *n_items = 0;
  if (chunk_len == 0 || n_chunks == 0) return CHUNKATTN_OK;
  const Plan p = window_plan(chunk_len, n_chunks, heads, block_rows, n_xcd);
  *n_items = p.n_items;
  for (int64_t slot = 0; slot < p.n_items && slot < cap; ++slot) {
    const chunkattn::Item it =
        chunkattn::decode(p, chunkattn::plan_slot_work(p, slot));
    int* r = items + slot * 7;
    r[0] = it.b;
    r[1] = it.h;
    r[2] = it.q0;
    r[3] = it.q_rows;
    r[4] = it.pred_rows > 0 ? it.b - 1 : -1;
    r[5] = it.pred_rows;
    r[6] = it.own_rows;
  }
  return CHUNKATTN_OK;
}

int chunkattn_validate_ring_step(const void* q_ring, const void* k_ring, const void* v_ring,
                                 const void* out_ring, int slots, int tail_slot, int n_live,
                                 int chunk_len, int heads, int head_dim, float scale,
                                 int dtype) {
  g_thread_err.clear();
  return validate_ring(&g_thread_err, q_ring, k_ring, v_ring, out_ring, slots, tail_slot, n_live,
                       chunk_len, heads, head_dim, scale, dtype);
}

int chunkattn_ring_step(chunkattn_ctx* ctx, const void* q_ring, const void* k_ring,
                        const void* v_ring, void* out_ring, int slots, int tail_slot,
                        int n_live, int chunk_len, int heads, int head_dim, float scale,
                        int dtype, void* hip_stream) {
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "ctx must be non-NULL");
  int rc = validate_ring(&ctx->err, q_ring, k_ring, v_ring, out_ring, slots, tail_slot, n_live,
                         chunk_len, heads, head_dim, scale, dtype);
  if (rc) return rc;
  if (chunk_len == 0 || n_live == 0) {
    ctx->err.clear();
    return CHUNKATTN_OK;
  }
  const int64_t per_chunk = (int64_t)chunk_len * heads * head_dim;
  KernelArgs a{};
  a.plan = chunkattn::make_plan(n_live, 1, heads, chunk_len, chunk_len, chunk_len,
                                call_block_rows(ctx, head_dim, dtype), ctx->n_xcd);
  a.q = q_ring;
  a.k = k_ring;
  a.v = v_ring;
  a.o = out_ring;
  a.q_bstride = per_chunk;
  a.o_bstride = per_chunk;
  a.kv_bstride = per_chunk;
  a.pk = k_ring;  // the predecessor is read in place from its slot
  a.pv = v_ring;
  a.p_bstride = per_chunk;
  a.pred_shift = 1;
  a.ring_slots = slots;
  a.ring_tail = tail_slot;
  a.row_stride = heads * head_dim;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  return run(ctx, a, head_dim, dtype, hip_stream);
}

struct chunkattn_fifo {
  chunkattn::Fifo q;
};

int chunkattn_fifo_create(chunkattn_fifo** out, int slots, int depth) {
  g_thread_err.clear();
  if (!out) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "out must be non-NULL");
  *out = nullptr;
  if (depth < 1 || slots < depth)
    return set_err(&g_thread_err, CHUNKATTN_EINVAL,
                   "need depth >= 1 and slots >= depth (got slots %d, depth %d)", slots, depth);
  chunkattn_fifo* f = new (std::nothrow) chunkattn_fifo{chunkattn::Fifo(slots, depth)};
  if (!f) return set_err(&g_thread_err, CHUNKATTN_ENOMEM, "cannot allocate the queue");
  *out = f;
  return CHUNKATTN_OK;
}

int chunkattn_fifo_destroy(chunkattn_fifo* f) {
  delete f;
  return CHUNKATTN_OK;
}

int chunkattn_fifo_push(chunkattn_fifo* f, int* slot) {
  g_thread_err.clear();
  if (!f || !slot) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "f and slot must be non-NULL");
  if (f->q.full())
    return set_err(&g_thread_err, CHUNKATTN_EINVAL, "queue full (%d chunks)", f->q.depth());
  *slot = f->q.push();
  return CHUNKATTN_OK;
}

int chunkattn_fifo_pop(chunkattn_fifo* f, int* slot) {
  g_thread_err.clear();
  if (!f || !slot) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "f and slot must be non-NULL");
  if (!f->q.head_clean())
    return set_err(&g_thread_err, CHUNKATTN_EINVAL,
                   "the head chunk has not done all %d steps (or the queue is empty)",
                   f->q.depth());
  *slot = f->q.pop();
  return CHUNKATTN_OK;
}

int chunkattn_fifo_live(const chunkattn_fifo* f, long long* ids, int* slots, int* steps_done,
                        int cap, int* n_live) {
  g_thread_err.clear();
  if (!f || !n_live || cap < 0)
    return set_err(&g_thread_err, CHUNKATTN_EINVAL, "bad fifo_live arguments");
  *n_live = f->q.live();
  for (int c = 0; c < f->q.live() && c < cap; ++c) {
    int64_t id;
    int s, d;
    f->q.at(c, &id, &s, &d);
    if (ids) ids[c] = id;
    if (slots) slots[c] = s;
    if (steps_done) steps_done[c] = d;
  }
  return CHUNKATTN_OK;
}

int chunkattn_fifo_advance(chunkattn_fifo* f) {
  g_thread_err.clear();
  if (!f) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "f must be non-NULL");
  if (f->q.live() == 0) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "queue empty");
  f->q.advance();
  return CHUNKATTN_OK;
}

int chunkattn_fifo_step(chunkattn_ctx* ctx, chunkattn_fifo* f, const void* q_ring,
                        const void* k_ring, const void* v_ring, void* out_ring, int chunk_len,
                        int heads, int head_dim, float scale, int dtype, void* hip_stream) {
  if (!f) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "f must be non-NULL");
  if (f->q.live() == 0) {
    std::string* sink = ctx ? &ctx->err : &g_thread_err;
    return set_err(sink, CHUNKATTN_EINVAL, "queue empty: push a chunk first");
  }
  const int rc = chunkattn_ring_step(ctx, q_ring, k_ring, v_ring, out_ring, f->q.slots(),
                                     f->q.tail_slot(), f->q.live(), chunk_len, heads, head_dim,
                                     scale, dtype, hip_stream);
  if (rc == CHUNKATTN_OK) f->q.advance();
  return rc;
}

int chunkattn_validate_noise_init(const void* pool, int pool_frames, long long frame_bytes,
                                  const void* keys, const void* prev_idx, int n_prev,
                                  int n_excl, int n_frames, const void* out,
                                  const void* idx_out) {
  g_thread_err.clear();
  std::string* err = &g_thread_err;
  if (pool_frames < 1 || pool_frames > chunkattn::kMaxNoisePool)
    return set_err(err, CHUNKATTN_EINVAL, "pool_frames must be in [1, %d] (got %d)",
                   chunkattn::kMaxNoisePool, pool_frames);
  if (n_frames < 1) return set_err(err, CHUNKATTN_EINVAL, "n_frames must be >= 1");
  if (n_prev < 0 || n_excl < 0 || n_excl > n_prev)
    return set_err(err, CHUNKATTN_EINVAL, "need 0 <= n_excl <= n_prev (got %d, %d)", n_excl,
                   n_prev);
  if (n_prev > 0 && !prev_idx)
    return set_err(err, CHUNKATTN_EINVAL, "prev_idx must be non-NULL when n_prev > 0");
  if ((long long)pool_frames - n_excl < n_frames)
    return set_err(err, CHUNKATTN_EINVAL,
                   "pool of %d frames minus %d excluded cannot give %d frames", pool_frames,
                   n_excl, n_frames);
  if (frame_bytes < 16 || frame_bytes % 16)
    return set_err(err, CHUNKATTN_EINVAL, "frame_bytes must be a positive multiple of 16");
  if ((long double)frame_bytes * pool_frames > 4.0e18L || frame_bytes / 16 / 256 >= (1LL << 31))
    return set_err(err, CHUNKATTN_EINVAL, "pool or frame size too large");
  if (!pool || !keys || !out || !idx_out)
    return set_err(err, CHUNKATTN_EINVAL, "pool, keys, out and idx_out must be non-NULL");
  if (!aligned16(pool) || !aligned16(out) || (reinterpret_cast<uintptr_t>(keys) & 3) ||
      (reinterpret_cast<uintptr_t>(idx_out) & 3) ||
      (prev_idx && (reinterpret_cast<uintptr_t>(prev_idx) & 3)))
    return set_err(err, CHUNKATTN_EINVAL,
                   "pool and out must be 16-byte aligned, keys and index arrays 4-byte aligned");
  const size_t pool_b = (size_t)pool_frames * frame_bytes, out_b = (size_t)n_frames * frame_bytes;
  if (overlaps(out, out_b, pool, pool_b) || overlaps(idx_out, 4 * (size_t)n_frames, out, out_b) ||
      overlaps(idx_out, 4 * (size_t)n_frames, keys, 4 * (size_t)pool_frames) ||
      (prev_idx && overlaps(idx_out, 4 * (size_t)n_frames, prev_idx, 4 * (size_t)n_prev)))
    return set_err(err, CHUNKATTN_EINVAL, "outputs overlap an input");
  return CHUNKATTN_OK;
}

int chunkattn_noise_init(chunkattn_ctx* ctx, const void* pool, int pool_frames,
                         long long frame_bytes, const void* keys, const void* prev_idx,
                         int n_prev, int n_excl, int n_frames, void* out, void* idx_out,
                         void* hip_stream) {
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "ctx must be non-NULL");
  int rc = chunkattn_validate_noise_init(pool, pool_frames, frame_bytes, keys, prev_idx, n_prev,
                                         n_excl, n_frames, out, idx_out);
  if (rc) {
    ctx->err = g_thread_err;
    return rc;
  }
  DeviceGuard g(ctx->device);
  if (!g.ok) return set_err(&ctx->err, CHUNKATTN_EDEVICE, "cannot make device current");
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  hipLaunchKernelGGL(chunkattn::noise_select, dim3(1), dim3(256), 0, st,
                     static_cast<const uint32_t*>(keys), pool_frames,
                     static_cast<const int*>(prev_idx), n_prev, n_excl, n_frames,
                     static_cast<int*>(idx_out));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_err(&ctx->err, CHUNKATTN_ELAUNCH, "noise_select launch failed: %s",
                   hipGetErrorString(e));
  const int64_t vecs = frame_bytes / 16;
  hipLaunchKernelGGL(chunkattn::noise_gather, dim3((unsigned)((vecs + 255) / 256), n_frames),
                     dim3(256), 0, st, static_cast<const uint4*>(pool), vecs,
                     static_cast<const int*>(idx_out), static_cast<uint4*>(out));
  e = hipGetLastError();
  if (e != hipSuccess)
    return set_err(&ctx->err, CHUNKATTN_ELAUNCH, "noise_gather launch failed: %s",
                   hipGetErrorString(e));
  ctx->err.clear();
  return CHUNKATTN_OK;
}

int chunkattn_mfma_probe(chunkattn_ctx* ctx, const void* operands, long long iters, void* out,
                         int* n_workgroups_out, double* flops_out, void* hip_stream) {
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "ctx must be non-NULL");
  if (!operands || !out || ((uintptr_t)operands & 15) || ((uintptr_t)out & 15))
    return set_err(&ctx->err, CHUNKATTN_EINVAL,
                   "operands and out must be non-NULL and 16-byte aligned");
  if (iters < 1 || iters > (1ll << 19))
    return set_err(&ctx->err, CHUNKATTN_EINVAL, "iters %lld outside [1, 2^19]", iters);
  DeviceGuard g(ctx->device);
  if (!g.ok) return set_err(&ctx->err, CHUNKATTN_EDEVICE, "cannot make device current");
  const int n_wg = ctx->n_cu;
  hipLaunchKernelGGL(chunkattn::mfma_peak_probe, dim3((unsigned)n_wg),
                     dim3(chunkattn::kProbeWaves * 64), 0, static_cast<hipStream_t>(hip_stream),
                     static_cast<const uint32_t*>(operands), iters, static_cast<float*>(out));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_err(&ctx->err, CHUNKATTN_ELAUNCH, "mfma_peak_probe launch failed: %s",
                   hipGetErrorString(e));
  if (n_workgroups_out) *n_workgroups_out = n_wg;
  // 16 x 16 x 32 multiply-adds per instruction, 2 FLOPs each
  if (flops_out)
    *flops_out = (double)n_wg * chunkattn::kProbeWaves * chunkattn::kProbeAcc * (double)iters *
                 (2.0 * 16 * 16 * 32);
  ctx->err.clear();
  return CHUNKATTN_OK;
}

int chunkattn_ctx_cu_count(const chunkattn_ctx* ctx) { return ctx ? ctx->n_cu : 0; }

const char* chunkattn_status_string(int status) {
  switch (status) {
    case CHUNKATTN_OK: return "ok";
    case CHUNKATTN_EINVAL: return "invalid argument";
    case CHUNKATTN_EUNSUPPORTED: return "unsupported";
    case CHUNKATTN_EDEVICE: return "device error";
    case CHUNKATTN_ENOMEM: return "out of host memory";
    case CHUNKATTN_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

const char* chunkattn_last_error(const chunkattn_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_thread_err.c_str();
}

int chunkattn_plan_debug(int chunk_len, int n_chunks, int heads, int n_xcd, int block_rows,
                         int* items, long long cap, long long* n_items) {
  g_thread_err.clear();
  if (!n_items) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "n_items must be non-NULL");
  if (block_rows == 0) block_rows = 384;
  if (chunk_len < 0 || n_chunks < 0 || heads < 1 || cap < 0 || (cap > 0 && !items) ||
      (block_rows != 128 && block_rows != 256 && block_rows != 384))
    return set_err(&g_thread_err, CHUNKATTN_EINVAL, "bad plan_debug arguments");
  *n_items = 0;
  if (chunk_len == 0 || n_chunks == 0) return CHUNKATTN_OK;
  const Plan p = chunkattn::make_plan(n_chunks, 1, heads, chunk_len, chunk_len, chunk_len,
                                      block_rows, n_xcd);
  *n_items = p.n_items;
  for (int64_t slot = 0; slot < p.n_items && slot < cap; ++slot) {
    const chunkattn::Item it =
        chunkattn::decode(p, chunkattn::plan_slot_work(p, slot));
    int* r = items + slot * 7;
    r[0] = it.b;
    r[1] = it.h;
    r[2] = it.q0;
    r[3] = it.q_rows;
    r[4] = it.pred_rows > 0 ? it.b - 1 : -1;
    r[5] = it.pred_rows;
    r[6] = it.own_rows;
  }
  return CHUNKATTN_OK;
}

int chunkattn_plan_device(chunkattn_ctx* ctx, int chunk_len, int n_chunks, int heads,
                          int* dev_items, long long cap, void* hip_stream) {
  if (!ctx) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "ctx must be non-NULL");
  if (chunk_len < 0 || n_chunks < 0 || heads < 1 || cap < 0 || (cap > 0 && !dev_items))
    return set_err(&ctx->err, CHUNKATTN_EINVAL, "bad plan_device arguments");
  if (chunk_len == 0 || n_chunks == 0 || cap == 0) return CHUNKATTN_OK;
  const Plan p = chunkattn::make_plan(n_chunks, 1, heads, chunk_len, chunk_len, chunk_len,
                                      call_block_rows(ctx, 128, CHUNKATTN_BF16), ctx->n_xcd);
  const int64_t n = p.n_items < cap ? p.n_items : cap;
  DeviceGuard g(ctx->device);
  if (!g.ok) return set_err(&ctx->err, CHUNKATTN_EDEVICE, "cannot make device current");
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(chunkattn::plan_dump, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(hip_stream), p, dev_items, (int64_t)cap);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_err(&ctx->err, CHUNKATTN_ELAUNCH, "plan_dump launch failed: %s",
                   hipGetErrorString(e));
  ctx->err.clear();
  return CHUNKATTN_OK;
}

}  // extern "C"
