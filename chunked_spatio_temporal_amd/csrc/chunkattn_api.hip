// C-ABI entry points of the chunk-attention library (declared in
// include/chunkattn.h): argument validation, the integer launch plan and the
// kernel launch.  No allocation happens on the hot calls.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "attn_kernel.h"
#include "attn_pingpong.h"
#include "chunkattn.h"
#include "fifo.h"
#include "noise.h"

// Work-queue slots of a context: each call of the persistent (256-row) main
// pass takes the next slot, so up to kQueueSlots calls may be in flight on
// different streams at once.  A slot is kQueueWords 64-bit words (one claim
// word per die, one finished-workgroup counter), zero between launches.
constexpr int kQueueSlots = 64;
constexpr int kQueueWords = 16;

struct chunkattn_ctx {
  int device = 0;
  int n_cu = 0;
  int n_xcd = 1;
  int waves = 8;  // waves per workgroup; a work item covers 32 * waves query rows
  unsigned long long* queue = nullptr;  // device, kQueueSlots * kQueueWords words
  std::atomic<unsigned> next_slot{0};
  std::string arch;
  std::string err;
};

namespace {

using chunkattn::KernelArgs;
using chunkattn::Plan;

constexpr int kDefaultWaves = 8;
constexpr int kMinBlockRows = 128;  // smallest work item (4 waves); bounds the grid

thread_local std::string g_thread_err;

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
      (long double)n * heads * ((long long)((q_rows + kMinBlockRows - 1) / kMinBlockRows));
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
      (long double)batch * heads * ((lq + kMinBlockRows - 1) / kMinBlockRows);
  if (items > 2147483647.0L)
    return set_err(err, CHUNKATTN_EUNSUPPORTED, "too many work items for one launch");
  return CHUNKATTN_OK;
}

}  // namespace

// Every kernel configuration the host can launch, instantiated explicitly.
namespace chunkattn {
template __global__ void chunk_attn_fwd_pingpong<128, __bf16>(KernelArgs);
template __global__ void chunk_attn_fwd_pingpong<128, float>(KernelArgs);
template __global__ void chunk_attn_fwd_pingpong<64, __bf16>(KernelArgs);
template __global__ void chunk_attn_fwd_pingpong<64, float>(KernelArgs);
template __global__ void chunk_attn_fwd<128, __bf16, 4>(KernelArgs);
template __global__ void chunk_attn_recheck<128, __bf16, 4>(KernelArgs);
template __global__ void chunk_attn_fwd<128, float, 4>(KernelArgs);
template __global__ void chunk_attn_recheck<128, float, 4>(KernelArgs);
template __global__ void chunk_attn_fwd<64, __bf16, 4>(KernelArgs);
template __global__ void chunk_attn_recheck<64, __bf16, 4>(KernelArgs);
template __global__ void chunk_attn_fwd<64, float, 4>(KernelArgs);
template __global__ void chunk_attn_recheck<64, float, 4>(KernelArgs);
template __global__ void chunk_attn_recheck<128, __bf16, 8>(KernelArgs);
template __global__ void chunk_attn_recheck<128, float, 8>(KernelArgs);
template __global__ void chunk_attn_recheck<64, __bf16, 8>(KernelArgs);
template __global__ void chunk_attn_recheck<64, float, 8>(KernelArgs);
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
template <int D, typename T, int W>
hipError_t launch_t(const KernelArgs& a, int n_persist, hipStream_t stream) {
  const dim3 grid((unsigned)a.plan.n_items);
  constexpr uint32_t kLds = chunkattn::kSyncLdsBytes<D>;
  if constexpr (W == 8) {
    if (!a.queue || n_persist < 1) return hipErrorInvalidValue;
    const hipError_t el = allow_pingpong_lds<D, T>();
    if (el != hipSuccess) return el;
    hipLaunchKernelGGL((chunkattn::chunk_attn_fwd_pingpong<D, T>), dim3((unsigned)n_persist),
                       dim3(512),
                       chunkattn::kPingPongLdsBytes<D>, stream, a);
  } else {
    hipLaunchKernelGGL((chunkattn::chunk_attn_fwd<D, T, W>), grid, dim3(64 * W), kLds, stream,
                       a);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((chunkattn::chunk_attn_recheck<D, T, W>), grid, dim3(64 * W), kLds, stream,
                     a);
  return hipGetLastError();
}

template <int W>
hipError_t launch_w(const KernelArgs& a, int n_persist, int head_dim, int dtype,
                    hipStream_t stream) {
  if (head_dim == 128)
    return dtype == CHUNKATTN_BF16 ? launch_t<128, __bf16, W>(a, n_persist, stream)
                                   : launch_t<128, float, W>(a, n_persist, stream);
  return dtype == CHUNKATTN_BF16 ? launch_t<64, __bf16, W>(a, n_persist, stream)
                                 : launch_t<64, float, W>(a, n_persist, stream);
}

hipError_t launch(const KernelArgs& a, int waves, int n_persist, int head_dim, int dtype,
                  hipStream_t stream) {
  return waves == 4 ? launch_w<4>(a, n_persist, head_dim, dtype, stream)
                    : launch_w<8>(a, n_persist, head_dim, dtype, stream);
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

int run(chunkattn_ctx* ctx, const KernelArgs& args, int head_dim, int dtype, void* stream) {
  DeviceGuard g(ctx->device);
  if (!g.ok) return set_err(&ctx->err, CHUNKATTN_EDEVICE, "cannot make device %d current",
                            ctx->device);
  KernelArgs a = args;
  a.queue = nullptr;
  if (ctx->waves == 8) {
    // one claim word per die and the finished count must fit in a slot
    if (a.plan.n_xcd >= kQueueWords) a.plan.n_xcd = 1;
    const unsigned slot = ctx->next_slot.fetch_add(1, std::memory_order_relaxed) % kQueueSlots;
    a.queue = ctx->queue + (size_t)slot * kQueueWords;
  }
  const int n_persist = (int)(a.plan.n_items < ctx->n_cu ? a.plan.n_items : ctx->n_cu);
  const hipError_t e =
      launch(a, ctx->waves, n_persist, head_dim, dtype, static_cast<hipStream_t>(stream));
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

int chunkattn_block_rows(void) { return 32 * kDefaultWaves; }

int chunkattn_ctx_block_rows(const chunkattn_ctx* ctx) { return ctx ? 32 * ctx->waves : 0; }

int chunkattn_create(chunkattn_ctx** out, int device_ordinal, unsigned flags) {
  if (!out) return set_err(&g_thread_err, CHUNKATTN_EINVAL, "out must be non-NULL");
  *out = nullptr;
  const unsigned known = CHUNKATTN_FLAG_BLOCK128 | CHUNKATTN_FLAG_BLOCK256;
  if ((flags & ~known) != 0 || flags == known)
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
  ctx->waves = (flags & CHUNKATTN_FLAG_BLOCK128) ? 4 : (flags & CHUNKATTN_FLAG_BLOCK256) ? 8
                                                                                       : kDefaultWaves;
  ctx->n_cu = prop.multiProcessorCount;
  ctx->arch = prop.gcnArchName;
  int xcc = 0;
  if (hipDeviceGetAttribute(&xcc, hipDeviceAttributeNumberOfXccs, device_ordinal) ==
          hipSuccess &&
      xcc > 0)
    ctx->n_xcd = xcc;
  if (ctx->waves == 8) {
    // the work queue of the persistent main pass, zeroed once here
    DeviceGuard g(device_ordinal);
    const size_t bytes = sizeof(unsigned long long) * kQueueSlots * kQueueWords;
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
  *out = ctx;
  return CHUNKATTN_OK;
}

int chunkattn_destroy(chunkattn_ctx* ctx) {
  if (ctx && ctx->queue) {
    DeviceGuard g(ctx->device);
    (void)hipFree(ctx->queue);
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

int chunkattn_queue_step(chunkattn_ctx* ctx, const void* q, const void* k, const void* v,
                         const void* kv_cache, void* out, int chunk_len, int n_chunks,
                         int heads, int head_dim, float scale, int dtype, void* hip_stream) {
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
                                32 * ctx->waves, ctx->n_xcd);
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
  return run(ctx, a, head_dim, dtype, hip_stream);
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
  a.plan = chunkattn::make_plan(batch, batch, heads, lq, lkv, 0, 32 * ctx->waves, ctx->n_xcd);
  a.q = q;
  a.k = k;
  a.v = v;
  a.pk = nullptr;
  a.pv = nullptr;
  a.o = out;
  a.q_bstride = (int64_t)lq * heads * head_dim;
  a.o_bstride = a.q_bstride;
  a.kv_bstride = kv_batch_stride;
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
  a.plan = window_plan(chunk_len, n_chunks, heads, 32 * ctx->waves, ctx->n_xcd);
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
  if (block_rows == 0) block_rows = 32 * kDefaultWaves;
  if (chunk_len < 0 || n_chunks < 0 || heads < 1 || cap < 0 || (cap > 0 && !items) ||
      (block_rows != 128 && block_rows != 256))
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
                                32 * ctx->waves, ctx->n_xcd);
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
  if (block_rows == 0) block_rows = 32 * kDefaultWaves;
  if (chunk_len < 0 || n_chunks < 0 || heads < 1 || cap < 0 || (cap > 0 && !items) ||
      (block_rows != 128 && block_rows != 256))
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
                                      32 * ctx->waves, ctx->n_xcd);
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
