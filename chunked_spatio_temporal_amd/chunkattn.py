"""ctypes binding of the chunk-attention C ABI (include/chunkattn.h).

Argument marshalling only: tensors become device pointers and sizes, the
current torch stream becomes the HIP stream, status codes become exceptions.
Every step of the computation runs in the HIP library; there is no fallback.
If the library is missing the first call raises ChunkAttnUnavailable.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# CHUNKATTN_LIBRARY names another build of the same library (the host-sanitized
# one of the CPU tests); by default the in-tree build.
LIB_PATH = os.environ.get("CHUNKATTN_LIBRARY") or os.path.join(PKG, "lib", "libchunkattn.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "chunkattn.h")

OK, EINVAL, EUNSUPPORTED, EDEVICE, ENOMEM, ELAUNCH = range(6)
BF16, F32 = 0, 1
FLAG_BLOCK128, FLAG_BLOCK256, FLAG_BLOCK384, FLAG_EXACT_SCALE = 1, 2, 4, 8
PLAN_FIELDS = ("chunk", "head", "q_row0", "q_rows", "pred_chunk", "pred_rows", "own_rows")


class ChunkAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"chunkattn status {status}: {message}")
        self.status = status


class ChunkAttnUnavailable(ImportError):
    pass


_lib = None


def load_library():
    """Loads lib/libchunkattn.so (raises ChunkAttnUnavailable if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ChunkAttnUnavailable(
            f"{LIB_PATH} is missing; build it with `python -m chunked_spatio_temporal_amd._build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float
    lib.chunkattn_block_rows.restype = i32
    lib.chunkattn_ctx_block_rows.restype = i32
    lib.chunkattn_ctx_block_rows.argtypes = [vp]
    lib.chunkattn_ctx_call_block_rows.restype = i32
    lib.chunkattn_ctx_call_block_rows.argtypes = [vp, i32, i32]
    lib.chunkattn_ctx_set_item_blocks.restype = i32
    lib.chunkattn_ctx_set_item_blocks.argtypes = [vp, i32]
    lib.chunkattn_ctx_set_tail_split.restype = i32
    lib.chunkattn_ctx_set_tail_split.argtypes = [vp, i32, i32]
    lib.chunkattn_create.restype = i32
    lib.chunkattn_create.argtypes = [ctypes.POINTER(vp), i32, ctypes.c_uint]
    lib.chunkattn_destroy.restype = i32
    lib.chunkattn_destroy.argtypes = [vp]
    lib.chunkattn_queue_step.restype = i32
    lib.chunkattn_queue_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp]
    lib.chunkattn_queue_step_noalloc.restype = i32
    lib.chunkattn_queue_step_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                                 i32, vp]
    lib.chunkattn_full.restype = i32
    lib.chunkattn_full.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, f32, i32, vp]
    lib.chunkattn_validate_queue_step.restype = i32
    lib.chunkattn_validate_queue_step.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32]
    lib.chunkattn_validate_full.restype = i32
    lib.chunkattn_validate_full.argtypes = [vp, vp, vp, vp, i32, i32, i32, i64, i32, i32, f32, i32]
    lib.chunkattn_status_string.restype = ctypes.c_char_p
    lib.chunkattn_status_string.argtypes = [i32]
    lib.chunkattn_last_error.restype = ctypes.c_char_p
    lib.chunkattn_last_error.argtypes = [vp]
    lib.chunkattn_plan_debug.restype = i32
    lib.chunkattn_plan_debug.argtypes = [i32, i32, i32, i32, i32, vp, i64, ctypes.POINTER(i64)]
    lib.chunkattn_plan_device.restype = i32
    lib.chunkattn_plan_device.argtypes = [vp, i32, i32, i32, vp, i64, vp]
    lib.chunkattn_window_step.restype = i32
    lib.chunkattn_window_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, f32, i32, vp]
    lib.chunkattn_validate_window_step.restype = i32
    lib.chunkattn_validate_window_step.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, f32,
                                                   i32]
    lib.chunkattn_window_plan_debug.restype = i32
    lib.chunkattn_window_plan_debug.argtypes = [i32, i32, i32, i32, i32, vp, i64,
                                                ctypes.POINTER(i64)]
    lib.chunkattn_ring_step.restype = i32
    lib.chunkattn_ring_step.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32,
                                        i32, vp]
    lib.chunkattn_validate_ring_step.restype = i32
    lib.chunkattn_validate_ring_step.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                 f32, i32]
    lib.chunkattn_fifo_create.restype = i32
    lib.chunkattn_fifo_create.argtypes = [ctypes.POINTER(vp), i32, i32]
    lib.chunkattn_fifo_destroy.restype = i32
    lib.chunkattn_fifo_destroy.argtypes = [vp]
    lib.chunkattn_fifo_push.restype = i32
    lib.chunkattn_fifo_push.argtypes = [vp, ctypes.POINTER(i32)]
    lib.chunkattn_fifo_pop.restype = i32
    lib.chunkattn_fifo_pop.argtypes = [vp, ctypes.POINTER(i32)]
    lib.chunkattn_fifo_live.restype = i32
    lib.chunkattn_fifo_live.argtypes = [vp, vp, vp, vp, i32, ctypes.POINTER(i32)]
    lib.chunkattn_fifo_advance.restype = i32
    lib.chunkattn_fifo_advance.argtypes = [vp]
    lib.chunkattn_fifo_step.restype = i32
    lib.chunkattn_fifo_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, f32, i32, vp]
    lib.chunkattn_noise_init.restype = i32
    lib.chunkattn_noise_init.argtypes = [vp, vp, i32, i64, vp, vp, i32, i32, i32, vp, vp, vp]
    lib.chunkattn_validate_noise_init.restype = i32
    lib.chunkattn_validate_noise_init.argtypes = [vp, i32, i64, vp, vp, i32, i32, i32, vp, vp]
    lib.chunkattn_ctx_xcd_count.restype = i32
    lib.chunkattn_ctx_xcd_count.argtypes = [vp]
    lib.chunkattn_ctx_cu_count.restype = i32
    lib.chunkattn_ctx_cu_count.argtypes = [vp]
    lib.chunkattn_mfma_probe.restype = i32
    lib.chunkattn_mfma_probe.argtypes = [vp, vp, i64, vp, ctypes.POINTER(i32),
                                         ctypes.POINTER(ctypes.c_double), vp]
    _lib = lib
    return lib


def declared_symbols() -> list[str]:
    """Names of the functions include/chunkattn.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(chunkattn_[a-z_]+)\s*\(", text)))


def _check(rc: int, ctx_handle=None):
    if rc != OK:
        lib = load_library()
        msg = lib.chunkattn_last_error(ctx_handle).decode()
        raise ChunkAttnError(rc, msg or lib.chunkattn_status_string(rc).decode())


def block_rows() -> int:
    return int(load_library().chunkattn_block_rows())


class Context:
    """Owns a chunkattn_ctx bound to one device (flags: 0 or FLAG_BLOCK128/256/384,
    optionally | FLAG_EXACT_SCALE)."""

    def __init__(self, device: int = 0, flags: int = 0):
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.chunkattn_create(ctypes.byref(h), int(device), int(flags)))
        self.handle = h
        self.device = int(device)
        self.flags = int(flags)

    def close(self):
        if getattr(self, "handle", None):
            load_library().chunkattn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def xcd_count(self) -> int:
        return int(load_library().chunkattn_ctx_xcd_count(self.handle))

    @property
    def cu_count(self) -> int:
        return int(load_library().chunkattn_ctx_cu_count(self.handle))

    @property
    def block_rows(self) -> int:
        """Query rows per work item of a bf16, head_dim-128 call."""
        return int(load_library().chunkattn_ctx_block_rows(self.handle))

    def call_block_rows(self, head_dim: int, dtype: int) -> int:
        """Query rows per work item of a call with this head_dim and dtype code."""
        return int(load_library().chunkattn_ctx_call_block_rows(self.handle, int(head_dim),
                                                                int(dtype)))

    def set_tail_split(self, items: int, parts: int = 0) -> None:
        """Key-axis split of the last `items` work items into `parts` (-1: chosen
        per call, 0: never)."""
        _check(load_library().chunkattn_ctx_set_tail_split(self.handle, int(items), int(parts)),
               self.handle)

    def set_item_blocks(self, blocks: int) -> None:
        """384-row query blocks per work item (0: chosen per call, 1..8: fixed)."""
        _check(load_library().chunkattn_ctx_set_item_blocks(self.handle, int(blocks)), self.handle)


_contexts: dict[tuple, Context] = {}


def create(device: int = 0, flags: int = 0) -> Context:
    """The process-wide context of (`device`, `flags`), created on first use."""
    key = (int(device), int(flags))
    ctx = _contexts.get(key)
    if ctx is None:
        ctx = _contexts[key] = Context(device, flags)
    return ctx


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"chunkattn: unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t, name, dev):
    if not t.is_cuda:
        raise ValueError(f"chunkattn: {name} must be a GPU tensor")
    if t.device != dev:
        raise ValueError(f"chunkattn: {name} is on {t.device}, q on {dev}")
    if not t.is_contiguous():
        raise ValueError(f"chunkattn: {name} must be contiguous")


def queue_step(q, k, v, kv_cache=None, out=None, scale=None, stream=None, ctx=None):
    """One queue step: chunk c attends over [predecessor K/V ; own K/V].

    q, k, v: [n_chunks, chunk_len, heads, head_dim] bf16/fp32 GPU tensors.
    kv_cache: optional [n_chunks, 2, chunk_len, heads, head_dim] (slot c = K/V
    of chunk c-1); None reads chunk c-1 from k/v in place.  Returns `out`.
    """
    import torch
    n, L, H, D = _queue_args("queue_step", q, k, v, kv_cache)
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", q.device)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("chunkattn.queue_step: out must match q")
    scale = D ** -0.5 if scale is None else float(scale)
    ctx = ctx or create(q.device.index or 0)
    rc = load_library().chunkattn_queue_step(
        ctx.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_cache), _ptr(out), L, n, H, D, scale,
        _dtype_code(q), _stream(q, stream))
    _check(rc, ctx.handle)
    return out


def queue_step_noalloc(q, k, v, kv_cache, out, scale=None, stream=None, ctx=None):
    """The queue step through chunkattn_queue_step_noalloc: same result as
    queue_step, with the work queue in the library's static device scratch
    (no allocation by the call; calls on one device must not overlap).  The
    caller passes `out`.  Returns `out`."""
    n, L, H, D = _queue_args("queue_step_noalloc", q, k, v, kv_cache)
    _require(out, "out", q.device)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("chunkattn.queue_step_noalloc: out must match q")
    scale = D ** -0.5 if scale is None else float(scale)
    ctx = ctx or create(q.device.index or 0)
    rc = load_library().chunkattn_queue_step_noalloc(
        ctx.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_cache), _ptr(out), L, n, H, D, scale,
        _dtype_code(q), _stream(q, stream))
    _check(rc, ctx.handle)
    return out


def _queue_args(fn, q, k, v, kv_cache):
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"chunkattn.{fn}: q, k, v must all be [n, L, H, D]")
    n, L, H, D = q.shape
    _require(q, "q", q.device)
    for name, t in (("k", k), ("v", v)):
        _require(t, name, q.device)
        if t.dtype != q.dtype:
            raise TypeError(f"chunkattn.{fn}: {name} dtype {t.dtype} != q dtype {q.dtype}")
    if kv_cache is not None:
        _require(kv_cache, "kv_cache", q.device)
        if kv_cache.shape != (n, 2, L, H, D) or kv_cache.dtype != q.dtype:
            raise ValueError(f"chunkattn.{fn}: kv_cache must be [n, 2, L, H, D] of q's dtype")
    return n, L, H, D


def window_step(q, k, v, kv_cache=None, out=None, scale=None, stream=None, ctx=None):
    """One window step: window c's queries (chunks c and c+1) attend over
    [chunk c-1's cached K/V ; own K/V of chunks c and c+1].

    q, k, v, kv_cache as for queue_step.  Returns `out`, [n, 2, L, H, D]:
    out[c, 0] = window c's rows of chunk c, out[c, 1] = its rows of chunk c+1
    (out[n-1, 1] is left as it was).
    """
    import torch
    n, L, H, D = _queue_args("window_step", q, k, v, kv_cache)
    if out is None:
        out = torch.empty((n, 2, L, H, D), dtype=q.dtype, device=q.device)
    else:
        _require(out, "out", q.device)
        if out.shape != (n, 2, L, H, D) or out.dtype != q.dtype:
            raise ValueError("chunkattn.window_step: out must be [n, 2, L, H, D] of q's dtype")
    scale = D ** -0.5 if scale is None else float(scale)
    ctx = ctx or create(q.device.index or 0)
    rc = load_library().chunkattn_window_step(
        ctx.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(kv_cache), _ptr(out), L, n, H, D, scale,
        _dtype_code(q), _stream(q, stream))
    _check(rc, ctx.handle)
    return out


def _ring_args(fn, q_ring, k_ring, v_ring, out_ring):
    if q_ring.dim() != 4 or k_ring.shape != q_ring.shape or v_ring.shape != q_ring.shape:
        raise ValueError(f"chunkattn.{fn}: q, k, v rings must all be [slots, L, H, D]")
    for name, t in (("q_ring", q_ring), ("k_ring", k_ring), ("v_ring", v_ring),
                    ("out_ring", out_ring)):
        _require(t, name, q_ring.device)
        if t.dtype != q_ring.dtype:
            raise TypeError(f"chunkattn.{fn}: {name} dtype {t.dtype} != {q_ring.dtype}")
    if out_ring.shape != q_ring.shape:
        raise ValueError(f"chunkattn.{fn}: out_ring must match q_ring")
    return q_ring.shape


def ring_step(q_ring, k_ring, v_ring, out_ring, tail_slot, n_live, scale=None, stream=None,
              ctx=None):
    """Queue step over the n_live chunks of ring buffers [slots, L, H, D]:
    chunk c (tail first) in slot (tail_slot - c) mod slots attends over its
    predecessor's slot (read in place) and its own.  Writes those slots of
    out_ring; returns out_ring."""
    S, L, H, D = _ring_args("ring_step", q_ring, k_ring, v_ring, out_ring)
    scale = D ** -0.5 if scale is None else float(scale)
    ctx = ctx or create(q_ring.device.index or 0)
    rc = load_library().chunkattn_ring_step(
        ctx.handle, _ptr(q_ring), _ptr(k_ring), _ptr(v_ring), _ptr(out_ring), S, int(tail_slot),
        int(n_live), L, H, D, scale, _dtype_code(q_ring), _stream(q_ring, stream))
    _check(rc, ctx.handle)
    return out_ring


class Fifo:
    """The streaming chunk queue's host bookkeeping (C++ object behind the C
    ABI): chunk g lives in slot g mod slots, each chunk stays `depth` steps."""

    def __init__(self, slots: int, depth: int):
        lib = load_library()
        h = ctypes.c_void_p()
        _check(lib.chunkattn_fifo_create(ctypes.byref(h), slots, depth))
        self.handle = h
        self.slots = slots
        self.depth = depth

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.chunkattn_fifo_destroy(h)
            self.handle = None

    def push(self) -> int:
        s = ctypes.c_int()
        _check(load_library().chunkattn_fifo_push(self.handle, ctypes.byref(s)))
        return s.value

    def pop(self) -> int:
        s = ctypes.c_int()
        _check(load_library().chunkattn_fifo_pop(self.handle, ctypes.byref(s)))
        return s.value

    def live(self):
        """[(chunk number, slot, steps done)] in processing order, tail first."""
        lib = load_library()
        n = ctypes.c_int()
        _check(lib.chunkattn_fifo_live(self.handle, None, None, None, 0, ctypes.byref(n)))
        ids = np.zeros(max(n.value, 1), np.int64)
        slots = np.zeros(max(n.value, 1), np.int32)
        done = np.zeros(max(n.value, 1), np.int32)
        _check(lib.chunkattn_fifo_live(self.handle, ids.ctypes.data_as(ctypes.c_void_p),
                                       slots.ctypes.data_as(ctypes.c_void_p),
                                       done.ctypes.data_as(ctypes.c_void_p), n.value,
                                       ctypes.byref(n)))
        return [(int(ids[i]), int(slots[i]), int(done[i])) for i in range(n.value)]

    def advance(self) -> None:
        """Mark one step done for every live chunk (no launch)."""
        _check(load_library().chunkattn_fifo_advance(self.handle))

    def step(self, q_ring, k_ring, v_ring, out_ring, scale=None, stream=None, ctx=None):
        """Attention of every live chunk (one launch), then every live chunk has
        done one more step."""
        S, L, H, D = _ring_args("Fifo.step", q_ring, k_ring, v_ring, out_ring)
        if S != self.slots:
            raise ValueError(f"chunkattn.Fifo.step: rings have {S} slots, queue {self.slots}")
        scale = D ** -0.5 if scale is None else float(scale)
        ctx = ctx or create(q_ring.device.index or 0)
        rc = load_library().chunkattn_fifo_step(
            ctx.handle, self.handle, _ptr(q_ring), _ptr(k_ring), _ptr(v_ring), _ptr(out_ring),
            L, H, D, scale, _dtype_code(q_ring), _stream(q_ring, stream))
        _check(rc, ctx.handle)
        return out_ring


def noise_init(pool, keys, n_frames, prev_idx=None, n_excl=0, out=None, idx_out=None,
               stream=None, ctx=None):
    """A new chunk's noise: n_frames frames of `pool` [P, ...] (any dtype), the
    candidates not used by the last n_excl entries of prev_idx, ranked by
    (keys, index); keys is an int32/uint32 tensor of P values (bit patterns
    compared as unsigned).  Returns (out [n_frames, ...], idx_out int32)."""
    import torch
    P = pool.shape[0]
    _require(pool, "pool", pool.device)
    _require(keys, "keys", pool.device)
    if keys.shape != (P,) or keys.element_size() != 4:
        raise ValueError("chunkattn.noise_init: keys must be P 32-bit values")
    frame_bytes = pool[0].numel() * pool.element_size() if P else 0
    n_prev = 0
    if prev_idx is not None:
        _require(prev_idx, "prev_idx", pool.device)
        if prev_idx.dtype != torch.int32 or prev_idx.dim() != 1:
            raise ValueError("chunkattn.noise_init: prev_idx must be 1-D int32")
        n_prev = prev_idx.numel()
    if out is None:
        out = torch.empty((n_frames,) + tuple(pool.shape[1:]), dtype=pool.dtype,
                          device=pool.device)
    if idx_out is None:
        idx_out = torch.empty(n_frames, dtype=torch.int32, device=pool.device)
    ctx = ctx or create(pool.device.index or 0)
    rc = load_library().chunkattn_noise_init(
        ctx.handle, _ptr(pool), P, frame_bytes, _ptr(keys), _ptr(prev_idx), n_prev, int(n_excl),
        int(n_frames), _ptr(out), _ptr(idx_out), _stream(pool, stream))
    _check(rc, ctx.handle)
    return out, idx_out


def validate_noise_init(pool_ptr, pool_frames, frame_bytes, keys_ptr, prev_ptr, n_prev, n_excl,
                        n_frames, out_ptr, idx_ptr):
    """(status, message) of the device-free argument checks of noise_init."""
    lib = load_library()
    rc = lib.chunkattn_validate_noise_init(pool_ptr, pool_frames, frame_bytes, keys_ptr,
                                           prev_ptr, n_prev, n_excl, n_frames, out_ptr, idx_ptr)
    return rc, lib.chunkattn_last_error(None).decode()


def full(q, k, v, out=None, scale=None, stream=None, ctx=None):
    """Non-chunked attention of every query row over all K/V rows of its batch item.

    q: [batch, lq, H, D]; k, v: [batch, lkv, H, D], or [1, lkv, H, D] shared by
    the whole batch (kv stride 0, e.g. text tokens of one prompt).
    """
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("chunkattn.full: q is [B, Lq, H, D]; k, v are [B or 1, Lkv, H, D]")
    B, lq, H, D = q.shape
    kb, lkv, Hk, Dk = k.shape
    if (Hk, Dk) != (H, D) or kb not in (1, B):
        raise ValueError("chunkattn.full: k/v heads/head_dim must match q; batch 1 or B")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _require(t, name, q.device)
        if t.dtype != q.dtype:
            raise TypeError(f"chunkattn.full: {name} dtype {t.dtype} != q dtype {q.dtype}")
    stride = 0 if (kb == 1 and B > 1) else lkv * H * D
    if out is None:
        out = torch.empty_like(q)
    else:
        _require(out, "out", q.device)
        if out.shape != q.shape or out.dtype != q.dtype:
            raise ValueError("chunkattn.full: out must match q")
    scale = D ** -0.5 if scale is None else float(scale)
    ctx = ctx or create(q.device.index or 0)
    rc = load_library().chunkattn_full(
        ctx.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, lq, lkv, stride, H, D, scale,
        _dtype_code(q), _stream(q, stream))
    _check(rc, ctx.handle)
    return out


def plan_debug(chunk_len: int, n_chunks: int, heads: int, n_xcd: int = 8,
               block_rows: int = 0) -> np.ndarray:
    """The queue-step launch plan computed on the host, [n_items, 7] int32."""
    lib = load_library()
    n = ctypes.c_longlong()
    _check(lib.chunkattn_plan_debug(chunk_len, n_chunks, heads, n_xcd, block_rows, None, 0,
                                    ctypes.byref(n)))
    items = np.zeros((n.value, 7), np.int32)
    _check(lib.chunkattn_plan_debug(chunk_len, n_chunks, heads, n_xcd, block_rows,
                                    items.ctypes.data_as(ctypes.c_void_p), n.value,
                                    ctypes.byref(n)))
    return items


def window_plan_debug(chunk_len: int, n_chunks: int, heads: int, n_xcd: int = 8,
                      block_rows: int = 0) -> np.ndarray:
    """The window-step launch plan computed on the host, [n_items, 7] int32."""
    lib = load_library()
    n = ctypes.c_longlong()
    _check(lib.chunkattn_window_plan_debug(chunk_len, n_chunks, heads, n_xcd, block_rows, None,
                                           0, ctypes.byref(n)))
    items = np.zeros((n.value, 7), np.int32)
    _check(lib.chunkattn_window_plan_debug(chunk_len, n_chunks, heads, n_xcd, block_rows,
                                           items.ctypes.data_as(ctypes.c_void_p), n.value,
                                           ctypes.byref(n)))
    return items


def plan_device(chunk_len: int, n_chunks: int, heads: int, device: int = 0, ctx=None):
    """The same plan as decoded by the device kernel, [n_items, 7] int32 (GPU)."""
    import torch
    lib = load_library()
    ctx = ctx or create(device)
    n = ctypes.c_longlong()
    _check(lib.chunkattn_plan_debug(chunk_len, n_chunks, heads, ctx.xcd_count, ctx.block_rows,
                                    None, 0, ctypes.byref(n)))
    dev = torch.device("cuda", ctx.device)
    items = torch.full((max(n.value, 1), 7), -7, dtype=torch.int32, device=dev)
    _check(lib.chunkattn_plan_device(ctx.handle, chunk_len, n_chunks, heads,
                                     ctypes.c_void_p(items.data_ptr()), n.value,
                                     _stream(items, None)), ctx.handle)
    return items[: n.value]


# floats the matrix-core probe writes per workgroup (8 waves x 8 accumulators
# x 64 lanes x 4)
PROBE_OUT_PER_WORKGROUP = 8 * 8 * 64 * 4
PROBE_WORDS = 64 * 32


def mfma_probe(operands, iters: int, out, ctx=None, stream=None):
    """Matrix-core rate probe (chunkattn_mfma_probe): operands is an int32
    device tensor of 64 x 32 words (bf16 pairs), out a float32 device tensor of
    at least ctx.cu_count * PROBE_OUT_PER_WORKGROUP elements.  Enqueues one
    launch; returns (workgroups, FLOPs of the launch)."""
    lib = load_library()
    ctx = ctx or create(operands.device.index or 0)
    if operands.numel() != PROBE_WORDS or operands.element_size() != 4:
        raise ValueError(f"chunkattn: operands must hold {PROBE_WORDS} 32-bit words")
    if out.dtype.itemsize != 4 or out.numel() < ctx.cu_count * PROBE_OUT_PER_WORKGROUP:
        raise ValueError("chunkattn: out must hold cu_count * PROBE_OUT_PER_WORKGROUP floats")
    for name, t in (("operands", operands), ("out", out)):
        _require(t, name, operands.device)
    n_wg = ctypes.c_int()
    flops = ctypes.c_double()
    _check(lib.chunkattn_mfma_probe(ctx.handle, ctypes.c_void_p(operands.data_ptr()), iters,
                                    ctypes.c_void_p(out.data_ptr()), ctypes.byref(n_wg),
                                    ctypes.byref(flops), _stream(out, stream)), ctx.handle)
    return n_wg.value, flops.value


def validate_queue_step(q_ptr, k_ptr, v_ptr, cache_ptr, out_ptr, chunk_len, n_chunks, heads,
                        head_dim, scale, dtype):
    """(status, message) of the device-free argument checks of queue_step."""
    lib = load_library()
    rc = lib.chunkattn_validate_queue_step(q_ptr, k_ptr, v_ptr, cache_ptr, out_ptr, chunk_len,
                                           n_chunks, heads, head_dim, scale, dtype)
    return rc, lib.chunkattn_last_error(None).decode()


def validate_full(q_ptr, k_ptr, v_ptr, out_ptr, batch, lq, lkv, kv_batch_stride, heads,
                  head_dim, scale, dtype):
    """(status, message) of the device-free argument checks of full."""
    lib = load_library()
    rc = lib.chunkattn_validate_full(q_ptr, k_ptr, v_ptr, out_ptr, batch, lq, lkv,
                                     kv_batch_stride, heads, head_dim, scale, dtype)
    return rc, lib.chunkattn_last_error(None).decode()


def validate_window_step(q_ptr, k_ptr, v_ptr, cache_ptr, out_ptr, chunk_len, n_chunks, heads,
                         head_dim, scale, dtype):
    """(status, message) of the device-free argument checks of window_step."""
    lib = load_library()
    rc = lib.chunkattn_validate_window_step(q_ptr, k_ptr, v_ptr, cache_ptr, out_ptr, chunk_len,
                                            n_chunks, heads, head_dim, scale, dtype)
    return rc, lib.chunkattn_last_error(None).decode()


def validate_ring_step(q_ptr, k_ptr, v_ptr, out_ptr, slots, tail_slot, n_live, chunk_len, heads,
                       head_dim, scale, dtype):
    """(status, message) of the device-free argument checks of ring_step."""
    lib = load_library()
    rc = lib.chunkattn_validate_ring_step(q_ptr, k_ptr, v_ptr, out_ptr, slots, tail_slot, n_live,
                                          chunk_len, heads, head_dim, scale, dtype)
    return rc, lib.chunkattn_last_error(None).decode()
