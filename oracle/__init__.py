"""fp64 CPU oracle for the chunk-attention queue step (TEST INFRASTRUCTURE).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  It wraps ``oracle.c`` (plain C, fp64,
OpenMP) through ctypes; array marshalling is all that happens here.  See the
header of ``oracle.c`` for what is computed and which passages it follows:
block-wise denoising over a FIFO chunk queue and the self-attention K/V
feature cache (DualParal write-up, sections 二 and 三), and plain
spatio-temporal softmax attention (video-diffusion survey, section 2.1).

Parity status of each entry point (what pins it, in tests/test_oracle_pins.py):
  queue_step / queue_rows  pinned: brute-force block-band masked attention over
                           the explicitly concatenated sequence, torch SDPA,
                           constant-V, permutation invariance, closed forms,
                           golden fixtures
  queue_probs              pinned: rows sum to 1, closed-form weights
  full / full_rows         pinned: torch SDPA, n_chunks=1 reduction, closed forms
  index_map                pinned: brute-force enumeration of the band mask
  window_step / window_rows
                           pinned: brute-force masked attention over the
                           concatenated sequence with the three-chunk window
                           mask, single-chunk reduction to full attention,
                           constant-V and closed forms, golden fixtures
  window_index_map         pinned: brute-force enumeration of the window mask
  ring_rows / ring_slot    pinned: the linear queue step on the chunks gathered
                           from their slots, wrap-around closed forms
  fifo.Fifo / fifo.run     pinned: the queue properties the page states (noise
                           falls from tail to head, depth steps per chunk,
                           arrival order kept, bounded length)
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# A test may point this at a deliberately broken build of oracle.c to check
# that the pins catch the planted mistake (tests/test_oracle_mutations.py).
LIB_PATH = os.environ.get("CHUNKATTN_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

BF16, F32, F64 = 0, 1, 2
SRC_PRED, SRC_OWN = 0, 1

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, dbl, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
    lib.oracle_num_threads.restype = i32
    lib.oracle_kv_set_size.restype = i64
    lib.oracle_kv_set_size.argtypes = [i64, i64]
    lib.oracle_index_map.restype = i64
    lib.oracle_index_map.argtypes = [i64, i64, i64, vp, vp, vp]
    lib.oracle_queue_rows.restype = i32
    lib.oracle_queue_rows.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i64, dbl, vp, i64, vp]
    lib.oracle_queue_step.restype = i32
    lib.oracle_queue_step.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i64, dbl, vp]
    lib.oracle_queue_probs.restype = i32
    lib.oracle_queue_probs.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i64, dbl,
                                       i64, i64, i64, vp, vp]
    lib.oracle_window_q_rows.restype = i64
    lib.oracle_window_q_rows.argtypes = [i64, i64, i64]
    lib.oracle_window_kv_set_size.restype = i64
    lib.oracle_window_kv_set_size.argtypes = [i64, i64, i64]
    lib.oracle_window_index_map.restype = i64
    lib.oracle_window_index_map.argtypes = [i64, i64, i64, vp, vp, vp]
    lib.oracle_window_rows.restype = i32
    lib.oracle_window_rows.argtypes = [i32, vp, vp, vp, vp, i64, i64, i64, i64, dbl, vp, i64,
                                       vp]
    lib.oracle_ring_slot.restype = i64
    lib.oracle_ring_slot.argtypes = [i64, i64, i64]
    lib.oracle_ring_rows.restype = i32
    lib.oracle_ring_rows.argtypes = [i32, vp, vp, vp, i64, i64, i64, i64, i64, i64, dbl, vp,
                                     i64, vp]
    lib.oracle_full_rows.restype = i32
    lib.oracle_full_rows.argtypes = [i32, vp, vp, vp, i64, i64, i64, i64, i64, i64, dbl,
                                     vp, i64, vp]
    _lib = lib
    return lib


def _as_host(x):
    """Return (contiguous numpy array holding the exact stored bits, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                x = x.cpu()
            x = x.contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            if x.dtype == torch.float64:
                return x.numpy(), F64
            raise TypeError(f"oracle: unsupported tensor dtype {x.dtype}")
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.uint16:
        return x, BF16
    raise TypeError(f"oracle: unsupported array dtype {x.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _common(q, k, v, kv_cache):
    qa, dt = _as_host(q)
    ka, dk = _as_host(k)
    va, dv = _as_host(v)
    if not (dt == dk == dv):
        raise TypeError("oracle: q, k, v must share one storage type")
    ca = None
    if kv_cache is not None:
        ca, dc = _as_host(kv_cache)
        if dc != dt:
            raise TypeError("oracle: kv_cache must share the storage type of q")
    if qa.ndim != 4 or ka.shape != qa.shape or va.shape != qa.shape:
        raise ValueError("oracle: q, k, v must all be [n_chunks][L][H][D]")
    n, L, H, D = qa.shape
    if ca is not None and ca.shape != (n, 2, L, H, D):
        raise ValueError("oracle: kv_cache must be [n_chunks][2][L][H][D]")
    return qa, ka, va, ca, dt, (n, L, H, D)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def kv_set_size(chunk_len: int, c: int) -> int:
    return int(_load().oracle_kv_set_size(chunk_len, c))


def index_map(chunk_len: int, n_chunks: int, c: int):
    """(src, chunk, row) int64 arrays describing R_c entry by entry."""
    lib = _load()
    m = kv_set_size(chunk_len, c)
    src = np.empty(m, np.int64)
    ch = np.empty(m, np.int64)
    row = np.empty(m, np.int64)
    got = lib.oracle_index_map(chunk_len, n_chunks, c, _ptr(src), _ptr(ch), _ptr(row))
    if got != m:
        raise ValueError("oracle_index_map: bad arguments")
    return src, ch, row


def queue_step(q, k, v, kv_cache=None, scale=None) -> np.ndarray:
    """Whole queue step; returns fp64 [n_chunks][L][H][D]."""
    qa, ka, va, ca, dt, (n, L, H, D) = _common(q, k, v, kv_cache)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty((n, L, H, D), np.float64)
    rc = _load().oracle_queue_step(dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(ca), L, n, H, D,
                                   scale, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_queue_step failed ({rc})")
    return out


def queue_rows(q, k, v, kv_cache, rows, scale=None) -> np.ndarray:
    """Selected output rows; rows is an (N, 3) array of (chunk, head, row)."""
    qa, ka, va, ca, dt, (n, L, H, D) = _common(q, k, v, kv_cache)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 3))
    out = np.empty((rows.shape[0], D), np.float64)
    rc = _load().oracle_queue_rows(dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(ca), L, n, H, D,
                                   scale, _ptr(rows), rows.shape[0], _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_queue_rows failed ({rc})")
    return out


def queue_probs(q, k, v, kv_cache, c, h, r, scale=None):
    """(softmax weights over R_c in index-map order, output row)."""
    qa, ka, va, ca, dt, (n, L, H, D) = _common(q, k, v, kv_cache)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    probs = np.empty(kv_set_size(L, c), np.float64)
    out = np.empty(D, np.float64)
    rc = _load().oracle_queue_probs(dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(ca), L, n, H, D,
                                    scale, c, h, r, _ptr(probs), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_queue_probs failed ({rc})")
    return probs, out


def _full_common(q, k, v):
    qa, dt = _as_host(q)
    ka, dk = _as_host(k)
    va, dv = _as_host(v)
    if not (dt == dk == dv):
        raise TypeError("oracle: q, k, v must share one storage type")
    if qa.ndim != 4 or ka.ndim != 4 or va.shape != ka.shape:
        raise ValueError("oracle: q is [batch][Lq][H][D], k/v are [kv_batch][Lkv][H][D]")
    batch, lq, H, D = qa.shape
    kvb, lkv, Hk, Dk = ka.shape
    if (Hk, Dk) != (H, D) or kvb not in (1, batch):
        raise ValueError("oracle: k/v must have batch 1 (shared) or the batch of q")
    stride = 0 if (kvb == 1 and batch > 1) else lkv * H * D
    return qa, ka, va, dt, batch, lq, lkv, stride, H, D


def full(q, k, v, scale=None) -> np.ndarray:
    """Full attention; k/v with batch 1 are shared by every batch item."""
    qa, ka, va, dt, batch, lq, lkv, stride, H, D = _full_common(q, k, v)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty((batch, lq, H, D), np.float64)
    rc = _load().oracle_full_rows(dt, _ptr(qa), _ptr(ka), _ptr(va), batch, lq, lkv, stride,
                                  H, D, scale, None, 0, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_full_rows failed ({rc})")
    return out


def full_rows(q, k, v, rows, scale=None) -> np.ndarray:
    """Selected rows of full attention; rows is (N, 3) of (batch, head, row)."""
    qa, ka, va, dt, batch, lq, lkv, stride, H, D = _full_common(q, k, v)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 3))
    out = np.empty((rows.shape[0], D), np.float64)
    rc = _load().oracle_full_rows(dt, _ptr(qa), _ptr(ka), _ptr(va), batch, lq, lkv, stride,
                                  H, D, scale, _ptr(rows), rows.shape[0], _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_full_rows failed ({rc})")
    return out


def window_q_rows(chunk_len: int, n_chunks: int, c: int) -> int:
    return int(_load().oracle_window_q_rows(chunk_len, n_chunks, c))


def window_kv_set_size(chunk_len: int, n_chunks: int, c: int) -> int:
    return int(_load().oracle_window_kv_set_size(chunk_len, n_chunks, c))


def window_index_map(chunk_len: int, n_chunks: int, c: int):
    """(src, chunk, row) int64 arrays describing W_c entry by entry."""
    lib = _load()
    m = window_kv_set_size(chunk_len, n_chunks, c)
    src = np.empty(m, np.int64)
    ch = np.empty(m, np.int64)
    row = np.empty(m, np.int64)
    got = lib.oracle_window_index_map(chunk_len, n_chunks, c, _ptr(src), _ptr(ch), _ptr(row))
    if got != m:
        raise ValueError("oracle_window_index_map: bad arguments")
    return src, ch, row


def window_step(q, k, v, kv_cache=None, scale=None) -> np.ndarray:
    """Whole window step; returns fp64 [n_chunks][2][L][H][D] (window c: chunk c's
    query rows, then chunk c+1's; the second half of the last window is NaN)."""
    qa, ka, va, ca, dt, (n, L, H, D) = _common(q, k, v, kv_cache)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    out = np.empty((n, 2, L, H, D), np.float64)
    rc = _load().oracle_window_rows(dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(ca), L, n, H, D,
                                    scale, None, 0, _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_window_rows failed ({rc})")
    return out


def window_rows(q, k, v, kv_cache, rows, scale=None) -> np.ndarray:
    """Selected window-step rows; rows is (N, 3) of (window, head, row in [0, 2L))."""
    qa, ka, va, ca, dt, (n, L, H, D) = _common(q, k, v, kv_cache)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 3))
    out = np.empty((rows.shape[0], D), np.float64)
    rc = _load().oracle_window_rows(dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(ca), L, n, H, D,
                                    scale, _ptr(rows), rows.shape[0], _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_window_rows failed ({rc})")
    return out


def ring_slot(slots: int, tail_slot: int, c: int) -> int:
    return int(_load().oracle_ring_slot(slots, tail_slot, c))


def ring_rows(q, k, v, tail_slot, n_live, rows, scale=None) -> np.ndarray:
    """Queue step over the n_live chunks of ring buffers q, k, v [S][L][H][D]
    (chunk c in processing order in slot (tail_slot - c) mod S); rows is (N, 3)
    of (chunk c, head, row).  Returns fp64 (N, D)."""
    qa, ka, va, _, dt, (S, L, H, D) = _common(q, k, v, None)
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 3))
    out = np.empty((rows.shape[0], D), np.float64)
    rc = _load().oracle_ring_rows(dt, _ptr(qa), _ptr(ka), _ptr(va), S, tail_slot, n_live, L, H,
                                  D, scale, _ptr(rows), rows.shape[0], _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_ring_rows failed ({rc})")
    return out
