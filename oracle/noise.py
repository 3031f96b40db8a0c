"""Coordinated noise initialization of a new chunk (TEST INFRASTRUCTURE).

Follows "双重并行：让AI视频生成突破时长限制" (techwalker write-up of DualParal),
section 三, second improvement: DiT video models keep global consistency when
the whole noise space is used, and degrade when the same noise recurs; so a
new chunk's noise is taken from a shared pool, leaving out the noise used by
the last NumC/2 latent frames of the chunk at the tail of the queue (its
temporal neighbour), and the chosen noise is shuffled before it initializes
the new chunk.

Reading used here.  The pool holds P noise frames.  A chunk has F latent
frames; E = NumC/2 frames of the tail chunk are excluded (NumC, undefined in
the write-up, is read as the latent frames per chunk, so E = F/2 by default).
The random draw is given as one 32-bit key per pool frame: the candidates
(pool frames not used by the tail chunk's last E frames) taken in ascending
(key, pool index) order, first F of them, are the new chunk's frames in order
- a uniformly random subset in uniformly random order when the keys are
uniform.  The new chunk's noise frame f is pool frame idx[f], copied exactly.

Only the tests import this module.
"""
import numpy as np


def select(pool_size, keys, n_frames, prev_idx=None, n_excl=0):
    """Pool indices of the new chunk's frames, in frame order.

    keys: P uint32 keys; prev_idx: the tail chunk's pool indices in frame order
    (None for the first chunk); n_excl: how many of its last frames to avoid."""
    keys = np.asarray(keys, np.uint32)
    if keys.shape != (pool_size,):
        raise ValueError("one key per pool frame")
    excluded = set()
    if prev_idx is not None and n_excl > 0:
        prev_idx = list(prev_idx)
        excluded = set(prev_idx[len(prev_idx) - n_excl:])
    candidates = [p for p in range(pool_size) if p not in excluded]
    if len(candidates) < n_frames:
        raise ValueError("pool too small for the frames after the exclusion")
    candidates.sort(key=lambda p: (int(keys[p]), p))
    return np.array(candidates[:n_frames], np.int64)


def init_chunk(pool, idx):
    """The new chunk's noise: pool frames idx, in order (exact copies)."""
    pool = np.asarray(pool)
    return pool[np.asarray(idx)].copy()
