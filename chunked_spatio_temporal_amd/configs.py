"""Workload registry: the five synthetic shapes the path is tested and timed on.

Token counts follow latent video grids: a chunk of F latent frames at an
h x w patch grid holds F*h*w tokens (Wan-class 480p latents are 30x52 patches,
720p latents 45x80).  FLOPs are counted as 4 * Lq * Lkv * D per (query block,
head): Q.K^T and P.V each 2 FLOPs per multiply-add; softmax is not counted.
Chunk 0 has a zero-length cache, so it is counted with Lkv = L.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "queue", "window", "stream", "full" or "cross"
    n: int                    # chunks (queue) or batch (full)
    L: int                    # tokens per chunk (queue) or Lq (full)
    H: int
    D: int
    dtype: str                # "bf16" or "f32"
    lkv: int = 0              # full attention only
    k_rho: float | None = None
    v_rho: float | None = None
    n_text: int = 0           # per-chunk cross-attention to shared text tokens
    seed: int = 0
    note: str = ""
    grid: tuple = field(default=())

    @property
    def scale(self) -> float:
        return self.D ** -0.5

    def self_flops(self) -> float:
        """Exact FLOPs of the self-attention call."""
        if self.kind in ("queue", "stream"):
            if self.n == 0:
                return 0.0
            kv_rows = self.L * self.L + (self.n - 1) * self.L * 2 * self.L
            return 4.0 * kv_rows * self.D * self.H
        if self.kind == "window":
            # window c: queries of chunks c and c+1 over chunks c-1, c, c+1
            pairs = 0
            for c in range(self.n):
                q_chunks = 2 if c + 1 < self.n else 1
                kv_chunks = 1 + (c >= 1) + (c + 1 < self.n)
                pairs += q_chunks * kv_chunks
            return 4.0 * pairs * self.L * self.L * self.D * self.H
        # full attention; cross-attention: every query row over the lkv shared text rows
        return 4.0 * self.n * self.L * self.lkv * self.D * self.H

    def nominal_flops(self) -> float:
        """Every chunk counted with a full 2L window (the nominal figure)."""
        return 4.0 * self.n * self.L * 2 * self.L * self.D * self.H

    def cross_flops(self) -> float:
        return 4.0 * self.n * self.L * self.n_text * self.D * self.H

    def total_flops(self) -> float:
        return self.self_flops() + self.cross_flops()


WORKLOADS = {
    "tiny": Workload("tiny", "queue", n=4, L=128, H=2, D=64, dtype="f32", seed=0,
                     grid=(2, 8, 8),
                     note="4 chunks x (2 frames x 8x8 patches), fp32 in/out, iid N(0,1)"),
    "wan1.3b": Workload("wan1.3b", "queue", n=8, L=6240, H=12, D=128, dtype="bf16",
                        k_rho=0.9, seed=1, grid=(4, 30, 52),
                        note="8 chunks x (4 frames x 30x52), K AR(1) rho 0.9"),
    "wan14b": Workload("wan14b", "queue", n=8, L=6240, H=40, D=128, dtype="bf16",
                       k_rho=0.9, seed=2, grid=(4, 30, 52),
                       note="8 chunks x (4 frames x 30x52), 40 heads, K AR(1) rho 0.9"),
    "full32k": Workload("full32k", "full", n=1, L=32760, lkv=32760, H=12, D=128,
                        dtype="bf16", seed=3, grid=(21, 30, 52),
                        note="non-chunked bidirectional attention, 21 frames x 30x52"),
    "720p16": Workload("720p16", "queue", n=16, L=14400, H=40, D=128, dtype="bf16",
                       k_rho=0.9, v_rho=0.9, n_text=512, seed=4, grid=(4, 45, 80),
                       note="16 chunks x (4 frames x 45x80), K and V AR(1) rho 0.9, "
                            "plus cross-attention to 512 shared text tokens"),
    "win14b": Workload("win14b", "window", n=8, L=6240, H=40, D=128, dtype="bf16",
                       k_rho=0.9, seed=5, grid=(4, 30, 52),
                       note="the 40-head queue in the three-chunk window form: window c's "
                            "queries are chunks c and c+1, its keys chunks c-1 (cached), c, c+1"),
    "stream14b": Workload("stream14b", "stream", n=8, L=6240, H=40, D=128, dtype="bf16",
                          k_rho=0.9, seed=6, grid=(4, 30, 52),
                          note="the 40-head queue as a stream in steady state: 8 live chunks "
                               "in a ring of 9 slots; each step a chunk enters, all 8 are "
                               "processed, the clean head leaves"),
    "wan14b_h5": Workload("wan14b_h5", "queue", n=8, L=6240, H=5, D=128, dtype="bf16",
                          k_rho=0.9, seed=2, grid=(4, 30, 52),
                          note="one GPU's share of the 40-head queue when its heads are split "
                               "over 8 GPUs: 5 heads"),
    "cross720p": Workload("cross720p", "cross", n=16, L=14400, H=40, D=128, dtype="bf16",
                          lkv=512, seed=4, grid=(4, 45, 80),
                          note="the 720p queue's per-chunk cross-attention alone: 16 x 14400 "
                               "queries over 512 shared text tokens"),
}

# The timed workload: the 40-head, 480p-latent queue step.
BENCH_WORKLOAD = "wan14b"


@dataclass(frozen=True)
class NoiseWorkload:
    """Coordinated noise initialization of one new chunk: `frames` latent
    frames from a pool of `pool_frames`, avoiding the `excl` frames used by
    the tail chunk's last latent frames."""
    name: str
    pool_frames: int
    frames: int
    excl: int
    frame_shape: tuple        # (channels, height, width) of one latent frame
    dtype: str
    seed: int = 0
    note: str = ""

    def bytes_per_init(self, elem_bytes: int) -> int:
        """Frames read from the pool plus frames written (the selection itself
        moves a few KB)."""
        n = 1
        for x in self.frame_shape:
            n *= x
        return 2 * self.frames * n * elem_bytes


NOISE_WORKLOADS = {
    # 4 latent frames per chunk (the 480p queue's chunk: 4 frames of 30x52
    # patches = 60x104 latents, 16 channels), pool of 2 chunks, NumC/2 = 2
    "noise480p": NoiseWorkload("noise480p", pool_frames=8, frames=4, excl=2,
                               frame_shape=(16, 60, 104), dtype="f32", seed=7,
                               note="one chunk's noise for the 480p queue"),
    # a whole 81-frame video's latents (21 frames) from a pool of 42
    "noise480p_video": NoiseWorkload("noise480p_video", pool_frames=42, frames=21, excl=10,
                                     frame_shape=(16, 60, 104), dtype="f32", seed=8,
                                     note="21 latent frames from a pool of 42"),
}
