"""Seeded synthetic inputs for the chunk-attention queue step.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  The GPU path and the CPU oracle both consume exactly the
tensors produced here.

Distributions (the pages run trained video DiTs on real prompts; there are no
weights or prompts here, so seeded Gaussian activations of the same shapes
stand in for them):

* Q, V and text K/V: i.i.d. N(0, 1).
* "Correlated" K (and V when asked): an elementwise AR(1) across chunks in
  processing order, x_0 = z_0, x_c = rho * x_{c-1} + innov * z_c, drawn in
  fp32 at equal (token, head, dim) positions, which mimics the temporal
  redundancy of neighbouring video chunks.  rho = 0.9 and innov = 0.44 keep
  the marginal variance at ~1 (0.9^2 + 0.44^2 = 1.0036).
* Storage rounding to bf16 is round-to-nearest-even (torch's conversion).

Every tensor comes from its own torch.Generator seeded with
``seed * 1000 + tensor_id``, on the device the tensor is created on.  The
same seed on a different device gives different values; a test always feeds
one generated set to both sides.
"""
from __future__ import annotations

import torch

Q_ID, K_ID, V_ID, QX_ID, KT_ID, VT_ID = 1, 2, 3, 4, 5, 6


def _gen(device, seed: int, tensor_id: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000 + int(tensor_id))
    return g


def normal(shape, seed: int, tensor_id: int, device="cpu", dtype=torch.bfloat16):
    """i.i.d. N(0,1) drawn in fp32, stored in ``dtype``."""
    g = _gen(device, seed, tensor_id)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def ar1_chunks(n, chunk_shape, seed: int, tensor_id: int, device="cpu",
               dtype=torch.bfloat16, rho: float = 0.9, innov: float = 0.44):
    """[n, *chunk_shape] with an elementwise AR(1) across the leading axis.

    Generated chunk by chunk in fp32 so host/device memory stays bounded by one
    fp32 chunk plus the stored output.
    """
    g = _gen(device, seed, tensor_id)
    out = torch.empty((n, *chunk_shape), device=device, dtype=dtype)
    prev = None
    for c in range(n):
        z = torch.randn(*chunk_shape, generator=g, device=device, dtype=torch.float32)
        cur = z if prev is None else prev.mul_(rho).add_(z, alpha=innov)
        out[c].copy_(cur)
        prev = cur
    return out


def queue_inputs(n, L, H, D, seed: int, device="cpu", dtype=torch.bfloat16,
                 k_rho: float | None = None, v_rho: float | None = None,
                 innov: float = 0.44):
    """(q, k, v), each [n][L][H][D].  k_rho / v_rho switch on the AR(1)."""
    q = normal((n, L, H, D), seed, Q_ID, device, dtype)
    if k_rho is None:
        k = normal((n, L, H, D), seed, K_ID, device, dtype)
    else:
        k = ar1_chunks(n, (L, H, D), seed, K_ID, device, dtype, k_rho, innov)
    if v_rho is None:
        v = normal((n, L, H, D), seed, V_ID, device, dtype)
    else:
        v = ar1_chunks(n, (L, H, D), seed, V_ID, device, dtype, v_rho, innov)
    return q, k, v


def build_cache(k, v, poison_slot0: bool = True):
    """Separate predecessor cache [n][2][L][H][D]: slot c holds (k[c-1], v[c-1]).

    Slot 0 is never read (chunk 0 has no predecessor); it is filled with NaN
    when ``poison_slot0`` so that any read of it shows in the output.
    """
    n = k.shape[0]
    cache = torch.empty((n, 2, *k.shape[1:]), device=k.device, dtype=k.dtype)
    if n > 0:
        cache[0].fill_(float("nan") if poison_slot0 else 0.0)
    if n > 1:
        cache[1:, 0].copy_(k[:-1])
        cache[1:, 1].copy_(v[:-1])
    return cache


def text_inputs(n_text, H, D, seed: int, device="cpu", dtype=torch.bfloat16):
    """Shared text K/V for cross-attention, each [1][n_text][H][D]."""
    kt = normal((1, n_text, H, D), seed, KT_ID, device, dtype)
    vt = normal((1, n_text, H, D), seed, VT_ID, device, dtype)
    return kt, vt


def cross_queries(n, L, H, D, seed: int, device="cpu", dtype=torch.bfloat16):
    """Per-chunk cross-attention queries [n][L][H][D]."""
    return normal((n, L, H, D), seed, QX_ID, device, dtype)


PROBE_ID = 7


def probe_operands(seed: int, device="cpu") -> torch.Tensor:
    """Operands of the matrix-core rate probe: 64 lanes x 32 words, each word a
    pair of bf16 values drawn uniformly from {-1, 0, 1} (low half first), as
    int32.  Small integers keep every product and sum of the probe exact."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 1000 + PROBE_ID)
    vals = torch.randint(-1, 2, (64, 64), generator=g).to(torch.float32)
    bits = vals.to(torch.bfloat16).view(torch.int16).to(torch.int32) & 0xFFFF
    words = bits[:, 0::2] | (bits[:, 1::2] << 16)
    return words.to(torch.int32).contiguous().to(device)
