"""fp32 calls computed in fp32 (chunk_attn_fwd_f32: fp32 matrix cores, fp32
running-maximum softmax, fp32 output), against the fp64 oracle over every
output element.

DualParal write-up, section 三: each chunk attends over the cached K/V of its
predecessor and its own; the fp32 configuration keeps fp32 storage, and here
fp32 arithmetic too, so the error is that of fp32 rounding rather than of bf16
operands (bf16 operand rounding alone gives a relative L2 error near 2e-3).

Bound per element (derived, not fitted).  A score S_j = c * sum_i q_i k_ji
accumulated in fp32 over D terms is off by at most (D + 1) 2^-24 c sum_i
|q_i k_ji|; a score error dS moves each normalised weight by at most 2 |dS|
relative, so the output by at most 2 max_j |dS_j| (max_j |V_jd - O_d|).  The
fp32 sums of the numerators and of P V over N keys add at most 2 (N + 1)
2^-24 relative, the exponentials and the final division a few ulps.  Every
element must lie within that bound; the relative L2 error, far below it in
practice, is held to 1e-5 for unit-scale inputs.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from chunked_spatio_temporal_amd import chunkattn as ca
from chunked_spatio_temporal_amd import configs, synth
from parity_util import error_stats, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EPS = 2.0 ** -24


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ca.load_library()
    yield


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def key_sets(q, k, v, cache):
    """Per chunk c: (K, V) of its key set, [N_c][H][D] fp64 (predecessor rows
    first; the cache, when given, holds the predecessor's K/V)."""
    kk, vv = to_f64(k), to_f64(v)
    cc = None if cache is None else to_f64(cache)
    out = []
    for c in range(kk.shape[0]):
        if c == 0:
            out.append((kk[0], vv[0]))
        else:
            pk, pv = (kk[c - 1], vv[c - 1]) if cc is None else (cc[c, 0], cc[c, 1])
            out.append((np.concatenate([pk, kk[c]]), np.concatenate([pv, vv[c]])))
    return out


def fp32_bound(qc, kc, vc, ref_c, scale):
    """Per-element bound for the rows of one chunk (or batch item): qc [L][H][D],
    kc/vc [N][H][D], ref_c [L][H][D] (fp64)."""
    D = qc.shape[-1]
    N = kc.shape[0]
    b = np.empty_like(ref_c)
    for h in range(qc.shape[1]):
        # max_j sum_i |q_i k_ji| per query row
        s_abs = np.abs(qc[:, h, :]) @ np.abs(kc[:, h, :]).T  # [L][N]
        ds = (D + 1) * EPS * scale * s_abs.max(axis=1)  # [L]
        spread = np.abs(vc[:, h, :]).max(axis=0)[None, :] + np.abs(ref_c[:, h, :])
        rel = 2.0 * ds[:, None] + 2.0 * (N + 1) * EPS + 16 * EPS
        b[:, h, :] = rel * spread
    return b + 1e-9


def check(got, ref, bound, what, rel_l2=1e-5):
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    worst = float((err / bound).max())
    s = error_stats(got, ref)
    say(what, "max-abs", s["max_abs"], "rel-L2", s["rel_l2"], "worst/bound", worst)
    assert worst <= 1.0, f"{what}: error {worst:.3f}x the fp32 bound"
    assert s["rel_l2"] <= rel_l2, f"{what}: relative L2 {s['rel_l2']:.3g}"
    return s


def queue_bound(q, k, v, cache, ref, scale):
    qq = to_f64(q)
    return np.stack([fp32_bound(qq[c], kc, vc, ref[c], scale)
                     for c, (kc, vc) in enumerate(key_sets(q, k, v, cache))])


@pytest.mark.parametrize("n,L,H,D", [(4, 128, 2, 64), (3, 300, 2, 128), (4, 97, 3, 64),
                                     (1, 1, 1, 128), (2, 1000, 3, 128), (8, 700, 8, 64)],
                         ids=["tiny", "300x128", "97x64", "single", "1000x128", "many-items"])
def test_queue_step_fp32(n, L, H, D):
    """Ragged tiles, a tile straddling the predecessor and own segments, a
    one-token queue, and a launch of 704 work items (more than the CUs)."""
    say("case f32 queue", (n, L, H, D))
    q, k, v = synth.queue_inputs(n, L, H, D, seed=700 + L, device=DEV, dtype=torch.float32,
                                 k_rho=0.9)
    cache = synth.build_cache(k, v)
    scale = D ** -0.5
    out_c = ca.queue_step(q, k, v, cache, scale=scale)
    out_a = ca.queue_step(q, k, v, None, scale=scale)
    torch.cuda.synchronize()
    assert out_c.dtype == torch.float32
    assert torch.equal(out_c, out_a), "cache and in-place predecessor differ"
    ref = oracle.queue_step(q, k, v, None, scale=scale)
    check(to_f64(out_c), ref, queue_bound(q, k, v, cache, ref, scale), f"queue {(n, L, H, D)}")


def test_tiny_workload_fp32():
    """The fp32 configuration itself (4 chunks x 128 tokens, 2 heads, d 64)."""
    w = configs.WORKLOADS["tiny"]
    q, k, v = synth.queue_inputs(w.n, w.L, w.H, w.D, w.seed, device=DEV, dtype=torch.float32)
    out = ca.queue_step(q, k, v, None, scale=w.scale)
    torch.cuda.synchronize()
    ref = oracle.queue_step(q, k, v, None, scale=w.scale)
    check(to_f64(out), ref, queue_bound(q, k, v, None, ref, w.scale), "tiny")


@pytest.mark.parametrize("std", [5.0, 20.0])
def test_peaked_logits_fp32(std):
    """Natural-logit std 5 and 20 (maxima far beyond fp32's exponent range
    without a maximum): the running maximum keeps every row in range."""
    n, L, H, D = 3, 400, 2, 128
    q = synth.normal((n, L, H, D), 801, synth.Q_ID, DEV, torch.float32) * std
    k = synth.normal((n, L, H, D), 801, synth.K_ID, DEV, torch.float32)
    v = synth.normal((n, L, H, D), 801, synth.V_ID, DEV, torch.float32)
    scale = D ** -0.5
    out = ca.queue_step(q, k, v, None, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.queue_step(q, k, v, None, scale=scale)
    check(to_f64(out), ref, queue_bound(q, k, v, None, ref, scale), f"peaked {std}",
          rel_l2=1e-4)


def test_window_step_fp32():
    n, L, H, D = 3, 200, 2, 128
    q, k, v = synth.queue_inputs(n, L, H, D, seed=802, device=DEV, dtype=torch.float32)
    cache = synth.build_cache(k, v)
    scale = D ** -0.5
    out = ca.window_step(q, k, v, cache, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.window_step(q, k, v, None, scale=scale)
    got = to_f64(out)
    qq, kk, vv = to_f64(q), to_f64(k), to_f64(v)
    for c in range(n):
        parts = [kk[c - 1]] if c >= 1 else []
        vparts = [vv[c - 1]] if c >= 1 else []
        rows = [qq[c]]
        parts.append(kk[c]); vparts.append(vv[c])
        if c + 1 < n:
            parts.append(kk[c + 1]); vparts.append(vv[c + 1]); rows.append(qq[c + 1])
        kc, vc = np.concatenate(parts), np.concatenate(vparts)
        nr = len(rows)
        rc = ref[c, :nr].reshape(nr * L, H, D)
        b = fp32_bound(np.concatenate(rows), kc, vc, rc, scale)
        check(got[c, :nr].reshape(nr * L, H, D), rc, b, f"window {c}")


@pytest.mark.parametrize("B,lq,lkv,H,D,shared", [(3, 200, 77, 2, 128, True),
                                                 (1, 1000, 1000, 2, 64, False),
                                                 (2, 129, 1, 1, 64, False)],
                         ids=["shared-kv", "1000", "one-key"])
def test_full_fp32(B, lq, lkv, H, D, shared):
    q = synth.normal((B, lq, H, D), 803, synth.Q_ID, DEV, torch.float32)
    kb = 1 if shared else B
    k = synth.normal((kb, lkv, H, D), 803, synth.K_ID, DEV, torch.float32)
    v = synth.normal((kb, lkv, H, D), 803, synth.V_ID, DEV, torch.float32)
    scale = D ** -0.5
    out = ca.full(q, k, v, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.full(q, k, v, scale=scale)
    qq, kk, vv, got = to_f64(q), to_f64(k), to_f64(v), to_f64(out)
    for b in range(B):
        kbi = 0 if shared else b
        check(got[b], ref[b], fp32_bound(qq[b], kk[kbi], vv[kbi], ref[b], scale),
              f"full b{b} {(B, lq, lkv, H, D)}")


def test_fp32_calls_use_the_fp32_kernel():
    """Every context runs fp32 calls on 64-row fp32 items, whatever its flags."""
    for flags in (0, ca.FLAG_BLOCK128, ca.FLAG_BLOCK256, ca.FLAG_EXACT_SCALE):
        ctx = ca.Context(0, flags)
        assert ctx.call_block_rows(128, ca.F32) == 64
        assert ctx.call_block_rows(64, ca.F32) == 64
