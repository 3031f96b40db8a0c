"""Every-element checks of the launches the benchmark times.

The full-size workloads run the persistent main pass with many work items per
workgroup (8000 items on 256 workgroups for the 40-head queue): the claim of
the next item, the hand-over to other dies' queues and the 64-bit offsets of
tensors over 2^31 bytes are exercised only there.  These tests check every
output element of such launches, not sampled rows:

* Range fingerprint at full size (DualParal write-up, section 三: the cached
  K/V of the neighbouring chunk must stand in exactly for the concatenated
  sequence).  With Q = 0 every weight is exactly 1, so output (c, r, h, d) is
  the number of key rows t of chunk c's key/value set whose one-hot V puts a 1
  in dimension d, over the size of that set: a closed form per (c, h, d) that
  numpy computes without the oracle.  The kernel's fp32 sums of ones are exact
  and the final division rounds to the same bf16 value, so the whole output is
  compared bit for bit.  A skipped, repeated, shifted or misplaced item, row,
  head or segment changes some entries.
* The output is prefilled with a finite sentinel that no correct output can
  take (outputs of the one-hot V lie in [0, 1]); a NaN prefill would not do,
  because the recheck pass recomputes every item whose first element is NaN.
* A launch with more work items than CUs at head_dim 64 and 128, compared
  with the fp64 oracle over the whole output.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from chunked_spatio_temporal_amd import chunkattn as ca
from chunked_spatio_temporal_amd import configs, synth
from parity_util import assert_parity, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = 7.0  # fingerprint outputs lie in [0, 1]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ca.load_library()
    yield


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def one_hot_v(n_tok, H, D, mult, modulus=None):
    """V[t, h, d] = 1 where (t + mult*h) mod modulus == d, else 0 (modulus D by
    default); shape [n_tok, H, D], bf16, built on the device."""
    m = D if modulus is None else modulus
    t = torch.arange(n_tok, device=DEV).view(n_tok, 1, 1)
    hh = torch.arange(H, device=DEV).view(1, H, 1)
    d = torch.arange(D, device=DEV).view(1, 1, D)
    return (((t + mult * hh) % m) == d).to(torch.bfloat16)


def range_counts(ranges, H, D, mult, modulus=None):
    """Closed form: for every (h, d), the number of tokens t in the union of the
    half-open ranges with (t + mult*h) mod modulus == d, i.e. t congruent to
    a = (d - mult*h) mod modulus: floor((hi-1-a)/m) - floor((lo-1-a)/m) per
    range.  Returns (counts [H, D] int64, total tokens)."""
    m = D if modulus is None else modulus
    h = np.arange(H).reshape(H, 1)
    d = np.arange(D).reshape(1, D)
    a = (d - mult * h) % m
    counts = np.zeros((H, D), np.int64)
    total = 0
    for lo, hi in ranges:
        counts += (hi - 1 - a) // m - (lo - 1 - a) // m
        total += hi - lo
    if m < D:
        counts[:, m:] = 0
    return counts, total


def expected_bf16(counts, total):
    return torch.from_numpy(counts / total).float().to(torch.bfloat16)


def mismatch_report(got, exp):
    bad = got != exp
    return (f"{int(bad.sum())} of {bad.numel()} elements differ; "
            f"{int((got == SENTINEL).sum())} still hold the sentinel")


# ------------------------------------------------------------------ queue step

@pytest.mark.slow
@pytest.mark.parametrize("name", ["wan14b", "720p16"])
@pytest.mark.parametrize("mode", ["cache", "alias"])
def test_queue_fingerprint_full_size_bit_exact(name, mode):
    w = configs.WORKLOADS[name]
    n, L, H, D = w.n, w.L, w.H, w.D
    mult = 7
    say("case queue fingerprint", name, mode, (n, L, H, D))
    q = torch.zeros((n, L, H, D), dtype=torch.bfloat16, device=DEV)
    k = synth.normal((n, L, H, D), w.seed, synth.K_ID, DEV)
    v = one_hot_v(n * L, H, D, mult).view(n, L, H, D)
    cache = synth.build_cache(k, v) if mode == "cache" else None
    out = torch.full_like(q, SENTINEL)
    ca.queue_step(q, k, v, cache, out=out, scale=w.scale)
    torch.cuda.synchronize()
    for c in range(n):
        lo = (c - 1) * L if c >= 1 else 0
        counts, total = range_counts([(lo, (c + 1) * L)], H, D, mult)
        exp = expected_bf16(counts, total).to(DEV)
        got = out[c]
        ok = torch.equal(got, exp.view(1, H, D).expand(L, H, D))
        assert ok, f"chunk {c}: " + mismatch_report(got, exp.view(1, H, D).expand(L, H, D))
    say(name, mode, "all", out.numel(), "elements exact")


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["cache", "alias"])
def test_window_fingerprint_full_size_bit_exact(mode):
    w = configs.WORKLOADS["win14b"]
    n, L, H, D = w.n, w.L, w.H, w.D
    mult = 5
    say("case window fingerprint", mode, (n, L, H, D))
    q = torch.zeros((n, L, H, D), dtype=torch.bfloat16, device=DEV)
    k = synth.normal((n, L, H, D), w.seed, synth.K_ID, DEV)
    v = one_hot_v(n * L, H, D, mult).view(n, L, H, D)
    cache = synth.build_cache(k, v) if mode == "cache" else None
    out = torch.full((n, 2, L, H, D), SENTINEL, dtype=torch.bfloat16, device=DEV)
    ca.window_step(q, k, v, cache, out=out, scale=w.scale)
    torch.cuda.synchronize()
    for c in range(n):
        lo = (c - 1) * L if c >= 1 else 0
        hi = min(c + 2, n) * L
        counts, total = range_counts([(lo, hi)], H, D, mult)
        exp = expected_bf16(counts, total).to(DEV).view(1, H, D)
        halves = 2 if c + 1 < n else 1
        for half in range(halves):
            got = out[c, half]
            assert torch.equal(got, exp.expand(L, H, D)), \
                f"window {c} half {half}: " + mismatch_report(got, exp.expand(L, H, D))
    # the last window has no second half: never written
    assert (out[n - 1, 1] == SENTINEL).all()


@pytest.mark.slow
def test_ring_fingerprint_full_size_bit_exact():
    """Steady state of the 40-head queue as a ring of 9 slots, depth 8, tail in
    slot 4 (wrapping round slot 0).  V is one-hot by physical token index
    slot*L + r, so chunk c's set is its own slot's range plus its
    predecessor's slot range; the one slot that is not live keeps the sentinel."""
    w = configs.WORKLOADS["wan14b"]
    S, depth, tail = 9, 8, 4
    L, H, D = w.L, w.H, w.D
    mult = 3
    say("case ring fingerprint", S, depth, tail, (L, H, D))
    q = torch.zeros((S, L, H, D), dtype=torch.bfloat16, device=DEV)
    k = synth.normal((S, L, H, D), 7, synth.K_ID, DEV)
    v = one_hot_v(S * L, H, D, mult).view(S, L, H, D)
    out = torch.full_like(q, SENTINEL)
    ca.ring_step(q, k, v, out, tail, depth, scale=w.scale)
    torch.cuda.synchronize()
    live = set()
    for c in range(depth):
        s = (tail - c) % S
        live.add(s)
        ranges = [(s * L, (s + 1) * L)]
        if c >= 1:
            p = (tail - c + 1) % S
            ranges.insert(0, (p * L, (p + 1) * L))
        counts, total = range_counts(ranges, H, D, mult)
        exp = expected_bf16(counts, total).to(DEV).view(1, H, D).expand(L, H, D)
        assert torch.equal(out[s], exp), f"chunk {c} (slot {s}): " + mismatch_report(out[s], exp)
    for s in set(range(S)) - live:
        assert (out[s] == SENTINEL).all(), f"slot {s} is not live but was written"


# ------------------------------------------------------------------ full attention

@pytest.mark.slow
def test_cross_attention_fingerprint_full_size_bit_exact():
    """The 720p queue's per-chunk cross-attention: 16 x 14400 queries over one
    shared set of 512 text rows (K/V batch stride 0).  V[j, h, d] = 1 where
    (j + 3h) mod 97 == d: dims below 97 count 5 or 6 of the 512 rows, the
    others none; 512 is a power of two, so every output is exact."""
    w = configs.WORKLOADS["720p16"]
    n, L, H, D, T = w.n, w.L, w.H, w.D, w.n_text
    say("case cross fingerprint", (n, L, H, D, T))
    qx = torch.zeros((n, L, H, D), dtype=torch.bfloat16, device=DEV)
    kt = synth.normal((1, T, H, D), w.seed, synth.K_ID, DEV)
    vt = one_hot_v(T, H, D, 3, modulus=97).view(1, T, H, D)
    ox = torch.full_like(qx, SENTINEL)
    ca.full(qx, kt, vt, out=ox, scale=w.scale)
    torch.cuda.synchronize()
    counts, total = range_counts([(0, T)], H, D, 3, modulus=97)
    exp = expected_bf16(counts, total).to(DEV).view(1, 1, H, D).expand(n, L, H, D)
    assert torch.equal(ox, exp), mismatch_report(ox, exp)


@pytest.mark.slow
def test_full_sequence_fingerprint_full_size_bit_exact():
    w = configs.WORKLOADS["full32k"]
    S, H, D = w.L, w.H, w.D
    say("case full32k fingerprint", (S, H, D))
    q = torch.zeros((1, S, H, D), dtype=torch.bfloat16, device=DEV)
    k = synth.normal((1, S, H, D), w.seed, synth.K_ID, DEV)
    v = one_hot_v(S, H, D, 11).view(1, S, H, D)
    out = torch.full_like(q, SENTINEL)
    ca.full(q, k, v, out=out, scale=w.scale)
    torch.cuda.synchronize()
    counts, total = range_counts([(0, S)], H, D, 11)
    exp = expected_bf16(counts, total).to(DEV).view(1, 1, H, D).expand(1, S, H, D)
    assert torch.equal(out, exp), mismatch_report(out, exp)


# ------------------------------------------------------------------ many items, oracle

_ORACLE = {}  # oracle outputs per shape, shared by the two work-item sizes


@pytest.mark.parametrize("flags", [pytest.param(0, id="default"),
                                   pytest.param(ca.FLAG_BLOCK256, id="bm256"),
                                   pytest.param(ca.FLAG_BLOCK128, id="bm128")])
@pytest.mark.parametrize("n,L,H,D", [(5, 800, 48, 64), (4, 900, 32, 128)],
                         ids=["d64", "d128"])
def test_many_items_whole_output_parity(n, L, H, D, flags):
    """More work items than CUs (960 and 512 at 256 rows per item, 1536 and
    896 at 128, 384 of 384 rows at head_dim 128 with the default context),
    ragged last query tiles, correlated keys: every output element against the
    fp64 oracle, the sentinel gone everywhere, and the in-place predecessor
    form bit-identical to the cache form."""
    say("case many items", (n, L, H, D), flags)
    ctx = ca.create(0, flags)
    q, k, v = synth.queue_inputs(n, L, H, D, seed=400 + D, device=DEV, k_rho=0.9)
    cache = synth.build_cache(k, v)
    out = torch.full_like(q, 2.0 ** 100)
    ca.queue_step(q, k, v, cache, out=out, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (out.float().abs() < 2.0 ** 99).all()
    key = (n, L, H, D)
    if key not in _ORACLE:
        _ORACLE[key] = oracle.queue_step(q, k, v, cache)
    ref = _ORACLE[key]
    s = assert_parity(to_f64(out), ref, f"many items {(n, L, H, D)}")
    say("stats", s)
    out2 = torch.full_like(q, 2.0 ** 100)
    ca.queue_step(q, k, v, None, out=out2, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
