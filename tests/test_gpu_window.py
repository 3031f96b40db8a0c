"""GPU parity of the HIP window step (DualParal write-up, section 三: window
[B_{i-1}, B_i] with the cached K/V of B_{i+1}) against the fp64 oracle.

Window c's queries are chunk c's and chunk c+1's rows; its keys/values are
chunk c-1's (cached) and chunks c and c+1's own.  Calls go through the C-ABI
library's Python binding; small shapes are compared over every existing output
row, the 40-head full-size workload on sampled rows that the oracle computes on
the sub-problem of chunks c-1, c, c+1.
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
SENTINEL = 12345.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ca.load_library()
    yield


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# the default context (384-row items for bf16 head_dim 128, 256 otherwise) and
# the two fixed work-item sizes
FLAGS = [pytest.param(0, id="default"), pytest.param(ca.FLAG_BLOCK256, id="bm256"),
         pytest.param(ca.FLAG_BLOCK128, id="bm128")]


def run_window(q, k, v, cache=None, scale=None, flags=0):
    n, L, H, D = q.shape
    out = torch.full((n, 2, L, H, D), SENTINEL, dtype=q.dtype, device=q.device)
    ca.window_step(q, k, v, cache, out=out, scale=scale, ctx=ca.create(0, flags))
    torch.cuda.synchronize()
    return out


def valid_rows(out):
    """Window outputs that exist, flattened [rows, H, D] (the last window has
    no second half)."""
    n, _, L, H, D = out.shape
    parts = [out[c].reshape(2 * L, H, D) for c in range(n - 1)]
    parts.append(out[n - 1, 0])
    return torch.cat(parts, 0)


def oracle_valid(ref):
    n, _, L, H, D = ref.shape
    parts = [ref[c].reshape(2 * L, H, D) for c in range(n - 1)] + [ref[n - 1, 0]]
    return np.concatenate(parts, 0)


SHAPES = [
    # n, L, H, D, dtype
    (1, 1, 1, 64, torch.bfloat16),
    (1, 130, 2, 128, torch.bfloat16),
    (2, 31, 1, 128, torch.bfloat16),
    (3, 64, 2, 64, torch.bfloat16),
    (4, 97, 3, 128, torch.bfloat16),
    (3, 128, 1, 128, torch.float32),
    (5, 100, 2, 128, torch.bfloat16),
    (2, 333, 1, 64, torch.float32),
]


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}x{s[2]}x{s[3]}"
                         f"{'bf16' if s[4] == torch.bfloat16 else 'f32'}")
def test_window_shapes_full_parity(shape, flags):
    n, L, H, D, dt = shape
    say("case window", shape, flags)
    q, k, v = synth.queue_inputs(n, L, H, D, seed=200 + L, device=DEV, dtype=dt, k_rho=0.9)
    cache = synth.build_cache(k, v)
    ref = oracle.window_step(q, k, v, None)
    a = run_window(q, k, v, None, flags=flags)
    b = run_window(q, k, v, cache, flags=flags)
    assert_parity(to_f64(valid_rows(a)), oracle_valid(ref), f"window {shape}")
    assert torch.equal(a, b), "alias and cache modes differ"
    # the absent half of the last window is not written
    assert (a[n - 1, 1] == SENTINEL).all()


@pytest.mark.parametrize("flags", FLAGS)
def test_window_fingerprint_bit_exact(flags):
    """Q = 0 makes every weight exactly 1: window c's output at (r, h, d) is the
    number of tokens t of chunks c-1..c+1 with (t + 5h) mod D == d, over |W_c|,
    t the global token index.  A key row shifted by one, a wrong chunk, head or
    segment changes some entries of the rounded rational."""
    n, L, H, D = 4, 150, 2, 128
    q = torch.zeros((n, L, H, D), dtype=torch.bfloat16, device=DEV)
    k = synth.normal((n, L, H, D), 19, 2, DEV)
    t = torch.arange(n * L, device=DEV).view(n, L, 1, 1)
    hh = torch.arange(H, device=DEV).view(1, 1, H, 1)
    d = torch.arange(D, device=DEV).view(1, 1, 1, D)
    v = (((t + 5 * hh) % D) == d).to(torch.bfloat16)
    cache = synth.build_cache(k, v)
    for cc in (None, cache):
        out = run_window(q, k, v, cc, flags=flags).cpu()
        for c in range(n):
            toks = np.arange(max(c - 1, 0) * L, min(c + 2, n) * L)
            rows = 2 * L if c + 1 < n else L
            for h in range(H):
                counts = np.bincount((toks + 5 * h) % D, minlength=D) / len(toks)
                exp = torch.from_numpy(counts).float().to(torch.bfloat16)
                got = out[c, :, :, h, :].reshape(2 * L, D)[:rows]
                assert torch.equal(got, exp.expand(rows, D)), f"window {c} head {h}"


@pytest.mark.parametrize("flags", FLAGS)
def test_window_reductions_to_queue_step_bitwise(flags):
    """The last window has exactly the queue step's key/value set for that chunk
    (its predecessor and its own rows) and the same tile walk, so the bits agree;
    a one-chunk queue's window is the queue step of that chunk."""
    n, L, H, D = 3, 200, 2, 128
    q, k, v = synth.queue_inputs(n, L, H, D, seed=77, device=DEV)
    ctx = ca.create(0, flags)
    win = run_window(q, k, v, None, flags=flags)
    que = ca.queue_step(q, k, v, None, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(win[n - 1, 0], que[n - 1])
    win1 = run_window(q[:1], k[:1], v[:1], None, flags=flags)
    que1 = ca.queue_step(q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(), None, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(win1[0, 0], que1[0])


@pytest.mark.parametrize("flags", FLAGS)
def test_window_score_overflow_falls_back_exactly(flags):
    """Scores far above every row's first tile overflow the fixed-maximum pass;
    the recheck pass must return the exact softmax: all weight on chunk 1's
    last 50 own rows, which every window sees."""
    n, L, H, D = 2, 200, 2, 128
    q = torch.full((n, L, H, D), 20.0, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((n, L, H, D), dtype=torch.bfloat16, device=DEV)
    k[1, 150:] = 1.0
    v = synth.normal((n, L, H, D), 25, 3, DEV)
    cache = synth.build_cache(k, v)
    out = run_window(q, k, v, cache, flags=flags)
    ref = oracle.window_step(q, k, v, cache)
    assert_parity(to_f64(valid_rows(out)), oracle_valid(ref), "window overflow")
    exp = v[1, 150:].float().mean(0)
    torch.testing.assert_close(valid_rows(out).float(), exp.expand(3 * L, H, D), atol=1e-2,
                               rtol=0)


def test_window_empty_is_a_noop():
    z = torch.empty((0, 16, 2, 128), dtype=torch.bfloat16, device=DEV)
    out = ca.window_step(z, z, z)
    assert out.shape == (0, 2, 16, 2, 128)


def sample_window_rows(n, L, H, rng, per=20):
    bm = ca.block_rows()
    windows = sorted({0, 1, n - 2, n - 1, int(rng.integers(0, n))} & set(range(n)))
    heads = sorted({0, H - 1, int(rng.integers(0, H))})
    rows = []
    for c in windows:
        nq = 2 * L if c + 1 < n else L
        fixed = {0, 1, bm - 1, bm, L - 1, L, L + 1, nq - 1, nq - 2, (nq // bm) * bm}
        for h in heads:
            rs = {r for r in fixed if 0 <= r < nq} | set(rng.integers(0, nq, per).tolist())
            rows += [(c, h, r) for r in sorted(rs)]
    return np.array(rows, np.int64)


def window_rows_oracle(q, k, v, cache, rows, scale):
    """Oracle rows of the full problem, computed on the sub-problem of chunks
    c-1, c, c+1 (window c's whole key/value set)."""
    n = q.shape[0]
    out = np.empty((len(rows), q.shape[-1]))
    for c in np.unique(rows[:, 0]):
        lo, hi = max(int(c) - 1, 0), min(int(c) + 2, n)
        sub = lambda t: t[lo:hi].cpu()
        sel = rows[:, 0] == c
        r = rows[sel].copy()
        r[:, 0] -= lo
        out[sel] = oracle.window_rows(sub(q), sub(k), sub(v),
                                      None if cache is None else sub(cache), r, scale)
    return out


@pytest.mark.slow
def test_window_workload_sampled_parity():
    w = configs.WORKLOADS["win14b"]
    say("case workload", w.name, w)
    q, k, v = synth.queue_inputs(w.n, w.L, w.H, w.D, w.seed, device=DEV, k_rho=w.k_rho,
                                 v_rho=w.v_rho)
    cache = synth.build_cache(k, v)
    out = torch.full((w.n, 2, w.L, w.H, w.D), SENTINEL, dtype=q.dtype, device=DEV)
    ca.window_step(q, k, v, cache, out=out, scale=w.scale)
    torch.cuda.synchronize()
    assert (out[w.n - 1, 1] == SENTINEL).all()
    vals = valid_rows(out)
    assert torch.isfinite(vals).all()
    assert vals.float().abs().amax().item() <= v.float().abs().amax().item() * (1 + 2 ** -7)
    rows = sample_window_rows(w.n, w.L, w.H, np.random.default_rng(w.seed))
    ref = window_rows_oracle(q, k, v, cache, rows, w.scale)
    idx = torch.from_numpy(rows).to(out.device)
    got = to_f64(out[idx[:, 0], idx[:, 2] // w.L, idx[:, 2] % w.L, idx[:, 1]])
    s = assert_parity(got, ref, w.name)
    say(w.name, "sampled rows", len(rows), s)
    out2 = ca.window_step(q, k, v, None, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(valid_rows(out), valid_rows(out2))
