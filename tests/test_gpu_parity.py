"""GPU parity of the HIP queue step and full attention against the fp64 oracle.

Every test calls the C-ABI library through its Python binding and compares
with the oracle on the same seeded inputs (chunked_spatio_temporal_amd.synth).
Small shapes are compared element by element over the whole output; the
full-size workloads (the same launch configuration the benchmark times) are
compared on sampled rows, which the oracle computes one by one on the
sub-problem of chunks c-1 and c, plus properties that hold at any size.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from chunked_spatio_temporal_amd import chunkattn as ca
from chunked_spatio_temporal_amd import configs, synth
from parity_util import assert_parity, error_stats, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ca.load_library()  # raises if the HIP library is not built
    yield


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# the default context (384-row items for bf16 head_dim 128, 256 otherwise) and
# the two fixed work-item sizes
FLAGS = [pytest.param(0, id="default"), pytest.param(ca.FLAG_BLOCK256, id="bm256"),
         pytest.param(ca.FLAG_BLOCK128, id="bm128")]
# the two persistent main passes (384- and 256-row items), which share the
# context's work-queue slots
PERSISTENT = [pytest.param(0, id="bm384"), pytest.param(ca.FLAG_BLOCK256, id="bm256")]


# Finite prefill of outputs that must be overwritten everywhere: above every
# output of finite inputs here, and not NaN (the recheck pass recomputes items
# whose first element is NaN, so a NaN prefill would hide a skipped item).
UNWRITTEN = 2.0 ** 100


def run_queue(q, k, v, cache=None, scale=None, flags=0):
    out = torch.full_like(q, UNWRITTEN)
    ca.queue_step(q, k, v, cache, out=out, scale=scale, ctx=ca.create(0, flags))
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------------ small / exact

@pytest.mark.parametrize("flags", FLAGS)
def test_tiny_config_full_parity(flags):
    w = configs.WORKLOADS["tiny"]
    say("case tiny", w, flags)
    q, k, v = synth.queue_inputs(w.n, w.L, w.H, w.D, w.seed, device=DEV, dtype=torch.float32)
    cache = synth.build_cache(k, v)
    ref = oracle.queue_step(q, k, v, None, scale=w.scale)
    out_alias = run_queue(q, k, v, None, w.scale, flags)
    out_cache = run_queue(q, k, v, cache, w.scale, flags)
    assert out_alias.dtype == torch.float32
    s = assert_parity(to_f64(out_alias), ref, "tiny alias")
    say("tiny stats", s)
    assert torch.equal(out_alias, out_cache), "alias and cache modes differ"


SHAPES = [
    # n, L, H, D, dtype
    (1, 1, 1, 64, torch.bfloat16),
    (5, 1, 2, 128, torch.bfloat16),
    (2, 31, 1, 128, torch.bfloat16),
    (3, 64, 2, 64, torch.bfloat16),
    (4, 97, 3, 128, torch.bfloat16),
    (2, 128, 1, 128, torch.float32),
    (3, 200, 2, 128, torch.bfloat16),
    (2, 333, 1, 64, torch.float32),
    (5, 129, 2, 128, torch.bfloat16),
    (1, 300, 3, 128, torch.bfloat16),
    # 384-row item boundaries: a 1-row last item, a full 256-row last item
    # (two query blocks per wave), whole 384-row items only
    (2, 385, 2, 128, torch.bfloat16),
    (2, 640, 1, 128, torch.bfloat16),
    (3, 768, 1, 128, torch.bfloat16),
]


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:4])) + str(s[4])[-4:])
def test_ragged_shapes_full_parity(shape, flags):
    n, L, H, D, dt = shape
    say("case ragged", shape, flags)
    q, k, v = synth.queue_inputs(n, L, H, D, seed=100 + L, device=DEV, dtype=dt, k_rho=0.9)
    cache = synth.build_cache(k, v)
    ref = oracle.queue_step(q, k, v, None)
    a = run_queue(q, k, v, None, flags=flags)
    b = run_queue(q, k, v, cache, flags=flags)
    assert_parity(to_f64(a), ref, f"ragged {shape}")
    assert torch.equal(a, b), "alias and cache modes differ"


def test_deterministic_and_order_independent_of_stream_state():
    q, k, v = synth.queue_inputs(4, 200, 3, 128, seed=7, device=DEV)
    a = run_queue(q, k, v)
    b = run_queue(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("flags", PERSISTENT)
def test_work_queue_slots_reused_across_many_calls(flags):
    """The 256-row main pass is persistent and takes its items from a work
    queue slot that a clearing kernel zeroes right before it; eager calls cycle
    through 64 slots.  150 back-to-back calls (every slot used twice or more),
    each into an output prefilled with a finite sentinel (NaN would be
    recomputed by the recheck pass), all give the first call's bits: no item is
    skipped or done twice after a slot is reused."""
    ctx = ca.create(0, flags)
    inputs = [synth.queue_inputs(4, 200, 3, 128, seed=s, device=DEV) for s in (21, 22)]
    refs = []
    for q, k, v in inputs:
        refs.append(ca.queue_step(q, k, v, None, ctx=ctx))
    torch.cuda.synchronize()
    outs = []
    for i in range(150):
        q, k, v = inputs[i % 2]
        o = torch.full_like(q, 2.0 ** 100)
        ca.queue_step(q, k, v, None, out=o, ctx=ctx)
        outs.append(o)
    torch.cuda.synchronize()
    say("calls", len(outs))
    for i, o in enumerate(outs):
        assert torch.equal(o, refs[i % 2]), f"call {i}"


@pytest.mark.parametrize("flags", PERSISTENT)
def test_work_queue_two_streams_interleaved(flags):
    """Calls of one context on two streams, launched alternately without
    synchronisation, use distinct queue slots and match the serial results."""
    ctx = ca.create(0, flags)
    a_in = synth.queue_inputs(8, 700, 5, 128, seed=31, device=DEV)
    b_in = synth.queue_inputs(3, 1000, 4, 64, seed=32, device=DEV)
    ref_a = ca.queue_step(*a_in, None, ctx=ctx)
    ref_b = ca.queue_step(*b_in, None, ctx=ctx)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for i in range(6):
        for st, inp in ((s1, a_in), (s2, b_in)):
            with torch.cuda.stream(st):
                o = torch.full_like(inp[0], 2.0 ** 100)
                ca.queue_step(*inp, None, out=o, ctx=ctx, stream=st)
            outs.append(o)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, ref_a if i % 2 == 0 else ref_b), f"launch {i}"


def unsplit_context(flags):
    ctx = ca.Context(0, flags)
    if ctx.call_block_rows(128, ca.BF16) == 384:
        ctx.set_tail_split(0)
    return ctx


@pytest.mark.parametrize("flags", PERSISTENT)
def test_work_queue_under_graph_replay(flags):
    """A queue step captured in a HIP graph and replayed several times, with
    eager calls of the same context and synchronisations between replays: the
    captured call has a work-queue slot of its own, cleared by a kernel node
    (no memset node) on every replay, so every replay gives the eager bits.
    Captured calls never cut items along the keys, so the context has the
    tail split off for the eager calls too."""
    ctx = unsplit_context(flags)
    q, k, v = synth.queue_inputs(4, 600, 3, 128, seed=41, device=DEV)
    ref = ca.queue_step(q, k, v, None, ctx=ctx)
    torch.cuda.synchronize()
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        ca.queue_step(q, k, v, None, out=out, ctx=ctx)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ca.queue_step(q, k, v, None, out=out, ctx=ctx)
    for rep in range(4):
        out.fill_(2.0 ** 100)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
        eager = ca.queue_step(q, k, v, None, ctx=ctx)
        torch.cuda.synchronize()
        assert torch.equal(eager, ref), f"eager call after replay {rep}"


@pytest.mark.parametrize("flags", PERSISTENT)
def test_two_graphs_on_two_streams_with_eager_calls(flags):
    """Two queue steps captured into two graphs, replayed at the same time on
    two streams while eager calls of the same context run on a third, for 70
    rounds (the eager calls wrap round all 64 eager slots): captured calls own
    their slots, so no two launches in flight share one, and every output
    equals its eager reference bit for bit (tail split off, as above)."""
    ctx = unsplit_context(flags)
    ins = [synth.queue_inputs(4, 600, 3, 128, seed=s, device=DEV) for s in (51, 52, 53)]
    refs = [ca.queue_step(*x, None, ctx=ctx) for x in ins]
    torch.cuda.synchronize()
    outs = [torch.empty_like(x[0]) for x in ins[:2]]
    graphs = []
    for i in range(2):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):  # warm-up on a side stream
            ca.queue_step(*ins[i], None, out=outs[i], ctx=ctx)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ca.queue_step(*ins[i], None, out=outs[i], ctx=ctx)
        graphs.append(g)
    s1, s2, s3 = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
    eager = torch.empty_like(ins[2][0])
    for rep in range(70):
        for o in outs + [eager]:
            o.fill_(2.0 ** 100)
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            graphs[0].replay()
        with torch.cuda.stream(s2):
            graphs[1].replay()
        with torch.cuda.stream(s3):
            ca.queue_step(*ins[2], None, out=eager, ctx=ctx, stream=s3)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], refs[0]), f"graph 0, round {rep}"
        assert torch.equal(outs[1], refs[1]), f"graph 1, round {rep}"
        assert torch.equal(eager, refs[2]), f"eager call, round {rep}"


def test_guard_bands_and_cache_slot0_never_read():
    n, L, H, D = 3, 150, 2, 128
    q, k, v = synth.queue_inputs(n, L, H, D, seed=8, device=DEV)
    pad = 4096  # elements of NaN before and after every tensor
    def padded(t):
        buf = torch.full((t.numel() + 2 * pad,), float("nan"), dtype=t.dtype, device=DEV)
        buf[pad:pad + t.numel()].copy_(t.reshape(-1))
        return buf, buf[pad:pad + t.numel()].view(t.shape)
    _, qp = padded(q)
    _, kp = padded(k)
    _, vp = padded(v)
    cache = synth.build_cache(k, v)  # slot 0 is NaN
    assert torch.isnan(cache[0]).all()
    _, cp = padded(cache)
    obuf, op = padded(torch.zeros_like(q))
    ca.queue_step(qp, kp, vp, cp, out=op)
    torch.cuda.synchronize()
    assert torch.isfinite(op).all()
    assert torch.isnan(obuf[:pad]).all() and torch.isnan(obuf[pad + q.numel():]).all(), \
        "writes outside out"
    ref = run_queue(q, k, v)
    assert torch.equal(op, ref)


@pytest.mark.parametrize("flags", FLAGS)
def test_range_fingerprint_bit_exact(flags):
    """Q = 0 makes every weight exactly 1, so O[c,r,h,d] = (number of tokens t
    in R_c with (t + 7h) mod D == d) / |R_c|, with t the token's global index.
    The kernel's fp32 sums of ones are exact, so the bf16 output must equal the
    rounded rational exactly: a key/value row shifted by one, a wrong chunk or
    head, or a dropped segment changes some entries."""
    n, L, H, D = 4, 300, 3, 128
    q = torch.zeros((n, L, H, D), dtype=torch.bfloat16, device=DEV)
    k = synth.normal((n, L, H, D), 9, 2, DEV)
    t = torch.arange(n * L, device=DEV).view(n, L, 1, 1)
    hh = torch.arange(H, device=DEV).view(1, 1, H, 1)
    d = torch.arange(D, device=DEV).view(1, 1, 1, D)
    v = (((t + 7 * hh) % D) == d).to(torch.bfloat16)
    cache = synth.build_cache(k, v)
    exp = np.zeros((n, L, H, D))
    for c in range(n):
        toks = np.arange(max(c - 1, 0) * L, (c + 1) * L)
        for h in range(H):
            counts = np.bincount((toks + 7 * h) % D, minlength=D)
            exp[c, :, h, :] = counts / len(toks)
    exp_bf16 = torch.from_numpy(exp).float().to(torch.bfloat16)
    for cc in (None, cache):
        out = run_queue(q, k, v, cc, flags=flags)
        assert torch.equal(out.cpu(), exp_bf16), "fingerprint mismatch"


@pytest.mark.parametrize("flags", FLAGS)
def test_constant_v_returned_exactly(flags):
    """Softmax weights sum to one, so a constant V row comes back.  Both
    kernels sum l from the same bf16-rounded P the P.V product uses, so l and
    the P.V sums differ only by fp32 summation order (relative 1e-7), far
    below half a bf16 step: the bf16 output equals V exactly."""
    n, L, H, D = 3, 257, 2, 128
    q, k, _ = synth.queue_inputs(n, L, H, D, seed=10, device=DEV)
    cvec = synth.normal((1, 1, H, D), 10, 9, DEV)
    v = cvec.expand(n, L, H, D).contiguous()
    out = run_queue(q, k, v, flags=flags)
    assert torch.equal(out, v)


def test_scale_zero_is_uniform_mean():
    n, L, H, D = 3, 100, 2, 64
    q, k, v = synth.queue_inputs(n, L, H, D, seed=11, device=DEV, dtype=torch.float32)
    out = run_queue(q, k, v, None, scale=0.0)
    ref = oracle.queue_step(q, k, v, None, scale=0.0)
    assert_parity(to_f64(out), ref, "scale 0")


def test_empty_inputs_are_noops():
    q = torch.empty((0, 16, 2, 128), dtype=torch.bfloat16, device=DEV)
    out = ca.queue_step(q, q, q)
    assert out.shape == q.shape
    q1 = torch.randn((2, 0, 2, 128), device=DEV).to(torch.bfloat16)
    assert ca.queue_step(q1, q1, q1).shape == q1.shape
    qf = torch.empty((0, 5, 2, 128), dtype=torch.bfloat16, device=DEV)
    kf = torch.randn((1, 7, 2, 128), device=DEV).to(torch.bfloat16)
    assert ca.full(qf, kf, kf).shape == qf.shape


def test_errors_are_raised_not_launched():
    q, k, v = synth.queue_inputs(2, 16, 2, 96, seed=1, device=DEV)
    with pytest.raises(ca.ChunkAttnError) as e:
        ca.queue_step(q, k, v)
    assert e.value.status == ca.EUNSUPPORTED
    q, k, v = synth.queue_inputs(2, 16, 2, 128, seed=1, device=DEV)
    with pytest.raises(ca.ChunkAttnError) as e:
        ca.queue_step(q, k, v, scale=-1.0)
    assert e.value.status == ca.EINVAL


@pytest.mark.parametrize("flags", FLAGS)
def test_device_plan_equals_host_plan(flags):
    ctx = ca.create(0, flags)
    say("xcd count", ctx.xcd_count, "block rows", ctx.block_rows)
    for (L, n, H) in [(128, 4, 2), (6240, 8, 40), (97, 5, 3), (14400, 16, 40)]:
        dev = ca.plan_device(L, n, H, ctx=ctx).cpu().numpy()
        host = ca.plan_debug(L, n, H, ctx.xcd_count, ctx.block_rows)
        np.testing.assert_array_equal(dev, host)


def test_block_sizes_agree():
    """The three launch configurations run different schedules (128-row items:
    the synchronous one, l summed on the vector ALU; 256-row items: the
    ping-pong one, no reference maximum and Q pre-scaled; 384-row items: the
    same on 16x16x32 MFMAs), so their sums round in a different order: they
    agree to a few bf16 rounding steps, well inside the parity bar each of them
    meets against the oracle."""
    q, k, v = synth.queue_inputs(5, 700, 3, 128, seed=14, device=DEV, k_rho=0.9)
    cache = synth.build_cache(k, v)
    a = run_queue(q, k, v, cache, flags=ca.FLAG_BLOCK128).float()
    b = run_queue(q, k, v, cache, flags=ca.FLAG_BLOCK256).float()
    c = run_queue(q, k, v, cache, flags=0).float()
    for what, x, y in (("128 vs 256", a, b), ("384 vs 256", c, b)):
        d = (x - y).abs()
        say("block", what, ": max", d.max().item(), "mean", d.mean().item())
        assert d.max().item() <= 4e-3 and d.mean().item() <= 2e-4


# -------------------------------------------------------------------- full attention

@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("B,lq,lkv,H,D,shared", [(1, 300, 300, 2, 128, False),
                                                 (3, 200, 77, 2, 128, True),
                                                 (2, 129, 1, 1, 64, False),
                                                 (4, 64, 512, 3, 128, True)])
def test_full_small_parity(B, lq, lkv, H, D, shared, flags):
    say("case full", B, lq, lkv, H, D, shared, flags)
    q = synth.normal((B, lq, H, D), 12, 1, DEV)
    kb = 1 if shared else B
    k = synth.normal((kb, lkv, H, D), 12, 2, DEV)
    v = synth.normal((kb, lkv, H, D), 12, 3, DEV)
    out = ca.full(q, k, v, ctx=ca.create(0, flags))
    torch.cuda.synchronize()
    ref = oracle.full(q, k, v)
    assert_parity(to_f64(out), ref, "full small")


def test_single_chunk_queue_equals_full_bitwise():
    q, k, v = synth.queue_inputs(1, 333, 2, 128, seed=13, device=DEV)
    a = run_queue(q, k, v)
    b = ca.full(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# -------------------------------------------------------------------- full-size workloads

def sample_rows(n, L, H, rng, per=24):
    bm = ca.block_rows()
    chunks = sorted(c for c in {0, 1, n - 1, int(rng.integers(0, n))} if c < n)
    heads = sorted({0, H - 1, int(rng.integers(0, H))})
    fixed = {0, 1, bm - 1, bm, L - 1, L - 2, (L // bm) * bm, max(L - bm, 0)}
    rows = []
    for c in chunks:
        for h in heads:
            rs = set(r for r in fixed if 0 <= r < L)
            rs |= set(rng.integers(0, L, per).tolist())
            rows += [(c, h, r) for r in sorted(rs)]
    return np.array(rows, np.int64)


def queue_rows_oracle(q, k, v, cache, rows, scale):
    """Oracle rows of the full problem, computed on the sub-problem [c-1, c]."""
    out = np.empty((len(rows), q.shape[-1]))
    for c in np.unique(rows[:, 0]):
        lo = max(int(c) - 1, 0)
        sub = lambda t: t[lo:c + 1].cpu()
        sel = rows[:, 0] == c
        r = rows[sel].copy()
        r[:, 0] -= lo
        out[sel] = oracle.queue_rows(sub(q), sub(k), sub(v),
                                     None if cache is None else sub(cache), r, scale)
    return out


def gather_rows(out, rows):
    idx = torch.from_numpy(rows).to(out.device)
    return to_f64(out[idx[:, 0], idx[:, 2], idx[:, 1]])


def check_any_size_properties(out, v):
    """Outputs are convex combinations of V rows: finite and within V's range.
    Outputs are prefilled with UNWRITTEN, so this also shows that every
    element was written."""
    assert torch.isfinite(out).all()
    vmax = v.float().abs().amax().item()
    assert out.float().abs().amax().item() <= vmax * (1 + 2 ** -7)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["wan1.3b", "wan14b", "720p16"])
def test_queue_workload_sampled_parity(name):
    w = configs.WORKLOADS[name]
    say("case workload", name, w)
    q, k, v = synth.queue_inputs(w.n, w.L, w.H, w.D, w.seed, device=DEV, k_rho=w.k_rho,
                                 v_rho=w.v_rho)
    cache = synth.build_cache(k, v)
    torch.cuda.synchronize()
    out = run_queue(q, k, v, cache, w.scale)
    check_any_size_properties(out, v)
    rng = np.random.default_rng(w.seed)
    rows = sample_rows(w.n, w.L, w.H, rng)
    ref = queue_rows_oracle(q, k, v, cache, rows, w.scale)
    s = assert_parity(gather_rows(out, rows), ref, name)
    say(name, "sampled rows", len(rows), s)
    # the in-place predecessor form gives the same bits
    out2 = run_queue(q, k, v, None, w.scale)
    assert torch.equal(out, out2)
    del out2, cache
    if w.n_text:
        qx = synth.cross_queries(w.n, w.L, w.H, w.D, w.seed, DEV)
        kt, vt = synth.text_inputs(w.n_text, w.H, w.D, w.seed, DEV)
        ox = torch.full_like(qx, UNWRITTEN)
        ca.full(qx, kt, vt, out=ox, scale=w.scale)
        torch.cuda.synchronize()
        check_any_size_properties(ox, vt)
        xrows = sample_rows(w.n, w.L, w.H, rng, per=8)
        refx = oracle.full_rows(qx[np.unique(xrows[:, 0])].cpu(), kt.cpu(), vt.cpu(),
                                _remap_batches(xrows), w.scale)
        sx = assert_parity(gather_rows(ox, xrows), refx, name + " cross")
        say(name, "cross sampled rows", len(xrows), sx)


def _remap_batches(rows):
    uniq = np.unique(rows[:, 0])
    r = rows.copy()
    r[:, 0] = np.searchsorted(uniq, rows[:, 0])
    return r


@pytest.mark.slow
def test_full_sequence_workload_sampled_parity():
    w = configs.WORKLOADS["full32k"]
    say("case workload", w.name, w)
    q = synth.normal((1, w.L, w.H, w.D), w.seed, synth.Q_ID, DEV)
    k = synth.normal((1, w.lkv, w.H, w.D), w.seed, synth.K_ID, DEV)
    v = synth.normal((1, w.lkv, w.H, w.D), w.seed, synth.V_ID, DEV)
    out = torch.full_like(q, UNWRITTEN)
    ca.full(q, k, v, out=out, scale=w.scale)
    torch.cuda.synchronize()
    check_any_size_properties(out, v)
    rows = sample_rows(1, w.L, w.H, np.random.default_rng(3), per=40)
    ref = oracle.full_rows(q.cpu(), k.cpu(), v.cpu(), rows, w.scale)
    s = assert_parity(gather_rows(out, rows), ref, "full32k")
    say("full32k sampled rows", len(rows), s)


@pytest.mark.parametrize("flags", FLAGS)
def test_score_overflow_falls_back_exactly(flags):
    """Scores that rise far above a row's first tile (2^300 in the exponent)
    overflow a fixed-maximum softmax; the kernel must still return the exact
    softmax (here all weight on the high-scoring keys), via its running-max
    fallback.  Chunk 1's own rows carry the high keys, chunk 0's do not."""
    n, L, H, D = 2, 200, 2, 128
    q = torch.full((n, L, H, D), 20.0, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((n, L, H, D), dtype=torch.bfloat16, device=DEV)
    k[1, 150:] = 1.0            # logical rows 350.. of chunk 1: score 20*128/sqrt(128) = 226
    v = synth.normal((n, L, H, D), 15, 3, DEV)
    cache = synth.build_cache(k, v)
    out = run_queue(q, k, v, cache, flags=flags)
    ref = oracle.queue_step(q, k, v, cache)
    assert_parity(to_f64(out), ref, "overflow fallback")
    # chunk 1 averages V over its 50 high-scoring own rows
    exp1 = v[1, 150:].float().mean(0)
    torch.testing.assert_close(out[1].float(), exp1.expand(L, H, D), atol=1e-2, rtol=0)


@pytest.mark.parametrize("flags", FLAGS)
def test_score_underflow_falls_back_exactly(flags):
    """Every score of a row far below zero (-226 / ln 2 in the exponent) sends
    the sum of weights out of fp32's range at the low end for a softmax
    without a maximum (the 256-row kernel marks l < 2^-64); the result must
    still be the exact softmax.  Chunk 1's last 50 own keys score 1/128 of
    the others' magnitude less negative, so they take almost all the weight;
    chunk 0's keys all score the same, so it returns the mean of its V."""
    n, L, H, D = 2, 200, 2, 128
    q = torch.full((n, L, H, D), -20.0, dtype=torch.bfloat16, device=DEV)
    k = torch.ones((n, L, H, D), dtype=torch.bfloat16, device=DEV)
    k[1, 150:] = 0.5            # score -113 instead of -226 for these keys
    v = synth.normal((n, L, H, D), 16, 3, DEV)
    cache = synth.build_cache(k, v)
    out = run_queue(q, k, v, cache, flags=flags)
    ref = oracle.queue_step(q, k, v, cache)
    assert_parity(to_f64(out), ref, "underflow fallback")
    exp0 = v[0].float().mean(0)
    torch.testing.assert_close(out[0].float(), exp0.expand(L, H, D), atol=1e-2, rtol=0)
    exp1 = v[1, 150:].float().mean(0)
    torch.testing.assert_close(out[1].float(), exp1.expand(L, H, D), atol=1e-2, rtol=0)
