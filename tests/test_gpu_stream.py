"""GPU parity of the streaming queue (DualParal write-up, section 二): the
ring-buffer queue step and the FIFO driver, against the fp64 oracle's ring step
and the plain queue simulation.

Chunk c of the queue (processing order, tail first) lives in ring slot
(tail - c) mod S and reads its predecessor in place from the slot of chunk c-1.
Calls go through the C-ABI library's Python binding.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import fifo as fifo_sim
from chunked_spatio_temporal_amd import chunkattn as ca
from chunked_spatio_temporal_amd import configs, synth
from parity_util import assert_parity, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = -777.0


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


def ring_inputs(S, L, H, D, seed, dt=torch.bfloat16):
    q = synth.normal((S, L, H, D), seed, 1, DEV, dt)
    k = synth.normal((S, L, H, D), seed, 2, DEV, dt)
    v = synth.normal((S, L, H, D), seed, 3, DEV, dt)
    return q, k, v


def all_rows(n, L, H):
    return np.array([(c, h, r) for c in range(n) for h in range(H) for r in range(L)], np.int64)


def gather(out_ring, tail, n, rows):
    S = out_ring.shape[0]
    idx = torch.from_numpy(rows).to(out_ring.device)
    slots = (tail - idx[:, 0]) % S
    return to_f64(out_ring[slots, idx[:, 2], idx[:, 1]])


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("S,tail,n,L,H,D,dt", [
    (5, 1, 4, 97, 2, 128, torch.bfloat16),   # wraps around slot 0
    (5, 4, 5, 64, 1, 64, torch.bfloat16),    # every slot live
    (3, 0, 2, 130, 2, 128, torch.float32),
    (4, 2, 1, 33, 3, 128, torch.bfloat16),   # one live chunk
], ids=["wrap", "full", "f32", "single"])
def test_ring_step_parity(S, tail, n, L, H, D, dt, flags):
    say("case ring", S, tail, n, L, H, D, dt, flags)
    q, k, v = ring_inputs(S, L, H, D, 300 + L, dt)
    out = torch.full_like(q, SENTINEL)
    ca.ring_step(q, k, v, out, tail, n, ctx=ca.create(0, flags))
    torch.cuda.synchronize()
    rows = all_rows(n, L, H)
    ref = oracle.ring_rows(q, k, v, tail, n, rows)
    assert_parity(gather(out, tail, n, rows), ref, "ring")
    live = {(tail - c) % S for c in range(n)}
    for s in range(S):
        if s not in live:
            assert (out[s] == SENTINEL).all(), f"slot {s} is not live but was written"


def test_ring_equals_queue_on_gathered_chunks_bitwise():
    S, tail, n, L, H, D = 6, 2, 5, 150, 2, 128
    q, k, v = ring_inputs(S, L, H, D, 31)
    out = torch.empty_like(q)
    ca.ring_step(q, k, v, out, tail, n)
    order = [(tail - c) % S for c in range(n)]
    lin = ca.queue_step(q[order].contiguous(), k[order].contiguous(), v[order].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(out[order], lin)


def test_fifo_streaming_run():
    """A whole video of 7 chunks through a queue of depth 4 in 5 slots: before
    every step the live chunks get fresh Q/K/V (the latents change each step),
    the step's outputs of every live chunk match the oracle, the queue's
    bookkeeping matches the plain simulation, and a chunk's output stays in its
    slot until the slot is reused."""
    total, S, depth, L, H, D = 7, 5, 4, 64, 2, 64
    f = ca.Fifo(S, depth)
    q = torch.zeros((S, L, H, D), dtype=torch.bfloat16, device=DEV)
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    out = torch.full_like(q, SENTINEL)
    left = total
    for step, (pushed, live, popped) in enumerate(fifo_sim.run(total, S, depth)):
        if left > 0:
            assert f.push() == pushed
            left -= 1
        assert f.live() == live
        for _, slot, _ in live:
            seed = 1000 * step + slot
            q[slot] = synth.normal((L, H, D), seed, 1, DEV)
            k[slot] = synth.normal((L, H, D), seed, 2, DEV)
            v[slot] = synth.normal((L, H, D), seed, 3, DEV)
        f.step(q, k, v, out)
        torch.cuda.synchronize()
        tail, n = live[0][1], len(live)
        rows = all_rows(n, L, H)
        assert_parity(gather(out, tail, n, rows), oracle.ring_rows(q, k, v, tail, n, rows),
                      f"stream step {step}")
        if popped >= 0:
            final = out[popped].clone()
            assert f.pop() == popped
            assert torch.equal(out[popped], final)
    assert f.live() == []


def test_fifo_step_on_empty_queue_is_rejected():
    f = ca.Fifo(3, 2)
    z = torch.zeros((3, 8, 1, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ca.ChunkAttnError):
        f.step(z, z.clone(), z.clone(), z.clone())
    assert f.live() == []


@pytest.mark.slow
def test_stream_workload_sampled_parity():
    """Steady state of the 40-head queue as a stream: 9 slots, depth 8, tail in
    slot 4 (the live chunks wrap around slot 0); sampled rows vs the oracle."""
    w = configs.WORKLOADS["wan14b"]
    S, depth, tail = 9, 8, 4
    say("case stream workload", S, depth, w)
    q, k, v = synth.queue_inputs(S, w.L, w.H, w.D, 7, device=DEV, k_rho=0.9)
    out = torch.full_like(q, SENTINEL)
    ca.ring_step(q, k, v, out, tail, depth, scale=w.scale)
    torch.cuda.synchronize()
    live = [(tail - c) % S for c in range(depth)]
    vmax = v.float().abs().amax().item()
    for s_ in range(S):
        if s_ in live:
            assert torch.isfinite(out[s_]).all()
            assert out[s_].float().abs().amax().item() <= vmax * (1 + 2 ** -7)
        else:
            assert (out[s_] == SENTINEL).all()
    rng = np.random.default_rng(7)
    rows = []
    for c in (0, 1, 4, 5, depth - 1):
        for h in (0, w.H - 1, int(rng.integers(0, w.H))):
            rs = {0, 255, 256, w.L - 1} | set(rng.integers(0, w.L, 12).tolist())
            rows += [(c, h, r) for r in sorted(rs)]
    rows = np.array(rows, np.int64)
    ref = oracle.ring_rows(q, k, v, tail, depth, rows, scale=w.scale)
    s = assert_parity(gather(out, tail, depth, rows), ref, "stream")
    say("stream sampled rows", len(rows), s)
