"""Key-axis split of the last work items (384-row items, one block each).

A launch with few items per CU ends when its last items do, so those items
may be cut into parts along their key tiles: the last items with a
predecessor segment in a queue step (the short items of the first chunk stay
whole), the last items of the launch when none has one.  The softmax carries
no maximum,
so the parts' unnormalised outputs and row sums add: O = sum_p O_p / sum_p l_p
(the same numerators, summed in another fp32 order).  Each part stores its
partial in a workspace; the part that finishes last adds all of them in part
order and writes the block.  Checked on every element against the fp64 oracle
and against the unsplit launch (DualParal write-up, section 三: each chunk
over the cached K/V of its predecessor and its own), for 2, 3 and 4 parts,
partly split launches, ragged blocks, one-tile parts, overflowing blocks
(the finishing part marks them for the recheck), and run-to-run
determinism.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from chunked_spatio_temporal_amd import chunkattn as ca
from chunked_spatio_temporal_amd import synth
from parity_util import assert_parity, error_stats, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SENTINEL = 2.0 ** 100


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ca.load_library()
    yield


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ctx_split(items, parts=0):
    c = ca.Context(0, 0)
    c.set_tail_split(items, parts)
    return c


def run(ctx, q, k, v, cache):
    out = torch.full_like(q, SENTINEL)
    ca.queue_step(q, k, v, cache, out=out, ctx=ctx)
    torch.cuda.synchronize()
    return out


def test_tail_split_setting_is_validated():
    c = ca.Context(0, 0)
    for items, parts in ((-2, 0), (5, 1), (5, 9)):
        with pytest.raises(ca.ChunkAttnError):
            c.set_tail_split(items, parts)
    c.set_tail_split(-1)
    c.set_tail_split(0)
    c.set_tail_split(7, 3)


# 3 chunks of 1000 rows: blocks of 384, 384 and 232 rows (a ragged block runs
# with two query blocks per wave); keys 1000 (chunk 0) or 1000 cached + 1000 own
N, L, H, D = 3, 1000, 2, 128
N_ITEMS = N * H * 3


@pytest.mark.parametrize("items,parts", [(N_ITEMS, 2), (N_ITEMS, 3), (N_ITEMS, 4), (5, 2)],
                         ids=["all-x2", "all-x3", "all-x4", "last5-x2"])
def test_split_queue_step_parity(items, parts):
    say("case split", items, parts)
    q, k, v = synth.queue_inputs(N, L, H, D, seed=601, device=DEV, k_rho=0.9)
    cache = synth.build_cache(k, v)
    ref = oracle.queue_step(q, k, v, cache)
    split = run(ctx_split(items, parts), q, k, v, cache)
    whole = run(ctx_split(0), q, k, v, cache)
    s = assert_parity(to_f64(split), ref, f"split {items}x{parts}")
    assert_parity(to_f64(whole), ref, "unsplit")
    # the same numerators in another summation order: at most a few bf16 steps apart
    d = error_stats(to_f64(split), to_f64(whole))
    assert d["max_abs"] <= 2e-3 and d["mean_abs"] <= 2e-5, d
    # alias mode (predecessor read in place) gives the same bits
    assert torch.equal(split, run(ctx_split(items, parts), q, k, v, None))
    say("stats", s, d)


def test_split_is_deterministic():
    q, k, v = synth.queue_inputs(N, L, H, D, seed=602, device=DEV)
    c = ctx_split(N_ITEMS, 3)
    a = run(c, q, k, v, None)
    for _ in range(5):
        assert torch.equal(run(c, q, k, v, None), a)


def test_split_one_tile_parts():
    """Chunks of 100 rows: 2 or 4 key tiles per item, cut into 4 parts (parts
    of one tile, and the single ragged tile of chunk 0's items)."""
    q, k, v = synth.queue_inputs(3, 100, 2, 128, seed=603, device=DEV)
    cache = synth.build_cache(k, v)
    out = run(ctx_split(6, 4), q, k, v, cache)
    assert_parity(to_f64(out), oracle.queue_step(q, k, v, cache), "one-tile parts")


def test_split_overflowing_blocks_are_rechecked():
    """Rows 400-700 of every chunk at scores far past fp32's range: the parts'
    sums overflow, the finishing part marks the block and the recheck
    recomputes it; every element matches the oracle."""
    q, k, v = synth.queue_inputs(N, L, H, D, seed=604, device=DEV)
    q = q.float()
    q[:, 400:700] = 20.0
    q = q.to(torch.bfloat16)
    k = k.float()
    k[:, 900:] = 1.0
    k = k.to(torch.bfloat16)
    cache = synth.build_cache(k, v)
    out = run(ctx_split(N_ITEMS, 2), q, k, v, cache)
    assert torch.isfinite(out).all()
    assert_parity(to_f64(out), oracle.queue_step(q, k, v, cache), "split overflow")


def test_short_launch_default_splits_match_oracle():
    """The default context cuts the last items of a launch with few items per
    CU: a 5-head queue shard of 8 chunks x 1000 rows (120 items), every element
    against the oracle."""
    q, k, v = synth.queue_inputs(8, 1000, 5, 128, seed=605, device=DEV, k_rho=0.9)
    cache = synth.build_cache(k, v)
    out = run(ca.create(0), q, k, v, cache)
    assert_parity(to_f64(out), oracle.queue_step(q, k, v, cache), "default split")


def test_split_without_predecessor_group():
    """Full attention (no item has a predecessor segment): the split takes the
    last items of the launch.  2 x 1000 query rows over 1000 keys, one block per
    item, the last 4 items in 3 parts: every element against the oracle and
    within 2e-3 of the unsplit launch."""
    B, lq, lkv, H, D = 2, 1000, 1000, 2, 128
    q = synth.normal((B, lq, H, D), 606, synth.Q_ID, DEV)
    k = synth.normal((B, lkv, H, D), 606, synth.K_ID, DEV)
    v = synth.normal((B, lkv, H, D), 606, synth.V_ID, DEV)
    outs = []
    for items, parts in ((4, 3), (0, 0)):
        c = ca.Context(0, 0)
        c.set_item_blocks(1)
        c.set_tail_split(items, parts)
        out = torch.full_like(q, SENTINEL)
        ca.full(q, k, v, out=out, ctx=c)
        torch.cuda.synchronize()
        outs.append(out)
    ref = oracle.full(q, k, v)
    assert_parity(to_f64(outs[0]), ref, "full split")
    d = error_stats(to_f64(outs[0]), to_f64(outs[1]))
    assert d["max_abs"] <= 2e-3 and d["mean_abs"] <= 2e-5, d
