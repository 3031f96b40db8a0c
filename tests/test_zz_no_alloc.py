"""The allocation-free queue step (chunkattn_queue_step_noalloc) against the
ordinary entry point: two calls in a row through the C ABI, the second with a
smaller input, each compared bit for bit with chunkattn_queue_step on the same
inputs (both run the same kernels; only the work queue's memory differs: the
library's static device scratch instead of the context's buffer).  Outputs are
prefilled with a finite sentinel, so an item the persistent pass skipped would
show (a NaN prefill would be recomputed by the recheck pass)."""
import sys

import pytest
import torch

from chunked_spatio_temporal_amd import chunkattn as ca
from chunked_spatio_temporal_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
UNWRITTEN = 2.0 ** 100


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ca.load_library()
    yield


@pytest.mark.parametrize("flags", [pytest.param(0, id="default"),
                                   pytest.param(ca.FLAG_BLOCK256, id="bm256"),
                                   pytest.param(ca.FLAG_BLOCK128, id="bm128")])
def test_noalloc_matches_queue_step_two_calls(flags):
    # the no-allocation entry point never cuts items along the keys; the
    # reference call uses a context with the tail split off
    ctx = ca.Context(0, flags)
    if ctx.call_block_rows(128, ca.BF16) == 384:
        ctx.set_tail_split(0)
    # the first call is larger than the second: the second must not see
    # anything the first left in the scratch
    for (n, L, H, D, seed, cached) in [(6, 900, 40, 128, 61, True), (3, 257, 5, 128, 62, False)]:
        print("case noalloc", (n, L, H, D), "cache" if cached else "alias", flags, flush=True)
        q, k, v = synth.queue_inputs(n, L, H, D, seed=seed, device=DEV, k_rho=0.9)
        cache = synth.build_cache(k, v) if cached else None
        ref = torch.full_like(q, UNWRITTEN)
        ca.queue_step(q, k, v, cache, out=ref, ctx=ctx)
        got = torch.full_like(q, UNWRITTEN)
        ca.queue_step_noalloc(q, k, v, cache, got, ctx=ctx)
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all() and (ref.float().abs() < 2.0 ** 99).all()
        assert torch.equal(got, ref), f"noalloc differs from queue_step at {(n, L, H, D)}"


def test_noalloc_validates_like_queue_step():
    q, k, v = synth.queue_inputs(2, 16, 2, 96, seed=1, device=DEV)
    with pytest.raises(ca.ChunkAttnError) as e:
        ca.queue_step_noalloc(q, k, v, None, torch.empty_like(q))
    assert e.value.status == ca.EUNSUPPORTED


def test_noalloc_fp32_matches_queue_step():
    """fp32 calls run the fp32 kernel, one workgroup per item and no work
    queue: the allocation-free entry point gives the same bits."""
    ctx = ca.Context(0, 0)
    for (n, L, H, D, seed) in [(4, 300, 3, 64, 63), (2, 129, 2, 128, 64)]:
        print("case noalloc fp32", (n, L, H, D), flush=True)
        q, k, v = synth.queue_inputs(n, L, H, D, seed=seed, device=DEV, dtype=torch.float32)
        cache = synth.build_cache(k, v)
        ref = torch.full_like(q, UNWRITTEN)
        ca.queue_step(q, k, v, cache, out=ref, ctx=ctx)
        got = torch.full_like(q, UNWRITTEN)
        ca.queue_step_noalloc(q, k, v, cache, got, ctx=ctx)
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all() and (ref.abs() < 2.0 ** 99).all()
        assert torch.equal(got, ref), f"noalloc differs from queue_step at {(n, L, H, D)}"
