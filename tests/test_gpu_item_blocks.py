"""Work items of several 384-row query blocks (bf16, head_dim 128).

A context may give each work item G consecutive 384-row query blocks of one
(chunk, head); the blocks then walk the same key/value tiles one after the
other as one stream, with the next block's Q loaded and the previous block
stored while the tiles keep flowing.  Each block's arithmetic is that of a
one-block item (the same tiles in the same order, the same accumulation
order), so the outputs must equal the one-block context's bit for bit, and
match the fp64 oracle over every element.

Cases: the queue step (predecessor segment straddling a tile, ragged last key
tile, ragged last query block inside a multi-block item), cross-attention of
per-chunk queries over 512 shared text rows (DualParal write-up, section 三:
cross-attention per chunk, without the cache), a single key tile per block,
and blocks that leave fp32's range at several positions of an item (the
recheck pass must find every marked block).  A shared K/V runs its items
head-major; that order must give the same bits as the same K/V copied per
batch item, in every kernel.
"""
import sys

import pytest
import torch

import oracle
from chunked_spatio_temporal_amd import chunkattn as ca
from chunked_spatio_temporal_amd import synth
from parity_util import assert_parity, to_f64

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


_CTX = {}


def ctx_blocks(g):
    """A context of the default (384-row) item size with g blocks per item and
    no key-axis split (items of several blocks are never split, so the
    one-block reference must not be either for the bitwise comparisons)."""
    if g not in _CTX:
        c = ca.Context(0, 0)
        c.set_item_blocks(g)
        c.set_tail_split(0)
        _CTX[g] = c
    return _CTX[g]


def test_item_blocks_setting_is_validated():
    c = ca.Context(0, 0)
    for bad in (-1, 9):
        with pytest.raises(ca.ChunkAttnError):
            c.set_item_blocks(bad)
    c.set_item_blocks(0)
    c.set_item_blocks(8)


@pytest.mark.parametrize("G", [2, 3, 8])
def test_queue_step_item_blocks(G):
    """3 chunks of 1000 rows (blocks of 384, 384, 232 rows): G = 2 gives items
    of two blocks and of the ragged one alone; G >= 3 one item per (chunk,
    head) whose last block is ragged.  Keys: 1000 cached + 1000 own rows, a
    tile straddling the two segments and a ragged last tile."""
    n, L, H, D = 3, 1000, 3, 128
    say("case queue item blocks", G, (n, L, H, D))
    q, k, v = synth.queue_inputs(n, L, H, D, seed=510, device=DEV, k_rho=0.9)
    cache = synth.build_cache(k, v)
    ref_out = torch.full_like(q, SENTINEL)
    ca.queue_step(q, k, v, cache, out=ref_out, ctx=ctx_blocks(1))
    out = torch.full_like(q, SENTINEL)
    ca.queue_step(q, k, v, cache, out=out, ctx=ctx_blocks(G))
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "multi-block items differ from one-block items"
    s = assert_parity(to_f64(out), oracle.queue_step(q, k, v, cache), f"queue G={G}")
    say("stats", s)


@pytest.mark.parametrize("G", [2, 5, 8])
def test_cross_attention_item_blocks(G):
    """Per-chunk queries (4 x 2000 rows: 6 blocks, the last of 80 rows) over
    one shared set of 512 text rows (8 key tiles per block)."""
    B, lq, T, H, D = 4, 2000, 512, 2, 128
    say("case cross item blocks", G, (B, lq, T, H, D))
    q = synth.cross_queries(B, lq, H, D, 511, DEV, torch.bfloat16)
    kt, vt = synth.text_inputs(T, H, D, 511, DEV, torch.bfloat16)
    ref_out = torch.full_like(q, SENTINEL)
    ca.full(q, kt, vt, out=ref_out, ctx=ctx_blocks(1))
    out = torch.full_like(q, SENTINEL)
    ca.full(q, kt, vt, out=out, ctx=ctx_blocks(G))
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "multi-block items differ from one-block items"
    s = assert_parity(to_f64(out), oracle.full(q, kt, vt), f"cross G={G}")
    say("stats", s)


@pytest.mark.parametrize("lkv", [40, 64, 100])
def test_short_key_walks_item_blocks(lkv):
    """One or two key tiles per block (40 and 64 rows: one tile, the first
    ragged; 100: two), 1500 query rows (4 blocks) in one item."""
    B, lq, H, D = 2, 1500, 2, 128
    say("case short key walk", lkv)
    q = synth.normal((B, lq, H, D), 512, synth.Q_ID, DEV)
    k = synth.normal((B, lkv, H, D), 512, synth.K_ID, DEV)
    v = synth.normal((B, lkv, H, D), 512, synth.V_ID, DEV)
    ref_out = torch.full_like(q, SENTINEL)
    ca.full(q, k, v, out=ref_out, ctx=ctx_blocks(1))
    out = torch.full_like(q, SENTINEL)
    ca.full(q, k, v, out=out, ctx=ctx_blocks(4))
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out), "multi-block items differ from one-block items"
    assert_parity(to_f64(out), oracle.full(q, k, v), f"short walk lkv={lkv}")


@pytest.mark.parametrize("hot", [(0, 2, 3), (1,), (4,), (0, 1, 2, 3, 4)],
                         ids=["b023", "b1", "b4", "all"])
def test_overflowing_blocks_inside_items(hot):
    """Blocks whose scores leave fp32's range without a maximum (Q = 20 on
    every dim against keys near 1: scores near 226 in natural units) at
    several positions of a 5-block item: the item marks blocks 0..2 itself,
    two blocks after each, and the last two at its end; the recheck pass must
    recompute exactly the marked ones.  Other blocks keep ordinary scores."""
    B, lq, lkv, H, D = 1, 5 * 384, 256, 2, 128
    say("case overflow blocks", hot)
    q = 0.5 * synth.normal((B, lq, H, D), 513, synth.Q_ID, DEV).float()
    for b in hot:
        q[:, b * 384:(b + 1) * 384] = 20.0
    q = q.to(torch.bfloat16)
    k = (1.0 + 0.1 * synth.normal((B, lkv, H, D), 513, synth.K_ID, DEV).float()).to(
        torch.bfloat16)
    v = synth.normal((B, lkv, H, D), 513, synth.V_ID, DEV)
    ref_out = torch.full_like(q, SENTINEL)
    ca.full(q, k, v, out=ref_out, ctx=ctx_blocks(1))
    out = torch.full_like(q, SENTINEL)
    ca.full(q, k, v, out=out, ctx=ctx_blocks(5))
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, ref_out), "multi-block items differ from one-block items"
    assert_parity(to_f64(out), oracle.full(q, k, v), f"overflow blocks {hot}")


def _shared_vs_replicated(q, kt, vt, ctx, what):
    """full() over one shared K/V (kv stride 0: items run head-major) against
    the same K/V copied per batch item (items in (chunk, head, tile) order):
    every output row is computed by one item with the same arithmetic, so the
    two must agree bit for bit, and every element must be written."""
    B = q.shape[0]
    kr = kt.expand(B, -1, -1, -1).contiguous()
    vr = vt.expand(B, -1, -1, -1).contiguous()
    sent = SENTINEL if q.dtype == torch.bfloat16 else 2.0 ** 120
    out_s = torch.full_like(q, sent)
    out_r = torch.full_like(q, sent)
    ca.full(q, kt, vt, out=out_s, ctx=ctx)
    ca.full(q, kr, vr, out=out_r, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.isfinite(out_s).all() and (out_s.float().abs() < sent / 2).all(), \
        f"{what}: output not fully written"
    assert torch.equal(out_s, out_r), f"{what}: shared K/V differs from replicated K/V"
    return out_s


@pytest.mark.parametrize("G", [1, 4])
def test_shared_kv_head_major_equals_replicated(G):
    """16 chunks x 2000 queries, 8 heads, over 512 shared text rows: 768
    one-block items (several per workgroup, claims across dies) or 256 items of
    up to 4 blocks; two chunks also against the fp64 oracle."""
    B, lq, T, H, D = 16, 2000, 512, 8, 128
    say("case shared kv head-major", G, (B, lq, T, H, D))
    q = synth.cross_queries(B, lq, H, D, 514, DEV, torch.bfloat16)
    kt, vt = synth.text_inputs(T, H, D, 514, DEV, torch.bfloat16)
    out = _shared_vs_replicated(q, kt, vt, ctx_blocks(G), f"G={G}")
    sel = [0, B - 1]
    assert_parity(to_f64(out[sel]), oracle.full(q[sel], kt, vt), f"shared kv G={G}")


@pytest.mark.parametrize("flags,dtype", [(ca.FLAG_BLOCK256, torch.bfloat16),
                                         (ca.FLAG_BLOCK128, torch.bfloat16),
                                         (0, torch.float32)],
                         ids=["bm256", "bm128", "fp32"])
def test_shared_kv_head_major_other_kernels(flags, dtype):
    """The 256- and 128-row kernels and the fp32 kernel take the same
    head-major order for a shared K/V: 6 items x 1000 queries, 5 heads, 300
    text rows (ragged last key tile)."""
    B, lq, T, H, D = 6, 1000, 300, 5, 128
    say("case shared kv head-major", flags, dtype, (B, lq, T, H, D))
    q = synth.normal((B, lq, H, D), 515, synth.Q_ID, DEV, dtype)
    kt = synth.normal((1, T, H, D), 515, synth.K_ID, DEV, dtype)
    vt = synth.normal((1, T, H, D), 515, synth.V_ID, DEV, dtype)
    ctx = ca.Context(0, flags)
    ctx.set_tail_split(0)
    _shared_vs_replicated(q, kt, vt, ctx, f"flags {flags} {dtype}")
