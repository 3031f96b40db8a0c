"""Device-free tests of the C-ABI library: symbols, validation, launch plan.

No compute call is made here (there may be no GPU); the plan and the argument
checks have device-free entry points.  The plan is compared bit for bit with
the oracle's integer index map of each chunk's key/value set.
"""
import ctypes
import os

import numpy as np
import pytest

import oracle
from chunked_spatio_temporal_amd import chunkattn as ca

lib = ca.load_library()


def test_every_declared_symbol_is_exported():
    names = ca.declared_symbols()
    assert "chunkattn_queue_step" in names and "chunkattn_full" in names
    assert "chunkattn_create" in names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in include/chunkattn.h but not exported"


def test_library_has_no_oracle_dependency():
    # the product library must not link or embed the oracle
    blob = open(ca.LIB_PATH, "rb").read()
    assert b"oracle_" not in blob
    assert b"liboracle" not in blob


def test_status_strings():
    for code in range(6):
        assert lib.chunkattn_status_string(code)
    assert lib.chunkattn_status_string(99) == b"unknown status"


# ---------------------------------------------------------------- validation

P = 1 << 20  # a fake 16-byte-aligned device address (never dereferenced)


def vq(**kw):
    a = dict(q=P, k=2 * P, v=3 * P, cache=None, out=4 * P, L=16, n=2, H=2, D=128,
             scale=0.1, dtype=ca.BF16)
    a.update(kw)
    return ca.validate_queue_step(a["q"], a["k"], a["v"], a["cache"], a["out"], a["L"], a["n"],
                                  a["H"], a["D"], a["scale"], a["dtype"])


def test_validate_queue_ok_and_empty():
    assert vq()[0] == ca.OK
    assert vq(cache=8 * P)[0] == ca.OK
    assert vq(D=64, dtype=ca.F32)[0] == ca.OK
    # empty problems are no-ops, pointers unused
    assert vq(n=0, q=None, k=None, v=None, out=None)[0] == ca.OK
    assert vq(L=0, q=None, k=None, v=None, out=None)[0] == ca.OK


@pytest.mark.parametrize("kw,code", [
    (dict(L=-1), ca.EINVAL),
    (dict(n=-3), ca.EINVAL),
    (dict(H=0), ca.EINVAL),
    (dict(D=96), ca.EUNSUPPORTED),
    (dict(D=256), ca.EUNSUPPORTED),
    (dict(dtype=7), ca.EUNSUPPORTED),
    (dict(scale=-0.5), ca.EINVAL),
    (dict(scale=float("nan")), ca.EINVAL),
    (dict(scale=float("inf")), ca.EINVAL),
    (dict(q=None), ca.EINVAL),
    (dict(out=None), ca.EINVAL),
    (dict(k=P + 2), ca.EINVAL),               # misaligned
    (dict(cache=8 * P + 8), ca.EINVAL),       # misaligned cache
    (dict(out=P), ca.EINVAL),                 # out aliases q
    (dict(out=2 * P + 64), ca.EINVAL),        # out overlaps k
    (dict(L=1 << 30, n=1 << 20, H=64), ca.EINVAL),  # 2^63 elements: offset overflow
])
def test_validate_queue_rejects(kw, code):
    rc, msg = vq(**kw)
    assert rc == code, msg
    assert msg


G = 1 << 34  # fake addresses far enough apart for rows of a quarter million heads


@pytest.mark.parametrize("H,D,dtype,code", [
    (262143, 128, ca.BF16, ca.OK),            # 64 rows span 2^32 - 16 KiB
    (262144, 128, ca.BF16, ca.EUNSUPPORTED),  # 64 rows span 2^32 bytes
    (131071, 128, ca.F32, ca.OK),
    (131072, 128, ca.F32, ca.EUNSUPPORTED),
    (524288, 64, ca.BF16, ca.EUNSUPPORTED),
])
def test_validate_rejects_rows_beyond_32bit_tile_offsets(H, D, dtype, code):
    """The kernels address a 64-row key/value tile by 32-bit byte offsets from
    its first row, so 64 rows of heads * head_dim elements must span under
    2^32 bytes; every entry point that launches the attention kernels checks it."""
    rc, msg = vq(q=G, k=2 * G, v=3 * G, out=4 * G, L=1, n=1, H=H, D=D, dtype=dtype)
    assert rc == code, msg
    rc, msg = vf(q=G, k=2 * G, v=3 * G, out=4 * G, B=1, lq=1, lkv=1, H=H, D=D, dtype=dtype)
    assert rc == code, msg
    rc, msg = vw(q=G, k=2 * G, v=3 * G, out=5 * G, L=1, n=1, H=H, D=D, dtype=dtype)
    assert rc == code, msg
    rc, msg = vr(q=G, k=2 * G, v=3 * G, out=4 * G, S=1, tail=0, n=1, L=1, H=H, D=D,
                 dtype=dtype)
    assert rc == code, msg


def vf(**kw):
    a = dict(q=P, k=2 * P, v=3 * P, out=4 * P, B=2, lq=16, lkv=8, stride=0, H=2, D=128,
             scale=0.1, dtype=ca.BF16)
    a.update(kw)
    return ca.validate_full(a["q"], a["k"], a["v"], a["out"], a["B"], a["lq"], a["lkv"],
                            a["stride"], a["H"], a["D"], a["scale"], a["dtype"])


def test_validate_full():
    assert vf()[0] == ca.OK
    assert vf(stride=8 * 2 * 128)[0] == ca.OK
    assert vf(B=0, q=None, k=None, v=None, out=None)[0] == ca.OK
    assert vf(lkv=0)[0] == ca.EINVAL           # attention over no keys
    assert vf(stride=-1)[0] == ca.EINVAL
    assert vf(stride=3)[0] == ca.EINVAL        # 6-byte stride breaks alignment
    assert vf(D=32)[0] == ca.EUNSUPPORTED
    assert vf(out=3 * P)[0] == ca.EINVAL


def vw(**kw):
    a = dict(q=P, k=2 * P, v=3 * P, cache=None, out=4 * P, L=16, n=2, H=2, D=128,
             scale=0.1, dtype=ca.BF16)
    a.update(kw)
    return ca.validate_window_step(a["q"], a["k"], a["v"], a["cache"], a["out"], a["L"],
                                   a["n"], a["H"], a["D"], a["scale"], a["dtype"])


def test_validate_window_step():
    assert vw()[0] == ca.OK
    assert vw(cache=8 * P)[0] == ca.OK
    assert vw(n=0, q=None, k=None, v=None, out=None)[0] == ca.OK
    # out holds two chunks' rows per window: [P - 16 KiB, P + 16 KiB) overlaps q,
    # while the queue step's out of half that size ends where q starts
    below_q = P - 16 * 2 * 128 * 2 * 2
    assert vq(out=below_q)[0] == ca.OK
    assert vw(out=below_q)[0] == ca.EINVAL
    # a window walks up to 3 * chunk_len key rows: chunk_len is capped at 2^29
    far = dict(q=1 << 40, k=2 << 40, v=3 << 40, out=4 << 40, n=1, H=1, D=64)
    assert vq(L=(1 << 29) + 1, **far)[0] == ca.OK
    assert vw(L=(1 << 29) + 1, **far)[0] == ca.EUNSUPPORTED
    assert vw(L=1 << 29, **far)[0] == ca.OK
    for kw, code in [(dict(D=96), ca.EUNSUPPORTED), (dict(scale=-1.0), ca.EINVAL),
                     (dict(k=P + 2), ca.EINVAL), (dict(out=P), ca.EINVAL)]:
        assert vw(**kw)[0] == code


def test_window_step_without_context_is_rejected():
    assert lib.chunkattn_window_step(None, P, 2 * P, 3 * P, None, 4 * P, 16, 2, 2, 128,
                                     ctypes.c_float(0.1), 0, None) == ca.EINVAL


def test_queue_step_without_context_is_rejected():
    assert lib.chunkattn_queue_step(None, P, 2 * P, 3 * P, None, 4 * P, 16, 2, 2, 128,
                                    ctypes.c_float(0.1), 0, None) == ca.EINVAL


# ---------------------------------------------------------------------- plan

def _slot_to_work_reference(n, n_xcd, n_first=0):
    """Die x runs slots x, x + n_xcd, ... in order.  It takes an even share of
    the long work items [0, n_first) (one contiguous piece), then as many short
    items [n_first, n) as it has slots left, again one contiguous piece."""
    order = np.empty(n, np.int64)
    long_pieces = np.array_split(np.arange(n_first), n_xcd)
    next_short = n_first
    for x in range(n_xcd):
        slots = np.arange(x, n, n_xcd)
        longs = long_pieces[x]
        assert len(longs) <= len(slots)
        shorts = np.arange(next_short, next_short + len(slots) - len(longs))
        next_short += len(shorts)
        order[slots] = np.r_[longs, shorts]
    assert next_short == n
    return order


@pytest.mark.parametrize("bm", [128, 256, 384])
@pytest.mark.parametrize("L,n,H,xcd", [(128, 4, 2, 8), (6240, 8, 12, 8), (97, 5, 3, 8),
                                       (1, 1, 1, 8), (300, 3, 7, 1), (6240, 8, 40, 8),
                                       (14400, 16, 40, 8), (200, 2, 3, 3)])
def test_plan_matches_oracle_index_map(L, n, H, xcd, bm):
    items = ca.plan_debug(L, n, H, xcd, bm)
    nq = -(-L // bm)
    assert items.shape == (n * H * nq, 7)
    # every (chunk, head, query row) exactly once
    c, h, q0, qr, pc, pr, orows = items.T.astype(np.int64)
    assert ((qr > 0) & (qr <= bm) & (q0 % bm == 0)).all()
    key = (c * H + h) * nq + q0 // bm
    assert sorted(key.tolist()) == list(range(n * H * nq))
    np.testing.assert_array_equal(qr, np.minimum(bm, L - q0))
    # each item's key/value set is the oracle's index map of its chunk, bit for bit
    for cc in range(n):
        sel = c == cc
        kv = np.unique(items[sel][:, 4:7], axis=0)
        assert kv.shape == (1, 3), "items of one chunk disagree on their key/value set"
        pcc, prr, oww = kv[0]
        src, ch, row = oracle.index_map(L, n, cc)
        plan_src = np.r_[np.full(prr, oracle.SRC_PRED), np.full(oww, oracle.SRC_OWN)]
        plan_ch = np.r_[np.full(prr, pcc), np.full(oww, cc)]
        plan_row = np.r_[np.arange(prr), np.arange(oww)]
        np.testing.assert_array_equal(plan_src, src)
        np.testing.assert_array_equal(plan_ch, ch)
        np.testing.assert_array_equal(plan_row, row)


@pytest.mark.parametrize("bm", [128, 256])
@pytest.mark.parametrize("L,n,H,xcd", [(128, 4, 2, 8), (97, 5, 3, 8), (1, 1, 1, 8),
                                       (300, 3, 7, 1), (6240, 8, 40, 8), (200, 2, 3, 3),
                                       (64, 1, 2, 8)])
def test_window_plan_matches_oracle_window_map(L, n, H, xcd, bm):
    items = ca.window_plan_debug(L, n, H, xcd, bm)
    c, h, q0, qr, pc, pr, orows = items.T.astype(np.int64)
    # every (window, head, query row) exactly once: 2L rows per window, L for the last
    expect = sum(H * -(-oracle.window_q_rows(L, n, cc) // bm) for cc in range(n))
    assert items.shape == (expect, 7)
    covered = set()
    for it in items:
        for r in range(it[2], it[2] + it[3]):
            covered.add((int(it[0]), int(it[1]), r))
    assert len(covered) == sum(it[3] for it in items)
    assert covered == {(cc, hh, r) for cc in range(n) for hh in range(H)
                       for r in range(oracle.window_q_rows(L, n, cc))}
    assert ((qr > 0) & (qr <= bm) & (q0 % bm == 0)).all()
    # each item's key/value set is the oracle's window map, bit for bit: the own
    # segment is read contiguously from chunk c (chunk c, then chunk c+1)
    for cc in range(n):
        kv = np.unique(items[c == cc][:, 4:7], axis=0)
        assert kv.shape == (1, 3), "items of one window disagree on their key/value set"
        pcc, prr, oww = kv[0]
        src, ch, row = oracle.window_index_map(L, n, cc)
        own = np.arange(oww)
        np.testing.assert_array_equal(
            np.r_[np.full(prr, oracle.SRC_PRED), np.full(oww, oracle.SRC_OWN)], src)
        np.testing.assert_array_equal(np.r_[np.full(prr, pcc), cc + own // L], ch)
        np.testing.assert_array_equal(np.r_[np.arange(prr), own % L], row)


def test_window_plan_order_longest_first():
    L, n, H, xcd = 6240, 8, 40, 8
    items = ca.window_plan_debug(L, n, H, xcd)
    bm = ca.block_rows()
    nq, nq_last = -(-2 * L // bm), -(-L // bm)
    n_first = int((items[:, 5] > 0).sum())
    by_work = items[np.argsort(_slot_to_work_reference(len(items), xcd, n_first))]
    # windows 1..n-2 (three segments), the last window, then window 0
    expect_c = np.r_[np.repeat(np.arange(1, n - 1), H * nq), np.full(H * nq_last, n - 1),
                     np.zeros(H * nq, int)]
    np.testing.assert_array_equal(by_work[:, 0], expect_c)


def test_default_block_rows():
    assert ca.block_rows() == 384  # bf16, head_dim 128 calls of a default context
    np.testing.assert_array_equal(ca.plan_debug(300, 3, 2, 8),
                                  ca.plan_debug(300, 3, 2, 8, ca.block_rows()))
    assert ca.plan_debug(300, 3, 2, 8, 128).shape[0] == 3 * 2 * 3
    assert ca.plan_debug(300, 3, 2, 8, 256).shape[0] == 3 * 2 * 2
    assert ca.plan_debug(800, 3, 2, 8, 384).shape[0] == 3 * 2 * 3
    with pytest.raises(ca.ChunkAttnError):
        ca.plan_debug(300, 3, 2, 8, 96)


def test_plan_order_longest_first_and_die_ranges():
    L, n, H, xcd = 6240, 8, 12, 8
    items = ca.plan_debug(L, n, H, xcd)
    nq = -(-L // ca.block_rows())
    # reconstruct the work index of every slot and check it is the reference bijection
    order = _slot_to_work_reference(len(items), xcd, int((items[:, 5] > 0).sum()))
    by_work = items[np.argsort(order)]
    # work order: chunks 1..n-1 (two segments) first, chunk 0 last; t fastest
    expect_c = np.r_[np.repeat(np.arange(1, n), H * nq), np.zeros(H * nq, int)]
    np.testing.assert_array_equal(by_work[:, 0], expect_c)
    np.testing.assert_array_equal(by_work[:, 1], np.tile(np.repeat(np.arange(H), nq), n))
    np.testing.assert_array_equal(by_work[:, 2], np.tile(np.arange(nq) * ca.block_rows(), n * H))


@pytest.mark.parametrize("n_items,xcd", [(1, 8), (7, 8), (8, 8), (9, 8), (4704, 8),
                                         (15680, 8), (1000, 3), (5, 1)])
def test_slot_to_work_is_a_bijection(n_items, xcd):
    # use a plan with one chunk, one head so n_items == number of query tiles
    bm = ca.block_rows()
    items = ca.plan_debug(bm * n_items, 1, 1, xcd)
    assert len(items) == n_items
    got = items[:, 2] // bm                      # tile index == work index here
    np.testing.assert_array_equal(got, _slot_to_work_reference(n_items, xcd))
    assert sorted(got.tolist()) == list(range(n_items))


@pytest.mark.parametrize("bm", [128, 256, 384])
@pytest.mark.parametrize("L,n,H,xcd", [(97, 5, 3, 8), (128, 4, 2, 8), (300, 3, 7, 8),
                                       (6240, 8, 40, 8), (6240, 8, 12, 8), (1000, 9, 5, 8),
                                       (200, 2, 3, 3), (64, 7, 1, 8), (1, 2, 1, 8)])
def test_die_order_is_the_two_class_split(L, n, H, xcd, bm):
    """Queue plans with long (predecessor) and short items: the slot -> work map
    is the reference two-class split, and every die walks about the same number
    of key rows (within one long item of the others)."""
    items = ca.plan_debug(L, n, H, xcd, bm)
    n_first = int((items[:, 5] > 0).sum())
    order = _slot_to_work_reference(len(items), xcd, n_first)
    by_work = items[np.argsort(order)]
    # work order: long items first
    assert (by_work[:n_first, 5] > 0).all() and (by_work[n_first:, 5] == 0).all()
    # the library's slots agree with the reference map item for item
    c, h, q0 = by_work[:, 0], by_work[:, 1], by_work[:, 2]
    nq = -(-L // bm)
    work_key = (c * H + h) * nq + q0 // bm
    pred_first = np.r_[np.arange(1, n), [0]] if n > 1 else np.array([0])
    expect_key = np.concatenate([(cc * H + np.repeat(np.arange(H), nq)) * nq + np.tile(np.arange(nq), H)
                                 for cc in pred_first])
    np.testing.assert_array_equal(work_key, expect_key)
    # balance: the dies' key-row totals differ by at most one long plus one short item
    rows = (items[:, 5] + items[:, 6]).astype(np.int64)
    per_die = np.array([rows[x::xcd].sum() for x in range(xcd)])
    assert per_die.max() - per_die.min() <= 2 * L + L


# ------------------------------------------------------- streaming queue (host)

from oracle import fifo as fifo_sim  # noqa: E402


@pytest.mark.parametrize("total,slots,depth", [(1, 1, 1), (5, 3, 3), (11, 5, 4), (20, 8, 8),
                                               (9, 12, 4), (3, 6, 4)])
def test_fifo_bookkeeping_matches_the_queue_simulation(total, slots, depth):
    """The C++ queue and the plain simulation of the page's FIFO agree on every
    step: which slot a new chunk gets, the live chunks in processing order with
    their slots and steps done, and which slot a clean chunk frees."""
    f = ca.Fifo(slots, depth)
    pushed_left = total
    for pushed, live, popped in fifo_sim.run(total, slots, depth):
        got_push = f.push() if pushed_left > 0 else -1
        pushed_left -= got_push >= 0
        assert got_push == pushed
        assert f.live() == live
        f.advance()
        head = f.live()[-1]
        got_pop = f.pop() if head[2] == depth else -1
        assert got_pop == popped
    assert f.live() == []


def test_fifo_rejects_misuse():
    with pytest.raises(ca.ChunkAttnError):
        ca.Fifo(3, 4)                  # fewer slots than depth
    with pytest.raises(ca.ChunkAttnError):
        ca.Fifo(3, 0)
    f = ca.Fifo(4, 2)
    with pytest.raises(ca.ChunkAttnError):
        f.advance()                    # empty
    with pytest.raises(ca.ChunkAttnError):
        f.pop()                        # empty
    f.push()
    f.push()
    with pytest.raises(ca.ChunkAttnError):
        f.push()                       # full
    f.advance()
    with pytest.raises(ca.ChunkAttnError):
        f.pop()                        # head has done 1 of 2 steps
    f.advance()
    assert f.pop() == 0 and f.push() == 2


def vr(**kw):
    a = dict(q=P, k=2 * P, v=3 * P, out=4 * P, S=5, tail=3, n=4, L=16, H=2, D=128, scale=0.1,
             dtype=ca.BF16)
    a.update(kw)
    return ca.validate_ring_step(a["q"], a["k"], a["v"], a["out"], a["S"], a["tail"], a["n"],
                                 a["L"], a["H"], a["D"], a["scale"], a["dtype"])


def test_validate_ring_step():
    assert vr()[0] == ca.OK
    assert vr(n=5)[0] == ca.OK
    assert vr(n=0, q=None, k=None, v=None, out=None)[0] == ca.OK
    for kw, code in [(dict(n=6), ca.EINVAL), (dict(tail=5), ca.EINVAL), (dict(tail=-1), ca.EINVAL),
                     (dict(S=0), ca.EINVAL), (dict(D=80), ca.EUNSUPPORTED),
                     (dict(out=P + 16), ca.EINVAL), (dict(q=None), ca.EINVAL)]:
        rc, msg = vr(**kw)
        assert rc == code, (kw, msg)


def test_ring_step_without_context_is_rejected():
    assert lib.chunkattn_ring_step(None, P, 2 * P, 3 * P, 4 * P, 5, 0, 2, 16, 2, 128,
                                   ctypes.c_float(0.1), 0, None) == ca.EINVAL


# ------------------------------------------------------ noise initialization

def vn(**kw):
    a = dict(pool=P, PF=12, fb=4096, keys=2 * P, prev=3 * P, n_prev=8, n_excl=4, F=8,
             out=4 * P, idx=5 * P)
    a.update(kw)
    return ca.validate_noise_init(a["pool"], a["PF"], a["fb"], a["keys"], a["prev"], a["n_prev"],
                                  a["n_excl"], a["F"], a["out"], a["idx"])


def test_validate_noise_init():
    assert vn()[0] == ca.OK
    assert vn(prev=None, n_prev=0, n_excl=0)[0] == ca.OK          # first chunk
    for kw in [dict(PF=0), dict(PF=4097), dict(F=0), dict(n_excl=9), dict(n_excl=-1),
               dict(prev=None), dict(F=9),                        # 12 - 4 < 9
               dict(fb=24), dict(fb=0), dict(pool=P + 8), dict(keys=2 * P + 2),
               dict(out=P + 4096), dict(idx=4 * P + 16)]:
        rc, msg = vn(**kw)
        assert rc == ca.EINVAL, (kw, msg)
