"""Pins for the fp64 CPU oracle, against things other than itself.

Each test checks the oracle against what the pages and the mathematics fix:
hand-derived closed forms (tests/golden), invariants of softmax attention, a
brute-force re-formulation (attention over the explicitly concatenated
sequence with a block-band mask, which is what the page's K/V cache replaces,
DualParal write-up section 三), torch's own scaled-dot-product attention, and
special cases that reduce to textbook attention.  The pins are chosen so that
plausible slips in the oracle (dropped cache rows, a wrong predecessor index,
a missing scale, V read from K, heads mixed) each fail at least one of them;
tests/test_oracle_mutations.py plants such slips and checks exactly that.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def band_masked_attention(q, k, v, scale):
    """Attention over the concatenated sequence of all chunks, with the block
    band mask: a query in chunk c sees keys of chunks c-1 and c only.

    This is the explicit-concatenation form that the page's cache avoids; it is
    written independently of the oracle (one dense score matrix per head).
    """
    n, L, H, D = q.shape
    S = n * L
    qs = q.reshape(S, H, D)
    ks = k.reshape(S, H, D)
    vs = v.reshape(S, H, D)
    chunk_of = np.arange(S) // L
    allowed = (chunk_of[None, :] == chunk_of[:, None]) | (chunk_of[None, :] == chunk_of[:, None] - 1)
    out = np.empty((S, H, D))
    for h in range(H):
        s = scale * qs[:, h, :] @ ks[:, h, :].T
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w /= w.sum(axis=1, keepdims=True)
        out[:, h, :] = w @ vs[:, h, :]
    return out.reshape(n, L, H, D)


def make_cache(k, v):
    n = k.shape[0]
    cache = np.full((n, 2) + k.shape[1:], np.nan)
    cache[1:, 0] = k[:-1]
    cache[1:, 1] = v[:-1]
    return cache


# --------------------------------------------------------------------------
# golden closed forms


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_golden_closed_forms(case):
    q = np.array(case["q"], np.float64)
    k = np.array(case["k"], np.float64)
    v = np.array(case["v"], np.float64)
    cache = None if case["cache"] is None else np.array(case["cache"], np.float64)
    exp = np.array(case["expected"], np.float64)
    got = oracle.queue_step(q, k, v, cache, scale=case["scale"])
    assert got.shape == exp.shape
    np.testing.assert_allclose(got, exp, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# (a) softmax weights of every row sum to one, and are the closed form


@pytest.mark.parametrize("c", [0, 1, 3])
def test_probs_sum_to_one(c):
    n, L, H, D = 4, 9, 2, 8
    q, k, v = rand((n, L, H, D), 1), rand((n, L, H, D), 2), rand((n, L, H, D), 3)
    for h in range(H):
        for r in (0, 4, L - 1):
            p, _ = oracle.queue_probs(q, k, v, None, c, h, r)
            assert p.shape == (L if c == 0 else 2 * L,)
            assert np.all(p > 0)
            assert abs(p.sum() - 1.0) <= 1e-12


def test_probs_match_closed_form_weights():
    # two keys with score gap ln 3 -> weights exactly (1/4, 3/4)
    q = np.zeros((2, 1, 1, 1))
    k = np.zeros((2, 1, 1, 1))
    v = np.zeros((2, 1, 1, 1))
    q[1, 0, 0, 0] = 1.0
    k[1, 0, 0, 0] = math.log(3.0)
    p, _ = oracle.queue_probs(q, k, v, None, 1, 0, 0, scale=1.0)
    np.testing.assert_allclose(p, [0.25, 0.75], rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# (b) constant V is returned exactly


@pytest.mark.parametrize("with_cache", [False, True])
def test_constant_v_returned(with_cache):
    n, L, H, D = 3, 7, 2, 5
    q, k = rand((n, L, H, D), 4), rand((n, L, H, D), 5)
    cvec = rand((1, 1, H, D), 6)
    v = np.broadcast_to(cvec, (n, L, H, D)).copy()
    cache = make_cache(k, v) if with_cache else None
    got = oracle.queue_step(q, k, v, cache)
    np.testing.assert_allclose(got, np.broadcast_to(cvec, got.shape), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# (c) cache form == explicit concatenation with a block-band mask


@pytest.mark.parametrize("shape", [(4, 16, 2, 8), (3, 5, 3, 4), (1, 6, 1, 3), (5, 1, 2, 2)])
@pytest.mark.parametrize("with_cache", [False, True])
def test_chunked_equals_band_masked_concatenation(shape, with_cache):
    n, L, H, D = shape
    q, k, v = rand(shape, 7), rand(shape, 8), rand(shape, 9)
    scale = 0.37
    cache = make_cache(k, v) if with_cache else None
    got = oracle.queue_step(q, k, v, cache, scale=scale)
    ref = band_masked_attention(q, k, v, scale)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_chunked_equals_torch_sdpa_with_band_mask():
    n, L, H, D = 4, 12, 3, 16
    q, k, v = rand((n, L, H, D), 10), rand((n, L, H, D), 11), rand((n, L, H, D), 12)
    got = oracle.queue_step(q, k, v, None)
    S = n * L
    tq = torch.from_numpy(q.reshape(S, H, D)).permute(1, 0, 2).unsqueeze(0)
    tk = torch.from_numpy(k.reshape(S, H, D)).permute(1, 0, 2).unsqueeze(0)
    tv = torch.from_numpy(v.reshape(S, H, D)).permute(1, 0, 2).unsqueeze(0)
    ch = torch.arange(S) // L
    mask = (ch[None, :] == ch[:, None]) | (ch[None, :] == ch[:, None] - 1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask,
                                                           scale=D ** -0.5)
    ref = ref.squeeze(0).permute(1, 0, 2).reshape(n, L, H, D).numpy()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_cache_mode_equals_alias_mode():
    shape = (5, 11, 2, 8)
    q, k, v = rand(shape, 13), rand(shape, 14), rand(shape, 15)
    a = oracle.queue_step(q, k, v, None)
    b = oracle.queue_step(q, k, v, make_cache(k, v))
    np.testing.assert_array_equal(a, b)


# --------------------------------------------------------------------------
# (d) joint permutation of key/value rows (across the cache/own boundary)


def test_joint_kv_permutation_invariance():
    n, L, H, D = 3, 10, 2, 6
    q, k, v = rand((n, L, H, D), 16), rand((n, L, H, D), 17), rand((n, L, H, D), 18)
    cache = make_cache(k, v)
    base = oracle.queue_step(q, k, v, cache)
    c = 1
    # R_c as one 2L-row array, permuted jointly for K and V, then split back
    kc = np.concatenate([cache[c, 0], k[c]], axis=0)
    vc = np.concatenate([cache[c, 1], v[c]], axis=0)
    perm = np.random.default_rng(19).permutation(2 * L)
    assert np.any(perm[:L] >= L)  # the permutation crosses the cache/own boundary
    k2, v2, cache2 = k.copy(), v.copy(), cache.copy()
    cache2[c, 0], k2[c] = kc[perm][:L], kc[perm][L:]
    cache2[c, 1], v2[c] = vc[perm][:L], vc[perm][L:]
    # chunk c+1 reads its predecessor from cache slot c+1, which is unchanged
    got = oracle.queue_step(q, k2, v2, cache2)
    np.testing.assert_allclose(got[c], base[c], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(got[c + 1], base[c + 1])


def test_query_permutation_permutes_output():
    n, L, H, D = 2, 9, 2, 4
    q, k, v = rand((n, L, H, D), 20), rand((n, L, H, D), 21), rand((n, L, H, D), 22)
    base = oracle.queue_step(q, k, v, None)
    perm = np.random.default_rng(23).permutation(L)
    q2 = q.copy()
    q2[1] = q[1][perm]
    got = oracle.queue_step(q2, k, v, None)
    np.testing.assert_allclose(got[1], base[1][perm], rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# reductions to textbook attention and closed forms


def _sdpa(q, k, v, scale):
    """torch fp64 attention for [B][L][H][D] arrays."""
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


def test_chunk0_is_plain_attention_on_itself():
    shape = (3, 14, 2, 8)
    q, k, v = rand(shape, 24), rand(shape, 25), rand(shape, 26)
    got = oracle.queue_step(q, k, v, None)
    ref = _sdpa(q[:1], k[:1], v[:1], 8 ** -0.5)
    np.testing.assert_allclose(got[:1], ref, rtol=0, atol=1e-12)


def test_single_chunk_equals_full():
    shape = (1, 17, 3, 8)
    q, k, v = rand(shape, 27), rand(shape, 28), rand(shape, 29)
    a = oracle.queue_step(q, k, v, None)
    b = oracle.full(q, k, v)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_full_matches_torch_sdpa_and_shared_kv():
    q = rand((3, 10, 2, 8), 30)
    kt, vt = rand((1, 7, 2, 8), 31), rand((1, 7, 2, 8), 32)
    got = oracle.full(q, kt, vt, scale=0.3)
    ref = _sdpa(q, np.broadcast_to(kt, (3, 7, 2, 8)).copy(),
                np.broadcast_to(vt, (3, 7, 2, 8)).copy(), 0.3)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    # per-batch K/V
    kb, vb = rand((3, 7, 2, 8), 33), rand((3, 7, 2, 8), 34)
    np.testing.assert_allclose(oracle.full(q, kb, vb), _sdpa(q, kb, vb, 8 ** -0.5),
                               rtol=0, atol=1e-12)


def test_full_rows_match_full():
    q, k, v = rand((2, 9, 2, 4), 35), rand((2, 5, 2, 4), 36), rand((2, 5, 2, 4), 37)
    allr = oracle.full(q, k, v)
    rows = np.array([[0, 0, 0], [1, 1, 8], [1, 0, 3]])
    got = oracle.full_rows(q, k, v, rows)
    for i, (b, h, r) in enumerate(rows):
        np.testing.assert_array_equal(got[i], allr[b, r, h])


@pytest.mark.parametrize("mode", ["zero_q", "zero_scale"])
def test_uniform_mean_when_scores_vanish(mode):
    n, L, H, D = 3, 4, 2, 3
    q, k = rand((n, L, H, D), 38), rand((n, L, H, D), 39)
    v = np.random.default_rng(40).integers(-8, 9, (n, L, H, D)).astype(np.float64)
    scale = 0.5
    if mode == "zero_q":
        q[:] = 0.0
    else:
        scale = 0.0
    got = oracle.queue_step(q, k, v, None, scale=scale)
    for c in range(n):
        lo = max(c - 1, 0)
        mean = v[lo:c + 1].reshape(-1, H, D).mean(axis=0)
        np.testing.assert_allclose(got[c], np.broadcast_to(mean, (L, H, D)), rtol=0, atol=1e-13)


def test_single_key_returns_its_value():
    q, k, v = rand((1, 1, 2, 4), 41), rand((1, 1, 2, 4), 42), rand((1, 1, 2, 4), 43)
    np.testing.assert_allclose(oracle.queue_step(q, k, v, None), v, rtol=0, atol=1e-15)


@pytest.mark.parametrize("j", [0, 5, 8, 13])
def test_dominant_key_selects_its_value(j):
    n, L, H, D = 2, 8, 1, 4
    q, k, v = rand((n, L, H, D), 44), 0.01 * rand((n, L, H, D), 45), rand((n, L, H, D), 46)
    qh = q[1, 3, 0] / np.linalg.norm(q[1, 3, 0])
    # key j of R_1: j < L is the predecessor's (chunk 0) row j, else own row j-L
    src_c, src_r = (0, j) if j < L else (1, j - L)
    k[src_c, src_r, 0] = 200.0 * qh
    got = oracle.queue_step(q, k, v, None, scale=1.0)
    np.testing.assert_allclose(got[1, 3, 0], v[src_c, src_r, 0], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# storage types: bf16 and fp32 inputs are widened exactly


def test_bf16_and_f32_inputs_widen_exactly():
    shape = (3, 6, 2, 8)
    tq = torch.from_numpy(rand(shape, 47)).to(torch.bfloat16)
    tk = torch.from_numpy(rand(shape, 48)).to(torch.bfloat16)
    tv = torch.from_numpy(rand(shape, 49)).to(torch.bfloat16)
    via_bf16 = oracle.queue_step(tq, tk, tv, None)
    via_f64 = oracle.queue_step(tq.double().numpy(), tk.double().numpy(), tv.double().numpy(),
                                None)
    np.testing.assert_array_equal(via_bf16, via_f64)
    via_f32 = oracle.queue_step(tq.float(), tk.float(), tv.float(), None)
    np.testing.assert_array_equal(via_f32, via_f64)


# --------------------------------------------------------------------------
# integer index map == brute-force enumeration of the band mask


@pytest.mark.parametrize("L,n", [(1, 1), (3, 4), (7, 2), (128, 4)])
def test_index_map_matches_band_enumeration(L, n):
    for c in range(n):
        src, ch, row = oracle.index_map(L, n, c)
        expect = []
        for cc in range(n):          # every key token of the concatenated sequence
            for r in range(L):
                if cc == c - 1:
                    expect.append((oracle.SRC_PRED, cc, r))
                elif cc == c:
                    expect.append((oracle.SRC_OWN, cc, r))
        got = list(zip(src.tolist(), ch.tolist(), row.tolist()))
        assert got == expect


def test_queue_rows_match_queue_step():
    shape = (4, 13, 3, 8)
    q, k, v = rand(shape, 50), rand(shape, 51), rand(shape, 52)
    cache = make_cache(k, v)
    allr = oracle.queue_step(q, k, v, cache)
    rows = np.array([[0, 0, 0], [3, 2, 12], [1, 1, 6], [2, 0, 0]])
    got = oracle.queue_rows(q, k, v, cache, rows)
    for i, (c, h, r) in enumerate(rows):
        np.testing.assert_array_equal(got[i], allr[c, r, h])


def test_cache_slot0_is_never_read():
    shape = (3, 5, 2, 4)
    q, k, v = rand(shape, 53), rand(shape, 54), rand(shape, 55)
    cache = make_cache(k, v)          # slot 0 is NaN
    assert np.isnan(cache[0]).all()
    got = oracle.queue_step(q, k, v, cache)
    assert np.isfinite(got).all()


# --------------------------------------------------------------------------
# window step (DualParal write-up, section 三: the window [B_{i-1}, B_i] with
# the cached K/V of B_{i+1}; chunk c+1 plays B_{i-1}, chunk c-1 B_{i+1})

WGOLDEN = os.path.join(os.path.dirname(__file__), "golden", "window_closed_forms.json")


def _window_golden_cases():
    with open(WGOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _window_golden_cases(), ids=lambda c: c["name"])
def test_window_golden_closed_forms(case):
    q = np.array(case["q"], np.float64)
    k = np.array(case["k"], np.float64)
    v = np.array(case["v"], np.float64)
    cache = None if case["cache"] is None else np.array(case["cache"], np.float64)
    got = oracle.window_step(q, k, v, cache, scale=case["scale"])
    flat = [np.nan if x is None else x for x in np.array(case["expected"], dtype=object).ravel()]
    exp = np.array(flat, np.float64).reshape(got.shape)
    np.testing.assert_allclose(got, exp, rtol=0, atol=1e-12)


def window_masked_attention(q, k, v, scale):
    """Brute force over the concatenated sequence: window c's queries are the
    tokens of chunks c and c+1, and each sees every key of chunks c-1, c, c+1
    that exists.  Written independently of the oracle (dense scores per head).
    Returns [n][2][L][H][D] with NaN for the absent half of the last window."""
    n, L, H, D = q.shape
    S = n * L
    qs, ks, vs = q.reshape(S, H, D), k.reshape(S, H, D), v.reshape(S, H, D)
    chunk_of = np.arange(S) // L
    out = np.full((n, 2, L, H, D), np.nan)
    for c in range(n):
        qtok = np.flatnonzero((chunk_of == c) | (chunk_of == c + 1))
        keys = np.flatnonzero((chunk_of >= c - 1) & (chunk_of <= c + 1))
        for h in range(H):
            s = scale * qs[qtok, h, :] @ ks[keys, h, :].T
            s -= s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w /= w.sum(axis=1, keepdims=True)
            o = w @ vs[keys, h, :]
            out[c].reshape(2 * L, H, D)[: len(qtok), h, :] = o
    return out


@pytest.mark.parametrize("shape", [(4, 6, 2, 8), (3, 5, 3, 4), (1, 7, 2, 3), (2, 1, 1, 2),
                                   (5, 3, 2, 5)])
@pytest.mark.parametrize("with_cache", [False, True])
def test_window_equals_masked_concatenation(shape, with_cache):
    q, k, v = rand(shape, 31), rand(shape, 32), rand(shape, 33)
    cache = make_cache(k, v) if with_cache else None
    got = oracle.window_step(q, k, v, cache, scale=0.7)
    exp = window_masked_attention(q, k, v, 0.7)
    np.testing.assert_allclose(got, exp, rtol=0, atol=1e-12)


def test_window_equals_torch_sdpa_with_window_mask():
    n, L, H, D = 4, 5, 2, 6
    q, k, v = rand((n, L, H, D), 41), rand((n, L, H, D), 42), rand((n, L, H, D), 43)
    got = oracle.window_step(q, k, v, None, scale=0.3)
    S = n * L
    chunk_of = torch.arange(S) // L
    qt = torch.tensor(q.reshape(S, H, D)).permute(1, 0, 2)
    kt = torch.tensor(k.reshape(S, H, D)).permute(1, 0, 2)
    vt = torch.tensor(v.reshape(S, H, D)).permute(1, 0, 2)
    for c in range(n):
        sel = (chunk_of == c) | (chunk_of == c + 1)
        mask = ((chunk_of[None, :] >= c - 1) & (chunk_of[None, :] <= c + 1)).expand(int(sel.sum()), S)
        o = torch.nn.functional.scaled_dot_product_attention(qt[:, sel], kt, vt, attn_mask=mask,
                                                              scale=0.3)
        o = o.permute(1, 0, 2).numpy()
        np.testing.assert_allclose(got[c].reshape(2 * L, H, D)[: o.shape[0]], o, rtol=0, atol=1e-12)


def test_window_single_chunk_equals_full_and_queue():
    L, H, D = 9, 2, 4
    q, k, v = rand((1, L, H, D), 51), rand((1, L, H, D), 52), rand((1, L, H, D), 53)
    got = oracle.window_step(q, k, v, None, scale=0.5)
    assert np.isnan(got[0, 1]).all()
    np.testing.assert_allclose(got[0, 0], oracle.full(q, k, v, scale=0.5)[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[0, 0], oracle.queue_step(q, k, v, None, scale=0.5)[0], rtol=0,
                               atol=1e-12)


def test_window_last_equals_queue_chunk():
    """The last window (no next chunk) has exactly the queue step's key/value
    set for that chunk: its predecessor and its own rows."""
    n, L, H, D = 3, 4, 2, 5
    q, k, v = rand((n, L, H, D), 61), rand((n, L, H, D), 62), rand((n, L, H, D), 63)
    got = oracle.window_step(q, k, v, None, scale=0.8)
    np.testing.assert_allclose(got[n - 1, 0], oracle.queue_step(q, k, v, None, scale=0.8)[n - 1],
                               rtol=0, atol=1e-12)


@pytest.mark.parametrize("with_cache", [False, True])
def test_window_constant_v_returned(with_cache):
    n, L, H, D = 3, 4, 2, 3
    q, k = rand((n, L, H, D), 71), rand((n, L, H, D), 72)
    v = np.broadcast_to(np.array([1.5, -2.0, 0.25]), (n, L, H, D)).copy()
    cache = make_cache(k, v) if with_cache else None
    got = oracle.window_step(q, k, v, cache)
    for c in range(n):
        rows = 2 * L if c + 1 < n else L
        np.testing.assert_allclose(got[c].reshape(2 * L, H, D)[:rows],
                                   np.broadcast_to(v[0, 0], (rows, H, D)), rtol=0, atol=1e-12)


def test_window_zero_query_is_mean_over_window():
    n, L, H, D = 4, 3, 1, 2
    k, v = rand((n, L, H, D), 81), rand((n, L, H, D), 82)
    q = np.zeros((n, L, H, D))
    got = oracle.window_step(q, k, v, None)
    for c in range(n):
        keys = v[max(c - 1, 0): min(c + 2, n)].reshape(-1, H, D)
        rows = 2 * L if c + 1 < n else L
        np.testing.assert_allclose(got[c].reshape(2 * L, H, D)[:rows],
                                   np.broadcast_to(keys.mean(0), (rows, H, D)), rtol=0,
                                   atol=1e-12)


def test_window_rows_match_window_step():
    n, L, H, D = 3, 5, 2, 4
    q, k, v = rand((n, L, H, D), 91), rand((n, L, H, D), 92), rand((n, L, H, D), 93)
    cache = make_cache(k, v)
    full = oracle.window_step(q, k, v, cache)
    rows = [(0, 1, 0), (0, 0, 7), (1, 1, 9), (2, 0, 4), (1, 0, 5)]
    got = oracle.window_rows(q, k, v, cache, rows)
    for i, (c, h, r) in enumerate(rows):
        np.testing.assert_array_equal(got[i], full[c, r // L, r % L, h])


@pytest.mark.parametrize("L,n", [(1, 1), (3, 4), (7, 2), (16, 5)])
def test_window_index_map_matches_mask_enumeration(L, n):
    for c in range(n):
        src, ch, row = oracle.window_index_map(L, n, c)
        exp = [(oracle.SRC_PRED, c - 1, r) for r in range(L)] if c >= 1 else []
        exp += [(oracle.SRC_OWN, cc, r) for cc in (c, c + 1) if cc < n for r in range(L)]
        assert list(zip(src.tolist(), ch.tolist(), row.tolist())) == exp
        assert oracle.window_kv_set_size(L, n, c) == len(exp)
        assert oracle.window_q_rows(L, n, c) == (2 * L if c + 1 < n else L)


# --------------------------------------------------------------------------
# streaming queue over a ring of slots (DualParal write-up, section 二)

from oracle import fifo as fifo_sim  # noqa: E402


@pytest.mark.parametrize("S,tail,n", [(5, 3, 4), (5, 1, 4), (4, 0, 4), (7, 6, 1), (3, 2, 3)])
def test_ring_step_is_the_queue_step_on_gathered_chunks(S, tail, n):
    L, H, D = 6, 2, 5
    q, k, v = rand((S, L, H, D), 101), rand((S, L, H, D), 102), rand((S, L, H, D), 103)
    order = [(tail - c) % S for c in range(n)]  # processing order, tail first
    lin = oracle.queue_step(q[order], k[order], v[order], None, scale=0.6)
    rows = [(c, h, r) for c in range(n) for h in range(H) for r in range(L)]
    got = oracle.ring_rows(q, k, v, tail, n, rows, scale=0.6)
    np.testing.assert_allclose(got, np.array([lin[c, r, h] for c, h, r in rows]), rtol=0,
                               atol=1e-12)


def test_ring_wraparound_closed_form():
    """S = 3, tail in slot 0: chunk 0 is slot 0, chunk 1 slot 2 (wrapped), and
    chunk 1's predecessor is chunk 0 in slot 0.  One token, D = 1, q = 1:
    chunk 1 sees keys (slot 0: ln 3, slot 2: 0), weights (3/4, 1/4), values
    (8, 4) -> 7; chunk 0 sees only its own key -> its value 8."""
    q = np.ones((3, 1, 1, 1))
    k = np.array([math.log(3.0), 50.0, 0.0]).reshape(3, 1, 1, 1)   # slot 1 unused
    v = np.array([8.0, -100.0, 4.0]).reshape(3, 1, 1, 1)
    got = oracle.ring_rows(q, k, v, 0, 2, [(0, 0, 0), (1, 0, 0)], scale=1.0)
    np.testing.assert_allclose(got[:, 0], [8.0, 7.0], rtol=0, atol=1e-12)
    assert [oracle.ring_slot(3, 0, c) for c in range(3)] == [0, 2, 1]


def test_fifo_follows_the_page():
    """Noise falls from tail to head (steps done rise), every chunk stays exactly
    `depth` steps, chunks leave in arrival order, the queue never exceeds depth,
    and live chunks always sit in distinct slots."""
    total, S, depth = 11, 5, 4
    sched = fifo_sim.run(total, S, depth)
    assert len(sched) == total + depth - 1
    entered, left = {}, []
    for step, (pushed, live, popped) in enumerate(sched):
        assert 1 <= len(live) <= depth
        dones = [d for _, _, d in live]
        assert dones == sorted(dones) and len(set(dones)) == len(dones)
        assert len({s for _, s, _ in live}) == len(live)
        assert [s for _, s, _ in live] == [(live[0][1] - c) % S for c in range(len(live))]
        for g, _, d in live:
            entered.setdefault(g, step - d)
        if popped >= 0:
            g_head = live[-1][0]
            assert popped == g_head % S and step - entered[g_head] + 1 == depth
            left.append(g_head)
    assert left == list(range(total))


def test_fifo_rejects_misuse():
    f = fifo_sim.Fifo(4, 2)
    with pytest.raises(ValueError):
        f.step()
    f.push()
    f.push()
    with pytest.raises(ValueError):
        f.push()           # full
    f.step()
    with pytest.raises(ValueError):
        f.pop()            # head has done 1 of 2 steps
    f.step()
    assert f.pop() == 0
    with pytest.raises(ValueError):
        fifo_sim.Fifo(3, 4)


# --------------------------------------------------------------------------
# coordinated noise initialization (DualParal write-up, section 三)

from oracle import noise as noise_sim  # noqa: E402


def test_noise_select_closed_forms():
    # keys order the candidates: pool 6, tail chunk used [4, 0, 5, 2] (last 2: 5, 2)
    keys = np.array([50, 10, 40, 30, 20, 60], np.uint32)
    idx = noise_sim.select(6, keys, 3, prev_idx=[4, 0, 5, 2], n_excl=2)
    # candidates {0, 1, 3, 4} by key: 1 (10), 4 (20), 3 (30), 0 (50)
    assert idx.tolist() == [1, 4, 3]
    # equal keys fall back to the pool index
    assert noise_sim.select(4, [7, 7, 7, 7], 4).tolist() == [0, 1, 2, 3]
    # the first chunk has nothing to avoid
    assert noise_sim.select(6, keys, 6).tolist() == [1, 4, 3, 2, 0, 5]
    # pool exactly F + E: the new chunk takes every frame the neighbour's tail did not use
    idx = noise_sim.select(6, keys, 4, prev_idx=[0, 1, 2, 3], n_excl=2)
    assert sorted(idx.tolist()) == [0, 1, 4, 5]


def test_noise_select_properties_over_a_long_video():
    """Chunk after chunk: frames are distinct within a chunk, never reuse what
    the neighbour's last E frames used, every pool frame keeps being used (the
    whole noise space), and the copies are exact."""
    P, F, E = 12, 8, 4
    rng = np.random.default_rng(5)
    pool = rng.standard_normal((P, 3, 5)).astype(np.float32)
    prev, used = None, set()
    for _ in range(40):
        keys = rng.integers(0, 2 ** 32, P, dtype=np.uint64).astype(np.uint32)
        idx = noise_sim.select(P, keys, F, prev, E)
        assert len(set(idx.tolist())) == F and ((0 <= idx) & (idx < P)).all()
        if prev is not None:
            assert not set(idx.tolist()) & set(prev[F - E:].tolist())
        chunk = noise_sim.init_chunk(pool, idx)
        assert np.array_equal(chunk, pool[idx])
        used |= set(idx.tolist())
        prev = idx
    assert used == set(range(P))


def test_noise_select_is_a_uniform_shuffle():
    """With uniform keys every candidate is equally likely at every position."""
    P, F = 5, 5
    rng = np.random.default_rng(11)
    counts = np.zeros((F, P))
    trials = 4000
    for _ in range(trials):
        keys = rng.integers(0, 2 ** 32, P, dtype=np.uint64).astype(np.uint32)
        for f, p in enumerate(noise_sim.select(P, keys, F)):
            counts[f, p] += 1
    assert np.abs(counts / trials - 1 / P).max() < 0.035


def test_noise_select_rejects_too_small_pool():
    with pytest.raises(ValueError):
        noise_sim.select(5, np.zeros(5, np.uint32), 4, prev_idx=[0, 1, 2, 3], n_excl=2)
