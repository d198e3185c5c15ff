"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

Each ``pin_*`` function takes the oracle module and raises AssertionError if
the oracle disagrees with a fact that does not come from the oracle itself:
printed numbers of the pages' worked examples (fixtures under tests/golden/),
closed forms, invariants of Eq. (1), special cases that reduce to plain
arithmetic, and a 50-digit brute-force evaluation on tiny shapes.  The pin
tests run them as they are; the mutation tests run them against copies of the
oracle with one planted mistake each and require that some pin fails.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


def _half_unit(printed: str) -> float:
    """Half a unit in the last printed digit of a decimal string."""
    if "." in printed:
        return 0.5 * 10.0 ** (-len(printed.split(".")[1]))
    return 0.5


def _worked_example():
    g = _load("worked_example_2d.json")
    q = np.array(g["query"], dtype=np.float64)
    K = np.array([e["k"] for e in g["keys"]], dtype=np.float64)
    return g, q, K


# --- worked example (《精读 …》, figure 「一句话里的注意力」) -------------------

def pin_worked_example_scores(so):
    """Printed scores q·k/√2 (two decimals) of the seven keys."""
    g, q, K = _worked_example()
    s = so.scores(q[None, :], K, 1.0 / math.sqrt(2.0))[0]
    for e, val in zip(g["keys"], s):
        p = e["printed_score"]
        assert abs(val - float(p)) <= _half_unit(p) + 1e-12, (e["token"], val, p)


def pin_worked_example_weights(so):
    """Printed weights (percent, two significant digits), through the full path.

    V = identity makes the output row equal to the weight row exactly
    (each output column j is w_j·1 plus zeros).  The scale is left to the
    oracle's default, so this also pins 1/√d_k with d_k = 2.
    """
    g, q, K = _worked_example()
    eye = np.eye(len(K))
    out = so.attention(q[None, None, None, :], K[None, None], eye[None, None])[0, 0, 0]
    for e, w in zip(g["keys"], out):
        p = e["printed_weight_percent"]
        assert abs(100.0 * w - float(p)) <= _half_unit(p) + 1e-9, (e["token"], 100 * w, p)
    assert abs(out.sum() - 1.0) < 1e-15
    # the largest weight sits on 猫 = [2, 0.4] and is about two thirds
    assert int(np.argmax(out)) == 1 and 0.65 < out[1] < 0.67


def pin_worked_example_causal(so):
    """Causal toggle: 它 is position 4 (0-based) of 7 and sees keys 0..4 only.

    The page prints no numbers for this view; the pin is that the masked
    softmax equals the unmasked weights of the visible keys renormalised,
    with exactly zero weight on the two later keys.
    """
    g, q, K = _worked_example()
    i = g["query_position"]
    Q = K.copy()
    Q[i] = q  # self-attention over the 7 tokens; only row i is checked
    eye = np.eye(len(K))
    full = so.attention(Q[None, None], K[None, None], eye[None, None])[0, 0, i]
    caus = so.attention(Q[None, None], K[None, None], eye[None, None], causal=True)[0, 0, i]
    assert np.all(caus[i + 1:] == 0.0)
    ref = full[: i + 1] / full[: i + 1].sum()
    assert np.allclose(caus[: i + 1], ref, rtol=0, atol=1e-14), (caus, ref)


# --- two-key saturation (《精读 …》, after footnote 4) ---------------------------

def pin_two_key_saturation(so):
    g = _load("two_key_saturation.json")
    for case in g["cases"]:
        s0, s1 = case["raw_scores"]
        # q·k1 = s0, q·k2 = s1 with q = [1, 0], k1 = [s0, 0], k2 = [s1, 1]
        q = np.array([[[[1.0, 0.0]]]])
        k = np.array([[[[s0, 0.0], [s1, 1.0]]]])
        v = np.eye(2)[None, None]
        w = so.attention(q, k, v, scale=case["scale"])[0, 0, 0]
        # closed form: softmax of two logits is the logistic function of their gap
        x = case["scale"] * (s0 - s1)
        assert abs(w[0] - 1.0 / (1.0 + math.exp(-x))) < 1e-15
        for got, p in zip(w, case["printed_weights"]):
            if p is not None:
                assert abs(got - float(p)) <= _half_unit(p) + 1e-12, (got, p)
        p1 = w[0] * (1.0 - w[0])
        assert abs(p1 - float(case["printed_p1mp"])) <= _half_unit(case["printed_p1mp"]) + 1e-12


# --- invariants and special cases of Eq. (1) -----------------------------------

def _rand(rng, *shape):
    return rng.standard_normal(shape)


def pin_rows_sum_and_exact_zeros(so):
    """Rows of weights sum to 1; illegal positions get weight exactly +0.0."""
    rng = np.random.default_rng(7)
    B, h, n, d = 3, 2, 9, 5
    m = n
    q, k = _rand(rng, B, h, n, d), _rand(rng, B, h, m, d)
    v = np.broadcast_to(np.eye(m), (B, h, m, m)).copy()
    key_lens = np.array([4, 9, 0], dtype=np.int32)
    for causal in (False, True):
        w = so.attention(q, k, v, causal=causal, key_lens=key_lens)
        for b in range(B):
            L = key_lens[b]
            for i in range(n):
                vis = np.array([(j < L) and (not causal or j <= i) for j in range(m)])
                row = w[b, :, i]
                assert np.all(row[:, ~vis] == 0.0) and not np.signbit(row[:, ~vis]).any()
                if vis.any():
                    assert np.allclose(row.sum(-1), 1.0, rtol=0, atol=1e-14)
                    assert np.all(row[:, vis] > 0.0)
                else:
                    assert np.all(row == 0.0)


def pin_zero_query_gives_mean(so):
    """Q = 0 ⇒ every legal score is 0 ⇒ the output is the mean of the legal V rows."""
    rng = np.random.default_rng(11)
    B, h, n, m, d, dv = 2, 3, 6, 6, 4, 5
    q = np.zeros((B, h, n, d))
    k, v = _rand(rng, B, h, m, d), _rand(rng, B, h, m, dv)
    key_lens = np.array([3, 6])
    for causal in (False, True):
        o = so.attention(q, k, v, causal=causal, key_lens=key_lens)
        for b in range(B):
            for i in range(n):
                hi = key_lens[b] if not causal else min(key_lens[b], i + 1)
                ref = v[b, :, :hi].mean(axis=1)
                assert np.allclose(o[b, :, i], ref, rtol=0, atol=1e-14)


def pin_single_visible_key(so):
    """One legal key ⇒ weight exactly 1 ⇒ output equals that value row bitwise."""
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 2, 2, 5, 3), _rand(rng, 2, 2, 5, 3), _rand(rng, 2, 2, 5, 4)
    o = so.attention(q, k, v, key_lens=np.array([1, 1]))
    assert np.array_equal(o, np.broadcast_to(v[:, :, :1], o.shape))
    o = so.attention(q, k, v, causal=True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])


def pin_permutation_equivariance(so):
    """Permuting (K, V) rows jointly leaves O unchanged; permuting Q permutes O."""
    rng = np.random.default_rng(17)
    B, h, n, m, d, dv = 2, 2, 5, 7, 3, 4
    q, k, v = _rand(rng, B, h, n, d), _rand(rng, B, h, m, d), _rand(rng, B, h, m, dv)
    key_lens = np.array([5, 7])
    o = so.attention(q, k, v, key_lens=key_lens)
    # permute keys inside the legal prefix of every batch element
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        p = rng.permutation(key_lens[b])
        k2[b][:, : key_lens[b]] = k[b][:, p]
        v2[b][:, : key_lens[b]] = v[b][:, p]
    assert np.allclose(so.attention(q, k2, v2, key_lens=key_lens), o, rtol=0, atol=1e-13)
    p = rng.permutation(n)
    assert np.allclose(so.attention(q[:, :, p], k, v, key_lens=key_lens), o[:, :, p], rtol=0, atol=1e-13)


def pin_shift_invariance(so):
    """K + 1wᵀ shifts each row's logits by a constant ⇒ O unchanged; V + 1cᵀ ⇒ O + cᵀ."""
    rng = np.random.default_rng(19)
    B, h, n, m, d, dv = 1, 2, 6, 6, 3, 3
    q, k, v = _rand(rng, B, h, n, d), _rand(rng, B, h, m, d), _rand(rng, B, h, m, dv)
    w = rng.standard_normal(d)
    c = rng.standard_normal(dv)
    for causal in (False, True):
        o = so.attention(q, k, v, causal=causal)
        assert np.allclose(so.attention(q, k + w, v, causal=causal), o, rtol=0, atol=1e-12)
        assert np.allclose(so.attention(q, k, v + c, causal=causal), o + c, rtol=0, atol=1e-12)


def pin_hard_limit(so):
    """Large scale with distinct scores ⇒ the softmax picks the arg-max key."""
    rng = np.random.default_rng(23)
    q, k, v = _rand(rng, 1, 1, 4, 3), _rand(rng, 1, 1, 6, 3), _rand(rng, 1, 1, 6, 2)
    o = so.attention(q, k, v, scale=1e4)
    best = np.argmax(q[0, 0] @ k[0, 0].T, axis=1)
    assert np.allclose(o[0, 0], v[0, 0, best], rtol=0, atol=1e-9)


def pin_cross_attention_shapes(so):
    """n ≠ m (encoder–decoder attention) and the multi-head shape walk.

    《精读 …》's ten-token walk: per head 10×64 queries, a 10×10 weight matrix,
    a 10×64 output; eight heads concatenate back to 10×512.
    """
    rng = np.random.default_rng(29)
    q, k, v = _rand(rng, 1, 8, 10, 64), _rand(rng, 1, 8, 10, 64), _rand(rng, 1, 8, 10, 64)
    o = so.attention(q, k, v)
    assert o.shape == (1, 8, 10, 64)
    assert o[0].transpose(1, 0, 2).reshape(10, 512).shape == (10, 512)
    q2 = _rand(rng, 2, 3, 4, 5)
    k2, v2 = _rand(rng, 2, 3, 7, 5), _rand(rng, 2, 3, 7, 6)
    assert so.attention(q2, k2, v2).shape == (2, 3, 4, 6)


def pin_brute_force_mp(so):
    """50-digit scalar-loop evaluation on tiny shapes, every mask kind."""
    from oracle.brute_mp import attention_mp

    rng = np.random.default_rng(31)
    shapes = [(2, 3, 4, 4, 3, 2), (2, 2, 3, 5, 2, 3), (1, 2, 5, 5, 4, 4)]
    for (B, h, n, m, d, dv) in shapes:
        q, k, v = _rand(rng, B, h, n, d), _rand(rng, B, h, m, d), _rand(rng, B, h, m, dv)
        kls = [None, rng.integers(0, m + 2, size=B)]
        for key_lens in kls:
            for causal in ([False, True] if n == m else [False]):
                scale = 0.7
                o = so.attention(q, k, v, scale=scale, causal=causal, key_lens=key_lens)
                ref = attention_mp(q.tolist(), k.tolist(), v.tolist(), scale, causal,
                                   None if key_lens is None else key_lens.tolist())
                ref = np.array([[[[float(x) for x in r] for r in hd] for hd in bb] for bb in ref])
                assert np.allclose(o, ref, rtol=0, atol=1e-13), (B, h, n, m, causal, key_lens)


def pin_nan_propagation(so):
    """IEEE arithmetic on Eq. (1): a NaN logit of a legal key makes that row's
    maximum, every weight and so the whole output row NaN; a NaN value
    component of a key every row sees reaches only that output column; a row
    with no legal key is the zero vector whatever its query holds, and rows
    that cannot see a key are untouched by a NaN in it."""
    rng = np.random.default_rng(19)
    B, h, n, m, d, dv = 2, 1, 6, 6, 3, 4
    q, k, v = _rand(rng, B, h, n, d), _rand(rng, B, h, m, d), _rand(rng, B, h, m, dv)
    q[0, 0, 2, 1] = np.nan  # batch 0: every key legal ⇒ row 2 all NaN
    q[1, 0, 4, 0] = np.nan  # batch 1: no legal key ⇒ row 4 zero
    o = so.attention(q, k, v, key_lens=np.array([6, 0]))
    assert np.isnan(o[0, 0, 2]).all()
    assert np.isfinite(np.delete(o[0, 0], 2, axis=0)).all()
    assert np.array_equal(o[1], np.zeros_like(o[1]))
    q[:] = _rand(rng, B, h, n, d)
    k[0, 0, 3, 2] = np.nan  # causal: rows 3.. see key 3, rows 0..2 do not
    v[1, 0, 0, 2] = np.nan  # causal: every row weighs key 0 > 0
    o = so.attention(q, k, v, causal=True)
    assert np.isnan(o[0, 0, 3:]).all() and np.isfinite(o[0, 0, :3]).all()
    assert np.isnan(o[1, 0, :, 2]).all()
    assert np.isfinite(np.delete(o[1, 0], 2, axis=1)).all()


def _window_slice(i, n, L, left, right, align):
    """Index range [lo, hi) of the legal keys of query i, by direct reading of the
    window's definition (no mask arithmetic shared with the oracle)."""
    p = i if align == "top_left" else i + L - n
    lo = 0 if left is None else max(0, p - left)
    hi = L if right is None else min(L, p + right + 1)
    return lo, max(lo, hi)


WINDOWS = [(2, 1, "top_left"), (0, 3, "top_left"), (None, 2, "top_left"), (3, None, "top_left"),
           (1, 1, "bottom_right"), (None, 0, "bottom_right"), (4, 0, "bottom_right")]


def pin_window_zero_query_gives_window_mean(so):
    """Restricted attention (《精读 …》 Table 1): Q = 0 ⇒ every legal score is 0 ⇒
    the output row is the plain mean of the value rows inside the query's
    window (and the zero vector when the window holds no legal key)."""
    rng = np.random.default_rng(23)
    B, h, n, m, d, dv = 2, 2, 5, 8, 3, 4
    q = np.zeros((B, h, n, d))
    k, v = _rand(rng, B, h, m, d), _rand(rng, B, h, m, dv)
    key_lens = np.array([8, 3])
    for left, right, align in WINDOWS:
        o = so.attention(q, k, v, key_lens=key_lens, window=(left, right, align))
        for b in range(B):
            for i in range(n):
                lo, hi = _window_slice(i, n, int(key_lens[b]), left, right, align)
                ref = v[b, :, lo:hi].mean(axis=1) if hi > lo else np.zeros((h, dv))
                assert np.allclose(o[b, :, i], ref, rtol=0, atol=1e-14), (left, right, align, b, i)


def pin_window_single_key(so):
    """Window (0, 0) on self-attention: each query sees only its own position,
    whose weight is exactly 1, so the output row is that value row bitwise."""
    rng = np.random.default_rng(29)
    q, k, v = _rand(rng, 2, 2, 6, 3), _rand(rng, 2, 2, 6, 3), _rand(rng, 2, 2, 6, 4)
    o = so.attention(q, k, v, window=(0, 0))
    assert np.array_equal(o, v)
    # bottom-right with one query: the last legal key only
    o = so.attention(q[:, :, :1], k, v, key_lens=np.array([6, 4]), window=(0, 0, "bottom_right"))
    assert np.array_equal(o[0, :, 0], v[0, :, 5]) and np.array_equal(o[1, :, 0], v[1, :, 3])


def pin_window_brute_force_mp(so):
    """The 50-digit evaluator on tiny shapes with every window kind."""
    from oracle.brute_mp import attention_mp

    rng = np.random.default_rng(31)
    B, h, n, m, d, dv = 2, 1, 4, 6, 3, 2
    q, k, v = _rand(rng, B, h, n, d), _rand(rng, B, h, m, d), _rand(rng, B, h, m, dv)
    key_lens = np.array([6, 2])
    for left, right, align in WINDOWS:
        o = so.attention(q, k, v, scale=0.7, key_lens=key_lens, window=(left, right, align))
        ref = attention_mp(q.tolist(), k.tolist(), v.tolist(), 0.7, key_lens=key_lens.tolist(),
                           window=(left, right, align))
        ref = np.array([[[[float(x) for x in row] for row in hd] for hd in bt] for bt in ref])
        assert np.allclose(o, ref, rtol=0, atol=1e-14), (left, right, align)


def pin_window_reduces_to_plain_masks(so):
    """An unbounded window is no mask; (None, 0) top-left on self-attention is
    the decoder's causal mask; a single bottom-right query with (None, 0) sees
    every legal key (it is the last position)."""
    rng = np.random.default_rng(37)
    q, k, v = _rand(rng, 2, 2, 5, 3), _rand(rng, 2, 2, 5, 3), _rand(rng, 2, 2, 5, 4)
    kl = np.array([5, 3])
    assert np.array_equal(so.attention(q, k, v, key_lens=kl, window=(None, None)),
                          so.attention(q, k, v, key_lens=kl))
    assert np.array_equal(so.attention(q, k, v, key_lens=kl, window=(None, 0)),
                          so.attention(q, k, v, key_lens=kl, causal=True))
    assert np.array_equal(so.attention(q[:, :, 4:], k, v, key_lens=kl, window=(None, 0, "bottom_right")),
                          so.attention(q[:, :, 4:], k, v, key_lens=kl))


def _mha_weights(rng, h, d_model, d_k, d_v, s=None):
    s = 1.0 / math.sqrt(d_model) if s is None else s
    return (s * rng.standard_normal((h, d_model, d_k)), s * rng.standard_normal((h, d_model, d_k)),
            s * rng.standard_normal((h, d_model, d_v)), s * rng.standard_normal((h * d_v, d_model)))


def pin_multihead_brute_force_mp(so):
    """The multi-head sublayer against scalar-loop 50-digit projections, heads
    and output projection (self- and cross-attention, padding, causal)."""
    from oracle.brute_mp import multihead_mp

    rng = np.random.default_rng(43)
    for (B, n, m, d_model, h, d_k, d_v, causal) in [(2, 3, 3, 6, 2, 3, 2, True), (1, 2, 4, 4, 3, 2, 3, False)]:
        xq = rng.standard_normal((B, n, d_model))
        xkv = xq if causal else rng.standard_normal((B, m, d_model))
        wq, wk, wv, wo = _mha_weights(rng, h, d_model, d_k, d_v, s=0.8)
        kl = np.array([n, 1][:B]) if causal else None
        o = so.multihead(xq, xkv, wq, wk, wv, wo, scale=0.6, causal=causal, key_lens=kl)
        ref = multihead_mp(xq.tolist(), xkv.tolist(), wq.tolist(), wk.tolist(), wv.tolist(),
                           wo.tolist(), 0.6, causal=causal, key_lens=None if kl is None else kl.tolist())
        ref = np.array([[[float(x) for x in r] for r in bb] for bb in ref])
        assert np.allclose(o, ref, rtol=0, atol=1e-13), (B, n, m, causal)


def pin_multihead_single_identity_head(so):
    """h = 1 with d_k = d_v = d_model and identity projections: the sublayer
    is plain Eq. (1) on the inputs themselves."""
    rng = np.random.default_rng(47)
    B, n, m, d = 2, 4, 5, 3
    xq, xkv = rng.standard_normal((B, n, d)), rng.standard_normal((B, m, d))
    eye = np.eye(d)[None]
    o = so.multihead(xq, xkv, eye, eye, eye, np.eye(d), key_lens=np.array([5, 2]))
    ref = so.attention(xq[:, None], xkv[:, None], xkv[:, None], key_lens=np.array([5, 2]))[:, 0]
    assert np.allclose(o, ref, rtol=0, atol=1e-14)


def pin_multihead_head_permutation(so):
    """Relabelling the heads (their three projections and their row block of
    W^O together) leaves the sublayer unchanged: Concat only orders the heads,
    and W^O's rows follow them."""
    rng = np.random.default_rng(53)
    B, n, d_model, h, d_k, d_v = 2, 5, 8, 4, 2, 3
    x = rng.standard_normal((B, n, d_model))
    wq, wk, wv, wo = _mha_weights(rng, h, d_model, d_k, d_v)
    perm = np.array([2, 0, 3, 1])
    wo_p = wo.reshape(h, d_v, d_model)[perm].reshape(h * d_v, d_model)
    o1 = so.multihead(x, x, wq, wk, wv, wo, causal=True)
    o2 = so.multihead(x, x, wq[perm], wk[perm], wv[perm], wo_p, causal=True)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13)
    # a permutation of the projections alone (W^O kept) does change the output
    o3 = so.multihead(x, x, wq[perm], wk[perm], wv[perm], wo, causal=True)
    assert not np.allclose(o1, o3, rtol=0, atol=1e-6)


def pin_multihead_page_shapes(so):
    """《精读 …》 multi-head section's walk-through: a 10-token input of width
    512 with h = 8 heads of d_k = d_v = 64 gives a 10 × 512 output, and the
    four projection matrices hold 4 · 512² = 1,048,576 weights."""
    rng = np.random.default_rng(59)
    h, d_model, d = 8, 512, 64
    x = rng.standard_normal((1, 10, d_model))
    wq, wk, wv, wo = _mha_weights(rng, h, d_model, d, d)
    assert wq.size + wk.size + wv.size + wo.size == 1_048_576
    assert so.multihead(x, x, wq, wk, wv, wo).shape == (1, 10, d_model)


def _row_masks(n, m, key_lens):
    """(causal, key_lens, window) combinations for the single-row helpers:
    every mask kind, each window kind with both alignments, with and without
    key lengths."""
    masks = [(False, None, None), (False, key_lens, None)]
    if n == m:
        masks += [(True, None, None), (True, key_lens, None)]
    masks += [(False, key_lens, w) for w in WINDOWS] + [(False, None, w) for w in WINDOWS[:3]]
    return masks


def pin_rows_brute_force_mp(so):
    """``attention_rows`` (one output row per pick, for checking full-size
    outputs row by row) against the 50-digit evaluator on tiny shapes: every
    mask kind, key lengths 0, inside and past m, every window kind with both
    alignments, n ≠ m, and picks in scrambled order, so that each row must use
    its own batch element's key length, its own position and its own window
    shift."""
    from oracle.brute_mp import attention_mp

    rng = np.random.default_rng(41)
    for (B, h, n, m, d, dv), kl in (((2, 2, 5, 5, 3, 2), [0, 7]), ((3, 2, 3, 6, 2, 3), [6, 1, 4]),
                                    ((2, 1, 6, 4, 3, 2), [3, 9])):
        q, k, v = _rand(rng, B, h, n, d), _rand(rng, B, h, m, d), _rand(rng, B, h, m, dv)
        picks = [(b, hh, i) for b in range(B) for hh in range(h) for i in range(n)]
        picks = [picks[t] for t in rng.permutation(len(picks))]
        for causal, key_lens, window in _row_masks(n, m, np.array(kl)):
            got = so.attention_rows(q, k, v, picks, scale=0.7, causal=causal, key_lens=key_lens,
                                    window=window)
            ref = attention_mp(q.tolist(), k.tolist(), v.tolist(), 0.7, causal,
                               None if key_lens is None else list(key_lens), window=window)
            for r, (b, hh, i) in enumerate(picks):
                assert np.allclose(got[r], [float(x) for x in ref[b][hh][i]], rtol=0, atol=1e-13), \
                    (B, h, n, m, causal, key_lens, window, (b, hh, i))


def pin_rows_match_whole_heads(so):
    """Rows from ``attention_rows`` equal the same rows of ``attention`` (pinned
    above) on heads longer than the oracle's 512-row evaluation slice: rows on
    both sides of the slice edge and the last row, causal, padded, windowed
    with both alignments, and n ≠ m."""
    rng = np.random.default_rng(43)
    for (B, h, n, m, kl) in ((2, 2, 600, 600, [600, 300]), (2, 1, 520, 700, [700, 0])):
        q, k, v = _rand(rng, B, h, n, 4), _rand(rng, B, h, m, 4), _rand(rng, B, h, m, 3)
        rows = [0, 1, 255, 256, 511, 512, 513, n - 1] + list(rng.integers(0, n, 3))
        picks = [(b, hh, int(i)) for b in range(B) for hh in range(h) for i in rows]
        masks = [(n == m, np.array(kl), None), (False, np.array(kl), (100, 0, "top_left")),
                 (False, np.array(kl), (None, 0, "bottom_right")), (False, None, (64, 64, "bottom_right"))]
        for causal, key_lens, window in masks:
            whole = so.attention(q, k, v, causal=causal, key_lens=key_lens, window=window)
            got = so.attention_rows(q, k, v, picks, causal=causal, key_lens=key_lens, window=window)
            ref = np.stack([whole[b, hh, i] for (b, hh, i) in picks])
            assert np.allclose(got, ref, rtol=0, atol=1e-13), (n, m, causal, kl, window)


ALL_PINS = [
    pin_worked_example_scores,
    pin_worked_example_weights,
    pin_worked_example_causal,
    pin_two_key_saturation,
    pin_rows_sum_and_exact_zeros,
    pin_zero_query_gives_mean,
    pin_single_visible_key,
    pin_permutation_equivariance,
    pin_shift_invariance,
    pin_hard_limit,
    pin_cross_attention_shapes,
    pin_brute_force_mp,
    pin_nan_propagation,
    pin_window_zero_query_gives_window_mean,
    pin_window_single_key,
    pin_window_brute_force_mp,
    pin_window_reduces_to_plain_masks,
    pin_multihead_brute_force_mp,
    pin_multihead_single_identity_head,
    pin_multihead_head_permutation,
    pin_multihead_page_shapes,
    pin_rows_brute_force_mp,
    pin_rows_match_whole_heads,
]


# --- gradient of Eq. (1) (oracle.sdpa_backward) --------------------------------
#
# The pages print no gradient, so these pins rest on the derivative itself
# (finite differences of the forward pass, at 60 digits and in fp64) and on
# invariants that follow from the form of Eq. (1).  Each takes the backward
# module ``sb``.

_BWD_MASKS = [  # (causal, key_lens, window) for B = 2
    (False, None, None),
    (True, None, None),
    (False, [3, 1], None),
    (False, None, (1, 0, "top_left")),
    (False, [4, 2], (None, 0, "bottom_right")),
]


def _bwd_case(rng, B, h, n, m, d, dv):
    return (_rand(rng, B, h, n, d), _rand(rng, B, h, m, d), _rand(rng, B, h, m, dv),
            _rand(rng, B, h, n, dv))


def pin_bwd_finite_difference_mp(sb):
    """Every gradient element against a 60-digit central difference of Eq. (1)."""
    from oracle.brute_mp import attention_grad_fd_mp

    rng = np.random.default_rng(71)
    for (n, m) in ((3, 3), (2, 4)):
        q, k, v, do = _bwd_case(rng, 2, 1, n, m, 3, 2)
        for causal, kl, win in _BWD_MASKS:
            if causal and n != m:
                continue
            got = sb.attention_backward(q, k, v, do, scale=0.7, causal=causal, key_lens=kl,
                                        window=win)
            ref = attention_grad_fd_mp(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 0.7,
                                       causal, kl, win)
            for name, a, r in zip(("dq", "dk", "dv"), got, ref):
                assert np.allclose(a, np.array(r), rtol=0, atol=1e-12), (name, n, m, causal, kl, win)


def pin_bwd_finite_difference_fp64(sb):
    """Larger shapes (several keys per row, ragged lengths, n ≠ m): fp64
    central differences of the forward oracle, step 1e-5 (error ~1e-9)."""
    from oracle import sdpa_oracle as so

    rng = np.random.default_rng(72)
    for (n, m, causal, kl, win) in ((6, 6, True, [6, 4], None), (5, 8, False, [8, 3], None),
                                    (7, 7, False, None, (2, 1, "top_left")),
                                    (3, 9, False, [9, 5], (None, 0, "bottom_right"))):
        q, k, v, do = _bwd_case(rng, 2, 1, n, m, 4, 3)
        got = sb.attention_backward(q, k, v, do, scale=0.6, causal=causal, key_lens=kl, window=win)
        loss = lambda q_, k_, v_: float(np.sum(do * so.attention(q_, k_, v_, scale=0.6, causal=causal,
                                                                  key_lens=kl, window=win)))
        h = 1e-5
        for which, x in enumerate((q, k, v)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                args = [q, k, v]
                up, dn = x.copy(), x.copy()
                up[idx] += h
                dn[idx] -= h
                args[which] = up
                lu = loss(*args)
                args[which] = dn
                fd[idx] = (lu - loss(*args)) / (2 * h)
            assert np.allclose(got[which], fd, rtol=0, atol=1e-7), (which, n, m, causal, kl, win)


def pin_bwd_key_shift_invariance(sb):
    """Adding one vector c to every key adds scale·q_i·c to all of row i's
    logits, which its softmax ignores: the derivative along that direction,
    Σ_j dK_j · c, is zero for every c, so Σ_j dK_j = 0 for every head."""
    rng = np.random.default_rng(73)
    q, k, v, do = _bwd_case(rng, 2, 2, 5, 7, 4, 3)
    for causal, kl, win in _BWD_MASKS:
        if causal:
            continue
        _, dk, _ = sb.attention_backward(q, k, v, do, scale=0.8, key_lens=kl, window=win)
        assert np.abs(dk.sum(axis=2)).max() < 1e-12, (kl, win)


def pin_bwd_bilinear_balance(sb):
    """The logits depend on q_i · k_j only, so Q → tQ, K → K/t changes
    nothing: d/dt at t = 1 gives ⟨dQ, Q⟩ = ⟨dK, K⟩ per head."""
    rng = np.random.default_rng(74)
    q, k, v, do = _bwd_case(rng, 2, 2, 6, 6, 4, 3)
    for causal, kl, win in _BWD_MASKS:
        dq, dk, _ = sb.attention_backward(q, k, v, do, scale=0.8, causal=causal, key_lens=kl,
                                          window=win)
        lhs = np.einsum("bhnd,bhnd->bh", dq, q)
        rhs = np.einsum("bhmd,bhmd->bh", dk, k)
        assert np.allclose(lhs, rhs, rtol=0, atol=1e-12), (causal, kl, win)


def pin_bwd_value_sum(sb):
    """o_i is linear in V with weights summing to 1 over the legal keys, so
    Σ_j dV_j = Σ_i dO_i over the rows that have a legal key."""
    rng = np.random.default_rng(75)
    q, k, v, do = _bwd_case(rng, 2, 1, 4, 6, 3, 2)
    # key_lens [6, 0]: batch 1 has no legal key at all
    _, _, dv = sb.attention_backward(q, k, v, do, scale=0.9, key_lens=[6, 0])
    assert np.allclose(dv[0].sum(axis=1), do[0].sum(axis=1), rtol=0, atol=1e-12)
    assert np.all(dv[1] == 0)


def pin_bwd_single_key(sb):
    """One legal key: every weight is 1 whatever the logits, so dQ = 0,
    dK = 0, and that key's dV is the sum of the output gradients."""
    rng = np.random.default_rng(76)
    q, k, v, do = _bwd_case(rng, 1, 2, 3, 5, 4, 2)
    dq, dk, dv = sb.attention_backward(q, k, v, do, scale=1.3, key_lens=[1])
    assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
    assert np.allclose(dv[0, :, 0], do[0].sum(axis=1), rtol=0, atol=1e-14)
    assert np.all(dv[0, :, 1:] == 0)


def pin_bwd_uniform_weights(sb):
    """q = 0 makes every legal weight 1/L.  Then dV_j = (1/L) Σ_i dO_i for the
    legal keys, and dQ_i = (scale/L) Σ_j (dO_i · (v_j − v̄)) k_j, the
    covariance of values and keys seen through dO_i (v̄ = mean legal value)."""
    rng = np.random.default_rng(77)
    _, k, v, do = _bwd_case(rng, 1, 1, 3, 5, 4, 2)
    q = np.zeros((1, 1, 3, 4))
    L, sc = 4, 0.5
    dq, _, dv = sb.attention_backward(q, k, v, do, scale=sc, key_lens=[L])
    assert np.allclose(dv[0, 0, :L], np.broadcast_to(do[0, 0].sum(axis=0) / L, (L, 2)), atol=1e-14)
    vc = v[0, 0, :L] - v[0, 0, :L].mean(axis=0)
    ref = np.array([[sc / L * sum((do[0, 0, i] @ vc[j]) * k[0, 0, j, t] for j in range(L))
                     for t in range(4)] for i in range(3)])
    assert np.allclose(dq[0, 0], ref, rtol=0, atol=1e-14)


def pin_bwd_empty_rows_pass_nothing(sb):
    """A query with no legal key has output 0 whatever Q, K, V: its dQ row is
    zero and its dO contributes to no dK or dV."""
    rng = np.random.default_rng(78)
    q, k, v, do = _bwd_case(rng, 1, 1, 4, 2, 3, 2)
    # bottom-right causal with 2 cached keys and 4 queries: rows 0 and 1 see nothing
    win = (None, 0, "bottom_right")
    dq, dk, dv = sb.attention_backward(q, k, v, do, scale=0.7, window=win)
    assert np.all(dq[0, 0, :2] == 0)
    do2 = do.copy()
    do2[0, 0, :2] = 123.0
    _, dk2, dv2 = sb.attention_backward(q, k, v, do2, scale=0.7, window=win)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def pin_lse_closed_forms(sb):
    """ln Σ_j exp(s_ij): q = 0 gives ln L; one legal key gives its logit; no
    legal key gives −∞; and exp(s − lse) sums to 1 over each row's legal keys
    (checked against 50-digit sums)."""
    import mpmath

    rng = np.random.default_rng(79)
    _, k, _, _ = _bwd_case(rng, 2, 1, 3, 6, 4, 2)
    q0 = np.zeros((2, 1, 3, 4))
    lse = sb.log_sum_exp(q0, k, scale=0.5, key_lens=[6, 0])
    assert np.allclose(lse[0], math.log(6), atol=1e-15) and np.all(lse[1] == -np.inf)
    q = rng.standard_normal((2, 1, 3, 4))
    lse1 = sb.log_sum_exp(q, k, scale=0.5, key_lens=[1, 6])
    assert np.allclose(lse1[0, 0], 0.5 * q[0, 0] @ k[0, 0, 0], atol=1e-14)
    with mpmath.workdps(50):
        for i in range(3):
            s = [mpmath.mpf(0.5) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                               for a, b in zip(q[1, 0, i], k[1, 0, j]))
                 for j in range(6)]
            assert abs(float(mpmath.log(mpmath.fsum(mpmath.exp(x) for x in s))) - lse1[1, 0, i]) < 1e-14


def pin_bwd_rows_finite_difference_mp(sb):
    """``backward_query_rows`` and ``backward_key_rows`` (gradient rows for
    checking full-size gradients) against the 60-digit central difference of
    Eq. (1): every pick in scrambled order, every mask kind, n ≠ m."""
    from oracle.brute_mp import attention_grad_fd_mp

    rng = np.random.default_rng(81)
    for (n, m) in ((3, 3), (2, 4)):
        q, k, v, do = _bwd_case(rng, 2, 2, n, m, 3, 2)
        for causal, kl, win in _BWD_MASKS:
            if causal and n != m:
                continue
            fd = attention_grad_fd_mp(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 0.7,
                                      causal, kl, win)
            picks = [(b, hh, i) for b in range(2) for hh in range(2) for i in range(n)]
            picks = [picks[t] for t in rng.permutation(len(picks))]
            dq = sb.backward_query_rows(q, k, v, do, picks, scale=0.7, causal=causal, key_lens=kl,
                                        window=win)
            for r, (b, hh, i) in enumerate(picks):
                assert np.allclose(dq[r], fd[0][b][hh][i], rtol=0, atol=1e-12), (n, m, causal, kl, win)
            for b in range(2):
                for hh in range(2):
                    keys = list(rng.permutation(m))
                    dk, dv = sb.backward_key_rows(q, k, v, do, b, hh, keys, scale=0.7, causal=causal,
                                                  key_lens=kl, window=win)
                    for r, j in enumerate(keys):
                        assert np.allclose(dk[r], fd[1][b][hh][j], rtol=0, atol=1e-12), (b, hh, j, win)
                        assert np.allclose(dv[r], fd[2][b][hh][j], rtol=0, atol=1e-12), (b, hh, j, win)


def pin_bwd_rows_match_whole(sb):
    """Gradient rows from the row helpers equal those of ``attention_backward``
    (pinned above) on heads longer than the 512-row evaluation slice, so the
    dK/dV helper must add up every slice of queries."""
    rng = np.random.default_rng(83)
    for (n, m, causal, kl, win) in ((600, 600, True, [600, 333], None),
                                    (530, 640, False, [640, 100], (None, 0, "bottom_right")),
                                    (600, 600, False, None, (50, 50, "top_left"))):
        q, k, v, do = _bwd_case(rng, 2, 1, n, m, 4, 3)
        dq, dk, dv = sb.attention_backward(q, k, v, do, causal=causal, key_lens=kl, window=win)
        picks = [(b, 0, i) for b in range(2) for i in (0, 1, 511, 512, n - 1)]
        got = sb.backward_query_rows(q, k, v, do, picks, causal=causal, key_lens=kl, window=win)
        assert np.allclose(got, np.stack([dq[b, hh, i] for (b, hh, i) in picks]), rtol=0, atol=1e-12)
        for b in range(2):
            keys = [0, 1, 99, 100, 332, 333, 511, 512, m - 1]
            gk, gv = sb.backward_key_rows(q, k, v, do, b, 0, keys, causal=causal, key_lens=kl,
                                          window=win)
            assert np.allclose(gk, dk[b, 0, keys], rtol=0, atol=1e-12), (n, m, b)
            assert np.allclose(gv, dv[b, 0, keys], rtol=0, atol=1e-12), (n, m, b)


BACKWARD_PINS = [
    pin_bwd_finite_difference_mp,
    pin_bwd_finite_difference_fp64,
    pin_bwd_key_shift_invariance,
    pin_bwd_bilinear_balance,
    pin_bwd_value_sum,
    pin_bwd_single_key,
    pin_bwd_uniform_weights,
    pin_bwd_empty_rows_pass_nothing,
    pin_lse_closed_forms,
    pin_bwd_rows_finite_difference_mp,
    pin_bwd_rows_match_whole,
]


# --- attention dropout (oracle.sdpa_dropout) ---------------------------------
#
# Dropout on the attention weights after the softmax, kept weights scaled by
# c = 1/(1 − p) (the reading the dropout oracle states).  Each pin takes the
# module ``oracle.sdpa_dropout``.

def _drop_case(rng, B, h, n, m, d, dv):
    q = rng.standard_normal((B, h, n, d))
    k = rng.standard_normal((B, h, m, d))
    v = rng.standard_normal((B, h, m, dv))
    return q, k, v


def pin_drop_unpack_bit_order(sd):
    """Bit j mod 32 of word ⌊j/32⌋ is key j (least significant bit first)."""
    words = np.array([[0x00000005, 0x80000002]], dtype=np.uint32)
    got = sd.unpack_keep(words, 64)[0]
    assert set(np.flatnonzero(got)) == {0, 2, 33, 63}
    assert sd.unpack_keep(words, 35)[0].tolist() == got[:35].tolist()


def pin_drop_all_kept_is_plain(sd):
    """Every weight kept and c = 1: Eq. (1) itself (the pinned oracle)."""
    import oracle.sdpa_oracle as so

    rng = np.random.default_rng(90)
    q, k, v = _drop_case(rng, 2, 2, 5, 7, 4, 3)
    keep = np.ones((2, 2, 5, 7), bool)
    for kw in (dict(), dict(key_lens=[7, 2]), dict(window=(1, 2, "top_left")),
               dict(window=(None, 0, "bottom_right"), key_lens=[3, 7])):
        assert np.array_equal(sd.attention_dropout(q, k, v, keep, 1.0, **kw), so.attention(q, k, v, **kw))


def pin_drop_all_dropped_is_zero(sd):
    rng = np.random.default_rng(91)
    q, k, v = _drop_case(rng, 1, 2, 4, 6, 3, 2)
    out = sd.attention_dropout(q, k, v, np.zeros((1, 2, 4, 6), bool), 1.25)
    assert np.all(out == 0.0)


def pin_drop_single_kept_key_closed_form(sd):
    """Two keys with scaled logits x0, x1 and only key 0 kept in row 0: the
    row is c · σ(x0 − x1) · v_0, with σ the logistic function (the softmax of
    two logits); in row 1 only key 1 is kept: c · σ(x1 − x0) · v_1."""
    c = 1.0 / (1.0 - 0.3)
    for s0, s1, scale in ((8.0, 0.0, 1.0 / 8.0), (2.0, -1.0, 0.5), (0.0, 0.0, 1.0)):
        q = np.array([[[[1.0, 0.0], [1.0, 0.0]]]])
        k = np.array([[[[s0, 0.0], [s1, 1.0]]]])
        v = np.array([[[[1.5, -2.0, 0.25], [-3.0, 0.5, 4.0]]]])
        keep = np.array([[[[True, False], [False, True]]]])
        out = sd.attention_dropout(q, k, v, keep, c, scale=scale)[0, 0]
        x = scale * (s0 - s1)
        sig = 1.0 / (1.0 + math.exp(-x))
        assert np.allclose(out[0], c * sig * v[0, 0, 0], rtol=1e-14, atol=1e-15)
        assert np.allclose(out[1], c * (1.0 - sig) * v[0, 0, 1], rtol=1e-14, atol=1e-15)


def pin_drop_expectation_over_masks(sd):
    """Averaging the output over every mask of a tiny head, each weighted by
    its probability (keep with 1 − p, independently), gives Eq. (1) without
    dropout: E[Z] = 1 − p and c = 1/(1 − p)."""
    import itertools

    import oracle.sdpa_oracle as so

    rng = np.random.default_rng(92)
    n, m, p = 2, 3, 0.3
    q, k, v = _drop_case(rng, 1, 1, n, m, 3, 2)
    for kw in (dict(), dict(key_lens=[2]), dict(window=(0, 1, "top_left"))):
        mean = np.zeros((1, 1, n, 2))
        for bits in itertools.product((0, 1), repeat=n * m):
            keep = np.array(bits, bool).reshape(1, 1, n, m)
            pr = (1 - p) ** keep.sum() * p ** (n * m - keep.sum())
            mean += pr * sd.attention_dropout(q, k, v, keep, 1.0 / (1.0 - p), **kw)
        assert np.allclose(mean, so.attention(q, k, v, **kw), rtol=0, atol=1e-13), kw


def pin_drop_disjoint_masks_add(sd):
    """The output is linear in Z: masks with no kept weight in common add."""
    rng = np.random.default_rng(93)
    q, k, v = _drop_case(rng, 2, 2, 6, 9, 4, 4)
    u = rng.random((2, 2, 6, 9))
    z1, z2 = u < 0.3, (u >= 0.3) & (u < 0.75)
    c = 1.7
    a = sd.attention_dropout(q, k, v, z1, c, causal=False, key_lens=[9, 4])
    b = sd.attention_dropout(q, k, v, z2, c, causal=False, key_lens=[9, 4])
    both = sd.attention_dropout(q, k, v, z1 | z2, c, causal=False, key_lens=[9, 4])
    assert np.allclose(a + b, both, rtol=0, atol=1e-13)


def pin_drop_brute_force_mp(sd):
    """50-digit scalar loops (``oracle.brute_mp.attention_mp`` with a mask):
    the legal keys fill the denominator, the kept ones the sum."""
    from oracle.brute_mp import attention_mp

    rng = np.random.default_rng(94)
    for (B, h, n, m, d, dv) in ((2, 2, 4, 4, 3, 2), (1, 2, 3, 5, 2, 3)):
        q, k, v = _drop_case(rng, B, h, n, m, d, dv)
        keep = rng.random((B, h, n, m)) < 0.6
        for causal, kl, win in ((False, None, None), (n == m, [m, 1][:B], None),
                                (False, [m, 2][:B], (1, 1, "top_left")), (False, None, (None, 0, "bottom_right"))):
            ref = np.array(attention_mp(q.tolist(), k.tolist(), v.tolist(), 0.6, causal, kl, window=win,
                                        keep=keep.tolist(), keep_scale=1.25), dtype=np.float64)
            got = sd.attention_dropout(q, k, v, keep, 1.25, scale=0.6, causal=causal, key_lens=kl, window=win)
            assert np.allclose(got, ref, rtol=0, atol=1e-14), (causal, kl, win)


def pin_drop_bwd_finite_difference_mp(sd):
    """Gradients against 60-digit central differences of the forward with the
    same mask (``attention_grad_fd_mp`` with ``keep``)."""
    from oracle.brute_mp import attention_grad_fd_mp

    rng = np.random.default_rng(95)
    for (n, m) in ((3, 3), (2, 4)):
        q, k, v = _drop_case(rng, 2, 1, n, m, 3, 2)
        do = rng.standard_normal((2, 1, n, 2))
        keep = rng.random((2, 1, n, m)) < 0.5
        for causal, kl, win in ((False, None, None), (n == m, [m, 1], None), (False, [m, 2], (1, 0, "top_left"))):
            fd = attention_grad_fd_mp(q.tolist(), k.tolist(), v.tolist(), do.tolist(), 0.7, causal, kl, win,
                                      keep=keep.tolist(), keep_scale=1.6)
            got = sd.attention_dropout_backward(q, k, v, do, keep, 1.6, scale=0.7, causal=causal, key_lens=kl,
                                                window=win)
            for g, f in zip(got, fd):
                assert np.allclose(g, np.array(f), rtol=0, atol=1e-12), (n, m, causal, kl, win)


def pin_drop_bwd_all_kept_is_plain(sd):
    import oracle.sdpa_backward as sb

    rng = np.random.default_rng(96)
    q, k, v = _drop_case(rng, 2, 1, 5, 6, 3, 4)
    do = rng.standard_normal((2, 1, 5, 4))
    keep = np.ones((2, 1, 5, 6), bool)
    for a, b in zip(sd.attention_dropout_backward(q, k, v, do, keep, 1.0, key_lens=[6, 3]),
                    sb.attention_backward(q, k, v, do, key_lens=[6, 3])):
        assert np.array_equal(a, b)


DROPOUT_PINS = [
    pin_drop_unpack_bit_order,
    pin_drop_all_kept_is_plain,
    pin_drop_all_dropped_is_zero,
    pin_drop_single_kept_key_closed_form,
    pin_drop_expectation_over_masks,
    pin_drop_disjoint_masks_add,
    pin_drop_brute_force_mp,
    pin_drop_bwd_finite_difference_mp,
    pin_drop_bwd_all_kept_is_plain,
]
