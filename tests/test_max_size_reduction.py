"""CPU check of the reduction the largest-head gradient tests rely on.

A head whose first R·P keys are one block of P keys repeated R times, followed
by t marker keys, has the gradient of a small head that holds the block once
with every logit raised by ln R (an extra input dimension: q gets ln R / scale,
block keys 1, marker keys 0): dQ is the same, each copy's dK and dV row is the
block row's divided by R, and the marker rows are the same.  Here both sides
come from the fp64 gradient oracle on a head small enough to build explicitly.
"""

import math

import numpy as np

import oracle.sdpa_backward as sb


def test_repeated_keys_reduce_to_a_shifted_small_head():
    rng = np.random.default_rng(11)
    n, d, P, R, t = 5, 8, 6, 7, 3
    scale = 1.0 / math.sqrt(d)
    q = rng.standard_normal((n, d))
    kb, vb = rng.standard_normal((P, d)), rng.standard_normal((P, d))
    do = rng.standard_normal((n, d))
    mv = 3.0
    k = np.concatenate([np.tile(kb, (R, 1)), kb[:t]])
    v = np.concatenate([np.tile(vb, (R, 1)), np.full((t, d), mv)])
    dq, dk, dv = sb.attention_head_backward(q, k, v, do, scale)

    qa = np.concatenate([q, np.full((n, 1), math.log(R) / scale)], axis=1)
    ka = np.concatenate([np.concatenate([kb, np.ones((P, 1))], axis=1),
                         np.concatenate([kb[:t], np.zeros((t, 1))], axis=1)])
    va = np.concatenate([vb, np.full((t, d), mv)])
    rq, rk, rv = sb.attention_head_backward(qa, ka, va, do, scale)

    assert np.allclose(dq, rq[:, :d], rtol=1e-12, atol=1e-12)
    for c in range(R):
        assert np.allclose(dk[c * P:(c + 1) * P], rk[:P, :d] / R, rtol=1e-12, atol=1e-12)
        assert np.allclose(dv[c * P:(c + 1) * P], rv[:P] / R, rtol=1e-12, atol=1e-12)
    assert np.allclose(dk[R * P:], rk[P:, :d], rtol=1e-12, atol=1e-12)
    assert np.allclose(dv[R * P:], rv[P:], rtol=1e-12, atol=1e-12)
