"""Plain fp64 CPU oracle for attention with dropout on the attention weights.

TEST INFRASTRUCTURE ONLY, like ``oracle.sdpa_oracle``: only the test suite,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU legs may use it, and the
HIP library never does.

What it computes
----------------
The pages train with dropout (《Attention Is All You Need：注意力就是你所需要的
一切》 §5.4 and the dropout paper it cites as [33]), and name attention
dropout among the settings tuned for parsing (same page, §6.3; 《精读 Attention
Is All You Need：原始 Transformer 论文》, its notes on the parsing experiment),
without saying where inside the attention it acts.  The reading taken here:
dropout acts on the attention weights after the softmax of Eq. (1), each
weight kept or zeroed on its own, and the kept ones scaled so that the
expected output is the output without dropout:

    P = row-wise softmax(S),  S = scale · Q Kᵀ with illegal logits −∞
    O = (P ∘ Z) V · c,         Z ∈ {0, 1}^{n×m}, c = 1 / (1 − p)

with Z drawn with Pr(Z_ij = 1) = 1 − p.  The softmax itself is unchanged
(its normaliser counts every legal key, kept or not).  The draw is an input
here (``keep``, a boolean [B, h, n, m]) and to the GPU path (a bit mask), so
both sides use the same Z.  Bits of illegal connections are irrelevant: those
weights are already exactly zero.

Gradient (same chain rule as ``oracle.sdpa_backward``, with P̃ = P ∘ Z · c):

    dV = P̃ᵀ dO,  dP̃ = dO Vᵀ,  dP = dP̃ ∘ Z · c,
    dS = P ∘ (dP − rowsum(P ∘ dP)),  dQ = scale · dS K,  dK = scale · dSᵀ Q

and rowsum(P ∘ dP) = dO_i · O_i as without dropout.

Pins (``tests/oracle_pins.py``): an all-kept mask with c = 1 is the oracle
without dropout; an all-dropped mask gives zeros; one kept key gives
c · p_ij · v_j in closed form; the average over every mask of a tiny head,
weighted by its probability, is the output without dropout; outputs add over
disjoint masks; a 50-digit brute force with the mask; and central finite
differences of this forward for the gradient.
"""

from __future__ import annotations

import numpy as np

from oracle import sdpa_backward as bwd
from oracle import sdpa_oracle as fwd

__all__ = ["attention_dropout", "attention_dropout_backward", "unpack_keep"]


def unpack_keep(words: np.ndarray, m: int) -> np.ndarray:
    """The bit mask of the GPU path as booleans: bit j mod 32 of word ⌊j/32⌋
    of a row is key j.  words: uint32 [..., ⌈m/32⌉] → bool [..., m]."""
    words = np.asarray(words, dtype=np.uint32)
    j = np.arange(m)
    return ((words[..., j // 32] >> (j % 32).astype(np.uint32)) & 1).astype(bool)


def dropped_weights(p: np.ndarray, keep: np.ndarray, keep_scale: float) -> np.ndarray:
    """P̃ = P ∘ Z · c: the weights that multiply the values."""
    return p * keep * keep_scale


def grad_through_dropout(dpt: np.ndarray, keep: np.ndarray, keep_scale: float) -> np.ndarray:
    """dP = dP̃ ∘ Z · c: the gradient of the softmax output from that of P̃."""
    return dpt * keep * keep_scale


def _weights(q, k, scale, vis):
    return fwd.row_softmax(fwd.apply_mask(fwd.scores(q, k, scale), vis))


def _vis(n, m, causal, key_len, window):
    pos = np.arange(n)
    if window is None:
        return fwd.visible_keys(pos, m, causal, key_len)
    return fwd.visible_keys(pos, m, causal, key_len, window=window)


def attention_dropout_head(q, k, v, keep, keep_scale: float, scale: float, causal=False, key_len=None,
                           window=None):
    """O for one head: q [n, d_k], k [m, d_k], v [m, d_v], keep bool [n, m]."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    p = _weights(q, k, scale, _vis(q.shape[0], k.shape[0], causal, key_len, window))
    return fwd.weighted_values(dropped_weights(p, np.asarray(keep, bool), keep_scale), v)


def attention_dropout(q, k, v, keep, keep_scale: float, scale=None, causal: bool = False, key_lens=None,
                      window=None) -> np.ndarray:
    """O over every (batch, head) pair of [B, h, len, d] arrays; keep is bool
    [B, h, n, m].  Other arguments as in ``oracle.sdpa_oracle.attention``."""
    if window is not None and causal:
        raise ValueError("give the causal mask as the window (None, 0) instead")
    B, h, n, m, d_k, d_v = fwd._check_shapes(q, k, v, causal)
    if np.shape(keep) != (B, h, n, m):
        raise ValueError("keep must be [B, h, n, m]")
    scale = fwd.default_scale(d_k) if scale is None else scale
    out = np.empty((B, h, n, d_v))
    for b in range(B):
        L = None if key_lens is None else int(key_lens[b])
        win = fwd._window_of(window, n, m, L)
        for hh in range(h):
            out[b, hh] = attention_dropout_head(q[b, hh], k[b, hh], v[b, hh], keep[b, hh], keep_scale, scale,
                                                causal, L, win)
    return out


def attention_dropout_head_backward(q, k, v, do, keep, keep_scale: float, scale: float, causal=False,
                                    key_len=None, window=None):
    """(dq, dk, dv) of one head, fp64."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    keep = np.asarray(keep, bool)
    p = _weights(q, k, scale, _vis(q.shape[0], k.shape[0], causal, key_len, window))
    pt = dropped_weights(p, keep, keep_scale)
    dv = bwd.grad_values(pt, do)
    dp = grad_through_dropout(bwd.grad_weights(do, v), keep, keep_scale)
    ds = bwd.grad_logits(p, dp)
    return bwd.grad_queries(ds, k, scale), bwd.grad_keys(ds, q, scale), dv


def attention_dropout_backward(q, k, v, do, keep, keep_scale: float, scale=None, causal: bool = False,
                               key_lens=None, window=None):
    """(dq, dk, dv) over every (batch, head) pair; arguments as in
    ``attention_dropout`` plus the upstream gradient do [B, h, n, d_v]."""
    B, h, n, m, d_k, d_v, scale = bwd._prep(q, k, v, do, scale, causal, window)
    dq, dk, dv = np.empty((B, h, n, d_k)), np.empty((B, h, m, d_k)), np.empty((B, h, m, d_v))
    for b in range(B):
        L = None if key_lens is None else int(key_lens[b])
        win = fwd._window_of(window, n, m, L)
        for hh in range(h):
            dq[b, hh], dk[b, hh], dv[b, hh] = attention_dropout_head_backward(
                q[b, hh], k[b, hh], v[b, hh], do[b, hh], keep[b, hh], keep_scale, scale, causal, L, win)
    return dq, dk, dv
