"""Plain fp64 CPU oracle for the gradient of scaled dot-product attention.

TEST INFRASTRUCTURE ONLY, like ``oracle.sdpa_oracle``: only the test suite,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU legs may use it, and the
HIP library never does.

What it computes
----------------
The pages print the forward pass only (Eq. (1) on the page 《精读 Attention Is
All You Need：原始 Transformer 论文》, section "缩放点积注意力：点积为什么要缩放";
《Attention Is All You Need：注意力就是你所需要的一切》 §3.2.1), and train the
model with it (same page §5: Adam on the full network), so the gradient of
Eq. (1) is needed but not written down.  It is derived here by the chain rule,
one (batch, head) pair at a time, with the forward steps of
``oracle.sdpa_oracle``:

    S = scale · Q Kᵀ, with illegal logits −∞        (``scores``, ``apply_mask``)
    P = row-wise softmax(S)                           (``row_softmax``)
    O = P V                                           (``weighted_values``)

Given an upstream gradient dO = ∂ℓ/∂O of any scalar ℓ:

    dV = Pᵀ dO                                        (``grad_values``)
    dP = dO Vᵀ                                        (``grad_weights``)
    dS = P ∘ (dP − rowsum(P ∘ dP))                    (``grad_logits``)
    dQ = scale · dS K                                 (``grad_queries``)
    dK = scale · dSᵀ Q                                (``grad_keys``)

The softmax line is the Jacobian of one row's softmax, ∂p_j/∂s_k =
p_j (δ_jk − p_k), applied to that row's dP.  A masked logit has p = 0 and so
dS = 0: masked connections get no gradient, and a row with no legal key (zero
output) passes none back.  rowsum(P ∘ dP) equals dO_i · O_i, which is how the
GPU computes it; here it is taken from its definition.

The log-sum-exp of each row, ln Σ_j exp(s_ij) over the legal keys (−∞ for a
row with none), is what a forward pass keeps for the backward pass: P is then
exp(s_ij − lse_i) without a second normalisation (``log_sum_exp``).

The steps are module-level functions that ``attention_head_backward`` looks up
at call time, so the pin tests can plant a mistake in exactly one of them.

Pins (``tests/oracle_pins.py``): central finite differences of the forward
oracle, the invariants Σ_j dK_j = 0 (shifting every key by one vector leaves
each row's softmax unchanged) and ⟨dQ, Q⟩ = ⟨dK, K⟩ (S is unchanged under
Q → tQ, K → K/t), Σ_j dV_j = Σ_i dO_i over rows with a legal key, closed forms
for a single key and for all-equal scores, and a 50-digit brute force.
"""

from __future__ import annotations

import numpy as np

from oracle import sdpa_oracle as fwd

__all__ = [
    "grad_values",
    "grad_weights",
    "grad_logits",
    "grad_queries",
    "grad_keys",
    "attention_head_backward",
    "attention_backward",
    "log_sum_exp",
    "backward_query_rows",
    "backward_key_rows",
]

_ROW_SLICE = 512


def grad_values(p: np.ndarray, do: np.ndarray) -> np.ndarray:
    """dV = Pᵀ dO: value j collects the output gradients weighted by p_ij."""
    return p.T @ do


def grad_weights(do: np.ndarray, v: np.ndarray) -> np.ndarray:
    """dP = dO Vᵀ: ∂ℓ/∂p_ij = dO_i · v_j, because o_i = Σ_j p_ij v_j."""
    return do @ v.T


def grad_logits(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """dS = P ∘ (dP − rowsum(P ∘ dP)), the softmax Jacobian applied row by row."""
    return p * (dp - np.sum(p * dp, axis=1, keepdims=True))


def grad_queries(ds: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """dQ = scale · dS K, because s_ij = scale · q_i · k_j."""
    return scale * (ds @ k)


def grad_keys(ds: np.ndarray, q: np.ndarray, scale: float) -> np.ndarray:
    """dK = scale · dSᵀ Q."""
    return scale * (ds.T @ q)


def _weights(q, k, scale, vis):
    return fwd.row_softmax(fwd.apply_mask(fwd.scores(q, k, scale), vis))


def _vis(query_pos, m, causal, key_len, window):
    if window is None:
        return fwd.visible_keys(query_pos, m, causal, key_len)
    return fwd.visible_keys(query_pos, m, causal, key_len, window=window)


def attention_head_backward(q, k, v, do, scale: float, causal: bool = False, key_len=None,
                            window=None):
    """Gradients of Eq. (1) for one head: q [n, d_k], k [m, d_k], v [m, d_v],
    do [n, d_v] → (dq [n, d_k], dk [m, d_k], dv [m, d_v]), fp64.

    ``window`` is (left, right, shift) as in ``oracle.sdpa_oracle.visible_keys``.
    Rows are processed in slices; dK and dV sum the slices' contributions.
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    n, m = q.shape[0], k.shape[0]
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    pos = np.arange(n)
    for r0 in range(0, n, _ROW_SLICE):
        r1 = min(r0 + _ROW_SLICE, n)
        p = _weights(q[r0:r1], k, scale, _vis(pos[r0:r1], m, causal, key_len, window))
        dv += grad_values(p, do[r0:r1])
        ds = grad_logits(p, grad_weights(do[r0:r1], v))
        dq[r0:r1] = grad_queries(ds, k, scale)
        dk += grad_keys(ds, q[r0:r1], scale)
    return dq, dk, dv


def _prep(q, k, v, do, scale, causal, window):
    if window is not None and causal:
        raise ValueError("give the causal mask as the window (None, 0) instead")
    B, h, n, m, d_k, d_v = fwd._check_shapes(q, k, v, causal)
    if do.shape != (B, h, n, d_v):
        raise ValueError("do must have the output's shape [B, h, n, d_v]")
    return B, h, n, m, d_k, d_v, fwd.default_scale(d_k) if scale is None else scale


def attention_backward(q, k, v, do, scale=None, causal: bool = False, key_lens=None,
                       window=None):
    """(dq, dk, dv) over every (batch, head) pair of [B, h, len, d] arrays, fp64.

    Arguments as in ``oracle.sdpa_oracle.attention``; ``do`` is [B, h, n, d_v].
    """
    B, h, n, m, d_k, d_v, scale = _prep(q, k, v, do, scale, causal, window)
    dq = np.empty((B, h, n, d_k))
    dk = np.empty((B, h, m, d_k))
    dv = np.empty((B, h, m, d_v))
    for b in range(B):
        L = None if key_lens is None else int(key_lens[b])
        win = fwd._window_of(window, n, m, L)
        for hh in range(h):
            dq[b, hh], dk[b, hh], dv[b, hh] = attention_head_backward(
                q[b, hh], k[b, hh], v[b, hh], do[b, hh], scale, causal, L, win)
    return dq, dk, dv


def log_sum_exp(q, k, scale=None, causal: bool = False, key_lens=None, window=None):
    """lse[b, h, i] = ln Σ_j exp(s_ij) over the legal keys j of row i; −∞ for a
    row with no legal key.  Shifted by the row maximum, like the softmax."""
    v = np.zeros(k.shape[:3] + (1,))
    B, h, n, m, d_k, _, scale = _prep(q, k, v, np.zeros(q.shape[:3] + (1,)), scale, causal, window)
    out = np.empty((B, h, n))
    pos = np.arange(n)
    for b in range(B):
        L = None if key_lens is None else int(key_lens[b])
        win = fwd._window_of(window, n, m, L)
        for hh in range(h):
            for r0 in range(0, n, _ROW_SLICE):
                r1 = min(r0 + _ROW_SLICE, n)
                s = fwd.apply_mask(fwd.scores(np.asarray(q[b, hh, r0:r1], np.float64),
                                              np.asarray(k[b, hh], np.float64), scale),
                                   _vis(pos[r0:r1], m, causal, L, win))
                mu = s.max(axis=1, keepdims=True)
                empty = np.all(s == -np.inf, axis=1)
                mu[empty] = 0.0
                with np.errstate(divide="ignore"):
                    out[b, hh, r0:r1] = (mu[:, 0] + np.log(np.exp(s - mu).sum(axis=1)))
    return out


def backward_query_rows(q, k, v, do, picks, scale=None, causal: bool = False, key_lens=None,
                        window=None):
    """dQ for selected rows only: ``picks`` is a list of (b, head, i) → [len, d_k].

    Row i of dQ needs only row i of P and dP (dS's row term is that row's own
    sum), so each pick costs one row of the head."""
    B, h, n, m, d_k, d_v, scale = _prep(q, k, v, do, scale, causal, window)
    out = np.empty((len(picks), d_k))
    for r, (b, hh, i) in enumerate(picks):
        L = None if key_lens is None else int(key_lens[b])
        win = fwd._window_of(window, n, m, L)
        kk = np.asarray(k[b, hh], np.float64)
        p = _weights(np.asarray(q[b, hh, i:i + 1], np.float64), kk, scale,
                     _vis(np.array([i]), m, causal, L, win))
        ds = grad_logits(p, grad_weights(np.asarray(do[b, hh, i:i + 1], np.float64),
                                         np.asarray(v[b, hh], np.float64)))
        out[r] = grad_queries(ds, kk, scale)[0]
    return out


def backward_key_rows(q, k, v, do, b, hh, keys, scale=None, causal: bool = False,
                      key_lens=None, window=None):
    """dK and dV rows ``keys`` of head (b, hh) → (dk [len, d_k], dv [len, d_v]).

    Column j of P and dS needs every query row (each row's softmax and its
    rowsum term), so this evaluates the whole head in row slices but keeps
    only the requested columns."""
    B, h, n, m, d_k, d_v, scale = _prep(q, k, v, do, scale, causal, window)
    L = None if key_lens is None else int(key_lens[b])
    win = fwd._window_of(window, n, m, L)
    qq, kk, vv, dd = (np.asarray(x[b, hh], np.float64) for x in (q, k, v, do))
    keys = np.asarray(keys)
    dk = np.zeros((len(keys), d_k))
    dv = np.zeros((len(keys), d_v))
    pos = np.arange(n)
    for r0 in range(0, n, _ROW_SLICE):
        r1 = min(r0 + _ROW_SLICE, n)
        p = _weights(qq[r0:r1], kk, scale, _vis(pos[r0:r1], m, causal, L, win))
        ds = grad_logits(p, grad_weights(dd[r0:r1], vv))
        dv += grad_values(p[:, keys], dd[r0:r1])
        dk += grad_keys(ds[:, keys], qq[r0:r1], scale)
    return dk, dv
