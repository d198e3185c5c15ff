"""Plain fp64 CPU oracle for scaled dot-product attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite (``tests/``), the smoke check
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or run anything under ``oracle/``.  The product path (the package
``transformer_attention_sdpa_amd`` and its HIP library) never imports it and
never falls back to it; the two share no code, constants or helpers.

What it computes
----------------
Eq. (1) of the pages, evaluated exactly as written, one (batch, head) pair at a
time, in float64:

    Attention(Q, K, V) = softmax(Q Kᵀ / √d_k) V

* Page 《精读 Attention Is All You Need：原始 Transformer 论文》, section
  "缩放点积注意力：点积为什么要缩放", Eq. (1): queries packed into Q, keys and
  values into K and V; the weights are a row-wise softmax of the scaled dot
  products and the output is the weighted sum of the values.
* Page 《Attention Is All You Need：注意力就是你所需要的一切》, §3.2 and
  §3.2.1: the weight of each value comes from the compatibility (dot product)
  of the query with the matching key, divided by √d_k, then a softmax.
* Same page, §3.2.3, and the page 《精读 …》 table of the three uses, which
  states that they compute the same thing: encoder self-attention, decoder
  self-attention and encoder–decoder attention run the identical computation; the decoder's
  illegal connections are set to −∞ inside the attention before the softmax,
  so their weights are exactly zero.  Decoder self-attention lets position i
  see every position up to and *including* i.
* Page 《企业官网建设流程全解析》 (its body is a Transformer explainer),
  §2.2: Q is n×d_k (n = number of queries), K is m×d_k and V is m×d_v
  (m = number of key/value pairs).

Readings taken where the pages are silent:
* a key-padding length ``key_lens[b]`` hides keys j ≥ key_lens[b] of every
  head of batch element b (queries are never masked), clamped to [0, m];
* a query row with no visible key returns the zero vector (every masked weight
  is exactly zero, so nothing is summed);
* the causal mask needs n == m (decoder self-attention) and is inclusive;
* restricted self-attention (《精读 …》 Table 1 and the discussion of long
  sequences after it; 《注意力就是你所需要的一切》 §4: each output position
  looks only at a neighbourhood of size r around it) is written as a key window
  [c_i − left, c_i + right] around the query's aligned position c_i, either
  side unbounded when None; a neighbourhood of size r centred on the query is
  left = right = ⌊r/2⌋.  c_i = i with top-left alignment, or i + (L − n) with
  bottom-right alignment, where the n queries are the last n positions of a
  sequence of L keys (a decoder step against its cached keys); L is the key
  length of the batch element (m without padding).  The decoder's causal mask
  is the window (None, 0) with top-left alignment and n == m.

The steps are module-level functions (``scores``, ``visible_keys``,
``apply_mask``, ``row_softmax``, ``weighted_values``) that
``attention_head`` looks up at call time, so the pin tests can plant a
mistake in exactly one step and show that a pin catches it.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "default_scale",
    "visible_keys",
    "scores",
    "apply_mask",
    "row_softmax",
    "weighted_values",
    "attention_head",
    "attention",
    "attention_rows",
    "project_heads",
    "concat_heads",
    "output_projection",
    "multihead",
]

# Rows of one head evaluated together.  Rows are independent in Eq. (1) (each
# query row is normalised on its own), so evaluating them in slices changes no
# arithmetic; it only bounds memory for the 8192×8192 case.
_ROW_SLICE = 512


def default_scale(d_k: int) -> float:
    """1/√d_k, the scale of Eq. (1) (《注意力就是你所需要的一切》 §3.2.1)."""
    return 1.0 / math.sqrt(d_k)


def visible_keys(query_pos: np.ndarray, m: int, causal: bool, key_len: int | None,
                 window=None) -> np.ndarray:
    """Boolean [len(query_pos), m]: True where query i may attend to key j.

    Causal (decoder self-attention, 《注意力就是你所需要的一切》 §3.2.3): key j is
    visible to the query at position i iff j ≤ i (inclusive).  Key padding:
    key j is visible iff j < clamp(key_len, 0, m).  Window (restricted
    attention): ``window = (left, right, shift)`` makes key j visible only if
    c − left ≤ j ≤ c + right, with c = i + shift and a None side unbounded.
    """
    j = np.arange(m)[None, :]
    vis = np.ones((len(query_pos), m), dtype=bool)
    if causal:
        vis &= j <= np.asarray(query_pos)[:, None]
    if key_len is not None:
        L = min(max(int(key_len), 0), m)
        vis &= j < L
    if window is not None:
        left, right, shift = window
        c = np.asarray(query_pos)[:, None] + int(shift)
        if left is not None:
            vis &= j >= c - int(left)
        if right is not None:
            vis &= j <= c + int(right)
    return vis


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """Scaled compatibilities s_ij = scale · q_i · k_j  (Eq. (1), Q Kᵀ/√d_k)."""
    return scale * (q @ k.T)


def apply_mask(s: np.ndarray, vis: np.ndarray) -> np.ndarray:
    """Set every illegal logit to −∞ before the softmax (§3.2.3)."""
    out = s.copy()
    out[~vis] = -np.inf
    return out


def row_softmax(s: np.ndarray) -> np.ndarray:
    """Softmax of each row on its own; a row whose logits are all −∞ (no
    legal key) gives zeros.

    Each row is a distribution over the keys that sums to 1 (each row of the
    worked example in 《精读 …》 is normalised on its own to 100 %).
    Subtracting the row maximum leaves the softmax unchanged and keeps exp()
    finite.
    """
    w = np.zeros_like(s)
    for i in range(s.shape[0]):
        row = s[i]
        if np.all(row == -np.inf):
            continue  # fully masked row: every weight is exactly zero
        mu = row.max()  # a NaN logit makes mu, and so the whole row, NaN
        e = np.exp(row - mu)  # exp(−∞) == 0.0 exactly
        w[i] = e / e.sum()
    return w


def weighted_values(w: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Output rows o_i = Σ_j w_ij v_j (the weighted sum of the values)."""
    return w @ v


def attention_head(q, k, v, scale: float, causal: bool = False, key_len=None, query_pos=None,
                   window=None):
    """Eq. (1) for one head.  q: [n', d_k], k: [m, d_k], v: [m, d_v] → [n', d_v].

    ``query_pos`` gives the sequence positions of the rows of q (default
    0..n'-1); only the causal mask and the window use it.  ``window`` is
    (left, right, shift) as in ``visible_keys``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if query_pos is None:
        query_pos = np.arange(q.shape[0])
    query_pos = np.asarray(query_pos)
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for r0 in range(0, q.shape[0], _ROW_SLICE):
        r1 = min(r0 + _ROW_SLICE, q.shape[0])
        s = scores(q[r0:r1], k, scale)
        if window is None:
            vis = visible_keys(query_pos[r0:r1], k.shape[0], causal, key_len)
        else:
            vis = visible_keys(query_pos[r0:r1], k.shape[0], causal, key_len, window=window)
        w = row_softmax(apply_mask(s, vis))
        out[r0:r1] = weighted_values(w, v)
    return out


def _window_of(window, n, m, key_len):
    """(left, right, shift) of one batch element from the user's window.

    ``window`` is None or (left, right) or (left, right, align) with align
    'top_left' (default) or 'bottom_right'."""
    if window is None:
        return None
    left, right = window[0], window[1]
    align = window[2] if len(window) > 2 else "top_left"
    for side in (left, right):
        if side is not None and int(side) < 0:
            raise ValueError("window sides are >= 0 or None (unbounded)")
    if align == "top_left":
        shift = 0
    elif align == "bottom_right":
        L = m if key_len is None else min(max(int(key_len), 0), m)
        shift = L - n
    else:
        raise ValueError(f"unknown alignment {align!r}")
    return (left, right, shift)


def _check_shapes(q, k, v, causal):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, h, len, d]")
    B, h, n, d_k = q.shape
    if k.shape[:2] != (B, h) or v.shape[:2] != (B, h):
        raise ValueError("batch/head dims differ")
    if k.shape[3] != d_k or k.shape[2] != v.shape[2]:
        raise ValueError("k must be [B,h,m,d_k] and v [B,h,m,d_v]")
    if causal and n != k.shape[2]:
        raise ValueError("the causal mask is defined for self-attention only (n == m)")
    return B, h, n, k.shape[2], d_k, v.shape[3]


def attention(q, k, v, scale=None, causal: bool = False, key_lens=None, window=None) -> np.ndarray:
    """Eq. (1) over every (batch, head) pair of [B, h, len, d] arrays, fp64.

    The heads are independent (《精读 …》 multi-head section: attention runs in
    parallel on each set of projections), so they are simply looped over.
    ``window``: None, or (left, right[, align]) for restricted attention (see
    the module notes); it is not combined with ``causal``.
    """
    if window is not None and causal:
        raise ValueError("give the causal mask as the window (None, 0) instead")
    B, h, n, m, d_k, d_v = _check_shapes(q, k, v, causal)
    if scale is None:
        scale = default_scale(d_k)
    out = np.empty((B, h, n, d_v), dtype=np.float64)
    for b in range(B):
        L = None if key_lens is None else int(key_lens[b])
        win = _window_of(window, n, m, L)
        for hh in range(h):
            if win is None:
                out[b, hh] = attention_head(q[b, hh], k[b, hh], v[b, hh], scale, causal, L)
            else:
                out[b, hh] = attention_head(q[b, hh], k[b, hh], v[b, hh], scale, causal, L,
                                            window=win)
    return out


def attention_rows(q, k, v, picks, scale=None, causal: bool = False, key_lens=None,
                   window=None):
    """Eq. (1) for selected output rows only: ``picks`` is a list of (b, head, i).

    Returns an array [len(picks), d_v].  Used to check full-size outputs row by
    row where evaluating every row would take too long.
    """
    if window is not None and causal:
        raise ValueError("give the causal mask as the window (None, 0) instead")
    B, h, n, m, d_k, d_v = _check_shapes(q, k, v, causal)
    if scale is None:
        scale = default_scale(d_k)
    out = np.empty((len(picks), d_v), dtype=np.float64)
    for r, (b, hh, i) in enumerate(picks):
        L = None if key_lens is None else int(key_lens[b])
        win = _window_of(window, n, m, L)
        if win is None:
            out[r] = attention_head(q[b, hh, i:i + 1], k[b, hh], v[b, hh], scale, causal, L,
                                    query_pos=np.array([i]))[0]
        else:
            out[r] = attention_head(q[b, hh, i:i + 1], k[b, hh], v[b, hh], scale, causal, L,
                                    query_pos=np.array([i]), window=win)[0]
    return out


def project_heads(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Per-head projections x W_i: x [B, len, d_model], w [h, d_model, d] →
    [B, h, len, d] (《精读 …》 multi-head section, head_i's inputs)."""
    return np.einsum("bld,hdk->bhlk", x, w)


def concat_heads(heads: np.ndarray) -> np.ndarray:
    """Concat(head_1, …, head_h): [B, h, n, d_v] → [B, n, h·d_v], head i in
    columns i·d_v … (i+1)·d_v − 1 of each row."""
    B, h, n, d_v = heads.shape
    return heads.transpose(0, 2, 1, 3).reshape(B, n, h * d_v)


def output_projection(concat: np.ndarray, wo: np.ndarray) -> np.ndarray:
    """Concat(…) W^O: [B, n, h·d_v] · [h·d_v, d_model] → [B, n, d_model]."""
    return concat @ wo


def multihead(xq, xkv, wq, wk, wv, wo, scale=None, causal: bool = False, key_lens=None,
              window=None) -> np.ndarray:
    """The multi-head attention sublayer, fp64 (《精读 …》 multi-head section;
    《注意力就是你所需要的一切》 §3.2.2):

        MultiHead(Q, K, V) = Concat(head_1, …, head_h) W^O,
        head_i = Attention(Q W_i^Q, K W_i^K, V W_i^V),

    with the queries taken from ``xq`` [B, n, d_model] and the keys and values
    from ``xkv`` [B, m, d_model] (the same array for self-attention, the
    encoder output for encoder–decoder attention, §3.2.3).  The projections
    are the pages' parameter matrices, stacked per head: ``wq`` [h, d_model,
    d_k] holds W_i^Q, ``wk`` [h, d_model, d_k], ``wv`` [h, d_model, d_v], and
    ``wo`` [h·d_v, d_model] is W^O.  The pages' projections carry no bias.
    Masking and scale follow ``attention``.  Returns [B, n, d_model].
    """
    xq = np.asarray(xq, dtype=np.float64)
    xkv = np.asarray(xkv, dtype=np.float64)
    wq, wk, wv, wo = (np.asarray(w, dtype=np.float64) for w in (wq, wk, wv, wo))
    h, d_model, d_k = wq.shape
    d_v = wv.shape[2]
    if xq.ndim != 3 or xkv.ndim != 3 or xq.shape[0] != xkv.shape[0]:
        raise ValueError("xq must be [B, n, d_model] and xkv [B, m, d_model]")
    if xq.shape[2] != d_model or xkv.shape[2] != d_model:
        raise ValueError("model width differs between inputs and projections")
    if wk.shape != (h, d_model, d_k) or wv.shape[:2] != (h, d_model) or wo.shape != (h * d_v, d_model):
        raise ValueError("projection shapes do not match")
    # The steps are looked up at call time (see the module notes).
    mod = globals()
    q = mod["project_heads"](xq, wq)
    k = mod["project_heads"](xkv, wk)
    v = mod["project_heads"](xkv, wv)
    heads = mod["attention"](q, k, v, scale=scale, causal=causal, key_lens=key_lens, window=window)
    return mod["output_projection"](mod["concat_heads"](heads), wo)
