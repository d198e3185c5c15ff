"""Plant one plausible mistake in the oracle at a time; some pin must catch it.

The mistakes are planted in the CPU oracle only (never in the GPU path), by
replacing one step function of ``oracle.sdpa_oracle`` for the duration of a
test.  Each mutant below is a mistake a careful reader could make when writing
Eq. (1) out: a dropped or wrong scale, a transposed operand, a strict instead
of inclusive causal mask, an off-by-one or misplaced key-padding mask, a finite
stand-in for −∞, a softmax over the wrong axis or without its normaliser, or a
key length taken from the wrong index.
"""

import numpy as np
import pytest

import oracle.sdpa_oracle as so
from tests.oracle_pins import ALL_PINS

_orig_visible = so.visible_keys


def _vis_strict_causal(query_pos, m, causal, key_len):
    vis = _orig_visible(query_pos, m, False, key_len)
    if causal:
        vis &= np.arange(m)[None, :] < np.asarray(query_pos)[:, None]
    return vis


def _vis_pad_off_by_one(query_pos, m, causal, key_len):
    return _orig_visible(query_pos, m, causal, None if key_len is None else key_len + 1)


def _vis_ignore_padding(query_pos, m, causal, key_len):
    return _orig_visible(query_pos, m, causal, None)


def _vis_pad_on_queries(query_pos, m, causal, key_len):
    vis = _orig_visible(query_pos, m, causal, None)
    if key_len is not None:
        vis &= (np.asarray(query_pos) < key_len)[:, None]
    return vis


def _vis_window_left_off_by_one(query_pos, m, causal, key_len, window=None):
    if window is not None and window[0] is not None:
        window = (window[0] - 1 if window[0] > 0 else 0, window[1], window[2])
    return _orig_visible(query_pos, m, causal, key_len, window=window) if window is not None \
        else _orig_visible(query_pos, m, causal, key_len)


def _vis_window_sides_swapped(query_pos, m, causal, key_len, window=None):
    if window is not None:
        window = (window[1], window[0], window[2])
    return _orig_visible(query_pos, m, causal, key_len, window=window) if window is not None \
        else _orig_visible(query_pos, m, causal, key_len)


def _vis_window_alignment_ignored(query_pos, m, causal, key_len, window=None):
    if window is not None:
        window = (window[0], window[1], 0)
    return _orig_visible(query_pos, m, causal, key_len, window=window) if window is not None \
        else _orig_visible(query_pos, m, causal, key_len)


def _mask_finite(s, vis):
    out = s.copy()
    out[~vis] = -1e9
    return out


def _softmax_cols(s):
    t = np.where(np.isfinite(s), s, -np.inf)
    mx = np.max(np.where(np.isfinite(t), t, -1e300), axis=0, keepdims=True)
    e = np.exp(t - mx)
    den = e.sum(axis=0, keepdims=True)
    return np.divide(e, den, out=np.zeros_like(e), where=den > 0)


def _softmax_unnormalised(s):
    out = np.zeros_like(s)
    for i in range(s.shape[0]):
        if np.isfinite(s[i]).any():
            out[i] = np.exp(s[i] - s[i][np.isfinite(s[i])].max())
    return out


def _softmax_no_max_guard_uniform(s):
    # fully masked rows become uniform instead of zero (a −1e9-style fill)
    w = so_row_softmax_orig(s)
    for i in range(s.shape[0]):
        if not np.isfinite(s[i]).any():
            w[i] = 1.0 / s.shape[1]
    return w


so_row_softmax_orig = so.row_softmax


MUTANTS = {
    "scale_dropped": ("scores", lambda q, k, scale: q @ k.T),
    "scale_squared": ("scores", lambda q, k, scale: scale * scale * (q @ k.T)),
    "scores_transposed": ("scores", lambda q, k, scale: (scale * (q @ k.T)).T),
    "keys_as_queries": ("scores", lambda q, k, scale: scale * (k[: q.shape[0]] @ k.T)),
    "causal_strict": ("visible_keys", _vis_strict_causal),
    "padding_off_by_one": ("visible_keys", _vis_pad_off_by_one),
    "padding_ignored": ("visible_keys", _vis_ignore_padding),
    "padding_on_queries": ("visible_keys", _vis_pad_on_queries),
    "window_left_off_by_one": ("visible_keys", _vis_window_left_off_by_one),
    "window_sides_swapped": ("visible_keys", _vis_window_sides_swapped),
    "window_alignment_ignored": ("visible_keys", _vis_window_alignment_ignored),
    "heads_concatenated_without_transpose": ("concat_heads",
                                             lambda hd: hd.reshape(hd.shape[0], hd.shape[2], -1)),
    "heads_projected_with_transposed_weights": ("project_heads",
                                                lambda x, w: np.einsum("bld,hkd->bhlk", x, w)
                                                if w.shape[1] == w.shape[2] else np.einsum("bld,hdk->bhlk", x, w[::-1])),
    "output_projection_transposed": ("output_projection",
                                     lambda c, wo: c @ wo.T if wo.shape[0] == wo.shape[1] else c @ wo[::-1]),
    "output_projection_dropped": ("output_projection", lambda c, wo: c[..., :wo.shape[1]]),
    "mask_finite_fill": ("apply_mask", _mask_finite),
    "mask_skipped": ("apply_mask", lambda s, vis: s.copy()),
    "softmax_over_columns": ("row_softmax", _softmax_cols),
    "softmax_unnormalised": ("row_softmax", _softmax_unnormalised),
    "masked_row_uniform": ("row_softmax", _softmax_no_max_guard_uniform),
    # only expressible when the weight matrix is square (n == m)
    "weights_transposed": ("weighted_values", lambda w, v: w.T @ v if w.shape[0] == w.shape[1] else w @ v),
    "values_dropped_last": ("weighted_values", lambda w, v: w[:, :-1] @ v[:-1]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(so, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(so)
        except Exception as e:  # an assertion or a shape error both count
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects mutant {name}"


def test_key_length_taken_from_head_index(monkeypatch):
    """A key length looked up by head instead of batch element must be caught."""
    def attention_wrong(q, k, v, scale=None, causal=False, key_lens=None):
        B, h, n, d_k = q.shape
        if scale is None:
            scale = so.default_scale(d_k)
        out = np.empty((B, h, n, v.shape[3]))
        for b in range(B):
            for hh in range(h):
                L = None if key_lens is None else int(key_lens[min(hh, len(key_lens) - 1)])
                out[b, hh] = so.attention_head(q[b, hh], k[b, hh], v[b, hh], scale, causal, L)
        return out

    monkeypatch.setattr(so, "attention", attention_wrong)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(so)
        except Exception:
            caught.append(pin.__name__)
    assert caught


# --- the gradient oracle ------------------------------------------------------
#
# Mistakes one could make deriving the gradient of Eq. (1) by hand: dropping
# the softmax's row term, flipping its sign, summing it over the wrong axis,
# forgetting the scale in dQ or dK, or a missing transpose in dK or dV
# (expressible when n == m).

import oracle.sdpa_backward as sb  # noqa: E402
from tests.oracle_pins import BACKWARD_PINS  # noqa: E402


def _sq(f, g):
    """f where the operands are square (the mistake is expressible), else g."""
    return lambda a, b, *rest: f(a, b, *rest) if a.shape[0] == a.shape[1] else g(a, b, *rest)


BWD_MUTANTS = {
    "softmax_row_term_dropped": ("grad_logits", lambda p, dp: p * dp),
    "softmax_row_term_sign": ("grad_logits", lambda p, dp: p * (np.sum(p * dp, axis=1, keepdims=True) - dp)),
    "softmax_term_over_columns": ("grad_logits", lambda p, dp: p * (dp - np.sum(p * dp, axis=0, keepdims=True))),
    "softmax_term_without_weights": ("grad_logits", lambda p, dp: p * (dp - np.sum(dp, axis=1, keepdims=True))),
    "dq_scale_dropped": ("grad_queries", lambda ds, k, scale: ds @ k),
    "dk_scale_dropped": ("grad_keys", lambda ds, q, scale: ds.T @ q),
    "dk_not_transposed": ("grad_keys", _sq(lambda ds, q, scale: scale * (ds @ q),
                                           lambda ds, q, scale: scale * (ds.T @ q))),
    "dv_not_transposed": ("grad_values", _sq(lambda p, do: p @ do, lambda p, do: p.T @ do)),
    "dp_transposed": ("grad_weights", lambda do, v: (do @ v.T) if do.shape[0] != v.shape[0]
                      else (do @ v.T).T),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_some_backward_pin_catches_mutant(name, monkeypatch):
    attr, fn = BWD_MUTANTS[name]
    monkeypatch.setattr(sb, attr, fn)
    caught = []
    for pin in BACKWARD_PINS:
        try:
            pin(sb)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects mutant {name}"


# --- the single-row helpers ---------------------------------------------------
#
# Mistakes one could make in a helper that evaluates chosen output rows: the
# row evaluated at position 0 instead of its own position, the window's
# bottom-right shift dropped, every batch element given the first one's key
# length, the neighbouring row returned, or (gradients) only the first slice
# of queries added into dK/dV.

_orig_rows = so.attention_rows


def _rows_query_pos_dropped(q, k, v, picks, scale=None, causal=False, key_lens=None, window=None):
    out = []
    for (b, hh, i) in picks:
        q0 = np.array(q, dtype=np.float64, copy=True)
        q0[b, hh, 0] = q[b, hh, i]
        out.append(_orig_rows(q0, k, v, [(b, hh, 0)], scale, causal, key_lens, window)[0])
    return np.array(out)


def _rows_shift_dropped(q, k, v, picks, scale=None, causal=False, key_lens=None, window=None):
    if window is not None:
        window = (window[0], window[1], "top_left")
    return _orig_rows(q, k, v, picks, scale, causal, key_lens, window)


def _rows_first_key_len(q, k, v, picks, scale=None, causal=False, key_lens=None, window=None):
    if key_lens is not None:
        key_lens = np.full(len(key_lens), key_lens[0])
    return _orig_rows(q, k, v, picks, scale, causal, key_lens, window)


def _rows_neighbour(q, k, v, picks, scale=None, causal=False, key_lens=None, window=None):
    n = q.shape[2]
    picks = [(b, hh, min(i + 1, n - 1) if i >= 1 else i) for (b, hh, i) in picks]
    return _orig_rows(q, k, v, picks, scale, causal, key_lens, window)


ROW_MUTANTS = {
    "rows_query_pos_dropped": _rows_query_pos_dropped,
    "rows_window_shift_dropped": _rows_shift_dropped,
    "rows_first_key_len_for_all": _rows_first_key_len,
    "rows_neighbour_returned": _rows_neighbour,
}


@pytest.mark.parametrize("name", sorted(ROW_MUTANTS))
def test_some_pin_catches_row_helper_mutant(name, monkeypatch):
    monkeypatch.setattr(so, "attention_rows", ROW_MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(so)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects mutant {name}"


_orig_qrows = sb.backward_query_rows
_orig_krows = sb.backward_key_rows


def _bwd_qrows_pos_dropped(q, k, v, do, picks, scale=None, causal=False, key_lens=None, window=None):
    out = []
    for (b, hh, i) in picks:
        q0, d0 = np.array(q, np.float64, copy=True), np.array(do, np.float64, copy=True)
        q0[b, hh, 0], d0[b, hh, 0] = q[b, hh, i], do[b, hh, i]
        out.append(_orig_qrows(q0, k, v, d0, [(b, hh, 0)], scale, causal, key_lens, window)[0])
    return np.array(out)


def _bwd_krows_first_slice(q, k, v, do, b, hh, keys, scale=None, causal=False, key_lens=None,
                           window=None):
    d0 = np.array(do, np.float64, copy=True)
    d0[:, :, 512:] = 0.0  # the later query slices contribute nothing
    return _orig_krows(q, k, v, d0, b, hh, keys, scale, causal, key_lens, window)


def _bwd_krows_shift_dropped(q, k, v, do, b, hh, keys, scale=None, causal=False, key_lens=None,
                             window=None):
    if window is not None:
        window = (window[0], window[1], "top_left")
    return _orig_krows(q, k, v, do, b, hh, keys, scale, causal, key_lens, window)


BWD_ROW_MUTANTS = {
    "bwd_query_rows_pos_dropped": ("backward_query_rows", _bwd_qrows_pos_dropped),
    "bwd_key_rows_first_slice_only": ("backward_key_rows", _bwd_krows_first_slice),
    "bwd_key_rows_window_shift_dropped": ("backward_key_rows", _bwd_krows_shift_dropped),
}


@pytest.mark.parametrize("name", sorted(BWD_ROW_MUTANTS))
def test_some_backward_pin_catches_row_helper_mutant(name, monkeypatch):
    attr, fn = BWD_ROW_MUTANTS[name]
    monkeypatch.setattr(sb, attr, fn)
    caught = []
    for pin in BACKWARD_PINS:
        try:
            pin(sb)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects mutant {name}"


# --- attention dropout ---------------------------------------------------------
#
# Mistakes one could make in the dropout step: the rescale 1/(1 − p) left
# out, the mask read transposed or inverted, the kept weights renormalised
# (a softmax over the kept keys only), the gradient passed through the mask
# unmasked or unscaled, or the mask's bits read most significant first.

import oracle.sdpa_dropout as sd  # noqa: E402
from tests.oracle_pins import DROPOUT_PINS  # noqa: E402


def _renormalised(p, keep, c):
    x = p * keep
    s = x.sum(axis=1, keepdims=True)
    return np.divide(x, s, out=np.zeros_like(x), where=s > 0)


def _msb_first(words, m):
    words = np.asarray(words, dtype=np.uint32)
    j = np.arange(m)
    return ((words[..., j // 32] >> (31 - j % 32).astype(np.uint32)) & 1).astype(bool)


DROPOUT_MUTANTS = {
    "keep_scale_dropped": ("dropped_weights", lambda p, keep, c: p * keep),
    "keep_inverted": ("dropped_weights", lambda p, keep, c: p * ~keep * c),
    "keep_transposed": ("dropped_weights", lambda p, keep, c: p * (keep.T if keep.shape[0] == keep.shape[1]
                                                                    else keep) * c),
    "kept_weights_renormalised": ("dropped_weights", _renormalised),
    "grad_not_masked": ("grad_through_dropout", lambda dpt, keep, c: dpt * c),
    "grad_not_scaled": ("grad_through_dropout", lambda dpt, keep, c: dpt * keep),
    "bits_msb_first": ("unpack_keep", _msb_first),
}


@pytest.mark.parametrize("name", sorted(DROPOUT_MUTANTS))
def test_some_dropout_pin_catches_mutant(name, monkeypatch):
    attr, fn = DROPOUT_MUTANTS[name]
    monkeypatch.setattr(sd, attr, fn)
    caught = []
    for pin in DROPOUT_PINS:
        try:
            pin(sd)
        except Exception as e:
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects mutant {name}"
