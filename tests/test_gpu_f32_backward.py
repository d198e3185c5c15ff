"""The fp32 gradient of Eq. (1) on the GPU against the fp64 gradient oracle.

The pages train the Transformer in single precision and print only the
forward pass (Eq. (1) of 《精读 Attention Is All You Need：原始 Transformer
论文》); ``oracle.sdpa_backward`` derives dQ, dK, dV by the chain rule and is
pinned by finite differences.  The GPU path: ``sdpa_forward_lse`` (fp32
output and per-row log-sum-exp), then ``sdpa_backward`` with dtype fp32.  Both
sides see the same fp32 values of Q, K, V and dO, all N(0, 1).

Bar: |got − ref| ≤ 2^-16 · (max|ref| + 1) per gradient tensor, about 1300×
tighter than the bf16 gradient bar.  Every weight is recomputed from the fp32
log-sum-exp, whose own error (≤ 10^-6 on these inputs) becomes a relative error
of each weight; the 64-term fp32 dot products (S, dP, D) and the fp32
accumulation of up to m terms in each gradient element add a few units of
2^-24 relative each (measured: ≤ 10^-6 of max|ref|).  The 2^-16 floor covers an
exactly-zero reference (a single legal key gives dQ = dK = 0), where the
device's dP − D cancels two fp32 dot products of 64 terms summed in different
orders, ≈ 64 · 2^-24 · |dO| |v| (measured 1.1·10^-6).  The measured errors are
printed.
"""

import numpy as np
import pytest

import oracle.sdpa_backward as sb
from sdpa_inputs import backward_case
from tests.gpu_cases import from_device, max_abs_err, to_device

pytestmark = pytest.mark.gpu

GRAD_REL = 2.0 ** -16
GRAD_ABS = 2.0 ** -16


def grad_bound(ref):
    return GRAD_REL * float(np.abs(ref).max()) + GRAD_ABS


def run_bwd(c):
    import torch

    from transformer_attention_sdpa_amd import backward, forward

    q, k, v, do = (to_device(c[x], "f32") for x in ("q", "k", "v", "do"))
    kl = None if c["key_lens"] is None else torch.from_numpy(np.asarray(c["key_lens"], np.int32)).cuda()
    kw = dict(causal=c["causal"], key_lens=kl, window=c["window"])
    out, lse = forward(q, k, v, return_lse=True, **kw)
    dq, dk, dv = backward(q, k, v, out, do, lse, **kw)
    torch.cuda.synchronize()
    assert dq.dtype == torch.float32 and dk.dtype == torch.float32 and dv.dtype == torch.float32
    return dq, dk, dv


def check(name, got, ref):
    msgs = []
    for g, r, what in zip(got, ref, ("dq", "dk", "dv")):
        mx, err = float(np.abs(r).max()), max_abs_err(g, r)
        msgs.append(f"{what} {err:.2e}/{mx:.2e}")
        assert np.all(np.isfinite(g)), (name, what)
        assert err <= grad_bound(r), (name, what, err, mx)
    print(f"f32 bwd {name}: " + ", ".join(msgs) + " (max abs err / max |ref|)")


CASES = [  # id, (B, h, n, m), options
    ("encoder_padded", (4, 2, 64, 64), dict(key_lens=[64, 8, 33, 50])),
    ("decoder_causal", (4, 2, 64, 64), dict(causal=True, key_lens=[64, 40, 17, 64])),
    ("cross_n_ne_m", (3, 2, 48, 64), dict(key_lens=[64, 16, 61])),
    ("ragged_tiles", (2, 2, 100, 130), dict(key_lens=[97, 130])),
    ("multi_tile_causal", (2, 2, 300, 300), dict(causal=True, key_lens=[260, 300])),
    ("window", (2, 2, 300, 300), dict(window=(40, 8), key_lens=[300, 211])),
    ("window_right_only", (1, 2, 200, 200), dict(window=(None, 30))),
    ("bottom_right_decode", (2, 2, 5, 200), dict(window=(None, 0, "bottom_right"), key_lens=[150, 3])),
    ("bottom_right_chunk", (2, 1, 70, 190), dict(window=(None, 0, "bottom_right"))),
    ("empty_batch_element", (2, 1, 64, 64), dict(key_lens=[0, 64])),
    ("single_query_key", (3, 1, 1, 1), {}),
    ("one_query_many_keys", (2, 3, 1, 333), dict(key_lens=[333, 5])),
]


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_f32_backward_parity(gpu_lib, i):
    name, (B, h, n, m), opts = CASES[i]
    c = backward_case(9800 + i, B, h, n, m, dtype="f32", **opts)
    got = tuple(from_device(t) for t in run_bwd(c))
    ref = sb.attention_backward(c["q"], c["k"], c["v"], c["do"], causal=c["causal"], key_lens=c["key_lens"],
                                window=c["window"])
    check(name, got, ref)
    if c["key_lens"] is not None:  # keys past each length get exactly zero gradient
        for b, L in enumerate(c["key_lens"]):
            assert np.all(got[1][b, :, L:] == 0.0) and np.all(got[2][b, :, L:] == 0.0)


def test_f32_backward_long_causal_sampled(gpu_lib):
    """1100 × 1100 causal heads (several query and key blocks, a ragged
    tail): dQ rows on both sides of every 64-row block edge of two heads, and
    the dK/dV rows of every key-block edge of one head."""
    B, h, n = 2, 4, 1100
    c = backward_case(9900, B, h, n, n, causal=True, dtype="f32")
    dq, dk, dv = (from_device(t) for t in run_bwd(c))
    picks = [(b, hh, q) for b, hh in ((0, 0), (B - 1, h - 1)) for e in range(64, n, 64) for q in (e - 1, e)]
    picks += [(0, 1, 0), (1, 2, n - 1)]
    ref_q = sb.backward_query_rows(c["q"], c["k"], c["v"], c["do"], picks, causal=True)
    got_q = np.stack([dq[b, hh, q] for b, hh, q in picks])
    keys = sorted({0, n - 1} | {x for e in range(64, n, 64) for x in (e - 1, e)})
    ref_k, ref_v = sb.backward_key_rows(c["q"], c["k"], c["v"], c["do"], 1, 3, keys, causal=True)
    check("long_causal_sampled", (got_q, dk[1, 3, keys], dv[1, 3, keys]), (ref_q, ref_k, ref_v))


def test_f32_backward_large_grid_sampled(gpu_lib):
    """128 heads of 520 (a ragged last block; 1152 blocks of 64 rows, so the
    launches that give each wave its own 32 rows and share tiles between
    waves): dQ rows at every 64-row block edge of two heads and the dK/dV rows
    at every edge of one, with key padding."""
    B, h, n = 4, 32, 520
    kl = [520, 333, 64, 1]
    c = backward_case(9903, B, h, n, n, key_lens=kl, dtype="f32")
    dq, dk, dv = (from_device(t) for t in run_bwd(c))
    picks = [(b, hh, q) for b, hh in ((0, 0), (1, 31)) for e in range(64, n, 64) for q in (e - 1, e)]
    picks += [(2, 5, 0), (3, 7, n - 1)]
    ref_q = sb.backward_query_rows(c["q"], c["k"], c["v"], c["do"], picks, key_lens=kl)
    got_q = np.stack([dq[b, hh, q] for b, hh, q in picks])
    keys = sorted({0, n - 1} | {x for e in range(64, n, 64) for x in (e - 1, e)})
    ref_k, ref_v = sb.backward_key_rows(c["q"], c["k"], c["v"], c["do"], 1, 9, keys, key_lens=kl)
    check("large_grid_sampled", (got_q, dk[1, 9, keys], dv[1, 9, keys]), (ref_q, ref_k, ref_v))


def test_f32_backward_deterministic(gpu_lib):
    """No atomics: two runs agree bit for bit."""
    import torch

    c = backward_case(9901, 2, 2, 300, 300, causal=True, dtype="f32")
    a = run_bwd(c)
    b = run_bwd(c)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))


def test_f32_backward_ignores_rows_past_key_length(gpu_lib):
    """NaN in the K/V rows at or past each key length leaves every gradient
    bitwise unchanged, and those rows' dK/dV are +0."""
    import torch

    c = backward_case(9902, 3, 2, 90, 150, key_lens=[150, 20, 0], dtype="f32")
    a = run_bwd(c)
    for b, L in enumerate(c["key_lens"]):
        c["k"][b, :, L:] = np.nan
        c["v"][b, :, L:] = np.nan
    b2 = run_bwd(c)
    for x, y in zip(a, b2):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    dk = b2[1].cpu().numpy()
    assert np.all(dk[2] == 0.0) and not np.signbit(dk[2]).any()
