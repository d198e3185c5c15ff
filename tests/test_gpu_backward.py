"""The gradient of Eq. (1) on the GPU against the fp64 gradient oracle.

The pages print only the forward pass (Eq. (1) of 《精读 Attention Is All You
Need：原始 Transformer 论文》); ``oracle.sdpa_backward`` derives dQ, dK, dV by
the chain rule and is pinned by finite differences.  The GPU path runs through
the C ABI: ``sdpa_forward_lse`` (forward output and per-row log-sum-exp), then
``sdpa_backward``.  Both sides see the same bf16 values of Q, K, V and dO.

Bar: the bf16 bar of the forward pass (2e-2), taken relative to the largest
magnitude of each gradient tensor, |got − ref| ≤ 2e-2 · max|ref| + 2^-16.  Each
gradient element is a sum of products in which P or dS was rounded to bf16
(≤ 2^-9 relative) and the result is rounded once more, and D_i = dO_i · O_i
uses the bf16 forward output; the measured errors are printed.  The 2^-16
floor covers an exactly-zero reference (a single legal key gives dQ = 0),
where the device's dP − D cancels two fp32 dot products of 64 terms summed
in different orders (≈ 64 · 2^-24 · |dO| |v|).  The
log-sum-exp is compared absolutely within 2^-8: the long kernel sums its
bf16-rounded weights, each within 2^-9 of its fp32 value, and ln turns a
relative error of the sum into an absolute one.
"""

import numpy as np
import pytest

import oracle.sdpa_backward as sb
from sdpa_inputs import backward_case
from tests.gpu_cases import from_device, max_abs_err, to_device

pytestmark = pytest.mark.gpu

GRAD_REL = 2e-2
GRAD_ABS = 2.0 ** -16


def grad_bound(ref):
    return GRAD_REL * float(np.abs(ref).max()) + GRAD_ABS
LSE_TOL = 2.0 ** -8


def run_bwd(c, lse_only=False):
    import torch

    from transformer_attention_sdpa_amd import backward, forward

    q, k, v, do = (to_device(c[x], "bf16") for x in ("q", "k", "v", "do"))
    kl = None if c["key_lens"] is None else torch.from_numpy(np.asarray(c["key_lens"], np.int32)).cuda()
    kw = dict(causal=c["causal"], key_lens=kl, window=c["window"])
    out, lse = forward(q, k, v, return_lse=True, **kw)
    if lse_only:
        torch.cuda.synchronize()
        return out, lse
    dq, dk, dv = backward(q, k, v, out, do, lse, **kw)
    torch.cuda.synchronize()
    return tuple(from_device(t) for t in (dq, dk, dv)), lse


def check_grads(name, got, ref):
    errs = []
    for g, r, what in zip(got, ref, ("dq", "dk", "dv")):
        mx = float(np.abs(r).max())
        err = max_abs_err(g, r)
        errs.append(f"{what} {err:.2e}/{mx:.2e}")
        assert np.all(np.isfinite(g)), (name, what)
        assert err <= grad_bound(r), (name, what, err, mx)
    print(f"bwd {name}: " + ", ".join(errs) + " (max abs err / max |ref|)")


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
]


@pytest.mark.parametrize("name,shape,opts", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(gpu_lib, name, shape, opts):
    B, h, n, m = shape
    c = backward_case(5000 + [x[0] for x in CASES].index(name), B, h, n, m, **opts)
    got, _ = run_bwd(c)
    ref = sb.attention_backward(c["q"], c["k"], c["v"], c["do"], causal=c["causal"],
                                key_lens=c["key_lens"], window=c["window"])
    check_grads(name, got, ref)


@pytest.mark.parametrize("name,shape,opts", CASES[:8], ids=[c[0] for c in CASES[:8]])
def test_lse_parity(gpu_lib, name, shape, opts):
    B, h, n, m = shape
    c = backward_case(6000 + [x[0] for x in CASES].index(name), B, h, n, m, **opts)
    _, lse = run_bwd(c, lse_only=True)
    got = lse.cpu().numpy().astype(np.float64)
    ref = sb.log_sum_exp(c["q"], c["k"], causal=c["causal"], key_lens=c["key_lens"], window=c["window"])
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf) and np.all(got[inf] == ref[inf]), name
    err = max_abs_err(got[~inf], ref[~inf])
    print(f"lse {name}: max abs err {err:.2e}")
    assert err <= LSE_TOL


def test_forward_lse_output_is_the_forward_output(gpu_lib):
    """sdpa_forward_lse writes the same output bits as sdpa_forward_window,
    on each forward kernel (sentence length, decode step, tiled)."""
    import torch

    from transformer_attention_sdpa_amd import forward

    for (B, h, n, m, opts) in ((4, 2, 64, 64, dict(causal=True)), (32, 8, 1, 300, dict(window=(None, 0, "bottom_right"))),
                               (2, 2, 300, 300, dict(window=(40, 8)))):
        c = backward_case(7001, B, h, n, m, **opts)
        q, k, v = (to_device(c[x], "bf16") for x in ("q", "k", "v"))
        o1 = forward(q, k, v, causal=c["causal"], window=c["window"])
        o2, _ = forward(q, k, v, causal=c["causal"], window=c["window"], return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), (B, h, n, m)


def test_backward_deterministic(gpu_lib):
    c = backward_case(7002, 2, 2, 300, 300, causal=True)
    a, _ = run_bwd(c)
    b, _ = run_bwd(c)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_ignores_rows_past_key_length(gpu_lib):
    """K and V rows at or past key_lens[b] may hold anything: NaN there changes
    no bit of the gradients, and their dK, dV rows are exactly zero."""
    c = backward_case(7003, 2, 2, 100, 150, key_lens=[120, 37])
    clean, _ = run_bwd(c)
    for b, L in enumerate(c["key_lens"]):
        c["k"][b, :, L:] = np.nan
        c["v"][b, :, L:] = np.nan
    dirty, _ = run_bwd(c)
    for x, y in zip(clean, dirty):
        assert np.array_equal(x, y)
    for b, L in enumerate(c["key_lens"]):
        assert np.all(dirty[1][b, :, L:] == 0) and np.all(dirty[2][b, :, L:] == 0)


def test_backward_four_wave_blocks_sampled(gpu_lib):
    """Enough heads for the four-wave workgroups (B·h·⌈n/128⌉ ≥ 1024): sampled
    dQ rows of every head, and every dK, dV row of two heads."""
    B, h, n = 8, 16, 1024
    c = backward_case(7004, B, h, n, n, causal=True)
    (dq, dk, dv), _ = run_bwd(c)
    rng = np.random.default_rng(7)
    picks = [(int(rng.integers(B)), int(rng.integers(h)), int(i)) for i in rng.integers(0, n, 48)]
    picks += [(0, 0, 0), (B - 1, h - 1, n - 1), (3, 5, 127), (3, 5, 128)]
    ref = sb.backward_query_rows(c["q"], c["k"], c["v"], c["do"], picks, causal=True)
    got = np.stack([dq[b, hh, i] for b, hh, i in picks])
    assert max_abs_err(got, ref) <= grad_bound(ref)
    for (b, hh) in ((0, 0), (B - 1, h - 1)):
        rk, rv = sb.backward_key_rows(c["q"], c["k"], c["v"], c["do"], b, hh, np.arange(n), causal=True)
        for g, r in ((dk[b, hh], rk), (dv[b, hh], rv)):
            err = max_abs_err(g, r)
            print(f"bwd 4-wave head {(b, hh)}: {err:.2e}/{np.abs(r).max():.2e}")
            assert err <= grad_bound(r)


def test_backward_long_causal_8k_sampled(gpu_lib):
    """The 8k causal shape (B = 4, h = 16, n = m = 8192): sampled dQ rows, and
    sampled dK, dV rows of one head (each key's column needs the whole head)."""
    from sdpa_inputs import WORKLOADS, grad_output, make_inputs

    wl = WORKLOADS["long_causal_8k"]
    c = make_inputs(wl, "bf16")
    c["do"] = grad_output(wl)
    (dq, dk, dv), _ = run_bwd(c)
    rng = np.random.default_rng(8)
    picks = [(int(rng.integers(wl.B)), int(rng.integers(wl.h)), int(i)) for i in rng.integers(0, wl.n, 24)]
    picks += [(0, 0, 0), (wl.B - 1, wl.h - 1, wl.n - 1)]
    ref = sb.backward_query_rows(c["q"], c["k"], c["v"], c["do"], picks, causal=True)
    got = np.stack([dq[b, hh, i] for b, hh, i in picks])
    err = max_abs_err(got, ref)
    print(f"bwd 8k dq rows: {err:.2e}/{np.abs(ref).max():.2e}")
    assert err <= grad_bound(ref)
    keys = np.concatenate([[0, 1, 63, 64, 4095, 8190, 8191], rng.integers(0, wl.m, 25)])
    rk, rv = sb.backward_key_rows(c["q"], c["k"], c["v"], c["do"], 1, 7, keys, causal=True)
    for g, r, what in ((dk[1, 7, keys], rk, "dk"), (dv[1, 7, keys], rv, "dv")):
        err = max_abs_err(g, r)
        print(f"bwd 8k {what} rows: {err:.2e}/{np.abs(r).max():.2e}")
        assert err <= grad_bound(r)
