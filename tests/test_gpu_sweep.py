"""Seeded random sweep over every entry point and dispatch path (GPU) against
the fp64 oracle.

Each case draws, from one PCG64 stream: the dtype, the head widths (every
pair the library takes: 64/64, 32, 128, 16, 512 and d_k = 16 or 32 against
d_v = 64 in bf16; 64/64 in fp32), the batch and head counts, the lengths (a
sentence-length regime with n, m ≤ 64, a tiled one up to a few hundred, and
decoder steps of 1..16 queries against longer key sets, with enough heads to
take the decode kernel), the mask (none, causal when n = m, or a key window
with either side open and either alignment), per-sequence key lengths from 0
to past m, the caller's layout (packed, or token-major views through
sdpa_forward_strided), the log-sum-exp output and the split-key workspace.
The gradient cases draw the backward widths (bf16 32, 64, 128; fp32 64) and
the dropout cases a keep probability and a width (32, 64 or 128, from a stream
of their own so that the other draws of a case do not depend on it).  Every case prints its draw, so a
failure names it.

Bars: the forward ones of the other parity tests (2e-2 bf16, 1e-5 fp32
absolute; log-sum-exp 2^-8 bf16, 2^-16 (1 + |lse|) fp32); gradients 2e-2 ·
max|ref| + 2^-16 in bf16 and 2^-16 (max|ref| + 1) in fp32, times the keep
factor with dropout (the reasons are given in the gradient and dropout tests).
The bf16 gradients add the bound of their one error term that does not
shrink with the gradient: D_i = dO_i · O_i is formed from the bf16-rounded
forward output, so |δD_i| ≤ 2^-9 Σ_t |dO_it| |O_it| (half an ulp of O under
round-to-nearest), which reaches dQ_i as scale · |δD_i| Σ_j P_ij |k_j| and dK_j as
scale · Σ_i P_ij |δD_i| |q_i|.  Where few keys are legal, dQ and dK are small
by cancellation while that term is not (a key length of 2 under a window: an
fp64 evaluation that rounds only O before D reproduces 8.6e-3 of the device's
8.7e-3 on dK, against max |dK| = 0.23).
"""

import numpy as np
import pytest

import oracle.sdpa_backward as sb
import oracle.sdpa_dropout as sd
import oracle.sdpa_oracle as so
from sdpa_inputs import pack_keep, random_case, random_keep, round_to_bf16
from tests.gpu_cases import TOL, from_device, max_abs_err, to_device

pytestmark = pytest.mark.gpu

SEED = 20261202
N_FWD, N_BWD, N_DROP = 160, 48, 24

BF16_WIDTHS = [(64, 64)] * 4 + [(32, 32), (128, 128), (16, 16), (16, 64), (32, 64), (512, 512)]


def _lens(rng, regime):
    if regime == "short":
        return int(rng.integers(1, 65)), int(rng.integers(1, 65))
    if regime == "tiled":
        return int(rng.integers(1, 400)), int(rng.integers(65, 400))
    return int(rng.integers(1, 17)), int(rng.integers(65, 700))  # decoder step


def _mask(rng, n, m):
    """(causal, window): causal only when n == m; windows with either side
    open (None) and either alignment."""
    r = rng.random()
    if r < 0.3:
        return False, None
    if r < 0.45 and n == m:
        return True, None
    left = None if rng.random() < 0.3 else int(rng.integers(0, max(2, m)))
    right = None if rng.random() < 0.3 else int(rng.integers(0, max(2, m // 2)))
    align = "bottom_right" if rng.random() < 0.5 else "top_left"
    return False, (left, right, align)


def _fwd_case(i):
    rng = np.random.default_rng([SEED, i])
    dt = "bf16" if rng.random() < 0.8 else "f32"
    dk, dv = BF16_WIDTHS[int(rng.integers(len(BF16_WIDTHS)))] if dt == "bf16" else (64, 64)
    regime = ["short", "tiled", "decode"][int(rng.integers(3))]
    n, m = _lens(rng, regime)
    if dk == 512:
        n, m = min(n, 130), min(m, 130)
    B, h = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    if regime == "decode" and dk == dv == 64 and dt == "bf16" and rng.random() < 0.5:
        B, h = 64, 4  # 256 heads: the decode kernel
    causal, window = _mask(rng, n, m)
    kl = rng.integers(0, m + 4, size=B).astype(np.int32) if rng.random() < 0.6 else None
    opts = dict(strided=bool(rng.random() < 0.3), lse=bool(rng.random() < 0.4),
                workspace=("auto" if rng.random() < 0.5 else None))
    c = random_case(rng, B, h, n, m, dk, dv, dtype=dt, causal=causal, key_lens=kl, window=window)
    return c, opts, dict(dtype=dt, B=B, h=h, n=n, m=m, d_k=dk, d_v=dv, causal=causal, window=window,
                         key_lens=None if kl is None else kl.tolist(), **opts)


def _kw(c):
    import torch

    kl = None if c["key_lens"] is None else torch.from_numpy(np.asarray(c["key_lens"], np.int32)).cuda()
    return dict(causal=c["causal"], key_lens=kl, window=c["window"])


def _token_major(t):
    return t.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("i", range(N_FWD))
def test_forward_sweep(gpu_lib, i):
    import torch

    from transformer_attention_sdpa_amd import forward

    c, opts, draw = _fwd_case(i)
    print(f"forward case {i}: {draw}", flush=True)
    dt = c["dtype"]
    q, k, v = (to_device(c[x], dt) for x in ("q", "k", "v"))
    out = None
    if opts["strided"]:
        q, k, v = _token_major(q), _token_major(k), _token_major(v)
        B, h, n, _ = q.shape
        out = _token_major(torch.empty((B, h, n, c["v"].shape[-1]), dtype=q.dtype, device="cuda"))
    res = forward(q, k, v, out=out, return_lse=opts["lse"], workspace=opts["workspace"], **_kw(c))
    torch.cuda.synchronize()
    o, lse = res if opts["lse"] else (res, None)
    ref = so.attention(c["q"], c["k"], c["v"], causal=c["causal"], key_lens=c["key_lens"], window=c["window"])
    err = max_abs_err(from_device(o), ref)
    print(f"  max abs err {err:.2e}")
    assert err <= TOL[dt]
    if lse is not None:
        ref_l = sb.log_sum_exp(c["q"], c["k"], causal=c["causal"], key_lens=c["key_lens"], window=c["window"])
        got_l = lse.cpu().numpy().astype(np.float64)
        inf = np.isinf(ref_l)
        assert np.array_equal(np.isinf(got_l), inf) and np.all(got_l[inf] == ref_l[inf])
        bar = 2.0 ** -8 if dt == "bf16" else 2.0 ** -16 * (1.0 + np.abs(ref_l[~inf]))
        assert np.all(np.abs(got_l[~inf] - ref_l[~inf]) <= bar)


def _bwd_case(i):
    rng = np.random.default_rng([SEED, 1000 + i])
    dt = "bf16" if rng.random() < 0.7 else "f32"
    d = int(rng.choice([32, 64, 128])) if dt == "bf16" else 64
    n, m = _lens(rng, ["short", "tiled", "decode"][int(rng.integers(3))])
    B, h = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    causal, window = _mask(rng, n, m)
    kl = rng.integers(0, m + 4, size=B).astype(np.int32) if rng.random() < 0.6 else None
    c = random_case(rng, B, h, n, m, d, d, dtype=dt, causal=causal, key_lens=kl, window=window)
    do = rng.standard_normal((B, h, n, d), dtype=np.float32)
    c["do"] = round_to_bf16(do) if dt == "bf16" else do
    return c, dict(dtype=dt, B=B, h=h, n=n, m=m, d=d, causal=causal, window=window,
                   key_lens=None if kl is None else kl.tolist())


def _grad_bar(dt, ref, c=1.0, d_term=0.0):
    mx = float(np.abs(ref).max())
    return (2e-2 * c * mx + 2.0 ** -16 + d_term) if dt == "bf16" else 2.0 ** -16 * (mx + 1.0)


def _d_term(c, keep=None, ks=1.0):
    """Bounds on the dQ and dK error from D_i = dO_i · O_i over the
    bf16-rounded output: (max_i scale |δD_i| Σ_j P_ij |k_j|,
    max_j scale Σ_i P_ij |δD_i| |q_i|) with |δD_i| ≤ 2^-9 Σ_t |dO_it| |O_it|."""
    B, h, n, d = c["q"].shape
    m = c["k"].shape[2]
    scale = 1.0 / np.sqrt(d)
    bq = bk = 0.0
    for b in range(B):
        L = None if c["key_lens"] is None else int(c["key_lens"][b])
        win = so._window_of(c["window"], n, m, L)
        vis = so.visible_keys(np.arange(n), m, c["causal"], L, window=win) if win is not None else \
            so.visible_keys(np.arange(n), m, c["causal"], L)
        for hh in range(h):
            q, k, v, do = (np.asarray(c[x][b, hh], np.float64) for x in ("q", "k", "v", "do"))
            P = so.row_softmax(so.apply_mask(so.scores(q, k, scale), vis))
            Pt = P if keep is None else P * keep[b, hh] * ks
            dD = 2.0 ** -9 * (np.abs(do) * np.abs(Pt @ v)).sum(1)
            bq = max(bq, float((scale * dD[:, None] * (P @ np.abs(k))).max()))
            bk = max(bk, float((scale * (P * dD[:, None]).T @ np.abs(q)).max()))
    return bq, bk


@pytest.mark.parametrize("i", range(N_BWD))
def test_backward_sweep(gpu_lib, i):
    import torch

    from transformer_attention_sdpa_amd import backward, forward

    c, draw = _bwd_case(i)
    print(f"backward case {i}: {draw}", flush=True)
    dt = c["dtype"]
    q, k, v, do = (to_device(c[x], dt) for x in ("q", "k", "v", "do"))
    out, lse = forward(q, k, v, return_lse=True, **_kw(c))
    grads = backward(q, k, v, out, do, lse, **_kw(c))
    torch.cuda.synchronize()
    ref = sb.attention_backward(c["q"], c["k"], c["v"], c["do"], causal=c["causal"], key_lens=c["key_lens"],
                                window=c["window"])
    dterm = _d_term(c) + (0.0,) if dt == "bf16" else (0.0, 0.0, 0.0)
    for g, r, what, dd in zip(grads, ref, ("dq", "dk", "dv"), dterm):
        g = from_device(g)
        err = max_abs_err(g, r)
        print(f"  {what}: max abs err {err:.2e} (max |ref| {np.abs(r).max():.2e}, D-term bound {dd:.1e})")
        assert np.all(np.isfinite(g)) and err <= _grad_bar(dt, r, d_term=dd), what


@pytest.mark.parametrize("i", range(N_DROP))
def test_dropout_sweep(gpu_lib, i):
    import torch

    from transformer_attention_sdpa_amd import backward_dropout, forward_dropout

    rng = np.random.default_rng([SEED, 2000 + i])
    n, m = _lens(rng, ["short", "tiled", "decode"][int(rng.integers(3))])
    B, h = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    causal, window = _mask(rng, n, m)
    kl = rng.integers(0, m + 4, size=B).astype(np.int32) if rng.random() < 0.6 else None
    p = float(rng.uniform(0.05, 0.5))
    d = int(np.random.default_rng([SEED, 2500 + i]).choice([32, 64, 64, 128]))
    c = random_case(rng, B, h, n, m, d, d, dtype="bf16", causal=causal, key_lens=kl, window=window)
    c["do"] = round_to_bf16(rng.standard_normal((B, h, n, d), dtype=np.float32))
    keep = random_keep(rng, B, h, n, m, p)
    ks = 1.0 / (1.0 - p)
    print(f"dropout case {i}: B={B} h={h} n={n} m={m} d={d} p={p:.2f} causal={causal} window={window} "
          f"key_lens={None if kl is None else kl.tolist()}", flush=True)
    q, k, v, do = (to_device(c[x], "bf16") for x in ("q", "k", "v", "do"))
    mask = torch.from_numpy(pack_keep(keep).view(np.int32)).cuda()
    out, lse = forward_dropout(q, k, v, mask, ks, return_lse=True, **_kw(c))
    grads = backward_dropout(q, k, v, out, do, lse, mask, ks, **_kw(c))
    torch.cuda.synchronize()
    kw = dict(causal=c["causal"], key_lens=c["key_lens"], window=c["window"])
    ref = sd.attention_dropout(c["q"], c["k"], c["v"], keep, ks, **kw)
    assert max_abs_err(from_device(out), ref) <= TOL["bf16"] * ks
    refg = sd.attention_dropout_backward(c["q"], c["k"], c["v"], c["do"], keep, ks, **kw)
    dterm = _d_term(c, keep, ks) + (0.0,)
    for g, r, what, dd in zip(grads, refg, ("dq", "dk", "dv"), dterm):
        g = from_device(g)
        err = max_abs_err(g, r)
        print(f"  {what}: max abs err {err:.2e} (max |ref| {np.abs(r).max():.2e}, D-term bound {dd:.1e})")
        assert np.all(np.isfinite(g)) and err <= _grad_bar("bf16", r, ks, dd), what
