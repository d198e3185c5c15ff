"""Head widths 32 and 128 (bf16) on the GPU against the fp64 oracle.

The pages' model variants use 16 heads of 32 and 4 heads of 128 beside the
base model's 8 heads of 64, and d_model = 256 / 1024 with 32- / 128-wide heads
(《精读 Attention Is All You Need：原始 Transformer 论文》 Table 3, rows (A)
and (C)).  Eq. (1) is the same at every width; the oracle takes any width.
Bar: the bf16 one, 2e-2 absolute; the log-sum-exp within 2^-8 (this kernel
sums fp32 weights, so it is far tighter in practice).
"""

import numpy as np
import pytest

import oracle.sdpa_backward as sb
import oracle.sdpa_oracle as so
from sdpa_inputs import random_case
from tests.gpu_cases import TOL, from_device, max_abs_err, run_gpu, to_device

pytestmark = pytest.mark.gpu

CASES = [  # id, (B, h, n, m, d), options
    ("A_h16_d32_encoder", (64, 16, 64, 64, 32), dict(key_lens=(8, 64))),
    ("A_h4_d128_encoder", (64, 4, 64, 64, 128), dict(key_lens=(8, 64))),
    ("C_dmodel256_d32_decoder", (16, 8, 64, 64, 32), dict(causal=True, key_lens=(8, 64))),
    ("C_dmodel1024_d128_cross", (8, 8, 48, 64, 128), dict(key_lens=(16, 64))),
    ("d32_ragged_tiles", (2, 2, 100, 130, 32), dict(key_lens=(1, 130))),
    ("d128_multi_tile_causal", (2, 2, 300, 300, 128), dict(causal=True)),
    ("d32_window", (2, 2, 300, 300, 32), dict(window=(40, 8))),
    ("d128_bottom_right", (4, 2, 5, 200, 128), dict(window=(None, 0, "bottom_right"), key_lens=(0, 200))),
    ("d32_four_wave_blocks", (8, 16, 1024, 1024, 32), dict(causal=True)),
    ("d128_four_wave_blocks", (8, 16, 1024, 1024, 128), dict(causal=True)),
    # sentence-length kernel (n, m <= 64) at both widths: windows in both
    # alignments, key lengths 0 and past m, ragged lengths, a lone query and
    # key, and queries that leave waves idle (n < 16, 33, 48)
    ("d32_short_window", (3, 2, 64, 64, 32), dict(window=(5, 3))),
    ("d128_short_window_causal_like", (3, 2, 40, 40, 128), dict(window=(None, 0), key_lens=(0, 40))),
    ("d128_short_bottom_right", (3, 2, 7, 50, 128), dict(window=(None, 0, "bottom_right"), key_lens=(0, 60))),
    ("d32_short_bottom_right_band", (2, 3, 12, 64, 32), dict(window=(6, 2, "bottom_right"), key_lens=(1, 64))),
    ("d128_short_ragged", (2, 3, 33, 17, 128), dict(key_lens=(0, 20))),
    ("d32_short_ragged_causal", (3, 1, 63, 63, 32), dict(causal=True, key_lens=(1, 63))),
    ("d32_short_one_by_one", (1, 1, 1, 1, 32), {}),
    ("d128_short_one_by_one", (2, 1, 1, 1, 128), dict(key_lens=(0, 1))),
]


def _case(i, shape, opts):
    B, h, n, m, d = shape
    rng = np.random.default_rng(8000 + i)
    opts = dict(opts)
    if isinstance(opts.get("key_lens"), tuple):
        lo, hi = opts["key_lens"]
        opts["key_lens"] = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    return random_case(rng, B, h, n, m, d, d, dtype="bf16", **opts)


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_width_parity(gpu_lib, i):
    name, shape, opts = CASES[i]
    c = _case(i, shape, opts)
    _, got = run_gpu(c)
    B, h, n, m, d = shape
    if B * h * n * m > 1 << 26:  # large: sampled rows (each costs one row of the head)
        rng = np.random.default_rng(9)
        picks = [(int(rng.integers(B)), int(rng.integers(h)), int(q)) for q in rng.integers(0, n, 64)]
        picks += [(0, 0, 0), (B - 1, h - 1, n - 1), (1, 3, 127), (1, 3, 128)]
        ref = so.attention_rows(c["q"], c["k"], c["v"], picks, causal=c["causal"], key_lens=c["key_lens"],
                                window=c["window"])
        got = np.stack([got[b, hh, q] for b, hh, q in picks])
    else:
        ref = so.attention(c["q"], c["k"], c["v"], causal=c["causal"], key_lens=c["key_lens"],
                           window=c["window"])
    err = max_abs_err(got, ref)
    print(f"width {name}: max abs err {err:.2e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("i", [0, 1, 5, 7], ids=[CASES[i][0] for i in (0, 1, 5, 7)])
def test_width_lse(gpu_lib, i):
    import torch

    from transformer_attention_sdpa_amd import forward

    name, shape, opts = CASES[i]
    c = _case(i, shape, opts)
    q, k, v = (to_device(c[x], "bf16") for x in ("q", "k", "v"))
    kl = None if c["key_lens"] is None else torch.from_numpy(c["key_lens"]).cuda()
    out, lse = forward(q, k, v, causal=c["causal"], key_lens=kl, window=c["window"], return_lse=True)
    o2 = forward(q, k, v, causal=c["causal"], key_lens=kl, window=c["window"])
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), o2.view(torch.int16))
    got = lse.cpu().numpy().astype(np.float64)
    ref = sb.log_sum_exp(c["q"], c["k"], causal=c["causal"], key_lens=c["key_lens"], window=c["window"])
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf) and np.all(got[inf] == ref[inf])
    err = max_abs_err(got[~inf], ref[~inf])
    print(f"width lse {name}: max abs err {err:.2e}")
    assert err <= 2.0 ** -8


def test_width_deterministic_and_ignores_padded_rows(gpu_lib):
    c = _case(0, (4, 2, 100, 150, 128), dict(key_lens=np.array([150, 37, 0, 99], np.int32)))
    _, a = run_gpu(c)
    for b, L in enumerate(c["key_lens"]):
        c["k"][b, :, L:] = np.nan
        c["v"][b, :, L:] = np.nan
    _, b2 = run_gpu(c)
    assert np.array_equal(a, b2)
    assert np.all(a[2] == 0)  # no legal key: zero rows


BWD_CASES = [  # id, (B, h, n, m, d), options
    ("d32_encoder_padded", (8, 4, 64, 64, 32), dict(key_lens=(8, 64))),
    ("d128_encoder_padded", (8, 2, 64, 64, 128), dict(key_lens=(8, 64))),
    ("d32_multi_tile_causal", (2, 2, 300, 300, 32), dict(causal=True)),
    ("d128_multi_tile_causal", (2, 2, 300, 300, 128), dict(causal=True)),
    ("d32_window_ragged", (2, 2, 200, 230, 32), dict(window=(30, 10), key_lens=(100, 230))),
    ("d128_bottom_right", (2, 2, 5, 200, 128), dict(window=(None, 0, "bottom_right"), key_lens=(0, 200))),
    ("d128_cross_padded", (3, 2, 70, 130, 128), dict(key_lens=(1, 130))),
    # sentence length (n, m <= 64): the fused one-launch kernel at both widths
    ("d32_short_causal_padded", (4, 3, 64, 64, 32), dict(causal=True, key_lens=(0, 64))),
    ("d128_short_window", (3, 2, 64, 64, 128), dict(window=(5, 3), key_lens=(1, 64))),
    ("d32_short_bottom_right", (3, 2, 7, 50, 32), dict(window=(None, 0, "bottom_right"), key_lens=(0, 60))),
    ("d128_short_ragged_cross", (2, 3, 33, 17, 128), dict(key_lens=(0, 20))),
    ("d32_short_n_gt_m", (2, 2, 64, 9, 32), {}),
    ("d128_short_one_by_one", (2, 1, 1, 1, 128), dict(key_lens=(0, 1))),
]


@pytest.mark.parametrize("i", range(len(BWD_CASES)), ids=[c[0] for c in BWD_CASES])
def test_width_backward_parity(gpu_lib, i):
    """dQ, dK, dV at widths 32 and 128 against the fp64 gradient oracle (bar as
    for width 64: 2e-2 of each tensor's largest magnitude, plus 2^-16)."""
    import torch

    from transformer_attention_sdpa_amd import backward, forward

    name, shape, opts = BWD_CASES[i]
    c = _case(100 + i, shape, opts)
    B, h, n, m, d = shape
    rng = np.random.default_rng(8500 + i)
    from sdpa_inputs import round_to_bf16

    c["do"] = round_to_bf16(rng.standard_normal((B, h, n, d), dtype=np.float32))
    q, k, v, do = (to_device(c[x], "bf16") for x in ("q", "k", "v", "do"))
    kl = None if c["key_lens"] is None else torch.from_numpy(c["key_lens"]).cuda()
    kw = dict(causal=c["causal"], key_lens=kl, window=c["window"])
    out, lse = forward(q, k, v, return_lse=True, **kw)
    grads = backward(q, k, v, out, do, lse, **kw)
    torch.cuda.synchronize()
    refs = sb.attention_backward(c["q"], c["k"], c["v"], c["do"], causal=c["causal"], key_lens=c["key_lens"],
                                 window=c["window"])
    msg = []
    for what, g, r in zip(("dq", "dk", "dv"), grads, refs):
        g = from_device(g)
        err = max_abs_err(g, r)
        bound = 2e-2 * float(np.abs(r).max()) + 2.0 ** -16
        msg.append(f"{what} {err:.2e}/{np.abs(r).max():.2e}")
        assert np.all(np.isfinite(g)) and err <= bound, (name, what, err, bound)
    print(f"width bwd {name}: " + ", ".join(msg))


@pytest.mark.parametrize("d", [32, 128])
def test_short_width_backward_ignores_rows_past_key_length(gpu_lib, d):
    """The fused sentence-length gradient: NaN in the K and V rows at or past
    each key length changes no bit of the gradients, and those rows' dK, dV
    are exactly zero."""
    import torch

    from transformer_attention_sdpa_amd import backward, forward

    c = _case(130 + d, (3, 2, 48, 64, d), dict(key_lens=np.array([64, 21, 0], np.int32)))
    rng = np.random.default_rng(8600 + d)
    from sdpa_inputs import round_to_bf16

    do_ = round_to_bf16(rng.standard_normal((3, 2, 48, d), dtype=np.float32))
    kl = torch.from_numpy(c["key_lens"]).cuda()

    def run():
        q, k, v, do = (to_device(x, "bf16") for x in (c["q"], c["k"], c["v"], do_))
        out, lse = forward(q, k, v, key_lens=kl, return_lse=True)
        g = backward(q, k, v, out, do, lse, key_lens=kl)
        torch.cuda.synchronize()
        return [x.view(torch.int16).cpu() for x in g]

    clean = run()
    for b, L in enumerate(c["key_lens"]):
        c["k"][b, :, L:] = np.nan
        c["v"][b, :, L:] = np.nan
    dirty = run()
    for x, y in zip(clean, dirty):
        assert torch.equal(x, y)
    for b, L in enumerate(c["key_lens"]):
        assert torch.all(dirty[1][b, :, L:] == 0) and torch.all(dirty[2][b, :, L:] == 0)


def test_width_backward_deterministic(gpu_lib):
    import torch

    from transformer_attention_sdpa_amd import backward, forward

    c = _case(120, (2, 2, 300, 300, 128), dict(causal=True))
    q, k, v = (to_device(c[x], "bf16") for x in ("q", "k", "v"))
    out, lse = forward(q, k, v, causal=True, return_lse=True)
    do = torch.randn_like(out)
    a = backward(q, k, v, out, do, lse, causal=True)
    b = backward(q, k, v, out, do, lse, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("d", [32, 128])
def test_short_width_padded_keys_are_never_read(gpu_lib, d):
    """Sentence-length kernel at width 32 and 128: NaN and huge values in the
    K/V rows at or past each key length leave the output bitwise unchanged."""
    import torch

    rng = np.random.default_rng(90 + d)
    B, h, n, m = 3, 2, 48, 64
    kl = np.array([m, 9, 40], np.int32)
    c = random_case(rng, B, h, n, m, d, d, dtype="bf16", key_lens=kl)
    o1, _ = run_gpu(c)
    for b in range(B):
        c["k"][b, :, kl[b]:] = np.nan
        c["v"][b, :, kl[b]:] = 3e38
    o2, got2 = run_gpu(c)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert np.isfinite(got2).all()


def test_short_width_masked_weights_are_exactly_zero(gpu_lib):
    """Width 128 holds the whole weight row (m = 64 <= d_v): V = [I | 0] makes
    O[:, :m] the weights, and every masked one must be +0.0 (causal and key
    padding on the sentence-length kernel)."""
    rng = np.random.default_rng(91)
    B, h, n, m, d = 4, 2, 64, 64, 128
    kl = np.array([64, 17, 1, 40], np.int32)
    c = random_case(rng, B, h, n, m, d, d, dtype="bf16", causal=True, key_lens=kl)
    c["v"] = np.zeros_like(c["v"])
    c["v"][:, :, np.arange(m), np.arange(m)] = 1.0
    _, got = run_gpu(c)
    j = np.arange(m)
    for b in range(B):
        for i in range(n):
            vis = (j < kl[b]) & (j <= i)
            row = got[b, :, i, :m]
            assert np.all(row[:, ~vis] == 0.0) and not np.signbit(row[:, ~vis]).any()
            assert np.allclose(row.sum(-1), 1.0, atol=4 * TOL["bf16"])
    assert np.all(got[..., m:] == 0.0)
    assert max_abs_err(got, so.attention(c["q"], c["k"], c["v"], causal=True, key_lens=kl)) <= TOL["bf16"]
