"""Attention dropout on the GPU (bf16, d_k = d_v = 32, 64 or 128) against the
fp64 dropout oracle.

The pages train with dropout and tune an attention dropout (《Attention Is All
You Need：注意力就是你所需要的一切》 §5.4, §6.3) without placing it; the
reading, stated in ``oracle.sdpa_dropout``, drops weights after the softmax of
Eq. (1) by a keep mask Z and scales the kept ones by c = 1/(1 − p).  The mask
is an input to both sides (``sdpa_inputs.random_keep``, packed by
``pack_keep``), so they see the same Z.

Bars: outputs within the bf16 bar times c (the kept weights are scaled by c
before the bf16-sized errors of the product); gradients within the backward
tests' bar times c, c · 2e-2 of each tensor's largest magnitude plus 2^-16.
The leading gradient error is the one the backward tests name: D_i = dO_i ·
O_i is formed from the bf16-rounded forward output, whose rounding error is
proportional to |O|, and the kept terms of O carry the factor c (on the
bottom-right decoder case an fp64 evaluation that rounds only O to bf16
before D accounts for 6.6e-3 of the kernel's 7.5e-3 on dK).  Where each
dropped weight's place is known (V = I), the zero pattern is compared exactly.
Width 64 runs through the 64-wide tiled kernel, widths 32 and 128 through the
kernel written for the other head widths; the cases cover both, with their
two launch shapes (2 and 4 waves per workgroup).
"""

import numpy as np
import pytest

import oracle.sdpa_backward as sb
import oracle.sdpa_dropout as sd
from sdpa_inputs import backward_case, pack_keep, random_keep
from tests.gpu_cases import TOL, from_device, max_abs_err, to_device

pytestmark = pytest.mark.gpu

GRAD_REL, GRAD_ABS = 2e-2, 2.0 ** -16

CASES = [  # id, (B, h, n, m), options, p
    ("encoder_padded", (8, 4, 64, 64), dict(key_lens=[64, 8, 33, 50, 64, 1, 0, 40]), 0.1),
    ("decoder_causal", (4, 4, 64, 64), dict(causal=True), 0.5),
    ("cross_ragged_words", (3, 2, 48, 70), dict(key_lens=[70, 33, 65]), 0.3),
    ("multi_tile_causal", (2, 2, 300, 300), dict(causal=True, key_lens=[260, 300]), 0.1),
    ("window", (2, 2, 300, 300), dict(window=(40, 8), key_lens=[300, 211]), 0.2),
    ("bottom_right_decode", (2, 2, 5, 200), dict(window=(None, 0, "bottom_right"), key_lens=[150, 3]), 0.1),
    ("single_query_key", (3, 1, 1, 1), {}, 0.5),
    ("four_wave_blocks", (4, 16, 1100, 1100), dict(causal=True), 0.1),
    ("w32_encoder_padded", (8, 4, 64, 64), dict(d=32, key_lens=[64, 8, 33, 50, 64, 1, 0, 40]), 0.1),
    ("w128_decoder_causal", (4, 4, 64, 64), dict(d=128, causal=True), 0.5),
    ("w32_multi_tile_causal", (2, 2, 300, 300), dict(d=32, causal=True, key_lens=[260, 300]), 0.1),
    ("w128_window_ragged_words", (2, 2, 300, 270), dict(d=128, window=(40, 8), key_lens=[270, 211]), 0.2),
    ("w128_bottom_right_decode", (2, 2, 5, 200), dict(d=128, window=(None, 0, "bottom_right"), key_lens=[150, 3]),
     0.1),
    ("w32_single_query_key", (3, 1, 1, 1), dict(d=32), 0.5),
    ("w128_four_wave_blocks", (2, 64, 1100, 1100), dict(d=128, causal=True), 0.1),
    ("w32_four_wave_blocks", (2, 64, 1100, 1100), dict(d=32, window=(300, 0)), 0.3),
]
LARGE = 1 << 24  # B·h·n·m above this: forward only, three whole heads against the oracle


def _large(i):
    B, h, n, m = CASES[i][1]
    return B * h * n * m > LARGE


def _case(i):
    name, (B, h, n, m), opts, p = CASES[i]
    c = backward_case(9100 + i, B, h, n, m, **opts)
    rng = np.random.default_rng(9200 + i)
    c["keep"] = random_keep(rng, B, h, n, m, p)
    c["keep_scale"] = 1.0 / (1.0 - p)
    return c


def _kw(c):
    import torch

    kl = None if c["key_lens"] is None else torch.from_numpy(np.asarray(c["key_lens"], np.int32)).cuda()
    return dict(causal=c["causal"], key_lens=kl, window=c["window"])


def _mask(c):
    import torch

    return torch.from_numpy(pack_keep(c["keep"]).view(np.int32)).cuda()


def _run(c, backward=False):
    import torch

    from transformer_attention_sdpa_amd import backward_dropout, forward_dropout

    q, k, v, do = (to_device(c[x], "bf16") for x in ("q", "k", "v", "do"))
    mask = _mask(c)
    out, lse = forward_dropout(q, k, v, mask, c["keep_scale"], return_lse=True, **_kw(c))
    grads = backward_dropout(q, k, v, out, do, lse, mask, c["keep_scale"], **_kw(c)) if backward else None
    torch.cuda.synchronize()
    return out, lse, grads


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_dropout_forward_parity(gpu_lib, i):
    c = _case(i)
    out, lse, _ = _run(c)
    got = from_device(out)
    B, h, n, m = CASES[i][1]
    kw = dict(causal=c["causal"], key_lens=c["key_lens"], window=c["window"])
    if _large(i):  # three whole heads
        errs = []
        for b, hh in ((0, 0), (B - 1, h - 1), (1, 5)):
            one = lambda x: x[b:b + 1, hh:hh + 1]  # noqa: E731
            kl = None if c["key_lens"] is None else c["key_lens"][b:b + 1]
            ref = sd.attention_dropout(one(c["q"]), one(c["k"]), one(c["v"]), one(c["keep"]), c["keep_scale"],
                                       causal=c["causal"], key_lens=kl, window=c["window"])
            errs.append(max_abs_err(one(got), ref))
        err = max(errs)
    else:
        ref = sd.attention_dropout(c["q"], c["k"], c["v"], c["keep"], c["keep_scale"], **kw)
        err = max_abs_err(got, ref)
    print(f"dropout fwd {CASES[i][0]}: max abs err {err:.2e} (c = {c['keep_scale']:.3f})")
    assert err <= TOL["bf16"] * c["keep_scale"]
    # the softmax (and so lse) does not see the mask
    if not _large(i):
        ref_l = sb.log_sum_exp(c["q"], c["k"], **kw)
        got_l = lse.cpu().numpy().astype(np.float64)
        inf = np.isinf(ref_l)
        assert np.array_equal(np.isinf(got_l), inf)
        assert max_abs_err(got_l[~inf], ref_l[~inf]) <= 2.0 ** -8


BWD = [i for i in range(len(CASES)) if not _large(i)]


@pytest.mark.parametrize("i", BWD, ids=[CASES[i][0] for i in BWD])
def test_dropout_backward_parity(gpu_lib, i):
    c = _case(i)
    _, _, grads = _run(c, backward=True)
    ref = sd.attention_dropout_backward(c["q"], c["k"], c["v"], c["do"], c["keep"], c["keep_scale"],
                                        causal=c["causal"], key_lens=c["key_lens"], window=c["window"])
    msgs = []
    for g, r, what in zip(grads, ref, ("dq", "dk", "dv")):
        g = from_device(g)
        mx, err = float(np.abs(r).max()), max_abs_err(g, r)
        msgs.append(f"{what} {err:.2e}/{mx:.2e}")
        assert np.all(np.isfinite(g)) and err <= GRAD_REL * c["keep_scale"] * mx + GRAD_ABS, (what, err, mx)
    print(f"dropout bwd {CASES[i][0]}: " + ", ".join(msgs))


@pytest.mark.parametrize("d,m", [(64, 64), (64, 45), (32, 32), (128, 100)])
def test_dropout_pattern_is_exact(gpu_lib, d, m):
    """V = I (m ≤ d_v) makes the output row i the dropped weights themselves:
    exactly 0 wherever Z_ij = 0 or the key is illegal, positive elsewhere."""
    B, h, n = 4, 3, 64
    seed = 9300 + m if d == 64 else 9350 + d
    c = backward_case(seed, B, h, n, m, causal=m == n, key_lens=[m, 17, 1, m - 5], d=d)
    c["v"] = np.zeros_like(c["v"])
    c["v"][:, :, np.arange(m), np.arange(m)] = 1.0
    rng = np.random.default_rng(9400 + m if d == 64 else 9450 + d)
    c["keep"] = random_keep(rng, B, h, n, m, 0.4)
    c["keep_scale"] = 1.0 / 0.6
    out, _, _ = _run(c)
    got = from_device(out)[..., :m]
    kw = dict(causal=c["causal"], key_lens=c["key_lens"])
    ref = sd.attention_dropout(c["q"], c["k"], c["v"], c["keep"], c["keep_scale"], **kw)[..., :m]
    assert np.array_equal(got == 0.0, ref == 0.0)
    assert not np.signbit(got[got == 0.0]).any()
    assert max_abs_err(got, ref) <= TOL["bf16"] * c["keep_scale"]


@pytest.mark.parametrize("d", [32, 64, 128])
def test_all_kept_equals_plain_bitwise(gpu_lib, d):
    """Every weight kept and c = 1: the same arithmetic as the plain tiled
    path (n, m > 64), so output, lse and gradients agree bit for bit."""
    import torch

    from transformer_attention_sdpa_amd import backward, backward_dropout, forward, forward_dropout

    c = backward_case(9500 if d == 64 else 9500 + d, 2, 4, 200, 260, key_lens=[260, 101], d=d)
    q, k, v, do = (to_device(c[x], "bf16") for x in ("q", "k", "v", "do"))
    kl = torch.from_numpy(np.asarray(c["key_lens"], np.int32)).cuda()
    ones = torch.full((2, 4, 200, (260 + 31) // 32), -1, dtype=torch.int32, device="cuda")
    o1, l1 = forward(q, k, v, key_lens=kl, return_lse=True)
    o2, l2 = forward_dropout(q, k, v, ones, 1.0, key_lens=kl, return_lse=True)
    g1 = backward(q, k, v, o1, do, l1, key_lens=kl)
    g2 = backward_dropout(q, k, v, o2, do, l2, ones, 1.0, key_lens=kl)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("window", [None, (9, 2, "bottom_right")])
def test_all_kept_equals_plain_bitwise_sentence_length(gpu_lib, d, window):
    """n, m <= 64 (the sentence-length forward kernel and the fused one-launch
    gradient): with every weight kept and c = 1 the dropout forms equal the
    plain ones bit for bit (output and lse; gradients from the same forward
    output and lse)."""
    import torch

    from transformer_attention_sdpa_amd import backward, backward_dropout, forward, forward_dropout

    c = backward_case(9600 + d, 3, 4, 64, 50, key_lens=[50, 17, 0], window=window, d=d)
    q, k, v, do = (to_device(c[x], "bf16") for x in ("q", "k", "v", "do"))
    kl = torch.from_numpy(np.asarray(c["key_lens"], np.int32)).cuda()
    ones = torch.full((3, 4, 64, 2), -1, dtype=torch.int32, device="cuda")
    o, lse = forward(q, k, v, key_lens=kl, window=window, return_lse=True)
    o2, l2 = forward_dropout(q, k, v, ones, 1.0, key_lens=kl, window=window, return_lse=True)
    g1 = backward(q, k, v, o, do, lse, key_lens=kl, window=window)
    g2 = backward_dropout(q, k, v, o, do, lse, ones, 1.0, key_lens=kl, window=window)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_keep_mask_helper(gpu_lib):
    """dropout_keep_mask: the layout the kernels read, with keep fraction
    1 − p within five standard deviations."""
    import torch

    from transformer_attention_sdpa_amd import dropout_keep_mask

    g = torch.Generator(device="cuda").manual_seed(3)
    B, h, n, m, p = 2, 4, 128, 100, 0.3
    words = dropout_keep_mask(B, h, n, m, p, generator=g)
    assert words.dtype == torch.int32 and tuple(words.shape) == (B, h, n, 4)
    keep = sd.unpack_keep(words.cpu().numpy().view(np.uint32), m)
    N = keep.size
    assert abs(keep.mean() - (1 - p)) <= 5 * np.sqrt(p * (1 - p) / N)
    with pytest.raises(ValueError):
        dropout_keep_mask(1, 1, 1, 1, 1.0)


def test_dropout_wrapper_errors(gpu_lib):
    import torch

    from transformer_attention_sdpa_amd import forward_dropout

    q = torch.zeros(1, 1, 8, 16, device="cuda", dtype=torch.bfloat16)
    mask = torch.zeros(1, 1, 8, 1, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError, match="unsupported"):
        forward_dropout(q, q, q, mask, 1.0)  # width 16: the dropout kernels take 32, 64, 128
    q64 = torch.zeros(1, 1, 8, 64, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="scale"):
        forward_dropout(q64, q64, q64, mask, float("inf"))
    with pytest.raises(ValueError, match="keep_mask"):
        forward_dropout(q64, q64, q64, mask[..., :0], 1.0)
