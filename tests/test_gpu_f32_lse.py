"""The per-row log-sum-exp of the fp32 forward kernels (GPU) against the fp64
oracle.

lse_i = ln Σ_j exp(s_ij) over the legal keys j of row i, s = scale · q_i · k_j
(the softmax denominator of Eq. (1) in 《精读 Attention Is All You Need：原始
Transformer 论文》, in log form), −∞ for a row with no legal key.  Both fp32
kernels, the sentence-length one (n, m ≤ 64) and the tiled one, write it
beside the output when asked, and the output must not change by a bit.

Bar: 2^-16 · (1 + |lse|).  An error δ in every score moves lse by at most δ;
the fp32 scores of N(0, 1) inputs at d_k = 64 carry about 64 · 2^-24 · |s|,
the hardware exp2 an ulp or two of each weight, the fp32 running sum (Kahan-
compensated in the tiled kernel) about m · 2^-24 relative, and the final
mc + log2 l one rounding of a number near |lse| · log2 e.  The measured errors
are printed.
"""

import numpy as np
import pytest

import oracle.sdpa_backward as sb
from sdpa_inputs import random_case
from tests.gpu_cases import max_abs_err, to_device

pytestmark = pytest.mark.gpu

CASES = [  # id, (B, h, n, m), options
    ("short_encoder_padded", (8, 4, 64, 64), dict(key_lens=(0, 64))),
    ("short_decoder_causal", (4, 4, 64, 64), dict(causal=True)),
    ("short_cross", (3, 2, 17, 50), dict(key_lens=(1, 50))),
    ("short_window_bottom_right", (2, 2, 5, 60), dict(window=(7, 0, "bottom_right"), key_lens=(3, 60))),
    ("short_one_by_one", (2, 1, 1, 1), {}),
    ("long_multi_tile_causal", (2, 2, 300, 300), dict(causal=True, key_lens=(200, 300))),
    ("long_window", (2, 2, 300, 300), dict(window=(40, 8), key_lens=(100, 300))),
    ("long_ragged_cross", (2, 3, 100, 517), dict(key_lens=(0, 517))),
    ("long_decode_step", (8, 4, 1, 700), dict(window=(None, 0, "bottom_right"), key_lens=(1, 700))),
    ("long_sharp_scores", (1, 2, 200, 260), dict(scale=1.0)),
]


def _case(i):
    name, (B, h, n, m), opts = CASES[i]
    opts = dict(opts)
    rng = np.random.default_rng(9600 + i)
    scale = opts.pop("scale", None)
    if isinstance(opts.get("key_lens"), tuple):
        lo, hi = opts["key_lens"]
        opts["key_lens"] = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    c = random_case(rng, B, h, n, m, 64, 64, dtype="f32", **opts)
    c["scale"] = scale
    return c


def _kw(c):
    import torch

    kl = None if c["key_lens"] is None else torch.from_numpy(c["key_lens"]).cuda()
    return dict(causal=c["causal"], key_lens=kl, window=c["window"], scale=c["scale"])


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_f32_lse_parity(gpu_lib, i):
    import torch

    from transformer_attention_sdpa_amd import forward

    c = _case(i)
    q, k, v = (to_device(c[x], "f32") for x in ("q", "k", "v"))
    out, lse = forward(q, k, v, return_lse=True, **_kw(c))
    plain = forward(q, k, v, **_kw(c))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), plain.view(torch.int32))
    got = lse.cpu().numpy().astype(np.float64)
    ref = sb.log_sum_exp(c["q"], c["k"], scale=c["scale"], causal=c["causal"], key_lens=c["key_lens"],
                         window=c["window"])
    inf = np.isinf(ref)
    assert np.array_equal(np.isinf(got), inf) and np.all(got[inf] == ref[inf])
    err = np.abs(got[~inf] - ref[~inf])
    bar = 2.0 ** -16 * (1.0 + np.abs(ref[~inf]))
    print(f"f32 lse {CASES[i][0]}: max abs err {max_abs_err(got[~inf], ref[~inf]):.2e}, "
          f"max |lse| {np.abs(ref[~inf]).max() if err.size else 0:.1f}")
    assert np.all(err <= bar)


def test_f32_lse_token_major_matches_packed(gpu_lib):
    """Token-major views through sdpa_forward_strided: the same output and
    lse bits as the packed call, on both fp32 kernels."""
    import torch

    from transformer_attention_sdpa_amd import forward

    def tm(t):
        return t.transpose(1, 2).contiguous().transpose(1, 2)

    for n, m in ((48, 64), (130, 190)):
        rng = np.random.default_rng(9700 + n)
        c = random_case(rng, 2, 4, n, m, 64, 64, dtype="f32",
                        key_lens=rng.integers(0, m, size=2, endpoint=True).astype(np.int32))
        q, k, v = (to_device(c[x], "f32") for x in ("q", "k", "v"))
        kl = torch.from_numpy(c["key_lens"]).cuda()
        o1, l1 = forward(q, k, v, key_lens=kl, return_lse=True)
        o2, l2 = forward(tm(q), tm(k), tm(v), key_lens=kl, out=tm(torch.empty_like(o1)), return_lse=True)
        torch.cuda.synchronize()
        assert torch.equal(o2.contiguous().view(torch.int32), o1.view(torch.int32)), (n, m)
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), (n, m)
