"""The remaining head widths of the pages' model variants (bf16, GPU) against
the fp64 oracle.

《精读 Attention Is All You Need：原始 Transformer 论文》 Table 3 varies the
head widths: row (A) runs 32 heads of d_k = d_v = 16 and one of 512, and row (B) keeps
d_v = 64 while it shrinks the key width d_k to 16 or 32.  Eq. (1) contracts
queries with keys over d_k and weights with values over d_v, so the two
widths are independent; the oracle takes any pair.  These widths run on the
sentence-length kernel when n, m ≤ 64 and on the width kernel beyond, and row
(A)'s single head of 512 on a kernel of its own.  Bar: the bf16 one, 2e-2 absolute; the
log-sum-exp within 2^-8.
"""

import numpy as np
import pytest

import oracle.sdpa_backward as sb
import oracle.sdpa_oracle as so
from sdpa_inputs import random_case
from tests.gpu_cases import TOL, from_device, max_abs_err, run_gpu, to_device

pytestmark = pytest.mark.gpu

CASES = [  # id, (B, h, n, m, d_k, d_v), options
    ("A_h32_d16_encoder", (64, 32, 64, 64, 16, 16), dict(key_lens=(8, 64))),
    ("B_dk16_dv64_encoder", (64, 8, 64, 64, 16, 64), dict(key_lens=(8, 64))),
    ("B_dk32_dv64_encoder", (64, 8, 64, 64, 32, 64), dict(key_lens=(8, 64))),
    ("B_dk16_dv64_decoder", (16, 8, 64, 64, 16, 64), dict(causal=True, key_lens=(8, 64))),
    ("A_d16_cross", (8, 32, 48, 64, 16, 16), dict(key_lens=(16, 64))),
    ("d16_multi_tile_causal", (2, 2, 300, 300, 16, 16), dict(causal=True)),
    ("dk32_dv64_multi_tile_causal", (2, 2, 300, 300, 32, 64), dict(causal=True)),
    ("dk16_dv64_window_ragged", (2, 2, 260, 260, 16, 64), dict(window=(40, 8), key_lens=(100, 260))),
    ("d16_window", (2, 2, 300, 300, 16, 16), dict(window=(40, 8))),
    ("dk32_dv64_bottom_right", (4, 2, 5, 200, 32, 64), dict(window=(None, 0, "bottom_right"), key_lens=(0, 200))),
    ("d16_bottom_right_band", (2, 3, 12, 64, 16, 16), dict(window=(6, 2, "bottom_right"), key_lens=(1, 64))),
    ("d16_ragged", (2, 3, 33, 17, 16, 16), dict(key_lens=(0, 20))),
    ("dk16_dv64_ragged_tiles", (2, 2, 100, 130, 16, 64), dict(key_lens=(1, 130))),
    ("d16_one_by_one", (1, 1, 1, 1, 16, 16), {}),
    ("dk32_dv64_one_by_one", (2, 1, 1, 1, 32, 64), dict(key_lens=(0, 1))),
    ("d16_four_wave_blocks", (8, 16, 1024, 1024, 16, 16), dict(causal=True)),
    ("dk32_dv64_four_wave_blocks", (8, 16, 1024, 1024, 32, 64), dict(causal=True)),
    # windows and empty key lengths on the sentence-length kernel (n, m <= 64)
    ("dk16_dv64_short_window", (4, 2, 40, 64, 16, 64), dict(window=(5, 3), key_lens=(0, 64))),
    ("dk32_dv64_short_bottom_right", (4, 2, 7, 60, 32, 64), dict(window=(None, 0, "bottom_right"), key_lens=(0, 60))),
    ("d16_short_window_ragged", (3, 4, 50, 50, 16, 16), dict(window=(9, 2), key_lens=(0, 50))),
    ("dk32_dv64_short_right_only", (2, 3, 64, 33, 32, 64), dict(window=(None, 4), key_lens=(1, 33))),
    # row (A)'s single head of 512
    ("A_h1_d512_encoder", (64, 1, 64, 64, 512, 512), dict(key_lens=(8, 64))),
    ("A_d512_decoder", (16, 1, 64, 64, 512, 512), dict(causal=True, key_lens=(8, 64))),
    ("d512_cross", (8, 1, 48, 64, 512, 512), dict(key_lens=(16, 64))),
    ("d512_multi_tile_causal", (2, 2, 300, 300, 512, 512), dict(causal=True)),
    ("d512_window_ragged", (2, 2, 260, 260, 512, 512), dict(window=(40, 8), key_lens=(100, 260))),
    ("d512_bottom_right", (4, 2, 5, 200, 512, 512), dict(window=(None, 0, "bottom_right"), key_lens=(0, 200))),
    ("d512_ragged", (2, 3, 33, 17, 512, 512), dict(key_lens=(0, 20))),
    ("d512_one_by_one", (1, 1, 1, 1, 512, 512), {}),
    # 320 query blocks: one workgroup per block (fewer than 256 blocks split
    # each block's output dims over two workgroups, as in every case above)
    ("d512_many_blocks", (64, 1, 130, 130, 512, 512), dict(key_lens=(8, 130))),
]


def _case(i, shape, opts, seed=8500):
    B, h, n, m, dk, dv = shape
    rng = np.random.default_rng(seed + i)
    opts = dict(opts)
    if isinstance(opts.get("key_lens"), tuple):
        lo, hi = opts["key_lens"]
        opts["key_lens"] = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    return random_case(rng, B, h, n, m, dk, dv, dtype="bf16", **opts)


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_table3_width_parity(gpu_lib, i):
    name, shape, opts = CASES[i]
    c = _case(i, shape, opts)
    _, got = run_gpu(c)
    B, h, n, m, dk, dv = shape
    assert got.shape == (B, h, n, dv)
    if B * h * n * m > 1 << 26:  # large: sampled rows, both sides of every 128-query block edge
        rng = np.random.default_rng(19)
        picks = [(int(rng.integers(B)), int(rng.integers(h)), int(q)) for q in rng.integers(0, n, 64)]
        picks += [(b, hh, q) for b, hh in ((0, 0), (B - 1, h - 1), (3, 7))
                  for e in range(128, n, 128) for q in (e - 1, e)]
        picks += [(0, 0, 0), (B - 1, h - 1, n - 1)]
        ref = so.attention_rows(c["q"], c["k"], c["v"], picks, causal=c["causal"], key_lens=c["key_lens"],
                                window=c["window"])
        got = np.stack([got[b, hh, q] for b, hh, q in picks])
    else:
        ref = so.attention(c["q"], c["k"], c["v"], causal=c["causal"], key_lens=c["key_lens"],
                           window=c["window"])
    err = max_abs_err(got, ref)
    print(f"table3 {name}: max abs err {err:.2e}")
    assert err <= TOL["bf16"]


LSE_CASES = [0, 1, 5, 9, 17, 18, 19, 20, 21, 24, 26]


@pytest.mark.parametrize("i", LSE_CASES, ids=[CASES[i][0] for i in LSE_CASES])
def test_table3_width_lse(gpu_lib, i):
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
    print(f"table3 lse {name}: max abs err {err:.2e}")
    assert err <= 2.0 ** -8


@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 64), (32, 64), (512, 512)])
def test_table3_padded_keys_are_never_read(gpu_lib, dk, dv):
    """NaN and huge values in the K/V rows at or past each key length leave
    the output bitwise unchanged; a head with no legal key gives zero rows."""
    import torch

    rng = np.random.default_rng(95 + dk + dv)
    B, h, n, m = 4, 2, 100, 150
    kl = np.array([m, 9, 0, 99], np.int32)
    c = random_case(rng, B, h, n, m, dk, dv, dtype="bf16", key_lens=kl)
    o1, a = run_gpu(c)
    for b in range(B):
        c["k"][b, :, kl[b]:] = np.nan
        c["v"][b, :, kl[b]:] = 3e38
    o2, got2 = run_gpu(c)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert np.isfinite(got2).all()
    assert np.all(a[2] == 0)


@pytest.mark.parametrize("dk,dv", [(16, 64), (512, 512)])
def test_table3_masked_weights_are_exactly_zero(gpu_lib, dk, dv):
    """m = 64 keys and d_v ≥ m: V = [I | 0] makes the output's first m columns
    the weight matrix itself, and every masked weight must be +0.0 (causal
    and key padding)."""
    rng = np.random.default_rng(96 + dk)
    B, h, n, m = 4, 2, 64, 64
    kl = np.array([64, 17, 1, 40], np.int32)
    c = random_case(rng, B, h, n, m, dk, dv, dtype="bf16", causal=True, key_lens=kl)
    c["v"] = np.zeros_like(c["v"])
    c["v"][:, :, np.arange(m), np.arange(m)] = 1.0
    _, got = run_gpu(c)
    assert np.all(got[..., m:] == 0.0)
    got = got[..., :m]
    j = np.arange(m)
    for b in range(B):
        for i in range(n):
            vis = (j < kl[b]) & (j <= i)
            row = got[b, :, i]
            assert np.all(row[:, ~vis] == 0.0) and not np.signbit(row[:, ~vis]).any()
            assert np.allclose(row.sum(-1), 1.0, atol=4 * TOL["bf16"])
    ref = so.attention(c["q"], c["k"], c["v"], causal=True, key_lens=kl)[..., :m]
    assert max_abs_err(got, ref) <= TOL["bf16"]


@pytest.mark.parametrize("n,m", [(130, 190), (48, 64)], ids=["tiled", "sentence"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (16, 64), (32, 64), (512, 512)])
def test_table3_token_major_matches_packed_bitwise(gpu_lib, dk, dv, n, m):
    """Token-major [B, len, h, d] views of q, k, v and out through
    sdpa_forward_strided: bitwise equal to the packed call, on the tiled
    kernels and on the sentence-length one (n, m ≤ 64)."""
    import torch

    from transformer_attention_sdpa_amd import forward

    rng = np.random.default_rng(97 + dk + dv + n)
    B, h = 3, 4
    c = random_case(rng, B, h, n, m, dk, dv, dtype="bf16", causal=False,
                    key_lens=rng.integers(1, m, size=B, endpoint=True).astype(np.int32))
    q, k, v = (to_device(c[x], "bf16") for x in ("q", "k", "v"))
    kl = torch.from_numpy(c["key_lens"]).cuda()

    def tm(t):
        return t.transpose(1, 2).contiguous().transpose(1, 2)

    packed = forward(q, k, v, key_lens=kl)
    out = tm(torch.empty_like(packed))
    got = forward(tm(q), tm(k), tm(v), key_lens=kl, out=out)
    torch.cuda.synchronize()
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.contiguous().view(torch.int16), packed.view(torch.int16))
    assert max_abs_err(from_device(packed), so.attention(c["q"], c["k"], c["v"], key_lens=c["key_lens"])) <= TOL["bf16"]
