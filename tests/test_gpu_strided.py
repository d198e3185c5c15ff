"""q, k, v and out at other strides than the packed [B, h, len, d] (GPU).

The multi-head section of 《精读 Attention Is All You Need：原始 Transformer
论文》 writes Concat(head_1, …, head_h) token by token, so projections produce
the token-major [B, len, h, d] layout.  ``sdpa_forward_strided`` reads and
writes such layouts in place.  Every forward kernel takes the strides and
runs the same arithmetic, so each strided result must equal the packed call
on the same values bit for bit, and both stay within the bf16 / fp32 bar of
the fp64 oracle.
"""

import numpy as np
import pytest

import oracle.sdpa_oracle as so
from sdpa_inputs import random_case
from tests.gpu_cases import TOL, from_device, max_abs_err, to_device

pytestmark = pytest.mark.gpu

CASES = [  # id, dtype, (B, h, n, m, d), options: every kernel family
    ("bf16_short_d64", "bf16", (4, 8, 64, 64, 64), dict(key_lens=(8, 64))),
    ("bf16_short_d64_causal", "bf16", (3, 4, 64, 64, 64), dict(causal=True, key_lens=(1, 64))),
    ("bf16_short_d32_window", "bf16", (3, 4, 40, 64, 32), dict(window=(None, 0, "bottom_right"), key_lens=(0, 64))),
    ("bf16_short_d128", "bf16", (3, 2, 48, 64, 128), dict(key_lens=(16, 64))),
    ("bf16_long_d64_causal", "bf16", (2, 3, 300, 300, 64), dict(causal=True)),
    ("bf16_long_d64_window", "bf16", (2, 2, 260, 260, 64), dict(window=(40, 8), key_lens=(100, 260))),
    ("bf16_width_d32", "bf16", (2, 3, 200, 150, 32), dict(key_lens=(1, 150))),
    ("bf16_width_d128_causal", "bf16", (2, 2, 130, 130, 128), dict(causal=True)),
    ("bf16_decode", "bf16", (64, 4, 2, 500, 64), dict(window=(None, 0, "bottom_right"), key_lens=(100, 500))),
    ("f32_short", "f32", (3, 4, 64, 64, 64), dict(key_lens=(8, 64))),
    ("f32_long", "f32", (2, 2, 100, 130, 64), dict(key_lens=(1, 130))),
]


def _case(i, dt, shape, opts):
    B, h, n, m, d = shape
    rng = np.random.default_rng(6100 + i)
    opts = dict(opts)
    if isinstance(opts.get("key_lens"), tuple):
        lo, hi = opts["key_lens"]
        opts["key_lens"] = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    return random_case(rng, B, h, n, m, d, d, dtype=dt, **opts)


def _token_major(t):
    """The same values in a [B, len, h, d] buffer, viewed as [B, h, len, d]."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def _run(c, q, k, v, out=None, workspace=None, return_lse=False):
    import torch

    from transformer_attention_sdpa_amd import forward

    kl = None if c["key_lens"] is None else torch.from_numpy(c["key_lens"]).cuda()
    r = forward(q, k, v, causal=c["causal"], key_lens=kl, window=c["window"], out=out,
                workspace=workspace, return_lse=return_lse)
    torch.cuda.synchronize()
    return r


def _bits(t):
    import torch

    return t.contiguous().view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_token_major_layout_matches_packed_bitwise(gpu_lib, i):
    import torch

    name, dt, shape, opts = CASES[i]
    c = _case(i, dt, shape, opts)
    q, k, v = (to_device(c[x], dt) for x in ("q", "k", "v"))
    packed = _run(c, q, k, v, workspace=None)
    qs, ks, vs = _token_major(q), _token_major(k), _token_major(v)
    assert not qs.is_contiguous() or shape[1] == 1
    out = _token_major(torch.empty_like(packed))  # the output written token-major too
    got = _run(c, qs, ks, vs, out=out, workspace=None)
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(_bits(got), _bits(packed)), name
    ref = so.attention(c["q"], c["k"], c["v"], causal=c["causal"], key_lens=c["key_lens"],
                       window=c["window"])
    err = max_abs_err(from_device(got), ref)
    print(f"strided {name}: bitwise equal to the packed call; max abs err {err:.2e}")
    assert err <= TOL[dt]


def test_fused_qkv_buffer_and_lse(gpu_lib):
    """q, k and v as views of one [B, len, 3, h, d] projection output (row
    stride 3·h·d), the output token-major, the log-sum-exp as well."""
    import torch

    B, h, n, d = 4, 8, 200, 64
    rng = np.random.default_rng(6200)
    c = random_case(rng, B, h, n, n, d, d, dtype="bf16", causal=True)
    q, k, v = (to_device(c[x], "bf16") for x in ("q", "k", "v"))
    fused = torch.empty((B, n, 3, h, d), dtype=torch.bfloat16, device="cuda")
    for j, t in enumerate((q, k, v)):
        fused[:, :, j] = t.transpose(1, 2)
    qs, ks, vs = (fused[:, :, j].transpose(1, 2) for j in range(3))
    assert qs.stride() == (n * 3 * h * d, d, 3 * h * d, 1)
    out = torch.empty((B, n, h, d), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o1, l1 = _run(c, q, k, v, return_lse=True)
    o2, l2 = _run(c, qs, ks, vs, out=out, return_lse=True)
    assert torch.equal(_bits(o1), _bits(o2)) and torch.equal(l1, l2)
    assert max_abs_err(from_device(o2), so.attention(c["q"], c["k"], c["v"], causal=True)) <= TOL["bf16"]


def test_one_kv_head_shared_by_all_query_heads(gpu_lib):
    """Head stride 0 on K and V: every query head reads the same K/V head, and
    the result equals the packed call on K/V repeated over the heads."""
    import torch

    B, h, n, m, d = 8, 8, 3, 700, 64
    rng = np.random.default_rng(6300)
    c = random_case(rng, B, 1, n, m, d, d, dtype="bf16", window=(None, 0, "bottom_right"))
    qc = random_case(rng, B, h, n, m, d, d, dtype="bf16")
    q = to_device(qc["q"], "bf16")
    k1, v1 = to_device(c["k"], "bf16"), to_device(c["v"], "bf16")
    ks, vs = k1.expand(B, h, m, d), v1.expand(B, h, m, d)
    assert ks.stride()[1] == 0
    case = {"key_lens": None, "causal": False, "window": (None, 0, "bottom_right")}
    got = _run(case, q, ks, vs)
    want = _run(case, q, ks.contiguous(), vs.contiguous())
    assert torch.equal(_bits(got), _bits(want))
    ref = so.attention(qc["q"], np.repeat(c["k"], h, axis=1), np.repeat(c["v"], h, axis=1),
                       window=(None, 0, "bottom_right"))
    assert max_abs_err(from_device(got), ref) <= TOL["bf16"]


def test_split_decoder_step_token_major(gpu_lib):
    """The split-key decoder path (workspace) with token-major q, k, v and out:
    bitwise equal to the packed call through the same path."""
    import torch

    from transformer_attention_sdpa_amd import sdpa_forward_workspace_bytes

    B, h, n, m, d = 1, 8, 2, 6000, 64
    rng = np.random.default_rng(6400)
    c = random_case(rng, B, h, n, m, d, d, dtype="bf16", window=(None, 0, "bottom_right"))
    q, k, v = (to_device(c[x], "bf16") for x in ("q", "k", "v"))
    need = sdpa_forward_workspace_bytes(B, h, n, m, d, d, 1)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    packed = _run(c, q, k, v, workspace=ws)
    out = _token_major(torch.empty_like(packed))
    got = _run(c, _token_major(q), _token_major(k), _token_major(v), out=out, workspace=ws)
    assert torch.equal(_bits(got), _bits(packed))
    ref = so.attention(c["q"], c["k"], c["v"], window=(None, 0, "bottom_right"))
    assert max_abs_err(from_device(got), ref) <= TOL["bf16"]
