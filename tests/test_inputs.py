"""The seeded input generator (CPU only)."""

import numpy as np
import pytest
import torch

from sdpa_inputs import WORKLOADS, bf16_bits, make_inputs, round_to_bf16


def test_same_seed_same_bytes():
    a = make_inputs("encoder_self_base", "bf16")
    b = make_inputs("encoder_self_base", "bf16")
    for key in ("q", "k", "v", "key_lens"):
        assert np.array_equal(a[key], b[key])
    c = make_inputs("encoder_self_base", "bf16", seed=5)
    assert not np.array_equal(a["q"], c["q"])


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * s for s in (1e-3, 1, 1e3)])
    x = np.concatenate([x, np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(x), ref)
    y = round_to_bf16(x)
    assert np.array_equal(torch.from_numpy(y).to(torch.bfloat16).float().numpy(), y)


@pytest.mark.parametrize("name", ["encoder_self_base", "decoder_causal_base", "cross_big"])
def test_key_lengths_in_range(name):
    wl = WORKLOADS[name]
    kl = make_inputs(name)["key_lens"]
    lo, hi = wl.key_len_range
    assert kl.dtype == np.int32 and kl.shape == (wl.B,)
    assert kl.min() >= lo and kl.max() <= hi


def test_shapes_follow_the_workloads():
    for name, wl in WORKLOADS.items():
        if wl.n * wl.m > 64 * 64:
            continue
        x = make_inputs(name)
        assert x["q"].shape == (wl.B, wl.h, wl.n, wl.d_k)
        assert x["k"].shape == (wl.B, wl.h, wl.m, wl.d_k)
        assert x["v"].shape == (wl.B, wl.h, wl.m, wl.d_v)


def test_dot_product_variance_is_dk():
    """Footnote 4 of §3.2.1: unit-variance independent components ⇒ Var(q·k) = d_k."""
    x = make_inputs("encoder_self_base", "f32")
    q, k = x["q"].astype(np.float64), x["k"].astype(np.float64)
    dots = np.einsum("bhid,bhid->bhi", q, k).ravel()
    assert abs(dots.mean()) < 0.1
    assert abs(dots.var() / 64.0 - 1.0) < 0.02
    scaled = dots / 8.0
    assert abs(scaled.var() - 1.0) < 0.02
