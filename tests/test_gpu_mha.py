"""The multi-head attention sublayer on the GPU against the fp64 oracle.

MultiHead = Concat(head_1..head_h) W^O, head_i = Attention(Q W_i^Q, K W_i^K,
V W_i^V) (the close-reading page's multi-head section; the translation's
§3.2.2).  The GPU path runs through the C ABI (``sdpa_mha_forward``).  The
oracle receives exactly the bf16 values the device sees, in fp64, and keeps
every intermediate unrounded.  The device also rounds Q, K, V, the weights P
and the head outputs to bf16, so the bar is the bf16 one (2e-2 absolute).
"""

import numpy as np
import pytest

import oracle.sdpa_oracle as so
from sdpa_inputs import bf16_bits, mha_case
from tests.gpu_cases import TOL, from_device, max_abs_err

pytestmark = pytest.mark.gpu


def _bf16(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bf16_bits(x)).view(np.int16)).cuda().view(torch.bfloat16)


def run_mha(c, **kw):
    """Marshal the pages' per-head matrices into the [out, in] layout and call the sublayer."""
    import torch

    from transformer_attention_sdpa_amd import mha_forward

    h, d_model, d = c["wq"].shape
    to_rows = lambda w: np.ascontiguousarray(w.transpose(0, 2, 1).reshape(h * d, d_model))
    xq = _bf16(c["xq"])
    xkv = xq if c["xkv"] is c["xq"] else _bf16(c["xkv"])
    kl = None if c["key_lens"] is None else torch.from_numpy(c["key_lens"]).cuda()
    out = mha_forward(xq, xkv, _bf16(to_rows(c["wq"])), _bf16(to_rows(c["wk"])),
                      _bf16(to_rows(c["wv"])), _bf16(np.ascontiguousarray(c["wo"].T)),
                      heads=h, key_lens=kl, **kw)
    torch.cuda.synchronize()
    return from_device(out)


CASES = [  # id, mha_case arguments, attention options
    ("encoder_base", dict(seed=2001, B=64, n=64, m=64, d_model=512, h=8, key_len_range=(8, 64)), {}),
    ("decoder_base_causal", dict(seed=2002, B=64, n=64, m=64, d_model=512, h=8, key_len_range=(8, 64)),
     dict(causal=True)),
    ("cross_big", dict(seed=2003, B=32, n=48, m=64, d_model=1024, h=16, self_attention=False,
                       key_len_range=(16, 64)), {}),
    ("ragged_cross", dict(seed=2004, B=3, n=50, m=70, d_model=128, h=2, self_attention=False,
                          key_len_range=(1, 70)), {}),
    ("long_window", dict(seed=2005, B=2, n=300, m=300, d_model=192, h=3), dict(window=(20, 5))),
    ("decode_step", dict(seed=2006, B=32, n=1, m=200, d_model=512, h=8, self_attention=False,
                         key_len_range=(1, 200)), dict(window=(None, 0, "bottom_right"))),
    # the model variants' head widths (《精读 …》 Table 3 rows (A) and (C))
    ("A_h16_d32", dict(seed=2011, B=16, n=64, m=64, d_model=512, h=16, d=32, key_len_range=(8, 64)), {}),
    ("A_h4_d128_causal", dict(seed=2012, B=16, n=64, m=64, d_model=512, h=4, d=128,
                              key_len_range=(8, 64)), dict(causal=True)),
    ("C_dmodel256_d32_cross", dict(seed=2013, B=8, n=48, m=64, d_model=256, h=8, d=32,
                                   self_attention=False, key_len_range=(1, 64)), {}),
    ("C_dmodel1024_d128_window", dict(seed=2014, B=4, n=100, m=100, d_model=1024, h=8, d=128),
     dict(window=(20, 5))),
]


@pytest.mark.parametrize("name,args,opts", CASES, ids=[c[0] for c in CASES])
def test_mha_parity(gpu_lib, name, args, opts):
    c = mha_case(**args)
    got = run_mha(c, **opts)
    ref = so.multihead(c["xq"], c["xkv"], c["wq"], c["wk"], c["wv"], c["wo"], key_lens=c["key_lens"],
                       **opts)
    err = max_abs_err(got, ref)
    print(f"mha {name}: out std {ref.std():.3f}, max abs err {err:.3e}")
    assert err <= TOL["bf16"]


def test_mha_matches_attention_on_projected_inputs(gpu_lib):
    """The sublayer equals its own steps: the projections computed here in
    fp64 from the same bf16 values, rounded to bf16 as the device stores them,
    attention through sdpa_forward, then Concat·W^O.  Checks the layout
    conversions of the two projection launches independently of the oracle's
    end-to-end tolerance."""
    import torch

    from tests.gpu_cases import run_gpu
    from sdpa_inputs import round_to_bf16

    c = mha_case(seed=2007, B=4, n=40, m=40, d_model=128, h=2, key_len_range=(5, 40))
    got = run_mha(c)
    q = round_to_bf16(np.einsum("bnd,hdk->bhnk", c["xq"].astype(np.float64), c["wq"]).astype(np.float32))
    k = round_to_bf16(np.einsum("bnd,hdk->bhnk", c["xkv"].astype(np.float64), c["wk"]).astype(np.float32))
    v = round_to_bf16(np.einsum("bnd,hdk->bhnk", c["xkv"].astype(np.float64), c["wv"]).astype(np.float32))
    _, heads = run_gpu({"q": q, "k": k, "v": v, "key_lens": c["key_lens"], "causal": False,
                        "dtype": "bf16"})
    heads = round_to_bf16(heads.astype(np.float32)).astype(np.float64)
    B, h, n, d = heads.shape
    ref = heads.transpose(0, 2, 1, 3).reshape(B, n, h * d) @ c["wo"].astype(np.float64)
    err = max_abs_err(got, ref)
    # The device rounds the output to bf16 once: half an ulp at the largest
    # magnitude, 2^(e − 8) for |out| in [2^e, 2^(e+1)); plus 1e-3 for the
    # fp32 accumulation order and the occasional Q/K/V value that fp32 and
    # fp64 sums round to neighbouring bf16 values.
    bound = 2.0 ** (np.floor(np.log2(np.abs(ref).max())) - 8) + 1e-3
    print(f"mha vs its own steps: max abs err {err:.3e} (bound {bound:.3e})")
    assert err <= bound


def test_mha_rejects_a_small_workspace(gpu_lib):
    import torch

    from transformer_attention_sdpa_amd import mha_forward

    c = mha_case(seed=2008, B=2, n=8, m=8, d_model=64, h=1)
    x = _bf16(c["xq"])
    w = _bf16(np.ascontiguousarray(c["wq"][0].T))
    with pytest.raises(RuntimeError, match="workspace"):
        mha_forward(x, x, w, w, w, w, heads=1, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
