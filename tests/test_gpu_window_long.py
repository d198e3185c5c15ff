"""Windows bounded on both sides on long sequences with many query blocks
(bf16, GPU).

Restricted self-attention (《精读 Attention Is All You Need：原始 Transformer
论文》 Table 1) gives each query a band of keys around its position; every
query row is an independent softmax over its band (Eq. (1)).  Such windows
run 2-wave workgroups over 128-query blocks.  These launches have more than
1024 query blocks and cover block boundaries, blocks whose queries see no key
(leading, trailing and between others), odd tile counts, bottom-right
alignment, the log-sum-exp output and token-major strides.  A head's result
must not depend on the rest of the launch: the same heads run alone give
bitwise the same outputs.
"""

import numpy as np
import pytest

import oracle.sdpa_oracle as so
from sdpa_inputs import random_case
from tests.gpu_cases import TOL, from_device, max_abs_err, to_device

pytestmark = pytest.mark.gpu

# (B, h, n, m, window, key_lens): each has B·h·⌈n/128⌉ > 1024 query blocks
CASES = [
    ("band_100_20_padded", (4, 8, 4500, 4500, (100, 20, "top_left"), [4500, 1000, 0, 2345])),
    ("band_256_256", (2, 16, 4160, 4160, (256, 256, "top_left"), None)),
    ("bottom_right_300_0", (2, 16, 4500, 5000, (300, 0, "bottom_right"), [5000, 4321])),
    ("narrow_band_ragged", (3, 12, 3900, 3999, (7, 3, "top_left"), [3999, 17, 2000])),
]


def _case(i):
    name, (B, h, n, m, win, kl) = CASES[i]
    rng = np.random.default_rng(7700 + i)
    c = random_case(rng, B, h, n, m, 64, 64, dtype="bf16",
                    key_lens=None if kl is None else np.array(kl, np.int32))
    c["window"] = win
    return c


def _forward(c, q=None, k=None, v=None, out=None, return_lse=False):
    import torch

    from transformer_attention_sdpa_amd import forward

    q = to_device(c["q"], "bf16") if q is None else q
    k = to_device(c["k"], "bf16") if k is None else k
    v = to_device(c["v"], "bf16") if v is None else v
    kl = None if c["key_lens"] is None else torch.from_numpy(np.asarray(c["key_lens"], np.int32)).cuda()
    r = forward(q, k, v, key_lens=kl, window=c["window"], out=out, workspace=None, return_lse=return_lse)
    torch.cuda.synchronize()
    return r


def _rows(n, rng):
    """Both sides of every 128-query block boundary, the first and last rows,
    and a few random rows."""
    rows = {0, 1, n - 1}
    for e in range(128, n, 128):
        rows |= {e - 1, e}
    rows |= {int(x) for x in rng.choice(n, 4, replace=False)}
    return sorted(rows)


def _band(i, n, L, win):
    left, right, align = win
    c = i if align == "top_left" else i + L - n
    lo = 0 if left is None else max(0, c - left)
    hi = L if right is None else min(L, c + right + 1)
    return lo, hi


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_window_parity_on_block_edges(gpu_lib, i):
    c = _case(i)
    B, h, n, m, win, kl = CASES[i][1]
    assert B * h * -(-n // 128) > 1024
    got = from_device(_forward(c))
    rng = np.random.default_rng(77 + i)
    picks = []
    for b in range(B):
        for hh in sorted({0, h - 1, int(rng.integers(h))}):
            picks += [(b, hh, q) for q in _rows(n, rng)]
    ref = so.attention_rows(c["q"], c["k"], c["v"], picks, key_lens=c["key_lens"], window=win)
    err = max_abs_err(np.stack([got[p] for p in picks]), ref)
    print(f"window {CASES[i][0]}: {len(picks)} rows, max abs err {err:.2e}")
    assert err <= TOL["bf16"]
    # every row whose band is empty is exactly zero, in every head
    for b in range(B):
        L = m if kl is None else min(kl[b], m)
        empty = [q for q in range(n) if _band(q, n, L, win)[1] <= _band(q, n, L, win)[0]]
        if empty:
            assert np.all(got[b][:, empty] == 0.0)


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_window_heads_match_when_run_alone(gpu_lib, i):
    """Each batch element alone (a launch of fewer blocks) gives bitwise the
    outputs and log-sum-exps of the whole batch."""
    import torch

    c = _case(i)
    B = CASES[i][1][0]
    o_all, l_all = _forward(c, return_lse=True)
    for b in range(B):
        cb = dict(c, q=c["q"][b:b + 1], k=c["k"][b:b + 1], v=c["v"][b:b + 1],
                  key_lens=None if c["key_lens"] is None else c["key_lens"][b:b + 1])
        o_b, l_b = _forward(cb, return_lse=True)
        assert torch.equal(o_b[0].view(torch.int16), o_all[b].view(torch.int16)), b
        assert torch.equal(l_b[0], l_all[b]), b


def test_window_token_major_bitwise(gpu_lib):
    """Token-major q, k, v and out views: bitwise the packed call."""
    import torch

    c = _case(1)
    q, k, v = (to_device(c[x], "bf16") for x in ("q", "k", "v"))

    def tm(t):
        return t.transpose(1, 2).contiguous().transpose(1, 2)

    packed = _forward(c, q, k, v)
    out = tm(torch.empty_like(packed))
    got = _forward(c, tm(q), tm(k), tm(v), out=out)
    assert got.data_ptr() == out.data_ptr()
    assert torch.equal(got.contiguous().view(torch.int16), packed.view(torch.int16))
