"""The largest heads the library accepts, on the GPU.

One head's K or V rows must span less than 2^31 bytes (the kernels address a
head with 32-bit byte offsets): m = 2^24 − 1 keys at width 64 in bf16, 2^23 − 1
at width 128 in bf16 or width 64 in fp32.  These cases put m at that maximum.

Expected values come from two properties of Eq. (1) (《注意力就是你所需要的一切》
§3.2.1), each exact in real arithmetic:
  * repetition: the first R·P keys are one random block of P rows repeated R
    times, so the copies of a key share one weight; together they weigh R times
    the block, and their weighted values are R times the block's;
  * disjoint union: softmax over two key sets merges from each set's output o
    and log-sum-exp λ as (e^λ₁·o₁ + e^λ₂·o₂) / (e^λ₁ + e^λ₂).
The last T legal keys (the highest offsets the kernels address) repeat the
block's first T keys with every value C = 2^16 (scaled down for more marker
rows), which moves the output by about
0.2 to 0.8, far above the bar, so a kernel that failed to read them fails.
With a key length below m, the rows past it hold NaN: reading any of them
would show.  Without key lengths (L = m) the markers end at the very last row,
so the highest addresses (just under 2^31 bytes into the head) are exercised,
as are the loads the split decoder path issues one step past that.  The
oracle computes o and λ of the block and of the marker rows (fp64).

Bar: the usual one for every dtype (2e-2 absolute for bf16, 1e-5 for fp32).
The fp32 kernel adds each 32-key tile into its running output and weight sum
with Kahan compensation, so its error does not grow with the key count.
"""

import math

import numpy as np
import pytest

import oracle.sdpa_backward as sb
import oracle.sdpa_oracle as so
from sdpa_inputs import random_case
from tests.gpu_cases import TOL, from_device, max_abs_err, to_device

pytestmark = pytest.mark.gpu

P = 4096       # rows of the repeated block
T = 64         # marker rows after the repeats
C = 65536.0    # marker value (exact in bf16)

CASES = [  # id, dtype, n, d, m, path, key length below m
    ("bf16_d64_one_query", "bf16", 1, 64, (1 << 24) - 1, "plain", True),  # one head: long kernel
    ("bf16_d64_decoder_split", "bf16", 3, 64, (1 << 24) - 1, "split", True),  # 16384 pieces
    ("bf16_d64_long", "bf16", 100, 64, (1 << 24) - 1, "plain", True),
    ("bf16_d128_width", "bf16", 40, 128, (1 << 23) - 1, "plain", True),
    ("f32_d64_long", "f32", 70, 64, (1 << 23) - 1, "plain", True),
    ("bf16_d64_decoder_split_full", "bf16", 3, 64, (1 << 24) - 1, "split", False),
    ("bf16_d64_long_full", "bf16", 100, 64, (1 << 24) - 1, "plain", False),
    ("f32_d64_long_full", "f32", 33, 64, (1 << 23) - 1, "plain", False),
]


def marker_value(t):
    """C for T marker rows, scaled down (by a power of two, exact in bf16) for
    t markers, so that they move the output by a similar amount."""
    return C * 2.0 ** round(math.log2(T / t))


def expected(c, R, t):
    """Output over R copies of the block followed by t marker rows."""
    o_b = so.attention(c["q"], c["k"], c["v"])
    lam_b = sb.log_sum_exp(c["q"], c["k"]) + math.log(R)
    lam_m = sb.log_sum_exp(c["q"], c["k"][:, :, :t])
    rho = np.exp(lam_m - lam_b)[..., None]  # marker weight / repeated-block weight
    return (o_b + rho * marker_value(t)) / (1.0 + rho)


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_largest_head(gpu_lib, i):
    import torch

    from transformer_attention_sdpa_amd import forward, sdpa_forward_workspace_bytes

    name, dt, n, d, m, path, padded = CASES[i]
    c = random_case(np.random.default_rng(9500 + i), 1, 1, n, P, d, d, dtype=dt)
    R = (m - T) // P
    t = T if padded else m - R * P  # without padding the markers run to the last row
    assert T <= t <= P
    L = R * P + t
    print(f"max size {name}: n={n} m={m} d={d} key length {L}", flush=True)
    q = to_device(c["q"], dt)
    kb, vb = to_device(c["k"], dt)[0, 0], to_device(c["v"], dt)[0, 0]
    k = torch.empty((1, 1, m, d), dtype=q.dtype, device="cuda")
    v = torch.empty_like(k)
    k[0, 0, :R * P] = kb.repeat(R, 1)
    v[0, 0, :R * P] = vb.repeat(R, 1)
    k[0, 0, R * P:L] = kb[:t]
    v[0, 0, R * P:L] = marker_value(t)
    k[0, 0, L:] = float("nan")
    v[0, 0, L:] = float("nan")
    kl = torch.tensor([L], dtype=torch.int32, device="cuda") if padded else None
    ws = None
    if path == "split":
        need = sdpa_forward_workspace_bytes(1, 1, n, m, d, d, 1)
        assert need > 0
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = forward(q, k, v, key_lens=kl, workspace=ws)
    torch.cuda.synchronize()
    got = from_device(out)
    del k, v
    ref = expected(c, R, t)
    err = max_abs_err(got, ref)
    tol = TOL[dt]
    shift = float(np.abs(ref - so.attention(c["q"], c["k"], c["v"])).max())
    print(f"max size {name}: max abs err {err:.2e} (bar {tol:.1e}; the markers move the output by {shift:.2f})")
    assert shift > 5 * tol
    assert np.all(np.isfinite(got)) and err <= tol
