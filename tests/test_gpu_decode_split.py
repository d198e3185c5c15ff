"""Decoder steps with a workspace: each head's keys split over several
workgroups, then merged (``sdpa_forward_ex``), against the fp64 oracle.

A decoder step asks a few new queries against the cached keys of its
sequence (《注意力就是你所需要的一切》 §3.1: the decoder consumes its own
earlier outputs), bottom-right aligned.  With ragged cache lengths one
workgroup per head leaves CUs idle; the split path gives every piece of keys
its own workgroup; with few heads (one sequence decoding alone) it is the
only path that spreads a head over several CUs.  Bar: bf16, 2e-2 absolute; the log-sum-exp within 2^-8;
the split and unsplit paths agree within the same bar.
"""

import numpy as np
import pytest

import oracle.sdpa_backward as sb
import oracle.sdpa_oracle as so
from sdpa_inputs import WORKLOADS, make_inputs, random_case
from tests.gpu_cases import TOL, from_device, max_abs_err, to_device

pytestmark = pytest.mark.gpu

BR = (None, 0, "bottom_right")
CASES = [  # id, (B, h, n, m), key lengths, window
    ("ragged_1q", (32, 8, 1, 3000), (1, 3000), BR),
    ("ragged_16q", (32, 8, 16, 2500), (1, 2500), BR),
    ("window_100", (32, 8, 4, 4100), (0, 4100), (100, 0, "bottom_right")),
    ("two_splits_exactly", (32, 8, 2, 2048), None, BR),
    ("full_no_mask", (16, 16, 3, 1500), (1500, 1500), None),
    # fewer than 256 heads: without a workspace the long kernel serves these
    ("one_sequence_8_heads", (1, 8, 1, 20000), (20000, 20000), BR),
    ("one_head_16q_ragged_tail", (1, 1, 16, 5000), (4321, 4321), BR),
    ("two_sequences_window", (2, 4, 2, 9000), (3000, 9000), (500, 0, "bottom_right")),
    ("one_sequence_short_cache", (1, 8, 5, 700), (300, 700), BR),  # 256-key pieces
]


def _case(i):
    name, (B, h, n, m), kl, win = CASES[i]
    rng = np.random.default_rng(9100 + i)
    key_lens = None
    if kl is not None:
        key_lens = rng.integers(kl[0], kl[1], size=B, endpoint=True).astype(np.int32)
        if kl[0] <= 1:
            key_lens[:3] = [0, 1, 5]  # empty, one key, a few keys: most splits empty
    return random_case(rng, B, h, n, m, 64, 64, dtype="bf16", key_lens=key_lens, window=win)


def _run(c, workspace: bool, lse=False):
    import torch

    from transformer_attention_sdpa_amd import forward, sdpa_forward_workspace_bytes

    q, k, v = (to_device(c[x], "bf16") for x in ("q", "k", "v"))
    B, h, n, _ = c["q"].shape
    m = c["k"].shape[2]
    kl = None if c["key_lens"] is None else torch.from_numpy(c["key_lens"]).cuda()
    ws = None
    if workspace:
        need = sdpa_forward_workspace_bytes(B, h, n, m, 64, 64, 1)
        assert need > 0, "the split path should apply to this shape"
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    r = forward(q, k, v, key_lens=kl, window=c["window"], workspace=ws, return_lse=lse)
    torch.cuda.synchronize()
    if lse:
        return from_device(r[0]), r[1].cpu().numpy().astype(np.float64)
    return from_device(r)


@pytest.mark.parametrize("i", range(len(CASES)), ids=[c[0] for c in CASES])
def test_split_decode_parity(gpu_lib, i):
    c = _case(i)
    got, lse = _run(c, True, lse=True)
    ref = so.attention(c["q"], c["k"], c["v"], key_lens=c["key_lens"], window=c["window"])
    err = max_abs_err(got, ref)
    plain = _run(c, False)
    gap = max_abs_err(got, plain)
    lref = sb.log_sum_exp(c["q"], c["k"], key_lens=c["key_lens"], window=c["window"])
    inf = np.isinf(lref)
    assert np.array_equal(np.isinf(lse), inf) and np.all(lse[inf] == lref[inf])
    lerr = max_abs_err(lse[~inf], lref[~inf])
    print(f"split {CASES[i][0]}: max abs err {err:.2e}, vs unsplit {gap:.2e}, lse {lerr:.2e}")
    assert err <= TOL["bf16"] and gap <= TOL["bf16"] and lerr <= 2.0 ** -8


def test_split_decode_long_cache_workload(gpu_lib):
    """The decode_long_cache workload (B = 32, h = 8, one query against
    2048–8192 cached keys) through the split path, every output row checked."""
    wl = WORKLOADS["decode_long_cache"]
    c = make_inputs(wl, "bf16")
    got = _run(c, True)
    ref = so.attention(c["q"], c["k"], c["v"], key_lens=c["key_lens"], window=wl.window)
    err = max_abs_err(got, ref)
    print(f"split decode_long_cache: max abs err {err:.2e}")
    assert err <= TOL["bf16"]


def test_split_decode_one_sequence_workload(gpu_lib):
    """The decode_one_sequence workload (one sequence, 8 heads, one query
    against a full 32768-key cache) through the split path, every row checked."""
    wl = WORKLOADS["decode_one_sequence"]
    c = make_inputs(wl, "bf16")
    got = _run(c, True)
    ref = so.attention(c["q"], c["k"], c["v"], key_lens=c["key_lens"], window=wl.window)
    err = max_abs_err(got, ref)
    print(f"split decode_one_sequence: max abs err {err:.2e}")
    assert err <= TOL["bf16"]


def test_split_decode_deterministic(gpu_lib):
    c = _case(1)
    a = _run(c, True)
    b = _run(c, True)
    assert np.array_equal(a, b)


def test_auto_workspace_splits_only_for_few_heads(gpu_lib):
    """forward()'s default workspace="auto" takes the split path below 256
    heads (bit-identical to an explicit workspace) and the unsplit one from
    256 heads on (bit-identical to no workspace)."""
    import torch

    from transformer_attention_sdpa_amd import forward

    for i in (5, 0):  # 8 heads, then 256 heads
        c = _case(i)
        q, k, v = (to_device(c[x], "bf16") for x in ("q", "k", "v"))
        kl = torch.from_numpy(c["key_lens"]).cuda()
        auto = forward(q, k, v, key_lens=kl, window=c["window"])
        torch.cuda.synchronize()
        split = _run(c, True)
        plain = _run(c, False)
        B, h = c["q"].shape[:2]
        want = split if B * h < 256 else plain
        assert np.array_equal(from_device(auto), want), CASES[i][0]

