"""sdpa_forward_ex_noalloc against sdpa_forward_ex with a caller's workspace (GPU).

The no-allocation entry point runs the same split-key decoder kernels with the
library's static scratch in place of the workspace, so its output and
log-sum-exp must equal the workspace call's bit for bit.  Two calls in a row,
the second smaller than the first: the scratch keeps the first call's
contents, and the second must read only what its own split launch wrote.
Each call is also held to the bf16 bar against the fp64 oracle.
"""

import numpy as np
import pytest

import oracle.sdpa_oracle as so
from sdpa_inputs import random_case
from tests.gpu_cases import TOL, from_device, max_abs_err, to_device

pytestmark = pytest.mark.gpu

CALLS = [  # B, h, n, m, key lengths
    (2, 8, 4, 8192, [8192, 5003]),
    (1, 8, 1, 2048, None),
]


def test_noalloc_matches_workspace_call_twice(gpu_lib):
    import torch

    from transformer_attention_sdpa_amd import (_lib, sdpa_forward_ex, sdpa_forward_ex_noalloc,
                                                sdpa_forward_workspace_bytes)

    stream = torch.cuda.current_stream().cuda_stream
    for i, (B, h, n, m, kl) in enumerate(CALLS):
        print(f"no-alloc call {i}: B={B} h={h} n={n} m={m} key_lens={kl}", flush=True)
        rng = np.random.default_rng(4200 + i)
        case = random_case(rng, B, h, n, m, 64, 64, dtype="bf16",
                           key_lens=None if kl is None else np.array(kl))
        q, k, v = (to_device(case[x], "bf16") for x in ("q", "k", "v"))
        klt = None if kl is None else torch.tensor(kl, dtype=torch.int32, device="cuda")
        need = sdpa_forward_workspace_bytes(B, h, n, m, 64, 64, _lib.SDPA_BF16)
        assert 0 < need <= _lib.SDPA_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        o_ref = torch.empty_like(q)
        o_got = torch.full_like(q, float("nan"))
        l_ref = torch.empty((B, h, n), dtype=torch.float32, device="cuda")
        l_got = torch.full_like(l_ref, float("nan"))
        # decoder step: n new queries at the end of each sequence's cache, causal
        args = (B, h, n, m, 64, 64, 0.125, -1, 0, _lib.SDPA_ALIGN_BOTTOM_RIGHT,
                None if klt is None else klt.data_ptr(), _lib.SDPA_BF16)
        rc = sdpa_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ref.data_ptr(),
                             l_ref.data_ptr(), *args, ws.data_ptr(), need, stream)
        assert rc == _lib.SDPA_OK, _lib.sdpa_strerror(rc)
        rc = sdpa_forward_ex_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_got.data_ptr(),
                                     l_got.data_ptr(), *args, stream)
        assert rc == _lib.SDPA_OK, _lib.sdpa_strerror(rc)
        torch.cuda.synchronize()
        assert torch.equal(o_got.view(torch.int16), o_ref.view(torch.int16)), i
        assert torch.equal(l_got, l_ref), i
        ref = so.attention(case["q"], case["k"], case["v"], key_lens=case["key_lens"],
                           window=(None, 0, "bottom_right"))
        err = max_abs_err(from_device(o_got), ref)
        print(f"no-alloc call {i}: bitwise equal to the workspace call; max abs err {err:.2e}",
              flush=True)
        assert err <= TOL["bf16"]
