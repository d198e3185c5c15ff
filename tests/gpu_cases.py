"""Helpers for GPU parity tests: move generator arrays to the device, run the
HIP path through the C ABI, and bring results back as float64.

No expected value is produced here: expected values come from ``oracle/``.
"""

from __future__ import annotations

import numpy as np

from sdpa_inputs import bf16_bits

TOL = {"f32": 1e-5, "bf16": 2e-2}  # max abs error against the fp64 oracle


def to_device(x: np.ndarray, dtype: str):
    import torch

    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    bits = bf16_bits(x).view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(bits)).cuda().view(torch.bfloat16)


def from_device(t) -> np.ndarray:
    import torch

    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def run_gpu(case: dict, scale=None, out=None, workspace=None):
    """Run the HIP path on a generator case; returns (device out tensor, float64 numpy).

    Without a workspace (the default here) the call goes through
    ``sdpa_forward`` / ``sdpa_forward_window``; ``workspace="auto"`` is the
    binding's own default."""
    import torch

    from transformer_attention_sdpa_amd import forward

    dt = case["dtype"]
    q, k, v = (to_device(case[x], dt) for x in ("q", "k", "v"))
    kl = None
    if case.get("key_lens") is not None:
        kl = torch.from_numpy(np.asarray(case["key_lens"], dtype=np.int32)).cuda()
    o = forward(q, k, v, causal=case.get("causal", False), key_lens=kl, scale=scale, out=out,
                window=case.get("window"), workspace=workspace)
    torch.cuda.synchronize()
    return o, from_device(o)


def max_abs_err(a, b) -> float:
    d = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    return float(d.max()) if d.size else 0.0
