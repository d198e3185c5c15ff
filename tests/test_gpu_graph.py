"""The library under HIP graph capture.

Every entry point only launches kernels on the caller's stream (no
allocation, no memset, no synchronisation), so a forward with its
log-sum-exp, the backward on it, the same two with attention dropout (a keep
mask copied in with the inputs), a split decoder step and the projected
sublayer can be captured into one graph and replayed.  Each replay gets new
inputs copied into the captured buffers, with eager work and a
synchronisation between replays, and must reproduce the eager call on the
same inputs bit for bit; the first replay's forward is also checked against
the fp64 oracle (Eq. (1) of 《注意力就是你所需要的一切》 §3.2.1).
"""

import numpy as np
import pytest

import oracle.sdpa_oracle as so
from sdpa_inputs import bf16_bits, mha_case, pack_keep, random_case, random_keep, round_to_bf16
from tests.gpu_cases import TOL, from_device, max_abs_err

pytestmark = pytest.mark.gpu

ENC = (64, 8, 64, 64)  # B, h, n, m: the base model's sentence-length self-attention
DEC = (32, 8, 1, 3000)  # one query against ragged caches: the split decoder path


def _bits(x):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bf16_bits(x)).view(np.int16)).view(torch.bfloat16)


def _inputs(seed):
    """Host tensors for one replay: encoder q/k/v/dout/key_lens, decoder q/k/v/key_lens, sublayer x."""
    import torch

    rng = np.random.default_rng(seed)
    B, h, n, m = ENC
    enc = random_case(rng, B, h, n, m, 64, 64, dtype="bf16",
                      key_lens=rng.integers(8, m, size=B, endpoint=True).astype(np.int32))
    dout = round_to_bf16(rng.standard_normal((B, h, n, 64), dtype=np.float32))
    B2, h2, n2, m2 = DEC
    kl2 = rng.integers(1, m2, size=B2, endpoint=True).astype(np.int32)
    kl2[:2] = [0, 1]
    dec = random_case(rng, B2, h2, n2, m2, 64, 64, dtype="bf16", key_lens=kl2,
                      window=(None, 0, "bottom_right"))
    x = round_to_bf16(rng.standard_normal((8, 64, 512), dtype=np.float32))
    host = {f"enc_{t}": _bits(enc[t]) for t in ("q", "k", "v")}
    host["enc_do"] = _bits(dout)
    host["enc_kl"] = torch.from_numpy(enc["key_lens"])
    host["enc_keep"] = torch.from_numpy(pack_keep(random_keep(rng, B, h, n, m, 0.2)).view(np.int32))
    host.update({f"dec_{t}": _bits(dec[t]) for t in ("q", "k", "v")})
    host["dec_kl"] = torch.from_numpy(dec["key_lens"])
    host["x"] = _bits(x)
    return host, enc


def _pipeline(s, w, ws_dec, ws_mha):
    """One pass over the six calls on the current stream; returns the outputs."""
    from transformer_attention_sdpa_amd import backward, backward_dropout, forward, forward_dropout, mha_forward

    out, lse = forward(s["enc_q"], s["enc_k"], s["enc_v"], key_lens=s["enc_kl"], return_lse=True)
    dq, dk, dv = backward(s["enc_q"], s["enc_k"], s["enc_v"], out, s["enc_do"], lse, key_lens=s["enc_kl"])
    o_d, l_d = forward_dropout(s["enc_q"], s["enc_k"], s["enc_v"], s["enc_keep"], 1.25, key_lens=s["enc_kl"],
                               return_lse=True)
    g_d = backward_dropout(s["enc_q"], s["enc_k"], s["enc_v"], o_d, s["enc_do"], l_d, s["enc_keep"], 1.25,
                           key_lens=s["enc_kl"])
    dec = forward(s["dec_q"], s["dec_k"], s["dec_v"], key_lens=s["dec_kl"], window=(None, 0, "bottom_right"),
                  workspace=ws_dec)
    y = mha_forward(s["x"], s["x"], *w, heads=8, workspace=ws_mha)
    return [out, lse, dq, dk, dv, o_d, l_d, *g_d, dec, y]


def test_graph_replays_match_eager(gpu_lib):
    import torch

    from transformer_attention_sdpa_amd import sdpa_forward_workspace_bytes, sdpa_mha_workspace_bytes

    host, _ = _inputs(7000)
    s = {k: t.cuda() for k, t in host.items()}
    c = mha_case(7100, 8, 64, 64, 512, 8)
    to_rows = lambda a: np.ascontiguousarray(a.transpose(0, 2, 1).reshape(512, 512))
    w = [_bits(to_rows(c[k])).cuda() for k in ("wq", "wk", "wv")] + [_bits(np.ascontiguousarray(c["wo"].T)).cuda()]
    B2, h2, n2, m2 = DEC
    need = sdpa_forward_workspace_bytes(B2, h2, n2, m2, 64, 64, 1)
    assert need > 0
    ws_dec = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws_mha = torch.empty(sdpa_mha_workspace_bytes(8, 64, 64, 8, 64, 64), dtype=torch.uint8, device="cuda")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _pipeline(s, w, ws_dec, ws_mha)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = _pipeline(s, w, ws_dec, ws_mha)
    torch.cuda.synchronize()

    names = ("out", "lse", "dq", "dk", "dv", "dropout out", "dropout lse", "dropout dq", "dropout dk",
             "dropout dv", "decoder", "sublayer")
    for r in range(3):
        host, enc = _inputs(7001 + r)
        for k, t in host.items():
            s[k].copy_(t)
        torch.cuda.synchronize()
        eager = [t.clone() for t in _pipeline(s, w, ws_dec, ws_mha)]
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, captured, eager):
            same = torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                               b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))
            assert same, f"replay {r}: {name} differs from the eager call"
        if r == 0:
            ref = so.attention(enc["q"], enc["k"], enc["v"], key_lens=enc["key_lens"])
            err = max_abs_err(from_device(captured[0]), ref)
            print(f"graph replay forward: max abs err {err:.2e}")
            assert err <= TOL["bf16"]
    print("graph: 3 replays bit-identical to eager")
