"""Seeded synthetic inputs for scaled dot-product attention.

This module only draws and rounds numbers; it holds none of the attention
arithmetic.  It is the one module that both the CPU oracle's tests and the GPU
path's tests and benchmark use, so that both sides see bit-identical inputs.

Distribution: Q, K and V components are iid N(0, 1).  That is the pages' own
model of query and key components (《Attention Is All You Need：注意力就是你所
需要的一切》 §3.2.1, footnote 4: independent components with mean 0 and
variance 1, so that q·k has mean 0 and variance d_k).  Shapes follow the base
model (h = 8, d_k = d_v = 64, d_model = 512) and the big model (h = 16,
d_k = d_v = 64, d_model = 1024) of Table 3 on the page 《精读 Attention Is All
You Need：原始 Transformer 论文》.  Synthetic N(0, 1) batches stand in for the
pages' WMT 2014 sentence batches, which are not used here.

Draw order for a seed: ``rng = numpy.random.default_rng(seed)`` (PCG64), then
Q, K, V via ``rng.standard_normal(shape, dtype=float32)``, then the per-sequence
key lengths via ``rng.integers(lo, hi, size=B, endpoint=True)``.  bf16 inputs
are the round-to-nearest-even bf16 values of those float32 draws; the arrays
returned here hold exactly the values the device sees (as float32).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "MHA_WORKLOADS", "backward_case", "grad_output", "make_inputs",
           "mha_case", "random_case",
           "round_to_bf16",
           "bf16_bits", "bits_to_f32"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    h: int
    n: int
    m: int
    d_k: int
    d_v: int
    causal: bool
    key_len_range: tuple | None  # inclusive (lo, hi) or None for no padding
    seed: int
    dtypes: tuple = field(default=("bf16",))
    what: str = ""
    window: tuple | None = None  # (left, right[, align]) key window, or None


WORKLOADS = {
    "single_head_16": Workload(
        "single_head_16", B=1, h=1, n=16, m=16, d_k=64, d_v=64, causal=False,
        key_len_range=None, seed=1001, dtypes=("f32",),
        what="one head, 16 queries over 16 keys, no mask"),
    "encoder_self_base": Workload(
        "encoder_self_base", B=64, h=8, n=64, m=64, d_k=64, d_v=64, causal=False,
        key_len_range=(8, 64), seed=1002, dtypes=("f32", "bf16"),
        what="encoder self-attention, base shape, key padding U[8,64]"),
    "decoder_causal_base": Workload(
        "decoder_causal_base", B=64, h=8, n=64, m=64, d_k=64, d_v=64, causal=True,
        key_len_range=(8, 64), seed=1003, dtypes=("bf16",),
        what="decoder masked self-attention, base shape, causal + key padding U[8,64]"),
    "cross_big": Workload(
        "cross_big", B=32, h=16, n=48, m=64, d_k=64, d_v=64, causal=False,
        key_len_range=(16, 64), seed=1004, dtypes=("bf16",),
        what="encoder-decoder cross-attention, big shape, 48 queries over 64 source keys, "
             "source key padding U[16,64]"),
    "long_causal_8k": Workload(
        "long_causal_8k", B=4, h=16, n=8192, m=8192, d_k=64, d_v=64, causal=True,
        key_len_range=None, seed=1005, dtypes=("bf16",),
        what="long-sequence causal self-attention, 8192 tokens, no padding"),
    # Restricted self-attention (《精读 …》 Table 1: each position attends to a
    # neighbourhood of size r around it, for long sequences): r = 513 keys
    # centred on the query, i.e. 256 on either side, on the 8k shape.
    "local_window_8k": Workload(
        "local_window_8k", B=4, h=16, n=8192, m=8192, d_k=64, d_v=64, causal=False,
        key_len_range=None, seed=1006, dtypes=("bf16",), window=(256, 256, "top_left"),
        what="long-sequence restricted self-attention, 8192 tokens, window of 256 keys "
             "either side of each query, no padding"),
    # The model variants' head widths at the base model's cost per layer
    # (h·d = 512; 《精读 …》 Table 3 row (A)): encoder batch as above.
    "encoder_h16_d32": Workload(
        "encoder_h16_d32", B=64, h=16, n=64, m=64, d_k=32, d_v=32, causal=False,
        key_len_range=(8, 64), seed=1009),
    "encoder_h4_d128": Workload(
        "encoder_h4_d128", B=64, h=4, n=64, m=64, d_k=128, d_v=128, causal=False,
        key_len_range=(8, 64), seed=1010),
    # Row (A)'s 32 heads of 16 and single head of 512, and row (B)'s narrow
    # keys (d_k = 16 or 32 against d_v = 64), encoder batch as above.
    "encoder_h32_d16": Workload(
        "encoder_h32_d16", B=64, h=32, n=64, m=64, d_k=16, d_v=16, causal=False,
        key_len_range=(8, 64), seed=1013, dtypes=("bf16",)),
    "encoder_dk16_dv64": Workload(
        "encoder_dk16_dv64", B=64, h=8, n=64, m=64, d_k=16, d_v=64, causal=False,
        key_len_range=(8, 64), seed=1014, dtypes=("bf16",)),
    "encoder_h1_d512": Workload(
        "encoder_h1_d512", B=64, h=1, n=64, m=64, d_k=512, d_v=512, causal=False,
        key_len_range=(8, 64), seed=1016, dtypes=("bf16",)),
    "encoder_dk32_dv64": Workload(
        "encoder_dk32_dv64", B=64, h=8, n=64, m=64, d_k=32, d_v=64, causal=False,
        key_len_range=(8, 64), seed=1015, dtypes=("bf16",)),
    # The 8k causal shape with 128-wide heads (same FLOPs as long_causal_8k).
    "long_causal_8k_d128": Workload(
        "long_causal_8k_d128", B=4, h=8, n=8192, m=8192, d_k=128, d_v=128, causal=True,
        key_len_range=None, seed=1011),
    # One autoregressive decoder step (《注意力就是你所需要的一切》 §3.1: the
    # decoder consumes its previously generated symbols; §6.1: beam search
    # with beam size 4): one new query per sequence against its cached keys,
    # the cache including the new token, so the query sits at the last
    # position (bottom-right aligned causal window).
    "decode_beam_base": Workload(
        "decode_beam_base", B=256, h=8, n=1, m=128, d_k=64, d_v=64, causal=False,
        key_len_range=(16, 128), seed=1007, dtypes=("bf16",), window=(None, 0, "bottom_right"),
        what="decoder self-attention step, base shape, 64 sentences x beam 4, one query "
             "against 16..128 cached keys"),
    "decode_long_cache": Workload(
        "decode_long_cache", B=32, h=8, n=1, m=8192, d_k=64, d_v=64, causal=False,
        key_len_range=(2048, 8192), seed=1008, dtypes=("bf16",), window=(None, 0, "bottom_right"),
        what="decoder self-attention step, base shape, one query against 2048..8192 cached "
             "keys (memory-bound stress case)"),
    "decode_one_sequence": Workload(
        "decode_one_sequence", B=1, h=8, n=1, m=32768, d_k=64, d_v=64, causal=False,
        key_len_range=None, seed=1012, dtypes=("bf16",), window=(None, 0, "bottom_right"),
        what="decoder self-attention step of one sequence alone, base model's 8 heads, one "
             "query against a full 32768-key cache (few heads: the split-key path)"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    return bits_to_f32(bf16_bits(x))


_CHUNK = 1 << 22  # elements per pass: keeps the temporaries small on 10^8-element tensors


def _bf16_bits_flat(u: np.ndarray, out: np.ndarray) -> None:
    # u + 0x7FFF + lsb stays below 2^32 for every non-NaN pattern (the largest,
    # −∞ = 0xFF800000, gains at most 0x8000); NaN patterns are replaced below.
    t = u >> 16
    t &= 1
    t += 0x7FFF
    t += u
    t >>= 16
    out[:] = t
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    if nan.any():
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)  # keep NaNs quiet NaNs


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of float32 ``x`` (round to nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    r = np.empty(u.shape, dtype=np.uint16)
    for i in range(0, u.size, _CHUNK):
        _bf16_bits_flat(u[i:i + _CHUNK], r[i:i + _CHUNK])
    return r.reshape(x.shape)


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """float32 values of uint16 bf16 bit patterns (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    flat = b.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint32)
    for i in range(0, flat.size, _CHUNK):
        o = out[i:i + _CHUNK]
        o[:] = flat[i:i + _CHUNK]
        o <<= 16
    return out.view(np.float32).reshape(b.shape)


def make_inputs(wl: Workload | str, dtype: str | None = None, seed: int | None = None):
    """Draw one batch for workload ``wl``.

    Returns a dict with float32 arrays ``q`` [B,h,n,d_k], ``k`` [B,h,m,d_k],
    ``v`` [B,h,m,d_v] holding exactly the device values (bf16-rounded when
    ``dtype == "bf16"``), ``key_lens`` (int32 [B] or None), ``causal``,
    ``window``, ``dtype`` and the workload.
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    dtype = dtype or wl.dtypes[-1]
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    q = rng.standard_normal((wl.B, wl.h, wl.n, wl.d_k), dtype=np.float32)
    k = rng.standard_normal((wl.B, wl.h, wl.m, wl.d_k), dtype=np.float32)
    v = rng.standard_normal((wl.B, wl.h, wl.m, wl.d_v), dtype=np.float32)
    key_lens = None
    if wl.key_len_range is not None:
        lo, hi = wl.key_len_range
        key_lens = rng.integers(lo, hi, size=wl.B, endpoint=True).astype(np.int32)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return {"q": q, "k": k, "v": v, "key_lens": key_lens, "causal": wl.causal,
            "window": wl.window, "dtype": dtype, "workload": wl}


# Multi-head sublayer workloads (mha_case arguments): the base model's encoder
# self-attention sublayer on the encoder batch, and the big model's
# encoder–decoder sublayer on the cross-attention batch (both models as in
# Table 3 of 《精读 Attention Is All You Need：原始 Transformer 论文》).
MHA_WORKLOADS = {
    "mha_encoder_base": dict(seed=3001, B=64, n=64, m=64, d_model=512, h=8, key_len_range=(8, 64)),
    "mha_cross_big": dict(seed=3002, B=32, n=48, m=64, d_model=1024, h=16, self_attention=False,
                          key_len_range=(16, 64)),
}


def mha_case(seed: int, B, n, m, d_model, h, d=64, self_attention=True, key_len_range=None):
    """Seeded inputs of the multi-head sublayer, bf16-rounded (returned as float32):

    ``xq`` [B, n, d_model] and ``xkv`` [B, m, d_model] (the same array for
    self-attention) with N(0, 1) components; the pages' projection matrices
    ``wq``, ``wk`` [h, d_model, d], ``wv`` [h, d_model, d] and ``wo``
    [h·d, d_model] with N(0, 1/d_model) components, so that the projected
    queries and keys again have unit-variance components; then the key
    lengths.  Draw order: xq, xkv (if separate), wq, wk, wv, wo, key lengths.
    """
    rng = np.random.default_rng(seed)
    xq = rng.standard_normal((B, n, d_model), dtype=np.float32)
    xkv = xq if self_attention else rng.standard_normal((B, m, d_model), dtype=np.float32)
    s = np.float32(1.0 / np.sqrt(d_model))
    wq = rng.standard_normal((h, d_model, d), dtype=np.float32) * s
    wk = rng.standard_normal((h, d_model, d), dtype=np.float32) * s
    wv = rng.standard_normal((h, d_model, d), dtype=np.float32) * s
    wo = rng.standard_normal((h * d, d_model), dtype=np.float32) * s
    key_lens = None
    if key_len_range is not None:
        lo, hi = key_len_range
        key_lens = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    r = round_to_bf16
    xq_r = r(xq)
    return {"xq": xq_r, "xkv": xq_r if self_attention else r(xkv), "wq": r(wq), "wk": r(wk),
            "wv": r(wv), "wo": r(wo), "key_lens": key_lens, "heads": h}


def grad_output(wl: Workload, dtype: str = "bf16") -> np.ndarray:
    """Seeded upstream gradient dO [B, h, n, d_v] for a workload's backward
    pass: N(0, 1) components from ``default_rng(seed + 10000)``, bf16-rounded
    for bf16 (the gradient of a loss Σ dO ∘ O)."""
    rng = np.random.default_rng(wl.seed + 10000)
    do = rng.standard_normal((wl.B, wl.h, wl.n, wl.d_v), dtype=np.float32)
    return round_to_bf16(do) if dtype == "bf16" else do


def backward_case(seed: int, B, h, n, m, causal=False, key_lens=None, window=None, dtype="bf16", d=64):
    """Free-shape case for the backward pass: ``random_case`` (q, k, v with
    d_k = d_v = d) from ``default_rng(seed)``, then dO [B, h, n, d] from the
    same generator, all N(0, 1) (bf16-rounded for dtype "bf16", fp32 as drawn
    for "f32")."""
    rng = np.random.default_rng(seed)
    c = random_case(rng, B, h, n, m, d, d, dtype=dtype, causal=causal, key_lens=key_lens,
                    window=window)
    do = rng.standard_normal((B, h, n, d), dtype=np.float32)
    c["do"] = round_to_bf16(do) if dtype == "bf16" else do
    return c


def random_case(rng: np.random.Generator, B, h, n, m, d_k, d_v, dtype="f32", causal=False,
                key_lens=None, window=None):
    """Free-shape N(0,1) case from an existing generator (for parity sweeps)."""
    q = rng.standard_normal((B, h, n, d_k), dtype=np.float32)
    k = rng.standard_normal((B, h, m, d_k), dtype=np.float32)
    v = rng.standard_normal((B, h, m, d_v), dtype=np.float32)
    if dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    kl = None if key_lens is None else np.asarray(key_lens, dtype=np.int32)
    return {"q": q, "k": k, "v": v, "key_lens": kl, "causal": causal, "window": window,
            "dtype": dtype}


def random_keep(rng: np.random.Generator, B, h, n, m, p: float):
    """Attention-dropout draw: bool [B, h, n, m], each entry True (kept) with
    probability 1 − p, independently."""
    return rng.random((B, h, n, m)) >= p


def pack_keep(keep) -> np.ndarray:
    """The keep mask in the layout the GPU path reads: uint32 [B, h, n, ⌈m/32⌉],
    bit (j mod 32) of word ⌊j/32⌋ for key j; bits past m are 0."""
    keep = np.asarray(keep, dtype=bool)
    m = keep.shape[-1]
    W = (m + 31) // 32
    padded = np.zeros(keep.shape[:-1] + (W * 32,), dtype=np.uint64)
    padded[..., :m] = keep
    weights = np.left_shift(np.uint64(1), np.arange(32, dtype=np.uint64))
    return (padded.reshape(keep.shape[:-1] + (W, 32)) * weights).sum(-1).astype(np.uint32)
