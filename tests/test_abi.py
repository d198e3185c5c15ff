"""The C ABI without a GPU: exports, constants and host-side validation.

Every call here fails validation, which happens on the host before any HIP
call, so nothing touches a device.
"""

import ctypes
import math
import os
import re

import pytest

from transformer_attention_sdpa_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sdpa.h")


def _header():
    with open(HEADER, encoding="utf-8") as f:
        return f.read()


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_every_declared_entry_point_is_exported(lib):
    names = re.findall(r"SDPA_API\s+[\w\s\*]+?\b(sdpa_\w+)\s*\(", _header())
    assert set(names) == {"sdpa_forward", "sdpa_forward_window", "sdpa_mha_forward",
                          "sdpa_mha_workspace_bytes", "sdpa_forward_lse", "sdpa_backward",
                          "sdpa_backward_workspace_bytes", "sdpa_forward_ex",
                          "sdpa_forward_ex_noalloc", "sdpa_forward_strided",
                          "sdpa_forward_workspace_bytes", "sdpa_forward_dropout",
                          "sdpa_backward_dropout", "sdpa_strerror", "sdpa_version"}
    for name in names:
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_header_constants_match_binding():
    defs = dict(re.findall(r"#define\s+(SDPA_[A-Z0-9_]+)\s+(-?\d+)", _header()))
    assert defs, "no constants parsed"
    for name, val in defs.items():
        assert getattr(_lib, name) == int(val), name


def test_version_and_strerror(lib):
    assert _lib.sdpa_version() >= 10000
    for code in range(-10, 1):
        msg = _lib.sdpa_strerror(code)
        assert msg and msg != "unknown status"
    assert _lib.sdpa_strerror(-1234) == "unknown status"


P = 1 << 20  # fake, 16-byte aligned "device" addresses; never dereferenced


def call(q=P, k=2 * P, v=3 * P, out=4 * P, B=2, h=2, n=8, m=8, d_k=64, d_v=64, scale=0.125,
         mask=0, key_lens=None, dtype=1):
    return _lib.sdpa_forward(q, k, v, out, B, h, n, m, d_k, d_v, scale, mask, key_lens, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SDPA_ERR_NULL),
    (dict(k=None), _lib.SDPA_ERR_NULL),
    (dict(v=None), _lib.SDPA_ERR_NULL),
    (dict(out=None), _lib.SDPA_ERR_NULL),
    (dict(B=0), _lib.SDPA_ERR_SHAPE),
    (dict(h=-1), _lib.SDPA_ERR_SHAPE),
    (dict(n=0), _lib.SDPA_ERR_SHAPE),
    (dict(m=0), _lib.SDPA_ERR_SHAPE),
    (dict(B=1 << 20, h=1 << 10, n=1 << 20), _lib.SDPA_ERR_SHAPE),
    # one head's rows reach 2^31 bytes (32-bit offsets within a head)
    (dict(B=1, h=1, n=1, m=1 << 24), _lib.SDPA_ERR_SHAPE),
    (dict(B=1, h=1, n=1 << 23, m=8, d_k=128, d_v=128), _lib.SDPA_ERR_SHAPE),
    (dict(B=1, h=1, n=1, m=1 << 23, dtype=0), _lib.SDPA_ERR_SHAPE),
    (dict(d_k=32, d_v=32, dtype=0), _lib.SDPA_ERR_UNSUPPORTED),  # other widths: bf16 only
    (dict(d_k=16, d_v=64, dtype=0), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=8, d_v=8), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=96, d_v=96), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=256, d_v=256), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=512, d_v=64), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=16, d_v=32), _lib.SDPA_ERR_UNSUPPORTED),            # d_k != d_v: only d_v = 64
    (dict(d_k=128, d_v=64), _lib.SDPA_ERR_UNSUPPORTED),           # ... with d_k = 16 or 32
    (dict(d_k=64, d_v=16), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_v=128), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(q=P + 8), _lib.SDPA_ERR_ALIGN),
    (dict(out=4 * P + 2), _lib.SDPA_ERR_ALIGN),
    (dict(key_lens=5 * P + 2), _lib.SDPA_ERR_ALIGN),
    (dict(mask=2), _lib.SDPA_ERR_MASK),
    (dict(mask=1, n=8, m=9), _lib.SDPA_ERR_MASK),
    (dict(dtype=2), _lib.SDPA_ERR_DTYPE),
    (dict(dtype=-1), _lib.SDPA_ERR_DTYPE),
    (dict(scale=math.nan), _lib.SDPA_ERR_SCALE),
    (dict(scale=math.inf), _lib.SDPA_ERR_SCALE),
    (dict(scale=0.0), _lib.SDPA_ERR_SCALE),
    (dict(scale=-0.125), _lib.SDPA_ERR_SCALE),
    (dict(out=P), _lib.SDPA_ERR_ALIAS),
    (dict(out=3 * P + 1024), _lib.SDPA_ERR_ALIAS),
    (dict(key_lens=4 * P + 64), _lib.SDPA_ERR_ALIAS),
])
def test_validation_rejects_before_any_hip_call(kw, code):
    assert call(**kw) == code


def call_window(wl=-1, wr=-1, align=0, **kw):
    args = dict(q=P, k=2 * P, v=3 * P, out=4 * P, B=2, h=2, n=8, m=8, d_k=64, d_v=64, scale=0.125,
                key_lens=None, dtype=1)
    args.update(kw)
    return _lib.sdpa_forward_window(args["q"], args["k"], args["v"], args["out"], args["B"],
                                    args["h"], args["n"], args["m"], args["d_k"], args["d_v"],
                                    args["scale"], wl, wr, align, args["key_lens"], args["dtype"],
                                    None)


@pytest.mark.parametrize("kw,code", [
    (dict(wl=-2), _lib.SDPA_ERR_MASK),
    (dict(wr=-7), _lib.SDPA_ERR_MASK),
    (dict(align=2), _lib.SDPA_ERR_MASK),
    (dict(align=-1), _lib.SDPA_ERR_MASK),
    (dict(q=None), _lib.SDPA_ERR_NULL),
    (dict(n=0), _lib.SDPA_ERR_SHAPE),
    (dict(d_k=128, d_v=128, dtype=0), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=128, d_v=32), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(dtype=3), _lib.SDPA_ERR_DTYPE),
    (dict(scale=math.inf), _lib.SDPA_ERR_SCALE),
    (dict(out=P), _lib.SDPA_ERR_ALIAS),
    (dict(q=P + 4), _lib.SDPA_ERR_ALIGN),
])
def test_window_validation_rejects_before_any_hip_call(kw, code, lib):
    """The window entry point shares sdpa_forward's checks and adds its own.

    Note: n != m is legal with a window (any alignment); only bad sides or an
    unknown alignment are mask errors."""
    assert call_window(**kw) == code


def call_mha(**kw):
    B, n, m, d_model, h = kw.get("B", 2), kw.get("n", 8), kw.get("m", 8), kw.get("d_model", 128), kw.get("h", 2)
    need = _lib.sdpa_mha_workspace_bytes(B, n, m, h, 64, 64)
    a = dict(x_q=P, x_kv=2 * P, w_q=3 * P, w_k=4 * P, w_v=5 * P, w_o=6 * P, out=7 * P, B=B, n=n, m=m,
             d_model=d_model, h=h, d_k=64, d_v=64, scale=0.125, wl=-1, wr=-1, align=0, key_lens=None,
             dtype=1, ws=8 * P, ws_bytes=need)
    a.update(kw)
    return _lib.sdpa_mha_forward(a["x_q"], a["x_kv"], a["w_q"], a["w_k"], a["w_v"], a["w_o"], a["out"],
                                 a["B"], a["n"], a["m"], a["d_model"], a["h"], a["d_k"], a["d_v"],
                                 a["scale"], a["wl"], a["wr"], a["align"], a["key_lens"], a["dtype"],
                                 a["ws"], a["ws_bytes"], None)


def test_mha_workspace_size(lib):
    # Q, K, V and the attention output in bf16, each rounded up to 256 bytes
    assert _lib.sdpa_mha_workspace_bytes(64, 64, 64, 8, 64, 64) == 4 * 64 * 8 * 64 * 64 * 2
    assert _lib.sdpa_mha_workspace_bytes(1, 3, 5, 1, 64, 64) == 2 * 512 + 2 * 768
    assert _lib.sdpa_mha_workspace_bytes(1, 3, 5, 1, 32, 64) == 0  # d_k != d_v
    assert _lib.sdpa_mha_workspace_bytes(2, 4, 4, 16, 32, 32) == 4 * 2 * 16 * 4 * 32 * 2
    assert _lib.sdpa_mha_workspace_bytes(2, 4, 4, 3, 32, 32) == 0  # h·d not a multiple of 64
    assert _lib.sdpa_mha_workspace_bytes(1, 2, 2, 1, 128, 128) == 4 * 512
    assert _lib.sdpa_mha_workspace_bytes(1, 2, 2, 1, 16, 16) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(x_q=None), _lib.SDPA_ERR_NULL),
    (dict(ws=None), _lib.SDPA_ERR_NULL),
    (dict(dtype=0), _lib.SDPA_ERR_UNSUPPORTED),  # the sublayer is bf16 only
    (dict(dtype=5), _lib.SDPA_ERR_DTYPE),
    (dict(d_model=96), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=32), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(h=0), _lib.SDPA_ERR_SHAPE),
    (dict(B=1 << 16, n=1 << 12, d_model=512), _lib.SDPA_ERR_SHAPE),
    (dict(wl=-3), _lib.SDPA_ERR_MASK),
    (dict(align=7), _lib.SDPA_ERR_MASK),
    (dict(scale=0.0), _lib.SDPA_ERR_SCALE),
    (dict(w_o=6 * P + 8), _lib.SDPA_ERR_ALIGN),
    (dict(ws_bytes=1024), _lib.SDPA_ERR_WORKSPACE),
    (dict(out=2 * P), _lib.SDPA_ERR_ALIAS),
    (dict(ws=P), _lib.SDPA_ERR_ALIAS),
    (dict(out=8 * P + 64), _lib.SDPA_ERR_ALIAS),
])
def test_mha_validation_rejects_before_any_hip_call(kw, code, lib):
    assert call_mha(**kw) == code


def call_lse(**kw):
    a = dict(q=P, k=2 * P, v=3 * P, out=4 * P, lse=5 * P, B=2, h=2, n=8, m=8, d_k=64, d_v=64,
             scale=0.125, wl=-1, wr=-1, align=0, key_lens=None, dtype=1)
    a.update(kw)
    return _lib.sdpa_forward_lse(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["h"], a["n"],
                                 a["m"], a["d_k"], a["d_v"], a["scale"], a["wl"], a["wr"], a["align"],
                                 a["key_lens"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(lse=None), _lib.SDPA_ERR_NULL),
    (dict(q=None), _lib.SDPA_ERR_NULL),
    (dict(lse=4 * P + 6000, dtype=0), _lib.SDPA_ERR_ALIAS),  # inside out's fp32 span (8 KiB), past its bf16 one
    (dict(dtype=4), _lib.SDPA_ERR_DTYPE),
    (dict(lse=5 * P + 2), _lib.SDPA_ERR_ALIGN),
    (dict(wr=-2), _lib.SDPA_ERR_MASK),
    (dict(align=3), _lib.SDPA_ERR_MASK),
    (dict(lse=4 * P + 64), _lib.SDPA_ERR_ALIAS),  # inside out
    (dict(lse=P), _lib.SDPA_ERR_ALIAS),
])
def test_forward_lse_validation_rejects_before_any_hip_call(kw, code, lib):
    assert call_lse(**kw) == code


def test_forward_workspace_size(lib):
    # only decoder steps (n <= 16) use one, for any number of heads, when their keys
    # fill two pieces: ceil(m / piece) splits × B·h heads × n queries × 68 floats,
    # pieces of 1024 keys, halved (to 256 at least) while B·h·splits < 1024
    assert _lib.sdpa_forward_workspace_bytes(32, 8, 1, 8192, 64, 64, 1) == 8 * 256 * 1 * 68 * 4
    assert _lib.sdpa_forward_workspace_bytes(32, 8, 4, 1025, 64, 64, 1) == 5 * 256 * 4 * 68 * 4  # 256
    assert _lib.sdpa_forward_workspace_bytes(32, 8, 1, 1024, 64, 64, 1) == 4 * 256 * 1 * 68 * 4  # 256
    assert _lib.sdpa_forward_workspace_bytes(16, 8, 1, 8192, 64, 64, 1) == 8 * 128 * 1 * 68 * 4
    assert _lib.sdpa_forward_workspace_bytes(1, 1, 16, 3000, 64, 64, 1) == 12 * 1 * 16 * 68 * 4  # 256
    assert _lib.sdpa_forward_workspace_bytes(1, 8, 1, 1000, 64, 64, 1) == 4 * 8 * 1 * 68 * 4  # 256
    assert _lib.sdpa_forward_workspace_bytes(1, 64, 1, 4096, 64, 64, 1) == 16 * 64 * 1 * 68 * 4  # 256
    assert _lib.sdpa_forward_workspace_bytes(64, 8, 1, 1000, 64, 64, 1) == 2 * 512 * 1 * 68 * 4  # 512
    assert _lib.sdpa_forward_workspace_bytes(1, 8, 1, 256, 64, 64, 1) == 0  # one piece
    assert _lib.sdpa_forward_workspace_bytes(128, 8, 1, 1000, 64, 64, 1) == 0  # one 1024-key piece
    assert _lib.sdpa_forward_workspace_bytes(1, 1, 1, 64, 64, 64, 1) == 0  # sentence-length kernel
    assert _lib.sdpa_forward_workspace_bytes(32, 8, 17, 8192, 64, 64, 1) == 0  # n > 16
    assert _lib.sdpa_forward_workspace_bytes(32, 8, 1, 8192, 64, 64, 0) == 0  # fp32
    assert _lib.sdpa_forward_workspace_bytes(32, 8, 1, 8192, 128, 128, 1) == 0


G = 1 << 32  # fake addresses far enough apart for the 134 MB K and V of this shape


def call_ex(**kw):
    a = dict(q=G, k=2 * G, v=3 * G, out=4 * G, lse=None, B=32, h=8, n=1, m=4096, d_k=64, d_v=64,
             scale=0.125, wl=-1, wr=0, align=1, key_lens=None, dtype=1, ws=5 * G, ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = _lib.sdpa_forward_workspace_bytes(a["B"], a["h"], a["n"], a["m"], a["d_k"],
                                                          a["d_v"], a["dtype"])
    return _lib.sdpa_forward_ex(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["h"], a["n"],
                                a["m"], a["d_k"], a["d_v"], a["scale"], a["wl"], a["wr"], a["align"],
                                a["key_lens"], a["dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SDPA_ERR_NULL),
    (dict(ws_bytes=100), _lib.SDPA_ERR_WORKSPACE),
    (dict(ws=5 * G + 8), _lib.SDPA_ERR_ALIGN),
    (dict(ws=4 * G), _lib.SDPA_ERR_ALIAS),              # workspace on out
    (dict(lse=4 * G + 40000, dtype=0), _lib.SDPA_ERR_ALIAS),  # inside out's fp32 span (64 KiB) only
    (dict(lse=6 * G + 1), _lib.SDPA_ERR_ALIGN),
    (dict(lse=G), _lib.SDPA_ERR_ALIAS),
    (dict(ws=6 * G, lse=6 * G + 64), _lib.SDPA_ERR_ALIAS),  # workspace on lse
    (dict(wl=-4), _lib.SDPA_ERR_MASK),
    (dict(scale=-1.0), _lib.SDPA_ERR_SCALE),
])
def test_forward_ex_validation_rejects_before_any_hip_call(kw, code, lib):
    assert call_ex(**kw) == code


def call_noalloc(**kw):
    a = dict(q=G, k=2 * G, v=3 * G, out=4 * G, lse=None, B=32, h=8, n=1, m=4096, d_k=64, d_v=64,
             scale=0.125, wl=-1, wr=0, align=1, key_lens=None, dtype=1)
    a.update(kw)
    return _lib.sdpa_forward_ex_noalloc(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["h"],
                                        a["n"], a["m"], a["d_k"], a["d_v"], a["scale"], a["wl"],
                                        a["wr"], a["align"], a["key_lens"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SDPA_ERR_NULL),
    (dict(out=4 * G + 8), _lib.SDPA_ERR_ALIGN),
    (dict(out=G), _lib.SDPA_ERR_ALIAS),
    (dict(lse=4 * G + 40000, dtype=0), _lib.SDPA_ERR_ALIAS),  # inside out's fp32 span (64 KiB) only
    (dict(lse=6 * G + 1), _lib.SDPA_ERR_ALIGN),
    (dict(lse=G), _lib.SDPA_ERR_ALIAS),
    (dict(wl=-4), _lib.SDPA_ERR_MASK),
    (dict(align=7), _lib.SDPA_ERR_MASK),
    (dict(scale=float("nan")), _lib.SDPA_ERR_SCALE),
    (dict(d_k=8, d_v=8), _lib.SDPA_ERR_UNSUPPORTED),
    # a split needing 64 pieces x 512 heads x 16 queries x 272 bytes = 142 MB > 8 MiB
    (dict(B=64, n=16, m=65536), _lib.SDPA_ERR_SCRATCH),
])
def test_forward_ex_noalloc_validation_rejects_before_any_hip_call(kw, code, lib):
    assert call_noalloc(**kw) == code


def test_noalloc_scratch_limit_covers_the_decoder_workloads(lib):
    """The static scratch holds the split workspace of the decoder-step shapes:
    256 heads of 8192 keys, one sequence of 8 heads over 32768 keys, and 8
    heads x 4 queries over 131072 keys; past it the call refuses."""
    for (B, h, n, m) in ((32, 8, 1, 8192), (1, 8, 1, 32768), (1, 8, 4, 131072)):
        need = _lib.sdpa_forward_workspace_bytes(B, h, n, m, 64, 64, _lib.SDPA_BF16)
        assert 0 < need <= _lib.SDPA_NOALLOC_SCRATCH_BYTES
    assert "SDPA_NOALLOC_SCRATCH_BYTES" in _lib.sdpa_strerror(_lib.SDPA_ERR_SCRATCH)
    assert re.search(r"#define\s+SDPA_NOALLOC_SCRATCH_BYTES\s+\(8u << 20\)", _header())


def call_strided(strides=None, **kw):
    """sdpa_forward_strided on fake addresses, 2 x 4 heads, n = 48, m = 80, bf16;
    ``strides`` defaults to the token-major [B, len, h, d] layout of all four."""
    a = dict(q=G, k=2 * G, v=3 * G, out=4 * G, lse=None, B=2, h=4, n=48, m=80, d_k=64, d_v=64,
             scale=0.125, wl=-1, wr=-1, align=0, key_lens=None, dtype=1, ws=None, ws_bytes=0)
    a.update(kw)
    B, h, n, m, d = a["B"], a["h"], a["n"], a["m"], a["d_k"]
    if strides is None:
        strides = [n * h * d, d, h * d, m * h * d, d, h * d, m * h * d, d, h * d, n * h * d, d, h * d]
    return _lib.sdpa_forward_strided(a["q"], a["k"], a["v"], a["out"], a["lse"], B, h, n, m, d,
                                     a["d_v"], a["scale"], a["wl"], a["wr"], a["align"], a["key_lens"],
                                     a["dtype"], strides, a["ws"], a["ws_bytes"], None)


def _bshd(B, h, n, m, d):
    return [n * h * d, d, h * d, m * h * d, d, h * d, m * h * d, d, h * d, n * h * d, d, h * d]


def _with(strides, i, v):
    s = list(strides)
    s[i] = v
    return s


BSHD = _bshd(2, 4, 48, 80, 64)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.SDPA_ERR_NULL),
    (dict(strides=_with(BSHD, 2, 63)), _lib.SDPA_ERR_SHAPE),          # q row stride < d_k
    (dict(strides=_with(BSHD, 5, 32)), _lib.SDPA_ERR_SHAPE),          # k row stride < d_k
    (dict(strides=_with(BSHD, 0, -8)), _lib.SDPA_ERR_SHAPE),          # negative batch stride
    (dict(strides=_with(BSHD, 7, 1 << 41)), _lib.SDPA_ERR_SHAPE),     # stride past 2^40
    (dict(strides=_with(BSHD, 8, 1 << 24)), _lib.SDPA_ERR_SHAPE),     # 64 rows past 2^31 bytes
    (dict(strides=_with(BSHD, 2, 260)), _lib.SDPA_ERR_ALIGN),         # 520-byte rows
    (dict(strides=_with(BSHD, 4, 4)), _lib.SDPA_ERR_ALIGN),           # 8-byte head stride
    (dict(strides=_with(BSHD, 10, 0)), _lib.SDPA_ERR_ALIAS),          # out heads on one another
    (dict(strides=_with(BSHD, 11, 64)), _lib.SDPA_ERR_ALIAS),         # out rows on the heads' rows
    (dict(out=G + 64), _lib.SDPA_ERR_ALIAS),                          # out inside q's span
    (dict(lse=4 * G + 256), _lib.SDPA_ERR_ALIAS),                     # lse inside out's span
    (dict(lse=4 * G + 60000, dtype=0), _lib.SDPA_ERR_ALIAS),          # inside out's fp32 span only
    (dict(wl=-3), _lib.SDPA_ERR_MASK),
    (dict(d_k=8, d_v=8), _lib.SDPA_ERR_UNSUPPORTED),
])
def test_forward_strided_validation_rejects_before_any_hip_call(kw, code, lib):
    assert call_strided(**kw) == code


def test_forward_strided_layout_rules_accept_shared_heads():
    """Head stride 0 on K and V (one K/V head shared by every query head) and
    a fused [B, len, 3, h, d] Q/K/V buffer pass the layout checks; the call
    is then refused by a later, launch-free check (out overlapping lse)."""
    B, h, n, d = 2, 4, 48, 64
    shared = _with(_with(BSHD, 4, 0), 7, 0)
    assert call_strided(strides=shared, lse=4 * G + 256) == _lib.SDPA_ERR_ALIAS
    fused = [n * 3 * h * d, d, 3 * h * d] * 3 + [n * h * d, d, h * d]
    assert call_strided(strides=fused, m=n, q=G, k=G + h * d * 2, v=G + 2 * h * d * 2,
                        lse=4 * G + 256) == _lib.SDPA_ERR_ALIAS


def call_bwd(**kw):
    B, h, n = kw.get("B", 2), kw.get("h", 2), kw.get("n", 8)
    a = dict(q=P, k=2 * P, v=3 * P, out=4 * P, dout=5 * P, lse=6 * P, dq=7 * P, dk=8 * P, dv=9 * P,
             B=B, h=h, n=n, m=8, d_k=64, d_v=64, scale=0.125, wl=-1, wr=-1, align=0, key_lens=None,
             dtype=1, ws=10 * P, ws_bytes=_lib.sdpa_backward_workspace_bytes(B, h, n))
    a.update(kw)
    return _lib.sdpa_backward(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"],
                              a["dv"], a["B"], a["h"], a["n"], a["m"], a["d_k"], a["d_v"], a["scale"],
                              a["wl"], a["wr"], a["align"], a["key_lens"], a["dtype"], a["ws"],
                              a["ws_bytes"], None)


def test_backward_workspace_size(lib):
    # D and lse·log2 e per query row, fp32, each rounded up to 256 bytes
    assert _lib.sdpa_backward_workspace_bytes(64, 8, 64) == 2 * 64 * 8 * 64 * 4
    assert _lib.sdpa_backward_workspace_bytes(1, 1, 3) == 2 * 256
    assert _lib.sdpa_backward_workspace_bytes(0, 1, 3) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dout=None), _lib.SDPA_ERR_NULL),
    (dict(lse=None), _lib.SDPA_ERR_NULL),
    (dict(dk=None), _lib.SDPA_ERR_NULL),
    (dict(ws=None), _lib.SDPA_ERR_NULL),
    (dict(q=None), _lib.SDPA_ERR_NULL),
    (dict(dtype=0, d_k=32, d_v=32), _lib.SDPA_ERR_UNSUPPORTED),    # the fp32 gradient takes width 64
    (dict(dtype=0, d_k=128, d_v=128), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(dtype=0, dk=7 * P + 6000), _lib.SDPA_ERR_ALIAS),         # inside dq's fp32 span (8 KiB) only
    (dict(dtype=9), _lib.SDPA_ERR_DTYPE),
    (dict(d_v=32), _lib.SDPA_ERR_UNSUPPORTED),
    # forward-only widths: the backward kernels take equal widths 32, 64, 128
    (dict(d_k=16, d_v=16), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=16, d_v=64), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=32, d_v=64), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(m=0), _lib.SDPA_ERR_SHAPE),
    (dict(scale=float("inf")), _lib.SDPA_ERR_SCALE),
    (dict(dq=7 * P + 4), _lib.SDPA_ERR_ALIGN),
    (dict(lse=6 * P + 2), _lib.SDPA_ERR_ALIGN),
    (dict(wl=-5), _lib.SDPA_ERR_MASK),
    (dict(align=2), _lib.SDPA_ERR_MASK),
    (dict(ws_bytes=16), _lib.SDPA_ERR_WORKSPACE),
    (dict(dq=P), _lib.SDPA_ERR_ALIAS),           # dq on q
    (dict(dv=5 * P + 64), _lib.SDPA_ERR_ALIAS),  # dv inside dout
    (dict(dk=7 * P), _lib.SDPA_ERR_ALIAS),       # dk on dq
    (dict(ws=9 * P), _lib.SDPA_ERR_ALIAS),       # workspace on dv
])
def test_backward_validation_rejects_before_any_hip_call(kw, code, lib):
    assert call_bwd(**kw) == code


def test_torch_wrapper_rejects_bad_windows():
    import torch

    from transformer_attention_sdpa_amd import forward

    x = torch.zeros(1, 1, 4, 64)
    for kw in (dict(window=(1, 1), causal=True), dict(window=(-1, 2)), dict(window=(1, 1, "middle"))):
        with pytest.raises(ValueError):
            forward(x, x, x, **kw)


@pytest.mark.parametrize("heads", [8, 512])
@pytest.mark.parametrize("return_lse", [False, True])
def test_torch_wrapper_rejects_causal_with_n_ne_m(heads, return_lse):
    """causal=True is the top-left inclusive j <= i rule of decoder self-attention
    and needs n == m.  The binding rejects n != m before it chooses an entry
    point, so the answer does not depend on the head count (fewer than 256
    heads take the workspace path) or on return_lse.  No launch happens: the
    check fires on CPU tensors, before the device checks."""
    import torch

    from transformer_attention_sdpa_amd import backward, forward

    q = torch.zeros(1, heads, 1, 64)
    kv = torch.zeros(1, heads, 4096, 64)
    with pytest.raises(ValueError, match="causal mask needs n == m"):
        forward(q, kv, kv, causal=True, return_lse=return_lse)
    with pytest.raises(ValueError, match="causal mask needs n == m"):
        backward(q, kv, kv, q, q, torch.zeros(1, heads, 1), causal=True)


def test_torch_wrapper_rejects_cpu_tensors():
    import torch

    from transformer_attention_sdpa_amd import forward

    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        forward(x, x, x)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without libsdpa.so every entry point of the binding raises."""
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libsdpa.so"))
    with pytest.raises(ImportError):
        _lib.load()
    with pytest.raises(ImportError):
        _lib.sdpa_version()
    with pytest.raises(ImportError):
        call()


# --- attention dropout -----------------------------------------------------------

def call_fwd_drop(**kw):
    a = dict(q=P, k=2 * P, v=3 * P, out=4 * P, lse=None, B=2, h=2, n=8, m=40, d_k=64, d_v=64, scale=0.125,
             wl=-1, wr=-1, align=0, key_lens=None, keep=11 * P, keep_scale=1.25, dtype=1)
    a.update(kw)
    return _lib.sdpa_forward_dropout(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["h"], a["n"], a["m"],
                                     a["d_k"], a["d_v"], a["scale"], a["wl"], a["wr"], a["align"], a["key_lens"],
                                     a["keep"], a["keep_scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(keep=None), _lib.SDPA_ERR_NULL),
    (dict(q=None), _lib.SDPA_ERR_NULL),
    (dict(dtype=0), _lib.SDPA_ERR_UNSUPPORTED),                  # bf16 only
    (dict(d_k=16, d_v=16), _lib.SDPA_ERR_UNSUPPORTED),           # equal widths 32, 64, 128 only
    (dict(d_k=512, d_v=512), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=16, d_v=64), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=32, d_v=64), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=32, d_v=32, dtype=0), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(dtype=5), _lib.SDPA_ERR_DTYPE),
    (dict(keep_scale=0.0), _lib.SDPA_ERR_SCALE),
    (dict(keep_scale=-1.0), _lib.SDPA_ERR_SCALE),
    (dict(keep_scale=math.nan), _lib.SDPA_ERR_SCALE),
    (dict(keep_scale=math.inf), _lib.SDPA_ERR_SCALE),
    (dict(keep=11 * P + 2), _lib.SDPA_ERR_ALIGN),
    (dict(lse=6 * P + 1), _lib.SDPA_ERR_ALIGN),
    (dict(wl=-2), _lib.SDPA_ERR_MASK),
    (dict(keep=4 * P + 16), _lib.SDPA_ERR_ALIAS),                # mask inside out
    (dict(keep=4 * P - 2 * 2 * 8 * 2 * 4 + 4), _lib.SDPA_ERR_ALIAS),  # mask's last word on out
    (dict(lse=11 * P + 8), _lib.SDPA_ERR_ALIAS),                 # lse on the mask
    (dict(lse=4 * P), _lib.SDPA_ERR_ALIAS),                      # lse on out
])
def test_forward_dropout_validation_rejects_before_any_hip_call(kw, code, lib):
    assert call_fwd_drop(**kw) == code


def call_bwd_drop(**kw):
    B, h, n = kw.get("B", 2), kw.get("h", 2), kw.get("n", 8)
    a = dict(q=P, k=2 * P, v=3 * P, out=4 * P, dout=5 * P, lse=6 * P, dq=7 * P, dk=8 * P, dv=9 * P,
             B=B, h=h, n=n, m=8, d_k=64, d_v=64, scale=0.125, wl=-1, wr=-1, align=0, key_lens=None,
             keep=11 * P, keep_scale=2.0, dtype=1, ws=10 * P, ws_bytes=_lib.sdpa_backward_workspace_bytes(B, h, n))
    a.update(kw)
    return _lib.sdpa_backward_dropout(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"],
                                      a["dv"], a["B"], a["h"], a["n"], a["m"], a["d_k"], a["d_v"], a["scale"],
                                      a["wl"], a["wr"], a["align"], a["key_lens"], a["keep"], a["keep_scale"],
                                      a["dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(keep=None), _lib.SDPA_ERR_NULL),
    (dict(dout=None), _lib.SDPA_ERR_NULL),
    (dict(dtype=0), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.SDPA_ERR_DTYPE),
    (dict(d_k=16, d_v=16), _lib.SDPA_ERR_UNSUPPORTED),    # equal widths 32, 64, 128 only
    (dict(d_k=512, d_v=512), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(d_k=128, d_v=128, dtype=0), _lib.SDPA_ERR_UNSUPPORTED),
    (dict(keep_scale=math.inf), _lib.SDPA_ERR_SCALE),
    (dict(keep=11 * P + 1), _lib.SDPA_ERR_ALIGN),
    (dict(ws_bytes=8), _lib.SDPA_ERR_WORKSPACE),
    (dict(dq=11 * P), _lib.SDPA_ERR_ALIAS),                # dq on the mask
    (dict(ws=11 * P + 16), _lib.SDPA_ERR_ALIAS),           # workspace on the mask
    (dict(dv=P), _lib.SDPA_ERR_ALIAS),
])
def test_backward_dropout_validation_rejects_before_any_hip_call(kw, code, lib):
    assert call_bwd_drop(**kw) == code
