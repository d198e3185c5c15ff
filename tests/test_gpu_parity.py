"""Parity of the HIP path with the fp64 oracle, element by element (GPU).

Bar: max abs error ≤ 1e-5 on the fp32 path and ≤ 2e-2 on the bf16 path; masked
weights exactly +0.0.  Every call goes through the C ABI (``sdpa_forward``) via
the thin Python binding.
"""

import json
import math
import os
import zlib

import numpy as np
import pytest

import oracle.sdpa_oracle as so
from sdpa_inputs import WORKLOADS, make_inputs, random_case, round_to_bf16
from tests.gpu_cases import TOL, from_device, max_abs_err, run_gpu, to_device

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _oracle(case, scale=None):
    return so.attention(case["q"], case["k"], case["v"], scale=scale, causal=case["causal"],
                        key_lens=case["key_lens"], window=case.get("window"))


# --- the five workloads at their real sizes ---------------------------------

SMALL = [("single_head_16", "f32"), ("encoder_self_base", "f32"), ("encoder_self_base", "bf16"),
         ("decoder_causal_base", "bf16"), ("cross_big", "bf16")]


@pytest.mark.parametrize("name,dt", SMALL, ids=[f"{a}-{b}" for a, b in SMALL])
def test_workload_full_parity(gpu_lib, name, dt):
    case = make_inputs(name, dt)
    _, got = run_gpu(case)
    ref = _oracle(case)
    err = max_abs_err(got, ref)
    print(f"{name} {dt}: max abs err {err:.3e}")
    assert err <= TOL[dt]


def _long_rows(n, head, rng):
    """Rows of one 8192-query head to check: both sides of every 64-query
    boundary (each wave's key range and tile skipping change there, and every
    fourth one is a 256-query workgroup edge, where the heavy-first block
    order changes), both sides of the 32-query sub-block edges inside one
    workgroup's block (a different block per head), the first two rows, the
    last row and two random rows."""
    rows = {0, 1, n - 1}
    for t in range(1, n // 64):
        rows |= {64 * t - 1, 64 * t}
    q0 = 256 * (head % (n // 256))
    for t in range(1, 8):
        rows |= {q0 + 32 * t - 1, q0 + 32 * t}
    rows |= {int(x) for x in rng.choice(n, 2, replace=False)}
    return sorted(rows)


def test_long_causal_8k_sampled_rows(gpu_lib):
    """n = m = 8192, 64 heads, causal, bf16: every head, every block edge."""
    case = make_inputs("long_causal_8k", "bf16")
    _, got = run_gpu(case)
    wl = WORKLOADS["long_causal_8k"]
    assert np.isfinite(got).all()
    rng = np.random.default_rng(99)
    picks = [(b, h, i) for b in range(wl.B) for h in range(wl.h)
             for i in _long_rows(wl.n, b * wl.h + h, rng)]
    q, k, v = (case[x].astype(np.float64) for x in ("q", "k", "v"))
    ref = so.attention_rows(q, k, v, picks, causal=True)
    g = np.stack([got[b, h, i] for (b, h, i) in picks])
    err = max_abs_err(g, ref)
    print(f"long_causal_8k: {len(picks)} sampled rows, max abs err {err:.3e}")
    assert err <= TOL["bf16"]
    # row 0 sees key 0 only: its output is v_0 exactly
    assert np.array_equal(got[:, :, 0], case["v"][:, :, 0])


# --- the pages' worked example through the GPU ------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_worked_example_on_gpu(gpu_lib, dt):
    """q = [2.2, 0] over seven 2-D keys, scale 1/√2, padded with zeros to d = 64.

    V = identity (padded) exposes the weights as the output row.
    """
    with open(os.path.join(GOLDEN, "worked_example_2d.json"), encoding="utf-8") as f:
        g = json.load(f)
    q = np.zeros((1, 1, 1, 64), np.float32)
    q[0, 0, 0, :2] = g["query"]
    k = np.zeros((1, 1, 7, 64), np.float32)
    k[0, 0, :, :2] = [e["k"] for e in g["keys"]]
    v = np.zeros((1, 1, 7, 64), np.float32)
    v[0, 0, np.arange(7), np.arange(7)] = 1.0
    if dt == "bf16":
        q, k = round_to_bf16(q), round_to_bf16(k)
    case = {"q": q, "k": k, "v": v, "key_lens": None, "causal": False, "dtype": dt}
    scale = 1.0 / math.sqrt(2.0)
    _, got = run_gpu(case, scale=scale)
    ref = _oracle(case, scale=scale)
    assert max_abs_err(got, ref) <= TOL[dt]
    assert np.all(got[0, 0, 0, 7:] == 0.0)
    w = got[0, 0, 0, :7]
    assert int(np.argmax(w)) == 1 and 0.64 < w[1] < 0.68  # about 66% on 猫 = [2, 0.4]
    if dt == "f32":
        for e, x in zip(g["keys"], w):
            p = e["printed_weight_percent"]
            half = 0.5 * 10.0 ** (-len(p.split(".")[1])) if "." in p else 0.5
            assert abs(100 * x - float(p)) <= half + 1e-3


# --- ragged shapes, several tiles, every mask kind ---------------------------

RAGGED = [
    # (B, h, n, m, causal, with key_lens)
    (1, 1, 1, 1, False, False),
    (1, 2, 1, 200, False, True),
    (2, 1, 5, 7, False, True),
    (1, 1, 33, 33, True, False),
    (2, 3, 65, 65, True, True),
    (1, 2, 100, 37, False, True),
    (1, 1, 127, 129, False, False),
    (2, 2, 129, 129, True, True),
    (1, 1, 200, 200, True, False),
    (1, 2, 300, 517, False, True),
    (1, 1, 513, 513, True, True),
    # sentence-length kernels at and around their 64-row limit, every mask kind
    (3, 2, 40, 40, True, True),
    (2, 2, 64, 64, True, True),
    (2, 2, 64, 63, False, True),
    (1, 3, 17, 64, False, True),
    (2, 1, 65, 64, False, True),
    (1, 2, 64, 65, False, False),
]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", RAGGED, ids=[str(s) for s in RAGGED])
def test_ragged_shapes(gpu_lib, shape, dt):
    B, h, n, m, causal, with_lens = shape
    rng = np.random.default_rng(zlib.crc32(repr((shape, dt)).encode()))
    kl = rng.integers(0, m + 3, size=B) if with_lens else None
    case = random_case(rng, B, h, n, m, 64, 64, dtype=dt, causal=causal, key_lens=kl)
    _, got = run_gpu(case)
    ref = _oracle(case)
    err = max_abs_err(got, ref)
    assert err <= TOL[dt], err


# --- masking is exact ---------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_masked_weights_are_exactly_zero(gpu_lib, dt, causal):
    """V = [I_m | 0] makes O[:, :m] the weight matrix: masked entries must be +0.0."""
    rng = np.random.default_rng(5)
    B, h, n, m = 4, 2, 64, 64
    kl = np.array([64, 17, 1, 40], np.int32)
    case = random_case(rng, B, h, n, m, 64, 64, dtype=dt, causal=causal, key_lens=kl)
    case["v"] = np.zeros_like(case["v"])
    case["v"][:, :, np.arange(m), np.arange(m)] = 1.0
    _, got = run_gpu(case)
    j = np.arange(m)
    for b in range(B):
        for i in range(n):
            vis = (j < kl[b]) & ((j <= i) if causal else True)
            row = got[b, :, i, :m]
            assert np.all(row[:, ~vis] == 0.0) and not np.signbit(row[:, ~vis]).any()
            assert np.all(row[:, vis] > 0.0) or dt == "bf16"
            assert np.allclose(row.sum(-1), 1.0, atol=TOL[dt] * 4)
    ref = _oracle(case)
    assert max_abs_err(got, ref) <= TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n,m", [(48, 100), (64, 64), (20, 50)])
def test_padded_keys_are_never_read(gpu_lib, dt, n, m):
    """Garbage (NaN, huge) in K/V rows at or beyond key_lens leaves O bitwise unchanged."""
    import torch

    rng = np.random.default_rng(8)
    B, h = 3, 2
    kl = np.array([m, 9, min(m, 40)], np.int32)
    case = random_case(rng, B, h, n, m, 64, 64, dtype=dt, key_lens=kl)
    o1, _ = run_gpu(case)
    for b in range(B):
        case["k"][b, :, kl[b]:] = np.nan
        case["v"][b, :, kl[b]:] = 1e30 if dt == "f32" else 3e38
    o2, got2 = run_gpu(case)
    assert torch.equal(o1.view(torch.int16) if dt == "bf16" else o1.view(torch.int32),
                       o2.view(torch.int16) if dt == "bf16" else o2.view(torch.int32))
    assert np.isfinite(got2).all()


NAN_CASES = [  # dtype, B, h, n, m, causal, key_lens: every kernel family
    ("bf16", 2, 2, 64, 64, False, [64, 40]),
    ("bf16", 1, 2, 200, 200, True, None),
    ("f32", 2, 2, 64, 64, False, [50, 64]),
    ("f32", 1, 2, 100, 130, False, [97]),
]


@pytest.mark.parametrize("dt,B,h,n,m,causal,kl", NAN_CASES,
                         ids=[f"{c[0]}-{c[3]}x{c[4]}{'-causal' if c[5] else ''}" for c in NAN_CASES])
def test_nan_in_legal_inputs_propagates(gpu_lib, dt, B, h, n, m, causal, kl):
    """NaN in a legal score or value reaches exactly the outputs the oracle says.

    A NaN query component or a NaN component of a legal key makes the whole
    row NaN for every query that sees it (its weights are NaN); a NaN value
    component makes only that output column NaN.  Everything else stays finite
    and within tolerance.  (The pages leave non-finite inputs open; NaN is
    propagated, never turned into zeros.)
    """
    rng = np.random.default_rng(17)
    case = random_case(rng, B, h, n, m, 64, 64, dtype=dt, causal=causal, key_lens=kl)
    case["q"][0, 0, 3, 5] = np.nan
    case["k"][B - 1, h - 1, 10, 7] = np.nan  # legal for every batch element here
    if not causal:  # a causally hidden NaN value would meet a zero weight: 0 · NaN
        case["v"][0, 1, 12, 3] = np.nan
    _, got = run_gpu(case)
    ref = _oracle(case)
    nan_ref = np.isnan(ref)
    assert nan_ref.any() and not nan_ref.all()
    assert np.array_equal(np.isnan(got), nan_ref)
    assert max_abs_err(got[~nan_ref], ref[~nan_ref]) <= TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_causal_future_keys_do_not_leak(gpu_lib, dt):
    """Changing key/value row j leaves query rows i < j bitwise unchanged."""
    import torch

    rng = np.random.default_rng(9)
    n = 300
    case = random_case(rng, 1, 2, n, n, 64, 64, dtype=dt, causal=True)
    o1, _ = run_gpu(case)
    j = 173
    case["k"][:, :, j] *= -3.0
    case["v"][:, :, j] += 5.0
    o2, _ = run_gpu(case)
    assert torch.equal(o1[:, :, :j], o2[:, :, :j])
    assert not torch.equal(o1[:, :, j:], o2[:, :, j:])


# --- special cases and invariants on the GPU ---------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fully_masked_rows_are_zero(gpu_lib, dt):
    rng = np.random.default_rng(10)
    case = random_case(rng, 3, 2, 40, 70, 64, 64, dtype=dt, key_lens=np.array([0, -5, 1000]))
    _, got = run_gpu(case)
    assert np.all(got[0] == 0.0) and np.all(got[1] == 0.0)
    ref = _oracle(case)  # lengths are clamped to [0, m] on both sides
    assert max_abs_err(got, ref) <= TOL[dt]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_single_visible_key_returns_that_value(gpu_lib, dt):
    rng = np.random.default_rng(12)
    case = random_case(rng, 2, 2, 70, 70, 64, 64, dtype=dt, key_lens=np.array([1, 1]))
    _, got = run_gpu(case)
    assert np.array_equal(got, np.broadcast_to(case["v"][:, :, :1], got.shape))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_zero_queries_average_the_legal_values(gpu_lib, dt):
    rng = np.random.default_rng(14)
    kl = np.array([5, 64, 33])
    case = random_case(rng, 3, 2, 64, 64, 64, 64, dtype=dt, causal=True, key_lens=kl)
    case["q"][:] = 0.0
    _, got = run_gpu(case)
    for b in range(3):
        for i in (0, 4, 5, 32, 63):
            hi = min(kl[b], i + 1)
            ref = case["v"][b, :, :hi].astype(np.float64).mean(axis=1)
            assert max_abs_err(got[b, :, i], ref) <= TOL[dt]


def test_deterministic_and_heads_independent(gpu_lib):
    """Bitwise run-to-run determinism; one B×h call equals B·h one-head calls."""
    import torch

    from transformer_attention_sdpa_amd import forward

    case = make_inputs("decoder_causal_base", "bf16")
    q, k, v = (to_device(case[x], "bf16") for x in ("q", "k", "v"))
    kl = torch.from_numpy(case["key_lens"]).cuda()
    o1 = forward(q, k, v, causal=True, key_lens=kl)
    o2 = forward(q, k, v, causal=True, key_lens=kl)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for b in (0, 17, 63):
        for h in (0, 5):
            one = forward(q[b:b + 1, h:h + 1].contiguous(), k[b:b + 1, h:h + 1].contiguous(),
                          v[b:b + 1, h:h + 1].contiguous(), causal=True, key_lens=kl[b:b + 1].contiguous())
            assert torch.equal(one[0, 0].view(torch.int16), o1[b, h].view(torch.int16))


def test_unscaled_and_custom_scale(gpu_lib):
    rng = np.random.default_rng(15)
    case = random_case(rng, 2, 2, 50, 90, 64, 64, dtype="f32")
    for scale in (1.0, 0.01, 0.3):
        _, got = run_gpu(case, scale=scale)
        assert max_abs_err(got, _oracle(case, scale=scale)) <= TOL["f32"]


def test_wrapper_errors(gpu_lib):
    import torch

    from transformer_attention_sdpa_amd import forward

    q = torch.zeros(1, 1, 4, 64, device="cuda", dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 5, 64, device="cuda", dtype=torch.bfloat16)
    # causal with n != m: the binding refuses before any entry point (ValueError);
    # the C ABI refuses the same call with SDPA_ERR_MASK
    with pytest.raises(ValueError, match="causal"):
        forward(q, k, k, causal=True)
    from transformer_attention_sdpa_amd import _lib, sdpa_forward

    o = torch.empty_like(q)
    rc = sdpa_forward(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), 1, 1, 4, 5, 64, 64,
                      0.125, _lib.SDPA_MASK_CAUSAL, None, _lib.SDPA_BF16,
                      torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.SDPA_ERR_MASK
    # widths: 64 everywhere; 16, 32, 128 (and d_k = 16 or 32 with d_v = 64) in
    # bf16 only; nothing else
    q8 = torch.zeros(1, 1, 4, 8, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="64"):
        forward(q8, q8, q8)
    q96 = torch.zeros(1, 1, 4, 96, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="unsupported"):
        forward(q96, q96, q96)
    q32f = torch.zeros(1, 1, 4, 32, device="cuda", dtype=torch.float32)
    with pytest.raises(RuntimeError, match="unsupported"):
        forward(q32f, q32f, q32f)


def test_pending_hip_error_is_not_reported_as_a_launch_failure(gpu_lib):
    """A failed HIP call that no one collected leaves an error pending on the
    thread; the library's own launch must still report SDPA_OK (it clears the
    pending error before launching) and produce the right output.  The pending
    error comes from hipSetDevice with an ordinal no device has (a host-side
    refusal, nothing reaches the GPU), through the HIP runtime already loaded
    in this process."""
    import ctypes

    import torch

    from transformer_attention_sdpa_amd import _lib, sdpa_forward

    maps = open("/proc/self/maps", encoding="utf-8").read().splitlines()
    paths = sorted({ln.split()[-1] for ln in maps if "libamdhip64" in ln})
    assert len(paths) == 1, paths
    hip = ctypes.CDLL(paths[0])
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    assert hip.hipSetDevice(12345) != 0
    case = random_case(np.random.default_rng(77), 2, 2, 40, 40, 64, 64, dtype="bf16")
    q, k, v = (to_device(case[x], "bf16") for x in ("q", "k", "v"))
    o = torch.empty_like(q)
    rc = sdpa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), 2, 2, 40, 40, 64, 64,
                      0.125, _lib.SDPA_MASK_NONE, None, _lib.SDPA_BF16,
                      torch.cuda.current_stream().cuda_stream)
    assert rc == _lib.SDPA_OK, _lib.sdpa_strerror(rc)
    torch.cuda.synchronize()
    assert max_abs_err(from_device(o), _oracle(case)) <= TOL["bf16"]


def test_concurrent_calls_on_separate_streams(gpu_lib):
    """The library keeps no state: calls from several host threads, each on its
    own stream, give the same bits as one call at a time."""
    import threading

    import torch

    rng = np.random.default_rng(31)
    cases = [random_case(rng, 4, 2, n, n, 64, 64, dtype="bf16", causal=c, key_lens=kl)
             for n, c, kl in ((64, False, [9, 64, 30, 1]), (200, True, None), (48, False, None),
                              (130, False, [100, 7, 130, 64]))]
    solo = [run_gpu(c)[1] for c in cases]
    results = [None] * len(cases)
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(5):
                    _, got = run_gpu(cases[i])
            s.synchronize()
            results[i] = got
        except Exception as e:  # surfaced below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for a, b in zip(solo, results):
        assert np.array_equal(a, b)


# --- larger-than-benchmark sizes, checked on sampled rows --------------------

@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_many_heads_sentence_length_sampled(gpu_lib, dt):
    """8192 heads of 64×64 (a 16× larger batch than the encoder workload)."""
    rng = np.random.default_rng(4242)
    B, h, n = 1024, 8, 64
    kl = rng.integers(0, n + 1, size=B)
    case = random_case(rng, B, h, n, n, 64, 64, dtype=dt, causal=False, key_lens=kl)
    _, got = run_gpu(case)
    picks = [(int(rng.integers(B)), int(rng.integers(h)), int(rng.integers(n))) for _ in range(300)]
    picks += [(B - 1, h - 1, n - 1), (0, 0, 0)]
    ref = so.attention_rows(case["q"], case["k"], case["v"], picks, key_lens=case["key_lens"])
    g = np.stack([got[b, hh, i] for (b, hh, i) in picks])
    assert max_abs_err(g, ref) <= TOL[dt]
    # rows of sequences with key length 0 are exactly zero
    for b in np.flatnonzero(case["key_lens"] == 0)[:4]:
        assert not got[b].any()


def test_long_causal_16k_sampled(gpu_lib):
    """n = m = 16384, causal, bf16: twice the benchmark length."""
    rng = np.random.default_rng(16384)
    n = 16384
    case = random_case(rng, 1, 2, n, n, 64, 64, dtype="bf16", causal=True)
    _, got = run_gpu(case)
    rows = [0, 1, 63, 64, 255, 256, 4095, 8191, 8192, 12345, 16319, 16320, 16383]
    picks = [(0, hh, i) for hh in range(2) for i in rows]
    ref = so.attention_rows(case["q"], case["k"], case["v"], picks, causal=True)
    g = np.stack([got[b, hh, i] for (b, hh, i) in picks])
    assert max_abs_err(g, ref) <= TOL["bf16"]


# --- restricted attention: key windows --------------------------------------

WIN_SHAPES = [  # B, h, n, m, key_lens: both kernel families, decode-like and ragged cases
    (2, 2, 64, 64, [64, 37]),
    (1, 2, 48, 64, [50]),
    (1, 2, 40, 64, [10]),       # bottom-right with fewer keys than queries: empty rows
    (2, 1, 1, 300, [300, 77]),  # one decoding query against cached keys
    (2, 2, 200, 200, None),
    (1, 2, 130, 300, [260]),
]
WINDOWS = [(2, 1, "top_left"), (0, 0, "top_left"), (None, 5, "top_left"), (7, None, "top_left"),
           (16, 16, "top_left"), (None, 0, "bottom_right"), (3, 0, "bottom_right"),
           (40, 40, "bottom_right"), (0, 0, "bottom_right")]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("shape", WIN_SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}x{s[3]}" for s in WIN_SHAPES])
def test_window_parity(gpu_lib, dt, shape):
    B, h, n, m, kl = shape
    rng = np.random.default_rng(zlib.crc32(repr((dt, shape)).encode()))
    base = random_case(rng, B, h, n, m, 64, 64, dtype=dt, key_lens=kl)
    worst = 0.0
    for win in WINDOWS:
        case = dict(base, window=win)
        _, got = run_gpu(case)
        ref = _oracle(case)
        err = max_abs_err(got, ref)
        worst = max(worst, err)
        assert err <= TOL[dt], (win, err)
        # rows with no legal key are exactly zero
        for b in range(B):
            L = m if kl is None else min(kl[b], m)
            for i in range(n):
                lo, hi = _window_range(i, n, L, win)
                if hi <= lo:
                    assert np.all(got[b, :, i] == 0.0), (win, b, i)
    print(f"windows {dt} {shape}: max abs err {worst:.3e}")


def _window_range(i, n, L, win):
    left, right, align = win
    c = i if align == "top_left" else i + L - n
    lo = 0 if left is None else max(0, c - left)
    hi = L if right is None else min(L, c + right + 1)
    return lo, hi


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("n", [64, 300])
def test_window_special_cases_are_bitwise_the_plain_masks(gpu_lib, dt, n):
    """(None, 0) top-left is the causal mask and (None, None) is no mask: the
    same kernels run, so the outputs agree bit for bit."""
    import torch

    rng = np.random.default_rng(41 + n)
    case = random_case(rng, 2, 2, n, n, 64, 64, dtype=dt, key_lens=[n, n // 2])
    o_causal, _ = run_gpu(dict(case, causal=True))
    o_win, _ = run_gpu(dict(case, window=(None, 0)))
    assert torch.equal(o_causal, o_win)
    o_plain, _ = run_gpu(case)
    o_open, _ = run_gpu(dict(case, window=(None, None)))
    assert torch.equal(o_plain, o_open)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_keys_outside_a_window_do_not_leak(gpu_lib, dt):
    """Changing key/value row j leaves bitwise unchanged every query whose
    window does not contain j."""
    import torch

    rng = np.random.default_rng(43)
    n, win = 400, (20, 10, "top_left")
    case = dict(random_case(rng, 1, 2, n, n, 64, 64, dtype=dt), window=win)
    o1, _ = run_gpu(case)
    j = 211
    case["k"][:, :, j] *= -3.0
    case["v"][:, :, j] += 5.0
    o2, _ = run_gpu(case)
    sees = [i for i in range(n) if i - 20 <= j <= i + 10]  # j inside [i - left, i + right]
    blind = [i for i in range(n) if i not in sees]
    assert torch.equal(o1[:, :, blind], o2[:, :, blind])
    assert not torch.equal(o1[:, :, sees], o2[:, :, sees])


def test_local_window_8k_sampled_rows(gpu_lib):
    """n = m = 8192, 64 heads, 256 keys either side of each query, bf16."""
    case = make_inputs("local_window_8k", "bf16")
    _, got = run_gpu(case)
    wl = WORKLOADS["local_window_8k"]
    assert np.isfinite(got).all()
    rng = np.random.default_rng(101)
    rows = [0, 1, 255, 256, 257, 511, 512, 1000, 4095, 4096, 7935, 7936, 8190, 8191]
    picks = []
    for b in range(wl.B):
        for h in range(wl.h):
            for i in rows[:3] + list(rng.choice(wl.n, size=3, replace=False)) + rows[-2:]:
                picks.append((b, h, int(i)))
    for i in rows:
        picks.append((2, 9, i))
    # both sides of every 128-query block edge (a workgroup walks four blocks)
    for b, h in ((0, 0), (3, 15)):
        for e in range(128, wl.n, 128):
            picks += [(b, h, e - 1), (b, h, e)]
    ref = so.attention_rows(case["q"], case["k"], case["v"], picks, window=wl.window)
    g = np.stack([got[b, h, i] for (b, h, i) in picks])
    err = max_abs_err(g, ref)
    print(f"local_window_8k: {len(picks)} sampled rows, max abs err {err:.3e}")
    assert err <= TOL["bf16"]


# --- decoder steps: a few queries against many cached keys ------------------

DECODE_WINDOWS = [(None, 0, "bottom_right"), (None, None, "top_left"), (3, 0, "bottom_right"),
                  (0, 0, "bottom_right"), (50, 5, "top_left"), (None, 7, "top_left")]


@pytest.mark.parametrize("n,m", [(1, 200), (2, 200), (5, 200), (16, 200), (1, 1100), (16, 1100)])
def test_decode_kernel_parity(gpu_lib, n, m):
    """bf16, n <= 16 queries against m keys over B·h = 256 heads (the decode
    kernel's range): ragged cache lengths including 0, 1 and m."""
    rng = np.random.default_rng(61 + n + m)
    B, h = 32, 8
    kl = rng.integers(0, m + 1, size=B).astype(np.int32)
    kl[:4] = [0, 1, m, 33]
    base = random_case(rng, B, h, n, m, 64, 64, dtype="bf16", key_lens=kl)
    worst = 0.0
    for win in DECODE_WINDOWS:
        case = dict(base, window=win)
        _, got = run_gpu(case)
        ref = _oracle(case)
        err = max_abs_err(got, ref)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (win, err)
        assert np.all(got[0] == 0.0)  # key length 0: no legal key anywhere
    # one key legal for the bottom-right causal query of batch element 1: v_0 exactly
    case = dict(base, window=(None, 0, "bottom_right"))
    _, got = run_gpu(case)
    if n == 1:
        assert np.array_equal(got[1, :, 0], base["v"][1, :, 0])
    print(f"decode kernel n={n} m={m}: max abs err {worst:.3e}")


@pytest.mark.parametrize("n", [1, 4, 16])
def test_decode_two_heads_per_workgroup(gpu_lib, n):
    """Short caches over many heads take two heads per workgroup; an odd head
    count (1025) leaves the last workgroup half empty.  Every decode window,
    ragged lengths including 0, 1 and m."""
    rng = np.random.default_rng(91 + n)
    B, h, m = 1025, 1, 200
    kl = rng.integers(0, m + 1, size=B).astype(np.int32)
    kl[:4] = [0, 1, m, 33]
    kl[-1] = m
    base = random_case(rng, B, h, n, m, 64, 64, dtype="bf16", key_lens=kl)
    worst = 0.0
    for win in DECODE_WINDOWS:
        case = dict(base, window=win)
        _, got = run_gpu(case)
        ref = _oracle(case)
        err = max_abs_err(got, ref)
        worst = max(worst, err)
        assert err <= TOL["bf16"], (win, err)
        assert np.all(got[0] == 0.0)
    print(f"decode two heads per workgroup n={n}: max abs err {worst:.3e}")


@pytest.mark.parametrize("name", ["decode_beam_base", "decode_long_cache"])
def test_decode_workloads_full_parity(gpu_lib, name):
    case = make_inputs(name, "bf16")
    _, got = run_gpu(case)
    ref = _oracle(case)
    err = max_abs_err(got, ref)
    print(f"{name}: max abs err {err:.3e}")
    assert err <= TOL["bf16"]


def test_decode_kernel_is_deterministic_and_matches_per_head_calls(gpu_lib):
    """Bitwise run-to-run; each head's row equals the tiled kernel's within
    tolerance (the two kernels sum in different orders)."""
    import torch

    rng = np.random.default_rng(71)
    B, h, n, m = 32, 8, 3, 500
    case = dict(random_case(rng, B, h, n, m, 64, 64, dtype="bf16",
                            key_lens=rng.integers(100, m + 1, size=B)),
                window=(None, 0, "bottom_right"))
    o1, g1 = run_gpu(case)
    o2, _ = run_gpu(case)
    assert torch.equal(o1, o2)
    # B·h = 2 heads takes the tiled kernel; compare a few batch elements
    for b in (0, 17, 31):
        sub = dict(case, q=case["q"][b:b + 1, :2], k=case["k"][b:b + 1, :2], v=case["v"][b:b + 1, :2],
                   key_lens=case["key_lens"][b:b + 1])
        _, gs = run_gpu(sub)
        assert max_abs_err(gs[0], g1[b, :2]) <= TOL["bf16"]
