"""The throughput accounting of bench.py, checked on the CPU.

The metric counts 4·d FLOPs per legal (query, key) pair and the HBM bytes of
Q, O and the legal K/V rows.  Here the closed forms in ``bench.algorithmic_work``
are compared with a brute-force count of the legal pairs taken from the
oracle's own visibility rule, for every workload shape (the 8k case on a
reduced batch, the count being per head).
"""

import dataclasses

import numpy as np
import pytest

import bench
import oracle.sdpa_oracle as so
from sdpa_inputs import WORKLOADS, make_inputs


def _brute(wl, key_lens):
    pairs = 0
    kv_rows = 0
    for b in range(wl.B):
        kl = None if key_lens is None else int(key_lens[b])
        if wl.window is None:
            vis = so.visible_keys(np.arange(wl.n), wl.m, wl.causal, kl)
        else:
            L = wl.m if kl is None else min(max(kl, 0), wl.m)
            align = wl.window[2] if len(wl.window) > 2 else "top_left"
            shift = L - wl.n if align == "bottom_right" else 0
            vis = so.visible_keys(np.arange(wl.n), wl.m, wl.causal, kl,
                                  window=(wl.window[0], wl.window[1], shift))
        pairs += wl.h * int(vis.sum())
        L = wl.m if kl is None else min(max(kl, 0), wl.m)
        kv_rows += wl.h * L
    return pairs, kv_rows


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_algorithmic_work_matches_brute_force(name):
    wl = WORKLOADS[name]
    if wl.B * wl.h * (wl.n + 2 * wl.m) * wl.d_k > 1 << 25:
        # the 8k and long-cache cases: one head is enough, the count is per head
        wl = dataclasses.replace(wl, B=1, h=1)
        key_lens = None
    else:
        key_lens = make_inputs(wl, wl.dtypes[0])["key_lens"]
    for dt, esz in (("bf16", 2), ("f32", 4)):
        flops, nbytes, dense = bench.algorithmic_work(wl, dt, key_lens)
        pairs, kv_rows = _brute(wl, key_lens)
        # 2·d_k per score and 2·d_v per weighted value; Q, O and the legal
        # K, V rows (d_k + d_v elements per query row and per key row)
        dk, dv = wl.d_k, wl.d_v
        assert flops == 2 * (dk + dv) * pairs
        assert dense == 2 * (dk + dv) * wl.B * wl.h * wl.n * wl.m
        assert nbytes == esz * (wl.B * wl.h * wl.n * (dk + dv) + kv_rows * (dk + dv))


def test_key_length_edge_cases():
    wl = dataclasses.replace(WORKLOADS["decoder_causal_base"], B=4, h=2)
    kl = np.array([0, 1, 64, 99], dtype=np.int32)  # empty, one key, full, beyond m
    flops, nbytes, _ = bench.algorithmic_work(wl, "bf16", kl)
    pairs, kv_rows = _brute(wl, kl)
    assert flops == 4 * 64 * pairs
    assert kv_rows == 2 * (0 + 1 + 64 + 64)
    assert nbytes == 2 * (2 * 4 * 2 * 64 * 64 + 2 * kv_rows * 64)


@pytest.mark.parametrize("window", [(3, 5, "top_left"), (0, 0, "top_left"), (None, 2, "bottom_right"),
                                    (7, None, "bottom_right"), (2, 0, "bottom_right")])
def test_window_pair_count(window):
    wl = dataclasses.replace(WORKLOADS["cross_big"], B=3, h=2, n=20, m=40, window=window)
    kl = np.array([0, 13, 40], dtype=np.int32)
    flops, _, _ = bench.algorithmic_work(wl, "bf16", kl)
    pairs, _ = _brute(wl, kl)
    assert flops == 4 * 64 * pairs


@pytest.mark.parametrize("name", ["encoder_self_base", "decoder_causal_base", "cross_big"])
def test_backward_work_matches_brute_force(name):
    """Five products per legal pair (S, dP, dV, dQ, dK: 2·d each); bytes at the
    element size: Q, O, dO, dQ of every query row, the fp32 log-sum-exp, the
    legal K, V rows read and every dK, dV row written."""
    wl = WORKLOADS[name]
    key_lens = make_inputs(wl, wl.dtypes[0])["key_lens"]
    pairs, kv_rows = _brute(wl, key_lens)
    rows_q = wl.B * wl.h * wl.n
    for dt, esz in (("bf16", 2), ("f32", 4)):
        flops, nbytes = bench.backward_work(wl, key_lens, dt)
        assert flops == 10 * 64 * pairs
        assert nbytes == (esz * 64 * (4 * rows_q + 2 * kv_rows + 2 * wl.B * wl.h * wl.m) + 4 * rows_q)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says so,
    before touching a device."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
