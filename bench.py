#!/usr/bin/env python3
"""Throughput of the fused attention forward on one MI355X (gfx950).

A "step" is one sdpa_forward over one batch of the workload (every step of the
path: staging, scores, masking, online softmax, weighted sum, store).  Inputs
are seeded synthetic N(0,1) tensors already resident in HBM; the timed steps
rotate over enough copies of the batch (> 2× the 256 MB Infinity Cache) that
the data really streams from HBM, and a 2 GiB read runs just before the timed
steps, so the sets they touch first are cold too, at any step count.  The K
timed steps are launched one after another behind that read (about 0.3 ms,
long enough for the host to enqueue all of them, so the kernels run back to
back) and timed with HIP events on the stream they run on.  The same steps
replayed from a HIP graph, and a graph replay of two passes over every set,
are reported beside them as cross-checks.

Prints ONE JSON line.  Default workload: the base-model encoder self-attention
batch (B=64, h=8, n=m=64, d_k=d_v=64, bf16, key padding U[8,64]).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--dtype bf16|f32]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sdpa_inputs import WORKLOADS, make_inputs  # noqa: E402

# MI355X published peaks (dense, no sparsity).
PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
INFINITY_CACHE_BYTES = 256 << 20

CSRC = os.path.join(ROOT, "transformer_attention_sdpa_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE = ("encoder_self_base", "bf16")
EXTRA = [("single_head_16", "f32"), ("encoder_self_base", "f32"), ("decoder_causal_base", "bf16"),
         ("cross_big", "bf16"), ("long_causal_8k", "bf16"), ("local_window_8k", "bf16"),
         ("decode_beam_base", "bf16"), ("decode_long_cache", "bf16"), ("encoder_h16_d32", "bf16"),
         ("encoder_h4_d128", "bf16"), ("long_causal_8k_d128", "bf16"), ("encoder_h32_d16", "bf16"),
         ("encoder_dk16_dv64", "bf16"), ("encoder_dk32_dv64", "bf16"), ("encoder_h1_d512", "bf16")]


def algorithmic_work(wl, dtype, key_lens):
    """FLOPs and HBM bytes one step must move, counting legal (query, key) pairs only.

    FLOPs: 2·d_k per score plus 2·d_v per weighted value, i.e. 4·d per legal
    pair (4·n·m·d per head when nothing is masked).  Bytes: Q and O in full,
    plus the K and V rows below each sequence's key length (padded rows are
    never read).
    """
    esz = 2 if dtype == "bf16" else 4
    pairs = 0
    kv_rows = 0
    for b in range(wl.B):
        L = wl.m if key_lens is None else min(max(int(key_lens[b]), 0), wl.m)
        if wl.window is not None:
            # query i sees keys [lo_i, hi_i) around its aligned position c_i
            import numpy as np

            left, right = wl.window[0], wl.window[1]
            align = wl.window[2] if len(wl.window) > 2 else "top_left"
            c = np.arange(wl.n, dtype=np.int64) + (L - wl.n if align == "bottom_right" else 0)
            lo = np.zeros_like(c) if left is None else np.clip(c - left, 0, L)
            hi = np.full_like(c, L) if right is None else np.clip(c + right + 1, 0, L)
            p = int(np.maximum(hi - lo, 0).sum())
        elif wl.causal:
            # query i sees min(i + 1, L) keys
            k = min(L, wl.n)
            p = k * (k + 1) // 2 + (wl.n - k) * L
        else:
            p = wl.n * L
        pairs += wl.h * p
        kv_rows += wl.h * L
    flops = 2 * (wl.d_k + wl.d_v) * pairs
    nbytes = esz * (wl.B * wl.h * wl.n * (wl.d_k + wl.d_v) + kv_rows * (wl.d_k + wl.d_v))
    dense_flops = 2 * (wl.d_k + wl.d_v) * wl.B * wl.h * wl.n * wl.m
    return flops, nbytes, dense_flops


# Source files of each measured kernel (its own file and the shared device header).
KERNEL_SOURCES = {
    "sdpa_short_bf16": ["sdpa_bf16_short.hip", "sdpa_common.hpp"],
    "sdpa_short_f32": ["sdpa_f32_short.hip", "sdpa_common.hpp"],
    "sdpa_long_bf16": ["sdpa_bf16.hip", "sdpa_common.hpp"],
    "sdpa_decode_bf16": ["sdpa_bf16_decode.hip", "sdpa_common.hpp"],
}


def kernel_source_hash(files=None) -> str:
    """Hash of device-code sources: the given files of csrc/ (the kernel whose
    traffic was measured), or every kernel source."""
    if files is None:
        files = sorted(n for n in os.listdir(CSRC) if n.endswith((".hip", ".hpp")))
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, dtype):
    """Per-launch HBM bytes from committed rocprofv3 counter runs, if still
    current: null once the measured kernel's sources changed."""
    path = os.path.join(PROFILES, f"traffic_{workload}_{dtype}.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        t = json.load(f)
    files = t.get("kernel_sources")
    if not files or t.get("kernel_source_hash") != kernel_source_hash(files):
        return None  # the kernel changed since the counters were taken
    return t.get("bytes_per_launch")


class CacheFlush:
    """Evicts the Infinity Cache (and L2) before a timed region: a read of eight
    times the cache's size (2 GiB, about 0.3 ms) on the timing stream.  It only
    reads, so it leaves no dirty lines whose write-back would land in the
    timed region, and it runs long enough for the host to enqueue every timed
    launch behind it."""

    def __init__(self, dev):
        import torch

        self.src = torch.ones(INFINITY_CACHE_BYTES, dtype=torch.int64, device=dev)
        self.nbytes = 8 * self.src.numel()

    def __call__(self):
        self.src.sum()


def timed_launches(launch, steps, stream, flush):
    """HIP-event time (ms) of ``steps`` launches issued one after another on
    ``stream`` right behind a cache flush.  The host enqueues them while the
    flush still runs, so the timed region holds the kernels back to back."""
    import torch

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    flush()
    e0.record()
    for i in range(steps):
        launch(i, stream)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def timed_replay(graph, flush):
    """HIP-event time (ms) of one replay of ``graph`` on the current stream,
    right behind a cache flush.  A replay carries a fixed cost of its own
    (about 15 µs here), so short replays read high per step; it is reported
    as a cross-check."""
    import torch

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    flush()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def time_workload(name, dtype, steps, warmup, clock_warm_s=0.0, case=None, split=False, dropout=0.0):
    """The forward pass of a workload, timed by the driver's protocol (plus a
    graph replay and a long rotation as cross-checks).  split: sdpa_forward_ex
    with a workspace.  dropout p > 0: sdpa_forward_dropout with a seeded keep
    mask per set (keep probability 1 − p, factor 1/(1 − p)), whose words count
    as read."""
    import torch

    from transformer_attention_sdpa_amd import _lib

    _lib.load()
    wl = WORKLOADS[name]
    if case is None:
        case = make_inputs(wl, dtype)
    dev = torch.device("cuda:0")
    if dtype == "bf16":
        from sdpa_inputs import bf16_bits
        import numpy as np

        def up(x):
            return torch.from_numpy(bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)
        tdt, code = torch.bfloat16, _lib.SDPA_BF16
    else:
        def up(x):
            return torch.from_numpy(x).to(dev)
        tdt, code = torch.float32, _lib.SDPA_F32
    q0, k0, v0 = up(case["q"]), up(case["k"]), up(case["v"])
    # Enough copies that one pass over them (Q, O and the legal K/V rows of
    # each copy) exceeds twice the Infinity Cache: a set is evicted before the
    # rotation comes back to it.  The timed replay starts right after a cache
    # flush, so the first sets it touches are cold too, at any step count.
    keep0 = None
    mask_bytes = 0
    if dropout > 0:
        import numpy as np

        from sdpa_inputs import pack_keep, random_keep
        keep0 = torch.from_numpy(pack_keep(random_keep(np.random.default_rng(1234), wl.B, wl.h, wl.n, wl.m,
                                                       dropout)).view(np.int32)).to(dev)
        mask_bytes = keep0.numel() * 4
    touched = algorithmic_work(wl, dtype, case["key_lens"])[1] + mask_bytes
    nsets = max(1, min(64, math.ceil(2 * INFINITY_CACHE_BYTES / touched)))
    sets = []
    for _ in range(nsets):
        q, k, v = q0.clone(), k0.clone(), v0.clone()
        o = torch.empty((wl.B, wl.h, wl.n, wl.d_v), dtype=tdt, device=dev)
        sets.append((q, k, v, o, None if keep0 is None else keep0.clone()))
    kl = None
    kl_ptr = None
    if case["key_lens"] is not None:
        kl = torch.from_numpy(case["key_lens"]).to(dev)
        kl_ptr = kl.data_ptr()
    scale = 1.0 / math.sqrt(wl.d_k)
    mask = _lib.SDPA_MASK_CAUSAL if wl.causal else _lib.SDPA_MASK_NONE
    ptrs = [(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), None if z is None else z.data_ptr())
            for (q, k, v, o, z) in sets]
    ws = None
    if split:  # sdpa_forward_ex with its workspace (decoder steps split into pieces of keys)
        need = _lib.sdpa_forward_workspace_bytes(wl.B, wl.h, wl.n, wl.m, wl.d_k, wl.d_v, code)
        if need == 0:
            raise ValueError(f"{name}: the split path does not apply")
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    if wl.window is not None:
        wleft = -1 if wl.window[0] is None else wl.window[0]
        wright = -1 if wl.window[1] is None else wl.window[1]
        walign = (_lib.SDPA_ALIGN_BOTTOM_RIGHT if len(wl.window) > 2 and wl.window[2] == "bottom_right"
                  else _lib.SDPA_ALIGN_TOP_LEFT)

    def launch(i, stream):
        p = ptrs[i % nsets]
        if p[4] is not None:
            wlft = -1 if wl.window is None else wleft
            wrgt = (0 if wl.causal else -1) if wl.window is None else wright
            wal = _lib.SDPA_ALIGN_TOP_LEFT if wl.window is None else walign
            rc = _lib.sdpa_forward_dropout(p[0], p[1], p[2], p[3], None, wl.B, wl.h, wl.n, wl.m, wl.d_k,
                                           wl.d_v, scale, wlft, wrgt, wal, kl_ptr, p[4], 1.0 / (1.0 - dropout),
                                           code, stream)
        elif ws is not None:
            wlft = -1 if wl.window is None else wleft
            wrgt = (0 if wl.causal else -1) if wl.window is None else wright
            wal = _lib.SDPA_ALIGN_TOP_LEFT if wl.window is None else walign
            rc = _lib.sdpa_forward_ex(p[0], p[1], p[2], p[3], None, wl.B, wl.h, wl.n, wl.m, wl.d_k,
                                      wl.d_v, scale, wlft, wrgt, wal, kl_ptr, code, ws.data_ptr(),
                                      ws.numel(), stream)
        elif wl.window is None:
            rc = _lib.sdpa_forward(p[0], p[1], p[2], p[3], wl.B, wl.h, wl.n, wl.m, wl.d_k, wl.d_v,
                                   scale, mask, kl_ptr, code, stream)
        else:
            rc = _lib.sdpa_forward_window(p[0], p[1], p[2], p[3], wl.B, wl.h, wl.n, wl.m, wl.d_k,
                                          wl.d_v, scale, wleft, wright, walign, kl_ptr, code,
                                          stream)
        if rc != _lib.SDPA_OK:
            raise RuntimeError(_lib.sdpa_strerror(rc))

    stream = torch.cuda.current_stream(dev).cuda_stream
    for i in range(warmup):
        launch(i, stream)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream(dev).cuda_stream
        for i in range(steps):
            launch(i, cs)
    graph.replay()  # first replay uploads the graph; not timed
    torch.cuda.synchronize()
    # Optional untimed replays so that the timed one does not start on clocks
    # that dropped while the host prepared this workload.
    t_warm = time.perf_counter() + clock_warm_s
    while time.perf_counter() < t_warm:
        graph.replay()
        torch.cuda.synchronize()

    flush = CacheFlush(dev)
    w0 = time.perf_counter()
    step_ms = timed_launches(launch, steps, stream, flush)
    wall = time.perf_counter() - w0
    graph_ms = timed_replay(graph, flush)

    # Cross-check over a long rotation: two full passes over every set (at
    # least twice the Infinity Cache of timed bytes whatever --steps is).
    rot = max(steps, 2 * nsets)
    graph_rot = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph_rot):
        cs = torch.cuda.current_stream(dev).cuda_stream
        for i in range(rot):
            launch(i, cs)
    graph_rot.replay()
    torch.cuda.synchronize()
    rot_ms = timed_replay(graph_rot, flush)

    flops, nbytes, dense = algorithmic_work(wl, dtype, case["key_lens"])
    nbytes += mask_bytes
    t = step_ms / 1e3 / steps
    del graph, graph_rot, sets, flush
    torch.cuda.empty_cache()
    return {
        "workload": name, "dtype": dtype, "steps": steps, "sets_rotated": nsets, "dropout": dropout,
        "ms_per_step": step_ms / steps, "ms_per_step_graph": graph_ms / steps,
        "bytes_touched_timed": nbytes * steps,
        "distinct_sets_timed": min(steps, nsets),
        "flushed_before_timing_bytes": 8 * INFINITY_CACHE_BYTES,
        "long_rotation": {"steps": rot, "ms_per_step": rot_ms / rot,
                          "bytes_touched_timed": nbytes * rot, "timing": "graph replay"},
        "wall_s_timed": wall,
        "alg_flops": flops, "dense_flops": dense, "alg_bytes": nbytes,
        "tflops": flops / t / 1e12, "gbs": nbytes / t / 1e9,
        "frac_mfma_peak": flops / t / 1e12 / PEAK_TFLOPS[dtype],
        "frac_hbm_peak": nbytes / t / 1e9 / PEAK_HBM_GBS,
    }


def backward_work(wl, key_lens, dtype="bf16"):
    """Algorithmic FLOPs and HBM bytes of one backward step.

    FLOPs: the five products per legal pair — S recomputed (2·d_k), dP (2·d_v),
    dV (2·d_v), dQ (2·d_k), dK (2·d_k) — i.e. 10·d per pair, 2.5× the forward
    count.  Bytes (at the dtype's element size; the log-sum-exp is fp32 either
    way): Q, O, dO and the log-sum-exp of every query row and the legal K/V
    rows read; dQ and every dK, dV row written.
    """
    esz = 2 if dtype == "bf16" else 4
    fwd_flops, _, _ = algorithmic_work(wl, dtype, key_lens)
    pairs = fwd_flops // (2 * (wl.d_k + wl.d_v))
    flops = 2 * (3 * wl.d_k + 2 * wl.d_v) * pairs
    kv_rows = sum(wl.h * (wl.m if key_lens is None else min(max(int(key_lens[b]), 0), wl.m))
                  for b in range(wl.B))
    rows_q = wl.B * wl.h * wl.n
    nbytes = (esz * rows_q * (wl.d_k + 2 * wl.d_v) + 4 * rows_q + esz * kv_rows * (wl.d_k + wl.d_v)
              + esz * rows_q * wl.d_k + esz * wl.B * wl.h * wl.m * (wl.d_k + wl.d_v))
    return flops, nbytes


def time_backward(name, steps, warmup, clock_warm_s=0.1, dtype="bf16", dropout=0.0):
    """sdpa_backward on a workload, in bf16 or fp32, with the forward output
    and log-sum-exp computed once beforehand (one fused launch per step at
    sentence length in bf16, else the dQ and dK/dV launches).  With dropout
    p > 0: sdpa_forward_dropout / sdpa_backward_dropout with a seeded keep mask
    (keep probability 1 − p, factor 1/(1 − p)), whose words count as read."""
    import numpy as np
    import torch

    from sdpa_inputs import bf16_bits, grad_output, pack_keep, random_keep
    from transformer_attention_sdpa_amd import _lib

    wl = WORKLOADS[name]
    case = make_inputs(wl, dtype)
    dev = torch.device("cuda:0")
    tdt, cdt = ((torch.bfloat16, _lib.SDPA_BF16) if dtype == "bf16" else (torch.float32, _lib.SDPA_F32))

    def up(x):
        if dtype != "bf16":
            return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)
        return torch.from_numpy(bf16_bits(x).view(np.int16)).to(dev).view(torch.bfloat16)

    q0, k0, v0, do0 = up(case["q"]), up(case["k"]), up(case["v"]), up(grad_output(wl, dtype))
    kl = torch.from_numpy(case["key_lens"]).to(dev) if case["key_lens"] is not None else None
    kl_ptr = None if kl is None else kl.data_ptr()
    B, h, n, m, d = wl.B, wl.h, wl.n, wl.m, wl.d_k
    scale = 1.0 / math.sqrt(d)
    if wl.window is None:
        wleft, wright, walign = -1, (0 if wl.causal else -1), _lib.SDPA_ALIGN_TOP_LEFT
    else:
        wleft = -1 if wl.window[0] is None else wl.window[0]
        wright = -1 if wl.window[1] is None else wl.window[1]
        walign = (_lib.SDPA_ALIGN_BOTTOM_RIGHT if len(wl.window) > 2 and wl.window[2] == "bottom_right"
                  else _lib.SDPA_ALIGN_TOP_LEFT)
    flops, nbytes = backward_work(wl, case["key_lens"], dtype)
    keep0, keep_scale = None, 1.0
    if dropout > 0:
        keep0 = torch.from_numpy(pack_keep(random_keep(np.random.default_rng(1234), B, h, n, m, dropout))
                                 .view(np.int32)).to(dev)
        keep_scale = 1.0 / (1.0 - dropout)
        nbytes += keep0.numel() * 4
    nsets = max(1, min(64, math.ceil(2 * INFINITY_CACHE_BYTES / nbytes)))
    need = _lib.sdpa_backward_workspace_bytes(B, h, n)
    stream = torch.cuda.current_stream(dev).cuda_stream
    sets = []
    for _ in range(nsets):
        q, k, v, do = q0.clone(), k0.clone(), v0.clone(), do0.clone()
        o = torch.empty((B, h, n, d), dtype=tdt, device=dev)
        lse = torch.empty((B, h, n), dtype=torch.float32, device=dev)
        keep = None if keep0 is None else keep0.clone()
        if keep is None:
            rc = _lib.sdpa_forward_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                       B, h, n, m, d, d, scale, wleft, wright, walign, kl_ptr, cdt, stream)
        else:
            rc = _lib.sdpa_forward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                           B, h, n, m, d, d, scale, wleft, wright, walign, kl_ptr,
                                           keep.data_ptr(), keep_scale, cdt, stream)
        if rc != _lib.SDPA_OK:
            raise RuntimeError(_lib.sdpa_strerror(rc))
        grads = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        sets.append((q, k, v, o, do, lse, *grads, ws, keep))

    def launch(i, st):
        q, k, v, o, do, lse, dq, dk, dv, ws, keep = sets[i % nsets]
        if keep is None:
            rc = _lib.sdpa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, h, n, m,
                                    d, d, scale, wleft, wright, walign, kl_ptr, cdt, ws.data_ptr(), need, st)
        else:
            rc = _lib.sdpa_backward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                            do.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                            dv.data_ptr(), B, h, n, m, d, d, scale, wleft, wright, walign,
                                            kl_ptr, keep.data_ptr(), keep_scale, cdt, ws.data_ptr(), need, st)
        if rc != _lib.SDPA_OK:
            raise RuntimeError(_lib.sdpa_strerror(rc))

    for i in range(warmup):
        launch(i, stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream(dev).cuda_stream
        for i in range(steps):
            launch(i, cs)
    graph.replay()
    torch.cuda.synchronize()
    t_warm = time.perf_counter() + clock_warm_s
    while time.perf_counter() < t_warm:
        graph.replay()
        torch.cuda.synchronize()
    flush = CacheFlush(dev)
    t = timed_launches(launch, steps, stream, flush) / 1e3 / steps
    t_graph = timed_replay(graph, flush) / 1e3 / steps
    del graph, sets, flush
    torch.cuda.empty_cache()
    return {"ms_per_step": t * 1e3, "ms_per_step_graph": t_graph * 1e3,
            "tflops": flops / t / 1e12, "gbs": nbytes / t / 1e9,
            "alg_flops": flops, "alg_bytes": nbytes,
            "frac_mfma_peak": flops / t / 1e12 / PEAK_TFLOPS[dtype],
            "frac_hbm_peak": nbytes / t / 1e9 / PEAK_HBM_GBS, "steps": steps, "sets_rotated": nsets,
            "launches_per_step": (1 if dtype == "bf16" and n <= 64 and m <= 64
                                  else 3 if dtype == "bf16" and d == 128 else 2),
            "dropout": dropout}


def mha_work(args, key_lens):
    """Algorithmic FLOPs and external HBM bytes of one multi-head sublayer step.

    FLOPs: the three input projections and the output projection (2 per
    multiply-add, dense), plus the attention's 4·d per legal pair.  Bytes: the
    sublayer's inputs, its four weight matrices and its output, each once (the
    projected Q, K, V and the head outputs are intermediate)."""
    from sdpa_inputs import Workload

    B, n, m, d_model, h = args["B"], args["n"], args["m"], args["d_model"], args["h"]
    hw = 64 * h
    proj = 2 * d_model * hw * (B * n + 2 * B * m) + 2 * B * n * hw * d_model
    wl = Workload("mha", B=B, h=h, n=n, m=m, d_k=64, d_v=64, causal=False,
                  key_len_range=args.get("key_len_range"), seed=0)
    att = algorithmic_work(wl, "bf16", key_lens)[0]
    self_att = args.get("self_attention", True)
    nbytes = 2 * (B * n * d_model * (2 if self_att else 1) + (0 if self_att else B * m * d_model)
                  + 4 * hw * d_model)
    return proj + att, nbytes, proj, att


def time_mha(name, steps, warmup, clock_warm_s=0.1):
    """The multi-head sublayer (three launches per step) on one of MHA_WORKLOADS."""
    import numpy as np
    import torch

    from sdpa_inputs import MHA_WORKLOADS, bf16_bits, mha_case
    from transformer_attention_sdpa_amd import _lib

    args = MHA_WORKLOADS[name]
    c = mha_case(**args)
    B, n, m, d_model, h = args["B"], args["n"], args["m"], args["d_model"], args["h"]
    dev = torch.device("cuda:0")

    def up(x):
        return torch.from_numpy(np.ascontiguousarray(bf16_bits(x)).view(np.int16)).to(dev).view(torch.bfloat16)

    rows = lambda w: np.ascontiguousarray(w.transpose(0, 2, 1).reshape(h * 64, d_model))
    wq, wk, wv, wo = up(rows(c["wq"])), up(rows(c["wk"])), up(rows(c["wv"])), up(np.ascontiguousarray(c["wo"].T))
    xq0 = up(c["xq"])
    xkv0 = xq0 if args.get("self_attention", True) else up(c["xkv"])
    need = _lib.sdpa_mha_workspace_bytes(B, n, m, h, 64, 64)
    flops, nbytes, _, _ = mha_work(args, c["key_lens"])
    per_set = nbytes + need
    nsets = max(1, min(64, math.ceil(2 * INFINITY_CACHE_BYTES / per_set)))
    sets = []
    for _ in range(nsets):
        xq = xq0.clone()
        xkv = xq if xkv0 is xq0 else xkv0.clone()
        sets.append((xq, xkv, torch.empty((B, n, d_model), dtype=torch.bfloat16, device=dev),
                     torch.empty(need, dtype=torch.uint8, device=dev)))
    kl = torch.from_numpy(c["key_lens"]).to(dev) if c["key_lens"] is not None else None

    def launch(i, stream):
        xq, xkv, out, ws = sets[i % nsets]
        rc = _lib.sdpa_mha_forward(xq.data_ptr(), xkv.data_ptr(), wq.data_ptr(), wk.data_ptr(),
                                   wv.data_ptr(), wo.data_ptr(), out.data_ptr(), B, n, m, d_model, h,
                                   64, 64, 0.125, -1, -1, 0, None if kl is None else kl.data_ptr(),
                                   _lib.SDPA_BF16, ws.data_ptr(), need, stream)
        if rc != _lib.SDPA_OK:
            raise RuntimeError(_lib.sdpa_strerror(rc))

    stream = torch.cuda.current_stream(dev).cuda_stream
    for i in range(warmup):
        launch(i, stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream(dev).cuda_stream
        for i in range(steps):
            launch(i, cs)
    graph.replay()
    torch.cuda.synchronize()
    t_warm = time.perf_counter() + clock_warm_s
    while time.perf_counter() < t_warm:
        graph.replay()
        torch.cuda.synchronize()
    flush = CacheFlush(dev)
    t = timed_launches(launch, steps, stream, flush) / 1e3 / steps
    t_graph = timed_replay(graph, flush) / 1e3 / steps
    del graph, sets, flush
    torch.cuda.empty_cache()
    return {"ms_per_step": t * 1e3, "ms_per_step_graph": t_graph * 1e3,
            "tflops": flops / t / 1e12, "gbs": nbytes / t / 1e9,
            "frac_mfma_peak": flops / t / 1e12 / PEAK_TFLOPS["bf16"],
            "frac_hbm_peak": nbytes / t / 1e9 / PEAK_HBM_GBS, "steps": steps, "sets_rotated": nsets,
            "launches_per_step": 3}


def copy_reference(steps, warmup, nbytes=256 << 20):
    """A plain device-to-device copy of known size: the yardstick that scales the
    FETCH_SIZE / WRITE_SIZE counters of the attention kernel to bytes."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "steps": steps,
            "ms_per_copy": t * 1e3, "gbs_read_plus_write": 2 * nbytes / t / 1e9}


def rocprof_summary(db_path) -> str:
    """Text summary of a rocprofv3 results database: per-kernel dispatch
    durations (kernel trace) and per-dispatch means of any PMC counters."""
    import sqlite3
    import statistics
    from collections import defaultdict

    con = sqlite3.connect(db_path)
    out = []
    rows = list(con.execute("select name, start, end from kernels order by start"))
    per = defaultdict(list)
    for name, t0, t1 in rows:
        per[name].append((t1 - t0) / 1e3)
    if per:
        out.append(f"{'kernel':64s} {'calls':>6s} {'mean_us':>9s} {'median_us':>9s} "
                   f"{'p10_us':>8s} {'p90_us':>8s}")
        for name, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            d2 = sorted(d)
            out.append(f"{name[:64]:64s} {len(d):6d} {statistics.mean(d):9.3f} "
                       f"{d2[len(d2) // 2]:9.3f} {d2[len(d2) // 10]:8.3f} {d2[9 * len(d2) // 10]:8.3f}")
    try:
        pmc = list(con.execute("select kernel_name, counter_name, value from counters_collection"))
    except sqlite3.Error:
        pmc = []
    if pmc:
        agg = defaultdict(list)
        for k, c, v in pmc:
            agg[(k, c)].append(v)
        out.append("")
        out.append(f"{'kernel':64s} {'counter':28s} {'dispatches':>10s} {'mean_per_dispatch':>18s}")
        for (k, c), v in sorted(agg.items()):
            out.append(f"{k[:64]:64s} {c:28s} {len(v):10d} {statistics.mean(v):18.6g}")
    return "\n".join(out)


def pmc_mean(db_path, kernel_substr, counter):
    import sqlite3
    import statistics

    con = sqlite3.connect(db_path)
    vals = [v for k, c, v in con.execute(
        "select kernel_name, counter_name, value from counters_collection")
        if kernel_substr in k and c == counter]
    if not vals:
        raise SystemExit(f"no {counter} samples for a kernel matching {kernel_substr!r} in {db_path}")
    return statistics.mean(vals)


def traffic_record(fetch_db, write_db, copy_fetch_db, copy_write_db, copy_bytes, kernel, workload,
                   dtype):
    """Per-launch HBM bytes of `kernel` from FETCH_SIZE / WRITE_SIZE runs, each
    scaled by what the same counter reads for a copy of `copy_bytes` bytes."""
    f = pmc_mean(fetch_db, kernel, "FETCH_SIZE")
    w = pmc_mean(write_db, kernel, "WRITE_SIZE")
    cf = pmc_mean(copy_fetch_db, "copyBuffer", "FETCH_SIZE")
    cw = pmc_mean(copy_write_db, "copyBuffer", "WRITE_SIZE")
    sf = copy_bytes / 1024.0 / cf
    sw = copy_bytes / 1024.0 / cw
    read_b = f * sf * 1024.0
    write_b = w * sw * 1024.0
    return {"kernel": kernel, "workload": workload, "dtype": dtype,
            "fetch_kib_per_dispatch": f, "write_kib_per_dispatch": w,
            "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw,
            "fetch_scale": sf, "write_scale": sw,
            "read_bytes_per_launch": read_b, "write_bytes_per_launch": write_b,
            "bytes_per_launch": read_b + write_b,
            "kernel_sources": KERNEL_SOURCES.get(kernel),
            "kernel_source_hash": kernel_source_hash(KERNEL_SOURCES.get(kernel))}


def _oracle_slice_worker(name, dtype, b0, b1, budget_s, ready, go, results):
    """One host core's share of the CPU baseline: the unchanged oracle on batch
    elements [b0, b1) of the workload, one BLAS thread, passes until the
    budget.  Runs in a spawned process that never touches the GPU."""
    import oracle.sdpa_oracle as so
    from threadpoolctl import threadpool_limits

    wl = WORKLOADS[name]
    case = make_inputs(wl, dtype)
    q, k, v = (case[x][b0:b1] for x in ("q", "k", "v"))
    kl = None if case["key_lens"] is None else case["key_lens"][b0:b1]
    with threadpool_limits(limits=1):
        ready.put(b0)
        go.wait()
        t0 = time.monotonic()
        reps = 0
        while True:
            so.attention(q, k, v, causal=wl.causal, key_lens=kl, window=wl.window)
            reps += 1
            t1 = time.monotonic()
            if t1 - t0 >= budget_s:
                break
    results.put((b0, b1, reps, t0, t1))


def cpu_worker_count(B: int) -> int:
    """Host cores the CPU baseline uses: every core this process may run on,
    at most 16 (one GPU's share of the host) and at most one per batch element."""
    return max(1, min(16, len(os.sched_getaffinity(0)), B))


def cpu_baseline(name, dtype, budget_s=10.0):
    """The fp64 oracle, as it stands, on the host cores: the batch is split over
    one process per usable core (each on one BLAS thread; the oracle's 64×64
    products gain nothing from more), every process repeats whole passes over
    its batch elements for the budget, and the rate is the work all of them
    finished over the span from the first start to the last end."""
    import dataclasses
    import multiprocessing as mp

    wl = WORKLOADS[name]
    key_lens = make_inputs(wl, dtype)["key_lens"]
    workers = cpu_worker_count(wl.B)
    bounds = [wl.B * i // workers for i in range(workers + 1)]
    ctx = mp.get_context("spawn")  # fresh interpreters: nothing of this process's GPU state
    ready, results, go = ctx.Queue(), ctx.Queue(), ctx.Event()
    procs = [ctx.Process(target=_oracle_slice_worker,
                         args=(name, dtype, bounds[i], bounds[i + 1], budget_s, ready, go, results))
             for i in range(workers)]
    for p in procs:
        p.start()
    for _ in procs:
        ready.get(timeout=300)
    go.set()
    done = [results.get(timeout=budget_s * 10 + 300) for _ in procs]
    for p in procs:
        p.join()
    flops = 0
    for b0, b1, reps, _, _ in done:
        part = dataclasses.replace(wl, B=b1 - b0)
        kl = None if key_lens is None else key_lens[b0:b1]
        flops += reps * algorithmic_work(part, dtype, kl)[0]
    span = max(r[4] for r in done) - min(r[3] for r in done)
    whole = algorithmic_work(wl, dtype, key_lens)[0]
    return {"value": flops / span / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"{name} ({wl.B * wl.h} heads, {dtype} values in fp64) split over {workers} "
                      f"processes by batch element, {flops / whole:.1f} whole-batch passes "
                      f"in {span:.1f} s, {span / (flops / whole) * 1e3:.1f} ms per pass",
            "host": host_description()}


def host_description() -> dict:
    """CPU model, usable cores and the BLAS numpy calls (recorded beside the oracle timing)."""
    import numpy as np

    model = "unknown"
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        b = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {})
        blas = f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:  # older numpy: no dict mode
        pass
    return {"cpu_model": model, "usable_cores": len(os.sched_getaffinity(0)), "blas": blas}


def _legal_keys(wl, key_lens, b, i):
    """Number of keys query row i of batch element b may attend to."""
    L = wl.m if key_lens is None else min(max(int(key_lens[b]), 0), wl.m)
    if wl.window is not None:
        left, right = wl.window[0], wl.window[1]
        c = i + (L - wl.n if len(wl.window) > 2 and wl.window[2] == "bottom_right" else 0)
        lo = 0 if left is None else min(max(c - left, 0), L)
        hi = L if right is None else min(max(c + right + 1, 0), L)
        return max(hi - lo, 0)
    return min(i + 1, L) if wl.causal else L


def oracle_pass(name, dtype, max_s=2.0, case=None):
    """The oracle on one workload, single BLAS thread: a whole batch when it is
    small, else a seeded sample of output rows (cost counted per legal pair)."""
    import numpy as np

    import oracle.sdpa_oracle as so
    from threadpoolctl import threadpool_limits

    wl = WORKLOADS[name]
    if case is None:
        case = make_inputs(wl, dtype)
    with threadpool_limits(limits=1):
        if wl.n * wl.m <= 64 * 64:
            flops, _, _ = algorithmic_work(wl, dtype, case["key_lens"])
            t0 = time.perf_counter()
            so.attention(case["q"], case["k"], case["v"], causal=wl.causal,
                         key_lens=case["key_lens"], window=wl.window)
            el = time.perf_counter() - t0
            return {"tflops": flops / el / 1e12, "ms_per_pass": el * 1e3, "sample": "whole batch"}
        rng = np.random.default_rng(7)
        picks, pairs = [], 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < max_s and len(picks) < 4096:
            b, hh, i = int(rng.integers(wl.B)), int(rng.integers(wl.h)), int(rng.integers(wl.n))
            so.attention_rows(case["q"], case["k"], case["v"], [(b, hh, i)], causal=wl.causal,
                              key_lens=case["key_lens"], window=wl.window)
            picks.append((b, hh, i))
            pairs += _legal_keys(wl, case["key_lens"], b, i)
        el = time.perf_counter() - t0
        flops_s = 2 * (wl.d_k + wl.d_v) * pairs / el
        full, _, _ = algorithmic_work(wl, dtype, case["key_lens"])
        return {"tflops": flops_s / 1e12, "ms_per_pass": full / flops_s * 1e3,
                "sample": f"{len(picks)} random output rows in {el:.1f} s; ms_per_pass extrapolated"}


def context(steps=400):
    """The practical matrix-core ceiling on this board: a plain bf16 GEMM through
    torch.matmul (hipBLASLt), sustained, so the board reaches the same
    power-limited state as the attention kernel, timed beside this library on
    the long causal workload's shape.  Context only; not a step."""
    import torch

    import transformer_attention_sdpa_amd as sdpa

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)

    def per_call(fn, iters, warm=3):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / iters

    out = {"what": "context: library GEMM ceiling on this GPU"}
    N = 8192
    a = torch.randn(N, N, device=dev, dtype=torch.bfloat16, generator=gen)
    b = torch.randn(N, N, device=dev, dtype=torch.bfloat16, generator=gen)
    c = torch.empty(N, N, device=dev, dtype=torch.bfloat16)
    t = per_call(lambda: torch.matmul(a, b, out=c), steps)
    out["gemm_bf16_8192cubed"] = {"calls": steps, "us_per_call": t * 1e6,
                                  "tflops": 2 * N ** 3 / t / 1e12,
                                  "frac_bf16_peak": 2 * N ** 3 / t / 1e12 / PEAK_TFLOPS["bf16"]}
    del a, b, c

    wl = WORKLOADS["long_causal_8k"]
    q, k, v = (torch.randn(wl.B, wl.h, wl.n, wl.d_k, device=dev, dtype=torch.bfloat16,
                           generator=gen) for _ in range(3))
    flops = 4 * wl.d_k * (wl.n * (wl.n + 1) // 2) * wl.B * wl.h
    ours = sdpa.forward(q, k, v, causal=True)
    t = per_call(lambda: sdpa.forward(q, k, v, causal=True, out=ours), 50)
    out["this_library_long_causal_8k"] = {"us_per_call": t * 1e6, "tflops": flops / t / 1e12}
    out["torch"] = torch.__version__
    return out


def context_gemm_shapes(iters=200):
    """The multi-head sublayer's projection GEMMs through torch.matmul
    (hipBLASLt), for a kernel trace beside this library's sublayer: per
    workload, Q, K, V as one GEMM when the sublayer attends to itself (Q
    alone and K, V together otherwise) and the output projection.  Per-call
    event times of these small GEMMs are bound by the host's launch rate;
    the kernel durations come from the trace.  Context only; not a step."""
    import torch

    from sdpa_inputs import MHA_WORKLOADS

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    out = {"what": "context: library GEMMs on the sublayer's projection shapes"}
    for name, a in MHA_WORKLOADS.items():
        B, n, m, dm, hw = a["B"], a["n"], a["m"], a["d_model"], 64 * a["h"]
        self_att = a.get("self_attention", True)
        shapes = ([("qkv", B * n, dm, 3 * hw)] if self_att else [("q", B * n, dm, hw), ("kv", B * m, dm, 2 * hw)])
        shapes.append(("out", B * n, hw, dm))
        for what, M, K, N in shapes:
            x = torch.randn(M, K, device=dev, dtype=torch.bfloat16, generator=gen)
            w = torch.randn(K, N, device=dev, dtype=torch.bfloat16, generator=gen)
            y = torch.empty(M, N, device=dev, dtype=torch.bfloat16)
            for _ in range(20):
                torch.matmul(x, w, out=y)
            torch.cuda.synchronize()
            for _ in range(iters):
                torch.matmul(x, w, out=y)
            torch.cuda.synchronize()
            out[f"{name}/{what}"] = {"M": M, "K": K, "N": N, "calls": 20 + iters}
    out["torch"] = torch.__version__
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=HEADLINE[0], choices=sorted(WORKLOADS))
    ap.add_argument("--dtype", default=HEADLINE[1], choices=["bf16", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split", action="store_true",
                    help="with --workload: time sdpa_forward_ex with its workspace (split decoder steps)")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a plain device copy instead (reference for HBM counters)")
    ap.add_argument("--copy-mib", type=float, default=256.0, help="size of --calibrate-copy")
    ap.add_argument("--rocprof-summary", nargs="+", metavar="DB",
                    help="print a text summary of rocprofv3 result databases and exit")
    ap.add_argument("--traffic-json", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB",
                                                        "COPY_WRITE_DB"),
                    help="print the per-launch HBM traffic record of --kernel and exit")
    ap.add_argument("--kernel", default="sdpa_short_bf16", help="kernel name for --traffic-json")
    ap.add_argument("--backward", choices=["encoder_self_base", "decoder_causal_base", "long_causal_8k",
                                           "encoder_h16_d32", "encoder_h4_d128", "long_causal_8k_d128"],
                    help="time only the backward pass of this workload (one JSON line)")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="attention dropout probability of the timed pass (--workload or --backward; "
                         "default 0: none)")
    ap.add_argument("--mha", choices=["mha_encoder_base", "mha_cross_big"],
                    help="time only this multi-head sublayer workload (one JSON line)")
    ap.add_argument("--context", action="store_true",
                    help="time a library bf16 GEMM (the matrix-core ceiling) beside this library")
    ap.add_argument("--context-gemm-shapes", action="store_true",
                    help="run library GEMMs of the sublayer's projection shapes (for a kernel trace)")
    args = ap.parse_args()

    if args.rocprof_summary:
        for db in args.rocprof_summary:
            print(f"== {db}")
            print(rocprof_summary(db))
        return
    if args.traffic_json:
        rec = traffic_record(*args.traffic_json, int(args.copy_mib * (1 << 20)), args.kernel,
                             args.workload, args.dtype)
        print(json.dumps(rec, indent=1))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every (batch, head) pair is independent and the "
              "library has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.context:
        print(json.dumps(context()), flush=True)
        return
    if args.context_gemm_shapes:
        print(json.dumps(context_gemm_shapes()), flush=True)
        return
    if args.backward:
        print(json.dumps({"workload": args.backward, "pass": "backward",
                          "dtype": args.dtype,
                          **time_backward(args.backward, args.steps, args.warmup, dtype=args.dtype,
                                          dropout=args.dropout)}), flush=True)
        return
    if args.mha:
        print(json.dumps({"workload": args.mha, **time_mha(args.mha, args.steps, args.warmup)}), flush=True)
        return
    if args.calibrate_copy:
        print(json.dumps(copy_reference(args.steps, args.warmup, int(args.copy_mib * (1 << 20)))),
              flush=True)
        return

    wl = WORKLOADS[args.workload]
    head = time_workload(args.workload, args.dtype, args.steps, args.warmup, split=args.split,
                         dropout=args.dropout)
    extra = {}
    if not args.no_extra:
        # Every GPU measurement first, then the CPU oracle passes.  Each extra
        # workload replays its graph untimed for 0.1 s before the timed replay,
        # since its inputs were generated on the host while the GPU idled.
        # Each workload's inputs are drawn once and serve its GPU timing and,
        # afterwards, its oracle pass.
        cases = {}
        for name, dt in EXTRA:
            if (name, dt) == (args.workload, args.dtype):
                continue
            st = 20 if name.endswith(("_8k", "_cache")) else max(10, min(args.steps, 200))
            cases[name, dt] = make_inputs(WORKLOADS[name], dt)
            r = time_workload(name, dt, st, min(args.warmup, 5), clock_warm_s=0.1,
                              case=cases[name, dt])
            extra[f"{name}-{dt}"] = {k: r[k] for k in (
                "ms_per_step", "tflops", "gbs", "frac_mfma_peak", "frac_hbm_peak", "steps",
                "sets_rotated", "ms_per_step_graph", "bytes_touched_timed", "long_rotation")}
            if args.no_cpu_baseline:
                del cases[name, dt]
        # decoder steps with each head's keys split over several workgroups
        # (sdpa_forward_ex with a workspace): 256 heads, and one sequence alone
        for name in ("decode_long_cache", "decode_one_sequence"):
            r = time_workload(name, "bf16", 20, min(args.warmup, 5), clock_warm_s=0.1, split=True)
            extra[f"{name}-bf16-split"] = {k: r[k] for k in (
                "ms_per_step", "tflops", "gbs", "frac_mfma_peak", "frac_hbm_peak", "steps",
                "sets_rotated", "ms_per_step_graph")}
        # attention dropout (p = 0.1) in the forward pass: sentence length and 8k causal
        for name in ("encoder_self_base", "long_causal_8k"):
            r = time_workload(name, "bf16", 20 if name.endswith("_8k") else max(10, min(args.steps, 200)),
                              min(args.warmup, 5), clock_warm_s=0.1, dropout=0.1)
            extra[f"{name}-bf16-dropout0.1"] = {k: r[k] for k in (
                "ms_per_step", "tflops", "gbs", "frac_mfma_peak", "frac_hbm_peak", "steps",
                "sets_rotated", "ms_per_step_graph")}
        for name in ("encoder_self_base", "long_causal_8k"):
            for dt in ("bf16", "f32"):
                extra[f"backward-{name}-{dt}"] = time_backward(
                    name, (20 if dt == "bf16" else 5) if name.endswith("_8k") else max(10, min(args.steps, 200)),
                    min(args.warmup, 3), dtype=dt)
        # Table 3 widths and attention dropout (p = 0.1) at sentence length
        for name, p in (("encoder_h16_d32", 0.0), ("encoder_h4_d128", 0.0), ("encoder_self_base", 0.1)):
            key = f"backward-{name}-bf16" + (f"-dropout{p}" if p else "")
            extra[key] = time_backward(name, max(10, min(args.steps, 200)), min(args.warmup, 3), dropout=p)
        for name in ("mha_encoder_base", "mha_cross_big"):
            extra[f"{name}-bf16"] = time_mha(name, max(10, min(args.steps, 200)),
                                             min(args.warmup, 5))
        if not args.no_cpu_baseline:
            for (name, dt), case in cases.items():
                extra[f"{name}-{dt}"]["cpu_oracle_1core"] = oracle_pass(name, dt, case=case)
            cases.clear()

    bound = "mfma" if head["alg_flops"] / head["alg_bytes"] > PEAK_TFLOPS[args.dtype] * 1e12 / (PEAK_HBM_GBS * 1e9) else "hbm"
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": head["gbs"] / PEAK_HBM_GBS}
    else:
        roof = {"bound": "mfma", "achieved": head["tflops"], "peak": PEAK_TFLOPS[args.dtype],
                "unit": "TFLOP/s", "frac": head["tflops"] / PEAK_TFLOPS[args.dtype]}
    roof["traffic"] = measured_traffic(args.workload, args.dtype)

    line = {
        "metric": "attention TFLOP/s and % of MI355X bf16 MFMA / HBM peak, h=8 d_k=64",
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic N(0,1), seeded",
        "config": {"workload": args.workload, "B": wl.B, "h": wl.h, "n": wl.n, "m": wl.m,
                   "d_k": wl.d_k, "d_v": wl.d_v, "causal": wl.causal,
                   "key_len_range": wl.key_len_range, "seed": wl.seed,
                   **({"dropout": args.dropout} if args.dropout else {})},
        "roofline": roof,
        "alg_bytes_per_step": head["alg_bytes"],
        "alg_flops_per_step": head["alg_flops"],
        "frac_hbm_peak": head["frac_hbm_peak"],
        "frac_mfma_peak": head["frac_mfma_peak"],
        "ms_per_step_graph": head["ms_per_step_graph"],
        "sets_rotated": head["sets_rotated"],
        "bytes_touched_timed": head["bytes_touched_timed"],
        "distinct_sets_timed": head["distinct_sets_timed"],
        "flushed_before_timing_bytes": head["flushed_before_timing_bytes"],
        "long_rotation": head["long_rotation"],
        "kernel_source_hash": kernel_source_hash(),
    }
    if extra:
        line["other_workloads"] = extra
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload, args.dtype)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
