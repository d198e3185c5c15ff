"""MI355X-native fused scaled dot-product attention (gfx950 HIP kernels).

``forward(q, k, v, *, causal=False, key_lens=None, scale=None, out=None)``
computes Eq. (1) of the pages, softmax(Q Kᵀ/√d_k) V, per (batch, head) on
[B, h, len, 64] tensors of dtype float32 or bfloat16 that live on the GPU.
PyTorch only supplies the device memory and the current stream; the work is
one launch of the HIP library ``libsdpa.so`` through its C ABI.
"""

from __future__ import annotations

import math

from . import _lib
from ._lib import (sdpa_backward, sdpa_backward_dropout, sdpa_backward_workspace_bytes,  # noqa: F401
                   sdpa_forward, sdpa_forward_dropout, sdpa_forward_ex, sdpa_forward_ex_noalloc,
                   sdpa_forward_lse, sdpa_forward_strided, sdpa_forward_window,
                   sdpa_forward_workspace_bytes, sdpa_mha_forward,
                   sdpa_mha_workspace_bytes, sdpa_strerror, sdpa_version)

__all__ = ["forward", "backward", "mha_forward", "dropout_keep_mask", "forward_dropout", "backward_dropout",
           "sdpa_forward", "sdpa_forward_window",
           "sdpa_forward_lse", "sdpa_forward_ex", "sdpa_forward_ex_noalloc", "sdpa_forward_strided",
           "sdpa_forward_workspace_bytes", "sdpa_forward_dropout", "sdpa_backward_dropout",
           "sdpa_backward", "sdpa_backward_workspace_bytes",
           "sdpa_mha_forward", "sdpa_mha_workspace_bytes", "sdpa_strerror", "sdpa_version"]


def _window_args(window, causal, n=None, m=None):
    """(window_left, window_right, align code) for the C ABI.

    The decoder's causal mask is the top-left window (unbounded, 0), which is
    the inclusive j <= i rule only when the queries and keys are the same
    sequence: with n != m it is rejected here, whichever entry point the call
    then takes (a bottom-right window is the decoder-step form)."""
    if window is None:
        if causal and n is not None and n != m:
            raise ValueError("the causal mask needs n == m; use window=(None, 0, 'bottom_right') "
                             "for queries at the end of a longer key sequence")
        return -1, (0 if causal else -1), _lib.SDPA_ALIGN_TOP_LEFT
    if causal:
        raise ValueError("give the causal mask as window=(None, 0) instead of combining both")
    left, right = window[0], window[1]
    align = window[2] if len(window) > 2 else "top_left"
    if align not in ("top_left", "bottom_right"):
        raise ValueError(f"unknown window alignment {align!r}")
    if any(x is not None and int(x) < 0 for x in (left, right)):
        raise ValueError("window sides are >= 0 or None (unbounded)")
    # the library treats any side wider than n + m as unbounded
    wl = -1 if left is None else min(int(left), 2**31 - 1)
    wr = -1 if right is None else min(int(right), 2**31 - 1)
    al = _lib.SDPA_ALIGN_BOTTOM_RIGHT if align == "bottom_right" else _lib.SDPA_ALIGN_TOP_LEFT
    return wl, wr, al


def mha_forward(x_q, x_kv, w_q, w_k, w_v, w_o, *, heads: int, causal: bool = False,
                key_lens=None, scale: float | None = None, window=None, out=None, workspace=None):
    """The multi-head attention sublayer, bf16 (``sdpa_mha_forward`` in
    include/sdpa.h): Concat(head_1..head_h) W^O with head_i =
    Attention(x_q W_i^Q, x_kv W_i^K, x_kv W_i^V).

    x_q [B, n, d_model] and x_kv [B, m, d_model] (pass the same tensor for
    self-attention); w_q, w_k, w_v [heads·d, d_model] and w_o [d_model,
    heads·d] in the [out, in] layout, d = 32, 64 or 128.  ``causal``, ``window``, ``key_lens``
    and ``scale`` as in ``forward``.  ``workspace``: a uint8 GPU tensor of at
    least ``sdpa_mha_workspace_bytes`` bytes, or None to have one allocated
    here (the library itself allocates nothing).  Returns ``out`` [B, n,
    d_model].
    """
    import torch

    for t in (x_q, x_kv, w_q, w_k, w_v, w_o):
        if not t.is_cuda or t.device != x_q.device:
            raise ValueError("all tensors must be on one GPU")
        if t.dtype != torch.bfloat16:
            raise ValueError("the sublayer runs in bf16")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    if x_q.dim() != 3 or x_kv.dim() != 3:
        raise ValueError("x_q must be [B, n, d_model] and x_kv [B, m, d_model]")
    B, n, d_model = x_q.shape
    m = x_kv.shape[1]
    if w_q.dim() != 2 or w_q.shape[0] % heads:
        raise ValueError("w_q must be [heads·d, d_model]")
    d = w_q.shape[0] // heads  # head width d_k = d_v
    hw = heads * d
    if (tuple(x_kv.shape) != (B, m, d_model) or tuple(w_q.shape) != (hw, d_model)
            or tuple(w_k.shape) != (hw, d_model) or tuple(w_v.shape) != (hw, d_model)
            or tuple(w_o.shape) != (d_model, hw)):
        raise ValueError("shape mismatch between inputs and projections")
    kl_ptr = None
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or key_lens.device != x_q.device or key_lens.numel() != B:
            raise ValueError("key_lens must be an int32 tensor of B elements on the inputs' device")
        key_lens = key_lens.contiguous()
        kl_ptr = key_lens.data_ptr()
    wl, wr, al = _window_args(window, causal, n, m)
    need = sdpa_mha_workspace_bytes(B, n, m, heads, d, d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x_q.device)
    if out is None:
        out = torch.empty((B, n, d_model), dtype=torch.bfloat16, device=x_q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    with torch.cuda.device(x_q.device):
        stream = torch.cuda.current_stream(x_q.device).cuda_stream
        rc = sdpa_mha_forward(x_q.data_ptr(), x_kv.data_ptr(), w_q.data_ptr(), w_k.data_ptr(),
                              w_v.data_ptr(), w_o.data_ptr(), out.data_ptr(), B, n, m, d_model,
                              heads, d, d, float(scale), wl, wr, al, kl_ptr, _lib.SDPA_BF16,
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                              stream)
    if rc != _lib.SDPA_OK:
        raise RuntimeError(f"sdpa_mha_forward failed ({rc}): {sdpa_strerror(rc)}")
    return out


def _lengths(q, k):
    """(n, m) of [B, h, n, d] queries and [B, h, m, d] keys (None when not 4-D;
    ``_check_qkv`` then rejects them)."""
    if q.dim() != 4 or k.dim() != 4:
        return None, None
    return q.shape[2], k.shape[2]


def _check_qkv(q, k, v, strided_ok=False):
    """Shapes and the dtype code of [B, h, n, d_k], [B, h, m, d_k], [B, h, m, d_v] GPU tensors
    (packed, or with ``strided_ok`` any strides whose last dimension is contiguous)."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, h, len, d]")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share one dtype")
    if q.dtype == torch.float32:
        dt = _lib.SDPA_F32
    elif q.dtype == torch.bfloat16:
        dt = _lib.SDPA_BF16
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    for t in (q, k, v):
        if strided_ok:
            if t.stride(-1) != 1 and t.shape[-1] != 1:
                raise ValueError("q, k, v need a contiguous last dimension")
        elif not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    B, h, n, d_k = q.shape
    m, d_v = k.shape[2], v.shape[3]
    if tuple(k.shape) != (B, h, m, d_k) or tuple(v.shape) != (B, h, m, d_v):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    return B, h, n, m, d_k, d_v, dt


def _key_lens_ptr(key_lens, B, device):
    import torch

    if key_lens is None:
        return None, None
    if key_lens.dtype != torch.int32 or key_lens.device != device or key_lens.numel() != B:
        raise ValueError("key_lens must be an int32 tensor of B elements on q's device")
    key_lens = key_lens.contiguous()
    return key_lens, key_lens.data_ptr()


def _like(t, shape, dtype, device, name):
    import torch

    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous {list(shape)} {dtype} tensor on q's device")
    return t


def backward(q, k, v, out, dout, lse, *, causal: bool = False, key_lens=None,
             scale: float | None = None, window=None, dq=None, dk=None, dv=None, workspace=None):
    """Gradients (dq, dk, dv) of Eq. (1) for the output gradient ``dout`` (bf16,
    or fp32 at d = 64), in q's dtype.

    ``out`` and ``lse`` come from ``forward(..., return_lse=True)`` with the same
    q, k, v, causal, key_lens, scale and window.  dq/dk/dv/workspace may be
    given to avoid allocations (workspace: a uint8 tensor of at least
    ``sdpa_backward_workspace_bytes(B, h, n)`` bytes).  Raises RuntimeError with
    the library's message on a nonzero status.
    """
    import torch

    wl, wr, al = _window_args(window, causal, *_lengths(q, k))
    B, h, n, m, d_k, d_v, dt = _check_qkv(q, k, v)
    for name, t, shape, dtype in (("out", out, (B, h, n, d_v), q.dtype),
                                  ("dout", dout, (B, h, n, d_v), q.dtype),
                                  ("lse", lse, (B, h, n), torch.float32)):
        _like(t, shape, dtype, q.device, name)
    key_lens, kl_ptr = _key_lens_ptr(key_lens, B, q.device)
    dq = _like(dq, (B, h, n, d_k), q.dtype, q.device, "dq")
    dk = _like(dk, (B, h, m, d_k), q.dtype, q.device, "dk")
    dv = _like(dv, (B, h, m, d_v), q.dtype, q.device, "dv")
    need = sdpa_backward_workspace_bytes(B, h, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = sdpa_backward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                           lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, h, n, m,
                           d_k, d_v, float(scale), wl, wr, al, kl_ptr, dt, workspace.data_ptr(),
                           workspace.numel() * workspace.element_size(), stream)
    if rc != _lib.SDPA_OK:
        raise RuntimeError(f"sdpa_backward failed ({rc}): {sdpa_strerror(rc)}")
    return dq, dk, dv


def forward(q, k, v, *, causal: bool = False, key_lens=None, scale: float | None = None,
            out=None, window=None, return_lse: bool = False, workspace="auto"):
    """Attention over [B, h, n, d_k] queries and [B, h, m, d] keys/values.

    The tensors may be views at any strides whose last dimension is contiguous
    (e.g. ``x.transpose(1, 2)`` of a token-major [B, len, h, d] tensor, or
    slices of a fused Q/K/V buffer); ``out`` may be such a view too.  Those
    calls go through ``sdpa_forward_strided`` with the tensors' own strides;
    packed tensors take the plain entry points.

    key_lens: None or an int32 tensor [B] on the same device (key j of batch
    element b is legal iff j < key_lens[b]).  window: None, or
    (left, right) / (left, right, align) for restricted attention: query i
    sees keys c_i - left .. c_i + right (None = unbounded side), where
    c_i = i for align "top_left" (default) and c_i = i + L - n for
    "bottom_right" (L = the batch element's key length); see
    ``sdpa_forward_window`` in include/sdpa.h.  Not combined with ``causal``.
    Returns ``out`` ([B, h, n, d_v], same dtype as q), or ``(out, lse)`` with
    ``return_lse`` (either dtype): lse [B, h, n] float32, the natural log of each
    row's softmax denominator, which ``backward`` takes.  ``workspace``: a
    uint8 GPU tensor of at least ``sdpa_forward_workspace_bytes(...)`` bytes,
    which lets decoder steps against long caches split each head's keys over
    several workgroups (see ``sdpa_forward_ex``); None for no workspace; or
    "auto" (the default): allocate one when the split applies and there are
    fewer than 256 heads, where a decoder step would otherwise run one
    workgroup per head on a mostly idle GPU (with 256 heads or more the two
    paths measure the same).  Raises RuntimeError with the library's message
    on a nonzero status.
    """
    import torch

    wl, wr, al = _window_args(window, causal, *_lengths(q, k))
    B, h, n, m, d_k, d_v, dt = _check_qkv(q, k, v, strided_ok=True)
    key_lens, kl_ptr = _key_lens_ptr(key_lens, B, q.device)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be a uint8 GPU tensor, None or "auto"')
        need = sdpa_forward_workspace_bytes(B, h, n, m, d_k, d_v, dt) if B * h < 256 else 0
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need > 0 else None
    if out is None:
        out = torch.empty((B, h, n, d_v), dtype=q.dtype, device=q.device)
    elif (tuple(out.shape) != (B, h, n, d_v) or out.dtype != q.dtype or out.device != q.device
          or (out.stride(-1) != 1 and d_v != 1)):
        raise ValueError("out must be a [B, h, n, d_v] tensor of q's dtype on q's device "
                         "with a contiguous last dimension")
    strided = not all(t.is_contiguous() for t in (q, k, v, out))
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    # The library launches on the calling thread's current HIP device.
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        lse = torch.empty((B, h, n), dtype=torch.float32, device=q.device) if return_lse else None
        if strided:
            strides = [s for t in (q, k, v, out) for s in t.stride()[:3]]
            rc = sdpa_forward_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                      None if lse is None else lse.data_ptr(), B, h, n, m, d_k, d_v,
                                      float(scale), wl, wr, al, kl_ptr, dt, strides,
                                      None if workspace is None else workspace.data_ptr(),
                                      0 if workspace is None else
                                      workspace.numel() * workspace.element_size(), stream)
        elif workspace is not None:
            rc = sdpa_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 None if lse is None else lse.data_ptr(), B, h, n, m, d_k, d_v,
                                 float(scale), wl, wr, al, kl_ptr, dt, workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size(), stream)
        elif return_lse:
            rc = sdpa_forward_lse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr(), B, h, n, m, d_k, d_v, float(scale), wl, wr, al,
                                  kl_ptr, dt, stream)
        elif window is None:
            rc = sdpa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, h, n,
                              m, d_k, d_v, float(scale),
                              _lib.SDPA_MASK_CAUSAL if causal else _lib.SDPA_MASK_NONE, kl_ptr,
                              dt, stream)
        else:
            rc = sdpa_forward_window(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B,
                                     h, n, m, d_k, d_v, float(scale), wl, wr, al, kl_ptr, dt,
                                     stream)
    if rc != _lib.SDPA_OK:
        raise RuntimeError(f"sdpa_forward failed ({rc}): {sdpa_strerror(rc)}")
    return (out, lse) if return_lse else out


# --- attention dropout ----------------------------------------------------------

def dropout_keep_mask(B: int, h: int, n: int, m: int, p: float, *, device="cuda", generator=None):
    """A keep mask for ``forward_dropout``: each weight (i, j) kept with
    probability 1 − p, packed as the library reads it, int32 [B, h, n, ⌈m/32⌉]
    with bit (j mod 32) of word ⌊j/32⌋ for key j.  Drawn with torch on
    ``device`` (input preparation, not a step of the attention path)."""
    import torch

    if not 0.0 <= p < 1.0:
        raise ValueError("the dropout probability p must be in [0, 1)")
    W = (m + 31) // 32
    u = torch.rand((B, h, n, W * 32), device=device, generator=generator)
    bits = (u >= p).view(B, h, n, W, 32).to(torch.int64)
    words = (bits << torch.arange(32, device=device, dtype=torch.int64)).sum(-1)
    return torch.where(words >= 1 << 31, words - (1 << 32), words).to(torch.int32)


def _check_keep(keep_mask, B, h, n, m, device):
    import torch

    W = (m + 31) // 32
    if (keep_mask.dtype != torch.int32 or tuple(keep_mask.shape) != (B, h, n, W)
            or not keep_mask.is_contiguous() or keep_mask.device != device):
        raise ValueError(f"keep_mask must be a contiguous int32 [{B}, {h}, {n}, {W}] tensor on q's device")


def forward_dropout(q, k, v, keep_mask, keep_scale: float, *, causal: bool = False, key_lens=None,
                    scale: float | None = None, window=None, out=None, return_lse: bool = False):
    """Eq. (1) with attention dropout: O = (P ∘ Z) V · keep_scale, the keep
    mask Z as ``dropout_keep_mask`` packs it (pass keep_scale = 1/(1 − p)).
    bf16, d_k = d_v = 32, 64 or 128, packed [B, h, len, d] tensors; other
    arguments as in ``forward``.  lse (with ``return_lse``) is the softmax's, unchanged by
    the mask, and is what ``backward_dropout`` takes."""
    import torch

    wl, wr, al = _window_args(window, causal, *_lengths(q, k))
    B, h, n, m, d_k, d_v, dt = _check_qkv(q, k, v)
    _check_keep(keep_mask, B, h, n, m, q.device)
    key_lens, kl_ptr = _key_lens_ptr(key_lens, B, q.device)
    out = _like(out, (B, h, n, d_v), q.dtype, q.device, "out")
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        lse = torch.empty((B, h, n), dtype=torch.float32, device=q.device) if return_lse else None
        rc = sdpa_forward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  None if lse is None else lse.data_ptr(), B, h, n, m, d_k, d_v, float(scale),
                                  wl, wr, al, kl_ptr, keep_mask.data_ptr(), float(keep_scale), dt, stream)
    if rc != _lib.SDPA_OK:
        raise RuntimeError(f"sdpa_forward_dropout failed ({rc}): {sdpa_strerror(rc)}")
    return (out, lse) if return_lse else out


def backward_dropout(q, k, v, out, dout, lse, keep_mask, keep_scale: float, *, causal: bool = False,
                     key_lens=None, scale: float | None = None, window=None, dq=None, dk=None, dv=None,
                     workspace=None):
    """Gradients (dq, dk, dv) of ``forward_dropout`` for the same mask and
    factor; ``out`` and ``lse`` are that forward's.  Arguments as in
    ``backward``."""
    import torch

    wl, wr, al = _window_args(window, causal, *_lengths(q, k))
    B, h, n, m, d_k, d_v, dt = _check_qkv(q, k, v)
    _check_keep(keep_mask, B, h, n, m, q.device)
    for name, t, shape, dtype in (("out", out, (B, h, n, d_v), q.dtype),
                                  ("dout", dout, (B, h, n, d_v), q.dtype),
                                  ("lse", lse, (B, h, n), torch.float32)):
        _like(t, shape, dtype, q.device, name)
    key_lens, kl_ptr = _key_lens_ptr(key_lens, B, q.device)
    dq = _like(dq, (B, h, n, d_k), q.dtype, q.device, "dq")
    dk = _like(dk, (B, h, m, d_k), q.dtype, q.device, "dk")
    dv = _like(dv, (B, h, m, d_v), q.dtype, q.device, "dv")
    need = sdpa_backward_workspace_bytes(B, h, n)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d_k)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = sdpa_backward_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                   lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, h, n, m,
                                   d_k, d_v, float(scale), wl, wr, al, kl_ptr, keep_mask.data_ptr(),
                                   float(keep_scale), dt, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(), stream)
    if rc != _lib.SDPA_OK:
        raise RuntimeError(f"sdpa_backward_dropout failed ({rc}): {sdpa_strerror(rc)}")
    return dq, dk, dv
