"""ctypes binding of libsdpa.so — argument marshalling only.

Every function here has the name of the C entry point it forwards to (see
include/sdpa.h); all arithmetic runs in the HIP kernels behind the C ABI.  The
library is looked up next to this file (built in-tree by ``build_lib``); if it
is missing, ``load()`` raises — there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsdpa.so")

# Mirrors of the #defines in include/sdpa.h (a CPU test checks they agree).
SDPA_OK = 0
SDPA_ERR_NULL = -1
SDPA_ERR_SHAPE = -2
SDPA_ERR_UNSUPPORTED = -3
SDPA_ERR_ALIGN = -4
SDPA_ERR_MASK = -5
SDPA_ERR_DTYPE = -6
SDPA_ERR_LAUNCH = -7
SDPA_ERR_SCALE = -8
SDPA_ERR_ALIAS = -9
SDPA_ERR_WORKSPACE = -10
SDPA_ERR_SCRATCH = -11
SDPA_NOALLOC_SCRATCH_BYTES = 8 << 20
SDPA_F32 = 0
SDPA_BF16 = 1
SDPA_MASK_NONE = 0
SDPA_MASK_CAUSAL = 1
SDPA_ALIGN_TOP_LEFT = 0
SDPA_ALIGN_BOTTOM_RIGHT = 1

_lib = None


def load() -> ctypes.CDLL:
    """Load libsdpa.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m transformer_attention_sdpa_amd.build_lib` "
            "(the attention path has no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    lib.sdpa_forward.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                 ctypes.c_float, i32, vp, i32, vp]
    lib.sdpa_forward.restype = ctypes.c_int
    lib.sdpa_forward_window.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                        ctypes.c_float, i32, i32, i32, vp, i32, vp]
    lib.sdpa_forward_window.restype = ctypes.c_int
    lib.sdpa_mha_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.sdpa_mha_workspace_bytes.restype = ctypes.c_size_t
    lib.sdpa_mha_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                     ctypes.c_float, i32, i32, i32, vp, i32, vp, ctypes.c_size_t, vp]
    lib.sdpa_mha_forward.restype = ctypes.c_int
    fp = ctypes.c_void_p
    lib.sdpa_forward_lse.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32,
                                     ctypes.c_float, i32, i32, i32, vp, i32, vp]
    lib.sdpa_forward_lse.restype = ctypes.c_int
    lib.sdpa_forward_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32, i32]
    lib.sdpa_forward_workspace_bytes.restype = ctypes.c_size_t
    lib.sdpa_forward_ex.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32, ctypes.c_float,
                                    i32, i32, i32, vp, i32, vp, ctypes.c_size_t, vp]
    lib.sdpa_forward_ex.restype = ctypes.c_int
    lib.sdpa_forward_strided.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32,
                                         ctypes.c_float, i32, i32, i32, vp, i32,
                                         ctypes.POINTER(ctypes.c_int64), vp, ctypes.c_size_t, vp]
    lib.sdpa_forward_strided.restype = ctypes.c_int
    lib.sdpa_forward_ex_noalloc.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32,
                                            ctypes.c_float, i32, i32, i32, vp, i32, vp]
    lib.sdpa_forward_ex_noalloc.restype = ctypes.c_int
    lib.sdpa_backward_workspace_bytes.argtypes = [i32, i32, i32]
    lib.sdpa_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.sdpa_backward.argtypes = [vp, vp, vp, vp, vp, fp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                  ctypes.c_float, i32, i32, i32, vp, i32, vp, ctypes.c_size_t, vp]
    lib.sdpa_backward.restype = ctypes.c_int
    lib.sdpa_forward_dropout.argtypes = [vp, vp, vp, vp, fp, i32, i32, i32, i32, i32, i32, ctypes.c_float,
                                         i32, i32, i32, vp, vp, ctypes.c_float, i32, vp]
    lib.sdpa_forward_dropout.restype = ctypes.c_int
    lib.sdpa_backward_dropout.argtypes = [vp, vp, vp, vp, vp, fp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                          ctypes.c_float, i32, i32, i32, vp, vp, ctypes.c_float, i32, vp,
                                          ctypes.c_size_t, vp]
    lib.sdpa_backward_dropout.restype = ctypes.c_int
    lib.sdpa_strerror.argtypes = [ctypes.c_int]
    lib.sdpa_strerror.restype = ctypes.c_char_p
    lib.sdpa_version.argtypes = []
    lib.sdpa_version.restype = ctypes.c_int
    _lib = lib
    return lib


def sdpa_forward(q, k, v, out, B, h, n, m, d_k, d_v, scale, mask_kind, key_lens, dtype,
                 stream) -> int:
    """Forward to the C entry point; pointers and the stream are plain integers (or None)."""
    return load().sdpa_forward(q, k, v, out, B, h, n, m, d_k, d_v, scale, mask_kind,
                               key_lens, dtype, stream)


def sdpa_forward_window(q, k, v, out, B, h, n, m, d_k, d_v, scale, window_left, window_right,
                        align, key_lens, dtype, stream) -> int:
    """Forward to the C entry point of the same name (restricted attention)."""
    return load().sdpa_forward_window(q, k, v, out, B, h, n, m, d_k, d_v, scale, window_left,
                                      window_right, align, key_lens, dtype, stream)


def sdpa_mha_workspace_bytes(B, n, m, h, d_k, d_v) -> int:
    """Forward to the C entry point of the same name."""
    return load().sdpa_mha_workspace_bytes(B, n, m, h, d_k, d_v)


def sdpa_mha_forward(x_q, x_kv, w_q, w_k, w_v, w_o, out, B, n, m, d_model, h, d_k, d_v, scale,
                     window_left, window_right, align, key_lens, dtype, workspace, workspace_bytes,
                     stream) -> int:
    """Forward to the C entry point of the same name (the multi-head sublayer)."""
    return load().sdpa_mha_forward(x_q, x_kv, w_q, w_k, w_v, w_o, out, B, n, m, d_model, h, d_k,
                                   d_v, scale, window_left, window_right, align, key_lens, dtype,
                                   workspace, workspace_bytes, stream)


def sdpa_forward_lse(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale, window_left, window_right,
                     align, key_lens, dtype, stream) -> int:
    """Forward to the C entry point of the same name (forward pass + row log-sum-exp)."""
    return load().sdpa_forward_lse(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale, window_left,
                                   window_right, align, key_lens, dtype, stream)


def sdpa_forward_workspace_bytes(B, h, n, m, d_k, d_v, dtype) -> int:
    """Forward to the C entry point of the same name."""
    return load().sdpa_forward_workspace_bytes(B, h, n, m, d_k, d_v, dtype)


def sdpa_forward_ex(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale, window_left, window_right, align,
                    key_lens, dtype, workspace, workspace_bytes, stream) -> int:
    """Forward to the C entry point of the same name (optional lse and workspace)."""
    return load().sdpa_forward_ex(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale, window_left,
                                  window_right, align, key_lens, dtype, workspace, workspace_bytes,
                                  stream)


def sdpa_forward_strided(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale, window_left, window_right,
                         align, key_lens, dtype, strides, workspace, workspace_bytes, stream) -> int:
    """Forward to the C entry point of the same name; ``strides`` is None or a
    sequence of 12 element strides (batch, head, row of q, k, v, out)."""
    arr = None
    if strides is not None:
        if len(strides) != 12:
            raise ValueError("strides: 12 values (batch, head, row of q, k, v and out)")
        arr = (ctypes.c_int64 * 12)(*[int(x) for x in strides])
    return load().sdpa_forward_strided(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale, window_left,
                                       window_right, align, key_lens, dtype, arr, workspace,
                                       workspace_bytes, stream)


def sdpa_forward_ex_noalloc(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale, window_left,
                            window_right, align, key_lens, dtype, stream) -> int:
    """Forward to the C entry point of the same name (sdpa_forward_ex with the
    library's static scratch in place of a workspace; allocates nothing)."""
    return load().sdpa_forward_ex_noalloc(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale,
                                          window_left, window_right, align, key_lens, dtype, stream)


def sdpa_backward_workspace_bytes(B, h, n) -> int:
    """Forward to the C entry point of the same name."""
    return load().sdpa_backward_workspace_bytes(B, h, n)


def sdpa_forward_dropout(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale, window_left, window_right, align,
                         key_lens, keep_mask, keep_scale, dtype, stream) -> int:
    """Forward to the C entry point of the same name (attention dropout)."""
    return load().sdpa_forward_dropout(q, k, v, out, lse, B, h, n, m, d_k, d_v, scale, window_left,
                                       window_right, align, key_lens, keep_mask, keep_scale, dtype, stream)


def sdpa_backward_dropout(q, k, v, out, dout, lse, dq, dk, dv, B, h, n, m, d_k, d_v, scale, window_left,
                          window_right, align, key_lens, keep_mask, keep_scale, dtype, workspace,
                          workspace_bytes, stream) -> int:
    """Forward to the C entry point of the same name (gradient with attention dropout)."""
    return load().sdpa_backward_dropout(q, k, v, out, dout, lse, dq, dk, dv, B, h, n, m, d_k, d_v, scale,
                                        window_left, window_right, align, key_lens, keep_mask, keep_scale,
                                        dtype, workspace, workspace_bytes, stream)


def sdpa_backward(q, k, v, out, dout, lse, dq, dk, dv, B, h, n, m, d_k, d_v, scale, window_left,
                  window_right, align, key_lens, dtype, workspace, workspace_bytes, stream) -> int:
    """Forward to the C entry point of the same name (the gradient of Eq. (1))."""
    return load().sdpa_backward(q, k, v, out, dout, lse, dq, dk, dv, B, h, n, m, d_k, d_v, scale,
                                window_left, window_right, align, key_lens, dtype, workspace,
                                workspace_bytes, stream)


def sdpa_strerror(status: int) -> str:
    return load().sdpa_strerror(status).decode()


def sdpa_version() -> int:
    return load().sdpa_version()
