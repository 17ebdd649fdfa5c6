"""MI355X (gfx950) gated-delta-rule forward pass.

Python face of the C ABI in ``include/gdn.h`` (``libgdn.so``): argument
marshalling only.  Every step of the computation runs in the HIP kernel; if
the library is missing this raises instead of falling back to anything else.

The rule (HyMo "Model Architecture Walkthrough", sections 5.2.1-5.2.2):
S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
o_t = S_t q_t, alpha_t = exp(g_t).
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["gdn_fwd", "gdn_fwd_train", "gdn_bwd_saved", "fwd_train", "gdn_fwd_scan", "gdn_fwd_scan_workspace_size", "fwd_scan", "gdn_fwd_recurrent", "gdn_diag_fwd", "gdn_diag_fwd_recurrent", "gdn_bwd",
           "gdn_bwd_workspace_size", "gdn_bwd_noalloc", "fwd", "fwd_recurrent", "diag_fwd", "diag_fwd_recurrent",
           "bwd", "gated_delta_rule", "GdnError", "lib_path", "load", "version"]

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDN_LIB_PATH names another build of the same library (the tests use it to
# run the host-side checks against a sanitizer-instrumented build).
_LIB_PATH = os.environ.get("GDN_LIB_PATH") or os.path.join(_HERE, "libgdn.so")
_lib = None

GDN_F32 = 0
GDN_BF16 = 1
GDN_FLAG_NO_SEGMENTS = 1


class GdnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gdn_fwd failed ({status}): {msg}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libgdn.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise OSError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m gated_deltanet_recurrence_delta_amd.build`")
        # torch first: libgdn.so names the HIP runtime by its soname, and the
        # process must hold one runtime.  Loaded before torch, the library
        # would bring in the system ROCm's copy next to torch's own, and its
        # launches fail.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.gdn_fwd.restype = I
        lib.gdn_fwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, P, I, I, I]
        lib.gdn_fwd_scan.restype = I
        lib.gdn_fwd_scan.argtypes = [P] * 9 + [I] * 5 + [P, I, I, P, ctypes.c_longlong]
        lib.gdn_fwd_scan_workspace_size.restype = ctypes.c_longlong
        lib.gdn_fwd_scan_workspace_size.argtypes = [I] * 8
        lib.gdn_fwd_recurrent.restype = I
        lib.gdn_fwd_recurrent.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, P, I]
        lib.gdn_diag_fwd.restype = I
        lib.gdn_diag_fwd.argtypes = [P] * 11 + [I] * 5 + [P, I, I]
        lib.gdn_diag_fwd_recurrent.restype = I
        lib.gdn_diag_fwd_recurrent.argtypes = [P] * 11 + [I] * 5 + [P, I]
        lib.gdn_fwd_train.restype = I
        lib.gdn_fwd_train.argtypes = [P] * 9 + [I] * 5 + [P, I, I, P, ctypes.c_longlong]
        lib.gdn_bwd.restype = I
        lib.gdn_bwd.argtypes = [P] * 16 + [ctypes.c_longlong] + [I] * 5 + [P, I]
        lib.gdn_bwd_saved.restype = I
        lib.gdn_bwd_saved.argtypes = [P] * 16 + [ctypes.c_longlong] + [I] * 5 + [P, I]
        lib.gdn_bwd_noalloc.restype = I
        lib.gdn_bwd_noalloc.argtypes = [P] * 15 + [I] * 5 + [P, I]
        lib.gdn_bwd_workspace_size.restype = ctypes.c_longlong
        lib.gdn_bwd_workspace_size.argtypes = [I] * 6
        lib.gdn_strerror.restype = ctypes.c_char_p
        lib.gdn_strerror.argtypes = [I]
        lib.gdn_version.restype = I
        lib.gdn_version.argtypes = []
        _lib = lib
    return _lib


def version() -> int:
    return load().gdn_version()


def strerror(status: int) -> str:
    return load().gdn_strerror(status).decode()


def gdn_fwd(q, k, v, g, beta, h0, cu_seqlens, out, hT, B, T, H, dk, dv,
            stream, dtype, chunk, flags=0) -> int:
    """Raw C call with integer pointers (0 = NULL).  Returns the status."""
    return load().gdn_fwd(q, k, v, g, beta, h0, cu_seqlens, out, hT,
                          int(B), int(T), int(H), int(dk), int(dv),
                          stream, int(dtype), int(chunk), int(flags))


def gdn_fwd_scan_workspace_size(B, T, H, dk, dv, packed, dtype, chunk=0) -> int:
    """Workspace bytes ``gdn_fwd_scan`` needs (negative: a status code)."""
    return load().gdn_fwd_scan_workspace_size(int(B), int(T), int(H), int(dk), int(dv), int(packed),
                                              int(dtype), int(chunk))


def gdn_fwd_scan(q, k, v, g, beta, h0, cu_seqlens, out, hT, B, T, H, dk, dv,
                 stream, dtype, chunk, workspace, workspace_bytes) -> int:
    """Raw C call of the chunk-map scan form (0 = NULL).  Returns the status."""
    return load().gdn_fwd_scan(q, k, v, g, beta, h0, cu_seqlens, out, hT,
                               int(B), int(T), int(H), int(dk), int(dv),
                               stream, int(dtype), int(chunk), workspace, int(workspace_bytes))


def gdn_fwd_train(q, k, v, g, beta, h0, cu_seqlens, out, hT, B, T, H, dk, dv,
                  stream, dtype, chunk, workspace, workspace_bytes) -> int:
    """Raw C call of the training forward (0 = NULL).  Returns the status."""
    return load().gdn_fwd_train(q, k, v, g, beta, h0, cu_seqlens, out, hT, int(B), int(T), int(H),
                                int(dk), int(dv), stream, int(dtype), int(chunk), workspace,
                                int(workspace_bytes))


def gdn_fwd_recurrent(q, k, v, g, beta, h0, cu_seqlens, out, hT, B, T, H, dk, dv,
                      stream, dtype) -> int:
    """Raw C call of the token-by-token form (0 = NULL).  Returns the status."""
    return load().gdn_fwd_recurrent(q, k, v, g, beta, h0, cu_seqlens, out, hT,
                                    int(B), int(T), int(H), int(dk), int(dv),
                                    stream, int(dtype))


def fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk: int = 0,
        out=None, hT=None, stream=None, segments: bool = True,
        check_cu_seqlens: bool = False):
    """Gated-delta-rule forward on torch device tensors (chunkwise form).

    q, k: (B,T,H,dk); v: (B,T,H,dv); g, beta: (B,T,H) float32 (packed:
    drop B and pass int32 ``cu_seqlens`` of length B+1).  q/k/v share one
    dtype, float32 or bfloat16.  h0: (B,H,dk,dv) float32 or None.
    Returns (out, hT); out has q's dtype, hT is float32.  Runs on the
    current stream (or ``stream``), asynchronously.  ``segments=False``
    passes GDN_FLAG_NO_SEGMENTS (every chain runs from its start).
    ``check_cu_seqlens=True`` copies cu_seqlens to the host (a
    synchronisation) and checks that it starts at 0, never decreases and
    ends at T before anything is launched.
    """
    a, out, hT = _marshal(q, k, v, g, beta, h0, cu_seqlens, out, hT, stream)
    if check_cu_seqlens and cu_seqlens is not None:
        check_offsets(cu_seqlens.cpu().numpy(), a[10])
    rc = gdn_fwd(*a, chunk, 0 if segments else GDN_FLAG_NO_SEGMENTS)
    if rc != 0:
        raise GdnError(rc, strerror(rc))
    return out, hT


def fwd_scan(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk: int = 0,
             out=None, hT=None, stream=None, workspace=None):
    """``fwd`` with exact segment starts from the chunk-map scan
    (``gdn_fwd_scan``): long sequences run as parallel segments whatever the
    decay.  ``workspace``: a uint8 device tensor of at least
    ``gdn_fwd_scan_workspace_size`` bytes, allocated here when None.
    Returns (out, hT)."""
    import torch

    a, out, hT = _marshal(q, k, v, g, beta, h0, cu_seqlens, out, hT, stream)
    B, T, H, dk, dv, dtype = a[9], a[10], a[11], a[12], a[13], a[15]
    need = gdn_fwd_scan_workspace_size(B, T, H, dk, dv, cu_seqlens is not None, dtype, chunk)
    if need < 0:
        raise GdnError(need, strerror(need))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be on q's device and hold {need} bytes")
    rc = gdn_fwd_scan(*a, chunk, workspace.data_ptr(), workspace.numel() * workspace.element_size())
    if rc != 0:
        raise GdnError(rc, strerror(rc))
    return out, hT


def fwd_recurrent(q, k, v, g, beta, h0=None, cu_seqlens=None, out=None, hT=None,
                  stream=None):
    """Token-by-token form of ``fwd`` (same arguments but no chunk length)."""
    a, out, hT = _marshal(q, k, v, g, beta, h0, cu_seqlens, out, hT, stream)
    rc = gdn_fwd_recurrent(*a)
    if rc != 0:
        raise GdnError(rc, strerror(rc))
    return out, hT


def check_offsets(cu, T: int) -> None:
    """Host check of packed-batch offsets: cu[0] == 0, non-decreasing,
    cu[-1] == T.  Raises ValueError otherwise."""
    import numpy as np

    cu = np.asarray(cu).reshape(-1)
    if cu.size < 1:
        raise ValueError("cu_seqlens must have at least one entry")
    if int(cu[0]) != 0:
        raise ValueError(f"cu_seqlens[0] must be 0, got {int(cu[0])}")
    if cu.size > 1 and bool(np.any(np.diff(cu.astype(np.int64)) < 0)):
        raise ValueError("cu_seqlens must be non-decreasing")
    if int(cu[-1]) != int(T):
        raise ValueError(f"cu_seqlens[-1] must equal the packed length {T}, got {int(cu[-1])}")


def _check_outputs(out, hT, out_shape, out_dtype, state_shape):
    """Caller-supplied outputs must have exactly the shapes and dtypes the
    kernel writes: a smaller buffer would be written past its end."""
    import torch

    if out is not None and (tuple(out.shape) != tuple(out_shape) or out.dtype != out_dtype):
        raise ValueError(f"out must be {out_dtype} of shape {tuple(out_shape)}, "
                         f"got {out.dtype} {tuple(out.shape)}")
    if hT is not None and (tuple(hT.shape) != tuple(state_shape) or hT.dtype != torch.float32):
        raise ValueError(f"hT must be float32 of shape {tuple(state_shape)}, "
                         f"got {hT.dtype} {tuple(hT.shape)}")


def _marshal(q, k, v, g, beta, h0, cu_seqlens, out, hT, stream):
    """Check the tensors, allocate missing outputs; the C arguments up to dtype."""
    import torch

    if q.dtype == torch.bfloat16:
        dtype = GDN_BF16
    elif q.dtype == torch.float32:
        dtype = GDN_F32
    else:
        raise TypeError(f"q/k/v dtype must be float32 or bfloat16, got {q.dtype}")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype:
            raise TypeError(f"{name} dtype {t.dtype} != q dtype {q.dtype}")
    for name, t in (("g", g), ("beta", beta)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        if q.dim() != 3:
            raise ValueError("packed q must be (T, H, dk)")
        T, H, dk = q.shape
        B = cu_seqlens.numel() - 1
        if B < 0:
            raise ValueError("cu_seqlens must have at least one entry")
    else:
        if q.dim() != 4:
            raise ValueError("q must be (B, T, H, dk)")
        B, T, H, dk = q.shape
    dv = v.shape[-1]
    if tuple(k.shape) != tuple(q.shape) or tuple(v.shape[:-1]) != tuple(q.shape[:-1]):
        raise ValueError("q, k, v shapes disagree")
    if tuple(g.shape) != tuple(q.shape[:-1]) or tuple(beta.shape) != tuple(q.shape[:-1]):
        raise ValueError("g/beta must have q's shape without the last dimension")
    if h0 is not None and (h0.dtype != torch.float32 or tuple(h0.shape) != (B, H, dk, dv)):
        raise ValueError("h0 must be float32 (B, H, dk, dv)")
    _check_outputs(out, hT, v.shape, v.dtype, (B, H, dk, dv))
    tensors = [q, k, v, g, beta] + [x for x in (h0, cu_seqlens, out, hT) if x is not None]
    dev = q.device
    for t in tensors:
        if t.device != dev or dev.type != "cuda":
            raise ValueError("all tensors must be on the same GPU device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if hT is None:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    args = (ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(h0), ptr(cu_seqlens),
            ptr(out), ptr(hT), B, T, H, dk, dv, stream.cuda_stream, dtype)
    return args, out, hT


# ------------------------------------------- diagonal-decay additive form ---

def gdn_diag_fwd(v, b, c, g, A_log, Dskip, gate, h0, cu_seqlens, out, hT, B, T, H, S, D,
                 stream, dtype, chunk) -> int:
    """Raw C call of the diagonal-decay form (0 = NULL).  Returns the status."""
    return load().gdn_diag_fwd(v, b, c, g, A_log, Dskip, gate, h0, cu_seqlens, out, hT,
                               int(B), int(T), int(H), int(S), int(D), stream, int(dtype),
                               int(chunk))


def gdn_diag_fwd_recurrent(v, b, c, g, A_log, Dskip, gate, h0, cu_seqlens, out, hT, B, T, H,
                           S, D, stream, dtype) -> int:
    """Raw C call of the diagonal-decay form, token by token.  Returns the status."""
    return load().gdn_diag_fwd_recurrent(v, b, c, g, A_log, Dskip, gate, h0, cu_seqlens, out,
                                         hT, int(B), int(T), int(H), int(S), int(D), stream,
                                         int(dtype))


def diag_fwd(v, b, c, g, A_log, D=None, gate=None, h0=None, cu_seqlens=None, chunk: int = 0,
             out=None, hT=None, stream=None):
    """HyMo's diagonal-decay recurrence with its epilogue, chunkwise form.

    v: (B,T,H,D); b, c: (B,T,H,S); g, gate: (B,T,H) float32; A_log: (H,S)
    float32; D: (H,) float32 or None; h0: (B,H,S,D) float32 or None (packed:
    drop B, pass int32 cu_seqlens).  v/b/c share one dtype.  Returns
    (out, hT); out has v's dtype, hT is float32.
    """
    a, out, hT = _marshal_diag(v, b, c, g, A_log, D, gate, h0, cu_seqlens, out, hT, stream)
    rc = gdn_diag_fwd(*a, chunk)
    if rc != 0:
        raise GdnError(rc, strerror(rc))
    return out, hT


def diag_fwd_recurrent(v, b, c, g, A_log, D=None, gate=None, h0=None, cu_seqlens=None,
                       out=None, hT=None, stream=None):
    """Token-by-token form of ``diag_fwd`` (same arguments but no chunk)."""
    a, out, hT = _marshal_diag(v, b, c, g, A_log, D, gate, h0, cu_seqlens, out, hT, stream)
    rc = gdn_diag_fwd_recurrent(*a)
    if rc != 0:
        raise GdnError(rc, strerror(rc))
    return out, hT


def _marshal_diag(v, b, c, g, A_log, Dskip, gate, h0, cu_seqlens, out, hT, stream):
    import torch

    if v.dtype == torch.bfloat16:
        dtype = GDN_BF16
    elif v.dtype == torch.float32:
        dtype = GDN_F32
    else:
        raise TypeError(f"v/b/c dtype must be float32 or bfloat16, got {v.dtype}")
    for name, t in (("b", b), ("c", c)):
        if t.dtype != v.dtype:
            raise TypeError(f"{name} dtype {t.dtype} != v dtype {v.dtype}")
    for name, t in (("g", g), ("A_log", A_log), ("D", Dskip), ("gate", gate), ("h0", h0)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        if v.dim() != 3:
            raise ValueError("packed v must be (T, H, D)")
        T, H, D = v.shape
        B = cu_seqlens.numel() - 1
        if B < 0:
            raise ValueError("cu_seqlens must have at least one entry")
    else:
        if v.dim() != 4:
            raise ValueError("v must be (B, T, H, D)")
        B, T, H, D = v.shape
    S = b.shape[-1]
    lead = tuple(v.shape[:-1])
    if tuple(b.shape) != lead + (S,) or tuple(c.shape) != lead + (S,):
        raise ValueError("b and c must be v's shape with S as the last dimension")
    if tuple(g.shape) != lead or (gate is not None and tuple(gate.shape) != lead):
        raise ValueError("g/gate must have v's shape without the last dimension")
    if tuple(A_log.shape) != (H, S):
        raise ValueError("A_log must be (H, S)")
    if Dskip is not None and tuple(Dskip.shape) != (H,):
        raise ValueError("D must be (H,)")
    if h0 is not None and tuple(h0.shape) != (B, H, S, D):
        raise ValueError("h0 must be (B, H, S, D)")
    _check_outputs(out, hT, v.shape, v.dtype, (B, H, S, D))
    tensors = [v, b, c, g, A_log] + [x for x in (Dskip, gate, h0, cu_seqlens, out, hT)
                                     if x is not None]
    dev = v.device
    for t in tensors:
        if t.device != dev or dev.type != "cuda":
            raise ValueError("all tensors must be on the same GPU device")
        if not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")
    if out is None:
        out = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if hT is None:
        hT = torch.empty((B, H, S, D), dtype=torch.float32, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    ptr = lambda t: 0 if t is None else t.data_ptr()
    args = (ptr(v), ptr(b), ptr(c), ptr(g), ptr(A_log), ptr(Dskip), ptr(gate), ptr(h0),
            ptr(cu_seqlens), ptr(out), ptr(hT), B, T, H, S, D, stream.cuda_stream, dtype)
    return args, out, hT


# ------------------------------------------------------------- backward ---

def gdn_bwd_workspace_size(B, T, H, dk, dv, packed) -> int:
    """Workspace bytes ``gdn_bwd`` needs (negative: a status code)."""
    return load().gdn_bwd_workspace_size(int(B), int(T), int(H), int(dk), int(dv), int(packed))


def gdn_bwd(q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg, dbeta, dh0,
            workspace, workspace_bytes, B, T, H, dk_, dv_, stream, dtype) -> int:
    """Raw C call of the backward pass (0 = NULL).  Returns the status."""
    return load().gdn_bwd(q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg, dbeta,
                          dh0, workspace, int(workspace_bytes), int(B), int(T), int(H),
                          int(dk_), int(dv_), stream, int(dtype))


def gdn_bwd_saved(q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg, dbeta, dh0,
                  workspace, workspace_bytes, B, T, H, dk_, dv_, stream, dtype) -> int:
    """Raw C call of the backward pass from records gdn_fwd_train left in the
    workspace (0 = NULL).  Returns the status."""
    return load().gdn_bwd_saved(q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg, dbeta,
                                dh0, workspace, int(workspace_bytes), int(B), int(T), int(H),
                                int(dk_), int(dv_), stream, int(dtype))


def train_records_supported(q, k, v, chunk: int = 0) -> bool:
    """Whether gdn_fwd_train / gdn_bwd_saved have records for this shape:
    bf16 storage, dk = dv = 128 and 64-token chunks (chunk 0 or 64)."""
    import torch

    return (q.dtype == torch.bfloat16 and q.shape[-1] == 128 and v.shape[-1] == 128
            and chunk in (0, 64))


def fwd_train(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk: int = 0,
              out=None, hT=None, workspace=None, stream=None):
    """``fwd`` that also leaves the backward pass's per-chunk records in a
    workspace (``gdn_fwd_train``), for ``bwd(..., saved=True)`` on the same
    inputs.  Only for bf16 with dk = dv = 128 and 64-token chunks
    (``train_records_supported``).  ``workspace``: a uint8 device tensor of
    at least ``gdn_bwd_workspace_size`` bytes, allocated here when None.
    Returns (out, hT, workspace)."""
    import torch

    a, out, hT = _marshal(q, k, v, g, beta, h0, cu_seqlens, out, hT, stream)
    B, T, H, dk, dv = a[9:14]
    need = gdn_bwd_workspace_size(B, T, H, dk, dv, cu_seqlens is not None)
    if need < 0:
        raise GdnError(need, strerror(need))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be on q's device and hold {need} bytes")
    rc = gdn_fwd_train(*a, chunk, workspace.data_ptr(), workspace.numel() * workspace.element_size())
    if rc != 0:
        raise GdnError(rc, strerror(rc))
    return out, hT, workspace


def bwd(q, k, v, g, beta, dout, h0=None, cu_seqlens=None, dhT=None, want_dh0=True,
        workspace=None, stream=None, saved=False):
    """Gradients of <dout, out> + <dhT, hT> for ``fwd``'s outputs (out, hT).

    Arguments as for ``fwd``; dout has out's shape and dtype, dhT is
    (B,H,dk,dv) float32 or None (zero).  Returns a dict with dq, dk, dv (the
    inputs' dtype), dg, dbeta (float32) and dh0 (float32, or None when
    ``want_dh0`` is false).  ``workspace``: a uint8 device tensor of at least
    ``gdn_bwd_workspace_size`` bytes, allocated here when None.  ``saved``:
    the workspace holds the records ``fwd_train`` wrote for these inputs
    (``gdn_bwd_saved``, which skips recomputing them).
    """
    import torch

    # out/hT slots carry dout/dhT so that nothing extra is allocated; unused
    a, _, _ = _marshal(q, k, v, g, beta, h0, cu_seqlens, dout, dhT, stream)
    B, T, H, dk_, dv_ = a[9:14]
    strm, dtype = a[14], a[15]
    dev = q.device
    if dout.dtype != v.dtype or tuple(dout.shape) != tuple(v.shape) or dout.device != dev:
        raise ValueError("dout must have v's shape, dtype and device")
    if not dout.is_contiguous():
        raise ValueError("dout must be contiguous")
    if dhT is not None and (dhT.dtype != torch.float32 or tuple(dhT.shape) != (B, H, dk_, dv_)
                            or dhT.device != dev or not dhT.is_contiguous()):
        raise ValueError("dhT must be contiguous float32 (B, H, dk, dv) on q's device")
    need = gdn_bwd_workspace_size(B, T, H, dk_, dv_, cu_seqlens is not None)
    if need < 0:
        raise GdnError(need, strerror(need))
    if saved and workspace is None:
        raise ValueError("saved=True needs the workspace fwd_train filled")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev or workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace must be on q's device and hold {need} bytes")
    grads = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
             "dg": torch.empty_like(g), "dbeta": torch.empty_like(beta),
             "dh0": torch.empty((B, H, dk_, dv_), dtype=torch.float32, device=dev)
             if want_dh0 else None}
    ptr = lambda t: 0 if t is None else t.data_ptr()
    call = gdn_bwd_saved if saved else gdn_bwd
    rc = call(a[0], a[1], a[2], a[3], a[4], a[5], a[6], ptr(dout), ptr(dhT),
              ptr(grads["dq"]), ptr(grads["dk"]), ptr(grads["dv"]), ptr(grads["dg"]),
              ptr(grads["dbeta"]), ptr(grads["dh0"]), ptr(workspace),
              workspace.numel() * workspace.element_size(), B, T, H, dk_, dv_, strm, dtype)
    if rc != 0:
        raise GdnError(rc, strerror(rc))
    return grads


NOALLOC_SCRATCH_BYTES = 64 << 20


def gdn_bwd_noalloc(q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg, dbeta, dh0,
                    B, T, H, dk_, dv_, stream, dtype) -> int:
    """Raw C call of the backward pass with the library's fixed per-GPU
    scratch instead of a workspace (0 = NULL).  Returns the status."""
    return load().gdn_bwd_noalloc(q, k, v, g, beta, h0, cu_seqlens, dout, dhT, dq, dk, dv, dg,
                                  dbeta, dh0, int(B), int(T), int(H), int(dk_), int(dv_), stream,
                                  int(dtype))


# -------------------------------------------------------------- autograd ---

def gated_delta_rule(q, k, v, g, beta, h0=None, cu_seqlens=None):
    """(out, hT) of ``fwd`` as a differentiable torch operation: the forward
    runs gdn_fwd and the backward gdn_bwd (from the saved inputs), giving
    gradients for q, k, v, g, beta and h0.  Where the training records exist
    (bf16, dk = dv = 128) the forward runs gdn_fwd_train instead and keeps
    its workspace for gdn_bwd_saved.  Arguments as for ``fwd``."""
    return _gdr_function().apply(q, k, v, g, beta, h0, cu_seqlens)


_GDR = None


def _gdr_function():
    global _GDR
    if _GDR is None:
        import torch

        class _GatedDeltaRule(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, g, beta, h0, cu_seqlens):
                ctx.workspace = None
                if train_records_supported(q, k, v):
                    out, hT, ctx.workspace = fwd_train(q, k, v, g, beta, h0, cu_seqlens)
                else:
                    out, hT = fwd(q, k, v, g, beta, h0, cu_seqlens)
                ctx.save_for_backward(q, k, v, g, beta, h0, cu_seqlens)
                ctx.has_h0 = h0 is not None
                return out, hT

            @staticmethod
            def backward(ctx, dout, dhT):
                q, k, v, g, beta, h0, cu_seqlens = ctx.saved_tensors
                dout = torch.zeros_like(v) if dout is None else dout.contiguous()
                dhT = None if dhT is None else dhT.contiguous()
                gr = bwd(q, k, v, g, beta, dout, h0=h0, cu_seqlens=cu_seqlens, dhT=dhT,
                         want_dh0=ctx.has_h0, workspace=ctx.workspace,
                         saved=ctx.workspace is not None)
                ctx.workspace = None
                return gr["dq"], gr["dk"], gr["dv"], gr["dg"], gr["dbeta"], gr["dh0"], None

        _GDR = _GatedDeltaRule
    return _GDR
