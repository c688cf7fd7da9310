"""Python binding of libkda.so, the MI355X KDA chunked forward library.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI of include/kda.h.  The names mirror that header:
``kda_fwd``, ``kda_workspace_size``, ``kda_is_supported``.  PyTorch provides
device memory and the current stream; there is no CPU or PyTorch fallback, and
importing this module fails if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

# torch first: its bundled HIP runtime carries the same SONAME
# (libamdhip64.so.7) that libkda.so links against, so loading torch first makes
# both use one runtime.  Loading libkda.so first would put a second HIP runtime
# in the process, and whichever initialises second sees no device.
import torch  # noqa: F401

__all__ = ["kda_fwd", "kda_workspace_size", "kda_is_supported", "KdaError", "STATUS",
           "library_path", "exported_symbols"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libkda.so")

STATUS = {0: "KDA_SUCCESS", 1: "KDA_ERR_INVALID", 2: "KDA_ERR_UNSUPPORTED",
          3: "KDA_ERR_WORKSPACE", 4: "KDA_ERR_LAUNCH"}
exported_symbols = ("kda_fwd", "kda_workspace_size", "kda_is_supported", "kda_status_string")


class KdaError(RuntimeError):
    """A non-zero kda_status_t returned by the library."""

    def __init__(self, status: int):
        self.status = status
        super().__init__(f"kda_fwd failed: {STATUS.get(status, status)}")


if not os.path.exists(library_path):
    raise ImportError(f"{library_path} is missing; build it with "
                      "`python -c 'import __graft_entry__ as g; g.build()'`")

_lib = ctypes.CDLL(library_path)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_lib.kda_workspace_size.argtypes = [_I64, _I64, _I64]
_lib.kda_workspace_size.restype = ctypes.c_size_t
_lib.kda_is_supported.argtypes = [_I64, _I64, ctypes.c_float]
_lib.kda_is_supported.restype = ctypes.c_int
_lib.kda_status_string.argtypes = [ctypes.c_int]
_lib.kda_status_string.restype = ctypes.c_char_p
_lib.kda_fwd.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, _P, ctypes.c_size_t, _P, _P,
                         ctypes.c_float, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P]
_lib.kda_fwd.restype = ctypes.c_int


def kda_workspace_size(T: int, H: int, N: int) -> int:
    """Workspace bytes for T packed tokens, H heads and N sequences."""
    return int(_lib.kda_workspace_size(T, H, N))


def kda_is_supported(K: int, V: int, lower_bound: float) -> bool:
    return bool(_lib.kda_is_supported(K, V, lower_bound))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def kda_fwd(q, k, v, raw_gate, raw_beta, scale, out, workspace, A_log, dt_bias, lower_bound,
            initial_state=None, final_state=None, cu_seqlens=None, stream=None):
    """Enqueue one KDA forward on ``stream`` (default: torch's current stream).

    Tensors are torch device tensors in the layouts of include/kda.h:
    q, k, raw_gate bf16 [B,T,H,K]; v and out bf16 [B,T,H,V]; raw_beta bf16 [B,T,H];
    workspace uint8 [>= kda_workspace_size(B*T, H, N)]; A_log fp32 [H];
    dt_bias fp32 [H,K]; initial_state / final_state fp32 [N,H,K,V] or None;
    cu_seqlens int32 [N+1] or None.  Raises KdaError on a non-zero status.
    """
    B, T, H, K = q.shape
    V = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("raw_gate", raw_gate), ("raw_beta", raw_beta),
                    ("out", out)):
        if t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bf16 device tensor")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias), ("initial_state", initial_state),
                    ("final_state", final_state)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda):
            raise ValueError(f"{name} must be a contiguous fp32 device tensor")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 device tensor")
    if tuple(k.shape) != (B, T, H, K) or tuple(raw_gate.shape) != (B, T, H, K) or \
            tuple(v.shape) != (B, T, H, V) or tuple(out.shape) != (B, T, H, V) or \
            tuple(raw_beta.shape) != (B, T, H):
        raise ValueError("inconsistent q/k/v/raw_gate/raw_beta/out shapes")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    for name, t in (("initial_state", initial_state), ("final_state", final_state)):
        if t is not None and tuple(t.shape) != (N, H, K, V):
            raise ValueError(f"{name} must have shape [N, H, K, V] = {(N, H, K, V)}")
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib.kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(raw_beta), float(scale),
                      _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                      _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                      _ptr(final_state), _ptr(cu_seqlens), B, T, H, K, V, N,
                      ctypes.c_void_p(int(stream)))
    if rc != 0:
        raise KdaError(rc)


def raw_call(*args):
    """Call the C entry point with already-marshalled ctypes arguments (tests)."""
    return _lib.kda_fwd(*args)
