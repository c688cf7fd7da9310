"""Python binding of libkda.so, the MI355X KDA chunked forward library.

Argument marshalling only: every step of the forward pass runs in the HIP
kernels behind the C ABI of include/kda.h.  The names mirror that header:
``kda_fwd``, ``kda_workspace_size``, ``kda_is_supported``, ``kda_shard_affine``,
``kda_shard_scan``, ``kda_decode``, ``kda_fwd_ex`` (with the ``FLAG_*`` variant bits),
``kda_bwd``, ``kda_bwd_ex``, ``kda_bwd_workspace_size``,
``kda_workspace_faults`` (with the ``FAULT_*`` bits) and ``kda_fwd_noalloc``.  PyTorch provides
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

__all__ = ["kda_fwd", "kda_fwd_ex", "kda_workspace_size", "kda_is_supported", "kda_shard_affine",
           "kda_shard_scan", "kda_decode", "kda_bwd", "kda_bwd_ex", "kda_bwd_workspace_size",
           "kda_workspace_faults", "kda_fwd_noalloc", "NOALLOC_SCRATCH_BYTES", "FAULT_WAIT_TIMEOUT", "FAULT_GATE_RANGE", "FAULT_QK_NORM", "KdaError", "STATUS", "library_path", "exported_symbols",
           "FLAG_GATE_GIVEN", "FLAG_BETA_GIVEN", "FLAG_NO_QK_NORM", "FLAG_STATE_VK", "FLAG_REUSE_RECORDS",
           "FLAG_KEEP_RECORDS", "FLAG_SINGLE_LAUNCH", "FAULT_PLACEMENT"]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libkda.so")

STATUS = {0: "KDA_SUCCESS", 1: "KDA_ERR_INVALID", 2: "KDA_ERR_UNSUPPORTED",
          3: "KDA_ERR_WORKSPACE", 4: "KDA_ERR_LAUNCH"}
exported_symbols = ("kda_fwd", "kda_workspace_size", "kda_is_supported", "kda_status_string",
                    "kda_shard_affine", "kda_shard_scan", "kda_decode", "kda_fwd_ex", "kda_bwd",
                    "kda_bwd_ex", "kda_bwd_workspace_size", "kda_workspace_faults", "kda_fwd_noalloc")
# kda_fwd_ex variant bits (KDA_FLAG_* in include/kda.h)
FLAG_GATE_GIVEN, FLAG_BETA_GIVEN, FLAG_NO_QK_NORM, FLAG_STATE_VK = 1, 2, 4, 8
# kda_fwd_ex, kda_bwd_ex: reuse the chunk records the previous call left in the workspace
FLAG_REUSE_RECORDS = 16
# kda_fwd_ex: leave every chunk record in the workspace, for a later FLAG_REUSE_RECORDS call
FLAG_KEEP_RECORDS = 32
# kda_fwd_ex: one-sequence calls with >= 16 heads run as one producer/chain launch
FLAG_SINGLE_LAUNCH = 64
# fault-word bits (KDA_FAULT_* in include/kda.h), read by kda_workspace_faults
FAULT_WAIT_TIMEOUT, FAULT_GATE_RANGE, FAULT_QK_NORM, FAULT_PLACEMENT = 1, 2, 4, 8
# size of the static device scratch behind kda_fwd_noalloc (KDA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 160 << 20


class KdaError(RuntimeError):
    """A non-zero kda_status_t returned by the library."""

    def __init__(self, status: int, what: str = "kda_fwd"):
        self.status = status
        super().__init__(f"{what} failed: {STATUS.get(status, status)}")


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
_lib.kda_fwd_ex.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, _P, ctypes.c_size_t, _P, _P,
                            ctypes.c_float, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, ctypes.c_uint, _P]
_lib.kda_fwd_ex.restype = ctypes.c_int
_lib.kda_shard_affine.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P, _P, ctypes.c_float,
                                  _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P]
_lib.kda_shard_affine.restype = ctypes.c_int
_lib.kda_shard_scan.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _P]
_lib.kda_shard_scan.restype = ctypes.c_int
_lib.kda_decode.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, ctypes.c_float, _P, _P,
                            _I64, _I64, _I64, _I64, _I64, _P]
_lib.kda_decode.restype = ctypes.c_int
_lib.kda_bwd_workspace_size.argtypes = [_I64, _I64, _I64]
_lib.kda_bwd_workspace_size.restype = ctypes.c_size_t
_lib.kda_bwd.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                         ctypes.c_size_t, _P, _P, ctypes.c_float, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _P]
_lib.kda_bwd.restype = ctypes.c_int
_lib.kda_bwd_ex.argtypes = _lib.kda_bwd.argtypes[:-1] + [ctypes.c_uint, _P]
_lib.kda_bwd_ex.restype = ctypes.c_int
_lib.kda_workspace_faults.argtypes = [_P, ctypes.POINTER(ctypes.c_uint32), _P]
_lib.kda_workspace_faults.restype = ctypes.c_int
_lib.kda_fwd_noalloc.argtypes = [_P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                                 _I64, _I64, _I64, _I64, _I64, _I64, _P]
_lib.kda_fwd_noalloc.restype = ctypes.c_int


def kda_workspace_size(T: int, H: int, N: int) -> int:
    """Workspace bytes for T packed tokens, H heads and N sequences."""
    return int(_lib.kda_workspace_size(T, H, N))


def kda_is_supported(K: int, V: int, lower_bound: float) -> bool:
    return bool(_lib.kda_is_supported(K, V, lower_bound))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_inputs(q, k, v, raw_gate, raw_beta, out, A_log, dt_bias, cu_seqlens):
    B, T, H, K = q.shape
    V = v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("raw_gate", raw_gate), ("raw_beta", raw_beta),
                    ("out", out)):
        if t is not None and (t.dtype != torch.bfloat16 or not t.is_contiguous() or not t.is_cuda):
            raise ValueError(f"{name} must be a contiguous bf16 device tensor")
    for name, t in (("A_log", A_log), ("dt_bias", dt_bias)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda):
            raise ValueError(f"{name} must be a contiguous fp32 device tensor")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda):
        raise ValueError("cu_seqlens must be an int32 device tensor")
    if tuple(k.shape) != (B, T, H, K) or tuple(raw_gate.shape) != (B, T, H, K) or \
            tuple(v.shape) != (B, T, H, V) or (out is not None and tuple(out.shape) != (B, T, H, V)) or \
            tuple(raw_beta.shape) != (B, T, H):
        raise ValueError("inconsistent q/k/v/raw_gate/raw_beta/out shapes")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    return B, T, H, K, V, N


def _check_f32(name, t, shape):
    if t is None:
        return
    if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name} must be a contiguous fp32 device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}")


def _stream(stream, dev):
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    return ctypes.c_void_p(int(stream))


def kda_fwd(q, k, v, raw_gate, raw_beta, scale, out, workspace, A_log, dt_bias, lower_bound,
            initial_state=None, final_state=None, cu_seqlens=None, stream=None):
    """Enqueue one KDA forward on ``stream`` (default: torch's current stream).

    Tensors are torch device tensors in the layouts of include/kda.h:
    q, k, raw_gate bf16 [B,T,H,K]; v and out bf16 [B,T,H,V]; raw_beta bf16 [B,T,H];
    workspace uint8 [>= kda_workspace_size(B*T, H, N)]; A_log fp32 [H];
    dt_bias fp32 [H,K]; initial_state / final_state fp32 [N,H,K,V] or None;
    cu_seqlens int32 [N+1] or None.  Raises KdaError on a non-zero status.
    """
    if out is None:
        raise ValueError("out is required")
    B, T, H, K, V, N = _check_inputs(q, k, v, raw_gate, raw_beta, out, A_log, dt_bias, cu_seqlens)
    _check_f32("initial_state", initial_state, (N, H, K, V))
    _check_f32("final_state", final_state, (N, H, K, V))
    rc = _lib.kda_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(raw_beta), float(scale),
                      _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                      _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                      _ptr(final_state), _ptr(cu_seqlens), B, T, H, K, V, N, _stream(stream, q.device))
    if rc != 0:
        raise KdaError(rc)


def kda_fwd_noalloc(q, k, v, raw_gate, raw_beta, scale, out, A_log, dt_bias, lower_bound,
                    initial_state=None, final_state=None, cu_seqlens=None, stream=None):
    """kda_fwd without a workspace: the library's static per-GPU scratch of
    NOALLOC_SCRATCH_BYTES is used instead (calls larger than it raise KdaError with
    KDA_ERR_WORKSPACE; calls that overlap on one GPU race)."""
    if out is None:
        raise ValueError("out is required")
    B, T, H, K, V, N = _check_inputs(q, k, v, raw_gate, raw_beta, out, A_log, dt_bias, cu_seqlens)
    _check_f32("initial_state", initial_state, (N, H, K, V))
    _check_f32("final_state", final_state, (N, H, K, V))
    rc = _lib.kda_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(raw_beta), float(scale),
                              _ptr(out), _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                              _ptr(final_state), _ptr(cu_seqlens), B, T, H, K, V, N, _stream(stream, q.device))
    if rc != 0:
        raise KdaError(rc, "kda_fwd_noalloc")


def kda_fwd_ex(q, k, v, raw_gate, raw_beta, scale, out, workspace, A_log, dt_bias, lower_bound,
               initial_state=None, final_state=None, cu_seqlens=None, flags=0, stream=None):
    """kda_fwd with variant flags (an OR of the FLAG_* bits).  With FLAG_GATE_GIVEN,
    A_log and dt_bias may be None; with FLAG_STATE_VK the states are [N,H,V,K];
    FLAG_KEEP_RECORDS leaves every chunk record in the workspace, and
    FLAG_REUSE_RECORDS skips the intra-chunk pass and uses the records that such a
    previous call on this workspace (same inputs but v and the states) left there."""
    if out is None:
        raise ValueError("out is required")
    if not flags & FLAG_GATE_GIVEN and (A_log is None or dt_bias is None):
        raise ValueError("A_log and dt_bias are required unless FLAG_GATE_GIVEN")
    B, T, H, K, V, N = _check_inputs(q, k, v, raw_gate, raw_beta, out, A_log, dt_bias, cu_seqlens)
    st_shape = (N, H, V, K) if flags & FLAG_STATE_VK else (N, H, K, V)
    _check_f32("initial_state", initial_state, st_shape)
    _check_f32("final_state", final_state, st_shape)
    rc = _lib.kda_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(raw_beta), float(scale),
                         _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size(),
                         _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                         _ptr(final_state), _ptr(cu_seqlens), B, T, H, K, V, N, int(flags),
                         _stream(stream, q.device))
    if rc != 0:
        raise KdaError(rc, "kda_fwd_ex")


def kda_shard_affine(q, k, v, raw_gate, raw_beta, workspace, A_log, dt_bias, lower_bound, P, R,
                     cu_seqlens=None, stream=None):
    """Enqueue the per-shard affine maps: every sequence n of the call (a shard)
    takes an entering state S to P[n] S + R[n].  P fp32 [N,H,K,K], R fp32 [N,H,K,V]."""
    B, T, H, K, V, N = _check_inputs(q, k, v, raw_gate, raw_beta, None, A_log, dt_bias, cu_seqlens)
    _check_f32("P", P, (N, H, K, K))
    _check_f32("R", R, (N, H, K, V))
    rc = _lib.kda_shard_affine(_ptr(q), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(raw_beta), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(A_log), _ptr(dt_bias),
                               float(lower_bound), _ptr(P), _ptr(R), _ptr(cu_seqlens), B, T, H, K, V, N,
                               _stream(stream, q.device))
    if rc != 0:
        raise KdaError(rc, "kda_shard_affine")


def kda_shard_scan(P, R, starts, initial_state=None, final_state=None, stream=None):
    """Enqueue the fold over consecutive shards: starts[0] = initial_state (or 0),
    starts[r+1] = P[r] starts[r] + R[r]; final_state gets the state after the last shard."""
    n, H, K, _ = P.shape
    V = R.shape[-1]
    _check_f32("P", P, (n, H, K, K))
    _check_f32("R", R, (n, H, K, V))
    _check_f32("starts", starts, (n, H, K, V))
    _check_f32("initial_state", initial_state, (H, K, V))
    _check_f32("final_state", final_state, (H, K, V))
    rc = _lib.kda_shard_scan(_ptr(P), _ptr(R), _ptr(initial_state), _ptr(starts), _ptr(final_state),
                             n, H, K, V, _stream(stream, P.device))
    if rc != 0:
        raise KdaError(rc, "kda_shard_scan")


def kda_decode(q, k, v, raw_gate, raw_beta, scale, out, A_log, dt_bias, lower_bound,
               initial_state=None, final_state=None, stream=None):
    """Enqueue the token-by-token step over B sequences of T tokens (layouts as for
    kda_fwd, states fp32 [B,H,K,V]; final_state may be initial_state for an in-place
    update).  Raises KdaError on a non-zero status."""
    if out is None:
        raise ValueError("out is required")
    B, T, H, K, V, _ = _check_inputs(q, k, v, raw_gate, raw_beta, out, A_log, dt_bias, None)
    _check_f32("initial_state", initial_state, (B, H, K, V))
    _check_f32("final_state", final_state, (B, H, K, V))
    rc = _lib.kda_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(raw_beta), float(scale), _ptr(out),
                         _ptr(A_log), _ptr(dt_bias), float(lower_bound), _ptr(initial_state),
                         _ptr(final_state), B, T, H, K, V, _stream(stream, q.device))
    if rc != 0:
        raise KdaError(rc, "kda_decode")


def kda_bwd_workspace_size(T: int, H: int, N: int) -> int:
    """Workspace bytes of kda_bwd for T packed tokens, H heads and N sequences."""
    return int(_lib.kda_bwd_workspace_size(T, H, N))


def kda_bwd(q, k, v, raw_gate, raw_beta, scale, d_out, dq, dk, dv, d_raw_gate, d_raw_beta, dA_log,
            d_dt_bias, workspace, A_log, dt_bias, lower_bound, initial_state=None, d_final=None,
            d_initial_state=None, cu_seqlens=None, stream=None):
    """Enqueue the gradients of one KDA forward (same inputs as kda_fwd) for the output
    gradient d_out (bf16 [B,T,H,V]) and the final-state gradient d_final (fp32 [N,H,K,V]
    or None for zero).  Writes dq, dk, d_raw_gate (bf16 [B,T,H,K]), dv (bf16 [B,T,H,V]),
    d_raw_beta (bf16 [B,T,H]), dA_log (fp32 [H]), d_dt_bias (fp32 [H,K]) and, if given,
    d_initial_state (fp32 [N,H,K,V])."""
    kda_bwd_ex(q, k, v, raw_gate, raw_beta, scale, d_out, dq, dk, dv, d_raw_gate, d_raw_beta, dA_log,
               d_dt_bias, workspace, A_log, dt_bias, lower_bound, initial_state, d_final, d_initial_state,
               cu_seqlens, flags=0, stream=stream, _name="kda_bwd")


def kda_bwd_ex(q, k, v, raw_gate, raw_beta, scale, d_out, dq, dk, dv, d_raw_gate, d_raw_beta, dA_log,
               d_dt_bias, workspace, A_log, dt_bias, lower_bound, initial_state=None, d_final=None,
               d_initial_state=None, cu_seqlens=None, flags=0, stream=None, _name="kda_bwd_ex"):
    """kda_bwd for the variants of kda_fwd_ex (an OR of the FLAG_* bits).  With
    FLAG_GATE_GIVEN, A_log, dt_bias, dA_log and d_dt_bias may be None; with FLAG_STATE_VK
    the states and their gradients are [N,H,V,K]."""
    if not flags & FLAG_GATE_GIVEN and (A_log is None or dt_bias is None or dA_log is None or d_dt_bias is None):
        raise ValueError("A_log, dt_bias, dA_log and d_dt_bias are required unless FLAG_GATE_GIVEN")
    B, T, H, K, V, N = _check_inputs(q, k, v, raw_gate, raw_beta, d_out, A_log, dt_bias, cu_seqlens)
    _check_inputs(q, dk, dv, d_raw_gate, d_raw_beta, None, None, None, None)
    if tuple(dq.shape) != tuple(q.shape) or dq.dtype != torch.bfloat16 or not dq.is_contiguous():
        raise ValueError("dq must be a contiguous bf16 tensor shaped like q")
    st_shape = (N, H, V, K) if flags & FLAG_STATE_VK else (N, H, K, V)
    _check_f32("initial_state", initial_state, st_shape)
    _check_f32("d_final", d_final, st_shape)
    _check_f32("d_initial_state", d_initial_state, st_shape)
    _check_f32("dA_log", dA_log, (H,))
    _check_f32("d_dt_bias", d_dt_bias, (H, K))
    rc = _lib.kda_bwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(raw_gate), _ptr(raw_beta), float(scale), _ptr(d_out),
                         _ptr(d_final), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(d_raw_gate), _ptr(d_raw_beta),
                         _ptr(dA_log), _ptr(d_dt_bias), _ptr(d_initial_state), _ptr(workspace),
                         workspace.numel() * workspace.element_size(), _ptr(A_log), _ptr(dt_bias),
                         float(lower_bound), _ptr(initial_state), _ptr(cu_seqlens), B, T, H, K, V, N,
                         int(flags), _stream(stream, q.device))
    if rc != 0:
        raise KdaError(rc, _name)


def kda_workspace_faults(workspace, stream=None) -> int:
    """The fault word (an OR of the FAULT_* bits) of the last call on ``workspace``,
    read after the work enqueued on ``stream`` has finished (this synchronises it)."""
    word = ctypes.c_uint32(0)
    rc = _lib.kda_workspace_faults(_ptr(workspace), ctypes.byref(word), _stream(stream, workspace.device))
    if rc != 0:
        raise KdaError(rc, "kda_workspace_faults")
    return int(word.value)


def raw_call(*args):
    """Call the C entry point with already-marshalled ctypes arguments (tests)."""
    return _lib.kda_fwd(*args)
