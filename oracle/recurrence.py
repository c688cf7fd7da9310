"""The oracle proper: fp64 token-by-token KDA recurrence (C, via ctypes).

Test infrastructure only; see the package docstring.

``oracle_fwd`` follows the per-token gated delta rule stated in
``kda_oracle.c`` (decay, delta-rule erase/write, output read from the updated
state), with q/k L2-normalised, beta = sigmoid(raw_beta) and the bounded gate
g = lower_bound * sigmoid(exp(A_log) * (raw_gate + dt_bias)); the argument
roles are those of the 14-argument FlashKDA call in the vLLM PR report
("关键源码片段") and the in-kernel flags of the chunk_kda call on the
instagit FlashKDA page ("Usage Examples").
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
            _build.build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.kda_oracle_fwd.argtypes = [P, P, P, P, P, ctypes.c_double, P, P, ctypes.c_double,
                                       P, P, I64, I64, I64, I64, I64, P, I64, P, P, ctypes.c_int,
                                       ctypes.c_int]
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def oracle_threads() -> int:
    """Number of OpenMP threads the oracle uses by default."""
    return int(_lib().kda_oracle_threads())


def _bits(t: torch.Tensor) -> np.ndarray:
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _f32(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().float().contiguous().numpy()
    return np.ascontiguousarray(t, dtype=np.float32)


# variant bits (the chunk_kda in-kernel switches on the instagit FlashKDA page)
GATE_GIVEN, BETA_GIVEN, NO_QK_NORM, STATE_VK = 1, 2, 4, 8


def oracle_fwd(q, k, v, raw_gate, raw_beta, scale, A_log, dt_bias, lower_bound,
               initial_state=None, cu_seqlens=None, heads=None, threads: int = 0,
               want_final: bool = True, flags: int = 0):
    """Run the fp64 recurrence.

    flags: GATE_GIVEN (raw_gate holds the log-decay g, which must lie in
    [lower_bound, 0]; other values raise ValueError), BETA_GIVEN (raw_beta holds beta), NO_QK_NORM (no L2
    norm of q, k), STATE_VK (states stored transposed, [N, H, V, K]).

    q, k, raw_gate: bf16 [B, T, H, K]; v: bf16 [B, T, H, V]; raw_beta: bf16 [B, T, H];
    A_log fp32 [H]; dt_bias fp32 [H, K]; initial_state fp32 [N, H, K, V] or None;
    cu_seqlens int32 [N+1] or None (then N = B sequences of length T).
    heads: optional list of head indices to evaluate (default: all).
    Returns (out fp64 [B*T, nh, V], final fp64 [N, nh, K, V] ([N, nh, V, K] with STATE_VK) or None).
    """
    B, T, H, K = q.shape
    V = v.shape[-1]
    assert k.shape == q.shape and raw_gate.shape == q.shape
    assert v.shape[:3] == q.shape[:3] and raw_beta.shape == q.shape[:3]
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int32) * T
    else:
        assert B == 1
        cu = np.ascontiguousarray(
            cu_seqlens.cpu().numpy() if isinstance(cu_seqlens, torch.Tensor) else cu_seqlens,
            dtype=np.int32)
    N = cu.size - 1
    hs = np.arange(H, dtype=np.int32) if heads is None else np.asarray(heads, dtype=np.int32)
    nh = hs.size
    qb, kb, vb, gb, bb = (_bits(x) for x in (q, k, v, raw_gate, raw_beta))
    al, dt = _f32(A_log), _f32(dt_bias)
    init = None if initial_state is None else _f32(initial_state)
    out = np.empty((B * T, nh, V), dtype=np.float64)
    # the C routine writes each final state in the layout the flags name: [V][K] with STATE_VK
    fin_shape = (N, nh, V, K) if flags & STATE_VK else (N, nh, K, V)
    fin = np.empty(fin_shape, dtype=np.float64) if want_final else None
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    rc = _lib().kda_oracle_fwd(ptr(qb), ptr(kb), ptr(vb), ptr(gb), ptr(bb), float(scale),
                               ptr(al), ptr(dt), float(lower_bound), ptr(init), ptr(cu),
                               N, B * T, H, K, V, ptr(hs), nh, ptr(out), ptr(fin), int(threads),
                               int(flags))
    if rc == -2:
        raise ValueError("given gate outside [lower_bound, 0]")
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return out, fin


def metrics(x: np.ndarray, ref: np.ndarray) -> dict:
    """Whole-tensor comparison of a result x with its reference ref (same shape):
    rel-L2 = |x-ref|_2/|ref|_2 (|x-ref|_2 itself when ref is all zero), max-abs
    = max |x-ref|, and whether every element of x is finite.  A shape mismatch
    or a non-finite reference raises ValueError: no broadcasting, and a broken
    reference never passes as a comparison."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if x.shape != ref.shape:
        raise ValueError(f"metrics: shape {x.shape} != reference shape {ref.shape}")
    if not np.isfinite(ref).all():
        raise ValueError("metrics: the reference holds non-finite values")
    finite = bool(np.isfinite(x).all())
    d = x - ref
    nref = float(np.linalg.norm(ref.ravel()))
    nd = float(np.linalg.norm(d.ravel())) if finite else float("inf")
    return {
        "rel_l2": nd / nref if nref > 0 else nd,
        "max_abs": float(np.abs(d).max()) if finite and d.size else (0.0 if finite else float("inf")),
        "finite": finite,
    }


def oracle_shard_affine(q, k, v, raw_gate, raw_beta, A_log, dt_bias, lower_bound, cu_seqlens=None,
                        heads=None, threads: int = 0):
    """Affine map of every sequence (shard) of the call, in fp64.

    Each token applies S -> (I - b k^ k^T) Diag(exp(g)) S + b k^ v^T, so a whole
    shard maps its entering state S to P S + R with
        R = the shard's final state from S = 0,
        P = the shard's final state with v = 0 from S = I   (needs K == V).
    This is the split that context parallelism over one sequence needs (the
    torchtitan PR page names KDA context parallelism without giving its form).
    Returns (P fp64 [N, nh, K, K], R fp64 [N, nh, K, V]).
    """
    B, T, H, K = q.shape
    V = v.shape[-1]
    if K != V:
        raise ValueError("the affine map is computed as a state, which needs K == V")
    _, R = oracle_fwd(q, k, v, raw_gate, raw_beta, 1.0, A_log, dt_bias, lower_bound, None,
                      cu_seqlens, heads, threads)
    N = B if cu_seqlens is None else (len(cu_seqlens) - 1)
    eye = np.broadcast_to(np.eye(K, dtype=np.float32), (N, H, K, K)).copy()
    _, P = oracle_fwd(q, k, torch.zeros_like(v), raw_gate, raw_beta, 1.0, A_log, dt_bias,
                      lower_bound, eye, cu_seqlens, heads, threads)
    return P, R


def oracle_shard_fold(P, R, initial_state=None):
    """Fold consecutive shards' maps in fp64: starts[0] = S0 (or 0),
    starts[r+1] = P[r] starts[r] + R[r].  P [n, H, K, K], R [n, H, K, V],
    initial_state [H, K, V] or None.  Returns (starts [n, H, K, V], final [H, K, V])."""
    P = np.asarray(P, dtype=np.float64)
    R = np.asarray(R, dtype=np.float64)
    n, H, K, V = R.shape
    S = np.zeros((H, K, V)) if initial_state is None else np.asarray(initial_state, dtype=np.float64).copy()
    starts = np.empty((n, H, K, V))
    for r in range(n):
        starts[r] = S
        S = np.matmul(P[r], S) + R[r]
    return starts, S
