"""Second CPU form of the KDA forward: fp64 chunk algebra (WY/UT form).

Test infrastructure only; see the package docstring.  This form exists to
check the token recurrence, so it shares none of its code (its own prep, its
own state update).  It is the chunked computation that the fla ``chunk_kda``
call on the instagit FlashKDA page ("Usage Examples") names, with 64-token
chunks and partial tail chunks as in the llm-atlas FlashKDA probe page (its
correctness suite covers one chunk, a partial tail and multiple chunks).  The
pages do not print the chunk algebra; it is derived from the token recurrence:

For one chunk of L tokens with start state S0, per-channel inclusive cumulative
log-decay G_i = sum_{s<=i} g_s (reset at every chunk), and normalised q^, k^:
  A_kk[i,j] = beta_i * sum_c k^_ic k^_jc exp(G_ic - G_jc)   (j < i, else 0)
  T  = (I + A_kk)^-1
  W  = T diag(beta) (K^ * exp(G))          U = T diag(beta) V
  D  = U - W S0                              (the per-token delta-rule errors)
  A_qk[i,j] = sum_c q^_ic k^_jc exp(G_ic - G_jc)              (j <= i, else 0)
  O  = scale * [ (Q^ * exp(G)) S0 + A_qk D ]
  S_L = Diag(exp(G_L)) S0 + (K^ * exp(G_L - G))^T D
exp(G_i - G_j) is evaluated pairwise, so no factor overflows.
"""

from __future__ import annotations

import numpy as np
import scipy.linalg
import torch


def _widen(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def _prep(q, k, raw_gate, raw_beta, A_log, dt_bias, lower_bound, eps=1e-6):
    """Per token and head: q^, k^, beta and the log-decay g (all fp64)."""
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + eps)
    kn = k / np.sqrt((k * k).sum(-1, keepdims=True) + eps)
    beta = 1.0 / (1.0 + np.exp(-raw_beta))
    x = np.exp(A_log)[:, None] * (raw_gate + dt_bias)          # [.., H, K]
    g = lower_bound / (1.0 + np.exp(-x))
    return qn, kn, beta, g


def _chunk(qn, kn, v, beta, g, S0, scale):
    """One chunk of one head: returns (O [L,V], S_L [K,V])."""
    L = qn.shape[0]
    G = np.cumsum(g, axis=0)                                   # [L, K]
    decay = np.exp(G[:, None, :] - G[None, :, :])              # [L, L, K] = exp(G_i - G_j)
    lower = np.tril(np.ones((L, L)), -1)
    incl = np.tril(np.ones((L, L)), 0)
    # the upper triangle of `decay` may hold large values; it is dropped by where()
    kk = np.where(lower > 0, np.einsum("ic,jc,ijc->ij", kn, kn, np.where(lower[:, :, None] > 0, decay, 0.0)), 0.0)
    A_kk = beta[:, None] * kk
    qk = np.einsum("ic,jc,ijc->ij", qn, kn, np.where(incl[:, :, None] > 0, decay, 0.0))
    A_qk = np.where(incl > 0, qk, 0.0)
    eye = np.eye(L)
    Gam = np.exp(G)
    rhs = np.concatenate([beta[:, None] * (kn * Gam), beta[:, None] * v], axis=1)
    WU = scipy.linalg.solve_triangular(eye + A_kk, rhs, lower=True, unit_diagonal=True)
    W, U = WU[:, :kn.shape[1]], WU[:, kn.shape[1]:]
    D = U - W @ S0
    O = scale * ((qn * Gam) @ S0 + A_qk @ D)
    GL = G[-1]
    S_L = np.exp(GL)[:, None] * S0 + (kn * np.exp(GL[None, :] - G)).T @ D
    return O, S_L


def chunked_fwd(q, k, v, raw_gate, raw_beta, scale, A_log, dt_bias, lower_bound,
                initial_state=None, cu_seqlens=None, chunk: int = 64):
    """Chunked fp64 forward with the same argument meaning as ``oracle_fwd``.

    Returns (out fp64 [B*T, H, V], final fp64 [N, H, K, V]).
    """
    B, T, H, K = q.shape
    V = v.shape[-1]
    qf = _widen(q).reshape(B * T, H, K)
    kf = _widen(k).reshape(B * T, H, K)
    vf = _widen(v).reshape(B * T, H, V)
    gf = _widen(raw_gate).reshape(B * T, H, K)
    bf = _widen(raw_beta).reshape(B * T, H)
    qn, kn, beta, g = _prep(qf, kf, gf, bf, _widen(A_log), _widen(dt_bias), float(lower_bound))
    if cu_seqlens is None:
        bounds = [(b * T, (b + 1) * T) for b in range(B)]
    else:
        cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        bounds = [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    N = len(bounds)
    out = np.zeros((B * T, H, V))
    fin = np.zeros((N, H, K, V))
    init = None if initial_state is None else _widen(initial_state)
    for n, (s, e) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((K, V)) if init is None else init[n, h].copy()
            for c0 in range(s, e, chunk):
                c1 = min(c0 + chunk, e)
                O, S = _chunk(qn[c0:c1, h], kn[c0:c1, h], vf[c0:c1, h], beta[c0:c1, h],
                              g[c0:c1, h], S, scale)
                out[c0:c1, h] = O
            fin[n, h] = S
    return out, fin
