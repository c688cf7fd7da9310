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


# ---------------------------------------------------------------------------
# Backward of the chunk algebra above.  Given dO = d loss / d O and
# dS_L = d loss / d S_L for one chunk, reverse-mode differentiation of the
# formulas in the module docstring gives (Tb = T diag(beta), KG = K^ exp(G),
# QG = Q^ exp(G), Kt = K^ exp(G_L - G)):
#   dD   = scale A_qk^T dO + Kt dS_L
#   dS0  = Diag(exp(G_L)) dS_L + scale QG^T dO - W^T dD
#   dA_qk = scale dO D^T (j <= i)       dKt = D dS_L^T       dW = -dD S0^T
#   dTb  = dD V^T + dW KG^T             dV = Tb^T dD         dKG = Tb^T dW
#   dT   = dTb diag(beta)               dbeta_j += sum_i dTb_ij T_ij
#   dA_kk = -(T^T dT T^T) (j < i)       dbeta_i += sum_j dA_kk_ij kk_ij
# and the pairwise products A[i,j] = sum_c x_ic k^_jc exp(G_ic - G_jc) send
# dA[i,j] * k^_j exp(G_i - G_j) to x_i, dA[i,j] * x_i exp(G_i - G_j) to k^_j,
# and +/- their channel-wise products to G_i / G_j.  The chunk-local
# cumulative sum G turns into a reverse cumulative sum for dg.
# ---------------------------------------------------------------------------


def _pair_grads(dA, x, kn, decay, mask):
    """Gradients of A[i,j] = sum_c x_ic kn_jc decay_ijc (mask_ij) w.r.t. x, kn and G."""
    dAm = np.where(mask > 0, dA, 0.0)
    P = np.where(mask[:, :, None] > 0, decay, 0.0) * dAm[:, :, None]   # [L, L, K]
    dx = np.einsum("ijc,jc->ic", P, kn)
    dk = np.einsum("ijc,ic->jc", P, x)
    prod = P * x[:, None, :] * kn[None, :, :]
    dG = prod.sum(axis=1) - prod.sum(axis=0)
    return dx, dk, dG


def _chunk_bwd(qn, kn, v, beta, g, S0, scale, dO, dSL):
    """One chunk of one head: gradients w.r.t. (qn, kn, v, beta, g, S0)."""
    L, K = qn.shape
    G = np.cumsum(g, axis=0)
    decay = np.exp(np.where(np.tril(np.ones((L, L)), 0)[:, :, None] > 0, G[:, None, :] - G[None, :, :], 0.0))
    lower = np.tril(np.ones((L, L)), -1)
    incl = np.tril(np.ones((L, L)), 0)
    kk = np.where(lower > 0, np.einsum("ic,jc,ijc->ij", kn, kn, decay), 0.0)
    A_kk = beta[:, None] * kk
    A_qk = np.where(incl > 0, np.einsum("ic,jc,ijc->ij", qn, kn, decay), 0.0)
    Tm = scipy.linalg.solve_triangular(np.eye(L) + A_kk, np.eye(L), lower=True, unit_diagonal=True)
    Gam = np.exp(G)
    GL = G[-1]
    KG, QG, Kt = kn * Gam, qn * Gam, kn * np.exp(GL[None, :] - G)
    Tb = Tm * beta[None, :]
    W, U = Tb @ KG, Tb @ v
    D = U - W @ S0

    dD = scale * A_qk.T @ dO + Kt @ dSL
    dS0 = np.exp(GL)[:, None] * dSL + scale * QG.T @ dO - W.T @ dD
    dGL = (dSL * S0).sum(axis=1) * np.exp(GL)
    dAqk = scale * dO @ D.T
    dKt = D @ dSL.T
    dW = -dD @ S0.T
    dTb = dD @ v.T + dW @ KG.T
    dv = Tb.T @ dD
    dKG = Tb.T @ dW
    dT = dTb * beta[None, :]
    dbeta = (dTb * Tm).sum(axis=0)
    dAkk = -(Tm.T @ dT @ Tm.T)
    dbeta += np.where(lower > 0, dAkk * kk, 0.0).sum(axis=1)
    dkk = dAkk * beta[:, None]

    dq1, dk1, dG1 = _pair_grads(dAqk, qn, kn, decay, incl)
    dka, dkb, dG2 = _pair_grads(dkk, kn, kn, decay, lower)
    dQG = scale * dO @ S0.T
    dqn = dq1 + dQG * Gam
    dkn = dk1 + dka + dkb + dKG * Gam + dKt * np.exp(GL[None, :] - G)
    dG = dG1 + dG2 + dQG * QG + dKG * KG - dKt * Kt
    dGL = dGL + (dKt * Kt).sum(axis=0)
    dG[-1] += dGL
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return dqn, dkn, dv, dbeta, dg, dS0


def chunked_bwd(q, k, v, raw_gate, raw_beta, scale, A_log, dt_bias, lower_bound, d_out, d_final=None,
                initial_state=None, cu_seqlens=None, chunk: int = 64):
    """Chunked fp64 backward with the argument meaning and return dict of ``oracle.grad.oracle_bwd``."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    qf = _widen(q).reshape(B * T, H, K)
    kf = _widen(k).reshape(B * T, H, K)
    vf = _widen(v).reshape(B * T, H, V)
    gf = _widen(raw_gate).reshape(B * T, H, K)
    bf = _widen(raw_beta).reshape(B * T, H)
    A_log_, dt_ = _widen(A_log), _widen(dt_bias)
    lb = float(lower_bound)
    qn, kn, beta, g = _prep(qf, kf, gf, bf, A_log_, dt_, lb)
    dO_all = _widen(d_out).reshape(B * T, H, V)
    if cu_seqlens is None:
        bounds = [(b * T, (b + 1) * T) for b in range(B)]
    else:
        cu = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
        bounds = [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    N = len(bounds)
    init = None if initial_state is None else _widen(initial_state)
    dfin = None if d_final is None else _widen(d_final)
    dqn, dkn = np.zeros_like(qn), np.zeros_like(kn)
    dv, dbeta, dg = np.zeros_like(vf), np.zeros_like(beta), np.zeros_like(g)
    dinit = np.zeros((N, H, K, V))
    for n, (s, e) in enumerate(bounds):
        starts = list(range(s, e, chunk))
        for h in range(H):
            S = np.zeros((K, V)) if init is None else init[n, h].copy()
            S_at = []
            for c0 in starts:
                c1 = min(c0 + chunk, e)
                S_at.append(S)
                _, S = _chunk(qn[c0:c1, h], kn[c0:c1, h], vf[c0:c1, h], beta[c0:c1, h], g[c0:c1, h], S, scale)
            dS = np.zeros((K, V)) if dfin is None else dfin[n, h].copy()
            for c0, S0 in reversed(list(zip(starts, S_at))):
                c1 = min(c0 + chunk, e)
                r = _chunk_bwd(qn[c0:c1, h], kn[c0:c1, h], vf[c0:c1, h], beta[c0:c1, h], g[c0:c1, h], S0,
                               scale, dO_all[c0:c1, h], dS)
                dqn[c0:c1, h], dkn[c0:c1, h], dv[c0:c1, h], dbeta[c0:c1, h], dg[c0:c1, h], dS = r
            dinit[n, h] = dS
    # back through the per-token preparation
    rq = np.sqrt((qf * qf).sum(-1, keepdims=True) + 1e-6)
    rk = np.sqrt((kf * kf).sum(-1, keepdims=True) + 1e-6)
    dq = (dqn - qn * (qn * dqn).sum(-1, keepdims=True)) / rq
    dk = (dkn - kn * (kn * dkn).sum(-1, keepdims=True)) / rk
    d_raw_beta = dbeta * beta * (1.0 - beta)
    a = np.exp(A_log_)[:, None]
    x = a * (gf + dt_)
    sx = 1.0 / (1.0 + np.exp(-x))
    dx = dg * lb * sx * (1.0 - sx)
    return {
        "dq": dq, "dk": dk, "dv": dv, "d_raw_gate": dx * a, "d_raw_beta": d_raw_beta,
        "dA_log": (dx * x).sum(axis=(0, 2)), "d_dt_bias": (dx * a).sum(axis=0),
        "d_initial_state": None if init is None else dinit,
    }
