"""40-digit decimal brute force of the KDA forward for tiny T.

Test infrastructure only; see the package docstring.  It checks the token
recurrence with a different formula: the unrolled solution of the linear
state recurrence with explicit K x K transition matrices,

  M_s = (I - beta_s k^_s k^_s^T) Diag(alpha_s)
  S_t = (M_t ... M_1) S_0 + sum_{s<=t} (M_t ... M_{s+1}) beta_s k^_s v_s^T
  o_t = scale * S_t^T q^_t

with every step (L2 norm, sigmoid, exp) evaluated in ``decimal`` at 40
significant digits.  The transition is the per-channel gated delta rule named
by the pages' kernel flags (instagit FlashKDA page, "Usage Examples"); the gate
g = lower_bound * sigmoid(exp(A_log) * (raw_gate + dt_bias)) is the adopted
reading.
"""

from __future__ import annotations

from decimal import Decimal, getcontext

import torch

EPS = Decimal("0.000001")


def _dec(x) -> Decimal:
    return Decimal(float(x))  # exact: every float is a finite binary fraction


def _sig(x: Decimal) -> Decimal:
    return Decimal(1) / (Decimal(1) + (-x).exp())


def _matmul(A, B):
    n, m, p = len(A), len(B), len(B[0])
    return [[sum((A[i][k] * B[k][j] for k in range(m)), Decimal(0)) for j in range(p)]
            for i in range(n)]


def brute_fwd(q, k, v, raw_gate, raw_beta, scale, A_log, dt_bias, lower_bound,
              initial_state=None, head: int = 0, digits: int = 40, gate_given=False,
              beta_given=False, no_qk_norm=False):
    """One sequence (B=1), one head.  Returns (out [T][V], final [K][V]) as Decimals.

    gate_given: raw_gate is the log-decay g itself, which must lie in [lower_bound, 0]
    (other values raise ValueError);
    beta_given: raw_beta is beta itself; no_qk_norm: q, k are used unnormalised."""
    getcontext().prec = digits
    _, T, H, K = q.shape
    V = v.shape[-1]
    to = lambda t: t.detach().cpu().to(torch.float64)  # noqa: E731  (exact widening)
    qf, kf, vf, gf, bf = to(q)[0, :, head], to(k)[0, :, head], to(v)[0, :, head], \
        to(raw_gate)[0, :, head], to(raw_beta)[0, :, head]
    al = _dec(to(A_log)[head])
    dt = [_dec(x) for x in to(dt_bias)[head].tolist()]
    lb = _dec(lower_bound)
    sc = _dec(scale)

    def norm(row):
        xs = [_dec(x) for x in row.tolist()]
        if no_qk_norm:
            return xs
        r = Decimal(1) / (sum((x * x for x in xs), Decimal(0)) + EPS).sqrt()
        return [x * r for x in xs]

    def given_gate(x):
        if x < lb or x > 0:
            raise ValueError("given gate outside [lower_bound, 0]")
        return x

    qn = [norm(qf[t]) for t in range(T)]
    kn = [norm(kf[t]) for t in range(T)]
    beta = [_dec(bf[t]) if beta_given else _sig(_dec(bf[t])) for t in range(T)]
    gm = al.exp()
    if gate_given:
        alpha = [[given_gate(_dec(gf[t, c])).exp() for c in range(K)] for t in range(T)]
    else:
        alpha = [[(lb * _sig(gm * (_dec(gf[t, c]) + dt[c]))).exp() for c in range(K)]
                 for t in range(T)]
    # transition matrices M_s = (I - beta k k^T) Diag(alpha)
    Ms = []
    for s in range(T):
        M = [[((Decimal(1) if i == j else Decimal(0)) - beta[s] * kn[s][i] * kn[s][j]) * alpha[s][j]
              for j in range(K)] for i in range(K)]
        Ms.append(M)
    if initial_state is None:
        S0 = [[Decimal(0)] * V for _ in range(K)]
    else:
        init = initial_state.detach().cpu().to(torch.float64)[0, head]
        S0 = [[_dec(init[i, j]) for j in range(V)] for i in range(K)]
    vdec = [[_dec(x) for x in vf[t].tolist()] for t in range(T)]
    outs = []
    S = None
    zero_start = initial_state is None
    for t in range(T):
        # P = M_t ... M_1 applied to S0 (skipped when S0 is zero)
        acc = S0
        if not zero_start:
            for s in range(t + 1):
                acc = _matmul(Ms[s], acc)
        S = acc
        for s in range(t + 1):
            # (M_t ... M_{s+1}) beta_s k_s v_s^T
            vec = [[beta[s] * kn[s][i]] for i in range(K)]
            for r in range(s + 1, t + 1):
                vec = _matmul(Ms[r], vec)
            S = [[S[i][j] + vec[i][0] * vdec[s][j] for j in range(V)] for i in range(K)]
        outs.append([sc * sum((S[i][j] * qn[t][i] for i in range(K)), Decimal(0)) for j in range(V)])
    return outs, S
