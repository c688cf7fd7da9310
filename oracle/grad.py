"""Gradients of the KDA forward: fp64 autograd of the token recurrence.

Test infrastructure only; see the package docstring.  The forward here is the
same per-token gated delta rule as ``kda_oracle.c`` (decay, delta-rule erase
and write, output read from the updated state; q, k L2-normalised, beta =
sigmoid(raw_beta), g = lower_bound * sigmoid(exp(A_log) (raw_gate + dt_bias)))
written with differentiable PyTorch CPU ops in fp64, so torch.autograd gives
the exact gradients of
    loss = <d_out, out> + <d_final, final_state>
with respect to every input.  The pages ask for a forward and its gradient
(the torchtitan PR page, "Summary") but print neither; this is the plain
definition.  ``fwd_torch`` (the same graph without gradients) is checked
against the C oracle, and the gradients against central finite differences of
``fwd_torch``.
"""

from __future__ import annotations

import torch

EPS = 1e-6


def _f64(t):
    return None if t is None else t.detach().cpu().to(torch.float64)


GATE_GIVEN, BETA_GIVEN, NO_QK_NORM, STATE_VK = 1, 2, 4, 8


def fwd_torch(q, k, v, raw_gate, raw_beta, scale, A_log, dt_bias, lower_bound, initial_state=None,
              cu_seqlens=None, flags=0):
    """fp64 token recurrence on fp64 tensors (differentiable).  Shapes as oracle_fwd:
    q, k, raw_gate [B, T, H, K]; v [B, T, H, V]; raw_beta [B, T, H]; A_log [H]; dt_bias [H, K];
    initial_state [N, H, K, V] ([N, H, V, K] with STATE_VK) or None.  ``flags`` are the variant
    switches of oracle_fwd: GATE_GIVEN (raw_gate is the natural-log decay, in
    [lower_bound, 0]; other values raise ValueError), BETA_GIVEN (raw_beta is beta), NO_QK_NORM, STATE_VK (transposed states).
    Returns (out [B*T, H, V], final [N, H, K, V] or [N, H, V, K])."""
    B, T, H, K = q.shape
    V = v.shape[-1]
    qf, kf, gf = (x.reshape(B * T, H, K) for x in (q, k, raw_gate))
    vf = v.reshape(B * T, H, V)
    bf = raw_beta.reshape(B * T, H)
    if cu_seqlens is None:
        bounds = [(b * T, (b + 1) * T) for b in range(B)]
    else:
        cu = [int(x) for x in cu_seqlens]
        bounds = [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    vk = bool(flags & STATE_VK)
    if flags & GATE_GIVEN and not bool(((gf >= lower_bound) & (gf <= 0.0)).all()):
        raise ValueError("given gate outside [lower_bound, 0]")
    a = None if flags & GATE_GIVEN else torch.exp(A_log)[:, None]          # [H, 1]
    outs, fins = [], []
    for n, (s, e) in enumerate(bounds):
        if initial_state is None:
            S = torch.zeros(H, K, V, dtype=torch.float64)
        else:
            S = initial_state[n].transpose(-1, -2) if vk else initial_state[n]
        for t in range(s, e):
            if flags & NO_QK_NORM:
                qh, kh = qf[t], kf[t]
            else:
                qh = qf[t] / torch.sqrt((qf[t] * qf[t]).sum(-1, keepdim=True) + EPS)   # [H, K]
                kh = kf[t] / torch.sqrt((kf[t] * kf[t]).sum(-1, keepdim=True) + EPS)
            beta = bf[t] if flags & BETA_GIVEN else torch.sigmoid(bf[t])            # [H]
            if flags & GATE_GIVEN:
                alpha = torch.exp(gf[t])
            else:
                alpha = torch.exp(lower_bound * torch.sigmoid(a * (gf[t] + dt_bias)))   # [H, K]
            S = alpha[:, :, None] * S
            pred = torch.einsum("hkv,hk->hv", S, kh)
            delta = beta[:, None] * (vf[t] - pred)
            S = S + kh[:, :, None] * delta[:, None, :]
            outs.append(scale * torch.einsum("hkv,hk->hv", S, qh))
        fins.append(S.transpose(-1, -2) if vk else S)
    out = torch.stack(outs) if outs else torch.zeros(0, H, V, dtype=torch.float64)
    return out, torch.stack(fins)


def oracle_bwd(q, k, v, raw_gate, raw_beta, scale, A_log, dt_bias, lower_bound, d_out, d_final=None,
               initial_state=None, cu_seqlens=None, flags=0):
    """Gradients (fp64) of <d_out, out> + <d_final, final> at the given inputs (bf16 inputs
    are widened exactly).  d_out [B, T, H, V] (or [B*T, H, V]), d_final [N, H, K, V] or None
    (states [N, H, V, K] with STATE_VK).  Returns a dict with dq, dk, dv, d_raw_gate
    ([B*T, H, *]), d_raw_beta [B*T, H], dA_log [H], d_dt_bias [H, K] (zero with GATE_GIVEN),
    d_initial_state (None without initial_state)."""
    xs = {n: _f64(t).requires_grad_(True) for n, t in
          (("q", q), ("k", k), ("v", v), ("raw_gate", raw_gate), ("raw_beta", raw_beta), ("A_log", A_log),
           ("dt_bias", dt_bias))}
    init = None if initial_state is None else _f64(initial_state).requires_grad_(True)
    cu = None if cu_seqlens is None else [int(x) for x in cu_seqlens]
    out, fin = fwd_torch(xs["q"], xs["k"], xs["v"], xs["raw_gate"], xs["raw_beta"], float(scale), xs["A_log"],
                         xs["dt_bias"], float(lower_bound), init, cu, flags)
    loss = (out * _f64(d_out).reshape(out.shape)).sum()
    if d_final is not None:
        loss = loss + (fin * _f64(d_final)).sum()
    loss.backward()
    B, T, H, K = q.shape
    V = v.shape[-1]
    g = {n: (xs[n].grad if xs[n].grad is not None else torch.zeros_like(xs[n])) for n in xs}
    return {
        "dq": g["q"].reshape(B * T, H, K).numpy(), "dk": g["k"].reshape(B * T, H, K).numpy(),
        "dv": g["v"].reshape(B * T, H, V).numpy(), "d_raw_gate": g["raw_gate"].reshape(B * T, H, K).numpy(),
        "d_raw_beta": g["raw_beta"].reshape(B * T, H).numpy(), "dA_log": g["A_log"].numpy(),
        "d_dt_bias": g["dt_bias"].numpy(),
        "d_initial_state": None if init is None else init.grad.numpy(),
    }
