"""A differentiable KDA chunked forward for PyTorch training code.

``kda_chunk`` allocates the outputs and workspaces with PyTorch and calls the
library's ``kda_fwd`` in the forward and ``kda_bwd`` in the backward; it adds
no arithmetic of its own.  Gradients flow to q, k, v, raw_gate, raw_beta,
A_log, dt_bias and initial_state from the output and from the final state.
"""

from __future__ import annotations

import torch

from . import (FLAG_KEEP_RECORDS, FLAG_REUSE_RECORDS, kda_bwd_ex, kda_bwd_workspace_size, kda_fwd_ex,
               kda_workspace_size)

__all__ = ["kda_chunk"]


def _sizes(q, v, cu_seqlens):
    B, T, H, K = q.shape
    V = v.shape[-1]
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    return B, T, H, K, V, N


class _KdaChunk(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, raw_gate, raw_beta, A_log, dt_bias, initial_state, scale, lower_bound,
                cu_seqlens, reuse_records):
        B, T, H, K, V, N = _sizes(q, v, cu_seqlens)
        out = torch.empty_like(v)
        final_state = torch.empty(N, H, K, V, dtype=torch.float32, device=q.device)
        size = kda_bwd_workspace_size(B * T, H, N) if reuse_records else kda_workspace_size(B * T, H, N)
        ws = torch.empty(max(size, 1), dtype=torch.uint8, device=q.device)
        kda_fwd_ex(q, k, v, raw_gate, raw_beta, scale, out, ws, A_log, dt_bias, lower_bound, initial_state,
                   final_state, cu_seqlens, flags=FLAG_KEEP_RECORDS if reuse_records else 0)
        ctx.save_for_backward(q, k, v, raw_gate, raw_beta, A_log, dt_bias, initial_state, cu_seqlens)
        ctx.scale, ctx.lower_bound = scale, lower_bound
        # the backward workspace starts with the forward's layout: keep it, records included
        ctx.ws = ws if reuse_records else None
        ctx.set_materialize_grads(False)
        return out, final_state

    @staticmethod
    def backward(ctx, d_out, d_final):
        q, k, v, raw_gate, raw_beta, A_log, dt_bias, initial_state, cu_seqlens = ctx.saved_tensors
        B, T, H, K, V, N = _sizes(q, v, cu_seqlens)
        d_out = torch.zeros_like(v) if d_out is None else d_out.to(torch.bfloat16).contiguous()
        d_final = None if d_final is None else d_final.to(torch.float32).contiguous()
        dq, dk, draw_gate = torch.empty_like(q), torch.empty_like(k), torch.empty_like(raw_gate)
        dv, draw_beta = torch.empty_like(v), torch.empty_like(raw_beta)
        dA_log, ddt_bias = torch.empty_like(A_log), torch.empty_like(dt_bias)
        dinit = None if initial_state is None else torch.empty_like(initial_state)
        if ctx.ws is not None:
            ws, flags = ctx.ws, FLAG_REUSE_RECORDS
        else:
            ws, flags = torch.empty(max(kda_bwd_workspace_size(B * T, H, N), 1), dtype=torch.uint8,
                                    device=q.device), 0
        kda_bwd_ex(q, k, v, raw_gate, raw_beta, ctx.scale, d_out, dq, dk, dv, draw_gate, draw_beta, dA_log,
                   ddt_bias, ws, A_log, dt_bias, ctx.lower_bound, initial_state=initial_state, d_final=d_final,
                   d_initial_state=dinit, cu_seqlens=cu_seqlens, flags=flags)
        ctx.ws = None
        return dq, dk, dv, draw_gate, draw_beta, dA_log, ddt_bias, dinit, None, None, None, None


def kda_chunk(q, k, v, raw_gate, raw_beta, A_log, dt_bias, *, scale=None, lower_bound=-5.0,
              initial_state=None, cu_seqlens=None, reuse_records=False):
    """Differentiable KDA forward; returns (out bf16 [B,T,H,V], final_state fp32 [N,H,K,V]).

    Inputs as for ``kda_fwd``: q, k, v, raw_gate bf16 [B,T,H,*]; raw_beta bf16 [B,T,H];
    A_log fp32 [H]; dt_bias fp32 [H,K]; initial_state fp32 [N,H,K,V] or None (zeros);
    cu_seqlens int32 [N+1] on the device (with B = 1) or None.  ``scale`` defaults to
    K^-1/2.  All tensors must be contiguous and on one GPU, and must not be modified in
    place between the forward and the backward.

    ``reuse_records`` runs the forward in a backward-sized workspace and keeps it until
    the backward, which then skips rebuilding the chunk records (KDA_FLAG_REUSE_RECORDS).
    It trades memory for time: the workspace (about 0.35 MB per chunk and head, 17 GB at
    T = 32768, H = 96) stays allocated from the forward to the backward, which uses the
    records up (a second backward would need the forward again).
    """
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return _KdaChunk.apply(q, k, v, raw_gate, raw_beta, A_log, dt_bias, initial_state, float(scale),
                           float(lower_bound), cu_seqlens, bool(reuse_records))
