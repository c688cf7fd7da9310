"""Run the HIP path (through the C ABI binding) on a KdaInputs workload."""

import numpy as np
import torch

import chunked_gated_delta_amd as kda


def to_dev(x, dev="cuda:0"):
    return None if x is None else x.to(dev)


def run_gpu(x, *, with_init=True, with_final=True, in_place=False, q_alias_k=None, dev="cuda:0",
            stream=None):
    """Returns (out fp64 numpy [B*T, H, V], final fp64 numpy [N, H, K, V] or None)."""
    q = to_dev(x.q, dev)
    k = q if (q_alias_k if q_alias_k is not None else x.q_is_k) else to_dev(x.k, dev)
    v, g, b = to_dev(x.v, dev), to_dev(x.raw_gate, dev), to_dev(x.raw_beta, dev)
    al, dt = to_dev(x.A_log, dev), to_dev(x.dt_bias, dev)
    cu = to_dev(x.cu_seqlens, dev)
    init = to_dev(x.initial_state, dev) if with_init else None
    out = torch.full_like(v, float("nan"))
    if in_place:
        assert init is not None
        fin = init
    elif with_final:
        fin = torch.full((x.N, x.H, x.K, x.V), float("nan"), dtype=torch.float32, device=dev)
    else:
        fin = None
    ws = torch.empty(kda.kda_workspace_size(x.B * x.T, x.H, x.N), dtype=torch.uint8, device=dev)
    kda.kda_fwd(q, k, v, g, b, x.scale, out, ws, al, dt, x.lower_bound, init, fin, cu,
                stream=stream)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy().reshape(x.B * x.T, x.H, x.V)
    f = None if fin is None else fin.double().cpu().numpy()
    return o, f
