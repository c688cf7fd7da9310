"""The differentiable wrapper ``kda_chunk`` (chunked_gated_delta_amd.function) through
torch autograd: its forward equals kda_fwd bit for bit, and the gradients autograd
delivers match the fp64 gradient oracle with the backward's tolerances."""

import numpy as np
import pytest
import torch

import chunked_gated_delta_amd as kda
import workloads as W
from gpu_run import run_gpu
from test_gpu_bwd import compare, cotangents, oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("lengths,reuse", [(None, False), ([70, 0, 5, 64], False), ([70, 0, 5, 64], True)])
def test_autograd_through_the_wrapper(lengths, reuse):
    from chunked_gated_delta_amd.function import kda_chunk

    T = 130 if lengths is None else sum(lengths)
    x = W.random_inputs("fn", 61, 1, T, 3, lengths=lengths)
    leaf = lambda t: t.to(DEV).requires_grad_(True)  # noqa: E731
    q, k, v, g, b = (leaf(t) for t in (x.q, x.k, x.v, x.raw_gate, x.raw_beta))
    al, dt, init = leaf(x.A_log), leaf(x.dt_bias), leaf(x.initial_state)
    cu = None if x.cu_seqlens is None else x.cu_seqlens.to(DEV)
    print(f"kda_chunk {x.name} T={T} lengths={lengths}", flush=True)
    out, fin = kda_chunk(q, k, v, g, b, al, dt, scale=x.scale, lower_bound=x.lower_bound,
                         initial_state=init, cu_seqlens=cu, reuse_records=reuse)
    o_ref, f_ref = run_gpu(x)
    assert np.array_equal(out.detach().double().cpu().numpy().reshape(o_ref.shape), o_ref)
    assert np.array_equal(fin.detach().double().cpu().numpy(), f_ref)

    d_out, d_fin = cotangents(x, 62)
    loss = (out.float() * d_out.to(DEV).float()).sum() + (fin * d_fin.to(DEV)).sum()
    loss.backward()
    torch.cuda.synchronize()
    B, H, K, V, N = x.B, x.H, x.K, x.V, x.N
    f = lambda t, *s: t.grad.double().cpu().numpy().reshape(*s)  # noqa: E731
    got = {"dq": f(q, B * T, H, K), "dk": f(k, B * T, H, K), "dv": f(v, B * T, H, V),
           "d_raw_gate": f(g, B * T, H, K), "d_raw_beta": f(b, B * T, H), "dA_log": f(al, H),
           "d_dt_bias": f(dt, H, K), "d_initial_state": f(init, N, H, K, V)}
    compare(got, oracle(x, d_out, d_fin))


def test_q_and_k_as_one_tensor_sum_their_gradients():
    """With q and k the same leaf, autograd adds dq and dk."""
    from chunked_gated_delta_amd.function import kda_chunk

    x = W.random_inputs("fn_qk", 63, 1, 100, 2)
    x.k = x.q
    qk = x.q.to(DEV).requires_grad_(True)
    v, g, b = x.v.to(DEV), x.raw_gate.to(DEV), x.raw_beta.to(DEV)
    al, dt, init = x.A_log.to(DEV), x.dt_bias.to(DEV), x.initial_state.to(DEV)
    out, fin = kda_chunk(qk, qk, v, g, b, al, dt, scale=x.scale, lower_bound=x.lower_bound, initial_state=init)
    d_out, d_fin = cotangents(x, 64)
    ((out.float() * d_out.to(DEV).float()).sum() + (fin * d_fin.to(DEV)).sum()).backward()
    ref = oracle(x, d_out, d_fin)
    got = qk.grad.double().cpu().numpy().reshape(x.T, x.H, x.K)
    compare({"dq": got}, {"dq": ref["dq"] + ref["dk"]}, names=("dq",))


def test_backward_on_the_forward_records_is_exact():
    """kda_bwd_ex with FLAG_REUSE_RECORDS after kda_fwd_ex with FLAG_KEEP_RECORDS on the
    same (backward-sized) workspace gives the same bits as kda_bwd rebuilding the records."""
    x = W.random_inputs("fn_reuse", 65, 1, 300, 3, lengths=[100, 200])
    t = {n: getattr(x, n).to(DEV) for n in ("q", "k", "v", "raw_gate", "raw_beta", "A_log", "dt_bias",
                                             "initial_state", "cu_seqlens")}
    d_out, d_fin = (c.to(DEV) for c in cotangents(x, 66))
    B, T, H, K, V, N = x.B, x.T, x.H, x.K, x.V, x.N
    size = kda.kda_bwd_workspace_size(B * T, H, N)

    def grads(ws, flags):
        gs = [torch.empty_like(t[n]) for n in ("q", "k", "v", "raw_gate", "raw_beta", "A_log", "dt_bias",
                                                "initial_state")]
        kda.kda_bwd_ex(t["q"], t["k"], t["v"], t["raw_gate"], t["raw_beta"], x.scale, d_out, gs[0], gs[1], gs[2],
                       gs[3], gs[4], gs[5], gs[6], ws, t["A_log"], t["dt_bias"], x.lower_bound,
                       initial_state=t["initial_state"], d_final=d_fin, d_initial_state=gs[7],
                       cu_seqlens=t["cu_seqlens"], flags=flags)
        return gs

    ws = torch.empty(size, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(t["v"])
    fin = torch.empty(N, H, K, V, device=DEV)
    print("kda_fwd then kda_bwd_ex(REUSE_RECORDS) on one workspace", flush=True)
    kda.kda_fwd_ex(t["q"], t["k"], t["v"], t["raw_gate"], t["raw_beta"], x.scale, out, ws, t["A_log"],
                   t["dt_bias"], x.lower_bound, t["initial_state"], fin, t["cu_seqlens"],
                   flags=kda.FLAG_KEEP_RECORDS)
    reused = grads(ws, kda.FLAG_REUSE_RECORDS)
    fresh = grads(torch.empty(size, dtype=torch.uint8, device=DEV), 0)
    torch.cuda.synchronize()
    for a, b in zip(reused, fresh):
        assert torch.equal(a, b)
