"""kda_fwd (both schedules) and kda_decode captured in a HIP graph (torch.cuda.CUDAGraph on ROCm).

Neither entry point records a memset or allocates, so both can be captured: the
forward's launches (chunk prefix or counter reset, intra, inter) and the decode
step replay on the captured buffers.  Every replay is checked against an eager
call on the same inputs, with eager work and synchronisations between replays.
"""

import numpy as np
import pytest
import torch

import chunked_gated_delta_amd as kda
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(x):
    return {n: (None if getattr(x, n) is None else getattr(x, n).to(DEV))
            for n in ("q", "k", "v", "raw_gate", "raw_beta", "A_log", "dt_bias", "initial_state", "cu_seqlens")}


@pytest.mark.parametrize("lengths,T", [(None, 200), ([130, 0, 64, 77], None), (None, 8192)])
def test_forward_replays_match_eager_calls(lengths, T):
    """T = 8192 with 3 heads runs the recurrence on 4 shards per sequence (shard map,
    R and P passes, fold, forward): every launch of that path is captured too."""
    T = sum(lengths) if lengths is not None else T
    xs = [W.random_inputs(f"graph_{i}", 500 + i, 1, T, 3, lengths=lengths) for i in range(3)]
    x0 = xs[0]
    st = dev(x0)  # the captured (static) input buffers
    out = torch.empty_like(st["v"])
    fin = torch.empty(x0.N, x0.H, x0.K, x0.V, device=DEV)
    ws = torch.empty(kda.kda_workspace_size(x0.B * x0.T, x0.H, x0.N), dtype=torch.uint8, device=DEV)

    def call(t, o, f, w):
        kda.kda_fwd(t["q"], t["k"], t["v"], t["raw_gate"], t["raw_beta"], x0.scale, o, w, t["A_log"],
                    t["dt_bias"], x0.lower_bound, t["initial_state"], f, t["cu_seqlens"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        call(st, out, fin, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print(f"capture kda_fwd T={T} lengths={lengths}", flush=True)
    with torch.cuda.graph(g):
        call(st, out, fin, ws)
    torch.cuda.synchronize()

    for i, x in enumerate(xs + xs[:1]):
        t = dev(x)
        for n in ("q", "k", "v", "raw_gate", "raw_beta", "A_log", "dt_bias", "initial_state"):
            st[n].copy_(t[n])
        print(f"replay {i}", flush=True)
        g.replay()
        # eager reference on separate buffers, launched between replays
        o_e = torch.empty_like(out)
        f_e = torch.empty_like(fin)
        w_e = torch.empty_like(ws)
        call(t, o_e, f_e, w_e)
        torch.cuda.synchronize()
        assert torch.equal(out, o_e) and torch.equal(fin, f_e), i


def test_decode_replays_advance_the_state_like_eager_steps():
    """A captured decode step updates its state in place on every replay."""
    B, H, steps = 4, 3, 5
    toks = [W.random_inputs(f"graph_dec_{i}", 600 + i, B, 1, H) for i in range(steps)]
    x0 = toks[0]
    st = dev(x0)
    state_g = st["initial_state"].clone()
    state_e = st["initial_state"].clone()
    out = torch.empty_like(st["v"])

    def step(t, o, s):
        kda.kda_decode(t["q"], t["k"], t["v"], t["raw_gate"], t["raw_beta"], x0.scale, o, t["A_log"],
                       t["dt_bias"], x0.lower_bound, s, s)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    scratch = state_g.clone()
    with torch.cuda.stream(side):
        step(st, out, scratch)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print(f"capture kda_decode B={B} H={H}", flush=True)
    with torch.cuda.graph(g):
        step(st, out, state_g)
    torch.cuda.synchronize()

    for i, x in enumerate(toks):
        t = dev(x)
        for n in ("q", "k", "v", "raw_gate", "raw_beta", "A_log", "dt_bias"):
            st[n].copy_(t[n])
        print(f"decode replay {i}", flush=True)
        g.replay()
        o_e = torch.empty_like(out)
        step(t, o_e, state_e)
        torch.cuda.synchronize()
        assert torch.equal(out, o_e), i
        assert torch.equal(state_g, state_e), i
    assert np.isfinite(state_g.cpu().numpy()).all()


def test_single_launch_forward_replays_match_eager_calls():
    """kda_fwd_ex with FLAG_SINGLE_LAUNCH captured: the ring-reset kernel (not a memset)
    and the persistent producer/chain launch replay on the captured workspace; every
    replay equals an eager call of the two-launch schedule bit for bit, and leaves the
    fault word clear."""
    xs = [W.random_inputs(f"graph_single_{i}", 700 + i, 1, 1000, 16) for i in range(3)]
    x0 = xs[0]
    st = dev(x0)
    out = torch.empty_like(st["v"])
    fin = torch.empty(x0.N, x0.H, x0.K, x0.V, device=DEV)
    ws = torch.empty(kda.kda_workspace_size(x0.B * x0.T, x0.H, x0.N), dtype=torch.uint8, device=DEV)

    def call(t, o, f, w, flags):
        kda.kda_fwd_ex(t["q"], t["k"], t["v"], t["raw_gate"], t["raw_beta"], x0.scale, o, w, t["A_log"],
                       t["dt_bias"], x0.lower_bound, t["initial_state"], f, t["cu_seqlens"], flags=flags)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(st, out, fin, ws, kda.FLAG_SINGLE_LAUNCH)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("capture kda_fwd_ex FLAG_SINGLE_LAUNCH T=1000 H=16", flush=True)
    with torch.cuda.graph(g):
        call(st, out, fin, ws, kda.FLAG_SINGLE_LAUNCH)
    torch.cuda.synchronize()

    for i, x in enumerate(xs + xs[:1]):
        t = dev(x)
        for n in ("q", "k", "v", "raw_gate", "raw_beta", "A_log", "dt_bias", "initial_state"):
            st[n].copy_(t[n])
        print(f"single-launch replay {i}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        assert kda.kda_workspace_faults(ws) == 0, i
        o_e = torch.empty_like(out)
        f_e = torch.empty_like(fin)
        w_e = torch.empty_like(ws)
        call(t, o_e, f_e, w_e, 0)
        torch.cuda.synchronize()
        assert torch.equal(out, o_e) and torch.equal(fin, f_e), i
