"""Parity of the token-by-token decode step (through the C ABI) against the
fp64 oracle recurrence.

The decode step computes in fp32, so beyond the forward's tolerances (out
rel-L2 <= 1e-2, max-abs <= 3e-2 after bf16 rounding) its states are held to
rel-L2 <= 1e-5.
"""

import numpy as np
import pytest
import torch

import chunked_gated_delta_amd as kda
import workloads as W
from oracle import metrics, oracle_fwd

pytestmark = pytest.mark.gpu

OUT_REL, OUT_ABS, ST_REL = 1e-2, 3e-2, 1e-5
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def d(t):
    return None if t is None else t.to(DEV)


def gpu_decode(x, in_place=False, init=True):
    s0 = d(x.initial_state) if init else None
    out = torch.full_like(d(x.v), float("nan"))
    if in_place:
        fin = s0
    else:
        fin = torch.full((x.B, x.H, x.K, x.V), float("nan"), device=DEV)
    kda.kda_decode(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, out, d(x.A_log),
                   d(x.dt_bias), x.lower_bound, s0, fin)
    torch.cuda.synchronize()
    return out.double().cpu().numpy().reshape(x.B * x.T, x.H, x.V), fin.double().cpu().numpy()


def check(o, f, ro, rf, label):
    mo, mf = metrics(o, ro), metrics(f, rf)
    print(f"{label}: out rel_l2={mo['rel_l2']:.3e} max_abs={mo['max_abs']:.3e} final rel_l2={mf['rel_l2']:.3e}",
          flush=True)
    assert mo["finite"] and mf["finite"]
    assert mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS, mo
    assert mf["rel_l2"] <= ST_REL, mf


def oracle(x, init=True, heads=None):
    return oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                      x.initial_state if init else None, heads=heads)


@pytest.mark.parametrize("B,T,H", [(8, 1, 4), (3, 5, 2), (1, 1, 1)])
def test_decode_matches_oracle(B, T, H):
    x = W.random_inputs("decode", 51 + T, B, T, H, init_std=0.3)
    o, f = gpu_decode(x)
    check(o, f, *oracle(x), f"B={B} T={T} H={H}")


def test_decode_in_place_and_without_initial_state():
    x = W.random_inputs("decode", 61, 4, 2, 3, init_std=0.3)
    ro, rf = oracle(x)
    o, f = gpu_decode(x, in_place=True)
    check(o, f, ro, rf, "in place")
    ro0, rf0 = oracle(x, init=False)
    o0, f0 = gpu_decode(x, init=False)
    check(o0, f0, ro0, rf0, "zero initial state")


def test_decode_zero_tokens_copies_the_state():
    x = W.random_inputs("decode", 62, 2, 0, 2, init_std=0.3)
    fin = torch.full((2, 2, 128, 128), float("nan"), device=DEV)
    out = torch.empty(2, 0, 2, 128, dtype=torch.bfloat16, device=DEV)
    kda.kda_decode(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, out, d(x.A_log),
                   d(x.dt_bias), x.lower_bound, d(x.initial_state), fin)
    torch.cuda.synchronize()
    assert torch.equal(fin.cpu(), x.initial_state)


@pytest.mark.parametrize("lb", [0.0, -1.0, -5.0])
def test_decode_gate_range_and_extremes(lb):
    x = W.random_inputs("decode", 63, 4, 3, 2, init_std=0.3, lower_bound=lb)
    x.raw_gate[0] = 30.0
    x.raw_gate[1] = -30.0
    x.raw_beta[2] = 20.0
    x.raw_beta[3] = -20.0
    o, f = gpu_decode(x)
    check(o, f, *oracle(x), f"lb={lb}")


def test_decode_continues_a_chunked_prefill():
    """kda_fwd over a 200-token prompt, then 3 decode steps from its final state,
    equals the oracle over all 203 tokens."""
    T0, T1 = 200, 3
    x = W.random_inputs("decode", 64, 1, T0 + T1, 4, init_std=0.1)
    pre = [t[:, :T0].contiguous() for t in (x.q, x.k, x.v, x.raw_gate, x.raw_beta)]
    dec = [t[:, T0:].contiguous() for t in (x.q, x.k, x.v, x.raw_gate, x.raw_beta)]
    state = d(x.initial_state.clone())
    out_p = torch.empty_like(d(pre[2]))
    ws = torch.empty(kda.kda_workspace_size(T0, x.H, 1), dtype=torch.uint8, device=DEV)
    kda.kda_fwd(*(d(t) for t in pre[:5]), x.scale, out_p, ws, d(x.A_log), d(x.dt_bias), x.lower_bound,
                state, state)
    out_d = torch.empty_like(d(dec[2]))
    kda.kda_decode(*(d(t) for t in dec[:5]), x.scale, out_d, d(x.A_log), d(x.dt_bias), x.lower_bound,
                   state, state)
    torch.cuda.synchronize()
    ro, rf = oracle(x)
    o = torch.cat([out_p, out_d], dim=1).double().cpu().numpy().reshape(T0 + T1, x.H, x.V)
    mo, mf = metrics(o, ro), metrics(state.double().cpu().numpy(), rf)
    print(f"prefill+decode: out rel_l2={mo['rel_l2']:.3e} final rel_l2={mf['rel_l2']:.3e}", flush=True)
    assert mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS, mo
    assert mf["rel_l2"] <= 1e-3, mf  # the chunked prefill's state tolerance


def test_decode_serving_shape_sampled_heads():
    x = W.random_inputs("decode", 65, 64, 1, 96, init_std=0.1)
    o, f = gpu_decode(x)
    heads = [0, 47, 95]
    ro, rf = oracle(x, heads=heads)
    check(o[:, heads], f[:, heads], ro, rf, "B=64 T=1 H=96, heads 0/47/95")


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64)])
def test_decode_other_head_dims(K, V):
    """Head dims 64 (instantiations of their own: K / 8 state rows per thread, V / 32
    column slices), in place, from a chunked prefill of the same head dims."""
    x = W.random_inputs(f"decode_{K}x{V}", 66 + K + V, 5, 3, 3, K=K, V=V, init_std=0.3)
    o, f = gpu_decode(x)
    check(o, f, *oracle(x), f"K={K} V={V}")
    o2, f2 = gpu_decode(x, in_place=True)
    assert np.array_equal(o, o2) and np.array_equal(f, f2)


def test_decode_continues_a_chunked_prefill_at_head_dim_64():
    T0, T1 = 130, 2
    x = W.random_inputs("decode64", 67, 1, T0 + T1, 3, K=64, V=64, init_std=0.1)
    pre = [t[:, :T0].contiguous() for t in (x.q, x.k, x.v, x.raw_gate, x.raw_beta)]
    dec = [t[:, T0:].contiguous() for t in (x.q, x.k, x.v, x.raw_gate, x.raw_beta)]
    state = d(x.initial_state.clone())
    out_p = torch.empty_like(d(pre[2]))
    ws = torch.empty(kda.kda_workspace_size(T0, x.H, 1), dtype=torch.uint8, device=DEV)
    kda.kda_fwd(*(d(t) for t in pre[:5]), x.scale, out_p, ws, d(x.A_log), d(x.dt_bias), x.lower_bound,
                state, state)
    out_d = torch.empty_like(d(dec[2]))
    kda.kda_decode(*(d(t) for t in dec[:5]), x.scale, out_d, d(x.A_log), d(x.dt_bias), x.lower_bound,
                   state, state)
    torch.cuda.synchronize()
    ro, rf = oracle(x)
    o = torch.cat([out_p, out_d], dim=1).double().cpu().numpy().reshape(T0 + T1, x.H, x.V)
    mo, mf = metrics(o, ro), metrics(state.double().cpu().numpy(), rf)
    print(f"prefill+decode K=V=64: out rel_l2={mo['rel_l2']:.3e} final rel_l2={mf['rel_l2']:.3e}", flush=True)
    assert mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS, mo
    assert mf["rel_l2"] <= 1e-3, mf
