"""Pins of the gradient oracle (CPU only).

  * its forward graph equals the C oracle's recurrence on the same inputs;
  * its autograd gradients equal central finite differences of that forward
    along random directions in every input (q, k, v, raw_gate, raw_beta,
    A_log, dt_bias, initial state), with and without a final-state cotangent;
  * the chunked second form of the backward (oracle/chunked.py) equals it.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import oracle_fwd
from oracle.grad import BETA_GIVEN, GATE_GIVEN, NO_QK_NORM, STATE_VK, fwd_torch, oracle_bwd

NAMES = ("q", "k", "v", "raw_gate", "raw_beta", "A_log", "dt_bias", "initial_state")


def f64(x):
    return x.detach().to(torch.float64)


def test_forward_graph_equals_the_c_oracle():
    x = W.random_inputs("grad", 111, 2, 37, 3, K=16, V=8, init_std=0.5)
    out, fin = fwd_torch(f64(x.q), f64(x.k), f64(x.v), f64(x.raw_gate), f64(x.raw_beta), x.scale, f64(x.A_log),
                         f64(x.dt_bias), x.lower_bound, f64(x.initial_state))
    ro, rf = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                        x.initial_state)
    assert np.abs(out.numpy() - ro).max() <= 1e-12
    assert np.abs(fin.numpy() - rf).max() <= 1e-12


@pytest.mark.parametrize("with_final", [True, False])
def test_gradients_match_central_differences(with_final):
    x = W.random_inputs("grad", 112, 1, 23, 2, K=8, V=8, init_std=0.5)
    g = torch.Generator().manual_seed(3)
    d_out = torch.randn(1, 23, 2, 8, generator=g, dtype=torch.float64)
    d_fin = torch.randn(1, 2, 8, 8, generator=g, dtype=torch.float64) if with_final else None
    grads = oracle_bwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                       d_out, d_fin, x.initial_state)
    base = {n: f64(getattr(x, n)) for n in NAMES}

    def loss(p):
        out, fin = fwd_torch(p["q"], p["k"], p["v"], p["raw_gate"], p["raw_beta"], x.scale, p["A_log"],
                             p["dt_bias"], x.lower_bound, p["initial_state"])
        val = (out * d_out.reshape(out.shape)).sum()
        return float(val + ((fin * d_fin).sum() if d_fin is not None else 0.0))

    key = {"q": "dq", "k": "dk", "v": "dv", "raw_gate": "d_raw_gate", "raw_beta": "d_raw_beta",
           "A_log": "dA_log", "dt_bias": "d_dt_bias", "initial_state": "d_initial_state"}
    h = 1e-5
    for n in NAMES:
        for trial in range(2):
            d = torch.randn(base[n].shape, generator=g, dtype=torch.float64)
            plus = dict(base); plus[n] = base[n] + h * d
            minus = dict(base); minus[n] = base[n] - h * d
            fd = (loss(plus) - loss(minus)) / (2 * h)
            an = float((torch.from_numpy(np.asarray(grads[key[n]])).reshape(d.shape) * d).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (n, fd, an)


@pytest.mark.parametrize("case", ["tail", "varlen", "no_init"])
def test_chunked_backward_equals_autograd(case):
    from oracle.chunked import chunked_bwd
    if case == "tail":
        x = W.random_inputs("grad", 113, 2, 150, 2, K=16, V=8, init_std=0.5)
    elif case == "varlen":
        x = W.random_inputs("grad", 114, 1, 170, 2, K=16, V=8, lengths=[1, 64, 105], init_std=0.5)
    else:
        x = W.random_inputs("grad", 115, 1, 70, 1, K=16, V=8, init_std=None)
    g = torch.Generator().manual_seed(7)
    d_out = torch.randn(x.B, x.T, x.H, x.V, generator=g, dtype=torch.float64)
    d_fin = torch.randn(x.N, x.H, x.K, x.V, generator=g, dtype=torch.float64)
    args = (x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound, d_out, d_fin,
            x.initial_state, x.cu_seqlens)
    a = oracle_bwd(*args)
    b = chunked_bwd(*args)
    for n in a:
        if a[n] is None:
            assert b[n] is None
            continue
        ref = np.asarray(a[n])
        assert np.abs(ref - np.asarray(b[n])).max() <= 1e-11 * max(1.0, np.abs(ref).max()), n


def variant_inputs(seed, T, H, K, V, flags):
    """Inputs in each variant's documented range (the same recipe as the forward variant pins)."""
    x = W.random_inputs("grad_variant", seed, 1, T, H, K=K, V=V, init_std=0.5)
    g = torch.Generator().manual_seed(seed + 500)
    if flags & GATE_GIVEN:
        x.raw_gate = (x.lower_bound * torch.sigmoid(torch.randn(x.raw_gate.shape, generator=g))).to(torch.bfloat16)
    if flags & BETA_GIVEN:
        x.raw_beta = torch.sigmoid(torch.randn(x.raw_beta.shape, generator=g)).to(torch.bfloat16)
    if flags & NO_QK_NORM:
        for name in ("q", "k"):
            t = getattr(x, name).float()
            setattr(x, name, (t / t.norm(dim=-1, keepdim=True)).to(torch.bfloat16))
    return x


@pytest.mark.parametrize("flags", [GATE_GIVEN, BETA_GIVEN, NO_QK_NORM, STATE_VK,
                                   GATE_GIVEN | BETA_GIVEN | NO_QK_NORM | STATE_VK])
def test_variant_forward_graph_and_gradients(flags):
    """Under each variant flag the forward graph equals the C oracle's, and its gradients equal
    central differences (the clamp of a given gate is never active at these inputs)."""
    x = variant_inputs(120 + flags, 21, 2, 8, 8, flags)
    ro, rf = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                        x.initial_state, flags=flags)
    out, fin = fwd_torch(f64(x.q), f64(x.k), f64(x.v), f64(x.raw_gate), f64(x.raw_beta), x.scale, f64(x.A_log),
                         f64(x.dt_bias), x.lower_bound, f64(x.initial_state), flags=flags)
    assert np.abs(out.numpy() - ro).max() <= 1e-12
    assert np.abs(fin.numpy() - rf).max() <= 1e-12
    g = torch.Generator().manual_seed(5)
    d_out = torch.randn(1, 21, 2, 8, generator=g, dtype=torch.float64)
    d_fin = torch.randn(1, 2, 8, 8, generator=g, dtype=torch.float64)
    grads = oracle_bwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                       d_out, d_fin, x.initial_state, flags=flags)
    base = {n: f64(getattr(x, n)) for n in NAMES}

    def loss(pp):
        o, f = fwd_torch(pp["q"], pp["k"], pp["v"], pp["raw_gate"], pp["raw_beta"], x.scale, pp["A_log"],
                         pp["dt_bias"], x.lower_bound, pp["initial_state"], flags=flags)
        return float((o * d_out.reshape(o.shape)).sum() + (f * d_fin).sum())

    key = {"q": "dq", "k": "dk", "v": "dv", "raw_gate": "d_raw_gate", "raw_beta": "d_raw_beta",
           "A_log": "dA_log", "dt_bias": "d_dt_bias", "initial_state": "d_initial_state"}
    h = 1e-6
    for n in NAMES:
        d = torch.randn(base[n].shape, generator=g, dtype=torch.float64)
        plus = dict(base); plus[n] = base[n] + h * d
        minus = dict(base); minus[n] = base[n] - h * d
        fd = (loss(plus) - loss(minus)) / (2 * h)
        an = float((torch.from_numpy(np.asarray(grads[key[n]])).reshape(d.shape) * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (flags, n, fd, an)
    if flags & GATE_GIVEN:
        assert not np.any(grads["dA_log"]) and not np.any(grads["d_dt_bias"])
