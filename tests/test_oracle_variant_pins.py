"""Pins of the oracle's variant flags (CPU only): the chunk_kda in-kernel
switches named on the instagit FlashKDA page ("Usage Examples").

  * the 40-digit decimal brute force (its own implementation of each switch)
    agrees with the fp64 recurrence under every flag and all of them at once;
  * the transposed state layout is the same computation with the states
    stored [N, H, V, K]: outputs equal and states transposed, exactly;
  * a given gate outside [lower_bound, 0] acts as its clamped value.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import oracle_fwd
from oracle.brute import brute_fwd
from oracle.recurrence import BETA_GIVEN, GATE_GIVEN, NO_QK_NORM, STATE_VK


def variant_inputs(seed, T, H, K, V, flags, init_std=0.5):
    x = W.random_inputs("variant", seed, 1, T, H, K=K, V=V, init_std=init_std)
    g = torch.Generator().manual_seed(seed + 500)
    if flags & GATE_GIVEN:  # natural-log decay in (lower_bound, 0)
        x.raw_gate = (x.lower_bound * torch.sigmoid(torch.randn(x.raw_gate.shape, generator=g))).to(torch.bfloat16)
    if flags & BETA_GIVEN:  # beta in (0, 1)
        x.raw_beta = torch.sigmoid(torch.randn(x.raw_beta.shape, generator=g)).to(torch.bfloat16)
    if flags & NO_QK_NORM:  # unit-scale keys and queries, as the variant requires
        for name in ("q", "k"):
            t = getattr(x, name).float()
            setattr(x, name, (t / t.norm(dim=-1, keepdim=True)).to(torch.bfloat16))
    return x


@pytest.mark.parametrize("flags", [GATE_GIVEN, BETA_GIVEN, NO_QK_NORM, GATE_GIVEN | BETA_GIVEN | NO_QK_NORM])
def test_brute_force_under_each_flag(flags):
    x = variant_inputs(81 + flags, 6, 2, 16, 12, flags)
    out, fin = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                          x.initial_state, flags=flags)
    for h in range(2):
        ob, fb = brute_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                           x.initial_state, head=h, gate_given=bool(flags & GATE_GIVEN),
                           beta_given=bool(flags & BETA_GIVEN), no_qk_norm=bool(flags & NO_QK_NORM))
        ob = np.array([[float(a) for a in r] for r in ob])
        fb = np.array([[float(a) for a in r] for r in fb])
        assert np.abs(out[:, h] - ob).max() <= 1e-13
        assert np.abs(fin[0, h] - fb).max() <= 1e-13


def test_transposed_state_layout_is_a_pure_relayout():
    x = W.random_inputs("variant", 91, 1, 90, 2, K=16, V=12, init_std=0.5)
    out, fin = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                          x.initial_state)
    init_t = x.initial_state.transpose(-1, -2).contiguous()
    out_t, fin_t = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                              x.lower_bound, init_t, flags=STATE_VK)
    assert np.array_equal(out, out_t)
    # fin_t holds S^T in memory: viewed as [N, H, V, K]
    assert np.array_equal(fin_t.reshape(1, 2, 12, 16), np.swapaxes(fin, -1, -2))


def test_given_gate_is_clamped_to_its_range():
    x = variant_inputs(92, 40, 2, 16, 16, GATE_GIVEN)
    lo = x.raw_gate.clone()
    lo[0, ::3] = -8.0   # below lower_bound = -5
    lo[0, 1::3] = 0.75  # above 0
    clamped = lo.clone()
    clamped[0, ::3] = x.lower_bound
    clamped[0, 1::3] = 0.0
    a = oracle_fwd(x.q, x.k, x.v, lo, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound, x.initial_state,
                   flags=GATE_GIVEN)
    b = oracle_fwd(x.q, x.k, x.v, clamped, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                   x.initial_state, flags=GATE_GIVEN)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
