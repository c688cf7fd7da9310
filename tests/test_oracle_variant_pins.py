"""Pins of the oracle's variant flags (CPU only): the chunk_kda in-kernel
switches named on the instagit FlashKDA page ("Usage Examples").

  * the 40-digit decimal brute force (its own implementation of each switch)
    agrees with the fp64 recurrence under every flag and all of them at once;
  * the transposed state layout is the same computation with the states
    stored [N, H, V, K]: outputs equal and states transposed, exactly;
  * a given gate is a natural-log decay: the decay factor exp(g) of a given g
    equals the in-kernel gate's once g holds that gate's value, and a value
    outside [lower_bound, 0] (no such gate maps there) is rejected by every
    oracle form.
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
    # with the flag the final state comes back as [N, H, V, K] (K = 16, V = 12 here)
    assert fin_t.shape == (1, 2, 12, 16)
    assert np.array_equal(fin_t, np.swapaxes(fin, -1, -2))


def test_given_gate_equals_the_in_kernel_gate_it_stands_for():
    """A given gate is the natural-log decay g of the same recurrence.  With A_log = 0,
    dt_bias = 0 and raw_gate in {-100, 0, 100}, the in-kernel gate lower_bound *
    sigmoid(raw_gate) is, in fp64, 0 to within 2e-43 (so exp(g) == 1.0 exactly),
    exactly lower_bound / 2, and exactly lower_bound; handing over g in {0,
    lower_bound / 2, lower_bound} (exact in bf16) must give the same bits, which also
    shows that both ends of [lower_bound, 0] are accepted."""
    x = W.random_inputs("variant", 93, 1, 48, 2, K=16, V=16, init_std=0.5)
    x.A_log = torch.zeros_like(x.A_log)
    x.dt_bias = torch.zeros_like(x.dt_bias)
    pick = torch.randint(0, 3, x.raw_gate.shape, generator=torch.Generator().manual_seed(94))
    raw = torch.tensor([100.0, 0.0, -100.0])[pick].to(torch.bfloat16)
    given = torch.tensor([x.lower_bound, x.lower_bound / 2, 0.0])[pick].to(torch.bfloat16)
    assert set(given.double().unique().tolist()) == {x.lower_bound, x.lower_bound / 2, 0.0}
    a = oracle_fwd(x.q, x.k, x.v, raw, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                   x.initial_state)
    b = oracle_fwd(x.q, x.k, x.v, given, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                   x.initial_state, flags=GATE_GIVEN)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_given_gate_outside_its_range_is_rejected():
    x = variant_inputs(92, 40, 2, 16, 16, GATE_GIVEN)
    for bad in (-8.0, 0.75):
        lo = x.raw_gate.clone()
        lo[0, 7, 1, 3] = bad
        with pytest.raises(ValueError):
            oracle_fwd(x.q, x.k, x.v, lo, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                       x.initial_state, flags=GATE_GIVEN)
        with pytest.raises(ValueError):
            brute_fwd(x.q[:, :8], x.k[:, :8], x.v[:, :8], lo[:, :8], x.raw_beta[:, :8], x.scale, x.A_log,
                      x.dt_bias, x.lower_bound, x.initial_state, head=1, gate_given=True)
    # the boundary values themselves are inside the range
    ok = x.raw_gate.clone()
    ok[0, 0] = x.lower_bound
    ok[0, 1] = 0.0
    oracle_fwd(x.q, x.k, x.v, ok, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound, x.initial_state,
               flags=GATE_GIVEN)
