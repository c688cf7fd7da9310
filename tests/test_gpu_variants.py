"""Parity of kda_fwd_ex's variant flags (through the C ABI) against the fp64
oracle run with the same flags.  Tolerances as for kda_fwd: out rel-L2 <= 1e-2
and max-abs <= 3e-2, final state rel-L2 <= 1e-3, all finite."""

import numpy as np
import pytest
import torch

import chunked_gated_delta_amd as kda
from oracle import metrics, oracle_fwd
from oracle.recurrence import BETA_GIVEN, GATE_GIVEN, NO_QK_NORM, STATE_VK
from test_oracle_variant_pins import variant_inputs

pytestmark = pytest.mark.gpu

OUT_REL, OUT_ABS, FIN_REL = 1e-2, 3e-2, 1e-3
DEV = "cuda:0"
ALL = GATE_GIVEN | BETA_GIVEN | NO_QK_NORM | STATE_VK


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def d(t):
    return None if t is None else t.to(DEV)


def run(x, flags, init, drop_gate_params=False):
    N = x.N
    shape = (N, x.H, x.V, x.K) if flags & STATE_VK else (N, x.H, x.K, x.V)
    out = torch.full_like(d(x.v), float("nan"))
    fin = torch.full(shape, float("nan"), device=DEV)
    ws = torch.empty(kda.kda_workspace_size(x.B * x.T, x.H, N), dtype=torch.uint8, device=DEV)
    al, dt = (None, None) if drop_gate_params else (d(x.A_log), d(x.dt_bias))
    kda.kda_fwd_ex(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, out, ws, al, dt,
                   x.lower_bound, d(init), fin, d(x.cu_seqlens), flags=flags)
    torch.cuda.synchronize()
    return out.double().cpu().numpy().reshape(x.B * x.T, x.H, x.V), fin.double().cpu().numpy()


def check(x, flags, **kw):
    init = x.initial_state
    if flags & STATE_VK and init is not None:
        init = init.transpose(-1, -2).contiguous()
    o, f = run(x, flags, init, **kw)
    ro, rf = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                        init, x.cu_seqlens, flags=flags)
    mo, mf = metrics(o, ro), metrics(f, rf)
    print(f"flags={flags}: out rel_l2={mo['rel_l2']:.3e} max_abs={mo['max_abs']:.3e} "
          f"final rel_l2={mf['rel_l2']:.3e}", flush=True)
    assert mo["finite"] and mf["finite"]
    assert mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS, mo
    assert mf["rel_l2"] <= FIN_REL, mf


@pytest.mark.parametrize("flags", [0, GATE_GIVEN, BETA_GIVEN, NO_QK_NORM, STATE_VK, ALL])
def test_variant_matches_oracle(flags):
    check(variant_inputs(101, 1000, 4, 128, 128, flags, init_std=0.1), flags)


def test_given_gate_without_gate_parameters_and_at_its_range_ends():
    """A_log and dt_bias absent; the given decays include both ends of [lower_bound, 0]
    (values outside it break the call's contract: test_gpu_faults.py)."""
    x = variant_inputs(102, 777, 3, 128, 128, GATE_GIVEN, init_std=0.1)
    x.raw_gate[0, ::5] = x.lower_bound
    x.raw_gate[0, 1::5] = 0.0
    check(x, GATE_GIVEN, drop_gate_params=True)


def test_variants_on_varlen_batch():
    x = variant_inputs(103, 3000, 2, 128, 128, ALL, init_std=0.1)
    x.cu_seqlens = torch.tensor([0, 5, 1290, 1290, 3000], dtype=torch.int32)
    x.initial_state = torch.randn(4, 2, 128, 128, generator=torch.Generator().manual_seed(9)) * 0.1
    check(x, ALL)
