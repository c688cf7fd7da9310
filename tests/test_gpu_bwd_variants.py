"""Parity of kda_bwd_ex (the gradients of the kda_fwd_ex variants) against the fp64
autograd oracle under the same flags (oracle/grad.py).  Inputs follow each variant's
documented range (the forward variant tests' recipe).  Tolerances as in test_gpu_bwd.py:
per gradient rel-L2 <= 1e-2 and max error <= 2e-2 of the largest reference magnitude."""

import numpy as np
import pytest
import torch

import chunked_gated_delta_amd as kda
from oracle.grad import oracle_bwd
from test_gpu_bwd import DEV, compare, d
from test_oracle_grad_pins import variant_inputs

pytestmark = pytest.mark.gpu

F = kda


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(flags, seed, T=150, H=2, with_params=True, K=128, V=128):
    x = variant_inputs(seed, T, H, K, V, flags)
    st = (1, H, V, K) if flags & F.FLAG_STATE_VK else (1, H, K, V)
    if x.initial_state.shape[1:] != st[1:]:  # the transposed layout of a non-square state
        x.initial_state = x.initial_state.transpose(-1, -2).contiguous()
    g = torch.Generator().manual_seed(seed + 7)
    d_out = torch.randn(1, T, H, V, generator=g).to(torch.bfloat16)
    d_fin = torch.randn(*st, generator=g)
    bf = lambda *s: torch.full(s, float("nan"), dtype=torch.bfloat16, device=DEV)  # noqa: E731
    dq, dk, dg, dv, db = bf(1, T, H, K), bf(1, T, H, K), bf(1, T, H, K), bf(1, T, H, V), bf(1, T, H)
    dinit = torch.full(st, float("nan"), device=DEV)
    gate_given = bool(flags & F.FLAG_GATE_GIVEN)
    dA = torch.full((H,), float("nan"), device=DEV) if with_params else None
    ddt = torch.full((H, K), float("nan"), device=DEV) if with_params else None
    al = d(x.A_log) if with_params or not gate_given else None
    dtb = d(x.dt_bias) if with_params or not gate_given else None
    ws = torch.empty(kda.kda_bwd_workspace_size(T, H, 1), dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)  # NaN bytes wherever a kernel reads what nothing wrote
    print(f"kda_bwd_ex flags={flags} T={T} H={H} K={K} V={V} params={with_params}", flush=True)
    kda.kda_bwd_ex(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, d(d_out), dq, dk, dv, dg, db,
                   dA, ddt, ws, al, dtb, x.lower_bound, initial_state=d(x.initial_state), d_final=d(d_fin),
                   d_initial_state=dinit, flags=flags)
    torch.cuda.synchronize()
    f = lambda t, *s: t.double().cpu().numpy().reshape(*s)  # noqa: E731
    got = {"dq": f(dq, T, H, K), "dk": f(dk, T, H, K), "dv": f(dv, T, H, V), "d_raw_gate": f(dg, T, H, K),
           "d_raw_beta": f(db, T, H), "d_initial_state": f(dinit, *st),
           "dA_log": None if dA is None else f(dA, H), "d_dt_bias": None if ddt is None else f(ddt, H, K)}
    ref = oracle_bwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                     d_out.double(), d_fin.double(), x.initial_state, flags=flags)
    return got, ref


@pytest.mark.parametrize("flags", [F.FLAG_BETA_GIVEN, F.FLAG_NO_QK_NORM, F.FLAG_STATE_VK])
def test_bwd_single_flag(flags):
    got, ref = run(flags, 300 + flags)
    compare(got, ref)


def test_bwd_gate_given_without_parameters():
    """With the decay given, A_log, dt_bias and their gradients may be absent."""
    got, ref = run(F.FLAG_GATE_GIVEN, 311, with_params=False)
    compare(got, ref, names=("dq", "dk", "dv", "d_raw_gate", "d_raw_beta", "d_initial_state"))


def test_bwd_gate_given_zero_fills_parameter_gradients():
    got, ref = run(F.FLAG_GATE_GIVEN, 312)
    compare(got, ref, names=("dq", "dk", "dv", "d_raw_gate", "d_raw_beta", "d_initial_state"))
    np.testing.assert_array_equal(got["dA_log"], 0.0)
    np.testing.assert_array_equal(got["d_dt_bias"], 0.0)


def test_bwd_all_flags():
    flags = F.FLAG_GATE_GIVEN | F.FLAG_BETA_GIVEN | F.FLAG_NO_QK_NORM | F.FLAG_STATE_VK
    got, ref = run(flags, 313, T=200, H=3)
    compare(got, ref, names=("dq", "dk", "dv", "d_raw_gate", "d_raw_beta", "d_initial_state"))


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64)])
def test_bwd_head_dims(K, V):
    """Head dims 64: the kernels keep their 128-channel layouts with the missing channels and
    columns held at zero (the workspace is filled with NaN bytes first, so a read of anything
    the call did not write shows up)."""
    got, ref = run(0, 320 + K + V // 2, T=200, H=3, K=K, V=V)
    compare(got, ref)


@pytest.mark.parametrize("K,V", [(64, 64), (128, 64)])
def test_bwd_all_flags_head_dims(K, V):
    flags = F.FLAG_GATE_GIVEN | F.FLAG_BETA_GIVEN | F.FLAG_NO_QK_NORM | F.FLAG_STATE_VK
    got, ref = run(flags, 330 + K + V // 2, T=130, H=2, K=K, V=V)
    compare(got, ref, names=("dq", "dk", "dv", "d_raw_gate", "d_raw_beta", "d_initial_state"))
