"""Head dims other than 128 through kda_fwd / kda_fwd_ex (K and V each 64 or 128)
against the fp64 oracle, with the whole-tensor bars of the other parity tests:
out relative L2 <= 1e-2 and max-abs <= 3e-2, final_state relative L2 <= 1e-3.

Shapes follow the C1 (T = 200, H = 2, one sequence) and C2 (B = 2, T = 4096,
H = 12, initial states) workloads with K = V = 64, plus mixed head dims,
ragged and packed sequences, the state variants and an in-place update.
"""

import numpy as np
import pytest
import torch

import chunked_gated_delta_amd as kda
import workloads as W
from gpu_run import run_gpu
from oracle import metrics, oracle_fwd

pytestmark = pytest.mark.gpu
OUT_REL, OUT_ABS, FIN_REL = 1e-2, 3e-2, 1e-3
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def oracle(x, heads=None, init=True, flags=0):
    st = x.initial_state if init else None
    return oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound, st,
                      x.cu_seqlens, heads=heads, flags=flags)


def check(o, f, ro, rf, label):
    mo = metrics(o, ro)
    msg = f"{label}: out rel_l2={mo['rel_l2']:.3e} max_abs={mo['max_abs']:.3e}"
    assert mo["finite"], label
    assert mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS, mo
    if f is not None:
        mf = metrics(f, rf)
        msg += f" final rel_l2={mf['rel_l2']:.3e}"
        assert mf["finite"] and mf["rel_l2"] <= FIN_REL, mf
    print(msg, flush=True)


def test_c1_shape_head_dim_64():
    x = W.random_inputs("c1_k64", 0, 1, 200, 2, K=64, V=64, a_log="zeros", dt_bias_std=0.0, init_std=None)
    assert kda.kda_is_supported(64, 64, x.lower_bound)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)


def test_c2_shape_head_dim_64():
    x = W.random_inputs("c2_k64", 1, 2, 4096, 12, K=64, V=64)
    heads = [0, 5, 11]
    o, f = run_gpu(x)
    ro, rf = oracle(x, heads=heads)
    check(o[:, heads], f[:, heads], ro, rf, x.name)


@pytest.mark.parametrize("K,V", [(64, 128), (128, 64), (64, 64)])
def test_mixed_head_dims_with_states(K, V):
    x = W.random_inputs(f"mixed_{K}x{V}", 40 + K + V, 1, 1000, 4, K=K, V=V)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)


def test_packed_sequences_head_dim_64():
    lengths = [1, 63, 64, 65, 300, 0, 129]
    x = W.random_inputs("varlen_k64", 41, 1, sum(lengths), 3, K=64, V=64, lengths=lengths)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)


def test_in_place_state_head_dim_64():
    x = W.random_inputs("inplace_k64", 42, 1, 777, 4, K=64, V=64)
    o, f = run_gpu(x, in_place=True)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)


@pytest.mark.parametrize("flags", [kda.FLAG_GATE_GIVEN, kda.FLAG_STATE_VK,
                                   kda.FLAG_GATE_GIVEN | kda.FLAG_BETA_GIVEN | kda.FLAG_NO_QK_NORM])
def test_variants_head_dim_64(flags):
    from test_oracle_variant_pins import variant_inputs
    x = variant_inputs(43 + flags, 500, 3, 64, 64, flags, init_std=0.1)
    d = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    init = d(x.initial_state)
    if flags & kda.FLAG_STATE_VK:
        init = init.transpose(-1, -2).contiguous()
    fin = torch.full_like(init, float("nan"))
    out = torch.full_like(d(x.v), float("nan"))
    ws = torch.empty(kda.kda_workspace_size(x.B * x.T, x.H, x.N), dtype=torch.uint8, device=DEV)
    al, dt = (None, None) if flags & kda.FLAG_GATE_GIVEN else (d(x.A_log), d(x.dt_bias))
    kda.kda_fwd_ex(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, out, ws, al, dt, x.lower_bound,
                   init, fin, d(x.cu_seqlens), flags=flags)
    assert kda.kda_workspace_faults(ws) == 0
    o = out.double().cpu().numpy().reshape(x.B * x.T, x.H, x.V)
    f = fin.double().cpu().numpy()
    init_o = x.initial_state
    if flags & kda.FLAG_STATE_VK:
        init_o = init_o.transpose(-1, -2).contiguous()
    ro, rf = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound, init_o,
                        x.cu_seqlens, flags=flags)
    check(o, f, ro, rf, f"variant flags={flags}")


def test_near_collinear_head_dim_64():
    """The near-collinear stress (one key repeated, beta ~ 1, decay ~ 1) at K = V = 64."""
    x = W.near_collinear(4, T=8192, D=64)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name + "_k64")


def test_other_entry_points_reject_head_dim_64():
    x = W.random_inputs("reject_k64", 44, 1, 64, 2, K=64, V=64)
    d = lambda t: t.to(DEV)  # noqa: E731
    P = torch.empty(1, 2, 64, 64, device=DEV)
    R = torch.empty(1, 2, 64, 64, device=DEV)
    ws = torch.empty(kda.kda_workspace_size(64, 2, 1), dtype=torch.uint8, device=DEV)
    with pytest.raises(kda.KdaError) as e:
        kda.kda_shard_affine(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), ws, d(x.A_log), d(x.dt_bias),
                             x.lower_bound, P, R)
    assert e.value.status == 2  # KDA_ERR_UNSUPPORTED
