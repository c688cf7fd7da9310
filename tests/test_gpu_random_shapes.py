"""Seeded sweep of mixed call shapes through kda_fwd against the fp64 oracle.

Each case draws, from one seeded generator, a combination that the targeted
parity tests cover only one axis at a time: batch or packed (varlen, empty
sequences included) layout, ragged lengths, 1-12 heads, head dims 64 or 128
for K and V independently, with or without an initial state, A_log zeros or
U(0, ln 16), and lower_bound anywhere in [-5, 0].  Two further cases are long
enough, with few enough heads, that the call splits its sequences into shards.
The bars are the whole-tensor ones of the other parity tests: out relative L2
<= 1e-2 and max-abs <= 3e-2, final_state relative L2 <= 1e-3, all finite.
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


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(i):
    """Shape and recipe of sweep case i (its own generator, so cases are independent)."""
    r = np.random.default_rng(1000 + i)
    K = int(r.choice([64, 128]))
    V = int(r.choice([64, 128]))
    H = int(r.integers(1, 13))
    lb = float(-5.0 * r.random()) if i % 4 else -5.0
    a_log = "uniform_ln16" if r.random() < 0.5 else "zeros"
    init = 0.1 if r.random() < 0.6 else None
    if r.random() < 0.5:
        n = int(r.integers(1, 7))
        lengths = [int(x) for x in r.integers(0, 700, size=n)]
        if n >= 2 and i % 3 == 0:
            lengths[1] = 0  # an empty sequence inside the pack
        if sum(lengths) == 0:
            lengths[0] = 1
        return dict(B=1, T=sum(lengths), H=H, K=K, V=V, lengths=lengths, lb=lb, a_log=a_log, init=init)
    B = int(r.integers(1, 4))
    T = int(r.integers(1, 1200))
    return dict(B=B, T=T, H=H, K=K, V=V, lengths=None, lb=lb, a_log=a_log, init=init)


def _run(i, c):
    x = W.random_inputs(f"sweep{i}", 2000 + i, c["B"], c["T"], c["H"], K=c["K"], V=c["V"], lengths=c["lengths"],
                        a_log=c["a_log"], init_std=c["init"], lower_bound=c["lb"])
    label = f"case {i}: " + ", ".join(f"{k}={v}" for k, v in c.items() if k != "lengths")
    if c["lengths"] is not None:
        label += f", lengths={c['lengths']}"
    print(label, flush=True)
    assert kda.kda_is_supported(c["K"], c["V"], c["lb"])
    o, f = run_gpu(x, with_init=c["init"] is not None)
    ro, rf = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                        x.initial_state, x.cu_seqlens)
    mo, mf = metrics(o, ro), metrics(f, rf)
    print(f"  out rel_l2={mo['rel_l2']:.3e} max_abs={mo['max_abs']:.3e} final rel_l2={mf['rel_l2']:.3e}", flush=True)
    assert mo["finite"] and mf["finite"], label
    assert mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS, (label, mo)
    assert mf["rel_l2"] <= FIN_REL, (label, mf)


@pytest.mark.parametrize("i", range(16))
def test_random_shape(i):
    _run(i, _case(i))


@pytest.mark.parametrize("i,B,T,H,lengths", [(100, 1, 9000, 2, None), (101, 1, 26000, 1, [9000, 0, 17000])])
def test_random_long_sequences_on_shards(i, B, T, H, lengths):
    r = np.random.default_rng(1000 + i)
    c = dict(B=B, T=T, H=H, K=128, V=128, lengths=lengths, lb=float(-5.0 * r.random()), a_log="uniform_ln16",
             init=0.1)
    _run(i, c)
