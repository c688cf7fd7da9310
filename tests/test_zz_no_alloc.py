"""kda_fwd_noalloc (through the C ABI) against kda_fwd with a caller workspace.

The no-allocation entry point runs the same kernels on a static per-GPU
scratch array, so its results must equal kda_fwd's bit for bit; both are also
held to the oracle's bar.  Two calls in a row, the second smaller than the
first (the array keeps the first call's contents, which the second must not
depend on), then a call too large for the array, which is refused on the host.
"""

import numpy as np
import pytest
import torch

import chunked_gated_delta_amd as kda
import workloads as W
from oracle import metrics, oracle_fwd

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
OUT_REL, OUT_ABS, FIN_REL = 1e-2, 3e-2, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def both(x):
    d = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    args = (d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta))
    outs = []
    for noalloc in (True, False):
        out = torch.full_like(args[2], float("nan"))
        fin = torch.full((x.N, x.H, x.K, x.V), float("nan"), device=DEV)
        if noalloc:
            kda.kda_fwd_noalloc(*args, x.scale, out, d(x.A_log), d(x.dt_bias), x.lower_bound, d(x.initial_state),
                                fin, d(x.cu_seqlens))
        else:
            ws = torch.empty(kda.kda_workspace_size(x.B * x.T, x.H, x.N), dtype=torch.uint8, device=DEV)
            kda.kda_fwd(*args, x.scale, out, ws, d(x.A_log), d(x.dt_bias), x.lower_bound, d(x.initial_state), fin,
                        d(x.cu_seqlens))
        torch.cuda.synchronize()
        outs.append((out.double().cpu().numpy().reshape(x.B * x.T, x.H, x.V), fin.double().cpu().numpy()))
    return outs


def check(x):
    (o1, f1), (o2, f2) = both(x)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2), x.name
    ro, rf = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
                        x.initial_state, x.cu_seqlens)
    mo, mf = metrics(o1, ro), metrics(f1, rf)
    print(f"{x.name}: noalloc == kda_fwd bitwise; out rel_l2={mo['rel_l2']:.3e} final rel_l2={mf['rel_l2']:.3e}",
          flush=True)
    assert mo["finite"] and mf["finite"]
    assert mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS and mf["rel_l2"] <= FIN_REL


def test_noalloc_equals_kda_fwd_then_smaller_call_then_refusal():
    check(W.c2_tp_share())          # B=2, T=4096, H=12 with initial states: about 142 MB of scratch
    x = W.random_inputs("noalloc_small", 55, 1, 200, 2, lengths=[0, 130, 70])
    check(x)                        # smaller, varlen with an empty sequence, on the same array
    big = W.random_inputs("noalloc_big", 56, 1, 64, 2)
    d = lambda t: t.to(DEV)  # noqa: E731
    out = torch.empty_like(d(big.v))
    # the layout of T=32768, H=96 (4.4 GB) does not fit: refused before any device work
    status = kda._lib.kda_fwd_noalloc(*(kda._ptr(d(t)) for t in (big.q, big.k, big.v, big.raw_gate,
                                                                  big.raw_beta)),
                                      float(big.scale), kda._ptr(out), kda._ptr(d(big.A_log)),
                                      kda._ptr(d(big.dt_bias)), float(big.lower_bound), None, None, None,
                                      1, 32768, 96, 128, 128, 1, None)
    assert status == 3  # KDA_ERR_WORKSPACE
