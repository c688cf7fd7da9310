"""Seeded sweep of mixed call shapes through kda_bwd against the fp64 gradient oracle.

The targeted backward tests vary one axis at a time; each case here draws a
combination from its own seeded generator: batch or packed (varlen, with an
empty sequence in some packs) layout, ragged lengths, 1-4 heads, head dims 64
or 128 for K and V independently, with or without an initial state and a
final-state gradient, A_log zeros or U(0, ln 16), lower_bound in [-5, 0].
The reference is the chunked fp64 reverse-mode form (oracle/chunked.py,
pinned to the autograd token recurrence), and the bars are those of the
other backward tests: relative L2 <= 1e-2 and max-abs <= 2e-2 of the
reference's largest magnitude per gradient, all values finite.
"""

import numpy as np
import pytest
import torch

import workloads as W
from test_gpu_bwd import compare, cotangents, gpu_bwd, oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(i):
    r = np.random.default_rng(3000 + i)
    K = int(r.choice([64, 128]))
    V = int(r.choice([64, 128]))
    H = int(r.integers(1, 5))
    lb = float(-5.0 * r.random()) if i % 3 else -5.0
    a_log = "uniform_ln16" if r.random() < 0.5 else "zeros"
    init = 0.1 if r.random() < 0.6 else None
    with_final = bool(r.random() < 0.7)
    if r.random() < 0.5:
        n = int(r.integers(2, 6))
        lengths = [int(x) for x in r.integers(0, 300, size=n)]
        if i % 2 == 0:
            lengths[1] = 0  # an empty sequence inside the pack
        if sum(lengths) == 0:
            lengths[0] = 1
        B, T = 1, sum(lengths)
    else:
        lengths = None
        B, T = int(r.integers(1, 3)), int(r.integers(1, 400))
    return dict(B=B, T=T, H=H, K=K, V=V, lengths=lengths, lb=lb, a_log=a_log, init=init, with_final=with_final)


@pytest.mark.parametrize("i", range(10))
def test_bwd_random_shape(i):
    c = _case(i)
    print(f"case {i}: {c}", flush=True)
    x = W.random_inputs(f"bwd_sweep{i}", 4000 + i, c["B"], c["T"], c["H"], K=c["K"], V=c["V"], lengths=c["lengths"],
                        a_log=c["a_log"], init_std=c["init"], lower_bound=c["lb"])
    d_out, d_fin = cotangents(x, 5000 + i, with_final=c["with_final"])
    got = gpu_bwd(x, d_out, d_fin, with_dinit=c["init"] is not None)
    compare(got, oracle(x, d_out, d_fin, chunked=True))
