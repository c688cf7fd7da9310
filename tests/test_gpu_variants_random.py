"""Seeded sweep of kda_fwd_ex variant-flag combinations on mixed shapes against the
fp64 oracle run with the same flags.

Each case draws from its own seeded generator a subset of the flags (gate given,
beta given, no q/k norm, transposed state layout), head dims 64 or 128 for K
and V independently, 1-6 heads, a ragged length, and either one sequence or a
packed batch with an empty sequence.  Inputs follow each flag's documented
range (the recipe of the variant pins).  Bars as for kda_fwd: out relative L2
<= 1e-2 and max-abs <= 3e-2, final state relative L2 <= 1e-3, all finite.
"""

import numpy as np
import pytest
import torch

from oracle.recurrence import BETA_GIVEN, GATE_GIVEN, NO_QK_NORM, STATE_VK
from test_gpu_variants import check
from test_oracle_variant_pins import variant_inputs

pytestmark = pytest.mark.gpu
FLAGS = (GATE_GIVEN, BETA_GIVEN, NO_QK_NORM, STATE_VK)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(i):
    r = np.random.default_rng(6000 + i)
    flags = 0
    for f in FLAGS:
        if r.random() < 0.5:
            flags |= f
    if flags == 0:
        flags = FLAGS[i % len(FLAGS)]
    K, V = int(r.choice([64, 128])), int(r.choice([64, 128]))
    H = int(r.integers(1, 7))
    T = int(r.integers(1, 900))
    cu = None
    if r.random() < 0.5 and T >= 3:
        a, b = sorted(int(x) for x in r.choice(np.arange(1, T), size=2, replace=False))
        cu = [0, a, a, b, T]  # the second sequence is empty
    return flags, K, V, H, T, cu


@pytest.mark.parametrize("i", range(12))
def test_variant_flags_random_shape(i):
    flags, K, V, H, T, cu = _case(i)
    print(f"case {i}: flags={flags} K={K} V={V} H={H} T={T} cu={cu}", flush=True)
    x = variant_inputs(7000 + i, T, H, K, V, flags, init_std=0.1)
    if cu is not None:
        x.cu_seqlens = torch.tensor(cu, dtype=torch.int32)
        x.initial_state = torch.randn(len(cu) - 1, H, K, V, generator=torch.Generator().manual_seed(8000 + i)) * 0.1
    check(x, flags)
