"""The workspace fault word (kda_workspace_faults): contract violations that the
kernels detect on the device are recorded there, through the C ABI.

  * a clean call leaves the word at zero;
  * KDA_FLAG_GATE_GIVEN with one decay outside [lower_bound, 0] sets
    FAULT_GATE_RANGE (a value at either end of the range does not);
  * KDA_FLAG_NO_QK_NORM with one key row of norm 2 sets FAULT_QK_NORM;
  * the next call on the same workspace starts from a clear word.
"""

import pytest
import torch

import chunked_gated_delta_amd as kda
import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def inputs(seed):
    x = W.random_inputs("faults", seed, 1, 200, 2)
    g = torch.Generator().manual_seed(seed)
    x.raw_gate = (x.lower_bound * torch.sigmoid(torch.randn(x.raw_gate.shape, generator=g))).to(torch.bfloat16)
    q, k = x.q.float(), x.k.float()
    x.q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    x.k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    return x


def run(x, flags, ws):
    d = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    out = torch.empty_like(d(x.v))
    fin = torch.empty(x.N, x.H, x.K, x.V, device=DEV)
    kda.kda_fwd_ex(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, out, ws, d(x.A_log),
                   d(x.dt_bias), x.lower_bound, d(x.initial_state), fin, d(x.cu_seqlens), flags=flags)
    return kda.kda_workspace_faults(ws)


def test_fault_word_records_contract_violations():
    x = inputs(61)
    ws = torch.empty(kda.kda_workspace_size(x.T, x.H, 1), dtype=torch.uint8, device=DEV)
    ws.fill_(0xFF)  # the call must clear the word itself
    G, N = kda.FLAG_GATE_GIVEN, kda.FLAG_NO_QK_NORM
    assert run(x, 0, ws) == 0
    assert run(x, G | N, ws) == 0
    edge = x.raw_gate.clone()
    edge[0, 3, 1, 5] = x.lower_bound
    edge[0, 4, 0, 9] = 0.0
    y = inputs(61)
    y.raw_gate = edge
    assert run(y, G, ws) == 0
    for bad in (x.lower_bound - 0.5, 0.25, float("nan")):
        g = x.raw_gate.clone()
        g[0, 150, 1, 77] = bad
        y.raw_gate = g
        print(f"given gate {bad}: faults", flush=True)
        assert run(y, G, ws) == kda.FAULT_GATE_RANGE
    assert run(x, G, ws) == 0  # cleared again by the next call
    k = x.k.clone()
    k[0, 66, 0] = 2.0 * k[0, 66, 0].float().to(torch.bfloat16)
    y = inputs(61)
    y.k = k
    assert run(y, N, ws) == kda.FAULT_QK_NORM
    assert run(y, 0, ws) == 0  # with the in-kernel norm the same row is fine
