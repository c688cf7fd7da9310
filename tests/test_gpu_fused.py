"""The single-launch schedule of one-sequence calls (kda_fwd_ex with
FLAG_SINGLE_LAUNCH, N == 1 and H >= 16): intra-chunk producers hand chunk
records through an L2 ring to the chain workgroups of each head.

It computes every product, operand split and accumulation in the order of the
two-launch schedule (records built first, recurrence after), which the same
call takes without the flag; so the two must agree bit for bit, and
both must meet the oracle's bar.  Every call must also leave the workspace's
fault word clear (no timed-out wait, no id residue split over two XCDs).
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
ALL = kda.FLAG_GATE_GIVEN | kda.FLAG_BETA_GIVEN | kda.FLAG_NO_QK_NORM | kda.FLAG_STATE_VK


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def run(x, flags, *, in_place=False, with_init=True):
    d = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    init = d(x.initial_state) if with_init else None
    if init is not None and flags & kda.FLAG_STATE_VK:
        init = init.transpose(-1, -2).contiguous()
    if in_place:
        init = init.clone()
        fin = init
    else:
        fin = torch.full((x.N, x.H, x.K, x.V), float("nan"), device=DEV)
    out = torch.full_like(d(x.v), float("nan"))
    ws = torch.empty(kda.kda_workspace_size(x.B * x.T, x.H, x.N), dtype=torch.uint8, device=DEV)
    ws.fill_(0xA5)
    al, dt = (None, None) if flags & kda.FLAG_GATE_GIVEN else (d(x.A_log), d(x.dt_bias))
    kda.kda_fwd_ex(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, out, ws, al, dt, x.lower_bound,
                   init, fin, d(x.cu_seqlens), flags=flags)
    faults = kda.kda_workspace_faults(ws)
    f = fin.double().cpu().numpy()
    if flags & kda.FLAG_STATE_VK:
        f = f.swapaxes(-1, -2)
    return out.double().cpu().numpy().reshape(x.B * x.T, x.H, x.V), f, faults


def check(x, flags=0, heads=None, **kw):
    o, f, faults = run(x, flags | kda.FLAG_SINGLE_LAUNCH, **kw)
    o2, f2, faults2 = run(x, flags, **kw)
    print(f"{x.name} flags={flags} {kw}: faults {faults}/{faults2}", flush=True)
    assert faults == 0 and faults2 == 0
    assert np.array_equal(o, o2), np.abs(o - o2).max()
    assert np.array_equal(f, f2), np.abs(f - f2).max()
    init = x.initial_state if kw.get("with_init", True) else None
    if flags & kda.FLAG_STATE_VK and init is not None:
        init = init.transpose(-1, -2).contiguous()
    ro, rf = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound, init,
                        x.cu_seqlens, heads=heads, flags=flags)
    if flags & kda.FLAG_STATE_VK:
        rf = rf.swapaxes(-1, -2)
    hs = slice(None) if heads is None else heads
    mo, mf = metrics(o[:, hs], ro), metrics(f[:, hs], rf)
    print(f"   out rel_l2={mo['rel_l2']:.3e} max_abs={mo['max_abs']:.3e} final rel_l2={mf['rel_l2']:.3e}",
          flush=True)
    assert mo["finite"] and mf["finite"]
    assert mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS and mf["rel_l2"] <= FIN_REL


@pytest.mark.parametrize("T,H", [(1, 16), (63, 16), (64, 17), (65, 24), (1000, 16), (777, 33), (4096, 96)])
def test_fused_equals_two_launch_schedule(T, H):
    """Ragged and whole last chunks, head counts that leave XCDs with 2, 3, 4 and 12 heads."""
    x = W.random_inputs(f"fused_T{T}_H{H}", 500 + T + H, 1, T, H)
    check(x, heads=[0, H // 2, H - 1] if H > 20 else None)


def test_fused_without_states_and_in_place():
    x = W.random_inputs("fused_states", 531, 1, 700, 16)
    check(x, with_init=False)
    check(x, in_place=True)


def test_fused_with_one_sequence_through_cu_seqlens():
    x = W.random_inputs("fused_cu", 532, 1, 555, 16, lengths=[555])
    check(x)


@pytest.mark.parametrize("flags", [kda.FLAG_GATE_GIVEN, kda.FLAG_STATE_VK, ALL])
def test_fused_variants(flags):
    from test_oracle_variant_pins import variant_inputs
    x = variant_inputs(533 + flags, 600, 16, 128, 128, flags, init_std=0.1)
    check(x, flags)


def test_fused_ring_wraps_many_times():
    """T = 32768 (512 chunks per head, the ring holds 8) with 40 heads (fewer chains
    would take the shard path instead): 5 heads per XCD, sampled."""
    x = W.random_inputs("fused_long", 534, 1, 32768, 40)
    check(x, heads=[0, 13, 39])
