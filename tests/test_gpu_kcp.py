"""Parity of the per-shard affine map and shard scan (through the C ABI)
against the fp64 oracle.

A long sequence is split into shards, passed as one varlen batch:
kda_shard_affine gives every shard's (P, R), kda_shard_scan folds them into
the shards' entering states, and kda_fwd over the shard batch from those
states must reproduce the unsplit sequence.  Tolerances as for the forward:
out rel-L2 <= 1e-2 and max-abs <= 3e-2, states rel-L2 <= 1e-3, all finite.
"""

import numpy as np
import pytest
import torch

import chunked_gated_delta_amd as kda
import workloads as W
from oracle import metrics, oracle_fwd, oracle_shard_affine, oracle_shard_fold

pytestmark = pytest.mark.gpu

OUT_REL, OUT_ABS, ST_REL = 1e-2, 3e-2, 1e-3
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def d(t):
    return None if t is None else t.to(DEV)


def gpu_affine(x, cu):
    n = len(cu) - 1
    P = torch.full((n, x.H, x.K, x.K), float("nan"), device=DEV)
    R = torch.full((n, x.H, x.K, x.V), float("nan"), device=DEV)
    ws = torch.empty(kda.kda_workspace_size(x.T, x.H, n), dtype=torch.uint8, device=DEV)
    kda.kda_shard_affine(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), ws, d(x.A_log),
                         d(x.dt_bias), x.lower_bound, P, R, cu_seqlens=torch.tensor(cu, dtype=torch.int32,
                                                                                     device=DEV))
    return P, R


def split_pipeline(x, cu):
    """shard maps -> scan -> per-shard forward from the scanned states."""
    n = len(cu) - 1
    cut = torch.tensor(cu, dtype=torch.int32, device=DEV)
    P, R = gpu_affine(x, cu)
    starts = torch.full((n, x.H, x.K, x.V), float("nan"), device=DEV)
    fin_scan = torch.full((x.H, x.K, x.V), float("nan"), device=DEV)
    init = None if x.initial_state is None else d(x.initial_state[0].contiguous())
    kda.kda_shard_scan(P, R, starts, initial_state=init, final_state=fin_scan)
    out = torch.full_like(d(x.v), float("nan"))
    fin = torch.full((n, x.H, x.K, x.V), float("nan"), device=DEV)
    ws = torch.empty(kda.kda_workspace_size(x.T, x.H, n), dtype=torch.uint8, device=DEV)
    kda.kda_fwd(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, out, ws, d(x.A_log),
                d(x.dt_bias), x.lower_bound, starts, fin, cut)
    torch.cuda.synchronize()
    return (out.double().cpu().numpy().reshape(x.T, x.H, x.V), fin[-1].double().cpu().numpy(),
            fin_scan.double().cpu().numpy())


def check_state(a, ref, label):
    m = metrics(a, ref)
    print(f"{label}: rel_l2={m['rel_l2']:.3e}", flush=True)
    assert m["finite"] and m["rel_l2"] <= ST_REL, m


def test_shard_maps_match_oracle():
    x = W.random_inputs("kcp-gpu", 41, 1, 4096, 4)
    cu = [0, 700, 1750, 1751, 2900, 4096]
    P, R = gpu_affine(x, cu)
    Pr, Rr = oracle_shard_affine(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.A_log, x.dt_bias, x.lower_bound,
                                 cu_seqlens=np.array(cu, dtype=np.int32))
    check_state(P.double().cpu().numpy(), Pr, "P")
    check_state(R.double().cpu().numpy(), Rr, "R")


@pytest.mark.parametrize("with_init", [True, False])
def test_split_sequence_equals_unsplit(with_init):
    x = W.random_inputs("kcp-gpu", 42, 1, 4096, 4, init_std=0.1 if with_init else None)
    cu = [0, 1000, 1064, 2100, 3333, 4096]
    o, f_last, f_scan = split_pipeline(x, cu)
    ro, rf = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                        x.lower_bound, x.initial_state)
    mo = metrics(o, ro)
    print(f"out rel_l2={mo['rel_l2']:.3e} max_abs={mo['max_abs']:.3e}", flush=True)
    assert mo["finite"] and mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS, mo
    check_state(f_last, rf[0], "final (last shard)")
    check_state(f_scan, rf[0], "final (scan)")


def test_near_collinear_split():
    x = W.c5_collinear(T=16384)
    o, f_last, f_scan = split_pipeline(x, [0, 4096, 8192, 12288, 16384])
    ro, rf = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                        x.lower_bound, None)
    mo = metrics(o, ro)
    print(f"out rel_l2={mo['rel_l2']:.3e} max_abs={mo['max_abs']:.3e}", flush=True)
    assert mo["finite"] and mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS, mo
    check_state(f_last, rf[0], "final (last shard)")
    check_state(f_scan, rf[0], "final (scan)")


@pytest.mark.parametrize("n", [1, 5])
def test_scan_matches_fp64_fold(n):
    g = torch.Generator().manual_seed(7 + n)
    H = 3
    P = torch.randn(n, H, 128, 128, generator=g) / 12.0
    R = torch.randn(n, H, 128, 128, generator=g)
    S0 = torch.randn(H, 128, 128, generator=g)
    starts = torch.full((n, H, 128, 128), float("nan"), device=DEV)
    fin = torch.full((H, 128, 128), float("nan"), device=DEV)
    kda.kda_shard_scan(d(P), d(R), starts, initial_state=d(S0), final_state=fin)
    torch.cuda.synchronize()
    rs, rf = oracle_shard_fold(P.double().numpy(), R.double().numpy(), S0.double().numpy())
    assert metrics(starts.double().cpu().numpy(), rs)["rel_l2"] <= 1e-5
    assert metrics(fin.double().cpu().numpy(), rf)["rel_l2"] <= 1e-5


def test_forward_reusing_the_shard_records_is_exact():
    """kda_fwd_ex with FLAG_REUSE_RECORDS on the workspace kda_shard_affine filled gives
    the same bits as a kda_fwd call that rebuilds the records."""
    x = W.random_inputs("kcp-reuse", 44, 1, 3000, 3)
    cu = [0, 640, 1000, 1001, 3000]
    n = len(cu) - 1
    cut = torch.tensor(cu, dtype=torch.int32, device=DEV)
    P = torch.empty(n, x.H, x.K, x.K, device=DEV)
    R = torch.empty(n, x.H, x.K, x.V, device=DEV)
    ws = torch.empty(kda.kda_workspace_size(x.T, x.H, n), dtype=torch.uint8, device=DEV)
    args = (d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta))
    al, dt = d(x.A_log), d(x.dt_bias)
    print("kda_shard_affine + scan + kda_fwd_ex(REUSE_RECORDS)", flush=True)
    kda.kda_shard_affine(*args, ws, al, dt, x.lower_bound, P, R, cu_seqlens=cut)
    starts = torch.empty(n, x.H, x.K, x.V, device=DEV)
    kda.kda_shard_scan(P, R, starts, initial_state=d(x.initial_state[0].contiguous()))
    out_r, fin_r = torch.empty_like(args[2]), torch.empty(n, x.H, x.K, x.V, device=DEV)
    kda.kda_fwd_ex(*args, x.scale, out_r, ws, al, dt, x.lower_bound, starts, fin_r, cut,
                   flags=kda.FLAG_REUSE_RECORDS)
    out_f, fin_f = torch.empty_like(out_r), torch.empty_like(fin_r)
    ws2 = torch.empty_like(ws)
    kda.kda_fwd(*args, x.scale, out_f, ws2, al, dt, x.lower_bound, starts, fin_f, cut)
    torch.cuda.synchronize()
    assert torch.equal(out_r, out_f) and torch.equal(fin_r, fin_f)
