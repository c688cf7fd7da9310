"""Pins of the oracle's per-shard affine map and shard fold (CPU only).

The per-token update S -> (I - b k^ k^T) Diag(exp(g)) S + b k^ v^T is affine in
the state, so a shard maps its entering state S to P S + R.  The oracle builds
R as the final state from S = 0 and P as the final state of the v = 0
recurrence from S = I.  These tests check that construction against facts
that do not reuse it:
  * P for one and two tokens equals the explicit product of the per-token
    matrices, built here with numpy from the gate and norm definitions;
  * superposition: final(v, S) = R + final(0, S), and linearity
    final(0, S) = P S, for a random S;
  * splitting a sequence into shards at ragged points, folding the maps and
    rerunning each shard from its folded entering state reproduces the
    unsplit run's outputs and final state.
"""

import math

import numpy as np
import torch

import workloads as W
from oracle import metrics, oracle_fwd, oracle_shard_affine, oracle_shard_fold

EPS = 1e-6


def sig(x):
    return 1.0 / (1.0 + math.exp(-x))


def token_matrix(x, t, h):
    """(I - b k^ k^T) Diag(exp(g)) of token t, head h, from the definitions."""
    k = x.k[0, t, h].double().numpy()
    kh = k / math.sqrt(float(k @ k) + EPS)
    b = sig(float(x.raw_beta[0, t, h].float()))
    a = math.exp(float(x.A_log[h]))
    g = np.array([x.lower_bound * sig(a * (float(x.raw_gate[0, t, h, c].float()) + float(x.dt_bias[h, c])))
                  for c in range(x.K)])
    return (np.eye(x.K) - b * np.outer(kh, kh)) @ np.diag(np.exp(g))


def test_affine_map_one_and_two_tokens_match_explicit_products():
    x = W.random_inputs("kcp2", 31, 1, 2, 2, K=16, V=16)
    for T in (1, 2):
        y = W.random_inputs("kcp2", 31, 1, 2, 2, K=16, V=16)
        y.q, y.k, y.v, y.raw_gate, y.raw_beta = (t[:, :T].contiguous() for t in (x.q, x.k, x.v, x.raw_gate,
                                                                                 x.raw_beta))
        P, R = oracle_shard_affine(y.q, y.k, y.v, y.raw_gate, y.raw_beta, y.A_log, y.dt_bias, y.lower_bound)
        for h in range(2):
            M = np.eye(16)
            for t in range(T):
                M = token_matrix(y, t, h) @ M
            assert np.abs(P[0, h] - M).max() <= 1e-13


def test_superposition_and_linearity():
    x = W.random_inputs("kcp", 32, 1, 150, 2, K=32, V=32)
    S0 = torch.randn(1, 2, 32, 32, generator=torch.Generator().manual_seed(5)) * 0.3
    P, R = oracle_shard_affine(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.A_log, x.dt_bias, x.lower_bound)
    _, full = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                         x.lower_bound, S0)
    _, hom = oracle_fwd(x.q, x.k, torch.zeros_like(x.v), x.raw_gate, x.raw_beta, x.scale, x.A_log,
                        x.dt_bias, x.lower_bound, S0)
    S = S0.double().numpy()
    assert np.abs(full - (R + hom)).max() <= 1e-12
    assert np.abs(hom - np.matmul(P, S)).max() <= 1e-12


def test_split_fold_rerun_equals_unsplit():
    x = W.random_inputs("kcp", 33, 1, 700, 3, K=32, V=32, init_std=0.2)
    cuts = [0, 131, 320, 321, 600, 700]  # ragged, one single-token shard
    cu = np.array(cuts, dtype=np.int32)
    P, R = oracle_shard_affine(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.A_log, x.dt_bias, x.lower_bound,
                               cu_seqlens=cu)
    starts, fin = oracle_shard_fold(P, R, x.initial_state[0].double().numpy())
    out_ref, fin_ref = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                                  x.lower_bound, x.initial_state)
    assert np.abs(fin - fin_ref[0]).max() <= 1e-11
    out2, fin2 = oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                            x.lower_bound, starts.astype(np.float32), cu_seqlens=cu)
    # the rerun starts from fp32-rounded entering states: agreement to fp32 level
    assert metrics(out2, out_ref)["rel_l2"] <= 1e-6
    assert metrics(fin2[-1], fin_ref[0])["rel_l2"] <= 1e-6
