"""Pins of the CPU oracle to things other than itself (CPU only).

Each test checks the fp64 token recurrence (oracle/recurrence.py) against a
fact fixed by the mathematics or by the pages:
  * decimal brute force of the unrolled product form (T <= 8) and a stored
    40-digit fixture (tests/golden/brute_k128_T5.json);
  * the second CPU form (chunk algebra) at chunk sizes 16, 32 and 64 with tails;
  * closed forms: decay only (beta = 0), gated linear attention when the erase
    term vanishes (distinct one-hot keys), exact stores (alpha = 1, beta = 1,
    one-hot keys) and the near-collinear scalar recurrence (the vLLM PR test);
  * invariants: packed varlen = per-document runs, split/resume through the
    state, power-of-two rescaling of q and k, head permutation, empty
    sequences.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import metrics, oracle_fwd
from oracle.brute import brute_fwd
from oracle.chunked import chunked_fwd

HERE = os.path.dirname(os.path.abspath(__file__))
EPS = 1e-6


def run(x, **kw):
    return oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                      x.lower_bound, x.initial_state, x.cu_seqlens, **kw)


def unit(v):
    v = np.asarray(v, dtype=np.float64)
    return v / math.sqrt(float((v * v).sum()) + EPS)


# ---------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed,T,K,V,with_state", [(11, 6, 16, 12, True), (12, 8, 8, 8, True),
                                                  (13, 7, 16, 16, False)])
def test_brute_force_small(seed, T, K, V, with_state):
    x = W.random_inputs("brute", seed, 1, T, 2, K=K, V=V, init_std=0.5 if with_state else None)
    out, fin = run(x)
    for h in range(2):
        ob, fb = brute_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                           x.lower_bound, x.initial_state, head=h)
        ob = np.array([[float(a) for a in r] for r in ob])
        fb = np.array([[float(a) for a in r] for r in fb])
        assert np.abs(out[:, h] - ob).max() <= 1e-13
        assert np.abs(fin[0, h] - fb).max() <= 1e-13


def test_brute_force_head_dim_64():
    """The head dim the forward also takes besides 128 (K = V = 64), against the decimal
    product form, with a carried initial state."""
    x = W.random_inputs("brute64", 21, 1, 4, 1, K=64, V=64, init_std=0.5)
    out, fin = run(x)
    ob, fb = brute_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                       x.lower_bound, x.initial_state, head=0)
    ob = np.array([[float(a) for a in r] for r in ob])
    fb = np.array([[float(a) for a in r] for r in fb])
    assert np.abs(out[:, 0] - ob).max() <= 1e-13
    assert np.abs(fin[0, 0] - fb).max() <= 1e-13


def test_brute_force_golden_k128():
    with open(os.path.join(HERE, "golden", "brute_k128_T5.json")) as f:
        doc = json.load(f)
    s = doc["spec"]
    x = W.random_inputs(s["name"], s["seed"], s["B"], s["T"], s["H"], s["K"], s["V"],
                        init_std=None)
    out, fin = run(x)
    ob = np.array([[float(a) for a in r] for r in doc["out"]])
    assert np.abs(out[:, s["head"]] - ob).max() <= 1e-14
    for r, row in zip(doc["final_rows"], doc["final"]):
        assert np.abs(fin[0, s["head"], r] - np.array([float(a) for a in row])).max() <= 1e-14


# ---------------------------------------------------------------------------
# chunked form
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_chunked_form_matches(chunk):
    lengths = [1, 63, 64, 65, 137]
    x = W.random_inputs("chunked", 5, 1, sum(lengths), 2, lengths=lengths)
    out, fin = run(x)
    o2, f2 = chunked_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                         x.lower_bound, x.initial_state, x.cu_seqlens, chunk=chunk)
    assert np.abs(out - o2).max() <= 1e-12
    assert np.abs(fin - f2).max() <= 1e-12


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64)])
def test_chunked_form_matches_at_other_head_dims(K, V):
    lengths = [1, 63, 64, 65, 137]
    x = W.random_inputs(f"chunked_{K}x{V}", 22, 1, sum(lengths), 2, K=K, V=V, lengths=lengths)
    out, fin = run(x)
    o2, f2 = chunked_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                         x.lower_bound, x.initial_state, x.cu_seqlens, chunk=64)
    assert out.shape == (sum(lengths), 2, V) and fin.shape == (len(lengths), 2, K, V)
    assert np.abs(out - o2).max() <= 1e-12
    assert np.abs(fin - f2).max() <= 1e-12


def test_chunked_form_c1_reference_case():
    x = W.c1_ref()
    out, fin = run(x)
    o2, f2 = chunked_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                         x.lower_bound, x.initial_state, x.cu_seqlens)
    assert np.abs(out - o2).max() <= 1e-12 and np.abs(fin - f2).max() <= 1e-12


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------

def test_decay_only_beta_zero():
    """raw_beta = -inf gives beta = 0: no writes, the state only decays.

    raw_gate = dt_bias = 0 puts every gate at sigmoid(0) = 1/2, so each step
    multiplies the state by exp(lower_bound / 2) and o_t = scale * S_t^T q^_t.
    """
    T, H, K, V = 9, 2, 16, 8
    x = W.random_inputs("decay", 7, 1, T, H, K=K, V=V, init_std=1.0)
    x.raw_beta = torch.full_like(x.raw_beta, -math.inf)
    x.raw_gate = torch.zeros_like(x.raw_gate)
    x.dt_bias = torch.zeros_like(x.dt_bias)
    out, fin = run(x)
    S0 = x.initial_state.double().numpy()[0]
    a = math.exp(x.lower_bound / 2)
    qf = x.q.double().numpy()[0]
    for h in range(H):
        for t in range(T):
            St = a ** (t + 1) * S0[h]
            ref = x.scale * St.T @ unit(qf[t, h])
            assert np.abs(out[t, h] - ref).max() <= 1e-14
        assert np.abs(fin[0, h] - a ** T * S0[h]).max() <= 1e-14
    # and with a zero start everything stays zero
    x.initial_state = None
    out, fin = run(x)
    assert not out.any() and not fin.any()


def test_unit_gate_keeps_state():
    """lower_bound = 0 gives alpha = 1; with beta = 0 the state is untouched."""
    x = W.random_inputs("lb0", 8, 1, 5, 1, K=8, V=8, init_std=1.0, lower_bound=0.0)
    x.raw_beta = torch.full_like(x.raw_beta, -math.inf)
    out, fin = run(x)
    assert np.array_equal(fin[0, 0], x.initial_state.double().numpy()[0, 0])


def test_reduces_to_gated_linear_attention():
    """Distinct one-hot keys and a zero start: the erase term vanishes.

    Then KDA is gated linear attention with write beta_t k^_t v_t^T, whose
    parallel (attention) form is
        o_t = scale * sum_{s<=t} beta_s <q^_t * decay(s->t), k^_s> v_s.
    Here raw_gate = dt_bias = 0 (every channel decays by exp(lb/2) per token)
    and raw_beta = 0 (beta = 1/2).
    """
    T, K, V = 12, 16, 8
    x = W.random_inputs("gla", 9, 1, T, 1, K=K, V=V, init_std=None)
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(3))[:T]
    k = torch.zeros_like(x.k)
    for t in range(T):
        k[0, t, 0, perm[t]] = 1.0 if t % 2 else -2.0
    x.k = k
    x.raw_gate = torch.zeros_like(x.raw_gate)
    x.dt_bias = torch.zeros_like(x.dt_bias)
    x.raw_beta = torch.zeros_like(x.raw_beta)
    out, fin = run(x)
    a = math.exp(x.lower_bound / 2)
    qf, kf, vf = (y.double().numpy()[0, :, 0] for y in (x.q, x.k, x.v))
    for t in range(T):
        ref = np.zeros(V)
        for s in range(t + 1):
            ref += 0.5 * a ** (t - s) * float(unit(qf[t]) @ unit(kf[s])) * vf[s]
        assert np.abs(out[t, 0] - x.scale * ref).max() <= 1e-15
    Sref = sum(0.5 * a ** (T - 1 - s) * np.outer(unit(kf[s]), vf[s]) for s in range(T))
    assert np.abs(fin[0, 0] - Sref).max() <= 1e-15


def test_one_hot_keys_store_values():
    """alpha = 1 (lower_bound 0), beta = 1 (raw_beta = +inf), one-hot keys.

    Writing key e_c replaces row c by v (up to the L2-norm epsilon): with
    kappa = 1/sqrt(1+eps), row c becomes (1 - kappa^2) row_c + kappa v and
    the other rows are untouched.  Repeated keys exercise the erase term.
    """
    T, K, V = 20, 8, 6
    x = W.random_inputs("store", 10, 1, T, 1, K=K, V=V, init_std=1.0, lower_bound=0.0)
    rows = [t % 5 for t in range(T)]
    k = torch.zeros_like(x.k)
    for t, c in enumerate(rows):
        k[0, t, 0, c] = 1.0
    x.k = k
    x.raw_beta = torch.full_like(x.raw_beta, math.inf)
    out, fin = run(x)
    kappa = 1.0 / math.sqrt(1.0 + EPS)
    S = x.initial_state.double().numpy()[0, 0].copy()
    vf, qf = x.v.double().numpy()[0, :, 0], x.q.double().numpy()[0, :, 0]
    for t, c in enumerate(rows):
        S[c] = (1 - kappa ** 2) * S[c] + kappa * vf[t]
        assert np.abs(out[t, 0] - x.scale * S.T @ unit(qf[t])).max() <= 1e-14
    assert np.abs(fin[0, 0] - S).max() <= 1e-14
    # "stores v exactly": the last value written to each row, up to eps
    for c in range(5):
        last = max(t for t in range(T) if rows[t] == c)
        assert np.abs(fin[0, 0, c] - vf[last]).max() <= 1e-5


@pytest.mark.parametrize("T", [256, 16384])
def test_near_collinear_closed_form(T):
    """The vLLM near-collinear test: q = k = one key, scalar gate, beta = sigmoid(8).

    With k^ fixed and every channel decaying by the same alpha, S_t = k^ s_t^T
    where s_t = alpha (1 - beta rho) s_{t-1} + beta v_t, rho = |k^|^2, and
    o_t = scale rho s_t.
    """
    x = W.c5_collinear(T=T)
    out, fin = run(x)
    key = x.k.double().numpy()[0, 0, 0]
    n2 = float(key @ key)
    rho = n2 / (n2 + EPS)
    kh = key / math.sqrt(n2 + EPS)
    beta = 1.0 / (1.0 + math.exp(-8.0))
    alpha = math.exp(-5.0 / (1.0 + math.exp(12.0)))
    vf = x.v.double().numpy()[0, :, 0]
    s = np.zeros(x.V)
    ref = np.empty((T, x.V))
    for t in range(T):
        s = alpha * (1 - beta * rho) * s + beta * vf[t]
        ref[t] = x.scale * rho * s
    m = metrics(out[:, 0], ref)
    # fp64 rounding accumulates over up to 16k steps: 1e-12 absolute
    assert m["finite"] and m["max_abs"] <= 1e-12
    assert np.abs(fin[0, 0] - np.outer(kh, s)).max() <= 1e-12


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------

def test_varlen_equals_per_document():
    lengths = [37, 1, 128, 90]
    x = W.random_inputs("varlen", 14, 1, sum(lengths), 3, lengths=lengths)
    out, fin = run(x)
    cu = x.cu_seqlens.tolist()
    for n in range(len(lengths)):
        s, e = cu[n], cu[n + 1]
        sub = lambda t: t[:, s:e].contiguous()  # noqa: E731
        o1, f1 = oracle_fwd(sub(x.q), sub(x.k), sub(x.v), sub(x.raw_gate), sub(x.raw_beta),
                            x.scale, x.A_log, x.dt_bias, x.lower_bound,
                            x.initial_state[n:n + 1], None)
        assert np.array_equal(o1, out[s:e]) and np.array_equal(f1[0], fin[n])


@pytest.mark.parametrize("T1", [1, 63, 64, 100, 137])
def test_split_resume_through_state(T1):
    T = 200
    x = W.random_inputs("split", 15, 1, T, 2)
    out, fin = run(x)
    a = lambda t: t[:, :T1].contiguous()  # noqa: E731
    b = lambda t: t[:, T1:].contiguous()  # noqa: E731
    o1, f1 = oracle_fwd(a(x.q), a(x.k), a(x.v), a(x.raw_gate), a(x.raw_beta), x.scale, x.A_log,
                        x.dt_bias, x.lower_bound, x.initial_state, None)
    o2, f2 = oracle_fwd(b(x.q), b(x.k), b(x.v), b(x.raw_gate), b(x.raw_beta), x.scale, x.A_log,
                        x.dt_bias, x.lower_bound, torch.from_numpy(f1).float(), None)
    # f1 is rounded to fp32 before it is fed back, as a caller's state would be
    assert np.abs(np.concatenate([o1, o2]) - out).max() <= 1e-6
    assert np.abs(f2 - fin).max() <= 1e-6
    # without the fp32 round trip the split is exact up to fp64 rounding
    o2x, f2x = oracle_fwd(b(x.q), b(x.k), b(x.v), b(x.raw_gate), b(x.raw_beta), x.scale, x.A_log,
                          x.dt_bias, x.lower_bound, None, None)
    assert o2x.shape == o2.shape


def test_power_of_two_rescaling_of_q_and_k():
    x = W.random_inputs("pow2", 16, 1, 150, 2)
    out, fin = run(x)
    x.q = (x.q.float() * 4.0).to(torch.bfloat16)
    x.k = (x.k.float() * 0.5).to(torch.bfloat16)
    o2, f2 = run(x)
    # only the epsilon inside the norm changes: relative effect ~ eps / |x|^2
    assert metrics(o2, out)["rel_l2"] <= 1e-7
    assert metrics(f2, fin)["rel_l2"] <= 1e-7


def test_head_permutation():
    x = W.random_inputs("perm", 17, 1, 90, 4)
    out, fin = run(x)
    p = [2, 0, 3, 1]
    y = W.random_inputs("perm", 17, 1, 90, 4)
    for name in ("q", "k", "v", "raw_gate", "raw_beta"):
        setattr(y, name, getattr(x, name)[:, :, p].contiguous())
    y.A_log = x.A_log[p].contiguous()
    y.dt_bias = x.dt_bias[p].contiguous()
    y.initial_state = x.initial_state[:, p].contiguous()
    o2, f2 = run(y)
    assert np.array_equal(o2, out[:, p]) and np.array_equal(f2, fin[:, p])


def test_head_subset_matches_full_run():
    x = W.random_inputs("subset", 18, 1, 70, 5)
    out, fin = run(x)
    o2, f2 = run(x, heads=[4, 1])
    assert np.array_equal(o2, out[:, [4, 1]]) and np.array_equal(f2, fin[:, [4, 1]])


def test_empty_sequence_passes_state_through():
    lengths = [5, 0, 7]
    x = W.random_inputs("empty", 19, 1, 12, 2, lengths=lengths)
    out, fin = run(x)
    assert np.array_equal(fin[1], x.initial_state[1].double().numpy())


def test_oracle_rejects_bad_cu_seqlens():
    x = W.random_inputs("bad", 20, 1, 10, 1, lengths=[4, 6])
    x.cu_seqlens = torch.tensor([0, 6, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        run(x)
