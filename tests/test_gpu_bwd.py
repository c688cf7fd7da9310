"""Parity of kda_bwd (through the C ABI) against the fp64 gradient oracle.

The oracle is torch autograd through the fp64 token recurrence
(oracle/grad.py) at small sizes, and the chunked fp64 reverse-mode form
(oracle/chunked.py, pinned to it) where the token loop's graph would not fit.
Tolerance, per gradient: relative L2 <= 1e-2 and max-abs error <= 2e-2 of the
reference's largest magnitude, all values finite.  Why 1e-2: the gradients
are written in bf16 (relative rounding 2^-9) and the forward states they use
come from the forward's fp16/bf16 operands (relative ~1e-3), so the expected
error is a few 1e-3; the forward's own output bar is the same 1e-2.
The varlen property test follows the torchtitan page's packed-versus-separate
documents check ("Results": forward and gradient).
"""

import numpy as np
import pytest
import torch

import chunked_gated_delta_amd as kda
import workloads as W
from oracle.chunked import chunked_bwd
from oracle.grad import oracle_bwd

pytestmark = pytest.mark.gpu

REL, MAXREL = 1e-2, 2e-2
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "d_raw_gate", "d_raw_beta", "dA_log", "d_dt_bias", "d_initial_state")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def d(t):
    return None if t is None else t.to(DEV)


def cotangents(x, seed, with_final=True):
    g = torch.Generator().manual_seed(seed)
    d_out = torch.randn(x.B, x.T, x.H, x.V, generator=g).to(torch.bfloat16)
    d_fin = torch.randn(x.N, x.H, x.K, x.V, generator=g) if with_final else None
    return d_out, d_fin


def gpu_bwd(x, d_out, d_fin, with_dinit=True):
    """Returns a dict of fp64 numpy gradients shaped like oracle_bwd's."""
    B, T, H, K, V, N = x.B, x.T, x.H, x.K, x.V, x.N
    nan_bf = lambda *s: torch.full(s, float("nan"), dtype=torch.bfloat16, device=DEV)  # noqa: E731
    dq, dk, dg = nan_bf(B, T, H, K), nan_bf(B, T, H, K), nan_bf(B, T, H, K)
    dv, db = nan_bf(B, T, H, V), nan_bf(B, T, H)
    dA = torch.full((H,), float("nan"), device=DEV)
    ddt = torch.full((H, K), float("nan"), device=DEV)
    dinit = torch.full((N, H, K, V), float("nan"), device=DEV) if with_dinit else None
    ws = torch.empty(kda.kda_bwd_workspace_size(B * T, H, N), dtype=torch.uint8, device=DEV)
    print(f"kda_bwd {x.name} B={B} T={T} H={H} N={N}", flush=True)
    kda.kda_bwd(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, d(d_out), dq, dk, dv, dg, db,
                dA, ddt, ws, d(x.A_log), d(x.dt_bias), x.lower_bound, initial_state=d(x.initial_state),
                d_final=d(d_fin), d_initial_state=dinit, cu_seqlens=d(x.cu_seqlens))
    torch.cuda.synchronize()
    f = lambda t, *s: t.double().cpu().numpy().reshape(*s)  # noqa: E731
    return {"dq": f(dq, B * T, H, K), "dk": f(dk, B * T, H, K), "dv": f(dv, B * T, H, V),
            "d_raw_gate": f(dg, B * T, H, K), "d_raw_beta": f(db, B * T, H), "dA_log": f(dA, H),
            "d_dt_bias": f(ddt, H, K), "d_initial_state": None if dinit is None else f(dinit, N, H, K, V)}


def compare(got, ref, names=NAMES):
    for n in names:
        if ref.get(n) is None or got.get(n) is None:
            continue
        r, g = np.asarray(ref[n], dtype=np.float64), np.asarray(got[n], dtype=np.float64)
        assert np.isfinite(g).all(), (n, "non-finite")
        if r.size == 0:
            continue
        scale_ = max(np.linalg.norm(r), 1e-30)
        rel = np.linalg.norm(g - r) / scale_
        mx = np.abs(g - r).max() / max(np.abs(r).max(), 1e-30)
        print(f"  {n}: rel_l2 {rel:.2e} max/maxref {mx:.2e}", flush=True)
        assert rel <= REL and mx <= MAXREL, (n, rel, mx)


def oracle(x, d_out, d_fin, chunked=False):
    fn = chunked_bwd if chunked else oracle_bwd
    return fn(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias, x.lower_bound,
              d_out.double(), None if d_fin is None else d_fin.double(), x.initial_state, x.cu_seqlens)


def test_bwd_one_tail_chunk():
    x = W.random_inputs("bwd_T40", 201, 1, 40, 2)
    d_out, d_fin = cotangents(x, 1)
    compare(gpu_bwd(x, d_out, d_fin), oracle(x, d_out, d_fin))


def test_bwd_reference_case_c1():
    """3 full chunks and an 8-token tail, zero initial state, A_log = dt_bias = 0."""
    x = W.c1_ref()
    d_out, d_fin = cotangents(x, 2)
    compare(gpu_bwd(x, d_out, d_fin, with_dinit=False), oracle(x, d_out, d_fin))


def test_bwd_batch_with_state_and_no_final_gradient():
    x = W.random_inputs("bwd_B2_T130", 202, 2, 130, 3)
    d_out, _ = cotangents(x, 3, with_final=False)
    compare(gpu_bwd(x, d_out, None), oracle(x, d_out, None))


def test_bwd_varlen_with_empty_and_ragged_sequences():
    lengths = [1, 0, 64, 70, 5, 0, 129]
    x = W.random_inputs("bwd_varlen", 203, 1, sum(lengths), 2, lengths=lengths)
    d_out, d_fin = cotangents(x, 4)
    compare(gpu_bwd(x, d_out, d_fin), oracle(x, d_out, d_fin))


def test_bwd_strong_decay_and_gate_parameters():
    """A_log at ln 16 everywhere: most channels decay near the floor (exp(-5) per token)."""
    x = W.random_inputs("bwd_decay", 204, 1, 192, 2, dt_bias_std=1.0)
    x.A_log.fill_(float(np.log(16.0)))
    d_out, d_fin = cotangents(x, 5)
    compare(gpu_bwd(x, d_out, d_fin), oracle(x, d_out, d_fin))


def check_sampled_heads(x, d_out, d_fin, heads):
    """GPU gradients of every head; the sampled heads against the chunked fp64 backward."""
    got = gpu_bwd(x, d_out, d_fin)
    for h in heads:
        xs = W.KdaInputs(name=f"{x.name}_head{h}", q=x.q[:, :, h:h + 1].contiguous(),
                         k=x.k[:, :, h:h + 1].contiguous(), v=x.v[:, :, h:h + 1].contiguous(),
                         raw_gate=x.raw_gate[:, :, h:h + 1].contiguous(),
                         raw_beta=x.raw_beta[:, :, h:h + 1].contiguous(), A_log=x.A_log[h:h + 1].contiguous(),
                         dt_bias=x.dt_bias[h:h + 1].contiguous(),
                         initial_state=x.initial_state[:, h:h + 1].contiguous(), cu_seqlens=None,
                         scale=x.scale, lower_bound=x.lower_bound)
        ref = oracle(xs, d_out[:, :, h:h + 1].contiguous(), d_fin[:, h:h + 1].contiguous(), chunked=True)
        sub = {n: (None if got[n] is None else got[n][:, h:h + 1] if n in ("dq", "dk", "dv", "d_raw_gate",
                                                                             "d_raw_beta", "d_initial_state")
                   else got[n][h:h + 1]) for n in NAMES}
        compare(sub, ref)


def test_bwd_tp_share_c2_sampled_heads():
    """B=2, T=4096, H=12 on the GPU; heads 0 and 7 checked against the chunked fp64 backward."""
    x = W.c2_tp_share()
    d_out, d_fin = cotangents(x, 6)
    check_sampled_heads(x, d_out, d_fin, (0, 7))


def test_bwd_c2_shape_head_dim_64():
    """The C2 shape (B=2, T=4096, H=12, initial states) with K = V = 64: heads 3 and 11."""
    x = W.random_inputs("c2_B2_T4096_H12_K64", 11, 2, 4096, 12, K=64, V=64)
    d_out, d_fin = cotangents(x, 16)
    check_sampled_heads(x, d_out, d_fin, (3, 11))


def test_bwd_packed_equals_separate_documents():
    """Gradients of a packed varlen call equal those of each document run alone (GPU vs GPU)."""
    lengths = [300, 64, 1, 257]
    x = W.random_inputs("bwd_pack", 205, 1, sum(lengths), 3, lengths=lengths)
    d_out, d_fin = cotangents(x, 7)
    packed = gpu_bwd(x, d_out, d_fin)
    cu = [0] + list(np.cumsum(lengths))
    dA_sum = np.zeros(x.H)
    ddt_sum = np.zeros((x.H, x.K))
    for n, (s, e) in enumerate(zip(cu[:-1], cu[1:])):
        xs = W.KdaInputs(name=f"doc{n}", q=x.q[:, s:e].contiguous(), k=x.k[:, s:e].contiguous(),
                         v=x.v[:, s:e].contiguous(), raw_gate=x.raw_gate[:, s:e].contiguous(),
                         raw_beta=x.raw_beta[:, s:e].contiguous(), A_log=x.A_log, dt_bias=x.dt_bias,
                         initial_state=x.initial_state[n:n + 1].contiguous(), cu_seqlens=None,
                         scale=x.scale, lower_bound=x.lower_bound)
        one = gpu_bwd(xs, d_out[:, s:e].contiguous(), d_fin[n:n + 1].contiguous())
        for name in ("dq", "dk", "dv", "d_raw_gate", "d_raw_beta"):
            np.testing.assert_allclose(packed[name][s:e], one[name], rtol=1e-2, atol=1e-2, err_msg=name)
        np.testing.assert_allclose(packed["d_initial_state"][n], one["d_initial_state"][0], rtol=1e-4,
                                   atol=1e-5)
        dA_sum += one["dA_log"]
        ddt_sum += one["d_dt_bias"]
    np.testing.assert_allclose(packed["dA_log"], dA_sum, rtol=1e-3, atol=1e-3)
    np.testing.assert_allclose(packed["d_dt_bias"], ddt_sum, rtol=1e-3, atol=1e-3)


def test_bwd_zero_tokens():
    x = W.random_inputs("bwd_empty", 206, 1, 0, 2)
    d_out, d_fin = cotangents(x, 8)
    got = gpu_bwd(x, d_out, d_fin)
    np.testing.assert_array_equal(got["dA_log"], 0.0)
    np.testing.assert_array_equal(got["d_dt_bias"], 0.0)
    np.testing.assert_array_equal(got["d_initial_state"], d_fin.double().numpy())


def test_bwd_near_collinear_c5():
    """One key repeated along T = 16384 as both q and k (raw_beta 8, raw_gate -12): against the
    chunked fp64 backward.  Two gradients need a bound other than the relative one:
      * dq is exactly zero: the state stays k^ s^T, so dq^ is parallel to q^ and the L2 norm's
        projection removes it (the fp64 reference holds ~1e-9 of rounding).  Its error is held to
        1e-2 of the largest |dk|, the companion gradient of the same key.
      * dA_log is a sum over every (token, channel) of d_raw_gate (raw_gate + dt_bias) whose terms
        cancel to ~1e-8 of their magnitude here.  It is held to the summation error bound:
        |error| <= 1e-2 * sum |term|, the terms taken from the oracle's own d_raw_gate.
    Every other gradient, d dt_bias included, meets the relative bar."""
    x = W.c5_collinear()
    d_out, d_fin = cotangents(x, 9)
    got = gpu_bwd(x, d_out, d_fin)
    ref = oracle(x, d_out, d_fin, chunked=True)
    compare(got, ref, names=tuple(n for n in NAMES if n not in ("dq", "dA_log")))
    err = np.abs(got["dq"] - ref["dq"]).max()
    print(f"  dq: max abs err {err:.2e} (|dk| max {np.abs(ref['dk']).max():.2e})", flush=True)
    assert np.isfinite(got["dq"]).all() and err <= 1e-2 * np.abs(ref["dk"]).max()
    z = (x.raw_gate.double().reshape(x.B * x.T, x.H, x.K) + x.dt_bias.double()).numpy()
    bound = np.abs(ref["d_raw_gate"] * z).sum(axis=(0, 2))
    err = np.abs(got["dA_log"] - ref["dA_log"])
    print(f"  dA_log: err/bound {np.max(err / bound):.2e}", flush=True)
    assert np.isfinite(got["dA_log"]).all() and (err <= 1e-2 * bound).all()


def test_bwd_varlen_c4_sampled():
    """The full C4 batch (16 packed sequences of lengths U[1, 8192], H = 32) on the GPU.  Sampled
    outputs: for heads 5 and 30, the token gradients and initial-state gradient of sequences 6, 11
    (the two shortest) and 14 (the longest) against the chunked fp64 backward of that sequence
    alone (sequences are independent).  The parameter gradients, sums over every sequence, are
    checked at C2 size and by the packed-versus-separate test."""
    x = W.c4_varlen()
    d_out, d_fin = cotangents(x, 10)
    got = gpu_bwd(x, d_out, d_fin)
    cu = x.cu_seqlens.tolist()
    per_token = ("dq", "dk", "dv", "d_raw_gate", "d_raw_beta")
    for n in (6, 11, 14):
        s_, e_ = cu[n], cu[n + 1]
        for h in (5, 30):
            xs = W.KdaInputs(name=f"c4_seq{n}_head{h}", q=x.q[:, s_:e_, h:h + 1].contiguous(),
                             k=x.k[:, s_:e_, h:h + 1].contiguous(), v=x.v[:, s_:e_, h:h + 1].contiguous(),
                             raw_gate=x.raw_gate[:, s_:e_, h:h + 1].contiguous(),
                             raw_beta=x.raw_beta[:, s_:e_, h:h + 1].contiguous(),
                             A_log=x.A_log[h:h + 1].contiguous(), dt_bias=x.dt_bias[h:h + 1].contiguous(),
                             initial_state=x.initial_state[n:n + 1, h:h + 1].contiguous(), cu_seqlens=None,
                             scale=x.scale, lower_bound=x.lower_bound)
            ref = oracle(xs, d_out[:, s_:e_, h:h + 1].contiguous(), d_fin[n:n + 1, h:h + 1].contiguous(),
                         chunked=True)
            sub = {k_: got[k_][s_:e_, h:h + 1] for k_ in per_token}
            sub["d_initial_state"] = got["d_initial_state"][n:n + 1, h:h + 1]
            compare(sub, ref, names=per_token + ("d_initial_state",))


def test_bwd_final_state_gradient_only():
    """d_out = 0: every gradient flows back from the final state alone."""
    x = W.random_inputs("bwd_fin_only", 207, 1, 150, 2)
    d_out, d_fin = cotangents(x, 11)
    d_out = torch.zeros_like(d_out)
    compare(gpu_bwd(x, d_out, d_fin), oracle(x, d_out, d_fin))


def test_bwd_initial_state_gradient_in_place():
    """d_initial_state may be the d_final buffer itself."""
    x = W.random_inputs("bwd_inplace", 208, 2, 100, 2)
    d_out, d_fin = cotangents(x, 12)
    ref = gpu_bwd(x, d_out, d_fin)
    B, T, H, K, V, N = x.B, x.T, x.H, x.K, x.V, x.N
    bf = lambda *s: torch.empty(s, dtype=torch.bfloat16, device=DEV)  # noqa: E731
    dq, dk, dg, dv, db = bf(B, T, H, K), bf(B, T, H, K), bf(B, T, H, K), bf(B, T, H, V), bf(B, T, H)
    dA, ddt = torch.empty(H, device=DEV), torch.empty(H, K, device=DEV)
    buf = d(d_fin).clone()
    ws = torch.empty(kda.kda_bwd_workspace_size(B * T, H, N), dtype=torch.uint8, device=DEV)
    kda.kda_bwd(d(x.q), d(x.k), d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, d(d_out), dq, dk, dv, dg, db, dA,
                ddt, ws, d(x.A_log), d(x.dt_bias), x.lower_bound, initial_state=d(x.initial_state), d_final=buf,
                d_initial_state=buf)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(buf.double().cpu().numpy(), ref["d_initial_state"])
    np.testing.assert_array_equal(dq.double().cpu().numpy().reshape(B * T, H, K), ref["dq"])


def test_bwd_long_sequence_with_few_heads_checkpoints_on_shards():
    """T = 8192 with 2 heads: the checkpointing forward pass runs on 4 shards per sequence
    from their folded entering states, and the reverse recurrence on the same shards from
    their folded leaving gradients (lower_bound -0.01, so state and gradient carry across
    shards); the gradients still match the chunked fp64 oracle."""
    x = W.random_inputs("bwd_split", 231, 1, 8192, 2, lower_bound=-0.01)
    d_out, d_fin = cotangents(x, 232)
    compare(gpu_bwd(x, d_out, d_fin), oracle(x, d_out, d_fin, chunked=True))


def test_bwd_two_long_sequences_fold_each_on_its_own_shards():
    """Two sequences of 8192 tokens, one head: 4 shards each, both folds (forward states and
    reverse gradients) per sequence, with the slowest decay (lower_bound -0.002) so that a
    shard's gradient reaches far back; every gradient matches the chunked fp64 oracle."""
    x = W.random_inputs("bwd_split2", 233, 2, 8192, 1, lower_bound=-0.002)
    d_out, d_fin = cotangents(x, 234)
    compare(gpu_bwd(x, d_out, d_fin), oracle(x, d_out, d_fin, chunked=True))


def test_bwd_split_ragged_tail_without_state_gradients():
    """T = 8229 (a 37-token tail in the last of 4 shards) with no final-state gradient and
    no d_initial_state requested: the reverse fold starts from zero and writes nothing for
    the initial state, and the gradients still match the chunked fp64 oracle."""
    x = W.random_inputs("bwd_split_tail", 235, 1, 8229, 2, lower_bound=-0.01)
    d_out, _ = cotangents(x, 236, with_final=False)
    compare(gpu_bwd(x, d_out, None, with_dinit=False), oracle(x, d_out, None, chunked=True))


def test_bwd_varlen_long_sequences_on_shards():
    """Two packed sequences of 9000 and 7500 tokens, 2 heads: the mean length gives 4 shards
    per sequence, each cut by its own length; both recurrences run on them and every
    gradient matches the chunked fp64 oracle."""
    lengths = [9000, 7500]
    x = W.random_inputs("bwd_split_varlen", 237, 1, sum(lengths), 2, lengths=lengths, lower_bound=-0.01)
    d_out, d_fin = cotangents(x, 238)
    compare(gpu_bwd(x, d_out, d_fin), oracle(x, d_out, d_fin, chunked=True))
