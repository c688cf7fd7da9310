"""Parity of the HIP path (through the C ABI) against the fp64 CPU oracle.

Tolerances (whole tensor): out relative L2 <= 1e-2 and max-abs <= 3e-2;
final_state relative L2 <= 1e-3; every value finite.
"""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_run import run_gpu
from oracle import metrics, oracle_fwd

pytestmark = pytest.mark.gpu

OUT_REL, OUT_ABS, FIN_REL = 1e-2, 3e-2, 1e-3


def oracle(x, heads=None, init=True):
    return oracle_fwd(x.q, x.k, x.v, x.raw_gate, x.raw_beta, x.scale, x.A_log, x.dt_bias,
                      x.lower_bound, x.initial_state if init else None, x.cu_seqlens,
                      heads=heads)


def check(o, f, ro, rf, label=""):
    mo = metrics(o, ro)
    print(f"{label}: out rel_l2={mo['rel_l2']:.3e} max_abs={mo['max_abs']:.3e}", end="")
    assert mo["finite"], "non-finite output"
    assert mo["rel_l2"] <= OUT_REL and mo["max_abs"] <= OUT_ABS, mo
    if f is not None:
        mf = metrics(f, rf)
        print(f" final rel_l2={mf['rel_l2']:.3e}", end="")
        assert mf["finite"], "non-finite final state"
        assert mf["rel_l2"] <= FIN_REL, mf
    print(flush=True)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def test_c1_reference_case():
    x = W.c1_ref()
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)


def test_c1_without_cu_seqlens():
    x = W.c1_ref()
    x.cu_seqlens = None
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name + " batch-mode")


def test_c2_tensor_parallel_share():
    x = W.c2_tp_share()
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)


def test_c4_varlen_packed():
    x = W.c4_varlen()
    assert x.T % 64 != 0
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)


def test_c5_near_collinear_keys():
    x = W.c5_collinear()
    o, f = run_gpu(x)           # q and k are one device buffer, as on the page
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)


def test_c5_near_collinear_keys_on_the_unsplit_chain():
    """C5 through the unsplit 256-chunk recurrence: an in-place state update and the
    transposed state layout both take it (the call above runs on 8 shards), and so
    does every call with 32 or more (sequence, head) chains."""
    import chunked_gated_delta_amd as kda
    x = W.c5_collinear()
    ro, rf = oracle(x)
    o, f = run_gpu(x, in_place=True)
    check(o, f, ro, rf, x.name + " (in place, unsplit)")
    dev = "cuda:0"
    d = lambda t: t.to(dev)  # noqa: E731
    out = torch.full_like(d(x.v), float("nan"))
    fin = torch.full((1, 1, 128, 128), float("nan"), device=dev)
    ws = torch.empty(kda.kda_workspace_size(x.T, 1, 1), dtype=torch.uint8, device=dev)
    qk = d(x.q)
    kda.kda_fwd_ex(qk, qk, d(x.v), d(x.raw_gate), d(x.raw_beta), x.scale, out, ws, d(x.A_log), d(x.dt_bias),
                   x.lower_bound, d(x.initial_state), fin, d(x.cu_seqlens), flags=kda.FLAG_STATE_VK)
    torch.cuda.synchronize()
    check(out.double().cpu().numpy().reshape(x.T, 1, 128), fin.double().cpu().numpy().swapaxes(-1, -2), ro, rf,
          x.name + " (transposed state, unsplit)")


@pytest.mark.parametrize("T", [32768, 65536])
def test_c5_near_collinear_keys_longer_than_the_page(T):
    """The page's stress case at 2x and 4x its length, on the split path (16 and 32 shards)
    and on the unsplit chain (in place).  With one repeated key and almost no decay the
    16-bit rounding of the state-update operands is the same every chunk, so its error
    adds up coherently along T (until the decay, 3e-5 per token, forgets it)."""
    x = W.c5_collinear(T=T)
    ro, rf = oracle(x)
    o, f = run_gpu(x)
    check(o, f, ro, rf, x.name + f" T={T} (shards)")
    o2, f2 = run_gpu(x, in_place=True)
    check(o2, f2, ro, rf, x.name + f" T={T} (in place, unsplit)")


def test_c3_headline_sampled_heads():
    """Full-size headline launch; the oracle recomputes three sampled heads."""
    x = W.c3_headline()
    o, f = run_gpu(x)
    heads = [0, 47, 95]
    ro, rf = oracle(x, heads=heads)
    check(o[:, heads], f[:, heads], ro, rf, x.name + f" heads {heads}")
    assert np.isfinite(o).all() and np.isfinite(f).all()


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 127, 129, 300])
def test_ragged_lengths(T):
    x = W.random_inputs(f"ragged_T{T}", 100 + T, 1, T, 3)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)


def test_varlen_with_empty_and_tiny_sequences():
    lengths = [0, 1, 64, 65, 0, 200, 17, 128]
    x = W.random_inputs("varlen_edges", 21, 1, sum(lengths), 4, lengths=lengths)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)
    # empty sequences pass the state through unchanged
    init = x.initial_state.double().numpy()
    assert np.array_equal(f[0], init[0]) and np.array_equal(f[4], init[4])


def test_packed_equals_per_document_bitwise():
    lengths = [70, 5, 130, 64]
    x = W.random_inputs("packed", 22, 1, sum(lengths), 2, lengths=lengths)
    o, f = run_gpu(x)
    cu = x.cu_seqlens.tolist()
    for n in range(len(lengths)):
        s, e = cu[n], cu[n + 1]
        y = W.random_inputs("packed", 22, 1, sum(lengths), 2, lengths=lengths)
        for name in ("q", "k", "v", "raw_gate", "raw_beta"):
            setattr(y, name, getattr(x, name)[:, s:e].contiguous())
        y.initial_state = x.initial_state[n:n + 1].contiguous()
        y.cu_seqlens = None
        o1, f1 = run_gpu(y)
        assert np.array_equal(o1, o[s:e]) and np.array_equal(f1[0], f[n])


def test_split_and_resume_through_state():
    T, T1 = 300, 137
    x = W.random_inputs("split", 23, 1, T, 2)
    o, f = run_gpu(x)
    a = W.random_inputs("split", 23, 1, T, 2)
    b = W.random_inputs("split", 23, 1, T, 2)
    for name in ("q", "k", "v", "raw_gate", "raw_beta"):
        setattr(a, name, getattr(x, name)[:, :T1].contiguous())
        setattr(b, name, getattr(x, name)[:, T1:].contiguous())
    o1, f1 = run_gpu(a)
    b.initial_state = torch.from_numpy(f1).float()
    o2, f2 = run_gpu(b)
    ro, rf = oracle(x)
    check(np.concatenate([o1, o2]), f2, ro, rf, "split at 137")


def test_in_place_state_and_null_states():
    x = W.random_inputs("inplace", 24, 1, 150, 2)
    ro, rf = oracle(x)
    o, f = run_gpu(x, in_place=True)
    check(o, f, ro, rf, "in-place state")
    o2, f2 = run_gpu(x, with_init=False)
    ro2, rf2 = oracle(x, init=False)
    check(o2, f2, ro2, rf2, "null initial state")
    o3, f3 = run_gpu(x, with_final=False)
    assert f3 is None
    check(o3, None, ro, None, "null final state")


def test_q_and_k_share_one_buffer():
    x = W.random_inputs("qk_alias", 25, 1, 200, 2)
    x.k = x.q
    o, f = run_gpu(x, q_alias_k=True)
    ro, rf = oracle(x)
    check(o, f, ro, rf, "q is k")


def test_batch_mode_several_sequences():
    x = W.random_inputs("batch", 26, 3, 100, 2)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, "B=3 batch mode")


@pytest.mark.parametrize("lb", [0.0, -1.0, -5.0])
def test_lower_bound_range(lb):
    x = W.random_inputs(f"lb{lb}", 27, 1, 200, 2, lower_bound=lb)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, f"lower_bound {lb}")


def test_extreme_gates_and_betas():
    """raw_beta = +-inf (beta 1 / 0) and saturated gates (raw_gate +-30)."""
    x = W.random_inputs("extreme", 28, 1, 160, 2)
    rb = x.raw_beta.float()
    rb[0, ::3] = float("inf")
    rb[0, 1::3] = -float("inf")
    x.raw_beta = rb.to(torch.bfloat16)
    rg = x.raw_gate.float()
    rg[0, ::2] = 30.0
    rg[0, 1::4] = -30.0
    x.raw_gate = rg.to(torch.bfloat16)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, "extreme gates")


def test_zero_keys_and_queries():
    x = W.random_inputs("zeros", 29, 1, 100, 2)
    q = x.q.clone()
    k = x.k.clone()
    q[0, 10:20] = 0
    k[0, 30:45] = 0
    x.q, x.k = q, k
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, "zero rows")


def test_head_permutation_is_exact():
    x = W.random_inputs("perm", 30, 1, 130, 4)
    o, f = run_gpu(x)
    p = [3, 1, 0, 2]
    y = W.random_inputs("perm", 30, 1, 130, 4)
    for name in ("q", "k", "v", "raw_gate", "raw_beta"):
        setattr(y, name, getattr(x, name)[:, :, p].contiguous())
    y.A_log = x.A_log[p].contiguous()
    y.dt_bias = x.dt_bias[p].contiguous()
    y.initial_state = x.initial_state[:, p].contiguous()
    o2, f2 = run_gpu(y)
    assert np.array_equal(o2, o[:, p]) and np.array_equal(f2, f[:, p])


def test_deterministic():
    x = W.random_inputs("det", 31, 1, 260, 3)
    o1, f1 = run_gpu(x)
    o2, f2 = run_gpu(x)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_runs_on_a_side_stream():
    x = W.random_inputs("stream", 32, 1, 200, 2)
    s = torch.cuda.Stream()
    o, f = run_gpu(x, stream=s.cuda_stream)
    ro, rf = oracle(x)
    check(o, f, ro, rf, "side stream")


def test_zero_tokens_copies_the_state():
    """B sequences of T = 0 tokens (empty, NULL-pointer tensors): final = initial."""
    import chunked_gated_delta_amd as kda
    dev = "cuda:0"
    x = W.random_inputs("empty", 71, 2, 0, 3, init_std=0.3)
    fin = torch.full((2, 3, 128, 128), float("nan"), device=dev)
    out = torch.empty(2, 0, 3, 128, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(kda.kda_workspace_size(0, 3, 2), 1), dtype=torch.uint8, device=dev)
    kda.kda_fwd(*(t.to(dev) for t in (x.q, x.k, x.v, x.raw_gate, x.raw_beta)), x.scale, out, ws,
                x.A_log.to(dev), x.dt_bias.to(dev), x.lower_bound, x.initial_state.to(dev), fin)
    torch.cuda.synchronize()
    assert torch.equal(fin.cpu(), x.initial_state)


@pytest.mark.parametrize("H", [40, 64])
def test_slice_width_changes_no_bit(H):
    """With few (sequence, head) chains the inter-chunk recurrence runs in narrower
    V slices per workgroup (on 256 CUs: H=2 gives 16 columns, H=40 gives 32, H=64
    the full 64).  Each output column is computed the same way at every width, so
    the two-head subset, run at H=2, reproduces the wide run bit for bit."""
    x = W.random_inputs(f"slices_H{H}", 300 + H, 1, 129, H)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)
    p = [0, H - 1]
    y = W.random_inputs(f"slices_H{H}", 300 + H, 1, 129, H)
    for name in ("q", "k", "v", "raw_gate", "raw_beta"):
        setattr(y, name, getattr(x, name)[:, :, p].contiguous())
    y.A_log = x.A_log[p].contiguous()
    y.dt_bias = x.dt_bias[p].contiguous()
    y.initial_state = x.initial_state[:, p].contiguous()
    o2, f2 = run_gpu(y)
    assert np.array_equal(o2, o[:, p]) and np.array_equal(f2, f[:, p])


@pytest.mark.parametrize("H", [2, 10, 20])
def test_varlen_at_every_slice_width(H):
    """Packed sequences with ragged tails and an empty one, at the head counts that pick
    16-, 32- and 64-column slices (4 sequences: 8, 40 and 80 (sequence, head) pairs)."""
    lengths = [130, 0, 64, 77]
    x = W.random_inputs(f"varlen_slices_H{H}", 400 + H, 1, sum(lengths), H, lengths=lengths)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)
    assert np.array_equal(f[1], x.initial_state[1].double().numpy())


@pytest.mark.parametrize("N", [300, 3000])
def test_many_short_sequences(N):
    """Hundreds to thousands of packed sequences of 0-70 (N = 300) or 0-5 tokens
    (N = 3000), empty ones included, through the longest-first sequence order."""
    g = np.random.default_rng(N)
    lengths = [int(v) for v in g.integers(0, 6 if N > 1000 else 71, size=N)]
    x = W.random_inputs(f"many_N{N}", 700 + N % 97, 1, sum(lengths), 2, lengths=lengths)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name)


@pytest.mark.parametrize("B,T,H,init,lb", [(1, 25600, 1, False, -5.0), (2, 16000, 2, True, -5.0),
                                             (1, 16421, 3, True, -0.01), (1, 20000, 1, True, -0.002)])
def test_long_sequences_with_few_heads_run_on_shards(B, T, H, init, lb):
    """Few (sequence, head) pairs and long sequences: the forward cuts every sequence into
    shards of at least 32 chunks (here 12, 7, 8 and 9 per sequence, ragged last shards
    included), folds their affine maps and runs the shards from the folded states.  With
    lower_bound -5 the state forgets a shard's start within it; the small lower bounds
    keep it, so the fold carries the state across shards.  An in-place state update takes
    the unsplit path, so the same inputs are checked both ways."""
    x = W.random_inputs(f"split_B{B}_T{T}_H{H}", 800 + T % 97, B, T, H, init_std=0.1 if init else None,
                        lower_bound=lb)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name + " (shards)")
    if init:
        o2, f2 = run_gpu(x, in_place=True)
        check(o2, f2, ro, rf, x.name + " (in place, unsplit)")


@pytest.mark.parametrize("lengths,H,lb", [([12000, 5000], 2, -0.01), ([33000, 0, 100, 64], 1, -0.002)])
def test_varlen_long_sequences_run_on_shards_of_their_own_length(lengths, H, lb):
    """Packed sequences whose mean length calls for 4 shards: each sequence is cut into 4
    shards of its own length (47 and 20 chunks; 0, 1 and 1 chunks, so empty shards and an
    empty sequence too), the folds carry the state across them, and the outputs and final
    states match the oracle and the unsplit in-place path."""
    x = W.random_inputs(f"split_varlen_{len(lengths)}_H{H}", 900 + len(lengths), 1, sum(lengths), H,
                        lengths=lengths, init_std=0.1, lower_bound=lb)
    o, f = run_gpu(x)
    ro, rf = oracle(x)
    check(o, f, ro, rf, x.name + " (shards)")
    o2, f2 = run_gpu(x, in_place=True)
    check(o2, f2, ro, rf, x.name + " (in place, unsplit)")
