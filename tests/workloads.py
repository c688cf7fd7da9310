"""Seeded synthetic KDA forward inputs.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic.  Both the oracle tests and the GPU path consume the
tensors it returns, so the two sides see bit-identical inputs.

The workloads follow the shapes and value distributions of the pages' calls:
  * the FlashKDA usage example on the instagit page (section "Usage Examples":
    q, k, v, g, beta bf16 [B,T,H,*], A_log fp32 [H], dt_bias fp32 [H,K],
    lower_bound -5.0);
  * the near-collinear-key test in the vLLM PR report (section "关键源码片段":
    one key repeated at every position and passed as both q and k, a 16-token
    value block tiled along T, raw_gate -12, raw_beta 8, T=16384, H=1, D=128,
    scale D**-0.5, cu_seqlens [0, T]).

Recipe (fixed here, documented in the design notes): a CPU ``torch.Generator``
seeded per workload draws float32 values in the order q, k, v, raw_gate,
raw_beta, A_log, dt_bias, initial_state, lengths; bf16 tensors are the float32
draws rounded to nearest-even by ``.to(torch.bfloat16)``.  "N(0, 0.1)" is read
as standard deviation 0.1.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import torch

K_DIM = 128
V_DIM = 128


@dataclass
class KdaInputs:
    """Host (CPU) tensors of one KDA forward call plus its sizes.

    Layouts (all contiguous):
      q, k, raw_gate: bf16 [B, T, H, K]
      v:              bf16 [B, T, H, V]
      raw_beta:       bf16 [B, T, H]
      A_log:          fp32 [H]
      dt_bias:        fp32 [H, K]
      initial_state:  fp32 [N, H, K, V] or None (zeros)
      cu_seqlens:     int32 [N + 1] or None (N = B sequences of length T)
    With cu_seqlens, B == 1 and T is the packed token count.
    """

    name: str
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    raw_gate: torch.Tensor
    raw_beta: torch.Tensor
    A_log: torch.Tensor
    dt_bias: torch.Tensor
    initial_state: Optional[torch.Tensor]
    cu_seqlens: Optional[torch.Tensor]
    scale: float
    lower_bound: float
    q_is_k: bool = False
    meta: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return self.q.shape[0]

    @property
    def T(self) -> int:
        return self.q.shape[1]

    @property
    def H(self) -> int:
        return self.q.shape[2]

    @property
    def K(self) -> int:
        return self.q.shape[3]

    @property
    def V(self) -> int:
        return self.v.shape[3]

    @property
    def N(self) -> int:
        return self.B if self.cu_seqlens is None else self.cu_seqlens.numel() - 1

    def seq_bounds(self):
        """(start, end) token offsets of every sequence in the flattened [B*T] axis."""
        if self.cu_seqlens is None:
            return [(b * self.T, (b + 1) * self.T) for b in range(self.B)]
        cu = self.cu_seqlens.tolist()
        return [(cu[n], cu[n + 1]) for n in range(len(cu) - 1)]

    def head_tokens(self) -> int:
        return self.B * self.T * self.H


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def random_inputs(
    name: str,
    seed: int,
    B: int,
    T: int,
    H: int,
    K: int = K_DIM,
    V: int = V_DIM,
    *,
    lengths: Optional[list] = None,
    a_log: str = "uniform_ln16",
    dt_bias_std: float = 0.1,
    init_std: Optional[float] = 0.1,
    lower_bound: float = -5.0,
    scale: Optional[float] = None,
) -> KdaInputs:
    """Standard-normal q/k/v/raw_gate/raw_beta with the given gate parameter recipe.

    ``lengths`` packs N sequences of those lengths (B must be 1 and T their sum)
    behind an int32 cu_seqlens.  ``a_log`` is "zeros" or "uniform_ln16"
    (U(0, ln 16)).  ``init_std`` None means no initial state (zeros).
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    if lengths is not None:
        assert B == 1 and sum(lengths) == T
    q = _bf16(torch.randn(B, T, H, K, generator=g))
    k = _bf16(torch.randn(B, T, H, K, generator=g))
    v = _bf16(torch.randn(B, T, H, V, generator=g))
    raw_gate = _bf16(torch.randn(B, T, H, K, generator=g))
    raw_beta = _bf16(torch.randn(B, T, H, generator=g))
    if a_log == "zeros":
        A_log = torch.zeros(H, dtype=torch.float32)
    elif a_log == "uniform_ln16":
        A_log = torch.rand(H, generator=g) * math.log(16.0)
    else:
        raise ValueError(a_log)
    if dt_bias_std == 0.0:
        dt_bias = torch.zeros(H, K, dtype=torch.float32)
    else:
        dt_bias = torch.randn(H, K, generator=g) * dt_bias_std
    N = B if lengths is None else len(lengths)
    if init_std is None:
        init = None
    else:
        init = torch.randn(N, H, K, V, generator=g) * init_std
    cu = None
    if lengths is not None:
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return KdaInputs(
        name=name, q=q, k=k, v=v, raw_gate=raw_gate, raw_beta=raw_beta,
        A_log=A_log.float().contiguous(), dt_bias=dt_bias.float().contiguous(),
        initial_state=None if init is None else init.float().contiguous(),
        cu_seqlens=cu, scale=(K ** -0.5) if scale is None else scale,
        lower_bound=lower_bound,
    )


def varlen_lengths(seed: int, n: int, lo: int, hi: int) -> list:
    """n integer lengths drawn uniformly from [lo, hi] by a generator of its own."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randint(lo, hi + 1, (n,), generator=g).tolist()


def near_collinear(seed: int = 4, T: int = 16384, H: int = 1, D: int = 128) -> KdaInputs:
    """One key vector repeated along T, used as both q and k; a tiled 16-token v block.

    Shapes and constants follow the near-collinear test in the vLLM PR report
    (raw_gate -12, raw_beta 8, A_log 0, dt_bias 0, lower_bound -5, zero state).
    """
    assert T % 16 == 0
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    key = _bf16(torch.randn(1, 1, H, D, generator=g))
    qk = key.expand(1, T, H, D).contiguous()
    vblock = _bf16(torch.randn(1, 16, H, D, generator=g))
    v = vblock.repeat(1, T // 16, 1, 1).contiguous()
    raw_gate = torch.full_like(qk, -12.0)
    raw_beta = torch.full((1, T, H), 8.0, dtype=torch.bfloat16)
    return KdaInputs(
        name="collinear", q=qk, k=qk, v=v, raw_gate=raw_gate, raw_beta=raw_beta,
        A_log=torch.zeros(H, dtype=torch.float32),
        dt_bias=torch.zeros(H, D, dtype=torch.float32),
        initial_state=torch.zeros(1, H, D, D, dtype=torch.float32),
        cu_seqlens=torch.tensor([0, T], dtype=torch.int32),
        scale=D ** -0.5, lower_bound=-5.0, q_is_k=True,
    )


# ---------------------------------------------------------------------------
# The five workloads.  C1 is the small reference case (3 full 64-token chunks
# plus an 8-token tail), C2 one tensor-parallel rank's share (12 of 96 heads),
# C3 the throughput headline, C4 a packed varlen batch, C5 near-collinear keys.
# ---------------------------------------------------------------------------

def c1_ref() -> KdaInputs:
    x = random_inputs("c1_ref_T200_H2", 0, 1, 200, 2, a_log="zeros", dt_bias_std=0.0,
                      init_std=None)
    return x


def c2_tp_share(T: int = 4096) -> KdaInputs:
    return random_inputs(f"c2_B2_T{T}_H12", 1, 2, T, 12)


def c3_headline(T: int = 32768, H: int = 96) -> KdaInputs:
    return random_inputs(f"c3_B1_T{T}_H{H}", 2, 1, T, H, init_std=None)


def c4_varlen(n: int = 16, max_len: int = 8192, H: int = 32) -> KdaInputs:
    lengths = varlen_lengths(3 + 1000, n, 1, max_len)
    return random_inputs(f"c4_varlen_N{n}_H{H}", 3, 1, sum(lengths), H, lengths=lengths)


def c5_collinear(T: int = 16384) -> KdaInputs:
    return near_collinear(4, T=T)
