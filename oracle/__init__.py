"""CPU oracle of the KDA forward pass — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import, call, link or execute anything in this package.  The
GPU product path never routes through it, and it shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing).

Contents
  recurrence.py  the oracle proper: fp64 token-by-token recurrence (plain C,
                 OpenMP over (sequence, head)), loaded through ctypes; the
                 per-shard affine map (P, R) of a sequence split into shards,
                 and the fold of consecutive shards' maps.
  chunked.py     a second, independent fp64 CPU form that processes 64-token
                 (or 16/32) chunks with the WY/UT chunk algebra; used only to
                 check the recurrence.
  grad.py        gradients of the forward: fp64 torch autograd through the
                 token recurrence (the definition of the backward), pinned by
                 central finite differences and by the C recurrence.
  chunked.py also holds the chunked backward (reverse-mode chunk algebra), a
                 second form checked against grad.py.
  brute.py       40-digit decimal brute force of the unrolled product form for
                 tiny T; used only to check the recurrence.
  build.py       compiles kda_oracle.c with gcc.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
and ``tests/test_oracle_kcp_pins.py`` / ``tests/test_oracle_grad_pins.py`` against closed forms, brute force,
invariants and special cases, with one
exception stated in the design notes: the gate formula itself (log alpha =
lower_bound * sigmoid(exp(A_log) * (raw_gate + dt_bias))) is a reading, since
the pages never print it, so agreement with FlashKDA's own gate is
"parity unpinned".
"""

from .recurrence import oracle_fwd, oracle_threads, metrics, oracle_shard_affine, oracle_shard_fold  # noqa: F401
