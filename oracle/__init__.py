"""CPU oracle of the routed MoE FFN layer -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy code that computes the layer from its definition.
Only `tests/`, the smoke check in `__graft_entry__.py` and the CPU-baseline leg of
`bench.py` may import it.  The HIP library and its Python binding never do, and
the oracle shares no code with them: the only thing both sides use is the seeded
input generator in `workloads/`, which holds none of the layer's arithmetic.

Modules:
  formats -- exact bf16 / fp8 e4m3fn decoding from the format definitions;
  moe     -- router, top-k softmax, permutation, expert FFN, combine, layer;
  brute   -- per-token dense evaluation without any permutation (tiny inputs).

Parity status: every function here is pinned by a `-m "not gpu"` test against
something other than itself (library routines, closed forms, brute force,
invariants).  The whole-layer values are not printed on the pages, so they are
pinned by the brute-force evaluation and the invariants rather than by a worked
example from the pages.
"""
from . import formats, moe, brute  # noqa: F401
