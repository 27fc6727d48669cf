"""CPU reference for the attention forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never does, and this
package imports nothing from it: the two share no code. The only module both
sides use is the seeded input generator, which holds none of the method's
arithmetic.

Contents
  attn_oracle(q, k, v, causal, scale, rows=None) -> (O, LSE)
      fp64 three-pass attention in C (``attn_oracle.c``), parallel over rows.
  attn_bwd_oracle(q, k, v, dout, causal, scale, qrows=None, krows=None) -> (dQ, dK, dV)
      fp64 attention gradients in C (``attn_bwd_oracle.c``), written out from
      their definitions; dQ per query row, dK and dV per key row.
  row_softmax(x) -> y
      fp64 three-pass row softmax of an M x N matrix (``softmax.py``), the
      pages' Kernel 2.
  attn_two_pass_np / attn_online_np
      tiny pure-NumPy fp64 variants used to pin the C oracle (brute force on
      small inputs); see ``variants.py``.

Parity status of each function is listed in ``variants.py`` and in the tests
that pin them (``tests/test_oracle.py``).
"""
from .native import (attn_oracle, oracle_threads, build_oracle, compile_oracle,  # noqa: F401
                     open_oracle_library, library_path, attn_bwd_oracle,
                     open_bwd_oracle_library, bwd_library_path)
from .variants import attn_two_pass_np, attn_online_np  # noqa: F401
from .softmax import row_softmax  # noqa: F401
