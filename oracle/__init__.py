"""CPU oracle for exact blockwise attention with running online-softmax state.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library, its
Python binding) may import, call or link anything in this package.  Only the
test suite, the smoke check of the package entry module and the CPU-baseline
leg of the benchmark use it.

The oracle is plain, slow and written to be checked by eye against the pages
it follows:

* ``oracle.attention`` -- NumPy float64.  The exact definition of attention
  (softmax of scaled logits plus optional causal mask, times V), the partial
  online-softmax state ``(m, l, O)`` over any key subset, the blockwise
  recurrence in the order the pages give it, the log-sum-exp merge of partial
  states, finalisation, the ring schedule and a multi-device ring emulation,
  and shared-prefix fan-out decode.
* ``oracle.brute`` -- pure-Python loops with ``math.fsum`` / ``math.exp``, an
  independent second implementation for tiny inputs.

Every function takes its inputs as float64 arrays holding exactly the values a
GPU kernel receives (bf16 or fp32 values upcast without rounding) and never
rounds intermediate results.
"""

from . import attention, brute  # noqa: F401
