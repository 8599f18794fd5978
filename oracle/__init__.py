"""CPU oracle for the fused LM-head log-prob — TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg may import or call
anything in this package.  The product path (the HIP library and its Python binding) never does;
the two share no code: only the seeded input generators in ``synth`` serve both.

Contents:
- ``fp64``  : the plain definition, written out in numpy float64 (full logits per row block,
              log-softmax over the whole vocabulary, gather, entropy, and the analytic backward).
- ``brute`` : the same definition in pure Python scalars with correctly rounded sums
              (``math.fsum``) for tiny shapes; a second, independent implementation used to pin
              ``fp64``.

Parity status of each function is stated in its module header.
"""
from . import fp64, brute  # noqa: F401
from .fp64 import forward, forward_rows, backward, grad_weight_rows, grad_hidden_rows, to_f64  # noqa: F401
