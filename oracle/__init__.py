"""fp64 CPU oracle for masked scaled dot-product attention over a CSR mask.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this package; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run it. It shares no code with the HIP path.

Two evaluations of the same definition are provided:

* :mod:`oracle.dense` -- the definition itself: a dense score matrix with -inf
  outside the pattern, a row softmax and a dense product with V, evaluated
  with NumPy GEMMs in row chunks (or row by row for sampled rows).
* :mod:`oracle.csr` -- the three sparse steps of the gluon-nlp proposal
  ("Unified Interface/Implementation for Sparse Attention", the three bullet
  points of the opening post): scores at the mask's nonzeros, a softmax over
  each sparse row, and the sparse-times-dense product, in fp64.
* :mod:`oracle.backward` -- the gradients with respect to q, k and v: the chain
  rule through the three steps, and torch autograd (fp64, CPU) of the dense
  definition.
* :mod:`oracle.mask` -- masks given as COO pairs, per-batch key lengths or packed
  variable-length sequences, turned into the CSR pattern and key mask.

Both follow the same conventions (see the module docstrings). Every function
here has a pin in ``tests/test_oracle_pins.py`` other than itself.
"""
from . import dense, csr, backward, mask  # noqa: F401
from .dense import attention_dense, attention_rows, pattern_rows  # noqa: F401
from .csr import sddmm, sparse_softmax, spmm, attention_csr  # noqa: F401
