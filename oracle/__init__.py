"""CPU oracle for SageBwd INT8 attention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The GPU library never calls it and shares no code
with it.  Everything here is plain NumPy on the host, written for a reader to
check against the method's description by eye, not for speed.

Modules
  sage     the SageBwd algorithm (quantise, forward, backward pre-pass,
           backward) with every numeric choice spelled out; also a
           quantisation-off mode in which it must reduce to exact attention.
  fpa      full-precision (float64) attention and its gradients, the
           textbook definition, used as the comparison baseline.
  metrics  cosine similarity, relative L2, relative L1 and RMSE.

Parity status: every function is pinned by CPU tests (tests/test_oracle_*.py)
against closed forms, library routines, finite differences, invariants and
the SageBwd paper's Table 1 trend.  No function is "parity unpinned".
"""
from . import fpa, metrics, sage  # noqa: F401
