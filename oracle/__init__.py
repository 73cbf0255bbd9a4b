"""Plain fp64 CPU oracle for SALAD's hybrid attention forward and backward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers or tables);
the two meet only in the seeded input generator, which holds none of the
method's arithmetic.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
library routines (torch CPU ``scaled_dot_product_attention`` in fp64, numpy
``argsort``), exact rational / high-precision brute force, invariants and,
for the backward pass, central finite differences of the forward.
"""

from . import salad_backward as _bwd
from . import salad_oracle as _fwd
from .salad_backward import *  # noqa: F401,F403
from .salad_oracle import *  # noqa: F401,F403

__all__ = list(_fwd.__all__) + list(_bwd.__all__)
