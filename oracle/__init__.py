"""fp64 CPU oracle for the retention forward pass and its gradients — TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. It shares no code with the HIP path and the HIP path never calls it. Pinned
by tests/test_oracle.py (brute force, closed forms, invariants, library special cases),
tests/test_oracle_backward.py (gradients against central finite differences of the
forward oracle), tests/test_oracle_vector.py (pair decays: reduction to the scalar
oracle, decomposition by coordinate pair, agreement of the forms) and
tests/test_oracle_layer.py (the gated multi-scale layer: explicit loops, identity
projections, head permutation); no function here is left unpinned.
"""
from .retention import *  # noqa: F401,F403
from .retention import __all__ as _fwd_all
from .backward import backward  # noqa: F401
from .vector_decay import *  # noqa: F401,F403
from .vector_decay import __all__ as _vec_all
from .layer import *  # noqa: F401,F403
from .layer import __all__ as _layer_all

__all__ = list(_fwd_all) + ["backward"] + list(_vec_all) + list(_layer_all)
