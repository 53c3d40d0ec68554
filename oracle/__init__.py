"""fp64 CPU oracle for AB-Attention block-sparse attention (test infrastructure).

Only the tests, the package's smoke check and the benchmark's CPU-baseline leg
may import this package.  The HIP library never calls it and shares no code
with it.
"""
from .absa_oracle import *  # noqa: F401,F403
from .absa_oracle import __all__ as _base_all
from .fp8_oracle import *  # noqa: F401,F403
from .fp8_oracle import __all__ as _fp8_all
from .cluster_oracle import *  # noqa: F401,F403
from .cluster_oracle import __all__ as _cluster_all

__all__ = list(_base_all) + list(_fp8_all) + list(_cluster_all)
