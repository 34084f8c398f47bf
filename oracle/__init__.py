"""CPU fp64 oracle for exact attention (test infrastructure only).

Only tests/, the smoke check and the bench's CPU-baseline leg use this
package. The HIP library neither imports it nor is imported by it.
"""
from . import attention  # noqa: F401
from . import blocks  # noqa: F401
from . import dropout  # noqa: F401
from . import rope  # noqa: F401
