"""fp64 CPU oracle for the fused decode-MLP path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
package.  It shares no code with the HIP library or its Python binding.
"""
from .decode_mlp import *  # noqa: F401,F403
