"""CPU float64 oracle for PISA's hot path -- TEST INFRASTRUCTURE ONLY.

Only tests, the smoke check and the benchmark's CPU-baseline leg may import this
package. The HIP library and its Python binding never import or call it.
"""
from .pisa_oracle import *  # noqa: F401,F403
