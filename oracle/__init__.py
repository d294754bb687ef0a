"""fp64 CPU oracle of the routed MoE layer.  TEST INFRASTRUCTURE ONLY: imported
by the tests, the smoke check and the benchmark's CPU-baseline leg, never by
the library path."""
from . import moe, adapter  # noqa: F401
