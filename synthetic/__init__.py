"""Seeded synthetic inputs shared by the oracle's tests and the HIP path (no layer arithmetic)."""
from .gen import (CONFIGS, CONFIG_ORDER, GRProblem, MoEConfig, Problem, make_audit_tensor,  # noqa: F401
                  make_gr_problem, make_problem)
