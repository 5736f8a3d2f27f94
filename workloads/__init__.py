"""Seeded synthetic workloads shared by the oracle tests, the GPU tests and the
benchmark.  Holds input generation only."""
from .gen import (CONFIGS, DEFAULT_BENCH, SMALL, Recipe, Shape, Workload, custom, generate, make_config,
                  router_logits)

__all__ = ["CONFIGS", "DEFAULT_BENCH", "SMALL", "Recipe", "Shape", "Workload", "custom",
           "generate", "make_config", "router_logits"]
