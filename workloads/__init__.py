"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests
and the bench; holds none of the method's arithmetic."""

from .configs import (BLOCK_SIZE, POISON, Case, Layout, Spec, build_layout, config, custom,
                      make_case, sequences_subset, spec_decode)

__all__ = ["BLOCK_SIZE", "POISON", "Case", "Layout", "Spec", "build_layout", "config", "custom",
           "make_case", "sequences_subset", "spec_decode"]
