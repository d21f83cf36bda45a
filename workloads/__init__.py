"""Seeded synthetic workloads shared by the oracle tests, the GPU parity tests and the bench.

Holds only input generation (no arithmetic of the method)."""
from .gen import (LayerShape, Workload, WORKLOADS, NANO, H8B, TINY, make_inputs,
                  seqlens_of, round_bf16, small_shape_inputs, group_channels, slice_group,
                  inproj_inputs)

__all__ = ["LayerShape", "Workload", "WORKLOADS", "NANO", "H8B", "TINY", "make_inputs",
           "seqlens_of", "round_bf16", "small_shape_inputs", "group_channels", "slice_group",
           "inproj_inputs"]
