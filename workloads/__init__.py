"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

This package only draws tree structures and random tensors. It holds none of the
method's arithmetic (no positions, no masks, no attention, no decision formula):
the HIP library and the CPU oracle each derive those on their own from what is
drawn here.
"""
from .configs import (  # noqa: F401
    Forward,
    Workload,
    Decisions,
    TreeDesc,
    make_config,
    CONFIG_NAMES,
)
