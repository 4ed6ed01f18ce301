"""CPU oracle for the Agent Attention forward -- test infrastructure only.

Imported by tests/, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.
"""
from .agent_oracle import (aggregate, broadcast, dwc, forward, pool_agents,  # noqa: F401
                           softmax_last, window_bounds)
