"""CPU oracle for the Agent Attention forward -- test infrastructure only.

Imported by tests/, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.
"""
from .agent_oracle import (aggregate, backward, broadcast, dwc, forward,  # noqa: F401
                           module_forward, pool_agents, pool_agents_backward, round_to_format,
                           softmax_backward, softmax_last, window_bounds)
