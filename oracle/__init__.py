"""CPU oracle for the Agent Attention forward -- test infrastructure only.

Imported by tests/, the smoke check and the benchmark's CPU-baseline leg;
never by the product path.
"""
from .agent_oracle import (aggregate, backward, broadcast, dwc, forward,  # noqa: F401
                           pool_agents, pool_agents_backward, softmax_backward, softmax_last,
                           window_bounds)
