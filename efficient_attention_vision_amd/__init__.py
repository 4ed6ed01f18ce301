"""Agent Attention forward for AMD Instinct MI355X (gfx950).

O = softmax(scale Q A^T) softmax(scale A K^T) V, where the agents A are the
2-D average pool of Q over the token grid or are supplied by the caller
("Agent Attention: On the Integration of Softmax and Linear Attention",
§4 Agent Transformer).  The computation runs in hand-written HIP kernels of
libagent_attn.so; this package is its thin Python binding.  The shared
library is loaded on first use.
"""
from ._binding import (AgentAttnError, EXPORTED, LIB_PATH, agent_attn_aggregate,  # noqa: F401
                       agent_attn_backward,
                       agent_attn_broadcast, agent_attn_forward, agent_attn_forward_cached,
                       agent_attn_forward_module, agent_attn_module_forward,
                       agent_attn_pool, agent_attn_read_faults, agent_attn_release,
                       agent_attn_set_wait_limit, agent_attn_workspace_bytes, lib)
