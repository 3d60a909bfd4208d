"""BF16 fused attention for AMD MI355X (gfx950) with the duplicate-max
stabilised safe softmax as a switchable mode.

The compute lives in libattn.so (hand-written HIP, C ABI in include/attn.h);
``binding`` marshals torch tensors to it; ``autograd`` wraps it as a
differentiable torch function and a GPT-2-shaped attention layer; ``inputs``
generates the seeded synthetic workloads.
"""
from .binding import (AttnError, abi_version, attn_bwd, attn_bwd_dkdv, attn_bwd_dq, attn_bwd_o32,
                      attn_bwd_workspace_bytes, attn_fwd, attn_fwd_o32, attn_tiecount, backward, forward,
                      fwd_key_tile, status_string, tiecount, workspace_for)

__all__ = ["AttnError", "abi_version", "attn_bwd", "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_o32",
           "attn_bwd_workspace_bytes", "attn_fwd", "attn_fwd_o32", "attn_tiecount", "backward", "forward",
           "fwd_key_tile", "status_string", "tiecount", "workspace_for"]
