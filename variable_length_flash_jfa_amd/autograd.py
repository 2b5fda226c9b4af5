"""torch.autograd wrapper over the C ABI forward and backward."""
from __future__ import annotations

import torch

from . import _binding


class _JaggedAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, offsets, broadcast_q, causal, scale):
        o, lse = _binding.fwd(q, k, v, offsets, broadcast_q=broadcast_q, causal=causal, scale=scale)
        ctx.save_for_backward(q, k, v, offsets, o, lse)
        ctx.flags = (broadcast_q, causal, scale)
        return o

    @staticmethod
    def backward(ctx, d_o):
        q, k, v, offsets, o, lse = ctx.saved_tensors
        broadcast_q, causal, scale = ctx.flags
        dq, dk, dv = _binding.bwd(q, k, v, offsets, o, lse, d_o.contiguous(),
                                  broadcast_q=broadcast_q, causal=causal, scale=scale)
        return dq, dk, dv, None, None, None, None


def jagged_attention(q, k, v, offsets, *, broadcast_q: bool, causal: bool = False, scale=None):
    """Differentiable jagged flash attention on packed bf16 tensors."""
    return _JaggedAttention.apply(q, k, v, offsets, broadcast_q, causal, scale)
