"""Autograd integration of the blocked vocabulary-projection cross-entropy.

The forward saves only the per-token normaliser lse [N] (fp32) and references
to H, W and the labels, never a slice of the N x V logits. The backward
recomputes the logits chunk by chunk from that normaliser in the library's
kernels ("Flattening Every Memory Peak in Long-Context Mixture-of-Experts
Training", full-text page, section 3.2: the backward recomputes strip by strip
from the saved normaliser). Because nothing larger than lse is saved, the
memory bound holds unchanged when the loss sits inside an activation
checkpoint and its forward is rerun during the backward (same page, section 2:
each operator's bound must survive checkpoint recomputation).

The upstream gradient reaches the library as a one-element device tensor, so
neither direction synchronises with the host. Gradients come out of the
library in fp32; autograd casts them to the dtype of H and W when those are
bf16, as it does for any function whose gradient dtype differs from its
input's.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import IGNORE_INDEX, backward, forward


class _VocabProjectionCE(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, labels, R, ignore_index, workspace):
        loss, lse = forward(H, W, labels, R, ignore_index, workspace)
        ctx.save_for_backward(H, W, labels, lse)
        ctx.R = R
        ctx.ignore_index = ignore_index
        ctx.workspace = workspace
        return loss

    @staticmethod
    def backward(ctx, dloss):
        H, W, labels, lse = ctx.saved_tensors
        need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_h or need_w):
            return None, None, None, None, None, None
        d = dloss.detach().reshape(1).to(torch.float32).contiguous()
        dH, dW = backward(H, W, labels, lse, d, ctx.R, ctx.ignore_index,
                          ctx.workspace)
        return (dH if need_h else None, dW if need_w else None,
                None, None, None, None)


def cross_entropy(H: torch.Tensor, W: torch.Tensor, labels: torch.Tensor,
                  R: int, ignore_index: int = IGNORE_INDEX,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Mean cross-entropy of softmax(H W^T) against labels as a
    differentiable scalar: gradients flow to H [N, d] and W [V, d].

    R is the number of vocabulary shards the product is blocked over (the
    result does not depend on it beyond fp32 summation order). A workspace of
    at least workspace_bytes(N, d, V, R) bytes may be passed to reuse one
    buffer across steps; otherwise each call allocates its own through
    torch's allocator.
    """
    return _VocabProjectionCE.apply(H, W, labels, R, ignore_index, workspace)
