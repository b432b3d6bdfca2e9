"""torch.autograd binding of libflce: per-token log-probs (and entropy) of a linear
LM head as a differentiable op, in the manner of the autograd function the
Liger-Kernel commit "native Blackwell tensor-parallel fused scaled linear
cross-entropy" lists among its code entry points ("Code entry points", PyTorch
autograd row).

Argument marshalling only: the forward is one flce.forward call, the backward one
flce.backward call with the incoming gradients as grad_logprob / grad_entropy.  The
logits are never materialised; the backward recomputes them on the GPU.
"""
from __future__ import annotations

import torch

from . import flce


class FusedLinearLogprob(torch.autograd.Function):
    """(logprob, entropy) = f(X, W) for targets; entropy only with compute_entropy."""

    @staticmethod
    def forward(ctx, X, W, targets, ignore_index: int, scale: float, compute_entropy: bool):
        lp, lse, ent = flce.forward(X, W, targets, ignore_index, scale, compute_entropy)
        ctx.save_for_backward(X, W, targets, lse, ent)
        ctx.cfg = (int(ignore_index), float(scale))
        # an unused output's gradient arrives as None rather than a tensor of zeros
        ctx.set_materialize_grads(False)
        if compute_entropy:
            return lp, ent
        return lp

    @staticmethod
    def backward(ctx, g_lp, g_ent=None):
        X, W, targets, lse, ent = ctx.saved_tensors
        ignore_index, scale = ctx.cfg
        glp = None if g_lp is None else g_lp.float().contiguous()
        gent = None if g_ent is None else g_ent.float().contiguous()
        dX = dW = None
        if ctx.needs_input_grad[0] or ctx.needs_input_grad[1]:
            dX, dW = flce.backward(X, W, targets, lse, ent if gent is not None else None, glp,
                                   gent, ignore_index, scale)
        return (dX if ctx.needs_input_grad[0] else None,
                dW if ctx.needs_input_grad[1] else None, None, None, None, None)


def linear_logprob(X, W, targets, ignore_index: int = -100, scale: float = 1.0,
                   compute_entropy: bool = False):
    """Differentiable per-token log-probs of targets under softmax(scale X W^T), and the
    per-token entropy when compute_entropy is set.  X [M, H], W [V, H] bf16 on the GPU,
    targets [M] int64; rows whose target is ignore_index or outside [0, V) give 0."""
    return FusedLinearLogprob.apply(X, W, targets, ignore_index, scale, compute_entropy)
