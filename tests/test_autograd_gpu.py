"""The autograd binding: gradients through linear_logprob equal a direct flce.backward
call bit for bit and match the fp64 oracle; an unused entropy output costs no
entropy gradient."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_autograd_matches_direct_backward_and_oracle():
    import torch
    from log_prob_amd import flce
    from log_prob_amd.autograd import linear_logprob
    c = inputs.make_case("ag", 601, 600, 320, 1500, ignore_frac=0.05, grad_mode="normal")
    X, W, t, glp, gent = gu.to_dev(c)
    Xg = X.clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    lp, ent = linear_logprob(Xg, Wg, t, c.ignore_index, c.scale, compute_entropy=True)
    ((lp * glp).sum() + (ent * gent).sum()).backward()
    _, lse, ent0 = flce.forward(X, W, t, c.ignore_index, c.scale, True)
    dX, dW = flce.backward(X, W, t, lse, ent0, glp, gent, c.ignore_index, c.scale)
    torch.cuda.synchronize()
    assert torch.equal(Xg.grad, dX) and torch.equal(Wg.grad, dW)
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                            c.grad_entropy)
    gu.check_grads(gu.bf16_to_np(Xg.grad), gu.bf16_to_np(Wg.grad), rdX, rdW, "autograd")


def test_autograd_logprob_only_and_unused_entropy():
    import torch
    from log_prob_amd import flce
    from log_prob_amd.autograd import linear_logprob
    c = inputs.make_case("ag2", 602, 300, 64, 700, grad_mode="normal_lp")
    X, W, t, glp, _ = gu.to_dev(c)
    Xg = X.clone().requires_grad_(True)
    Wg = W.clone().requires_grad_(True)
    lp = linear_logprob(Xg, Wg, t, c.ignore_index, c.scale)
    (lp * glp).sum().backward()
    _, lse, _ = flce.forward(X, W, t, c.ignore_index, c.scale, False)
    dX, dW = flce.backward(X, W, t, lse, None, glp, None, c.ignore_index, c.scale)
    torch.cuda.synchronize()
    assert torch.equal(Xg.grad, dX) and torch.equal(Wg.grad, dW)
    # entropy computed but not used in the loss: the same gradients as logprob alone
    Xg2 = X.clone().requires_grad_(True)
    Wg2 = W.clone().requires_grad_(True)
    lp2, _ent = linear_logprob(Xg2, Wg2, t, c.ignore_index, c.scale, compute_entropy=True)
    (lp2 * glp).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(Xg2.grad, dX) and torch.equal(Wg2.grad, dW)
