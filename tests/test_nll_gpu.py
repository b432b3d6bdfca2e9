"""GPU parity of the scalar cross-entropy reductions (sum / count / mean NLL over the
valid rows) and of the mean-NLL log-prob gradient, against the fp64 oracle."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _targets(rng, M, V, ignore_index):
    t = rng.integers(0, V, M)
    t[rng.random(M) < 0.07] = ignore_index
    t[rng.random(M) < 0.01] = V + 5       # out of range: not valid
    t[rng.random(M) < 0.01] = -1
    return t


@pytest.mark.parametrize("M", [1, 1023, 1024, 1025, 3_000_001])
def test_nll_reduce_matches_oracle_sum(M):
    """The reduction alone, on stored log-probs: fp64 sums in a different order agree
    to rounding, the count is exact, and a second call is bitwise equal."""
    import torch
    from log_prob_amd import flce
    rng = np.random.default_rng(1000 + M)
    V, ign = 50257, -100
    lp = -(rng.standard_exponential(M) * 3.0).astype(np.float32)
    t = _targets(rng, M, V, ign)
    print(f"[nll] reduce M={M}", flush=True)
    out = flce.nll_reduce(torch.from_numpy(lp).cuda(), torch.from_numpy(t).cuda(), V, ign)
    again = flce.nll_reduce(torch.from_numpy(lp).cuda(), torch.from_numpy(t).cuda(), V, ign)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    total, n, mean = ref.nll_reduce(lp, t, V, ign)
    assert got[1] == n
    np.testing.assert_allclose(got[0], total, rtol=1e-12, atol=0)
    if n:
        np.testing.assert_allclose(got[2], mean, rtol=1e-12, atol=0)
    assert torch.equal(out, again)


def test_nll_reduce_no_valid_row():
    import torch
    from log_prob_amd import flce
    lp = torch.tensor([-1.0, -2.0, -3.0], device="cuda")
    t = torch.tensor([-100, -100, 9], device="cuda")
    got = flce.nll_reduce(lp, t, 9).cpu().numpy()
    assert got[0] == 0.0 and got[1] == 0.0 and np.isnan(got[2])
    g = flce.nll_mean_grad(t, 9, flce.nll_reduce(lp, t, 9)).cpu().numpy()
    assert np.all(g == 0.0)


def test_mean_nll_loss_forward_backward():
    """The scalar loss path on the device: forward -> mean NLL -> its log-prob
    gradient -> backward, against the oracle's loss and gradients."""
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("nll_e2e", 301, 600, 320, 1500, ignore_frac=0.05, grad_mode="none")
    c.targets[::37] = c.V + 1                     # out of range: ignored too
    X, W, t, _, _ = gu.to_dev(c)
    lp, lse, _ = flce.forward(X, W, t, c.ignore_index, c.scale, False)
    red = flce.nll_reduce(lp, t, c.V, c.ignore_index)
    g = flce.nll_mean_grad(t, c.V, red, c.ignore_index)
    dX, dW = flce.backward(X, W, t, lse, None, g, None, c.ignore_index, c.scale)
    torch.cuda.synchronize()
    o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, False)
    total, n, mean = ref.nll_reduce(o["logprob"], c.targets, c.V, c.ignore_index)
    got = red.cpu().numpy()
    assert got[1] == n
    # |mean error| <= max |logprob error| <= the forward tolerance
    assert abs(got[2] - mean) <= gu.FWD_ATOL, (got[2], mean)
    rg = ref.nll_mean_grad(c.targets, c.V, c.ignore_index, n)
    assert np.array_equal(g.cpu().numpy(), rg.astype(np.float32))
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale,
                            rg.astype(np.float32), None)
    gu.check_grads(gu.bf16_to_np(dX), gu.bf16_to_np(dW), rdX, rdW, "nll_e2e")
