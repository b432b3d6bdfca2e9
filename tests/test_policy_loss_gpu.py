"""GPU parity of the clipped policy loss on the per-token log-probs against the fp64
oracle: per-token loss, clip flags, the fp64 reductions, the gradient, the caller's
normaliser, the on-policy case, bitwise repeatability, and the gradient fed through
flce_backward end to end.  The kernel computes each token in fp64, as the oracle does,
so both take the clip decision in the same precision; the inputs keep every ratio at
least 1e-6 away from the clip boundaries, where a last-ulp difference in exp could
flip it."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
IGN = -100


def _draw(seed, M, V=50257, spread=0.4, ignore_frac=0.1, eps=(0.2, 0.28)):
    rng = np.random.default_rng(np.random.SeedSequence([2026, 77, seed]))
    lp = (-rng.exponential(2.0, M)).astype(np.float32)
    old = (lp + rng.normal(0.0, spread, M)).astype(np.float32)
    adv = rng.standard_normal(M).astype(np.float32)
    adv[rng.random(M) < 0.02] = 0.0
    t = rng.integers(0, V, M)
    t[rng.random(M) < ignore_frac] = IGN
    # keep the ratios off the clip boundaries (see the module docstring)
    r = np.exp(lp.astype(np.float64) - old.astype(np.float64))
    for b in (1 - eps[0], 1 + eps[1]):
        near = np.abs(r - b) < 1e-6
        old[near] = np.float32(old[near] - np.float32(1e-3))
    return lp, old, adv, t


def _dev(*arrs):
    import torch
    return [None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs]


def _run(lp, old, adv, t, V, el, eh, den=0.0):
    import torch
    from log_prob_amd import flce
    dlp, dold, dadv, dt = _dev(lp, old, adv, t)
    ptl, clip, out = flce.policy_loss_reduce(dlp, dold, dadv, dt, V, IGN, el, eh, den)
    g = flce.policy_loss_grad(dlp, dold, dadv, dt, V, out, IGN, el, eh, den)
    torch.cuda.synchronize()
    return ptl.cpu().numpy(), clip.cpu().numpy().astype(bool), out.cpu().numpy(), g.cpu().numpy()


def _check(lp, old, adv, t, V, el, eh, den, name):
    ptl, clip, out, g = _run(lp, old, adv, t, V, el, eh, den)
    o_old = None if old is None else old.astype(np.float64)
    loss, is_clip, total, n, n_clip, mean = ref.policy_loss(
        lp.astype(np.float64), o_old, adv.astype(np.float64), t, V, IGN, el, eh, den)
    N = den if den > 0 else n
    gr = ref.policy_loss_grad(lp.astype(np.float64), o_old, adv.astype(np.float64), t, V, IGN,
                              el, eh, N)
    # per-token values: fp64 on both sides, then one rounding to fp32 on the GPU
    np.testing.assert_allclose(ptl, loss, rtol=2e-7, atol=1e-30, err_msg=name)
    np.testing.assert_array_equal(clip, is_clip, err_msg=name)
    assert int(out[1]) == n and int(out[2]) == n_clip, name
    assert out[0] == pytest.approx(total, rel=1e-12, abs=1e-12), name
    if N > 0:
        assert out[3] == pytest.approx(mean, rel=1e-12, abs=1e-15), name
    else:
        assert np.isnan(out[3]), name
    np.testing.assert_allclose(g, gr, rtol=2e-7, atol=1e-30, err_msg=name)
    return out


@pytest.mark.parametrize("seed,M,eps", [(1, 5000, (0.2, 0.2)), (2, 1023, (0.2, 0.28)),
                                        (3, 1, (0.1, 0.2)), (4, 70001, (0.2, 0.28))])
def test_policy_loss_matches_oracle(seed, M, eps):
    V = 50257
    lp, old, adv, t = _draw(seed, M, V, eps=eps)
    print(f"[policy] seed={seed} M={M} eps={eps}", flush=True)
    out = _check(lp, old, adv, t, V, eps[0], eps[1], 0.0, f"seed{seed}")
    if M > 100:
        assert 0 < out[2] < out[1]      # both branches of the minimum are exercised


def test_policy_loss_normaliser_and_on_policy():
    V = 32000
    lp, old, adv, t = _draw(5, 3000, V)
    _check(lp, old, adv, t, V, 0.2, 0.2, 8192.0, "normaliser")
    # on-policy: ratio 1, loss -A, nothing clipped, gradient -A / N
    ptl, clip, out, g = _run(lp, None, adv, t, V, 0.2, 0.2)
    valid = t != IGN
    assert not clip.any() and int(out[2]) == 0
    np.testing.assert_array_equal(ptl[valid], -adv[valid])
    np.testing.assert_allclose(g[valid], -adv[valid].astype(np.float64) / valid.sum(), rtol=2e-7)
    assert np.all(g[~valid] == 0) and np.all(ptl[~valid] == 0)


def test_policy_loss_nothing_valid_and_repeatable():
    V = 1000
    lp, old, adv, t = _draw(6, 2048, V)
    t[:] = IGN
    ptl, clip, out, g = _run(lp, old, adv, t, V, 0.2, 0.2)
    assert int(out[1]) == 0 and out[0] == 0 and np.isnan(out[3])
    assert np.all(g == 0) and np.all(ptl == 0) and not clip.any()
    # an empty batch of tokens: sums and counts 0, the mean NaN (0 / 0), or 0 over a
    # positive normaliser
    e = np.zeros(0, np.float32)
    ptl, clip, out, g = _run(e, e, e, np.zeros(0, np.int64), V, 0.2, 0.2)
    assert ptl.size == 0 and g.size == 0 and list(out[:3]) == [0, 0, 0] and np.isnan(out[3])
    _, _, out, _ = _run(e, e, e, np.zeros(0, np.int64), V, 0.2, 0.2, den=64.0)
    assert out[3] == 0.0
    lp, old, adv, t = _draw(7, 100003, V)
    a = _run(lp, old, adv, t, V, 0.2, 0.28)
    b = _run(lp, old, adv, t, V, 0.2, 0.28)
    for x, y in zip(a, b):
        assert np.array_equal(x, y, equal_nan=True)


def test_policy_loss_gradient_through_backward():
    """forward -> policy loss -> grad_logprob -> flce_backward, against the oracle's
    backward driven by the oracle's gradient of the same loss."""
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("policy_e2e", 601, 600, 320, 1500, ignore_frac=0.05, grad_mode="none")
    X, W, t, _, _ = gu.to_dev(c)
    lp, lse, ent = flce.forward(X, W, t, c.ignore_index, c.scale, False)
    rng = np.random.default_rng(np.random.SeedSequence([2026, 78]))
    lp_h = lp.cpu().numpy()
    old_h = (lp_h + rng.normal(0.0, 0.3, c.M)).astype(np.float32)
    adv_h = rng.standard_normal(c.M).astype(np.float32)
    old, adv = _dev(old_h, adv_h)
    _, _, out = flce.policy_loss_reduce(lp, old, adv, t, c.V, c.ignore_index, 0.2, 0.28)
    g = flce.policy_loss_grad(lp, old, adv, t, c.V, out, c.ignore_index, 0.2, 0.28)
    dX, dW = flce.backward(X, W, t, lse, None, g, None, c.ignore_index, c.scale)
    torch.cuda.synchronize()
    # oracle: the same loss on the oracle's own log-probs, its gradient, its backward
    o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, False)
    _, _, _, n, _, _ = ref.policy_loss(o["logprob"], old_h.astype(np.float64),
                                       adv_h.astype(np.float64), c.targets, c.V, c.ignore_index,
                                       0.2, 0.28)
    g_ref = ref.policy_loss_grad(o["logprob"], old_h.astype(np.float64), adv_h.astype(np.float64),
                                 c.targets, c.V, c.ignore_index, 0.2, 0.28, n)
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, g_ref, None)
    # the two sides take the same clip decisions: their log-probs differ by far less
    # than any ratio's distance to a clip boundary in this case (asserted, not assumed)
    gg = g.cpu().numpy()
    assert np.array_equal(gg == 0, g_ref == 0)
    gu.check_grads(gu.bf16_to_np(dX), gu.bf16_to_np(dW), rdX, rdW, "policy_e2e")


def test_policy_loss_targets_beyond_32_bits():
    """Targets whose low 32 bits name a vocabulary column but which lie outside [0, V)
    as 64-bit values leave their tokens out of the loss, the counts and the gradient."""
    V = 50257
    lp, old, adv, t = _draw(8, 4000, V)
    rows = np.array([0, 17, 2047, 3999])
    t[rows] = np.array([2**32 + 5, -2**32 + 7, 2**63 - 1, -2**63], dtype=np.int64)
    print("[policy] 64-bit targets", flush=True)
    out = _check(lp, old, adv, t, V, 0.2, 0.28, 0.0, "t64")
    assert int(out[1]) == int(np.sum((t != IGN) & (t >= 0) & (t < V)))
    ptl, _, _, g = _run(lp, old, adv, t, V, 0.2, 0.28)
    assert np.all(ptl[rows] == 0) and np.all(g[rows] == 0)
