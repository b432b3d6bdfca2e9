"""Pins of the oracle's clipped policy loss (token-mean aggregated) and its gradient
with respect to the per-token log-probs: hand-worked cases on both sides of the clip
range, the on-policy closed form, finite differences and torch autograd of the
gradient, ignored rows and the normaliser."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import flce_ref as ref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
V, IGN = 1000, -100


def _worked():
    with open(os.path.join(GOLDEN, "policy_loss_worked.json")) as f:
        return json.load(f)


def test_hand_worked_cases():
    g = _worked()
    for c in g["cases"]:
        old = np.array([g["old_logprob"]])
        lp = old + np.log(c["ratio"])
        loss, clipped, total, n, n_clip, mean = ref.policy_loss(
            lp, old, np.array([c["adv"]]), np.array([3]), V, IGN, c["eps_low"], c["eps_high"])
        assert loss[0] == pytest.approx(c["loss"], abs=1e-12), c
        assert bool(clipped[0]) == c["clipped"], c
        assert (n, n_clip) == (1, int(c["clipped"]))
        assert mean == pytest.approx(c["loss"], abs=1e-12)


def test_on_policy_closed_form():
    """old_logprob = logprob (or None): every ratio is 1, inside any clip range, so the
    loss is -A per token, nothing is clipped and the gradient is -A / N."""
    rng = np.random.default_rng(5)
    M = 50
    lp = -rng.exponential(2.0, M)
    A = rng.standard_normal(M)
    t = rng.integers(0, V, M)
    t[[3, 17, 40]] = IGN
    valid = t != IGN
    for old in (None, lp.copy()):
        loss, clipped, total, n, n_clip, mean = ref.policy_loss(lp, old, A, t, V, IGN, 0.2, 0.28)
        np.testing.assert_allclose(loss[valid], -A[valid], rtol=0, atol=1e-15)
        assert not clipped.any() and n == M - 3 and n_clip == 0
        assert mean == pytest.approx(-A[valid].sum() / n, rel=1e-13)
        gr = ref.policy_loss_grad(lp, old, A, t, V, IGN, 0.2, 0.28, n)
        np.testing.assert_allclose(gr[valid], -A[valid] / n, rtol=1e-13)
        assert np.all(gr[~valid] == 0)


def _random(seed, M=64):
    rng = np.random.default_rng(seed)
    lp = -rng.exponential(2.0, M)
    old = lp + rng.normal(0.0, 0.3, M)   # ratios spread over both sides of the range
    A = rng.standard_normal(M)
    t = rng.integers(0, V, M)
    t[rng.random(M) < 0.1] = IGN
    return lp, old, A, t


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_gradient_by_finite_differences(seed):
    lp, old, A, t = _random(seed)
    el, eh = 0.2, 0.28
    _, clipped, _, n, _, _ = ref.policy_loss(lp, old, A, t, V, IGN, el, eh)
    g = ref.policy_loss_grad(lp, old, A, t, V, IGN, el, eh, n)
    r = np.exp(lp - old)
    h = 1e-6
    for m in range(len(lp)):
        # skip tokens within reach of a clip boundary (the loss has a kink there)
        if min(abs(r[m] - (1 - el)), abs(r[m] - (1 + eh))) < 1e-4:
            continue
        up, dn = lp.copy(), lp.copy()
        up[m] += h
        dn[m] -= h
        fd = (ref.policy_loss(up, old, A, t, V, IGN, el, eh)[5] -
              ref.policy_loss(dn, old, A, t, V, IGN, el, eh)[5]) / (2 * h)
        assert fd == pytest.approx(g[m], abs=1e-9), m


def test_gradient_against_torch_autograd():
    """torch autograd of the surrogate written with torch.clamp / torch.minimum (a
    library derivative, not the oracle's closed form)."""
    lp, old, A, t = _random(7, M=200)
    el, eh = 0.2, 0.2
    _, _, _, n, _, mean = ref.policy_loss(lp, old, A, t, V, IGN, el, eh)
    g = ref.policy_loss_grad(lp, old, A, t, V, IGN, el, eh, n)
    x = torch.tensor(lp, dtype=torch.float64, requires_grad=True)
    r = torch.exp(x - torch.tensor(old))
    At = torch.tensor(A)
    obj = torch.minimum(r * At, torch.clamp(r, 1 - el, 1 + eh) * At)
    mask = torch.tensor(t != IGN, dtype=torch.float64)
    L = -(obj * mask).sum() / n
    L.backward()
    assert float(L.detach()) == pytest.approx(mean, rel=1e-12)
    np.testing.assert_allclose(g, x.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_wide_clip_range_is_importance_weighted_policy_gradient():
    lp, old, A, t = _random(11)
    valid = t != IGN
    _, clipped, _, n, n_clip, mean = ref.policy_loss(lp, old, A, t, V, IGN, 1.0, 1e9)
    assert n_clip == 0
    r = np.exp(lp - old)
    assert mean == pytest.approx(-(r * A)[valid].sum() / n, rel=1e-12)


def test_normaliser_and_empty_batch():
    lp, old, A, t = _random(13)
    _, _, total, n, _, mean = ref.policy_loss(lp, old, A, t, V, IGN, 0.2, 0.2)
    _, _, total2, n2, _, mean2 = ref.policy_loss(lp, old, A, t, V, IGN, 0.2, 0.2, denominator=4096)
    assert total2 == total and n2 == n and mean2 == pytest.approx(total / 4096, rel=1e-14)
    g = ref.policy_loss_grad(lp, old, A, t, V, IGN, 0.2, 0.2, n)
    g2 = ref.policy_loss_grad(lp, old, A, t, V, IGN, 0.2, 0.2, 4096)
    np.testing.assert_allclose(g2 * 4096, g * n, rtol=1e-13)
    # nothing valid: NaN mean, zero gradient
    tt = np.full(len(t), IGN)
    _, _, total, n, _, mean = ref.policy_loss(lp, old, A, tt, V, IGN, 0.2, 0.2)
    assert n == 0 and total == 0 and np.isnan(mean)
    assert np.all(ref.policy_loss_grad(lp, old, A, tt, V, IGN, 0.2, 0.2, 0) == 0)


# --- planted mistakes: each must fail at least one of the pins above -------------
import inspect  # noqa: E402
import types  # noqa: E402

_SRC = inspect.getsource(ref)
MUTANTS = {
    "min_to_max": ("loss = np.where(valid, -np.minimum(unclipped, clipped), 0.0)",
                   "loss = np.where(valid, -np.maximum(unclipped, clipped), 0.0)"),
    "loss_unmasked": ("loss = np.where(valid, -np.minimum(unclipped, clipped), 0.0)",
                      "loss = -np.minimum(unclipped, clipped)"),
    "eps_swapped": ("c = np.minimum(np.maximum(r, 1.0 - float(eps_low)), 1.0 + float(eps_high))",
                    "c = np.minimum(np.maximum(r, 1.0 - float(eps_high)), 1.0 + float(eps_low))"),
    "ratio_inverted": ("    r = np.exp(lp - old)\n    c = ", "    r = np.exp(old - lp)\n    c = "),
    "tie_counts_as_clipped": ("is_clipped = valid & (clipped < unclipped)",
                              "is_clipped = valid & (clipped <= unclipped)"),
    "grad_sign": ("g[keep] = -r[keep] * np.asarray(advantages, np.float64)[keep] / float(N)",
                  "g[keep] = r[keep] * np.asarray(advantages, np.float64)[keep] / float(N)"),
    "grad_keeps_clipped": ("keep = valid & ~is_clipped", "keep = valid"),
    "grad_drops_ratio": ("g[keep] = -r[keep] * np.asarray(advantages, np.float64)[keep] / float(N)",
                         "g[keep] = -np.asarray(advantages, np.float64)[keep] / float(N)"),
    "mean_over_all_rows": ("N = float(denominator) if denominator > 0 else float(n)",
                           "N = float(denominator) if denominator > 0 else float(len(valid))"),
}


def _mutant(old, new):
    assert _SRC.count(old) == 1, f"mutation site not found: {old}"
    mod = types.ModuleType("flce_ref_policy_mutant")
    exec(compile(_SRC.replace(old, new), "flce_ref_policy_mutant", "exec"), mod.__dict__)
    return mod


def _pins_pass(m):
    """True iff the module passes every pin of this file."""
    global ref
    saved = ref
    ref = m
    try:
        for fn in (test_hand_worked_cases, test_on_policy_closed_form,
                   test_gradient_against_torch_autograd,
                   test_wide_clip_range_is_importance_weighted_policy_gradient,
                   test_normaliser_and_empty_batch):
            fn()
        for seed in (1, 2, 3):
            test_gradient_by_finite_differences(seed)
        return True
    except AssertionError:
        return False
    finally:
        ref = saved


def test_the_real_oracle_passes_the_pins():
    assert _pins_pass(ref)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    assert not _pins_pass(_mutant(*MUTANTS[name])), f"mutant {name} passed every pin"
