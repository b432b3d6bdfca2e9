"""Planted mistakes in a copy of the oracle must each be caught by some pin (CPU only).

Each mutant rewrites one line of the oracle's source (a dropped term, a wrong
sign, a wrong index or operand, a missing scale or mask) and executes it as a
separate module; the real oracle module is never modified.  The pins below are
the ones test_oracle.py applies: closed forms, the pure-Python brute force,
torch float64 autograd, and the zero-sum invariant.
"""
import inspect
import math
import types

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import flce_ref
from tests import test_oracle as pins
from synth import inputs

SRC = inspect.getsource(flce_ref)

MUTANTS = {
    "logprob_sign": ("logprob = np.where(valid, z_t - lse, 0.0)",
                     "logprob = np.where(valid, lse - z_t, 0.0)"),
    "lse_drops_max": ("lse = zmax + np.log(np.exp(Z - zmax[:, None]).sum(axis=1))",
                      "lse = np.log(np.exp(Z - zmax[:, None]).sum(axis=1))"),
    "entropy_unmasked": ("entropy = np.where(valid, -(P * logP).sum(axis=1), 0.0)",
                         "entropy = -(P * logP).sum(axis=1)"),
    "entropy_sign": ("entropy = np.where(valid, -(P * logP).sum(axis=1), 0.0)",
                     "entropy = np.where(valid, (P * logP).sum(axis=1), 0.0)"),
    "dz_softmax_sign": ("dZ = -a[:, None] * P", "dZ = a[:, None] * P"),
    "dz_onehot_dropped": ("dZ[np.arange(R)[valid], t[valid]] += a[valid]", "pass"),
    "dz_entropy_term_dropped": ("dZ += b[:, None] * P * (E[:, None] - Z)", "pass"),
    "dz_entropy_term_sign": ("dZ += b[:, None] * P * (E[:, None] - Z)",
                             "dZ += b[:, None] * P * (Z - E[:, None])"),
    "target_off_by_one": ("z_t = Z[np.arange(R), safe_t]",
                          "z_t = Z[np.arange(R), np.minimum(safe_t + 1, V - 1)]"),
    "grad_unmasked": ("a = np.where(valid, a, 0.0)", "pass"),
    "dx_missing_scale": ("dX[r] = s * (dZ @ Wd)", "dX[r] = dZ @ Wd"),
    "dw_wrong_operand": ("dW += s * (dZ.T @ Xr)", "dW += s * (dZ.T @ Xr[::-1])"),
    "scale_not_applied": ("return s * (Xd @ Wd.T)", "return Xd @ Wd.T"),
    "valid_ignores_range": ("return (t != ignore_index) & (t >= 0) & (t < V)",
                            "return (t != ignore_index)"),
    # mistakes that only a run over several row blocks can show
    "dw_block_overwrites": ("dW += s * (dZ.T @ Xr)", "dW = s * (dZ.T @ Xr)"),
    "dx_rows_block_misplaced": ("out[i:i + step] = s * (o[\"dZ\"] @ Wd)",
                                "out[:len(r)] = s * (o[\"dZ\"] @ Wd)"),
    "forward_block_skips_tail": ("for r0 in range(0, M, step):\n        r = slice(r0, min(M, r0 + step))",
                                 "for r0 in range(0, M - step, step):\n        r = slice(r0, min(M, r0 + step))"),
    "dw_rows_block_misplaced": ("out[i:i + step] = s * (dZc.T @ Xd)",
                                "out[:len(vb)] = s * (dZc.T @ Xd)"),
}


def _mutant(old, new):
    assert SRC.count(old) >= 1, f"mutation site not found: {old}"
    mod = types.ModuleType("flce_ref_mutant")
    exec(compile(SRC.replace(old, new), "flce_ref_mutant", "exec"), mod.__dict__)
    return mod


def _pin_closed_forms(ref):
    for case in pins._golden_cases():
        z = np.array([[pins._eval(e) for e in case["z"]]])
        o = ref.from_logits(z, np.array([case["t"]]), -100, True,
                            grad_logprob=[pins._eval(case["a"])], grad_entropy=[pins._eval(case["b"])])
        assert abs(o["lse"][0] - pins._eval(case["lse"])) <= 1e-9 * max(1, abs(z).max())
        assert abs(o["logprob"][0] - pins._eval(case["logprob"])) <= 1e-9
        assert abs(o["entropy"][0] - pins._eval(case["entropy"])) <= 1e-9
        assert np.allclose(o["dZ"][0], [pins._eval(e) for e in case["dz"]], atol=1e-9, rtol=0)


def _pin_brute(ref):
    X, W, t, s, glp, gent = pins._tiny_problem(1)
    Xl = [[brute.bf16_to_float(v) for v in row] for row in X]
    Wl = [[brute.bf16_to_float(v) for v in row] for row in W]
    bf = brute.solve(Xl, Wl, [int(v) for v in t], -100, s, list(map(float, glp)),
                     list(map(float, gent)))
    o = ref.forward(X, W, t, -100, s, True)
    dX, dW = ref.backward(X, W, t, -100, s, glp, gent)
    for k in ("lse", "logprob", "entropy"):
        assert np.allclose(o[k], bf[k], atol=1e-10, rtol=0)
    assert np.allclose(dX, bf["dX"], atol=1e-10, rtol=0)
    assert np.allclose(dW, bf["dW"], atol=1e-10, rtol=0)


def _pin_zero_sum(ref):
    c = inputs.make_case("inv", 901, 20, 16, 61, ignore_frac=0.1, grad_mode="normal")
    _, dW = ref.backward(c.X, c.W, c.targets, -100, 1.0, c.grad_logprob, c.grad_entropy)
    assert np.abs(dW.sum(0)).max() <= 1e-10 * np.abs(dW).sum(0).max()


def _pin_torch(ref):
    rng = np.random.default_rng(11)
    M, H, V = 6, 8, 23
    X = pins._bits(rng.standard_normal((M, H)))
    W = pins._bits(rng.standard_normal((V, H)) / 4)
    t = rng.integers(0, V, M)
    t[2] = -100
    s = float(np.float32(1 / 0.7))
    glp, gent = rng.standard_normal(M), rng.standard_normal(M)
    o = ref.forward(X, W, t, -100, s, True)
    dX, dW = ref.backward(X, W, t, -100, s, glp, gent)
    Xt = torch.tensor(flce_ref.decode_bf16(X), requires_grad=True)
    Wt = torch.tensor(flce_ref.decode_bf16(W), requires_grad=True)
    Z = s * (Xt @ Wt.T)
    nll = torch.nn.functional.cross_entropy(Z, torch.tensor(t), ignore_index=-100, reduction="none")
    lp = torch.log_softmax(Z, 1)
    ent = torch.where(torch.tensor(t) != -100, -(lp.exp() * lp).sum(1), torch.zeros((), dtype=torch.float64))
    assert np.allclose(o["logprob"], (-nll).detach().numpy(), atol=1e-10)
    assert np.allclose(o["entropy"], ent.detach().numpy(), atol=1e-10)
    ((torch.tensor(glp) * -nll).sum() + (torch.tensor(gent) * ent).sum()).backward()
    assert np.allclose(dX, Xt.grad.numpy(), atol=1e-10)
    assert np.allclose(dW, Wt.grad.numpy(), atol=1e-10)


def _pin_blocked(ref):
    """The row loops over many small blocks against the brute force."""
    M, H, V = 8, 6, 11
    X, W, t, s, glp, gent = pins._tiny_problem(5, M=M, H=H, V=V)
    saved = ref.ROW_BLOCK_BYTES
    ref.ROW_BLOCK_BYTES = 8 * max(M, V) * 2       # 2 rows / vocabulary entries per block
    try:
        rows = np.array([6, 0, 7, 3, 2])
        vrows = np.array([10, 0, 4, 5, 9, 1])
        o = ref.forward(X, W, t, -100, s, True)
        dX, dW = ref.backward(X, W, t, -100, s, glp, gent)
        dxr = ref.dx_rows(X, W, t, rows, -100, s, glp, gent)
        dwr = ref.dw_rows(X, W, t, vrows, -100, s, o["lse"], o["E"], glp, gent)
    finally:
        ref.ROW_BLOCK_BYTES = saved
    Xl = [[brute.bf16_to_float(v) for v in row] for row in X]
    Wl = [[brute.bf16_to_float(v) for v in row] for row in W]
    bf = brute.solve(Xl, Wl, [int(v) for v in t], -100, s, list(map(float, glp)),
                     list(map(float, gent)))
    for k in ("lse", "logprob", "entropy"):
        assert np.allclose(o[k], bf[k], atol=1e-10, rtol=0)
    bdX, bdW = np.array(bf["dX"]), np.array(bf["dW"])
    assert np.allclose(dX, bdX, atol=1e-10, rtol=0) and np.allclose(dW, bdW, atol=1e-10, rtol=0)
    assert np.allclose(dxr, bdX[rows], atol=1e-10, rtol=0)
    assert np.allclose(dwr, bdW[vrows], atol=1e-10, rtol=0)


PINS = [_pin_closed_forms, _pin_brute, _pin_zero_sum, _pin_torch, _pin_blocked]


def test_pins_pass_on_real_oracle():
    for pin in PINS:
        pin(flce_ref)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
