"""Pins of the fp64 oracle to things other than itself (CPU only).

* closed forms derived by hand (tests/golden/closed_forms.json),
* an independent pure-Python brute force on tiny shapes,
* PyTorch's own cross_entropy / logsumexp / autograd in float64 (library routines
  the definitions reduce to),
* central finite differences of a*logprob + b*entropy for dX and dW,
* invariants: d-logit rows sum to zero, so dW columns sum to zero; bounds on
  logprob, entropy and lse; shift and vocabulary-permutation invariance;
  ignored rows are inert; large-magnitude rows stay finite.
"""
import ast
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle import flce_ref as ref
from synth import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _eval(expr: str) -> float:
    """Evaluate a closed-form expression: numbers, + - * /, log, exp."""
    allowed = {"log": math.log, "exp": math.exp}

    def ev(n):
        if isinstance(n, ast.Expression):
            return ev(n.body)
        if isinstance(n, ast.Constant) and isinstance(n.value, (int, float)):
            return float(n.value)
        if isinstance(n, ast.UnaryOp) and isinstance(n.op, (ast.USub, ast.UAdd)):
            v = ev(n.operand)
            return -v if isinstance(n.op, ast.USub) else v
        if isinstance(n, ast.BinOp) and isinstance(n.op, (ast.Add, ast.Sub, ast.Mult, ast.Div)):
            a, b = ev(n.left), ev(n.right)
            if isinstance(n.op, ast.Add):
                return a + b
            if isinstance(n.op, ast.Sub):
                return a - b
            if isinstance(n.op, ast.Mult):
                return a * b
            return a / b
        if isinstance(n, ast.Call) and isinstance(n.func, ast.Name) and n.func.id in allowed:
            return allowed[n.func.id](*[ev(x) for x in n.args])
        raise ValueError(f"unsupported expression: {expr}")

    return ev(ast.parse(expr, mode="eval"))


def _golden_cases():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_closed_forms_from_logits(case):
    z = np.array([[_eval(e) for e in case["z"]]])
    t = np.array([case["t"]])
    a, b = _eval(case["a"]), _eval(case["b"])
    o = ref.from_logits(z, t, -100, True, grad_logprob=[a], grad_entropy=[b])
    tol = 1e-12 * max(1.0, abs(z).max())
    assert abs(o["lse"][0] - _eval(case["lse"])) <= tol
    assert abs(o["logprob"][0] - _eval(case["logprob"])) <= tol
    assert abs(o["entropy"][0] - _eval(case["entropy"])) <= 1e-12
    np.testing.assert_allclose(o["dZ"][0], [_eval(e) for e in case["dz"]], rtol=0, atol=1e-12)


def _bits(x):
    return inputs.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_row_blocks_many_against_one_and_brute_force(monkeypatch):
    """Every block loop of the oracle (rows of the forward, the backward and dx_rows;
    vocabulary entries of dw_rows) run over many small blocks gives the single-block
    results and the pure-Python brute force's.  A loop that overwrote instead of
    accumulating, or wrote a block to the wrong rows, fails here."""
    M, H, V = 8, 6, 11
    X, W, t, s, glp, gent = _tiny_problem(5, M=M, H=H, V=V)
    rows = np.array([6, 0, 7, 3, 2])
    vrows = np.array([10, 0, 4, 5, 9, 1, int(t[0])])

    def run():
        o = ref.forward(X, W, t, -100, s, True)
        dX, dW = ref.backward(X, W, t, -100, s, glp, gent)
        dxr = ref.dx_rows(X, W, t, rows, -100, s, glp, gent)
        dwr = ref.dw_rows(X, W, t, vrows, -100, s, o["lse"], o["E"], glp, gent)
        return o, dX, dW, dxr, dwr

    one = run()
    assert ref.row_block(V) >= M and ref.row_block(M) >= len(vrows)
    monkeypatch.setattr(ref, "ROW_BLOCK_BYTES", 8 * max(M, V) * 2)   # 2 rows / entries per block
    assert ref.row_block(V) == 2 and ref.row_block(M) == 2
    many = run()
    Xl = [[brute.bf16_to_float(v) for v in row] for row in X]
    Wl = [[brute.bf16_to_float(v) for v in row] for row in W]
    bf = brute.solve(Xl, Wl, [int(v) for v in t], -100, s, [float(g) for g in glp],
                     [float(g) for g in gent])
    bdX, bdW = np.array(bf["dX"]), np.array(bf["dW"])
    for res in (one, many):
        o, dX, dW, dxr, dwr = res
        for k in ("lse", "logprob", "entropy"):
            np.testing.assert_allclose(o[k], bf[k], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dX, bdX, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dW, bdW, rtol=0, atol=1e-13)
        np.testing.assert_allclose(dxr, bdX[rows], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dwr, bdW[vrows], rtol=0, atol=1e-13)


def test_closed_forms_through_linear_head():
    """Uniform and two-level logits built from crafted bf16 X and W."""
    # W = 0: every logit is 0 -> lse = log V, logprob = -log V, entropy = log V
    M, H, V = 3, 8, 37
    X = _bits(np.random.default_rng(0).standard_normal((M, H)))
    W = _bits(np.zeros((V, H)))
    t = np.array([0, 36, 5])
    o = ref.forward(X, W, t, -100, 1.0, True)
    np.testing.assert_allclose(o["lse"], math.log(V), atol=1e-14)
    np.testing.assert_allclose(o["logprob"], -math.log(V), atol=1e-14)
    np.testing.assert_allclose(o["entropy"], math.log(V), atol=1e-14)
    # two-level: X row = (c, 0, ...), W[t] = (1, 0, ...), other W rows 0, scale s
    c, s = 1.5, 2.0
    Xc = np.zeros((1, H)); Xc[0, 0] = c
    Wc = np.zeros((V, H)); Wc[7, 0] = 1.0
    o = ref.forward(_bits(Xc), _bits(Wc), np.array([7]), -100, s, True)
    cz = c * s
    lse = math.log(math.exp(cz) + V - 1)
    assert abs(o["lse"][0] - lse) < 1e-13
    assert abs(o["logprob"][0] - (cz - lse)) < 1e-13
    assert abs(o["entropy"][0] - (lse - cz * math.exp(cz) / (math.exp(cz) + V - 1))) < 1e-13


def _tiny_problem(seed, M=5, H=6, V=7, scale=0.8):
    rng = np.random.default_rng(seed)
    X = _bits(rng.standard_normal((M, H)))
    W = _bits(rng.standard_normal((V, H)) * 0.7)
    t = rng.integers(0, V, M)
    t[1] = -100          # ignore_index
    t[3] = V + 2         # out of range -> ignored
    glp = rng.standard_normal(M).astype(np.float32)
    gent = rng.standard_normal(M).astype(np.float32)
    return X, W, t, float(np.float32(scale)), glp, gent


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_brute_force_agreement(seed):
    X, W, t, s, glp, gent = _tiny_problem(seed)
    Xl = [[brute.bf16_to_float(v) for v in row] for row in X]
    Wl = [[brute.bf16_to_float(v) for v in row] for row in W]
    bf = brute.solve(Xl, Wl, [int(v) for v in t], -100, s, [float(g) for g in glp],
                     [float(g) for g in gent])
    o = ref.forward(X, W, t, -100, s, True)
    dX, dW = ref.backward(X, W, t, -100, s, glp, gent)
    np.testing.assert_allclose(o["lse"], bf["lse"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(o["logprob"], bf["logprob"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(o["entropy"], bf["entropy"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dX, bf["dX"], rtol=0, atol=1e-13)
    np.testing.assert_allclose(dW, bf["dW"], rtol=0, atol=1e-13)


def test_against_torch_library_fp64():
    """cross_entropy, logsumexp and autograd of torch (float64, CPU) agree."""
    rng = np.random.default_rng(11)
    M, H, V = 9, 16, 53
    X = _bits(rng.standard_normal((M, H)))
    W = _bits(rng.standard_normal((V, H)) / 4)
    t = rng.integers(0, V, M)
    t[[2, 6]] = -100
    s = float(np.float32(1 / 0.7))
    glp = rng.standard_normal(M)
    gent = rng.standard_normal(M)
    o = ref.forward(X, W, t, -100, s, True)
    dX, dW = ref.backward(X, W, t, -100, s, glp, gent)

    Xt = torch.tensor(ref.decode_bf16(X), requires_grad=True)
    Wt = torch.tensor(ref.decode_bf16(W), requires_grad=True)
    tt = torch.tensor(t)
    Z = s * (Xt @ Wt.T)
    nll = torch.nn.functional.cross_entropy(Z, tt, ignore_index=-100, reduction="none")
    valid = tt != -100
    logp_all = torch.log_softmax(Z, dim=1)
    ent = torch.where(valid, -(logp_all.exp() * logp_all).sum(1), torch.zeros(()).double())
    np.testing.assert_allclose(o["lse"], torch.logsumexp(Z, 1).detach().numpy(), atol=1e-13)
    np.testing.assert_allclose(o["logprob"], (-nll).detach().numpy(), atol=1e-13)
    np.testing.assert_allclose(o["entropy"], ent.detach().numpy(), atol=1e-13)
    L = (torch.tensor(glp) * (-nll)).sum() + (torch.tensor(gent) * ent).sum()
    L.backward()
    np.testing.assert_allclose(dX, Xt.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dW, Wt.grad.numpy(), atol=1e-12)


def test_finite_differences():
    rng = np.random.default_rng(5)
    M, H, V = 3, 5, 7
    Xd = rng.standard_normal((M, H))
    Wd = rng.standard_normal((V, H)) * 0.6
    t = np.array([2, -100, 6])
    s = 1.25
    a = rng.standard_normal(M)
    b = rng.standard_normal(M)

    def L(Xd_, Wd_):
        o = ref.forward_f64(Xd_, Wd_, t, -100, s, True)
        return float((a * o["logprob"]).sum() + (b * o["entropy"]).sum())

    dX, dW = ref.backward_f64(Xd, Wd, t, -100, s, a, b)
    h = 1e-6
    for arr, grad in ((Xd, dX), (Wd, dW)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + h; lp = L(Xd, Wd)
            arr[idx] = old - h; lm = L(Xd, Wd)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        assert np.abs(num - grad).max() <= 1e-7 * max(1.0, np.abs(grad).max())
    # the ignored row gets an exactly-zero gradient
    assert np.all(dX[1] == 0.0)


def test_invariants_on_random_case():
    c = inputs.make_case("inv", 901, 40, 32, 211, scale=1.3, ignore_frac=0.1, grad_mode="normal")
    o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, True)
    Xd, Wd = ref.decode_bf16(c.X), ref.decode_bf16(c.W)
    Z = ref.logits(Xd, Wd, c.scale)
    d = ref.from_logits(Z, c.targets, c.ignore_index, True, c.grad_logprob, c.grad_entropy)
    # rows of d-logits sum to zero (softmax minus one-hot, and the entropy term)
    assert np.abs(d["dZ"].sum(1)).max() <= 1e-14 * np.abs(d["dZ"]).sum(1).max() + 1e-16
    dX, dW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                          c.grad_entropy)
    assert np.abs(dW.sum(0)).max() <= 1e-12 * np.abs(dW).sum(0).max()
    valid = ref.valid_rows(c.targets, c.V, c.ignore_index)
    assert np.all(o["logprob"] <= 0)
    assert np.all(o["entropy"] >= 0) and np.all(o["entropy"] <= math.log(c.V) + 1e-12)
    zmax = Z.max(1)
    assert np.all(o["lse"] >= zmax) and np.all(o["lse"] <= zmax + math.log(c.V) + 1e-12)
    assert np.all(o["logprob"][~valid] == 0) and np.all(o["entropy"][~valid] == 0)
    assert np.all(dX[~valid] == 0)
    # entropy == lse - E (the two forms agree)
    np.testing.assert_allclose(o["entropy"][valid], (o["lse"] - o["E"])[valid], atol=1e-12)


def test_shift_invariance_constant_feature():
    """Appending a constant feature column shifts every logit of a row by X[m,H]*w0."""
    rng = np.random.default_rng(3)
    M, H, V = 6, 8, 29
    X = rng.standard_normal((M, H)); W = rng.standard_normal((V, H)) / 3
    t = rng.integers(0, V, M)
    o1 = ref.forward_f64(X, W, t, -100, 1.0, True)
    shift = rng.standard_normal(M)
    X2 = np.concatenate([X, shift[:, None]], 1)
    W2 = np.concatenate([W, np.ones((V, 1))], 1)
    o2 = ref.forward_f64(X2, W2, t, -100, 1.0, True)
    np.testing.assert_allclose(o2["logprob"], o1["logprob"], atol=1e-12)
    np.testing.assert_allclose(o2["entropy"], o1["entropy"], atol=1e-12)
    np.testing.assert_allclose(o2["lse"], o1["lse"] + shift, atol=1e-12)


def test_vocab_permutation_equivariance():
    c = inputs.make_case("perm", 902, 12, 16, 41, ignore_frac=0.2, grad_mode="normal")
    perm = np.random.default_rng(4).permutation(c.V)
    inv = np.argsort(perm)
    t2 = np.where((c.targets >= 0) & (c.targets < c.V), inv[np.clip(c.targets, 0, c.V - 1)],
                  c.targets)
    o1 = ref.forward(c.X, c.W, c.targets, -100, 1.0, True)
    o2 = ref.forward(c.X, c.W[perm], t2, -100, 1.0, True)
    for k in ("logprob", "lse", "entropy"):
        np.testing.assert_allclose(o2[k], o1[k], atol=1e-12)
    _, dW1 = ref.backward(c.X, c.W, c.targets, -100, 1.0, c.grad_logprob, c.grad_entropy)
    _, dW2 = ref.backward(c.X, c.W[perm], t2, -100, 1.0, c.grad_logprob, c.grad_entropy)
    np.testing.assert_allclose(dW2, dW1[perm], atol=1e-12)


def test_ignored_rows_are_inert():
    c = inputs.make_case("ign", 903, 16, 16, 50, ignore_frac=0.25, grad_mode="normal")
    ign = c.targets == -100
    X2 = c.X.copy()
    X2[ign] = _bits(np.random.default_rng(9).standard_normal((ign.sum(), c.H)) * 5)
    dX1, dW1 = ref.backward(c.X, c.W, c.targets, -100, 1.0, c.grad_logprob, c.grad_entropy)
    dX2, dW2 = ref.backward(X2, c.W, c.targets, -100, 1.0, c.grad_logprob, c.grad_entropy)
    np.testing.assert_array_equal(dW1, dW2)
    np.testing.assert_array_equal(dX1[~ign], dX2[~ign])
    o1 = ref.forward(c.X, c.W, c.targets, -100, 1.0, True)
    o2 = ref.forward(X2, c.W, c.targets, -100, 1.0, True)
    np.testing.assert_array_equal(o1["logprob"], o2["logprob"])
    np.testing.assert_array_equal(o1["entropy"], o2["entropy"])


@pytest.mark.parametrize("factor", [64.0, 1e4])
def test_large_magnitude_rows_finite(factor):
    c = inputs.make_case("big", 904, 8, 64, 300, grad_mode="normal")
    Xd = ref.decode_bf16(c.X) * factor
    Wd = ref.decode_bf16(c.W)
    o = ref.forward_f64(Xd, Wd, c.targets, -100, 1.0, True)
    dX, dW = ref.backward_f64(Xd, Wd, c.targets, -100, 1.0, c.grad_logprob, c.grad_entropy)
    for v in (o["lse"], o["logprob"], o["entropy"], dX, dW):
        assert np.all(np.isfinite(v))
    Z = ref.logits(Xd, Wd, 1.0)
    assert np.all(o["lse"] >= Z.max(1)) and np.all(o["entropy"] >= 0)
    assert np.all(o["entropy"] <= math.log(c.V) + 1e-9)


def test_subset_helpers_match_full():
    c = inputs.make_case("sub", 905, 30, 24, 97, ignore_frac=0.1, grad_mode="normal", scale=0.9)
    o = ref.forward(c.X, c.W, c.targets, -100, c.scale, True)
    dX, dW = ref.backward(c.X, c.W, c.targets, -100, c.scale, c.grad_logprob, c.grad_entropy)
    rows = np.array([0, 7, 29, 3])
    orow = ref.forward_rows(c.X, c.W, c.targets, rows, -100, c.scale, True)
    for k in ("logprob", "lse", "entropy"):
        np.testing.assert_allclose(orow[k], o[k][rows], atol=1e-13)
    np.testing.assert_allclose(ref.dx_rows(c.X, c.W, c.targets, rows, -100, c.scale,
                                           c.grad_logprob, c.grad_entropy), dX[rows], atol=1e-13)
    vrows = np.array([0, 96, 50, int(c.targets[5])])
    np.testing.assert_allclose(
        ref.dw_rows(c.X, c.W, c.targets, vrows, -100, c.scale, o["lse"], o["E"],
                    c.grad_logprob, c.grad_entropy), dW[vrows], atol=1e-13)


def test_nll_reduce_against_torch_cross_entropy():
    """Sum and mean NLL over valid rows equal torch's cross_entropy reductions (fp64 CPU
    library routine, independent of the oracle's arithmetic)."""
    rng = np.random.default_rng(23)
    M, H, V = 13, 16, 41
    X = _bits(rng.standard_normal((M, H)))
    W = _bits(rng.standard_normal((V, H)) / 4)
    t = rng.integers(0, V, M)
    t[[1, 5, 9]] = -100
    s = float(np.float32(0.9))
    o = ref.forward(X, W, t, -100, s, False)
    total, n, mean = ref.nll_reduce(o["logprob"], t, V, -100)
    Z = s * (torch.tensor(ref.decode_bf16(X)) @ torch.tensor(ref.decode_bf16(W)).T)
    tt = torch.tensor(t)
    ce_sum = torch.nn.functional.cross_entropy(Z, tt, ignore_index=-100, reduction="sum")
    ce_mean = torch.nn.functional.cross_entropy(Z, tt, ignore_index=-100, reduction="mean")
    assert n == M - 3
    np.testing.assert_allclose(total, float(ce_sum), rtol=1e-13)
    np.testing.assert_allclose(mean, float(ce_mean), rtol=1e-13)
    # the gradient of the mean NLL through the log-probs: torch autograd of the mean
    Zg = Z.clone().requires_grad_(True)
    torch.nn.functional.cross_entropy(Zg, tt, ignore_index=-100, reduction="mean").backward()
    g = ref.nll_mean_grad(t, V, -100, n)
    dZ = ref.from_logits(Z.numpy(), t, -100, False, grad_logprob=g)["dZ"]
    np.testing.assert_allclose(dZ, Zg.grad.numpy(), atol=1e-14)


def test_nll_reduce_special_cases():
    # no valid row: sum 0, count 0, mean undefined (NaN), zero gradient
    t = np.array([-100, 7, -3])
    total, n, mean = ref.nll_reduce(np.array([1.0, 2.0, 3.0]), t, 5, -100)
    assert total == 0.0 and n == 0 and np.isnan(mean)
    assert np.all(ref.nll_mean_grad(t, 5, -100, 0) == 0.0)
    # brute force on a tiny case: a plain loop over the rows
    lp = np.array([-0.5, -1.25, -3.0, -0.125])
    t = np.array([0, 2, 9, 1])        # row 2 is out of range
    acc, cnt = 0.0, 0
    for i in range(4):
        if t[i] != -100 and 0 <= t[i] < 4:
            acc += -lp[i]
            cnt += 1
    assert ref.nll_reduce(lp, t, 4, -100) == (acc, cnt, acc / cnt)
