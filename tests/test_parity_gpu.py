"""GPU parity: libflce (through the C ABI) against the fp64 oracle, element by element,
on seeded inputs small enough for the oracle, spanning several 256 x 256 tiles and
ragged tails in M, V and K, plus the degenerate cases of the method."""
import sys

import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# name, case_id, M, H, V, make_case kwargs
CASES = [
    ("config1_tiny", 1, 64, 128, 1000, dict(ignore_frac=0.05, grad_mode="inv_m")),
    ("multi_tile_ragged", 101, 600, 320, 1500, dict(ignore_frac=0.05, grad_mode="normal")),
    ("aligned_tiles", 102, 512, 256, 2048, dict(grad_mode="inv_m", ignore_frac=0.02)),
    ("logprob_only_T07", 103, 257, 72, 257,
     dict(scale=1 / 0.7, compute_entropy=False, grad_mode="normal_lp")),
    ("big_rows_x64", 104, 513, 136, 3000,
     dict(ignore_frac=0.1, big_rows_frac=0.1, big_factor=64.0, grad_mode="normal")),
    ("k_tail_H200", 105, 300, 200, 700, dict(grad_mode="normal", ignore_frac=0.1)),
    ("single_row", 106, 1, 64, 1000, dict(grad_mode="normal")),
    ("single_vocab", 107, 100, 64, 1, dict(grad_mode="normal")),
    ("min_H8", 108, 70, 8, 300, dict(grad_mode="normal")),
    ("odd_vocab_50257", 109, 40, 64, 50257, dict(grad_mode="normal", ignore_frac=0.05)),
    ("negative_scale", 110, 128, 64, 500, dict(scale=-0.5, grad_mode="normal")),
    ("m_4097_tail", 111, 4097, 64, 300, dict(grad_mode="normal", ignore_frac=0.02)),
]


def _case(spec):
    name, cid, M, H, V, kw = spec
    return inputs.make_case(name, cid, M, H, V, **kw)


def _oracle(c):
    o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, True)
    dX, dW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                          c.grad_entropy)
    return o, dX, dW


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_parity_small(spec):
    c = _case(spec)
    print(f"[parity] {spec[0]} M={c.M} H={c.H} V={c.V}", flush=True)
    res = gu.run_flce(c)
    o, dX, dW = _oracle(c)
    gu.check_forward(res, o, c.compute_entropy, spec[0])
    gu.check_grads(res["dX"], res["dW"], dX, dW, spec[0])
    # ignored rows: exact zeros
    valid = ref.valid_rows(c.targets, c.V, c.ignore_index)
    assert np.all(res["logprob"][~valid] == 0.0)
    if c.compute_entropy:
        assert np.all(res["entropy"][~valid] == 0.0)
    assert np.all(res["dX"][~valid] == 0.0)


def test_strongly_negative_rows():
    """Every logit of a row far below zero (about -200): lse must still be exact-ish."""
    c = inputs.make_case("neg", 120, 300, 64, 900, grad_mode="normal")
    X = inputs.decode_bf16_to_f32(c.X).copy()
    W = inputs.decode_bf16_to_f32(c.W).copy()
    X[:, 0] = -200.0    # a bias feature: every logit of every row shifted by -200 * W[:, 0]
    W[:, 0] = 1.0
    c.X = inputs.f32_to_bf16_bits(X)
    c.W = inputs.f32_to_bf16_bits(W)
    res = gu.run_flce(c)
    o, dX, dW = _oracle(c)
    assert np.all(o["lse"] < -150)
    gu.check_forward(res, o, True, "strongly_negative")
    gu.check_grads(res["dX"], res["dW"], dX, dW, "strongly_negative")


def test_ignore_index_inside_vocab_and_out_of_range_targets():
    c = inputs.make_case("ign", 121, 200, 64, 700, grad_mode="normal")
    c.ignore_index = 5
    c.targets[::7] = 5
    c.targets[3] = 700          # == V: out of range, treated as ignored
    c.targets[4] = -3           # negative, not ignore_index: ignored
    res = gu.run_flce(c)
    o, dX, dW = _oracle(c)
    gu.check_forward(res, o, True, "ignore_inside")
    gu.check_grads(res["dX"], res["dW"], dX, dW, "ignore_inside")
    assert res["logprob"][3] == 0.0 and res["logprob"][4] == 0.0


def test_chunked_backward_matches():
    """The smallest workspace forces 256-column chunks and the fp32 dX accumulator."""
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("chunk", 122, 300, 136, 1300, grad_mode="normal", ignore_frac=0.1)
    mn = flce.backward_workspace_min(c.M, c.H, c.V)
    assert flce.backward_chunk_cols(c.M, c.H, c.V, mn) == 256
    ws = torch.empty(mn, dtype=torch.uint8, device="cuda")
    res_small = gu.run_flce(c, bwd_ws=ws)
    res_full = gu.run_flce(c)
    o, dX, dW = _oracle(c)
    gu.check_grads(res_small["dX"], res_small["dW"], dX, dW, "chunked")
    # dW is computed chunk by chunk either way: identical; dX differs only in fp32 order
    np.testing.assert_array_equal(res_small["dW"], res_full["dW"])
    # one bf16 ulp (2^-8 relative) at most, from fp32 summation order before rounding
    assert gu.rel_max(res_small["dX"], res_full["dX"]) <= 5e-3


def test_forward_token_waves_bitwise():
    """Token waves of 256 and 1024 rows (a ragged last wave: 5000 = 4 * 1024 + 904)
    give the same bits as one wave, and match the oracle."""
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("waves", 126, 5000, 64, 300, grad_mode="normal", ignore_frac=0.05)
    print(f"[parity] token waves M={c.M} H={c.H} V={c.V}", flush=True)
    X, W, t, _, _ = gu.to_dev(c)
    full, _ = flce.workspace_query(c.M, c.H, c.V, True)
    mn = flce.forward_workspace_min(c.M, c.H, c.V, True)
    w1k = mn * 4  # room for four 256-row tiles of partials per wave
    assert flce.forward_wave_rows(c.M, c.H, c.V, w1k) == 1024
    assert flce.forward_wave_rows(c.M, c.H, c.V, mn) == 256
    outs = []
    for nbytes in (full, mn, w1k):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        outs.append([v.clone() for v in flce.forward(X, W, t, c.ignore_index, c.scale, True,
                                                      workspace=ws)])
    torch.cuda.synchronize()
    for other in outs[1:]:
        for a, b in zip(outs[0], other):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, True)
    res = {k: v.cpu().numpy().astype(np.float64) for k, v in zip(("logprob", "lse", "entropy"),
                                                                 outs[1])}
    gu.check_forward(res, o, True, "token_waves")


def test_zero_grads_write_zeros():
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("zero", 123, 100, 64, 300, grad_mode="none")
    X, W, t, _, _ = gu.to_dev(c)
    lp, lse, ent = flce.forward(X, W, t)
    dX = torch.full_like(X, 3.0)
    dW = torch.full_like(W, 3.0)
    flce.backward(X, W, t, lse, None, None, None, out=(dX, dW))
    torch.cuda.synchronize()
    assert torch.count_nonzero(dX).item() == 0 and torch.count_nonzero(dW).item() == 0


def test_repeat_is_bitwise_deterministic_and_poison_safe():
    """Two runs give identical bits, also when the workspace starts full of NaN bytes."""
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("det", 124, 700, 136, 2100, grad_mode="normal", ignore_frac=0.05)
    X, W, t, glp, gent = gu.to_dev(c)
    fb, bb = flce.workspace_query(c.M, c.H, c.V, True)
    outs = []
    for poison in (False, True):
        ws = torch.empty(max(fb, bb), dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF if poison else 0)
        lp, lse, ent = flce.forward(X, W, t, workspace=ws)
        ws.fill_(0xFF if poison else 0)
        dX, dW = flce.backward(X, W, t, lse, ent, glp, gent, workspace=ws)
        torch.cuda.synchronize()
        outs.append([v.clone() for v in (lp, lse, ent, dX, dW)])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_grad_zero_sum_property():
    """Rows of d-logits sum to zero, so every dW column sums to ~0 (at any size)."""
    c = inputs.make_case("zs", 125, 1024, 256, 4096, grad_mode="normal")
    res = gu.run_flce(c)
    dW = res["dW"]
    assert np.abs(dW.sum(0)).max() <= 2e-2 * np.abs(dW).sum(0).max()


@pytest.mark.parametrize("how", ["scale_zero", "weight_zero"])
def test_uniform_softmax_closed_forms(how):
    """Every logit 0 (scale 0, or W = 0): the softmax is uniform, so on valid rows
    lse = entropy = ln V and logprob = -ln V; ignored rows give 0.  With scale 0 both
    gradients vanish exactly (every d-logit carries a factor of the scale); with W = 0, dX
    vanishes exactly and dW = dz^T X is checked against the oracle.  The vocabulary is
    ragged (1500 and 700 columns), so the masked tail of the last tile must stay out of
    the sums however the scale treats it."""
    import math
    if how == "scale_zero":
        c = inputs.make_case("uniform_s0", 122, 600, 136, 1500, scale=0.0, ignore_frac=0.1,
                             grad_mode="normal")
    else:
        c = inputs.make_case("uniform_w0", 123, 300, 64, 700, ignore_frac=0.1, grad_mode="normal")
        c.W = np.zeros_like(c.W)
    print(f"[parity] uniform {how} M={c.M} H={c.H} V={c.V}", flush=True)
    res = gu.run_flce(c)
    valid = ref.valid_rows(c.targets, c.V, c.ignore_index)
    assert 0 < valid.sum() < c.M
    lnV = math.log(c.V)
    np.testing.assert_allclose(res["lse"], lnV, rtol=0, atol=2e-6)
    np.testing.assert_allclose(res["logprob"][valid], -lnV, rtol=0, atol=2e-6)
    np.testing.assert_allclose(res["entropy"][valid], lnV, rtol=0, atol=2e-6)
    assert np.all(res["logprob"][~valid] == 0.0) and np.all(res["entropy"][~valid] == 0.0)
    assert np.all(res["dX"] == 0.0)
    if how == "scale_zero":
        assert np.all(res["dW"] == 0.0)
    else:
        o, dX, dW = _oracle(c)
        assert np.all(dX == 0.0) and np.max(np.abs(dW)) > 0
        gu.check_forward(res, o, True, "uniform_w0")
        gu.check_grads(res["dX"], res["dW"], dX, dW, "uniform_w0")


@pytest.mark.parametrize("col", [0, 255, 256, 1299])
def test_every_target_in_one_column(col):
    """Every valid row targets the same vocabulary column (the first, the edges of the
    first 256-column tile, the last column of a ragged last tile): the target-logit
    correction of the d-logits, rare on random targets, is taken by every row of every
    tile that holds that column."""
    c = inputs.make_case("one_col", 124, 700, 128, 1300, ignore_frac=0.05, grad_mode="normal")
    valid = ref.valid_rows(c.targets, c.V, c.ignore_index)
    c.targets = np.where(valid, col, c.targets).astype(np.int64)
    print(f"[parity] one column {col} M={c.M} H={c.H} V={c.V}", flush=True)
    res = gu.run_flce(c)
    o, dX, dW = _oracle(c)
    gu.check_forward(res, o, True, f"one_col{col}")
    gu.check_grads(res["dX"], res["dW"], dX, dW, f"one_col{col}")


def test_targets_beyond_32_bits_are_not_valid():
    """Targets are 64-bit: values whose low 32 bits name a vocabulary column
    (2^32 + 5, -2^32 + 7, 2^63 - 1, -2^63) are out of range, so those rows are ignored
    by the forward, the backward and the scalar NLL reduction alike."""
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("t64", 125, 400, 64, 900, grad_mode="normal")
    big = np.array([2**32 + 5, -2**32 + 7, 2**63 - 1, -2**63], dtype=np.int64)
    rows = np.array([0, 1, 255, 399])
    c.targets[rows] = big
    print(f"[parity] 64-bit targets M={c.M} H={c.H} V={c.V}", flush=True)
    res = gu.run_flce(c)
    o, dX, dW = _oracle(c)
    assert not ref.valid_rows(c.targets, c.V, c.ignore_index)[rows].any()
    gu.check_forward(res, o, True, "t64")
    gu.check_grads(res["dX"], res["dW"], dX, dW, "t64")
    assert np.all(res["logprob"][rows] == 0) and np.all(res["entropy"][rows] == 0)
    assert np.all(res["dX"][rows] == 0)
    lp = torch.from_numpy(res["logprob"].astype(np.float32)).cuda()
    red = flce.nll_reduce(lp, torch.from_numpy(c.targets).cuda(), c.V, c.ignore_index)
    total, n, _ = ref.nll_reduce(res["logprob"].astype(np.float64), c.targets, c.V, c.ignore_index)
    r = red.cpu().numpy()
    assert int(r[1]) == n == c.M - len(rows)
    assert r[0] == pytest.approx(total, rel=1e-12)


@pytest.mark.parametrize("H", [16384, 65544])
def test_long_hidden_dimension(H):
    """K loops of 256 and 1025 steps (65544 = 1024 * 64 + 8: a last K step with a single
    16-byte chunk of each row), with ragged M and V, against the oracle."""
    c = inputs.make_case("long_h", 126, 100, H, 300, ignore_frac=0.05, grad_mode="normal")
    print(f"[parity] long H M={c.M} H={c.H} V={c.V}", flush=True)
    res = gu.run_flce(c)
    o, dX, dW = _oracle(c)
    gu.check_forward(res, o, True, f"long_h{H}")
    gu.check_grads(res["dX"], res["dW"], dX, dW, f"long_h{H}")


def test_target_is_the_dominant_logit():
    """Rows whose target holds nearly all of the probability (the usual row of a trained
    policy): X[m] = k_m W[t_m], so z_t = k_m |W_t|^2 stands far above the row's other
    logits, with k_m up to 64 x 4.  logprob is at most 0 exactly, 0 <= entropy <= ln V,
    and every output matches the oracle."""
    M, H, V = 700, 256, 3000
    c = inputs.make_case("dominant", 131, M, H, V, ignore_frac=0.05, grad_mode="normal")
    rng = np.random.default_rng(131)
    valid = ref.valid_rows(c.targets, V, c.ignore_index)
    Wf = inputs.decode_bf16_to_f32(c.W)
    k = (64.0 * rng.uniform(0.05, 4.0, M)).astype(np.float32)
    k[: M // 4] = rng.uniform(3.0, 12.0, M // 4)        # also targets only moderately ahead
    X = k[:, None] * Wf[np.where(valid, c.targets, 0)]
    c.X[valid] = inputs.f32_to_bf16_bits(X[valid])
    print(f"[parity] dominant target M={M} H={H} V={V}", flush=True)
    res = gu.run_flce(c)
    o, dX, dW = _oracle(c)
    assert np.all(res["logprob"] <= 0.0)
    assert np.all(res["entropy"] >= 0.0) and np.all(res["entropy"] <= np.log(V) + 1e-6)
    assert np.max(o["logprob"][valid]) > -1e-6          # the oracle's rows are dominant
    gu.check_forward(res, o, True, "dominant")
    gu.check_grads(res["dX"], res["dW"], dX, dW, "dominant")


def _guarded(numel, dtype, guard_bytes=4096):
    """A tensor of `numel` elements with `guard_bytes` of canary bytes on both sides."""
    import torch
    esz = torch.empty(0, dtype=dtype).element_size()
    g = guard_bytes // esz
    buf = torch.empty(numel + 2 * g, dtype=dtype, device="cuda")
    buf.view(torch.uint8).fill_(0xA5)
    return buf, buf[g:g + numel], g


def _guards_intact(buf, g):
    import torch
    b = buf.view(torch.uint8)
    n = g * buf.element_size()
    return bool((b[:n] == 0xA5).all()) and bool((b[-n:] == 0xA5).all())


@pytest.mark.parametrize("ws_kind", ["preferred", "minimum", "minimum_plus"])
def test_guard_regions_untouched(ws_kind):
    """Nothing is written outside the outputs or past the workspace bytes a call is given:
    canary bytes before and after logprob, lse, entropy, dX, dW and the workspace keep
    their value, for the preferred workspace, the smallest one (256-row forward waves,
    256-column backward chunks with the fp32 dX accumulator) and a size just above it."""
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("guards", 132, 600, 136, 3000, ignore_frac=0.05, grad_mode="normal")
    X, W, t, glp, gent = gu.to_dev(c)
    fwd_b, bwd_b = flce.workspace_query(c.M, c.H, c.V, True)
    if ws_kind == "preferred":
        sizes = (fwd_b, bwd_b)
    else:
        extra = 0 if ws_kind == "minimum" else 1000
        sizes = (flce.forward_workspace_min(c.M, c.H, c.V, True) + extra,
                 flce.backward_workspace_min(c.M, c.H, c.V) + extra)
    bufs = [_guarded(c.M, torch.float32) for _ in range(3)]
    dxb = _guarded(c.M * c.H, torch.bfloat16)
    dwb = _guarded(c.V * c.H, torch.bfloat16)
    wsf = _guarded(sizes[0], torch.uint8)
    wsb = _guarded(sizes[1], torch.uint8)
    print(f"[parity] guards, workspaces {sizes}", flush=True)
    lp, lse, ent = (b[1] for b in bufs)
    flce.forward(X, W, t, c.ignore_index, c.scale, True, workspace=wsf[1], out=(lp, lse, ent))
    dX, dW = dxb[1].view(c.M, c.H), dwb[1].view(c.V, c.H)
    flce.backward(X, W, t, lse, ent, glp, gent, c.ignore_index, c.scale, workspace=wsb[1],
                  out=(dX, dW))
    torch.cuda.synchronize()
    for name, (buf, _, g) in zip(("logprob", "lse", "entropy", "dX", "dW", "forward workspace",
                                  "backward workspace"), bufs + [dxb, dwb, wsf, wsb]):
        assert _guards_intact(buf, g), f"{name}: a guard byte changed"
    o, rdX, rdW = _oracle(c)
    res = dict(logprob=gu.to_np(lp), lse=gu.to_np(lse), entropy=gu.to_np(ent))
    gu.check_forward(res, o, True, "guards")
    gu.check_grads(gu.bf16_to_np(dX), gu.bf16_to_np(dW), rdX, rdW, "guards")
