"""GPU parity of the vocabulary-shard entry points.

One GPU runs every shard of a vocabulary in turn.  Two buffers stand in for the
exchange between ranks: the shards' forward partials are gathered into one buffer
(shard r at byte r * stride), and the fp32 dX terms are summed in shard order
(accumulate = 1 after the first shard).  The results are checked against the fp64
oracle on the whole, unsharded vocabulary.  Sharding changes only the fp32
summation order, so the tolerances are those of the unsharded tests.
"""
import os

import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu
from tests.test_configs_gpu import _fingerprint

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# name, case_id, M, H, V, shard offsets, make_case kwargs
CASES = [
    ("ragged_3", 201, 600, 320, 1500, [0, 300, 1024, 1500],
     dict(ignore_frac=0.05, grad_mode="normal")),
    ("aligned_4", 202, 512, 256, 2048, [0, 512, 1024, 1536, 2048],
     dict(grad_mode="inv_m", ignore_frac=0.02)),
    ("one_row_shard_lp_T07", 203, 257, 72, 700, [0, 1, 257, 700],
     dict(scale=1 / 0.7, compute_entropy=False, grad_mode="normal_lp")),
    ("odd_vocab_8", 204, 300, 64, 50257,
     [round(r * 50257 / 8) for r in range(9)], dict(grad_mode="normal", ignore_frac=0.05)),
    ("single_shard", 205, 300, 200, 700, [0, 700], dict(grad_mode="normal", ignore_frac=0.1)),
]


def run_sharded(case, offsets, lse_in=None, ent_in=None):
    """Forward partials per shard, merge, then backward per shard; torch results."""
    import torch
    from log_prob_amd import flce
    X, W, t, glp, gent = gu.to_dev(case)
    M, H = case.M, case.H
    need_ent = case.compute_entropy or gent is not None
    P = len(offsets) - 1
    stride = max(flce.workspace_query(M, H, offsets[r + 1] - offsets[r], need_ent)[0]
                 for r in range(P))
    stride = (stride + 255) // 256 * 256
    # poisoned: any read of a byte no shard wrote shows up as NaN
    gathered = torch.full((P * stride,), 0xFF, dtype=torch.uint8, device="cuda")
    for r in range(P):
        lo, hi = offsets[r], offsets[r + 1]
        flce.forward_partials_shard(X, W[lo:hi], t, lo, case.ignore_index, case.scale, need_ent,
                                    workspace=gathered[r * stride:(r + 1) * stride])
    lp, lse, ent = flce.forward_merge_shards(t, offsets, gathered, stride, case.ignore_index,
                                             need_ent)
    lse_b = lse if lse_in is None else lse_in
    ent_b = ent if ent_in is None else ent_in
    dXp = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
    dW = torch.full_like(W, float("nan"))
    for r in range(P):
        lo, hi = offsets[r], offsets[r + 1]
        flce.backward_shard(X, W[lo:hi], t, lo, case.V, lse_b,
                            ent_b if gent is not None else None, glp, gent, dX_partial=dXp,
                            accumulate=r > 0, ignore_index=case.ignore_index, scale=case.scale,
                            dW_shard=dW[lo:hi])
    torch.cuda.synchronize()
    if not case.compute_entropy:
        ent = None
    return lp, lse, ent, dXp, dW


def _np(t):
    return None if t is None else t.detach().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_shards_match_oracle(spec):
    name, cid, M, H, V, offsets, kw = spec
    c = inputs.make_case(name, cid, M, H, V, **kw)
    print(f"[shards] {name} M={M} H={H} V={V} shards={len(offsets) - 1}", flush=True)
    lp, lse, ent, dXp, dW = run_sharded(c, offsets)
    res = dict(logprob=_np(lp), lse=_np(lse), entropy=_np(ent))
    o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, True)
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                            c.grad_entropy)
    gu.check_forward(res, o, c.compute_entropy, name)
    gu.check_grads(_np(dXp), gu.bf16_to_np(dW), rdX, rdW, name)
    valid = ref.valid_rows(c.targets, c.V, c.ignore_index)
    assert np.all(res["logprob"][~valid] == 0.0)
    assert np.all(_np(dXp)[~valid] == 0.0)


def test_shard_targets_outside_every_shard_and_ignore_inside():
    """Targets past V_total and an ignore_index that is a real id: rows stay ignored."""
    c = inputs.make_case("ign_sh", 206, 200, 64, 700, grad_mode="normal")
    c.ignore_index = 5
    t = c.targets.copy()
    t[::7] = 5
    t[3::11] = 700 + 3     # past the vocabulary
    t[5::13] = -1
    c.targets = t
    lp, lse, ent, dXp, dW = run_sharded(c, [0, 128, 256, 700])
    o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, True)
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                            c.grad_entropy)
    gu.check_forward(dict(logprob=_np(lp), lse=_np(lse), entropy=_np(ent)), o, True, "ign_sh")
    gu.check_grads(_np(dXp), gu.bf16_to_np(dW), rdX, rdW, "ign_sh")


def test_shard_zero_grads_and_accumulate_flag():
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("zg_sh", 207, 300, 64, 600, grad_mode="none")
    X, W, t, _, _ = gu.to_dev(c)
    lp, lse, ent = flce.forward(X, W, t, c.ignore_index, c.scale, True)
    dXp = torch.full((c.M, c.H), 3.0, dtype=torch.float32, device="cuda")
    dW = torch.full_like(W, 7.0)
    # accumulate = 1 leaves the running sum as it is; the shard's dW rows become zero
    flce.backward_shard(X, W[100:400], t, 100, c.V, lse, dX_partial=dXp, accumulate=True,
                        dW_shard=dW[100:400])
    torch.cuda.synchronize()
    assert bool((dXp == 3.0).all())
    assert int(torch.count_nonzero(dW[100:400])) == 0
    assert bool((dW[:100].float() == 7.0).all()) and bool((dW[400:].float() == 7.0).all())
    # accumulate = 0 overwrites
    flce.backward_shard(X, W[0:100], t, 0, c.V, lse, dX_partial=dXp, accumulate=False,
                        dW_shard=dW[0:100])
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dXp)) == 0


def test_shard_matches_unsharded_path_bitwise_where_tiles_align():
    """With shard edges on 256-column tiles and the same lse, every dW tile sees the same
    d-logits and the same K order as in the unsharded call: dW is bitwise equal."""
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("bit_sh", 208, 700, 320, 2304, grad_mode="normal", ignore_frac=0.05)
    X, W, t, glp, gent = gu.to_dev(c)
    lp, lse, ent = flce.forward(X, W, t, c.ignore_index, c.scale, True)
    dX, dW = flce.backward(X, W, t, lse, ent, glp, gent, c.ignore_index, c.scale)
    offsets = [0, 768, 1024, 2304]
    lp2, lse2, ent2, dXp, dW2 = run_sharded(c, offsets, lse_in=lse, ent_in=ent)
    assert torch.equal(dW, dW2)
    assert float((lse - lse2).abs().max()) <= 1e-5
    assert float((lp - lp2).abs().max()) <= 1e-5
    assert float((ent - ent2).abs().max()) <= 1e-5
    # dX: one fp32 sum over all columns rounded once vs a sum of fp32 shard terms
    ex = float((dX.float() - dXp).abs().max()) / float(dXp.abs().max())
    assert ex <= 1e-2, ex


@pytest.mark.parametrize("cfg,n_shards", [(2, 4), (3, 8)])
def test_shards_full_size_against_golden(cfg, n_shards):
    """Workloads 2 and 3 split over 4 and 8 ranks (the pages' tensor-parallel degrees;
    workload 3's 128256 ids split at non-tile edges), against the oracle: every row of
    the forward outputs and of the largest gradient magnitudes (stored by
    make_golden.py), and dX rows and dW rows on both sides of every shard boundary
    element by element (oracle on the host), relative to the whole-tensor maxima."""
    import torch
    from tests import oracle_runner as run
    case = inputs.config_case(cfg)
    V = case.V
    offsets = [round(r * V / n_shards) for r in range(n_shards + 1)]
    print(f"[shards] config {cfg}: M={case.M} H={case.H} V={V} shards={n_shards}", flush=True)
    g = np.load(os.path.join(GOLDEN, f"config{cfg}.npz"))
    assert str(g["fingerprint"]) == _fingerprint(case), "inputs differ from the golden run"
    lp, lse, ent, dXp, dW = run_sharded(case, offsets)
    res = dict(logprob=_np(lp), lse=_np(lse), entropy=_np(ent))
    exp = dict(logprob=g["logprob"], lse=g["lse"], entropy=g["entropy"])
    gu.check_forward(res, exp, case.compute_entropy, f"config{cfg} x{n_shards}")
    assert bool(torch.isfinite(dXp).all()) and bool(torch.isfinite(dW).all())
    ex = float(np.abs(_np(dXp.abs().amax(1)) - g["dx_rowmax"]).max()) / float(g["dx_absmax"])
    ew = float(np.abs(_np(dW.float().abs().amax(1)) - g["dw_rowmax"]).max()) / float(g["dw_absmax"])
    assert ex <= gu.GRAD_RTOL and ew <= gu.GRAD_RTOL, f"row maxima: dX {ex:.3g} dW {ew:.3g}"
    rng = np.random.default_rng(np.random.SeedSequence([2026, cfg, 97]))
    rows = np.sort(rng.choice(case.M, 32, replace=False))
    vrows = sorted({v for b in offsets[1:-1] for v in (b - 1, b)} | {0, V - 1})
    with run.Pool(case, lse=g["lse"], E=g["E"]) as pool:
        rdx = pool.rows("dx", rows)
        rdw = pool.rows("dw", np.array(vrows))
    got_dx = _np(dXp.index_select(0, torch.from_numpy(rows).cuda()))
    got_dw = gu.bf16_to_np(dW.index_select(0, torch.tensor(vrows).cuda()))
    ex = gu.max_abs(got_dx, rdx) / float(g["dx_absmax"])
    ew = gu.max_abs(got_dw, rdw) / float(g["dw_absmax"])
    assert ex <= gu.GRAD_RTOL and ew <= gu.GRAD_RTOL, f"dX rel {ex:.3g} dW rel {ew:.3g}"


def _random_splits(n=8, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M, H, V = int(rng.integers(1, 900)), int(8 * rng.integers(1, 60)), int(rng.integers(2, 4000))
        P = int(rng.integers(2, min(V, 9) + 1))
        offsets = [0] + sorted(set(int(x) for x in rng.integers(1, V, P - 1))) + [V]
        mode = str(rng.choice(["inv_m", "normal", "normal_lp"]))
        out.append((i, M, H, V, offsets, mode, float(rng.choice([1.0, 1 / 0.7, -0.5]))))
    return out


@pytest.mark.parametrize("spec", _random_splits(), ids=lambda s: f"r{s[0]}_M{s[1]}_V{s[3]}_P{len(s[4]) - 1}")
def test_random_shard_splits(spec):
    """Seeded random shapes split at random vocabulary boundaries (shards of any width,
    down to one column), against the oracle on the whole vocabulary."""
    i, M, H, V, offsets, mode, scale = spec
    c = inputs.make_case(f"rsh{i}", 210 + i, M, H, V, scale=scale, grad_mode=mode,
                         compute_entropy=True, ignore_frac=0.05)
    print(f"[shards] random {spec}", flush=True)
    lp, lse, ent, dXp, dW = run_sharded(c, offsets)
    o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, True)
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                            c.grad_entropy)
    gu.check_forward(dict(logprob=_np(lp), lse=_np(lse), entropy=_np(ent)), o, True, f"rsh{i}")
    gu.check_grads(_np(dXp), gu.bf16_to_np(dW), rdX, rdW, f"rsh{i}")
