"""GPU parity when the caller's workspaces are of any size between the minimum and the
preferred one: the forward then runs in token waves of the height the workspace allows
and the backward in vocabulary chunks of the width it allows (fp32 dX accumulation over
the chunks), on seeded random shapes, against the fp64 oracle."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _specs(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 1400))
        H = int(8 * rng.integers(1, 90))
        V = int(rng.integers(1, 6000))
        scale = float(rng.choice([1.0, 1 / 0.7, -0.5]))
        mode = str(rng.choice(["inv_m", "normal", "normal_lp"]))
        ent = mode == "normal" or bool(rng.integers(0, 2))
        ign = float(rng.choice([0.0, 0.1]))
        fq, bq = float(rng.random()), float(rng.random())
        out.append((i, M, H, V, scale, ent, mode, ign, fq, bq))
    return out


@pytest.mark.parametrize("spec", _specs(), ids=lambda s: f"w{s[0]}_M{s[1]}_H{s[2]}_V{s[3]}")
def test_any_workspace_size(spec):
    import torch
    from log_prob_amd import flce
    i, M, H, V, scale, ent, mode, ign, fq, bq = spec
    c = inputs.make_case(f"ws{i}", 800 + i, M, H, V, scale=scale, compute_entropy=ent,
                         grad_mode=mode, ignore_frac=ign)
    fmin = flce.forward_workspace_min(M, H, V, ent)
    ffull, bfull = flce.workspace_query(M, H, V, ent)
    bmin = flce.backward_workspace_min(M, H, V)
    fb = fmin + int(fq * (ffull - fmin))
    bb = bmin + int(bq * max(0, bfull - bmin))
    waves = flce.forward_wave_rows(M, H, V, fb, ent)
    chunk = flce.backward_chunk_cols(M, H, V, bb)
    print(f"[workspace] {spec} wave={waves} chunk={chunk}", flush=True)
    fws = torch.empty(fb, dtype=torch.uint8, device="cuda")
    bws = torch.empty(bb, dtype=torch.uint8, device="cuda")
    res = gu.run_flce(c, fwd_ws=fws, bwd_ws=bws)
    o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, True)
    gu.check_forward(res, o, c.compute_entropy, f"ws{i}")
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                            c.grad_entropy)
    gu.check_grads(res["dX"], res["dW"], rdX, rdW, f"ws{i}")
    valid = ref.valid_rows(c.targets, c.V, c.ignore_index)
    assert np.all(res["logprob"][~valid] == 0.0) and np.all(res["dX"][~valid] == 0.0)
