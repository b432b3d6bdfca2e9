"""GPU parity on a seeded sweep of random small shapes: ragged M, H and V tails in every
combination, both signs of the scale, ignored and out-of-range targets, entropy on and
off, and each gradient mode, against the fp64 oracle element by element."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _shapes(n=16, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([1, 2, 31, 255, 256, 257]) if i % 3 == 0 else rng.integers(1, 700))
        H = int(8 * rng.integers(1, 66))                      # 8 .. 520
        V = int(rng.choice([1, 255, 256, 257]) if i % 4 == 1 else rng.integers(1, 3000))
        scale = float(rng.choice([1.0, 1 / 0.7, 0.25, -0.5, 3.0]))
        ent = bool(rng.integers(0, 2))
        mode = str(rng.choice(["inv_m", "normal", "normal_lp", "none"]))
        if mode == "normal" and not ent:
            ent = True          # grad_entropy needs the entropy output
        ign = float(rng.choice([0.0, 0.05, 0.3]))
        out.append((i, M, H, V, scale, ent, mode, ign))
    return out


@pytest.mark.parametrize("spec", _shapes(), ids=lambda s: f"s{s[0]}_M{s[1]}_H{s[2]}_V{s[3]}")
def test_random_shape_parity(spec):
    i, M, H, V, scale, ent, mode, ign = spec
    c = inputs.make_case(f"rand{i}", 700 + i, M, H, V, scale=scale, compute_entropy=ent,
                         grad_mode=mode, ignore_frac=ign)
    if i % 5 == 2 and M > 3:      # a few targets outside [0, V)
        c.targets[:3] = [V, V + 7, -5]
    print(f"[random] {spec}", flush=True)
    res = gu.run_flce(c)
    o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, True)
    gu.check_forward(res, o, c.compute_entropy, f"rand{i}")
    valid = ref.valid_rows(c.targets, c.V, c.ignore_index)
    assert np.all(res["logprob"][~valid] == 0.0)
    if mode == "none":
        assert np.all(res["dX"] == 0.0) and np.all(res["dW"] == 0.0)
    else:
        rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                                c.grad_entropy)
        gu.check_grads(res["dX"], res["dW"], rdX, rdW, f"rand{i}")
        assert np.all(res["dX"][~valid] == 0.0)
