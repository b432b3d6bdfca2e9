"""The d-logit tile's vocabulary masking and target correction, through dX and dW,
element by element against the fp64 oracle.

The d-logit kernel computes each 256 x 256 tile transposed (vocabulary rows, token
columns), two waves of 128 vocabulary rows per token column: in the last tile of a
ragged V the second wave has some, or no, existing rows, whose d-logits must be 0, and
a token's target row may fall in either wave, in any of a lane's four consecutive rows.
Swept over the size of the last vocabulary tile (1 ... 256 entries, and vocabularies of
a single tile), both signs of the scale, and with and without an entropy gradient; the
targets are drawn so that many fall in the last tile."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

LAST = [1, 64, 127, 128, 129, 200, 255, 256]
CASES = ([(512 + r, s, g) for r in LAST for s in (1.0, -0.8) for g in ("normal", "normal_lp")] +
         [(v, s, "normal") for v in (1, 100, 129) for s in (1.0, -0.8)])


@pytest.mark.parametrize("V,scale,grad_mode", CASES)
def test_backward_ragged_vocabulary_tiles(V, scale, grad_mode):
    import torch
    from log_prob_amd import flce
    M, H = 300, 64
    c = inputs.make_case(f"bwd_edge_{V}", 192, M, H, V, scale=scale, ignore_frac=0.05,
                         grad_mode=grad_mode)
    # half of the targets in the last vocabulary tile, where the masking applies
    rng = np.random.default_rng(V)
    last0 = (V - 1) // 256 * 256
    valid = ref.valid_rows(c.targets, V, c.ignore_index)
    pick = valid & (rng.random(M) < 0.5)
    c.targets[pick] = rng.integers(last0, V, int(pick.sum()))
    X, W, t, glp, gent = gu.to_dev(c)
    lp, lse, ent = flce.forward(X, W, t, c.ignore_index, c.scale, True)
    nan = lambda *shape: torch.full(shape, float("nan"), dtype=torch.bfloat16, device="cuda")
    dX, dW = flce.backward(X, W, t, lse, ent if gent is not None else None, glp, gent,
                           c.ignore_index, c.scale, out=(nan(M, H), nan(V, H)))
    torch.cuda.synchronize()
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                            c.grad_entropy)
    gu.check_grads(gu.bf16_to_np(dX), gu.bf16_to_np(dW), rdX, rdW,
                   f"V={V} scale={scale} grads={grad_mode}")
