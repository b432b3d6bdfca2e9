"""The forward tile's vocabulary masking, element by element against the fp64 oracle.

The forward computes each 256 x 256 logit tile transposed (vocabulary rows, token
columns) with two waves of 128 vocabulary rows per token column, so the last vocabulary
tile of a ragged V leaves the second wave with some, or no, existing rows; its maxima
and sums must skip the rows past V.  Swept over the size of that last tile (1 ... 256
entries, including vocabularies of a single tile), both signs of the scale (a negative
scale takes the maximum of the negated logits), and with and without entropy.  Every
row is also checked against the bounds logprob <= 0 and 0 <= entropy <= ln V."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

LAST = [1, 64, 127, 128, 129, 200, 255, 256]
CASES = ([(512 + r, s, e) for r in LAST for s in (1.0, -0.8) for e in (True, False)] +
         [(v, s, True) for v in (1, 100, 128, 129) for s in (1.0, -0.8)])


@pytest.mark.parametrize("V,scale,ent", CASES)
def test_forward_ragged_vocabulary_tiles(V, scale, ent):
    import torch
    from log_prob_amd import flce
    M, H = 300, 64
    c = inputs.make_case(f"fwd_edge_{V}", 191, M, H, V, scale=scale, ignore_frac=0.05,
                         big_rows_frac=0.05)
    X, W, t, _, _ = gu.to_dev(c)
    nan = lambda: torch.full((M,), float("nan"), device="cuda")
    out = (nan(), nan(), nan() if ent else None)
    flce.forward(X, W, t, c.ignore_index, c.scale, ent, out=out)
    torch.cuda.synchronize()
    got = dict(logprob=gu.to_np(out[0]), lse=gu.to_np(out[1]),
               entropy=None if out[2] is None else gu.to_np(out[2]))
    want = ref.forward_f64(ref.decode_bf16(c.X), ref.decode_bf16(c.W), c.targets,
                           c.ignore_index, c.scale, ent)
    gu.check_forward(got, want, ent, f"V={V} scale={scale} entropy={ent}")
    assert np.all(got["logprob"] <= 0.0)
    if ent:
        assert np.all(got["entropy"] >= 0.0) and np.all(got["entropy"] <= np.log(V) + 1e-6)
