"""The allocation-free forward (flce_forward_noalloc, through the C ABI) against
flce_forward with a workspace, on two calls in a row, the second with a smaller input.

flce_forward_noalloc runs the same kernels through the library's static device
scratch, in token waves sized to it; a row's tiles and merge do not depend on its
wave, so its outputs must equal flce_forward's bit for bit.  The first call's
vocabulary makes the scratch hold fewer rows than the batch (two waves); the second
call is smaller, with entropy off, and reuses the scratch the first one left behind.
Both are also checked against the fp64 oracle on a sample of rows."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CALLS = [
    # case id, M, H, V, entropy, make_case options
    (141, 6000, 256, 131072, True, dict(ignore_frac=0.05, big_rows_frac=0.05)),
    (142, 700, 128, 50257, False, dict(scale=1 / 0.7)),
]


def test_noalloc_matches_forward_on_two_calls():
    import torch
    from log_prob_amd import flce
    for cid, M, H, V, ent, kw in CALLS:
        c = inputs.make_case(f"noalloc{cid}", cid, M, H, V, compute_entropy=ent,
                             grad_mode="none", **kw)
        rows = flce.forward_wave_rows(M, H, V, flce.FLCE_NOALLOC_SCRATCH_BYTES, ent)
        print(f"[noalloc] M={M} H={H} V={V} entropy={ent}: waves of {rows} rows", flush=True)
        if cid == 141:
            assert rows < M          # the scratch takes this batch in more than one wave
        X, W, t, _, _ = gu.to_dev(c)
        want = flce.forward(X, W, t, c.ignore_index, c.scale, ent)
        out = tuple(torch.full((M,), float("nan"), device="cuda") if (k < 2 or ent) else None
                    for k in range(3))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        flce.forward_noalloc(X, W, t, c.ignore_index, c.scale, ent, out=out)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before   # nothing allocated through torch
        got = out
        for name, a, b in zip(("logprob", "lse", "entropy"), got, want):
            if b is None:
                assert a is None
                continue
            assert torch.equal(a, b), f"{name} differs from flce_forward"
        sample = np.unique(np.concatenate([np.arange(0, M, max(1, M // 48)), [M - 1]]))
        o = ref.forward_rows(c.X, c.W, c.targets, sample, c.ignore_index, c.scale, True)
        res = {k: (None if v is None else gu.to_np(v)[sample])
               for k, v in zip(("logprob", "lse", "entropy"), got)}
        gu.check_forward(res, o, ent, f"noalloc {cid}")
