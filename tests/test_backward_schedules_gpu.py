"""Every kind of backward schedule against the fp64 oracle: one launch per step
(pipelined: a step's dW and dX tiles with the next step's d-logit tiles, over two
d-logit buffers) and three launches per step, each with one and with several vocabulary
chunks and token waves.  The workspace size selects the schedule; sizes are scanned
between the smallest and twice the preferred one and the first size of each kind is run,
with NaN bit patterns in the workspace so that a stale read would show."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _kinds(M, H, V):
    from log_prob_amd import flce
    lo = flce.backward_workspace_min(M, H, V)
    hi = 2 * flce.workspace_query(M, H, V, True)[1]
    Mpad, Vpad = -(-M // 256) * 256, -(-V // 256) * 256
    found = {}
    for b in np.unique(np.geomspace(lo, hi, 64).astype(np.int64)):
        rows, chunk, pipe = flce.backward_schedule(M, H, V, int(b))
        key = (pipe, chunk < Vpad, rows < Mpad)   # pipelined, several chunks, several waves
        found.setdefault(key, int(b))
    return found


@pytest.mark.parametrize("M,H,V", [(600, 136, 3000), (4097, 64, 1000), (300, 200, 20000)])
def test_every_schedule_kind_matches_oracle(M, H, V):
    import torch
    from log_prob_amd import flce
    c = inputs.make_case(f"sched{M}", 161, M, H, V, ignore_frac=0.05, big_rows_frac=0.05,
                         grad_mode="normal")
    found = _kinds(M, H, V)
    print(f"[schedules] M={M} H={H} V={V}: {found}", flush=True)
    assert (True, True, False) in found or (True, True, True) in found   # pipelined, chunked
    assert (False, True, False) in found or (False, True, True) in found  # sequential, chunked
    X, W, t, glp, gent = gu.to_dev(c)
    lp, lse, ent = flce.forward(X, W, t, c.ignore_index, c.scale, True)
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                            c.grad_entropy)
    for key, b in sorted(found.items()):
        ws = torch.full((b,), 0xFF, dtype=torch.uint8, device="cuda")
        dX, dW = flce.backward(X, W, t, lse, ent, glp, gent, c.ignore_index, c.scale,
                               workspace=ws)
        torch.cuda.synchronize()
        gu.check_grads(gu.bf16_to_np(dX), gu.bf16_to_np(dW), rdX, rdW,
                       f"M={M} schedule {flce.backward_schedule(M, H, V, b)}")
