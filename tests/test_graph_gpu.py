"""The library's calls inside a captured HIP graph: every kernel launch is captured
(no allocation, no memset, no host synchronisation inside a call), and replays give
the eager results bit for bit, also with eager work and synchronisation between them."""
import pytest

from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_forward_backward_graph_replays_match_eager():
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("graph", 401, 700, 320, 1500, ignore_frac=0.05, grad_mode="normal")
    X, W, t, glp, gent = gu.to_dev(c)
    fb, bb = flce.workspace_query(c.M, c.H, c.V, True)
    ws = torch.empty(max(fb, bb), dtype=torch.uint8, device="cuda")
    lp = torch.empty(c.M, device="cuda")
    lse = torch.empty_like(lp)
    ent = torch.empty_like(lp)
    dX = torch.empty_like(X)
    dW = torch.empty_like(W)

    def step():
        flce.forward(X, W, t, c.ignore_index, c.scale, True, workspace=ws, out=(lp, lse, ent))
        flce.backward(X, W, t, lse, ent, glp, gent, c.ignore_index, c.scale, workspace=ws,
                      out=(dX, dW))

    # eager reference
    step()
    torch.cuda.synchronize()
    ref = [v.clone() for v in (lp, lse, ent, dX, dW)]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(3):
        for v in (lp, lse, ent, dX, dW):
            v.zero_()
        # unrelated eager work between replays
        junk = (X.float() @ X.float().T).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("logprob", "lse", "entropy", "dX", "dW"),
                              (lp, lse, ent, dX, dW), ref):
            assert torch.equal(a, b), f"replay {i}: {name} differs"
        del junk
