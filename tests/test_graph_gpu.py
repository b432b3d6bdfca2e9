"""The library's calls inside a captured HIP graph: every kernel launch is captured
(no allocation, no memset, no host synchronisation inside a call), and replays give
the eager results bit for bit, also with eager work and synchronisation between them.
At the larger shape the forward, d-logit and dW launches hand out their last tiles
through counters in the workspace, which kernels of the same call zero: every replay
must find them cleared."""
import pytest

from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(700, 320, 1500), (4096, 8192, 65836)],
                         ids=["small", "queued_tiles"])
def test_forward_backward_graph_replays_match_eager(shape):
    import torch
    from log_prob_amd import flce
    M, H, V = shape
    c = inputs.make_case("graph", 401, M, H, V, ignore_frac=0.05, grad_mode="normal")
    fb, bb = flce.workspace_query(c.M, c.H, c.V, True)
    if M > 700:
        # three launches per step, each of at least 2048 tiles (256 per XCD)
        rows, chunk, pipe = flce.backward_schedule(M, H, V, bb)
        tiles = lambda n: -(-n // 256)
        assert not pipe and rows >= M
        assert min(tiles(M) * tiles(V), tiles(M) * tiles(chunk), tiles(chunk) * tiles(H)) >= 2048
    X, W, t, glp, gent = gu.to_dev(c)
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


@pytest.mark.parametrize("loss", ["mean_nll", "policy"])
def test_full_training_step_graph(loss):
    """One captured training step with no host synchronisation: forward, the scalar
    loss reduced on the device (mean NLL, or the clipped policy loss), its log-prob
    gradient with the token count read on the device, and the backward. Replays give
    the eager results bit for bit."""
    import numpy as np
    import torch
    from log_prob_amd import flce
    c = inputs.make_case("graph_step", 402, 900, 136, 2600, ignore_frac=0.1, grad_mode="none")
    X, W, t, _, _ = gu.to_dev(c)
    fb, bb = flce.workspace_query(c.M, c.H, c.V, False)
    ws = torch.empty(max(fb, bb), dtype=torch.uint8, device="cuda")
    lp = torch.empty(c.M, device="cuda")
    lse = torch.empty_like(lp)
    dX = torch.empty_like(X)
    dW = torch.empty_like(W)
    g = torch.empty(c.M, device="cuda")
    per_tok = torch.empty(c.M, device="cuda")
    clipped = torch.empty(c.M, dtype=torch.uint8, device="cuda")
    red = torch.empty(4 if loss == "policy" else 3, dtype=torch.float64, device="cuda")
    rng = np.random.default_rng(np.random.SeedSequence([2026, 402, 9]))
    old = torch.from_numpy(rng.normal(-8.0, 1.0, c.M).astype(np.float32)).cuda()
    adv = torch.from_numpy(rng.standard_normal(c.M).astype(np.float32)).cuda()

    def step():
        flce.forward(X, W, t, c.ignore_index, c.scale, False, workspace=ws, out=(lp, lse, None))
        if loss == "mean_nll":
            flce.nll_reduce(lp, t, c.V, c.ignore_index, out=red)
            flce.nll_mean_grad(t, c.V, red, c.ignore_index, out=g)
        else:
            flce.policy_loss_reduce(lp, old, adv, t, c.V, c.ignore_index, 0.2, 0.28,
                                    out=(per_tok, clipped, red))
            flce.policy_loss_grad(lp, old, adv, t, c.V, red, c.ignore_index, 0.2, 0.28, out=g)
        flce.backward(X, W, t, lse, None, g, None, c.ignore_index, c.scale, workspace=ws,
                      out=(dX, dW))

    outs = (lp, red, g, per_tok, clipped, dX, dW)
    names = ("logprob", "reduced", "grad_logprob", "per_token_loss", "is_clipped", "dX", "dW")
    step()
    torch.cuda.synchronize()
    ref = [v.clone() for v in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for i in range(3):
        for v in outs:
            v.zero_()
        junk = (X.float() @ X.float().T).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, ref):
            if loss == "mean_nll" and name in ("per_token_loss", "is_clipped"):
                continue
            assert torch.equal(a, b), f"{loss} replay {i}: {name} differs"
        del junk
    assert float(ref[1][1]) == float((t != c.ignore_index).sum())
    if loss == "policy":
        assert 0 < int(ref[1][2]) < int(ref[1][1])   # both branches of the minimum occur
