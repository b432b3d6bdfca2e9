"""Calls on several streams at once: the library keeps no state between calls (every
buffer is the caller's, the tile-queue counters included), so work enqueued on several
streams, or from several host threads, gives the same bits as the same calls run one
after another.  The third case's forward, d-logit and dW launches (at least 2048 tiles
each) hand out their last tiles through the counters of their own workspace."""
import threading

import pytest

from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    dict(name="s_a", case_id=501, M=700, H=320, V=1500, ignore_frac=0.05, grad_mode="normal"),
    dict(name="s_b", case_id=502, M=513, H=136, V=2600, scale=1 / 0.7, grad_mode="normal_lp"),
    dict(name="s_q", case_id=503, M=4096, H=8192, V=65836, ignore_frac=0.05, grad_mode="normal"),
]


def _setup(spec):
    import torch
    from log_prob_amd import flce
    kw = dict(spec)
    c = inputs.make_case(kw.pop("name"), kw.pop("case_id"), kw.pop("M"), kw.pop("H"),
                         kw.pop("V"), **kw)
    X, W, t, glp, gent = gu.to_dev(c)
    fb, bb = flce.workspace_query(c.M, c.H, c.V, True)
    ws = torch.empty(max(fb, bb), dtype=torch.uint8, device="cuda")
    outs = (torch.empty(c.M, device="cuda"), torch.empty(c.M, device="cuda"),
            torch.empty(c.M, device="cuda"), torch.empty_like(X), torch.empty_like(W))
    return c, (X, W, t, glp, gent), ws, outs


def _step(c, data, ws, outs):
    from log_prob_amd import flce
    X, W, t, glp, gent = data
    lp, lse, ent, dX, dW = outs
    flce.forward(X, W, t, c.ignore_index, c.scale, True, workspace=ws, out=(lp, lse, ent))
    flce.backward(X, W, t, lse, ent if gent is not None else None, glp, gent, c.ignore_index,
                  c.scale, workspace=ws, out=(dX, dW))


def _serial_reference(setups):
    import torch
    refs = []
    for c, data, ws, outs in setups:
        _step(c, data, ws, outs)
        torch.cuda.synchronize()
        refs.append([o.clone() for o in outs])
    return refs


def _check(setups, refs, what):
    import torch
    for (c, _, _, outs), ref in zip(setups, refs):
        for name, a, b in zip(("logprob", "lse", "entropy", "dX", "dW"), outs, ref):
            assert torch.equal(a, b), f"{what}: {c.name} {name} differs from the serial run"


def test_two_streams_match_serial():
    import torch
    setups = [_setup(s) for s in CASES]
    refs = _serial_reference(setups)
    for _, _, _, outs in setups:
        for o in outs:
            o.zero_()
    streams = [torch.cuda.Stream() for _ in setups]
    torch.cuda.synchronize()
    for _ in range(3):
        for st, (c, data, ws, outs) in zip(streams, setups):
            with torch.cuda.stream(st):
                _step(c, data, ws, outs)
    torch.cuda.synchronize()
    _check(setups, refs, "two streams")


def test_two_host_threads_match_serial():
    import torch
    setups = [_setup(s) for s in CASES]
    refs = _serial_reference(setups)
    for _, _, _, outs in setups:
        for o in outs:
            o.zero_()
    streams = [torch.cuda.Stream() for _ in setups]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            c, data, ws, outs = setups[i]
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    _step(c, data, ws, outs)
            streams[i].synchronize()
        except Exception as e:  # reported on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(setups))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    _check(setups, refs, "two threads")
