"""Tail queues of the tile kernels.  In a launch of at least 2048 tiles (256 per XCD),
the forward, d-logit and dW kernels hand out the last tiles of each XCD's stream at run
time, through counters in the workspace that the launch before them on the stream
clears, with spare workgroups that take tiles from the back of a slower XCD's queue.
Which workgroup runs a tile must not change any result.

* The forward at a ragged shape whose 3078 tiles are queued (n mod 8 = 6 tiles past
  the eight streams), element by element against the fp64 oracle, with the workspace
  and outputs filled with 0xFF bytes first (NaN partials, all-ones counters): a tile
  left out would leave a NaN, and uncleared counters would hand out the wrong tiles.
  Two calls through one workspace, the allocation-free entry point and 256-row token
  waves (1026 tiles a launch: no queue) all give the same bits.
* The backward in token waves whose dW launches (2080 tiles) are queued and add in
  fp32 across the waves: the only launches where a tile taken twice would change the
  result.  Its dX rows are sampled against the oracle; its dX equals, and its dW is
  compared with, that of the one-wave schedule of the same problem.  (The fp64 oracle
  over the whole problem, about 7e13 FLOP, is out of reach; the one-wave d-logit and dW
  launches of the large workloads are compared with the oracle over whole tensors in
  the workload tests.)
"""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

QUEUED = 2048  # tiles of a launch from which its last tiles are queued


def _tiles(n):
    return -(-n // 256)


def _nan(*shape, bf16=False):
    import torch
    return torch.full(shape, float("nan"), device="cuda",
                      dtype=torch.bfloat16 if bf16 else torch.float32)


def test_forward_queued_tiles_match_oracle_from_any_workspace():
    import torch
    from log_prob_amd import flce
    M, H, V = 600, 256, 262444
    assert _tiles(M) * _tiles(V) >= QUEUED and (_tiles(M) * _tiles(V)) % 8 != 0
    c = inputs.make_case("tile_queue_fwd", 181, M, H, V, ignore_frac=0.05, big_rows_frac=0.05)
    X, W, t, _, _ = gu.to_dev(c)
    fb, _ = flce.workspace_query(M, H, V, True)
    ws = torch.empty(fb, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)

    def run(fn, **kw):
        out = (_nan(M), _nan(M), _nan(M))
        fn(X, W, t, c.ignore_index, c.scale, True, out=out, **kw)
        torch.cuda.synchronize()
        return dict(zip(("logprob", "lse", "entropy"), (gu.to_np(o) for o in out)))

    first = run(flce.forward, workspace=ws)
    second = run(flce.forward, workspace=ws)        # counters left by the first call
    noalloc = run(flce.forward_noalloc)
    small = torch.empty(flce.forward_workspace_min(M, H, V, True), dtype=torch.uint8,
                        device="cuda")
    small.fill_(0xFF)
    assert flce.forward_wave_rows(M, H, V, small.numel()) == 256
    waves = run(flce.forward, workspace=small)
    for k in first:
        for name, other in (("second call", second), ("no-alloc", noalloc),
                            ("256-row waves", waves)):
            assert np.array_equal(first[k], other[k]), f"{k}: {name} differs"

    want = ref.forward_f64(ref.decode_bf16(c.X), ref.decode_bf16(c.W), c.targets,
                           c.ignore_index, c.scale, True)
    e_lp, e_lse = gu.check_forward(first, want, True, "queued forward")
    print(f"[tile queue] forward M={M} H={H} V={V}: {_tiles(M) * _tiles(V)} tiles, max abs "
          f"error logprob {e_lp:.3g} lse {e_lse:.3g}", flush=True)


def test_backward_queued_dw_across_waves():
    import torch
    from log_prob_amd import flce
    M, H, V = 65536, 4096, 33068
    b = int(1.856 * 2**30) // 256 * 256
    rows, chunk, pipe = flce.backward_schedule(M, H, V, b)
    n_dw = (chunk // 256) * _tiles(H)
    # token waves, three launches per step, a queued dW launch that adds across waves
    assert not pipe and rows < M and n_dw >= QUEUED, (rows, chunk, pipe, n_dw)
    _, pref = flce.workspace_query(M, H, V, True)
    r1, c1, p1 = flce.backward_schedule(M, H, V, pref)
    assert r1 >= M and not p1, (r1, c1, p1)
    print(f"[tile queue] backward M={M} H={H} V={V}: {rows}-row waves x {chunk} columns "
          f"({n_dw} dW tiles a launch) against one wave x {c1} columns", flush=True)

    c = inputs.make_case("tile_queue_bwd", 182, M, H, V, ignore_frac=0.05, big_rows_frac=0.05,
                         grad_mode="normal")
    X, W, t, glp, gent = gu.to_dev(c)
    lp, lse, ent = flce.forward(X, W, t, c.ignore_index, c.scale, True)

    def run(nbytes):
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)
        out = (_nan(M, H, bf16=True), _nan(V, H, bf16=True))
        flce.backward(X, W, t, lse, ent, glp, gent, c.ignore_index, c.scale, workspace=ws,
                      out=out)
        torch.cuda.synchronize()
        res = gu.bf16_to_np(out[0]), gu.bf16_to_np(out[1])
        del ws, out
        torch.cuda.empty_cache()
        return res

    dX, dW = run(b)
    dX1, dW1 = run(pref)
    assert np.all(np.isfinite(dX)) and np.all(np.isfinite(dW))
    # both schedules take the same chunk: a row's d-logits and dX do not depend on its wave
    assert c1 == chunk and np.array_equal(dX, dX1)
    ew = gu.rel_max(dW, dW1)
    print(f"[tile queue] waves vs one wave: dX equal, dW rel {ew:.3g}", flush=True)
    assert ew <= gu.GRAD_RTOL

    # dX rows against the oracle: the first and last row of every wave, a few more
    rng = np.random.default_rng(182)
    pick = {0, M - 1, *rng.choice(M, size=6, replace=False).tolist()}
    for w0 in range(0, M, rows):
        pick.update((w0, min(M, w0 + rows) - 1))
    pick = np.array(sorted(pick), dtype=np.int64)
    want = ref.dx_rows(c.X, c.W, c.targets, pick, c.ignore_index, c.scale, c.grad_logprob,
                       c.grad_entropy)
    e = gu.rel_max(dX[pick], want)
    print(f"[tile queue] dX rows {len(pick)} against the oracle: rel {e:.3g}", flush=True)
    assert e <= gu.GRAD_RTOL
