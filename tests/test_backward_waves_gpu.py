"""The backward in token waves (workspaces too small for one wave of every row) against
the fp64 oracle, element by element: dW stored by the first wave and accumulated in
fp32 across later waves, dX completed wave by wave.  Shapes from the pages' wave cases
(Liger-Kernel commit "native Blackwell tensor-parallel fused scaled linear
cross-entropy", section "Correctness": 4097-token boundaries, 5000-token tails) and a
batch past 2^20 tokens, with workspaces too small for one wave of every row (the wave
height is whatever the schedule takes for that size); the smallest workspace does not
grow with the number of tokens."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _single_wave_min(M, H, V):
    """Bytes of the smallest one-wave schedule: 256-column chunks with the fp32 dX
    accumulator of every row, or one chunk of every column."""
    Mpad, Vpad = -(-M // 256) * 256, -(-V // 256) * 256
    return min(Mpad * 256 * 2 + M * H * 4, Mpad * Vpad * 2)


def _multi_wave_sizes(M, H, V):
    """The smallest workspace and one halfway to the smallest one-wave schedule: both
    must run the backward in more than one token wave."""
    from log_prob_amd import flce
    lo = flce.backward_workspace_min(M, H, V)
    hi = _single_wave_min(M, H, V)
    assert lo < hi
    return [lo, (lo + hi) // 2 // 256 * 256]


def _run(c, ws_bytes):
    import torch
    from log_prob_amd import flce
    X, W, t, glp, gent = gu.to_dev(c)
    lp, lse, ent = flce.forward(X, W, t, c.ignore_index, c.scale, True)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)                          # NaN bit patterns: stale data would show
    dX, dW = flce.backward(X, W, t, lse, ent if gent is not None else None, glp, gent,
                           c.ignore_index, c.scale, workspace=ws)
    torch.cuda.synchronize()
    return gu.bf16_to_np(dX), gu.bf16_to_np(dW)


@pytest.mark.parametrize("M,which", [(4097, 0), (4097, 1), (5000, 0), (5000, 1)])
def test_waves_match_oracle(M, which):
    from log_prob_amd import flce
    H, V = 64, 1000
    c = inputs.make_case(f"waves{M}", 151, M, H, V, ignore_frac=0.05, big_rows_frac=0.05,
                         grad_mode="normal")
    b = _multi_wave_sizes(M, H, V)[which]
    rows, chunk = flce.backward_wave_rows(M, H, V, b), flce.backward_chunk_cols(M, H, V, b)
    assert rows < M                                     # more than one wave, a ragged tail
    print(f"[waves] M={M} H={H} V={V}: {b} workspace bytes -> {rows}-row waves, "
          f"{chunk}-column chunks", flush=True)
    dX, dW = _run(c, b)
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                            c.grad_entropy)
    gu.check_grads(dX, dW, rdX, rdW, f"waves M={M}")
    valid = ref.valid_rows(c.targets, V, c.ignore_index)
    assert np.all(dX[~valid] == 0.0)


def test_minimum_workspace_does_not_grow_with_tokens():
    from log_prob_amd import flce
    H, V = 64, 512
    sizes = {M: flce.backward_workspace_min(M, H, V) for M in (4097, 5000, (1 << 20) + 1, 1 << 24)}
    assert len(set(sizes.values())) == 1, sizes
    # and it is the 256-row, 256-column schedule with the fp32 dW accumulator (and the
    # 256 bytes of tile-queue counters)
    assert sizes[4097] == 256 * 256 * 2 + 256 * H * 4 + V * H * 4 + 256


@pytest.mark.parametrize("which", [0, 1])
def test_more_than_2_20_tokens_bounded_workspace(which):
    from log_prob_amd import flce
    M, H, V = (1 << 20) + 1, 64, 512
    c = inputs.make_case("waves_2e20", 152, M, H, V, ignore_frac=0.02, grad_mode="normal")
    b = _multi_wave_sizes(M, H, V)[which]
    rows = flce.backward_wave_rows(M, H, V, b)
    assert rows < M
    print(f"[waves] M={M}: {b} workspace bytes -> {rows}-row waves", flush=True)
    dX, dW = _run(c, b)
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                            c.grad_entropy)
    gu.check_grads(dX, dW, rdX, rdW, f"waves M={M} rows={rows}")


def test_shard_backward_in_waves():
    """Every shard of a split vocabulary with a workspace that forces token waves: the
    fp32 dX terms summed over shards and the shards' dW rows match the oracle."""
    import torch
    from log_prob_amd import flce
    M, H, V = 4097, 64, 1000
    offs = [0, 300, 301, 1000]
    c = inputs.make_case("shard_waves", 153, M, H, V, ignore_frac=0.05, grad_mode="normal")
    X, W, t, glp, gent = gu.to_dev(c)
    lp, lse, ent = flce.forward(X, W, t, c.ignore_index, c.scale, True)
    dXp = torch.empty((M, H), dtype=torch.float32, device="cuda")
    dW = torch.empty_like(W)
    for r in range(len(offs) - 1):
        Vs = offs[r + 1] - offs[r]
        lo, _ = flce.backward_shard_workspace_query(M, H, Vs)
        ws = torch.full((lo,), 0xFF, dtype=torch.uint8, device="cuda")
        flce.backward_shard(X, W[offs[r]:offs[r + 1]], t, offs[r], V, lse, ent, glp, gent,
                            dX_partial=dXp, accumulate=r > 0, ignore_index=c.ignore_index,
                            scale=c.scale, workspace=ws, dW_shard=dW[offs[r]:offs[r + 1]])
    torch.cuda.synchronize()
    rdX, rdW = ref.backward(c.X, c.W, c.targets, c.ignore_index, c.scale, c.grad_logprob,
                            c.grad_entropy)
    gu.check_grads(gu.to_np(dXp), gu.bf16_to_np(dW), rdX, rdW, "shard waves")
