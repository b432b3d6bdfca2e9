"""GPU parity at the extremes of the accepted sizes: an empty batch, a token count just
past 2^20 and a vocabulary just past 2^21 (the widest d-logit chunk, so the backward
takes two chunks).  Rows the oracle checks are sampled; properties that hold at any
size are checked on whole tensors."""
import numpy as np
import pytest

from oracle import flce_ref as ref
from synth import inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def test_empty_batch():
    import torch
    from log_prob_amd import flce
    H, V = 64, 1000
    X = torch.empty((0, H), dtype=torch.bfloat16, device="cuda")
    W = torch.ones((V, H), dtype=torch.bfloat16, device="cuda")  # never read
    t = torch.empty(0, dtype=torch.int64, device="cuda")
    lp, lse, ent = flce.forward(X, W, t)
    assert lp.numel() == 0 and lse.numel() == 0 and ent.numel() == 0
    dW = torch.full_like(W, 3.0)
    dX, dW = flce.backward(X, W, t, lse, ent, torch.empty(0, device="cuda"),
                           torch.empty(0, device="cuda"), out=(torch.empty_like(X), dW))
    red = flce.nll_reduce(lp, t, V)
    torch.cuda.synchronize()
    assert dX.numel() == 0 and int(torch.count_nonzero(dW)) == 0
    r = red.cpu().numpy()
    assert r[0] == 0.0 and r[1] == 0.0 and np.isnan(r[2])
    dWs = torch.full_like(W[100:600], 5.0)
    flce.backward_shard(X, W[100:600], t, 100, V, lse, dX_partial=torch.empty((0, H), device="cuda"),
                        dW_shard=dWs)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(dWs)) == 0


def _check_case(c, rows, vrows, all_rows_forward):
    import torch
    from log_prob_amd import flce
    X, W, t, glp, gent = gu.to_dev(c)
    lp, lse, ent = flce.forward(X, W, t, c.ignore_index, c.scale, True)
    dX, dW = flce.backward(X, W, t, lse, ent, glp, gent, c.ignore_index, c.scale)
    torch.cuda.synchronize()
    Wd = ref.decode_bf16(c.W)
    if all_rows_forward:
        o = ref.forward(c.X, c.W, c.targets, c.ignore_index, c.scale, True, Wd=Wd)
        sel = rows
        got = {k: v.cpu().numpy().astype(np.float64) for k, v in
               (("logprob", lp), ("lse", lse), ("entropy", ent))}
        gu.check_forward(got, o, True, c.name)
    else:
        o = ref.forward_rows(c.X, c.W, c.targets, rows, c.ignore_index, c.scale, True, Wd=Wd)
        got = {k: v.cpu().numpy().astype(np.float64)[rows] for k, v in
               (("logprob", lp), ("lse", lse), ("entropy", ent))}
        gu.check_forward(got, o, True, c.name)
    rdx = ref.dx_rows(c.X, c.W, c.targets, rows, c.ignore_index, c.scale, c.grad_logprob,
                      c.grad_entropy, Wd=Wd)
    got_dx = gu.bf16_to_np(dX.index_select(0, torch.from_numpy(rows).cuda()))
    if all_rows_forward:
        rdw = ref.dw_rows(c.X, c.W, c.targets, vrows, c.ignore_index, c.scale, o["lse"], o["E"],
                          c.grad_logprob, c.grad_entropy)
        got_dw = gu.bf16_to_np(dW.index_select(0, torch.from_numpy(vrows).cuda()))
        gu.check_grads(got_dx, got_dw, rdx, rdw, c.name)
    else:
        assert gu.rel_max(got_dx, rdx) <= gu.GRAD_RTOL, c.name
    assert bool(torch.isfinite(dX).all()) and bool(torch.isfinite(dW).all())
    assert bool(torch.isfinite(lse).all())
    colsum = dW.float().sum(0).abs().max().item()
    colabs = dW.float().abs().sum(0).max().item()
    assert colsum <= 2e-2 * colabs, (colsum, colabs)
    return lp, dX


def test_token_count_past_2_pow_20():
    M = (1 << 20) + 1
    c = inputs.make_case("m_2e20", 501, M, 64, 512, grad_mode="normal", ignore_frac=0.01)
    print(f"[sizes] M={M} H=64 V=512", flush=True)
    rng = np.random.default_rng(7)
    rows = np.sort(np.concatenate([rng.choice(M, 61, replace=False), [0, M - 2, M - 1]]))
    _check_case(c, rows, None, all_rows_forward=False)


def test_vocabulary_past_2_pow_21_two_chunks():
    from log_prob_amd import flce
    V = (1 << 21) + 3
    c = inputs.make_case("v_2e21", 502, 64, 64, V, grad_mode="normal", ignore_frac=0.05)
    assert flce.backward_chunk_cols(64, 64, V, flce.workspace_query(64, 64, V)[1]) < V
    print(f"[sizes] M=64 H=64 V={V}", flush=True)
    rng = np.random.default_rng(8)
    vrows = np.sort(np.concatenate([rng.choice(V, 29, replace=False), [0, (1 << 21) - 1,
                                                                       1 << 21, V - 1]]))
    # the targets of a few rows at the far end of the vocabulary, past the first chunk
    c.targets[:4] = [V - 1, V - 2, 1 << 21, (1 << 21) - 1]
    _check_case(c, np.arange(64), vrows, all_rows_forward=True)
