"""Helpers shared by the GPU tests: upload synthetic cases, run libflce, compare.

Tolerances: forward outputs (logprob, lse, entropy) max |gpu - oracle| <= 2e-3;
dX and dW max |gpu - oracle| / max |oracle| <= 1e-2.
"""
import numpy as np

FWD_ATOL = 2e-3
GRAD_RTOL = 1e-2


def to_dev(case, device="cuda"):
    import torch
    X = torch.from_numpy(case.X.view(np.int16)).view(torch.bfloat16).to(device)
    W = torch.from_numpy(case.W.view(np.int16)).view(torch.bfloat16).to(device)
    t = torch.from_numpy(case.targets).to(device)
    glp = None if case.grad_logprob is None else torch.from_numpy(case.grad_logprob).to(device)
    gent = None if case.grad_entropy is None else torch.from_numpy(case.grad_entropy).to(device)
    return X, W, t, glp, gent


def bf16_to_np(t):
    """bf16 torch tensor -> float64 numpy (exact)."""
    import torch
    bits = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def to_np(t):
    """Any torch tensor -> float64 numpy."""
    return t.detach().cpu().numpy().astype(np.float64)


def bf16_bits(t):
    """bf16 torch tensor -> its uint16 bit patterns as numpy."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_np(bits):
    """bf16 bit patterns (uint16 numpy) -> float64 numpy (exact)."""
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def run_flce(case, fwd_ws=None, bwd_ws=None, need_backward=True):
    """Forward (+ backward) through the C ABI; returns numpy float64 results."""
    import torch
    from log_prob_amd import flce
    X, W, t, glp, gent = to_dev(case)
    lp, lse, ent = flce.forward(X, W, t, case.ignore_index, case.scale, case.compute_entropy,
                                workspace=fwd_ws)
    need_ent_in = gent is not None
    ent_in = ent
    if need_ent_in and ent is None:
        # grad_entropy needs the entropy output: run a second forward with it on
        _, _, ent_in = flce.forward(X, W, t, case.ignore_index, case.scale, True)
    out = dict(logprob=lp, lse=lse, entropy=ent)
    if need_backward:
        dX, dW = flce.backward(X, W, t, lse, ent_in if need_ent_in else None, glp, gent,
                               case.ignore_index, case.scale, workspace=bwd_ws)
        out.update(dX=dX, dW=dW)
    torch.cuda.synchronize()
    res = {}
    for k, v in out.items():
        if v is None:
            res[k] = None
        elif v.dtype == torch.bfloat16:
            res[k] = bf16_to_np(v)
        else:
            res[k] = v.detach().cpu().numpy().astype(np.float64)
    return res


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def rel_max(a, ref):
    den = float(np.max(np.abs(ref))) if np.size(ref) else 0.0
    num = max_abs(a, ref)
    if den == 0.0:
        return num
    return num / den


def check_forward(res, ref, compute_entropy, label=""):
    e_lp = max_abs(res["logprob"], ref["logprob"])
    e_lse = max_abs(res["lse"], ref["lse"])
    msg = f"{label} logprob {e_lp:.3g} lse {e_lse:.3g}"
    assert np.all(np.isfinite(res["logprob"])) and np.all(np.isfinite(res["lse"])), msg
    assert e_lp <= FWD_ATOL and e_lse <= FWD_ATOL, msg
    if compute_entropy:
        e_ent = max_abs(res["entropy"], ref["entropy"])
        assert np.all(np.isfinite(res["entropy"])), label
        assert e_ent <= FWD_ATOL, f"{msg} entropy {e_ent:.3g}"
    return e_lp, e_lse


def check_grads(dX, dW, rdX, rdW, label=""):
    ex, ew = rel_max(dX, rdX), rel_max(dW, rdW)
    assert np.all(np.isfinite(dX)) and np.all(np.isfinite(dW)), label
    assert ex <= GRAD_RTOL and ew <= GRAD_RTOL, f"{label} dX rel {ex:.3g} dW rel {ew:.3g}"
    return ex, ew
