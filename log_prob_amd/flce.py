"""Thin ctypes binding of libflce (the C ABI in include/flce.h).

Only argument marshalling lives here: every step of the computation runs in the
HIP kernels of libflce.so.  torch supplies device memory and the current stream.
If the library is missing, loading fails loudly; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libflce.so")

FLCE_OK = 0
# bytes of the static device scratch flce_forward_noalloc uses (FLCE_NOALLOC_SCRATCH_BYTES)
FLCE_NOALLOC_SCRATCH_BYTES = 32 << 20
STATUS = {0: "FLCE_OK", 1: "FLCE_ERR_INVALID_VALUE", 2: "FLCE_ERR_UNSUPPORTED",
          3: "FLCE_ERR_WORKSPACE_TOO_SMALL", 4: "FLCE_ERR_HIP"}

# Every symbol include/flce.h declares.
EXPORTS = ("flce_workspace_query", "flce_forward_workspace_min", "flce_forward_wave_rows",
           "flce_backward_workspace_min", "flce_backward_chunk_cols",
           "flce_backward_wave_rows", "flce_backward_schedule", "flce_forward",
           "flce_forward_noalloc", "flce_forward_partials", "flce_forward_merge", "flce_backward",
           "flce_forward_partials_shard", "flce_forward_merge_shards",
           "flce_backward_shard_workspace_query", "flce_backward_shard", "flce_nll_reduce",
           "flce_nll_mean_grad", "flce_policy_loss_reduce", "flce_policy_loss_grad",
           "flce_status_string",
           "flce_last_error_message", "flce_version")

_lib = None


class FlceError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libflce.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libflce.so not built at {path}; run `python -m log_prob_amd.build`")
    lib = ctypes.CDLL(path)
    c = ctypes
    P, I64, SZ = c.c_void_p, c.c_int64, c.c_size_t
    lib.flce_workspace_query.argtypes = [I64, I64, I64, c.c_int, c.POINTER(SZ), c.POINTER(SZ)]
    lib.flce_forward_workspace_min.argtypes = [I64, I64, I64, c.c_int, c.POINTER(SZ)]
    lib.flce_forward_wave_rows.argtypes = [I64, I64, I64, c.c_int, SZ, c.POINTER(I64)]
    lib.flce_backward_workspace_min.argtypes = [I64, I64, I64, c.POINTER(SZ)]
    lib.flce_backward_chunk_cols.argtypes = [I64, I64, I64, SZ, c.POINTER(I64)]
    lib.flce_backward_wave_rows.argtypes = [I64, I64, I64, SZ, c.POINTER(I64)]
    lib.flce_backward_schedule.argtypes = [I64, I64, I64, SZ, c.POINTER(I64), c.POINTER(I64),
                                           c.POINTER(c.c_int)]
    lib.flce_forward.argtypes = [P, P, P, I64, I64, I64, I64, c.c_float, c.c_int, P, P, P, P, SZ, P]
    lib.flce_forward_noalloc.argtypes = [P, P, P, I64, I64, I64, I64, c.c_float, c.c_int, P, P, P,
                                         P]
    lib.flce_forward_partials.argtypes = [P, P, P, I64, I64, I64, I64, c.c_float, c.c_int, P, SZ,
                                          P]
    lib.flce_forward_merge.argtypes = [P, I64, I64, I64, I64, c.c_int, P, P, P, P, SZ, P]
    lib.flce_backward.argtypes = [P, P, P, I64, I64, I64, I64, c.c_float, P, P, P, P, P, P, P,
                                  SZ, P]
    lib.flce_forward_partials_shard.argtypes = [P, P, P, I64, I64, I64, I64, I64, c.c_float,
                                                c.c_int, P, SZ, P]
    lib.flce_forward_merge_shards.argtypes = [P, I64, I64, c.POINTER(I64), I64, c.c_int, P, P, P,
                                              P, SZ, P]
    lib.flce_backward_shard_workspace_query.argtypes = [I64, I64, I64, c.POINTER(SZ),
                                                        c.POINTER(SZ)]
    lib.flce_backward_shard.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, c.c_float, P, P, P,
                                        P, P, c.c_int, P, P, SZ, P]
    lib.flce_nll_reduce.argtypes = [P, P, I64, I64, I64, P, P]
    lib.flce_nll_mean_grad.argtypes = [P, I64, I64, I64, P, P, P]
    D = c.c_double
    lib.flce_policy_loss_reduce.argtypes = [P, P, P, P, I64, I64, I64, D, D, D, P, P, P, P]
    lib.flce_policy_loss_grad.argtypes = [P, P, P, P, I64, I64, I64, D, D, D, P, P, P]
    for name in ("flce_nll_reduce", "flce_nll_mean_grad", "flce_policy_loss_reduce",
                 "flce_policy_loss_grad", "flce_workspace_query",
                 "flce_forward_workspace_min", "flce_forward_wave_rows",
                 "flce_backward_workspace_min", "flce_backward_chunk_cols",
                 "flce_backward_wave_rows", "flce_backward_schedule", "flce_forward",
           "flce_forward_noalloc", "flce_forward_partials", "flce_forward_merge", "flce_backward",
                 "flce_forward_partials_shard", "flce_forward_merge_shards",
                 "flce_backward_shard_workspace_query", "flce_backward_shard"):
        getattr(lib, name).restype = c.c_int
    lib.flce_status_string.argtypes = [c.c_int]
    lib.flce_status_string.restype = c.c_char_p
    lib.flce_last_error_message.argtypes = []
    lib.flce_last_error_message.restype = c.c_char_p
    lib.flce_version.argtypes = []
    lib.flce_version.restype = c.c_char_p
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != FLCE_OK:
        raise FlceError(status, load().flce_last_error_message().decode())


def workspace_query(M: int, H: int, V: int, compute_entropy: bool = True) -> Tuple[int, int]:
    fwd, bwd = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().flce_workspace_query(M, H, V, int(bool(compute_entropy)), ctypes.byref(fwd),
                                       ctypes.byref(bwd)))
    return fwd.value, bwd.value


def forward_workspace_min(M: int, H: int, V: int, compute_entropy: bool = True) -> int:
    b = ctypes.c_size_t()
    _check(load().flce_forward_workspace_min(M, H, V, int(bool(compute_entropy)), ctypes.byref(b)))
    return b.value


def forward_wave_rows(M: int, H: int, V: int, workspace_bytes: int,
                      compute_entropy: bool = True) -> int:
    r = ctypes.c_int64()
    _check(load().flce_forward_wave_rows(M, H, V, int(bool(compute_entropy)), workspace_bytes,
                                         ctypes.byref(r)))
    return r.value


def backward_workspace_min(M: int, H: int, V: int) -> int:
    b = ctypes.c_size_t()
    _check(load().flce_backward_workspace_min(M, H, V, ctypes.byref(b)))
    return b.value


def backward_chunk_cols(M: int, H: int, V: int, workspace_bytes: int) -> int:
    c = ctypes.c_int64()
    _check(load().flce_backward_chunk_cols(M, H, V, workspace_bytes, ctypes.byref(c)))
    return c.value


def backward_wave_rows(M: int, H: int, V: int, workspace_bytes: int) -> int:
    r = ctypes.c_int64()
    _check(load().flce_backward_wave_rows(M, H, V, workspace_bytes, ctypes.byref(r)))
    return r.value


def backward_schedule(M: int, H: int, V: int, workspace_bytes: int):
    """(rows per token wave, chunk columns, pipelined) of flce_backward's schedule."""
    r, cc, pp = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int()
    _check(load().flce_backward_schedule(M, H, V, workspace_bytes, ctypes.byref(r),
                                         ctypes.byref(cc), ctypes.byref(pp)))
    return r.value, cc.value, bool(pp.value)


def backward_shard_workspace_query(M: int, H: int, V_shard: int) -> Tuple[int, int]:
    lo, pref = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load().flce_backward_shard_workspace_query(M, H, V_shard, ctypes.byref(lo),
                                                      ctypes.byref(pref)))
    return lo.value, pref.value


# ----------------------------------------------------------------------------
# torch-facing wrappers
def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _require(t, name, dtype, shape):
    import torch
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def alloc_workspace(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def forward(X, W, targets, ignore_index: int = -100, scale: float = 1.0,
            compute_entropy: bool = True, workspace=None, out=None):
    """(logprob, lse, entropy-or-None) as fp32 [M] tensors, on X's device and stream."""
    import torch
    M, H = X.shape
    V = W.shape[0]
    _require(X, "X", torch.bfloat16, (M, H))
    _require(W, "W", torch.bfloat16, (V, H))
    _require(targets, "targets", torch.int64, (M,))
    dev = X.device
    if out is None:
        logprob = torch.empty(M, dtype=torch.float32, device=dev)
        lse = torch.empty(M, dtype=torch.float32, device=dev)
        entropy = torch.empty(M, dtype=torch.float32, device=dev) if compute_entropy else None
    else:
        logprob, lse, entropy = out
    if workspace is None:
        fwd_b, _ = workspace_query(M, H, V, compute_entropy)
        workspace = alloc_workspace(fwd_b, dev)
    _check(load().flce_forward(_ptr(X), _ptr(W), _ptr(targets), M, H, V, int(ignore_index),
                               float(scale), int(bool(compute_entropy)), _ptr(logprob), _ptr(lse),
                               _ptr(entropy), _ptr(workspace), workspace.numel(), _stream(dev)))
    return logprob, lse, entropy


def forward_noalloc(X, W, targets, ignore_index: int = -100, scale: float = 1.0,
                    compute_entropy: bool = True, out=None):
    """flce_forward_noalloc: the forward through the library's static device scratch (no
    workspace).  With `out` = (logprob, lse, entropy-or-None) nothing is allocated here
    either; calls overlapping on one GPU share the scratch and must not run concurrently."""
    import torch
    M, H = X.shape
    V = W.shape[0]
    _require(X, "X", torch.bfloat16, (M, H))
    _require(W, "W", torch.bfloat16, (V, H))
    _require(targets, "targets", torch.int64, (M,))
    dev = X.device
    if out is None:
        logprob = torch.empty(M, dtype=torch.float32, device=dev)
        lse = torch.empty(M, dtype=torch.float32, device=dev)
        entropy = torch.empty(M, dtype=torch.float32, device=dev) if compute_entropy else None
    else:
        logprob, lse, entropy = out
    _check(load().flce_forward_noalloc(_ptr(X), _ptr(W), _ptr(targets), M, H, V,
                                       int(ignore_index), float(scale),
                                       int(bool(compute_entropy)), _ptr(logprob), _ptr(lse),
                                       _ptr(entropy), _stream(dev)))
    return logprob, lse, entropy


def forward_partials(X, W, targets, ignore_index: int = -100, scale: float = 1.0,
                     compute_entropy: bool = True, workspace=None):
    """Run only the fused GEMM + online-softmax kernel; partials stay in `workspace`."""
    import torch
    M, H = X.shape
    V = W.shape[0]
    _require(X, "X", torch.bfloat16, (M, H))
    _require(W, "W", torch.bfloat16, (V, H))
    _require(targets, "targets", torch.int64, (M,))
    if workspace is None:
        workspace = alloc_workspace(workspace_query(M, H, V, compute_entropy)[0], X.device)
    _check(load().flce_forward_partials(_ptr(X), _ptr(W), _ptr(targets), M, H, V,
                                        int(ignore_index), float(scale),
                                        int(bool(compute_entropy)), _ptr(workspace),
                                        workspace.numel(), _stream(X.device)))
    return workspace


def forward_merge(targets, M: int, H: int, V: int, workspace, ignore_index: int = -100,
                  compute_entropy: bool = True, out=None):
    """Merge partials left by forward_partials into (logprob, lse, entropy-or-None)."""
    import torch
    _require(targets, "targets", torch.int64, (M,))
    dev = targets.device
    if out is None:
        logprob = torch.empty(M, dtype=torch.float32, device=dev)
        lse = torch.empty(M, dtype=torch.float32, device=dev)
        entropy = torch.empty(M, dtype=torch.float32, device=dev) if compute_entropy else None
    else:
        logprob, lse, entropy = out
    _check(load().flce_forward_merge(_ptr(targets), M, H, V, int(ignore_index),
                                     int(bool(compute_entropy)), _ptr(logprob), _ptr(lse),
                                     _ptr(entropy), _ptr(workspace), workspace.numel(),
                                     _stream(dev)))
    return logprob, lse, entropy


def backward(X, W, targets, lse, entropy=None, grad_logprob=None, grad_entropy=None,
             ignore_index: int = -100, scale: float = 1.0, workspace=None, out=None):
    """(dX, dW) as bf16 tensors shaped like X and W."""
    import torch
    M, H = X.shape
    V = W.shape[0]
    _require(X, "X", torch.bfloat16, (M, H))
    _require(W, "W", torch.bfloat16, (V, H))
    _require(targets, "targets", torch.int64, (M,))
    _require(lse, "lse", torch.float32, (M,))
    for name, t in (("entropy", entropy), ("grad_logprob", grad_logprob),
                    ("grad_entropy", grad_entropy)):
        if t is not None:
            _require(t, name, torch.float32, (M,))
    dev = X.device
    if out is None:
        dX = torch.empty_like(X)
        dW = torch.empty_like(W)
    else:
        dX, dW = out
    if workspace is None:
        _, bwd_b = workspace_query(M, H, V, entropy is not None)
        workspace = alloc_workspace(bwd_b, dev)
    _check(load().flce_backward(_ptr(X), _ptr(W), _ptr(targets), M, H, V, int(ignore_index),
                                float(scale), _ptr(lse), _ptr(entropy), _ptr(grad_logprob),
                                _ptr(grad_entropy), _ptr(dX), _ptr(dW), _ptr(workspace),
                                workspace.numel(), _stream(dev)))
    return dX, dW


# ----------------------------------------------------------------------------
# vocabulary shards: what one rank of a vocabulary-parallel group runs
def forward_partials_shard(X, W_shard, targets, v_offset: int, ignore_index: int = -100,
                           scale: float = 1.0, compute_entropy: bool = True, workspace=None):
    """Partials of the shard W_shard = rows [v_offset, v_offset + V_shard) of W."""
    import torch
    M, H = X.shape
    Vs = W_shard.shape[0]
    _require(X, "X", torch.bfloat16, (M, H))
    _require(W_shard, "W_shard", torch.bfloat16, (Vs, H))
    _require(targets, "targets", torch.int64, (M,))
    if workspace is None:
        workspace = alloc_workspace(workspace_query(M, H, Vs, compute_entropy)[0], X.device)
    _check(load().flce_forward_partials_shard(_ptr(X), _ptr(W_shard), _ptr(targets), M, H, Vs,
                                              int(v_offset), int(ignore_index), float(scale),
                                              int(bool(compute_entropy)), _ptr(workspace),
                                              workspace.numel(), _stream(X.device)))
    return workspace


def forward_merge_shards(targets, shard_offsets, gathered, shard_stride_bytes: int,
                         ignore_index: int = -100, compute_entropy: bool = True, out=None):
    """Merge gathered shard partials (shard r at byte r * stride of `gathered`)."""
    import torch
    M = targets.shape[0]
    _require(targets, "targets", torch.int64, (M,))
    offs = (ctypes.c_int64 * len(shard_offsets))(*[int(v) for v in shard_offsets])
    dev = targets.device
    if out is None:
        logprob = torch.empty(M, dtype=torch.float32, device=dev)
        lse = torch.empty(M, dtype=torch.float32, device=dev)
        entropy = torch.empty(M, dtype=torch.float32, device=dev) if compute_entropy else None
    else:
        logprob, lse, entropy = out
    _check(load().flce_forward_merge_shards(_ptr(targets), M, len(shard_offsets) - 1, offs,
                                            int(ignore_index), int(bool(compute_entropy)),
                                            _ptr(logprob), _ptr(lse), _ptr(entropy),
                                            _ptr(gathered), int(shard_stride_bytes),
                                            _stream(dev)))
    return logprob, lse, entropy


def backward_shard(X, W_shard, targets, v_offset: int, V_total: int, lse, entropy=None,
                   grad_logprob=None, grad_entropy=None, dX_partial=None, accumulate=False,
                   ignore_index: int = -100, scale: float = 1.0, workspace=None, dW_shard=None):
    """(dX_partial fp32 [M, H], dW_shard bf16) of one shard; dX is the sum over shards."""
    import torch
    M, H = X.shape
    Vs = W_shard.shape[0]
    _require(X, "X", torch.bfloat16, (M, H))
    _require(W_shard, "W_shard", torch.bfloat16, (Vs, H))
    _require(targets, "targets", torch.int64, (M,))
    _require(lse, "lse", torch.float32, (M,))
    for name, t in (("entropy", entropy), ("grad_logprob", grad_logprob),
                    ("grad_entropy", grad_entropy)):
        if t is not None:
            _require(t, name, torch.float32, (M,))
    dev = X.device
    if dX_partial is None:
        dX_partial = torch.empty((M, H), dtype=torch.float32, device=dev)
    _require(dX_partial, "dX_partial", torch.float32, (M, H))
    if dW_shard is None:
        dW_shard = torch.empty_like(W_shard)
    if workspace is None:
        workspace = alloc_workspace(backward_shard_workspace_query(M, H, Vs)[1], dev)
    _check(load().flce_backward_shard(_ptr(X), _ptr(W_shard), _ptr(targets), M, H, Vs,
                                      int(v_offset), int(V_total), int(ignore_index),
                                      float(scale), _ptr(lse), _ptr(entropy),
                                      _ptr(grad_logprob), _ptr(grad_entropy), _ptr(dX_partial),
                                      int(bool(accumulate)), _ptr(dW_shard), _ptr(workspace),
                                      workspace.numel(), _stream(dev)))
    return dX_partial, dW_shard


# ----------------------------------------------------------------------------
# scalar cross-entropy reductions on the log-probs
def nll_reduce(logprob, targets, V: int, ignore_index: int = -100, out=None):
    """fp64 device tensor [sum of -logprob over valid rows, valid rows, mean NLL]."""
    import torch
    M = logprob.shape[0]
    _require(logprob, "logprob", torch.float32, (M,))
    _require(targets, "targets", torch.int64, (M,))
    if out is None:
        out = torch.empty(3, dtype=torch.float64, device=logprob.device)
    _require(out, "out", torch.float64, (3,))
    _check(load().flce_nll_reduce(_ptr(logprob), _ptr(targets), M, int(V), int(ignore_index),
                                  _ptr(out), _stream(logprob.device)))
    return out


def nll_mean_grad(targets, V: int, reduced, ignore_index: int = -100, out=None):
    """grad_logprob of the mean NLL (-1/n on valid rows) from nll_reduce's output."""
    import torch
    M = targets.shape[0]
    _require(targets, "targets", torch.int64, (M,))
    _require(reduced, "reduced", torch.float64, (3,))
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=targets.device)
    _require(out, "grad_logprob", torch.float32, (M,))
    _check(load().flce_nll_mean_grad(_ptr(targets), M, int(V), int(ignore_index), _ptr(reduced),
                                     _ptr(out), _stream(targets.device)))
    return out


def _policy_inputs(logprob, old_logprob, advantages, targets):
    import torch
    M = logprob.shape[0]
    _require(logprob, "logprob", torch.float32, (M,))
    if old_logprob is not None:
        _require(old_logprob, "old_logprob", torch.float32, (M,))
    _require(advantages, "advantages", torch.float32, (M,))
    _require(targets, "targets", torch.int64, (M,))
    return M


def policy_loss_reduce(logprob, old_logprob, advantages, targets, V: int,
                       ignore_index: int = -100, eps_low: float = 0.2, eps_high: float = 0.2,
                       denominator: float = 0.0, with_clip_flags: bool = True, out=None):
    """Clipped policy loss on the log-probs, token-mean aggregated (see include/flce.h):
    (per-token loss fp32 [M], clip flags uint8 [M] or None, fp64 device tensor [loss sum,
    valid rows, clipped rows, loss sum / N]).  `out` may supply those three buffers."""
    import torch
    M = _policy_inputs(logprob, old_logprob, advantages, targets)
    dev = logprob.device
    if out is not None:
        per_token, clipped, out = out
    else:
        per_token = torch.empty(M, dtype=torch.float32, device=dev)
        clipped = torch.empty(M, dtype=torch.uint8, device=dev) if with_clip_flags else None
        out = torch.empty(4, dtype=torch.float64, device=dev)
    _require(per_token, "per_token_loss", torch.float32, (M,))
    if clipped is not None:
        _require(clipped, "is_clipped", torch.uint8, (M,))
    _require(out, "out", torch.float64, (4,))
    _check(load().flce_policy_loss_reduce(
        _ptr(logprob), _ptr(old_logprob), _ptr(advantages), _ptr(targets), M, int(V),
        int(ignore_index), float(eps_low), float(eps_high), float(denominator), _ptr(per_token),
        _ptr(clipped), _ptr(out), _stream(dev)))
    return per_token, clipped, out


def policy_loss_grad(logprob, old_logprob, advantages, targets, V: int, reduced=None,
                     ignore_index: int = -100, eps_low: float = 0.2, eps_high: float = 0.2,
                     denominator: float = 0.0, out=None):
    """grad_logprob of the loss of policy_loss_reduce; `reduced` is its fp64 output
    (needed when denominator <= 0)."""
    import torch
    M = _policy_inputs(logprob, old_logprob, advantages, targets)
    if out is None:
        out = torch.empty(M, dtype=torch.float32, device=logprob.device)
    _require(out, "grad_logprob", torch.float32, (M,))
    if reduced is not None:
        _require(reduced, "reduced", torch.float64, (4,))
    _check(load().flce_policy_loss_grad(
        _ptr(logprob), _ptr(old_logprob), _ptr(advantages), _ptr(targets), M, int(V),
        int(ignore_index), float(eps_low), float(eps_high), float(denominator), _ptr(reduced),
        _ptr(out), _stream(logprob.device)))
    return out
