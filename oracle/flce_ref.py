"""fp64 CPU oracle for the fused LM-head linear + cross-entropy (log-prob) path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or load
this module: only the tests, the smoke check of the graft entry point and the
CPU-baseline leg of the benchmark do.  It shares no code with the HIP library.

What it computes is the plain definition, written out with the [rows, V]
logits materialised (in row blocks) and every step in float64:

  z[m, v]   = s * sum_k X[m, k] * W[v, k]        logits of a scaled linear head
  lse[m]    = log sum_v exp(z[m, v])             (two passes: max, then sum)
  logprob   = z[m, t[m]] - lse[m]                per-token target log-prob
  entropy   = -sum_v p log p,  p = softmax(z)    optional
  dZ        = a (onehot(t) - p) + b p (E - z),   E = sum_v p z
  dX        = s dZ W,   dW = s dZ^T X

Sources (web pages; cited by title and section):
* Liger-Kernel commit "native Blackwell tensor-parallel fused scaled linear
  cross-entropy" (mirror page of Liger-Kernel test/transformers, tag v0.8.3),
  section "Summary": the classifier GEMM fused with NLL/LSE and optional
  entropy; "Performance methodology": bf16 inputs, fp32 accumulation, four
  classifier GEMMs (logits, recomputed logits for dZ, dX, dW).
* SkyRL PR 2141 "perf(megatron): autotune fused LM-head Triton kernels",
  sections "Summary" and "Overview": per-token log-probs and optional entropy
  (compute_entropy), LSE seeded from the true row maximum.
* Liger-Kernel PR 1294 "Triton MoE improvements and chunked GRPO improvements",
  section "Chunked Triton GRPO loss": the (N, V) logits are never materialised
  by the method (the oracle does materialise them; that is its point), and
  "Correctness": per-token logp/lse are checked against an fp32 ground truth.

Readings where the pages are silent (each is listed in the design notes):
* the scale multiplies the fp32 accumulator of bf16 products (temperature
  applied to the logits, not to the inputs); the oracle uses float64(float32(s));
* natural logarithms; entropy of softmax(z) after the scale;
* a row is valid iff t != ignore_index and 0 <= t < V.  Invalid rows get
  logprob = 0, entropy = 0, a zero d-logit row, so they add nothing to dX or
  dW; lse is still the row's true value;
* grad_logprob is dL/dlogprob (so the NLL case is grad_logprob = -1) and
  grad_entropy is dL/dentropy; the entropy gradient is p_j (E - z_j).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "decode_bf16", "valid_rows", "logits", "from_logits", "forward_f64", "forward",
    "forward_rows", "backward_f64", "backward", "dx_rows", "dw_rows", "row_block",
    "nll_reduce", "nll_mean_grad", "policy_loss", "policy_loss_grad",
]


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  Exact: bf16 is the top half of fp32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def valid_rows(t: np.ndarray, V: int, ignore_index: int) -> np.ndarray:
    """Rows that take part in the loss: not ignore_index and a target in [0, V)."""
    t = np.asarray(t, dtype=np.int64)
    return (t != ignore_index) & (t >= 0) & (t < V)


def logits(Xd: np.ndarray, Wd: np.ndarray, scale: float) -> np.ndarray:
    """z = s * X W^T in float64 (s is the float32 scale widened to float64)."""
    s = float(np.float64(np.float32(scale)))
    return s * (Xd @ Wd.T)


def from_logits(Z: np.ndarray, t: np.ndarray, ignore_index: int, compute_entropy: bool = True,
                grad_logprob=None, grad_entropy=None) -> dict:
    """Every per-token quantity of the method, given materialised logits Z [R, V].

    Returns logprob, lse, entropy (None if not requested and not needed), E
    (the softmax-weighted mean logit) and, if any grad is given, dZ.
    """
    Z = np.asarray(Z, dtype=np.float64)
    R, V = Z.shape
    t = np.asarray(t, dtype=np.int64)
    valid = valid_rows(t, V, ignore_index)
    # two-pass log-sum-exp: exact row maximum first, then the shifted sum
    zmax = Z.max(axis=1)
    lse = zmax + np.log(np.exp(Z - zmax[:, None]).sum(axis=1))
    logP = Z - lse[:, None]
    P = np.exp(logP)
    safe_t = np.where(valid, t, 0)
    z_t = Z[np.arange(R), safe_t]
    logprob = np.where(valid, z_t - lse, 0.0)
    E = (P * Z).sum(axis=1)
    need_ent = compute_entropy or grad_entropy is not None
    entropy = None
    if need_ent:
        # Shannon entropy in nats of the softmax distribution
        entropy = np.where(valid, -(P * logP).sum(axis=1), 0.0)
    out = dict(logprob=logprob, lse=lse, entropy=entropy if compute_entropy else None,
               E=E, valid=valid)
    if grad_logprob is not None or grad_entropy is not None:
        a = np.zeros(R) if grad_logprob is None else np.asarray(grad_logprob, np.float64)
        b = np.zeros(R) if grad_entropy is None else np.asarray(grad_entropy, np.float64)
        a = np.where(valid, a, 0.0)
        b = np.where(valid, b, 0.0)
        dZ = -a[:, None] * P
        dZ[np.arange(R)[valid], t[valid]] += a[valid]
        dZ += b[:, None] * P * (E[:, None] - Z)
        out["dZ"] = dZ
    return out


# Bytes of one [rows, V] float64 logit block.  Only the memory footprint depends on it:
# rows are independent, so the blocks' results are the rows' results.  The pins force
# small values so that every row loop runs over many blocks.
ROW_BLOCK_BYTES = 1 << 29


def row_block(V: int, budget_bytes=None) -> int:
    """Rows per block so that one [rows, V] float64 block stays within the budget."""
    b = ROW_BLOCK_BYTES if budget_bytes is None else budget_bytes
    return max(1, int(b // (8 * max(V, 1))))


def forward_f64(Xd, Wd, t, ignore_index, scale, compute_entropy=True):
    """logprob, lse, entropy (None if off) and E for every row, from float64 X and W."""
    Xd = np.asarray(Xd, np.float64)
    Wd = np.asarray(Wd, np.float64)
    M, V = Xd.shape[0], Wd.shape[0]
    t = np.asarray(t, np.int64)
    res = {k: np.zeros(M) for k in ("logprob", "lse", "entropy", "E")}
    step = row_block(V)
    for r0 in range(0, M, step):
        r = slice(r0, min(M, r0 + step))
        o = from_logits(logits(Xd[r], Wd, scale), t[r], ignore_index, True)
        for k in res:
            res[k][r] = o[k]
    if not compute_entropy:
        res["entropy"] = None
    return res


def forward_rows(X_bits, W_bits, t, rows, ignore_index, scale, compute_entropy=True, Wd=None):
    """Forward outputs for a subset of rows (rows are independent of each other)."""
    rows = np.asarray(rows, dtype=np.int64)
    Wd = decode_bf16(W_bits) if Wd is None else Wd
    return forward_f64(decode_bf16(X_bits[rows]), Wd, np.asarray(t, np.int64)[rows],
                       ignore_index, scale, compute_entropy)


def forward(X_bits, W_bits, t, ignore_index, scale, compute_entropy=True, Wd=None):
    """logprob, lse, entropy (and E) for every row, from bf16 bit arrays."""
    Wd = decode_bf16(W_bits) if Wd is None else Wd
    return forward_f64(decode_bf16(X_bits), Wd, t, ignore_index, scale, compute_entropy)


def _ab(rows, valid, grad_logprob, grad_entropy):
    a = np.zeros(len(rows)) if grad_logprob is None else np.asarray(grad_logprob, np.float64)[rows]
    b = np.zeros(len(rows)) if grad_entropy is None else np.asarray(grad_entropy, np.float64)[rows]
    return np.where(valid, a, 0.0), np.where(valid, b, 0.0)


def backward_f64(Xd, Wd, t, ignore_index, scale, grad_logprob=None, grad_entropy=None):
    """dX [M, H] and dW [V, H] in float64 from float64 X and W (row-blocked)."""
    Xd = np.asarray(Xd, np.float64)
    Wd = np.asarray(Wd, np.float64)
    M, H = Xd.shape
    V = Wd.shape[0]
    s = float(np.float64(np.float32(scale)))
    dX = np.zeros((M, H))
    dW = np.zeros((V, H))
    step = row_block(V)
    for r0 in range(0, M, step):
        r = np.arange(r0, min(M, r0 + step))
        Xr = Xd[r]
        Z = logits(Xr, Wd, scale)
        o = from_logits(Z, t[r], ignore_index, False,
                        grad_logprob=np.zeros(len(r)) if grad_logprob is None else np.asarray(grad_logprob)[r],
                        grad_entropy=None if grad_entropy is None else np.asarray(grad_entropy)[r])
        dZ = o["dZ"]
        dX[r] = s * (dZ @ Wd)
        dW += s * (dZ.T @ Xr)
    return dX, dW


def backward(X_bits, W_bits, t, ignore_index, scale, grad_logprob=None, grad_entropy=None):
    """dX [M, H] and dW [V, H] in float64 from bf16 bit arrays."""
    return backward_f64(decode_bf16(X_bits), decode_bf16(W_bits), t, ignore_index, scale,
                        grad_logprob, grad_entropy)


def dx_rows(X_bits, W_bits, t, rows, ignore_index, scale, grad_logprob=None, grad_entropy=None,
            Wd=None):
    """dX for a subset of rows: each needs only its own row of d-logits."""
    rows = np.asarray(rows, dtype=np.int64)
    Wd = decode_bf16(W_bits) if Wd is None else Wd
    s = float(np.float64(np.float32(scale)))
    out = np.zeros((len(rows), Wd.shape[1]))
    step = row_block(Wd.shape[0])
    for i in range(0, len(rows), step):
        r = rows[i:i + step]
        Z = logits(decode_bf16(X_bits[r]), Wd, scale)
        o = from_logits(Z, t[r], ignore_index, False,
                        grad_logprob=np.zeros(len(r)) if grad_logprob is None else np.asarray(grad_logprob)[r],
                        grad_entropy=None if grad_entropy is None else np.asarray(grad_entropy)[r])
        out[i:i + step] = s * (o["dZ"] @ Wd)
    return out


def dw_rows(X_bits, W_bits, t, vrows, ignore_index, scale, lse, E,
            grad_logprob=None, grad_entropy=None):
    """dW rows for a subset of vocabulary entries.

    Column v of the d-logits needs every token's lse and E, which the caller
    passes from this module's own forward().  dW[v] = s * sum_m dZ[m, v] X[m].
    """
    vrows = np.asarray(vrows, dtype=np.int64)
    Xd = decode_bf16(X_bits)
    M = Xd.shape[0]
    V = W_bits.shape[0]
    s = float(np.float64(np.float32(scale)))
    t = np.asarray(t, np.int64)
    valid = valid_rows(t, V, ignore_index)
    a, b = _ab(np.arange(M), valid, grad_logprob, grad_entropy)
    lse = np.asarray(lse, np.float64)
    E = np.asarray(E, np.float64)
    out = np.zeros((len(vrows), Xd.shape[1]))
    step = row_block(M)                             # entries per [M, entries] block
    for i in range(0, len(vrows), step):
        vb = vrows[i:i + step]
        Zc = logits(Xd, decode_bf16(W_bits[vb]), scale)   # [M, len(vb)]
        Pc = np.exp(Zc - lse[:, None])
        onehot = (t[:, None] == vb[None, :]) & valid[:, None]
        dZc = a[:, None] * (onehot - Pc) + b[:, None] * Pc * (E[:, None] - Zc)
        out[i:i + step] = s * (dZc.T @ Xd)
    return out


def nll_reduce(logprob, t, V, ignore_index):
    """Scalar cross-entropy reductions over the valid rows: (sum of -logprob, number of
    valid rows, their mean; NaN when no row is valid).

    The mean token-level NLL is the usual scalar loss of the fused linear
    cross-entropy (Liger-Kernel commit "native Blackwell tensor-parallel fused scaled
    linear cross-entropy", "Summary": NLL fused with the classifier GEMM); SkyRL PR
    2141, "Summary", keeps such reductions out of the per-token log-prob kernels, so
    here they run on the log-probs.
    """
    valid = valid_rows(t, V, ignore_index)
    lp = np.asarray(logprob, np.float64)
    total = float(-np.sum(lp[valid]))
    n = int(np.count_nonzero(valid))
    return total, n, (total / n if n else float("nan"))


def nll_mean_grad(t, V, ignore_index, n_valid):
    """dL/dlogprob of L = mean NLL over the valid rows: -1/n on valid rows, 0 elsewhere."""
    valid = valid_rows(t, V, ignore_index)
    g = np.zeros(len(valid))
    if n_valid:
        g[valid] = -1.0 / n_valid
    return g


def policy_loss(logprob, old_logprob, advantages, t, V, ignore_index, eps_low, eps_high,
                denominator=0.0):
    """Clipped policy-gradient loss on the per-token log-probs, token-mean aggregated.

    Liger-Kernel PR 1294, "Chunked Triton GRPO loss": the loss sits on the per-token
    log-probs of the fused linear path ("Setup": loss_type "dapo", clip eps 0.2/0.2,
    num_items_in_batch; "Correctness": per-token loss and is_clipped outputs).  The page
    names these settings without formulas; the reading here is the plainest one, the
    clipped surrogate of proximal policy optimisation with a token-level ratio and the
    DAPO token mean:

      r_m   = exp(logprob_m - old_logprob_m)       (old_logprob None: r = 1)
      c_m   = min(max(r_m, 1 - eps_low), 1 + eps_high)
      l_m   = -min(r_m A_m, c_m A_m)               per-token loss, 0 on invalid rows
      clip_m = c_m A_m < r_m A_m                   the minimum takes the clipped term
      L     = sum of l_m over valid rows / N,      N = denominator if > 0, else the
                                                   number of valid rows

    Returns (per_token_loss [M], is_clipped bool [M], sum of l_m, valid rows, clipped
    rows, L; NaN when N is 0).  Everything in float64.
    """
    valid = valid_rows(t, V, ignore_index)
    lp = np.asarray(logprob, np.float64)
    old = lp if old_logprob is None else np.asarray(old_logprob, np.float64)
    A = np.asarray(advantages, np.float64)
    r = np.exp(lp - old)
    c = np.minimum(np.maximum(r, 1.0 - float(eps_low)), 1.0 + float(eps_high))
    unclipped, clipped = r * A, c * A
    loss = np.where(valid, -np.minimum(unclipped, clipped), 0.0)
    is_clipped = valid & (clipped < unclipped)
    n = int(np.count_nonzero(valid))
    total = float(np.sum(loss))
    N = float(denominator) if denominator > 0 else float(n)
    return (loss, is_clipped, total, n, int(np.count_nonzero(is_clipped)),
            total / N if N > 0 else float("nan"))


def policy_loss_grad(logprob, old_logprob, advantages, t, V, ignore_index, eps_low, eps_high,
                     N):
    """dL/dlogprob of the token-mean clipped loss above: -r_m A_m / N on valid rows whose
    minimum takes the unclipped term (d r_m / d logprob_m = r_m), 0 on clipped and
    invalid rows and everywhere when N is 0."""
    loss, is_clipped, _, _, _, _ = policy_loss(logprob, old_logprob, advantages, t, V,
                                               ignore_index, eps_low, eps_high)
    valid = valid_rows(t, V, ignore_index)
    lp = np.asarray(logprob, np.float64)
    old = lp if old_logprob is None else np.asarray(old_logprob, np.float64)
    r = np.exp(lp - old)
    g = np.zeros(len(valid))
    if N > 0:
        keep = valid & ~is_clipped
        g[keep] = -r[keep] * np.asarray(advantages, np.float64)[keep] / float(N)
    return g
