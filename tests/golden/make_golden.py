"""Write the oracle's expected values for the full-size workloads (configs 2-5).

Calls only the fp64 oracle (oracle/flce_ref.py, through tests/oracle_runner.py, which
runs the oracle's own functions on disjoint row ranges in worker processes) on the
seeded inputs of synth/inputs.py; nothing here touches the HIP library.  For each
config it stores
  * logprob, lse, entropy and E (the softmax-weighted mean logit) of every row, fp64;
  * the largest magnitude of every row of dX and of every row of dW (fp32) and the
    whole-tensor maxima max|dX| and max|dW| (fp64; the denominators of the
    relative-to-max tolerance on the gradients), from the oracle's dX of every token
    row and dW of every vocabulary entry;
  * a SHA-256 fingerprint of the generated X, W and targets, so a test can confirm
    it regenerated exactly the same inputs.
Before writing, a few rows of dX and dW are computed again by one plain call of the
oracle in this process and must match what the workers returned.

    python tests/golden/make_golden.py [--out DIR] [config ...]   # default: 2 3 4 5
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle import flce_ref as ref  # noqa: E402
from synth import inputs  # noqa: E402
from tests import oracle_runner as run  # noqa: E402


def fingerprint(case) -> str:
    h = hashlib.sha256()
    for a in (case.X, case.W, case.targets):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def make(cfg: int, out_dir: str = HERE) -> str:
    t0 = time.time()
    case = inputs.config_case(cfg)
    with run.Pool(case) as pool:
        parts = pool.map("forward", run.ranges(case.M, 4 * pool.workers),
                         label=f"config {cfg} forward")
    fwd = {k: np.concatenate([p[k] for p in parts]) for k in ("logprob", "lse", "entropy", "E")}
    with run.Pool(case, lse=fwd["lse"], E=fwd["E"]) as pool:
        n = 8 * pool.workers
        dx_rowmax = np.concatenate(pool.map("dx_rowmax", run.ranges(case.M, n),
                                            label=f"config {cfg} dX"))
        dw_rowmax = np.concatenate(pool.map("dw_rowmax", run.ranges(case.V, n),
                                            label=f"config {cfg} dW"))
    # cross-check a few rows with one plain oracle call in this process
    rng = np.random.default_rng(np.random.SeedSequence([2026, cfg, 98]))
    rows = np.sort(rng.choice(case.M, 6, replace=False))
    vrows = np.sort(np.concatenate([rng.choice(case.V, 5, replace=False),
                                    [int(np.argmax(dw_rowmax))]]))
    chk_dx = ref.dx_rows(case.X, case.W, case.targets, rows, case.ignore_index, case.scale,
                         case.grad_logprob, case.grad_entropy)
    chk_dw = ref.dw_rows(case.X, case.W, case.targets, vrows, case.ignore_index, case.scale,
                         fwd["lse"], fwd["E"], case.grad_logprob, case.grad_entropy)
    assert np.allclose(np.abs(chk_dx).max(1), dx_rowmax[rows], rtol=1e-12, atol=0)
    assert np.allclose(np.abs(chk_dw).max(1), dw_rowmax[vrows], rtol=1e-12, atol=0)
    out = os.path.join(out_dir, f"config{cfg}.npz")
    np.savez_compressed(
        out, fingerprint=np.array(fingerprint(case)),
        logprob=fwd["logprob"], lse=fwd["lse"], entropy=fwd["entropy"], E=fwd["E"],
        dx_absmax=np.float64(dx_rowmax.max()), dw_absmax=np.float64(dw_rowmax.max()),
        dx_rowmax=dx_rowmax.astype(np.float32), dw_rowmax=dw_rowmax.astype(np.float32))
    print(f"config {cfg}: wrote {out} in {time.time() - t0:.0f} s "
          f"(max|dX| {dx_rowmax.max():.6g}, max|dW| {dw_rowmax.max():.6g})", flush=True)
    return out


if __name__ == "__main__":
    args = sys.argv[1:]
    out_dir = HERE
    if args[:1] == ["--out"]:
        out_dir = args[1]
        os.makedirs(out_dir, exist_ok=True)
        args = args[2:]
    for c in [int(a) for a in args] or [2, 3, 4, 5]:
        make(c, out_dir)
