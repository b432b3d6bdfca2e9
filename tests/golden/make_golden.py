"""Write the oracle's expected values for the full-size workloads (configs 2-5).

Calls only the fp64 oracle (oracle/flce_ref.py) on the seeded inputs of
synth/inputs.py; nothing here touches the HIP library.  For each config it stores
  * logprob, lse, entropy of every row (float32 is ample for the 2e-3 tolerance),
  * dX for a sample of rows and dW for a sample of vocabulary entries (float32),
  * a SHA-256 fingerprint of the generated X, W and targets, so a test can
    confirm it regenerated exactly the same inputs.

    python tests/golden/make_golden.py [config ...]     # default: 2 3 4 5
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

N_SAMPLE = 16


def fingerprint(case) -> str:
    h = hashlib.sha256()
    for a in (case.X, case.W, case.targets):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def sample_rows(case, rng):
    M = case.M
    rows = set(rng.choice(M, size=min(M, N_SAMPLE - 4), replace=False).tolist())
    rows.update({0, M - 1})
    ign = np.where(case.targets == case.ignore_index)[0]
    if len(ign):
        rows.add(int(ign[0]))
    # the row with the largest-norm input (a x64 row where the config has them)
    norms = np.abs(inputs.decode_bf16_to_f32(case.X[: min(M, 4096)])).sum(1)
    rows.add(int(np.argmax(norms)))
    return np.array(sorted(rows), dtype=np.int64)


def sample_vocab(case, rng):
    V = case.V
    vs = set(rng.choice(V, size=min(V, N_SAMPLE - 4), replace=False).tolist())
    vs.update({0, V - 1})
    valid_t = case.targets[(case.targets >= 0) & (case.targets < V)]
    if len(valid_t):
        vs.update(int(x) for x in valid_t[:2])
    return np.array(sorted(vs), dtype=np.int64)


def make(cfg: int) -> str:
    t0 = time.time()
    case = inputs.config_case(cfg)
    rng = np.random.default_rng(np.random.SeedSequence([2026, cfg, 99]))
    rows = sample_rows(case, rng)
    vrows = sample_vocab(case, rng)
    Wd = ref.decode_bf16(case.W)
    fwd = ref.forward(case.X, case.W, case.targets, case.ignore_index, case.scale, True, Wd=Wd)
    print(f"config {cfg}: forward {time.time() - t0:.0f} s", flush=True)
    dx = ref.dx_rows(case.X, case.W, case.targets, rows, case.ignore_index, case.scale,
                     case.grad_logprob, case.grad_entropy, Wd=Wd)
    del Wd
    dw = ref.dw_rows(case.X, case.W, case.targets, vrows, case.ignore_index, case.scale,
                     fwd["lse"], fwd["E"], case.grad_logprob, case.grad_entropy)
    out = os.path.join(HERE, f"config{cfg}.npz")
    np.savez_compressed(
        out, fingerprint=np.array(fingerprint(case)), logprob=fwd["logprob"].astype(np.float32),
        lse=fwd["lse"].astype(np.float32), entropy=fwd["entropy"].astype(np.float32),
        dx_rows=rows, dx=dx.astype(np.float32), dw_rows=vrows, dw=dw.astype(np.float32),
        dx_absmax_sample=np.float64(np.abs(dx).max()))
    print(f"config {cfg}: wrote {out} in {time.time() - t0:.0f} s", flush=True)
    return out


if __name__ == "__main__":
    cfgs = [int(a) for a in sys.argv[1:]] or [2, 3, 4, 5]
    for c in cfgs:
        make(c)
