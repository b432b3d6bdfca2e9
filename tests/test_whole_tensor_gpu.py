"""Every element of dX and dW of the full-size workloads 2-5 against the fp64 oracle,
in the launch configuration bench.py times.

The oracle runs here, on the host, in worker processes (tests/oracle_runner.py) over
disjoint pieces: dX over ranges of token rows (each row's d-logits need only that
row), dW over ranges of vocabulary entries (each entry's column of d-logits needs
every token's lse and E, taken from the oracle's stored forward,
tests/golden/config*.npz).  Each piece is its own test so that progress is visible;
the GPU outputs of a workload are computed once and kept on the host while its pieces
run.  Errors are relative to the maximum magnitude of the oracle's whole tensor
(stored by make_golden.py), and each piece also checks that its own oracle values
stay within that maximum."""
import numpy as np
import pytest

from synth import inputs
from tests import gpu_util as gu
from tests import oracle_runner as run
from tests.test_configs_gpu import golden, run_config

pytestmark = pytest.mark.gpu

# pieces per workload and tensor: a test each, about 10-20 s of oracle work on 16 cores
PIECES = {2: 1, 3: 2, 4: 4, 5: 8}
_STATE = {}


def _state(cfg):
    if _STATE.get("cfg") != cfg:
        if "pool" in _STATE:
            _STATE["pool"].close()
        _STATE.clear()
        case = inputs.config_case(cfg)
        res = run_config(case)
        g = golden(cfg)
        pool = run.Pool(case, lse=g["lse"], E=g["E"], gdX=res["dX"], gdW=res["dW"])
        _STATE.update(cfg=cfg, case=case, g=g, pool=pool)
    return _STATE


@pytest.fixture(scope="module", autouse=True)
def _close_pool():
    yield
    if "pool" in _STATE:
        _STATE["pool"].close()
    _STATE.clear()


CASES = [(c, kind, k) for c in sorted(PIECES) for kind in ("dX", "dW") for k in range(PIECES[c])]


@pytest.mark.parametrize("cfg,kind,part", CASES, ids=[f"c{c}-{t}-{k}" for c, t, k in CASES])
def test_whole_tensor(cfg, kind, part):
    st = _state(cfg)
    case, g, pool = st["case"], st["g"], st["pool"]
    n = case.M if kind == "dX" else case.V
    r0, r1 = run.ranges(n, PIECES[cfg])[part]
    print(f"[whole] config {cfg} {kind} rows [{r0}, {r1})", flush=True)
    sub = [(r0 + a, r0 + b) for a, b in run.ranges(r1 - r0, 2 * pool.workers)]
    res = pool.map("dx_cmp" if kind == "dX" else "dw_cmp", sub)
    err = max(e for e, _ in res)
    big = max(m for _, m in res)
    den = float(g["dx_absmax"] if kind == "dX" else g["dw_absmax"])
    print(f"[whole] config {cfg} {kind} rows [{r0}, {r1}): rel {err / den:.3g}", flush=True)
    assert big <= den * (1 + 1e-9), (big, den)
    assert err / den <= gu.GRAD_RTOL, f"config {cfg} {kind} [{r0}, {r1}): rel {err / den:.3g}"
