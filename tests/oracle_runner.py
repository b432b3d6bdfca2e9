"""Run the fp64 oracle over many rows in worker processes (test infrastructure only).

Rows are independent in every function of the oracle, so a large workload is split
into disjoint row (or vocabulary-entry) ranges and each worker process calls the
oracle's own functions on one range.  The workers are fresh interpreters (spawned: no
GPU state, no torch) that memory-map the case's arrays from files the parent writes,
so nothing large is copied through pipes, and each worker's BLAS has its own share of
the host cores.  (Worker threads in one process were tried first and gave some wrong
dW rows on a larger host; separate processes share no BLAS state.)
Nothing here computes any part of the method itself; the workers return either the
oracle's values for their range or, to keep the traffic small, their comparison with
the GPU's values for the same range (largest difference, largest oracle magnitude) or
the largest magnitude of each row.
"""
from __future__ import annotations

import atexit
import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import sys
import tempfile
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def cores() -> int:
    return len(os.sched_getaffinity(0))


def ranges(n: int, parts: int):
    b = np.linspace(0, n, parts + 1).astype(np.int64)
    return [(int(a), int(c)) for a, c in zip(b[:-1], b[1:]) if c > a]


# ---------------------------------------------------------------------------------
# worker side: module globals set by _init in each worker process
_G = {}


def _init(paths, scalars, blas_threads):
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    from threadpoolctl import threadpool_limits
    _G["limits"] = threadpool_limits(limits=blas_threads, user_api="blas")
    _G.update({k: (None if p is None else np.load(p, mmap_mode="r")) for k, p in paths.items()})
    _G.update(scalars)


def _wd():
    from oracle import flce_ref as ref
    if "Wd" not in _G:
        _G["Wd"] = ref.decode_bf16(_G["W"])
    return _G["Wd"]


def _grads():
    return _G.get("glp"), _G.get("gent")


def _forward(a, b):
    from oracle import flce_ref as ref
    o = ref.forward_f64(ref.decode_bf16(_G["X"][a:b]), _wd(), np.asarray(_G["t"][a:b]),
                        _G["ignore_index"], _G["scale"], True)
    return {k: o[k] for k in ("logprob", "lse", "entropy", "E")}


def _dx(rows):
    from oracle import flce_ref as ref
    glp, gent = _grads()
    return ref.dx_rows(_G["X"], _G["W"], np.asarray(_G["t"]), np.asarray(rows), _G["ignore_index"],
                       _G["scale"], None if glp is None else np.asarray(glp),
                       None if gent is None else np.asarray(gent), Wd=_wd())


def _dw(vrows):
    from oracle import flce_ref as ref
    glp, gent = _grads()
    return ref.dw_rows(_G["X"], _G["W"], np.asarray(_G["t"]), np.asarray(vrows),
                       _G["ignore_index"], _G["scale"], np.asarray(_G["lse"]), np.asarray(_G["E"]),
                       None if glp is None else np.asarray(glp),
                       None if gent is None else np.asarray(gent))


def _bits_to_f64(bits):
    return (np.asarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _task(kind, idx):
    """kind: forward (rows), dx (token rows), dw (vocabulary entries): the oracle's values;
    dx_rowmax / dw_rowmax: the largest magnitude of each of those rows; dx_cmp / dw_cmp:
    (largest |GPU - oracle|, largest |oracle|) over those rows, against the GPU's bf16
    bits.  idx: the rows (a range for forward)."""
    idx = np.asarray(idx, np.int64)
    if kind == "forward":
        return _forward(int(idx[0]), int(idx[-1]) + 1)
    if kind in ("dx", "dx_rowmax", "dx_cmp"):
        want = _dx(idx)
        got = _G.get("gdX")
    else:
        want = _dw(idx)
        got = _G.get("gdW")
    if kind in ("dx", "dw"):
        return want
    if kind.endswith("rowmax"):
        return np.abs(want).max(1)
    return float(np.max(np.abs(_bits_to_f64(got[idx]) - want))), float(np.abs(want).max())


# ---------------------------------------------------------------------------------
# parent side
class Pool:
    """Worker processes over one case.  `extra` holds more arrays by name (lse, E of
    the oracle's forward; gdX, gdW: the GPU's gradients as bf16 bits)."""

    def __init__(self, case, workers=None, **extra):
        self.workers = workers or max(1, min(8, cores() // 4))
        base = "/dev/shm" if os.path.isdir("/dev/shm") else None
        self.dir = tempfile.mkdtemp(prefix="flce_oracle_", dir=base)
        atexit.register(shutil.rmtree, self.dir, True)
        arrays = dict(X=case.X, W=case.W, t=case.targets, glp=case.grad_logprob,
                      gent=case.grad_entropy, **extra)
        paths = {}
        for k, v in arrays.items():
            if v is None:
                paths[k] = None
                continue
            paths[k] = os.path.join(self.dir, k + ".npy")
            np.save(paths[k], np.ascontiguousarray(v))
        scalars = dict(scale=case.scale, ignore_index=case.ignore_index)
        threads = max(1, cores() // self.workers)
        self.ex = cf.ProcessPoolExecutor(self.workers, mp_context=mp.get_context("spawn"),
                                         initializer=_init, initargs=(paths, scalars, threads))

    def rows(self, kind, idx, parts=None):
        """The oracle's dx or dw values of the rows idx, split over the workers."""
        idx = np.asarray(idx, np.int64)
        n = parts or self.workers
        pieces = [idx[a:b] for a, b in ranges(len(idx), n)]
        return np.concatenate(self.map(kind, pieces))

    def map(self, kind, pieces, label=None):
        """Results of _task(kind, idx) for every piece, in order; a piece is an index
        array or an (a, b) range."""
        t0 = time.time()
        futs = [self.ex.submit(_task, kind, np.arange(*p) if isinstance(p, tuple) else p)
                for p in pieces]
        out = []
        for i, f in enumerate(futs):
            out.append(f.result())
            if label and ((i + 1) % self.workers == 0 or i + 1 == len(futs)):
                print(f"{label}: {i + 1}/{len(futs)} pieces, {time.time() - t0:.0f} s", flush=True)
        return out

    def close(self):
        self.ex.shutdown(wait=True)
        shutil.rmtree(self.dir, True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
