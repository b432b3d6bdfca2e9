"""Benchmark of the fused LM-head linear + cross-entropy path on one gfx950 GPU.

A step is one forward (logprob, lse, entropy) plus one backward (dX, dW) of the
M=8192, H=8192, V=131072 bf16 workload with entropy on and grad_logprob = 1/M,
through the libflce C ABI.  Inputs are seeded synthetic bf16 (no dataset), resident
in HBM before timing starts.  FLOPs follow the four-classifier-GEMM convention:
2MHV for the forward, 8MHV for forward + backward (forward logits, recomputed
logits, dX, dW).

Prints one JSON line.  Also measures, with HIP events on the launch stream, the
dominant kernel (the fused GEMM + online-softmax forward kernel, launched alone
through flce_forward_partials) against the dense bf16 MFMA peak, and times the fp64
CPU oracle on a bounded sample of the same workload.
"""
import os

# the oracle's BLAS must use every core this job may run on; set before numpy loads
_CORES = len(os.sched_getaffinity(0))
for _v in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(_CORES))

import argparse  # noqa: E402
import json  # noqa: E402
import sys  # noqa: E402
import time  # noqa: E402

import numpy as np  # noqa: E402

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
METRIC = "fwd & fwd+bwd TFLOP/s (% bf16 MFMA peak), M=8192 H=8192 V=131072"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=4, help="workload config (default 4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-shard-bench", action="store_true",
                    help="skip the per-rank vocabulary-shard timings (profiling runs)")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of the oracle sample (0: sized for ~15 s)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--kernel-only", choices=["fwd"], default=None,
                    help="only launch the fused forward kernel three times (for counter passes)")
    ap.add_argument("--blas-reference", action="store_true",
                    help="only time the library bf16 GEMM (torch.matmul) of the same logits shape")
    return ap.parse_args()


def blas_reference(case, steps):
    """Context, not a product path: the vendor bf16 GEMM (torch.matmul, hipBLASLt) on the
    shapes and memory orders of the four GEMMs of a step: z = X W^T (forward and the
    d-logit recompute; the library materialises the logits the fused kernels never
    write), dX = dz W and dW = dz^T X, dz a [M, V] bf16 matrix."""
    import torch
    M, H, V = case.M, case.H, case.V
    g = torch.Generator(device="cuda").manual_seed(0)
    X = torch.randn(M, H, device="cuda", dtype=torch.bfloat16, generator=g)
    W = torch.randn(V, H, device="cuda", dtype=torch.bfloat16, generator=g)
    dz = torch.randn(M, V, device="cuda", dtype=torch.bfloat16, generator=g)
    z = torch.empty(M, V, device="cuda", dtype=torch.bfloat16)
    dX = torch.empty(M, H, device="cuda", dtype=torch.bfloat16)
    dW = torch.empty(V, H, device="cuda", dtype=torch.bfloat16)
    cases = (("z = X @ W^T", lambda: torch.matmul(X, W.t(), out=z)),
             ("dX = dz @ W", lambda: torch.matmul(dz, W, out=dX)),
             ("dW = dz^T @ X", lambda: torch.matmul(dz.t(), X, out=dW)))
    for name, fn in cases:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = 2.0 * M * H * V / (ms * 1e-3) / 1e12
        print(json.dumps({"blas_reference": f"torch.matmul bf16 {name}", "M": M, "H": H,
                          "V": V, "ms": round(ms, 4), "tflops": round(tf, 2),
                          "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}), flush=True)


PROFILE = os.path.join(ROOT, "profiles", "fwd_bwd_M8192_H8192_V131072.md")
KERNEL_SOURCES = ("log_prob_amd/csrc/flce_kernels.hip", "log_prob_amd/csrc/flce_internal.h")


def kernel_source_hash():
    """SHA-256 of the kernel sources with comments and blank space removed, so that a
    change to a comment does not disown the committed counter figures."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                 # line comments
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def profile_figures():
    """From the committed rocprofv3 summary: HBM bytes per fwd_tile launch (counters)
    and the traced average duration of the launches the roofline loop times; both None
    if the kernel sources changed since that profile was taken."""
    try:
        kv = {}
        with open(PROFILE) as f:
            for line in f:
                if ":" in line and not line.startswith(("|", "#")):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None, None
        return (float(kv["fwd_tile_traffic_bytes_per_launch"]),
                float(kv.get("fwd_tile_roofline_loop_avg_ms", "nan")))
    except (OSError, KeyError, ValueError):
        return None, None


def copy_probe(mib):
    """A plain copy kernel of known size: reads and writes mib MiB, three times."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


def cpu_baseline(case, rows_req):
    """Time the fp64 oracle (forward, then backward) on the first R tokens of the workload.

    The oracle's forward forms the logits of the R rows (2RHV fp64 FLOP); its backward
    forms them again, then dX and dW (6RHV): 8RHV performed in all, the same count as
    the GPU step's four classifier GEMMs."""
    from oracle import flce_ref as ref
    M, H, V = case.M, case.H, case.V
    Wd = ref.decode_bf16(case.W)
    # grow the sample until one timed pass takes 10-30 s of CPU work (the first
    # call also warms up the BLAS threads)
    _run_oracle_rows(ref, case, Wd, 8)
    R = rows_req if rows_req > 0 else 64
    while True:
        tf, tb = _run_oracle_rows(ref, case, Wd, R)
        dt = tf + tb
        if rows_req > 0 or dt >= 10.0 or R >= M:
            break
        R = int(min(M, max(R + 1, R * min(8.0, 15.0 / max(dt, 1e-3)))))
    rhv = float(R) * H * V
    return {"value": 8.0 * rhv / dt / 1e12, "unit": "TFLOP/s", "cores": _CORES,
            "kind": "oracle",
            "sample": f"fp64 NumPy oracle on the first {R} of {M} tokens (H={H}, V={V}, full "
                      f"vocabulary): forward {tf:.1f} s (2RHV fp64 FLOP: the logits) + backward "
                      f"{tb:.1f} s (6RHV: the logits again, dX, dW); value = the 8RHV fp64 FLOP "
                      f"performed / {dt:.1f} s",
            "forward_tflops": 2.0 * rhv / tf / 1e12,
            "backward_tflops": 6.0 * rhv / tb / 1e12,
            "step_equivalent_s": dt * M / R}


def _run_oracle_rows(ref, case, Wd, R):
    """Seconds of the oracle's forward and of its backward over the first R rows."""
    rows = np.arange(R)
    t0 = time.perf_counter()
    ref.forward_rows(case.X, case.W, case.targets, rows, case.ignore_index, case.scale,
                     case.compute_entropy, Wd=Wd)
    t1 = time.perf_counter()
    Xd = ref.decode_bf16(case.X[:R])
    glp = None if case.grad_logprob is None else case.grad_logprob[:R]
    gent = None if case.grad_entropy is None else case.grad_entropy[:R]
    ref.backward_f64(Xd, Wd, case.targets[:R], case.ignore_index, case.scale, glp, gent)
    return t1 - t0, time.perf_counter() - t1


def main():
    args = parse()
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch
    from log_prob_amd import flce
    from synth import inputs
    from tests.gpu_util import to_dev

    cfg = args.config
    if args.blas_reference:
        import types
        blas_reference(types.SimpleNamespace(**{k: inputs.CONFIGS[cfg][k] for k in "MHV"}),
                       max(args.steps, 5))
        return
    case = inputs.config_case(cfg)
    M, H, V = case.M, case.H, case.V
    dev = torch.device("cuda:0")
    X, W, t, glp, gent = to_dev(case, dev)
    ent = case.compute_entropy or gent is not None
    fwd_b, bwd_b = flce.workspace_query(M, H, V, ent)
    ws = torch.empty(max(fwd_b, bwd_b), dtype=torch.uint8, device=dev)
    logprob = torch.empty(M, dtype=torch.float32, device=dev)
    lse = torch.empty_like(logprob)
    entropy = torch.empty_like(logprob) if ent else None
    dX = torch.empty_like(X)
    dW = torch.empty_like(W)
    stream = torch.cuda.current_stream(dev)

    def fwd():
        flce.forward(X, W, t, case.ignore_index, case.scale, ent, workspace=ws,
                     out=(logprob, lse, entropy))

    def step():
        fwd()
        flce.backward(X, W, t, lse, entropy if gent is not None else None, glp, gent,
                      case.ignore_index, case.scale, workspace=ws, out=(dX, dW))

    def timed(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs]

    if args.kernel_only == "fwd":
        for _ in range(3):
            flce.forward_partials(X, W, t, case.ignore_index, case.scale, ent, workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"kernel_only": "fwd_tile", "launches": 3}), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # whole-job timing: exactly K steps bracketed by synchronisation (wall clock); HIP
    # events around each step give the per-step spread
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in evs]
    ms = wall * 1e3 / args.steps
    ms_med = float(np.median(step_ms))

    # forward alone and the dominant kernel alone (HIP events on the launch stream)
    for _ in range(2):
        fwd()
    fwd_ms = float(np.median(timed(fwd, max(args.steps, 5))))
    # the same step with an entropy gradient as well: grad_entropy = N(0,1)/M
    ent_grad = None
    if ent and gent is None:
        gen = torch.Generator(device=dev).manual_seed(2026)
        gent_v = torch.randn(M, device=dev, dtype=torch.float32, generator=gen) / M

        def step_entgrad():
            fwd()
            flce.backward(X, W, t, lse, entropy, glp, gent_v, case.ignore_index, case.scale,
                          workspace=ws, out=(dX, dW))
        step_entgrad()
        eg_ms = float(np.median(timed(step_entgrad, max(args.steps, 5))))
        ent_grad = {"ms": round(eg_ms, 4),
                    "tflops": round(8.0 * M * H * V / (eg_ms * 1e-3) / 1e12, 2),
                    "grad_entropy": "N(0,1)/M"}
    # token waves: the same forward with a workspace that holds 4096-row waves of partials
    wave_rows = min(4096, -(-M // 256) * 256)
    ws_wave = torch.empty(flce.forward_workspace_min(M, H, V, ent) * (wave_rows // 256),
                          dtype=torch.uint8, device=dev)
    assert flce.forward_wave_rows(M, H, V, ws_wave.numel(), ent) == wave_rows
    fwd_wave = lambda: flce.forward(X, W, t, case.ignore_index, case.scale, ent,
                                    workspace=ws_wave, out=(logprob, lse, entropy))
    fwd_wave()
    fwd_wave_ms = float(np.median(timed(fwd_wave, max(args.steps, 5))))
    part = lambda: flce.forward_partials(X, W, t, case.ignore_index, case.scale, ent, workspace=ws)
    part()
    k_ms = timed(part, max(args.steps, 5))
    k_avg = float(np.mean(k_ms))

    # one rank's share of a vocabulary-parallel split of the same workload: the rank's
    # forward partials, the merge over all ranks' gathered partials, and the rank's
    # backward (compute only: the all-gather and the dX all-reduce are the caller's)
    shard_out = {}
    dXp = torch.empty((M, H), dtype=torch.float32, device=dev)
    for P in (() if args.no_shard_bench else (2, 4, 8)):
        if V % P or (V // P) % 256:
            continue
        Vs = V // P
        offs = [r * Vs for r in range(P + 1)]
        stride = -(-flce.workspace_query(M, H, Vs, ent)[0] // 256) * 256
        gathered = torch.empty(P * stride, dtype=torch.uint8, device=dev)
        for r in range(P):
            flce.forward_partials_shard(X, W[offs[r]:offs[r + 1]], t, offs[r], case.ignore_index,
                                        case.scale, ent, workspace=gathered[r * stride:(r + 1) * stride])

        def rank_fwd():
            flce.forward_partials_shard(X, W[0:Vs], t, 0, case.ignore_index, case.scale, ent,
                                        workspace=gathered[0:stride])
            flce.forward_merge_shards(t, offs, gathered, stride, case.ignore_index, ent,
                                      out=(logprob, lse, entropy))

        def rank_bwd():
            flce.backward_shard(X, W[0:Vs], t, 0, V, lse, entropy if gent is not None else None,
                                glp, gent, dX_partial=dXp, ignore_index=case.ignore_index,
                                scale=case.scale, workspace=ws, dW_shard=dW[0:Vs])
        rank_fwd()
        rank_bwd()
        sf = float(np.median(timed(rank_fwd, max(args.steps, 5))))
        sb = float(np.median(timed(rank_bwd, max(args.steps, 5))))
        shard_out[f"tp{P}"] = {"V_shard": Vs, "fwd_ms": round(sf, 4),
                               "fwd_tflops": round(2.0 * M * H * Vs / (sf * 1e-3) / 1e12, 2),
                               "fwd_bwd_ms": round(sf + sb, 4),
                               "fwd_bwd_tflops": round(8.0 * M * H * Vs / ((sf + sb) * 1e-3) / 1e12, 2)}
        del gathered

    # the committed profile covers the bench workload only
    traffic, prof_ms = profile_figures() if cfg == 4 else (None, None)
    flop_f = 2.0 * M * H * V
    flop_fb = 8.0 * M * H * V
    tf_fb = flop_fb / (ms * 1e-3) / 1e12
    tf_f = flop_f / (fwd_ms * 1e-3) / 1e12
    k_tf = flop_f / (k_avg * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": round(tf_fb, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"fused linear+CE forward+backward, M={M} H={H} V={V} bf16, "
                               f"entropy {'on' if ent else 'off'}, scale={case.scale:g}",
                   "M": M, "H": H, "V": V, "flops_per_step": flop_fb},
        "pct_peak": round(100.0 * tf_fb / PEAK_BF16_TFLOPS, 2),
        "ms_per_step_event_median": round(ms_med, 4),
        "fwd_ms": round(fwd_ms, 4),
        "fwd_tflops": round(tf_f, 2),
        "fwd_pct_peak": round(100.0 * tf_f / PEAK_BF16_TFLOPS, 2),
        "wall_s_timed": round(wall, 3),
        "fwd_bwd_with_grad_entropy": ent_grad,
        "fwd_workspace_bytes": fwd_b,
        "bwd_workspace_bytes": bwd_b,
        "bwd_chunk_cols": flce.backward_chunk_cols(M, H, V, bwd_b),
        "fwd_token_waves": {"wave_rows": wave_rows, "ms": round(fwd_wave_ms, 4),
                            "tflops": round(flop_f / (fwd_wave_ms * 1e-3) / 1e12, 2),
                            "workspace_bytes": int(ws_wave.numel()), "full_workspace_bytes": fwd_b},
        "vocab_shard_rank": shard_out,
        "roofline": {"bound": "mfma", "kernel": "fwd_tile_kernel (fused GEMM + online softmax)",
                     "achieved": round(k_tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(k_tf / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes/launch (rocprofv3 FETCH_SIZE+WRITE_SIZE, scaled)",
                     "algorithmic_bytes": 2 * M * H + 2 * V * H + 8 * M + 12 * M,
                     "avg_launch_ms": round(k_avg, 4), "flops_per_launch": flop_f,
                     "profile_avg_launch_ms": prof_ms,
                     "note": "achieved = flops_per_launch / avg_launch_ms, HIP events around "
                             "each of the last steps launches (the forward kernel plus the "
                             "0.04 ms target-logit kernel); profile_avg_launch_ms = the same "
                             "launches in the committed rocprofv3 trace of this command"},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
