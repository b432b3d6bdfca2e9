"""The C ABI on the CPU: the library loads, exports what include/flce.h declares, and
rejects bad arguments before touching HIP (so no device is needed here)."""
import ctypes
import os
import re

import numpy as np
import pytest

from log_prob_amd import flce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    with open(os.path.join(ROOT, "include", "flce.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(flce_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = flce.load()
    declared = _header_functions()
    assert declared == sorted(flce.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings():
    lib = flce.load()
    assert re.fullmatch(rb"\d+\.\d+\.\d+", lib.flce_version())
    for code, name in flce.STATUS.items():
        assert lib.flce_status_string(code).decode() == name


def test_workspace_query_values():
    # forward: m, s, u partials of [ceil(V/256), Mpad] fp32 + zt [Mpad] + 256 bytes of
    # tile-queue counters
    fwd, bwd = flce.workspace_query(8192, 8192, 131072, True)
    assert fwd == 3 * 512 * 8192 * 4 + 8192 * 4 + 256
    fwd0, _ = flce.workspace_query(8192, 8192, 131072, False)
    assert fwd0 == 2 * 512 * 8192 * 4 + 8192 * 4 + 256
    # backward preferred: one d-logit chunk (2 GiB, within the 4 GiB budget) covers the
    # whole vocabulary here
    assert bwd == 8192 * 131072 * 2 + 256
    assert flce.backward_chunk_cols(8192, 8192, 131072, bwd) == 131072
    # smaller workspaces shrink the chunk, down to one 256-column tile plus fp32 dX
    mn = flce.backward_workspace_min(8192, 8192, 131072)
    assert mn == 8192 * 256 * 2 + 8192 * 8192 * 4 + 256
    assert flce.backward_chunk_cols(8192, 8192, 131072, mn) == 256
    # ragged shapes are padded to whole tiles
    fwd, _ = flce.workspace_query(64, 128, 1000, True)
    assert fwd == 3 * 4 * 256 * 4 + 256 * 4 + 256
    _, bwd = flce.workspace_query(32767, 2048, 151936, True)
    c = flce.backward_chunk_cols(32767, 2048, 151936, bwd)
    assert c % 256 == 0 and 256 <= c < 151936 + 256
    # d-logits past the 4 GiB chunk budget: 65536-column chunks (4 GiB of bf16 over
    # 32768 padded rows) plus the fp32 dX accumulator
    assert c == 65536
    assert bwd == 32768 * 65536 * 2 + 32767 * 2048 * 4 + 256


def test_forward_token_waves():
    # one 256-row wave: 3 partial arrays of [512 tiles, 256 rows] fp32 + the target logits
    mn = flce.forward_workspace_min(8192, 8192, 131072, True)
    assert mn == 3 * 512 * 256 * 4 + 256 * 4 + 256
    assert flce.forward_workspace_min(8192, 8192, 131072, False) == 2 * 512 * 256 * 4 + 256 * 4 + 256
    full, _ = flce.workspace_query(8192, 8192, 131072, True)
    assert flce.forward_wave_rows(8192, 8192, 131072, full) == 8192
    assert flce.forward_wave_rows(8192, 8192, 131072, mn) == 256
    w4k = 3 * 512 * 4096 * 4 + 4096 * 4 + 256
    assert flce.forward_wave_rows(8192, 8192, 131072, w4k) == 4096
    assert flce.forward_wave_rows(8192, 8192, 131072, w4k - 1) == 3840
    # the wave never exceeds the padded token count
    assert flce.forward_wave_rows(300, 64, 1000, 1 << 30) == 512
    with pytest.raises(flce.FlceError) as e:
        flce.forward_wave_rows(8192, 8192, 131072, mn - 1)
    assert e.value.status == 3


def _status(fn, *args):
    return fn(*args)


P = ctypes.c_void_p


def _fwd(lib, X=16, W=16, t=16, M=4, H=8, V=3, ign=-100, scale=1.0, ent=1, lp=16, lse=16,
         entropy=16, ws=256, wsb=1 << 20):
    return lib.flce_forward(X, W, t, M, H, V, ign, scale, ent, lp, lse, entropy, ws, wsb, None)


def test_forward_argument_errors():
    lib = flce.load()
    INV, UNS, WS = 1, 2, 3
    assert _fwd(lib, X=None) == INV
    assert _fwd(lib, t=None) == INV
    assert _fwd(lib, lse=None) == INV
    assert _fwd(lib, ws=None) == INV
    assert _fwd(lib, M=-1) == INV
    assert _fwd(lib, V=-1) == INV
    assert _fwd(lib, ent=2) == INV
    assert _fwd(lib, entropy=None) == INV
    assert _fwd(lib, scale=float("nan")) == INV
    assert _fwd(lib, scale=float("inf")) == INV
    assert _fwd(lib, H=12) == UNS
    assert _fwd(lib, X=24) == UNS
    assert _fwd(lib, ws=128) == UNS
    assert _fwd(lib, M=1 << 31) == UNS
    assert _fwd(lib, wsb=100) == WS
    assert b"workspace" in lib.flce_last_error_message()


def test_forward_entropy_null_allowed_when_off():
    lib = flce.load()
    # passes validation and only then fails on the (absent) device: anything but 1/2/3
    st = _fwd(lib, ent=0, entropy=None, wsb=10)
    assert st == 3   # still too small a workspace: validation order is arguments first


def _bwd(lib, X=16, W=16, t=16, M=4, H=8, V=3, ign=-100, scale=1.0, lse=16, ent=16, glp=16,
         gent=16, dX=16, dW=16, ws=256, wsb=1 << 20):
    return lib.flce_backward(X, W, t, M, H, V, ign, scale, lse, ent, glp, gent, dX, dW, ws, wsb,
                             None)


def test_backward_argument_errors():
    lib = flce.load()
    INV, UNS, WS = 1, 2, 3
    assert _bwd(lib, lse=None) == INV
    assert _bwd(lib, dX=None) == INV
    assert _bwd(lib, dW=None) == INV
    assert _bwd(lib, ent=None) == INV          # grad_entropy needs the entropy output
    assert _bwd(lib, H=0) == INV
    assert _bwd(lib, scale=float("-inf")) == INV
    assert _bwd(lib, H=4) == UNS
    assert _bwd(lib, dW=18) == UNS
    assert _bwd(lib, wsb=0) == WS
    mn = flce.backward_workspace_min(4, 8, 3)
    assert _bwd(lib, wsb=mn - 1) == WS


def test_python_wrapper_raises():
    with pytest.raises(flce.FlceError) as e:
        flce.workspace_query(-1, 8, 8)
    assert e.value.status == 1
    with pytest.raises(flce.FlceError):
        flce.backward_chunk_cols(100, 64, 1000, 10)


def test_shard_workspace_query():
    # d-logits (+ 256 bytes of tile-queue counters)
    lo, pref = flce.backward_shard_workspace_query(8192, 8192, 16384)
    assert lo == 8192 * 256 * 2 + 256
    assert pref == 8192 * 16384 * 2 + 256    # the whole shard in one chunk
    lo, pref = flce.backward_shard_workspace_query(300, 64, 1000)
    assert lo == 512 * 256 * 2 + 256 and pref == 512 * 1024 * 2 + 256


def _fps(lib, X=16, W=16, t=16, M=4, H=8, Vs=3, off=0, ign=-100, scale=1.0, ent=1, ws=256,
         wsb=1 << 20):
    return lib.flce_forward_partials_shard(X, W, t, M, H, Vs, off, ign, scale, ent, ws, wsb, None)


def _merge(lib, offs, t=16, M=4, ign=-100, ent=1, lp=16, lse=16, entropy=16, g=256,
           stride=1 << 16):
    arr = None if offs is None else (ctypes.c_int64 * len(offs))(*offs)
    n = 0 if offs is None else len(offs) - 1
    return lib.flce_forward_merge_shards(t, M, n, arr, ign, ent, lp, lse, entropy, g, stride,
                                         None)


def _bws(lib, X=16, W=16, t=16, M=4, H=8, Vs=3, off=0, Vt=3, ign=-100, scale=1.0, lse=16,
         ent=16, glp=16, gent=16, dXp=16, acc=0, dW=16, ws=256, wsb=1 << 20):
    return lib.flce_backward_shard(X, W, t, M, H, Vs, off, Vt, ign, scale, lse, ent, glp, gent,
                                   dXp, acc, dW, ws, wsb, None)


def test_shard_argument_errors():
    lib = flce.load()
    INV, UNS, WS = 1, 2, 3
    # forward partials of a shard
    assert _fps(lib, off=-1) == INV
    assert _fps(lib, off=(1 << 30) - 2) == INV   # shard would end past 2^30 ids
    assert _fps(lib, W=None) == INV
    assert _fps(lib, W=24) == UNS
    assert _fps(lib, wsb=16) == WS
    # merge of gathered partials
    assert _merge(lib, None) == INV
    assert _merge(lib, [0]) == UNS                       # no shard
    assert _merge(lib, list(range(0, 66 * 256, 256))) == UNS   # 65 shards
    assert _merge(lib, [1, 5, 9]) == INV                 # must start at 0
    assert _merge(lib, [0, 5, 5]) == INV                 # empty shard
    assert _merge(lib, [0, 5, 3]) == INV                 # reversed
    assert _merge(lib, [0, 5, 9], g=128) == UNS
    assert _merge(lib, [0, 5, 9], stride=1000) == UNS
    assert _merge(lib, [0, 5, 9], stride=256) == WS      # below one shard's partials
    assert _merge(lib, [0, 5, 9], ent=1, entropy=None) == INV
    # backward of a shard
    assert _bws(lib, off=-1) == INV
    assert _bws(lib, off=1, Vs=3, Vt=3) == INV           # shard past V_total
    assert _bws(lib, Vt=1 << 31) == UNS
    assert _bws(lib, acc=2) == INV
    assert _bws(lib, dXp=None) == INV
    assert _bws(lib, ent=None) == INV                    # grad_entropy needs entropy
    assert _bws(lib, dXp=20) == UNS
    mn, _ = flce.backward_shard_workspace_query(4, 8, 3)
    assert _bws(lib, wsb=mn - 1) == WS


def test_nll_argument_errors():
    lib = flce.load()
    INV, UNS = 1, 2
    assert lib.flce_nll_reduce(None, 16, 4, 3, -100, 16, None) == INV
    assert lib.flce_nll_reduce(16, 16, -1, 3, -100, 16, None) == INV
    assert lib.flce_nll_reduce(16, 16, 4, 0, -100, 16, None) == INV
    assert lib.flce_nll_reduce(16, 16, 1 << 31, 3, -100, 16, None) == UNS
    assert lib.flce_nll_reduce(18, 16, 4, 3, -100, 16, None) == UNS
    assert lib.flce_nll_reduce(16, 16, 4, 3, -100, 20, None) == UNS
    assert lib.flce_nll_mean_grad(16, 4, 3, -100, None, 16, None) == INV
    assert lib.flce_nll_mean_grad(16, -1, 3, -100, 16, 16, None) == INV
    assert lib.flce_nll_mean_grad(12, 4, 3, -100, 16, 16, None) == UNS


def test_policy_loss_argument_errors():
    """Every invalid call of the policy-loss entry points fails on the host, before any
    HIP call (fake, aligned device addresses; nothing is dereferenced)."""
    lib = flce.load()
    INV, UNS = 1, 2

    def red(lp=16, old=None, adv=16, t=16, M=4, V=3, el=0.2, eh=0.2, den=0.0, ptl=16, out=16):
        return lib.flce_policy_loss_reduce(lp, old, adv, t, M, V, -100, el, eh, den, ptl, None,
                                           out, None)

    def grad(lp=16, old=None, adv=16, t=16, M=4, V=3, el=0.2, eh=0.2, den=0.0, reduced=16,
             g=16):
        return lib.flce_policy_loss_grad(lp, old, adv, t, M, V, -100, el, eh, den, reduced, g,
                                         None)

    assert red(lp=None) == INV and red(adv=None) == INV and red(t=None) == INV
    assert red(ptl=None) == INV and red(out=None) == INV
    assert red(M=-1) == INV and red(V=0) == INV
    assert red(M=1 << 31) == UNS
    assert red(el=-0.1) == INV and red(eh=float("inf")) == INV and red(el=float("nan")) == INV
    assert red(den=float("nan")) == INV
    assert red(lp=18) == UNS and red(old=18) == UNS and red(t=20) == UNS and red(out=20) == UNS
    assert grad(g=None) == INV
    assert grad(reduced=None) == INV                    # the count is read from `reduced`
    assert grad(V=0) == INV and grad(el=-1.0) == INV
    assert grad(reduced=20) == UNS and grad(g=18) == UNS
    # an empty batch of tokens launches nothing
    assert grad(M=0, lp=None, adv=None, t=None, g=None, reduced=None) == 0


def test_empty_batch_needs_no_device():
    """M = 0 is a valid, empty call: sizes are 0 and the forward and the merges return
    FLCE_OK before any HIP call, with every pointer NULL."""
    lib = flce.load()
    assert flce.workspace_query(0, 64, 1000, True) == (0, 0)
    assert flce.forward_workspace_min(0, 64, 1000) == 0
    assert flce.forward_wave_rows(0, 64, 1000, 0) == 0
    assert flce.backward_workspace_min(0, 64, 1000) == 0
    assert flce.backward_chunk_cols(0, 64, 1000, 0) == 1024
    assert _fwd(lib, X=None, W=None, t=None, M=0, lp=None, lse=None, entropy=None, ws=None,
                wsb=0) == 0
    assert lib.flce_forward_partials(None, None, None, 0, 64, 1000, -100, 1.0, 1, None, 0,
                                     None) == 0
    assert lib.flce_forward_merge(None, 0, 64, 1000, -100, 1, None, None, None, None, 0,
                                  None) == 0
    assert _merge(lib, [0, 5, 9], t=None, M=0, lp=None, lse=None, entropy=None, g=None) == 0
    assert lib.flce_nll_mean_grad(None, 0, 1000, -100, None, None, None) == 0
    # still checked: H, V and the flags
    assert _fwd(lib, M=0, V=0) == 1
    assert _fwd(lib, M=0, H=12) == 2
    assert _fwd(lib, M=0, ent=3) == 1
    # the empty backward must write dW = 0, so it needs dW (checked before any launch)
    assert _bwd(lib, M=0, dW=None) == 1
    assert _bwd(lib, M=0, dW=18) == 2


def _fwd_noalloc(lib, X=16, W=16, t=16, M=4, H=8, V=3, ign=-100, scale=1.0, ent=1, lp=16,
                 lse=16, entropy=16):
    return lib.flce_forward_noalloc(X, W, t, M, H, V, ign, scale, ent, lp, lse, entropy, None)


def test_forward_noalloc_rejections_need_no_device():
    """The allocation-free forward checks its arguments like flce_forward, and rejects a
    vocabulary whose one 256-row wave of partials does not fit its static scratch, all
    before any HIP call.  (Only rejected calls are made here: a call that passes would
    launch kernels on these placeholder pointers.)"""
    lib = flce.load()
    INV, UNS = 1, 2
    assert flce.FLCE_NOALLOC_SCRATCH_BYTES == 32 << 20
    assert _fwd_noalloc(lib, X=None) == INV
    assert _fwd_noalloc(lib, t=None) == INV
    assert _fwd_noalloc(lib, lse=None) == INV
    assert _fwd_noalloc(lib, ent=2) == INV
    assert _fwd_noalloc(lib, entropy=None) == INV
    assert _fwd_noalloc(lib, scale=float("nan")) == INV
    assert _fwd_noalloc(lib, H=12) == UNS
    assert _fwd_noalloc(lib, X=24) == UNS
    assert _fwd_noalloc(lib, M=1 << 31) == UNS
    # the partials of a 256-row wave: 3 (entropy) or 2 arrays of 256 fp32 per vocabulary
    # tile, each array rounded up to 256 bytes, plus 1 KiB of target logits
    for ent, arrays in ((1, 3), (0, 2)):
        n_vt = (flce.FLCE_NOALLOC_SCRATCH_BYTES - 1024) // (arrays * 1024)
        assert flce.forward_wave_rows(256, 8, 256 * n_vt, flce.FLCE_NOALLOC_SCRATCH_BYTES,
                                      bool(ent)) == 256
        assert _fwd_noalloc(lib, V=256 * n_vt + 1, ent=ent) == UNS
        assert b"scratch" in lib.flce_last_error_message()
    # an empty batch is a valid call that touches nothing
    assert _fwd_noalloc(lib, X=None, W=None, t=None, M=0, lp=None, lse=None, entropy=None) == 0


def test_size_limits_match_the_header():
    """Each edge of the documented size limits: 0 <= M <= 2^30, 8 <= H <= 2^20 with
    H % 8 == 0, 1 <= V <= 2^30."""
    lib = flce.load()
    fb, bb = ctypes.c_size_t(), ctypes.c_size_t()

    def q(M, H, V):
        return lib.flce_workspace_query(M, H, V, 1, ctypes.byref(fb), ctypes.byref(bb))
    assert q(0, 8, 1) == 0
    assert q(1 << 30, 8, 1) == 0 and q((1 << 30) + 1, 8, 1) == 2
    assert q(1, 1 << 20, 1) == 0 and q(1, (1 << 20) + 8, 1) == 2
    assert q(1, 8, 1 << 30) == 0 and q(1, 8, (1 << 30) + 1) == 2
    assert q(-1, 8, 1) == 1 and q(1, 0, 1) == 1 and q(1, 8, 0) == 1
    assert q(1, 4, 1) == 2 and q(1, 12, 1) == 2


MAX_WG = 0xFFFFFFFF // 256      # workgroups of 256 threads in one dispatch


@pytest.mark.parametrize("M,H,V", [(1 << 30, 8, 1 << 18), (1 << 20, 1 << 20, 1 << 20),
                                   ((1 << 26) + 5, 64, 3000), (1 << 30, 1 << 20, 1)])
def test_every_launch_within_the_dispatch_limit(M, H, V):
    """Shapes whose single-launch grids would pass 2^32 work-items: the forward and the
    backward plan smaller token waves (and chunks) so that every grid fits; the
    one-launch partials call refuses them."""
    big = 1 << 62
    rows = flce.forward_wave_rows(M, H, V, big)
    n_vt = -(-V // 256)
    assert rows % 256 == 0 and 256 <= rows and (rows // 256) * n_vt <= MAX_WG
    assert rows * 64 <= 0xFFFFFFFF                      # the target-logit kernel's grid
    fb, _ = flce.workspace_query(M, H, V, True)
    assert flce.forward_wave_rows(M, H, V, fb) == rows  # the preferred size is one such wave
    r, c, pipe = flce.backward_schedule(M, H, V, big)
    n_mt, n_ct, n_ht = -(-r // 256), -(-c // 256), -(-H // 256)
    grids = (n_mt * n_ct, n_ct * n_ht, n_mt * n_ht)
    assert (sum(grids) + 24 if pipe else max(grids)) <= MAX_WG, (r, c, pipe, grids)
    lo = flce.backward_workspace_min(M, H, V)
    r, c, pipe = flce.backward_schedule(M, H, V, lo)
    n_mt, n_ct = -(-r // 256), -(-c // 256)
    assert max(n_mt * n_ct, n_ct * n_ht, n_mt * n_ht) <= MAX_WG
    lib = flce.load()
    if -(-M // 256) * n_vt > MAX_WG:
        assert lib.flce_forward_partials(16, 16, 16, M, H, V, -100, 1.0, 1, 256, big, None) == 2
        assert b"waves" in lib.flce_last_error_message()


@pytest.mark.parametrize("M,H,V", [(4096, 4096, 512), (4097, 64, 1000), (600, 136, 3000),
                                   (8192, 8192, 131072), (32767, 2048, 151936), (1, 8, 1),
                                   ((1 << 20) + 1, 64, 512)])
def test_backward_schedule_sizes(M, H, V):
    """The smallest backward workspace is never above the preferred one, is accepted
    (and one byte less is not), and the preferred size runs every row in one wave."""
    Mpad = -(-M // 256) * 256
    lo = flce.backward_workspace_min(M, H, V)
    _, pref = flce.workspace_query(M, H, V, True)
    assert lo <= pref
    assert flce.backward_wave_rows(M, H, V, pref) == Mpad
    rows = flce.backward_wave_rows(M, H, V, lo)
    assert rows % 256 == 0 and 256 <= rows <= Mpad
    assert flce.backward_chunk_cols(M, H, V, lo) % 256 == 0
    with pytest.raises(flce.FlceError):
        flce.backward_wave_rows(M, H, V, lo - 1)
    with pytest.raises(flce.FlceError):
        flce.backward_chunk_cols(M, H, V, lo - 1)


def test_backward_schedule_choices():
    """The smallest workspace runs three launches per step (the two d-logit buffers of a
    pipelined schedule need more); the preferred one pipelines small steps (M = H = 4096,
    V = 32768: one step of 3.3e12 FLOP) and not large ones (M = H = 8192, V = 131072)."""
    for M, H, V in ((4096, 4096, 32768), (8192, 8192, 131072), (600, 136, 3000)):
        lo = flce.backward_workspace_min(M, H, V)
        assert flce.backward_schedule(M, H, V, lo)[2] is False
    assert flce.backward_schedule(4096, 4096, 32768,
                                  flce.workspace_query(4096, 4096, 32768)[1]) == (4096, 32768, True)
    assert flce.backward_schedule(8192, 8192, 131072,
                                  flce.workspace_query(8192, 8192, 131072)[1]) == (8192, 131072, False)
    rows, chunk, _ = flce.backward_schedule(600, 136, 3000, 1 << 30)
    assert (rows, chunk) == (flce.backward_wave_rows(600, 136, 3000, 1 << 30),
                             flce.backward_chunk_cols(600, 136, 3000, 1 << 30))


def _schedule_bytes(M, H, V, rows, chunk, pipe):
    """Workspace a schedule uses, from its description in include/flce.h: the bf16
    d-logits of one wave over one chunk (two buffers when pipelined over more than one
    step), the fp32 dX accumulator of one wave when a wave takes several chunks, the fp32
    dW accumulator when there are several waves, 256 bytes of tile-queue counters; each
    part rounded up to 256 bytes."""
    up = lambda x: -(-x // 256) * 256
    Mpad, Vpad = up(M), up(V)
    steps = -(-M // rows) * -(-Vpad // chunk)
    b = (2 if pipe and steps > 1 else 1) * up(rows * chunk * 2)
    if chunk < Vpad:
        b += up(min(rows, M) * H * 4)
    if rows < Mpad:
        b += up(V * H * 4)
    return b + 256


def test_backward_schedules_fit_their_workspace():
    """Seeded random shapes and workspace sizes: the reported schedule fits the bytes
    given, keeps every launch within the dispatch limit, and pipelines only small steps;
    below the minimum the call is refused."""
    rng = np.random.default_rng(20261202)
    for _ in range(400):
        M = int(rng.choice([int(rng.integers(1, 2000)), int(rng.integers(1, 1 << 22))]))
        H = 8 * int(rng.integers(1, 1 << int(rng.integers(3, 14))))
        V = int(rng.choice([int(rng.integers(1, 5000)), int(rng.integers(1, 1 << 21))]))
        lo = flce.backward_workspace_min(M, H, V)
        _, pref = flce.workspace_query(M, H, V, True)
        for b in (lo, int(rng.integers(lo, 2 * pref + 2)), pref):
            rows, chunk, pipe = flce.backward_schedule(M, H, V, b)
            Mpad = -(-M // 256) * 256
            assert rows % 256 == 0 and chunk % 256 == 0 and 256 <= rows <= Mpad
            assert _schedule_bytes(M, H, V, rows, chunk, pipe) <= b, (M, H, V, b, rows, chunk, pipe)
            n_mt, n_ct, n_ht = rows // 256, chunk // 256, -(-H // 256)
            grids = (n_mt * n_ct, n_ct * n_ht, n_mt * n_ht)
            assert (sum(grids) + 24 if pipe else max(grids)) <= MAX_WG
            if pipe:
                assert 6.0 * rows * H * chunk <= 8e12
        with pytest.raises(flce.FlceError):
            flce.backward_schedule(M, H, V, lo - 1)
