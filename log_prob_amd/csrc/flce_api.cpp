// libflce C ABI: argument validation, workspace carve-up and the launch sequence.
// Every check runs on the host before the first HIP call, so a rejected call
// enqueues nothing and needs no device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "flce.h"
#include "flce_internal.h"

namespace {

thread_local char g_last_error[512] = "";

flce_status_t fail(flce_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

flce_status_t ok() {
  g_last_error[0] = '\0';
  return FLCE_OK;
}

constexpr int64_t kTile = flce::kTile;
constexpr int64_t kMaxM = int64_t(1) << 30;
constexpr int64_t kMaxV = int64_t(1) << 30;
constexpr int64_t kMaxH = int64_t(1) << 20;
// A dispatch covers at most 2^32 - 1 work-items per dimension: the tile kernels run
// 256 threads per workgroup, the target-logit kernel 64 per row, the merge 16 per row.
constexpr int64_t kMaxWorkgroups = flce::kMaxWorkgroups;
constexpr int64_t kMaxWaveRows = (0xFFFFFFFFLL / 64) / 256 * 256;
constexpr size_t kAlign = 256;
// Preferred size of one d-logit chunk buffer: 4 GiB.  Wider chunks mean fewer passes
// over the fp32 dX accumulator and fewer launches; past about 2000 K steps the dX GEMM's
// tiles drift apart in L2 (M=32767, H=2048, V=151936: 3 chunks of 65536 columns -0.8 to
// -1.8% against 5 of 32768, one chunk of 152064 +2%).
constexpr size_t kDzBudget = size_t(4) << 30;
// Widest d-logit chunk: keeps every byte offset the kernels form inside one
// 256-row tile of the chunk buffer below 2^30.
constexpr int64_t kMaxChunk = int64_t(1) << 21;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// M = 0 (an empty batch of tokens) is valid: the forward writes nothing and the
// backward writes dW = 0.
flce_status_t check_shape(int64_t M, int64_t H, int64_t V) {
  if (M < 0 || H <= 0 || V <= 0)
    return fail(FLCE_ERR_INVALID_VALUE,
                "M must be >= 0, H and V positive (got M=%lld H=%lld V=%lld)", (long long)M,
                (long long)H, (long long)V);
  if (M > kMaxM || V > kMaxV || H > kMaxH)
    return fail(FLCE_ERR_UNSUPPORTED, "shape too large (limits M, V <= 2^30, H <= 2^20)");
  if (H % 8 != 0)
    return fail(FLCE_ERR_UNSUPPORTED, "H must be a multiple of 8 (got %lld)", (long long)H);
  return FLCE_OK;
}

struct FwdLayout {
  int64_t n_mt, n_vt, Mpad;
  size_t off_m, off_s, off_u, off_zt, off_q, total;
};

// Forward workspace for a wave of `rows` token rows (rows <= Mpad of the call).
FwdLayout fwd_layout(int64_t rows, int64_t V, bool ent) {
  FwdLayout L;
  L.n_mt = cdiv(rows, flce::kFwdTileM);
  L.n_vt = cdiv(V, flce::kFwdTileN);
  L.Mpad = cdiv(rows, kTile) * kTile;
  const size_t part = align_up(size_t(L.n_vt) * size_t(L.Mpad) * sizeof(float));
  L.off_m = 0;
  L.off_s = part;
  L.off_u = 2 * part;
  L.off_zt = (ent ? 3 : 2) * part;
  L.off_q = L.off_zt + align_up(size_t(L.Mpad) * sizeof(float));
  L.total = L.Mpad > 0 ? L.off_q + flce::kQueueBytes : 0;  // no rows: no launch
  return L;
}

// Tallest forward wave one set of launches can take: the tile grid and the per-row
// kernels within the dispatch limits (at least 256 rows for every V <= 2^30).
int64_t max_wave_rows(int64_t V) {
  const int64_t by_grid = kMaxWorkgroups / cdiv(V, flce::kFwdTileN) * flce::kFwdTileM;
  const int64_t r = by_grid < kMaxWaveRows ? by_grid : kMaxWaveRows;
  return r / kTile * kTile;
}

// Tallest wave (a multiple of 256 rows, at most Mpad and max_wave_rows) whose forward
// partials fit in `bytes`; 0 if not even one 256-row wave fits.
int64_t wave_rows_for_workspace(int64_t M, int64_t V, bool ent, size_t bytes) {
  int64_t Mpad = cdiv(M, kTile) * kTile;
  if (Mpad > max_wave_rows(V)) Mpad = max_wave_rows(V);
  if (fwd_layout(Mpad, V, ent).total <= bytes) return Mpad;
  int64_t lo = 0, hi = Mpad / kTile;  // in tiles: lo fits (or 0), hi does not
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) / 2;
    if (fwd_layout(mid * kTile, V, ent).total <= bytes) lo = mid; else hi = mid;
  }
  return lo * kTile;
}

// The backward's schedule: token waves of `rows` rows (a multiple of 256; rows >= Mpad
// is one wave of every row) and vocabulary chunks of `chunk` columns.  The workspace
// holds the bf16 d-logits of one wave's chunk, then, when a wave takes more than one
// chunk and dX is bf16, the fp32 dX accumulator of one wave, then, when there is more
// than one wave, the fp32 dW accumulator of the whole vocabulary (dW of wave 0 is
// stored into it, later waves add, the last one writes bf16): the token-wave form of
// the backward in the Liger-Kernel commit "native Blackwell tensor-parallel fused
// scaled linear cross-entropy", sections "Implementation / Backward" and "Correctness".
struct BwdPlan {
  int64_t rows = 0, chunk = 0;
  bool pipe = false;               // grouped launches over two d-logit buffers
  int nbuf = 1;                    // d-logit buffers
  bool dx_acc = false, dw_acc = false;
  size_t dz_bytes = 0, off_dx = 0, off_dw = 0, off_q = 0, total = 0;
};

// Steps (token waves x vocabulary chunks) of a schedule.
int64_t plan_steps(int64_t M, int64_t V, int64_t rows, int64_t chunk) {
  return cdiv(M, rows) * cdiv(cdiv(V, kTile) * kTile, chunk);
}

// Every launch of a schedule within the dispatch limits: the d-logit, dW and dX grids
// of the largest step (their sum when pipelined).
bool grids_ok(int64_t H, int64_t rows, int64_t chunk, bool pipe) {
  const int64_t n_mt = cdiv(rows, kTile), n_ct = cdiv(chunk, kTile), n_ht = cdiv(H, kTile);
  const int64_t dl = n_mt * n_ct, dw = n_ct * n_ht, dx = n_mt * n_ht;
  if (pipe) return dl + dw + dx + 24 <= kMaxWorkgroups;
  return dl <= kMaxWorkgroups && dw <= kMaxWorkgroups && dx <= kMaxWorkgroups;
}

BwdPlan bwd_plan(int64_t M, int64_t H, int64_t V, int64_t rows, int64_t chunk, bool dx_bf16,
                 bool pipe) {
  const int64_t Mpad = cdiv(M, kTile) * kTile;
  const int64_t Vpad = cdiv(V, kTile) * kTile;
  BwdPlan p;
  p.rows = rows < Mpad ? rows : Mpad;
  p.chunk = chunk;
  p.pipe = pipe;
  p.nbuf = (pipe && Mpad > 0 && plan_steps(M, V, p.rows, chunk) > 1) ? 2 : 1;
  const int64_t wave_m = p.rows < M ? p.rows : M;  // token rows of the largest wave
  p.dz_bytes = align_up(size_t(p.rows) * size_t(chunk) * 2);
  size_t b = size_t(p.nbuf) * p.dz_bytes;
  p.dx_acc = dx_bf16 && chunk < Vpad;
  if (p.dx_acc) {
    p.off_dx = b;
    b += align_up(size_t(wave_m) * size_t(H) * sizeof(float));
  }
  p.dw_acc = p.rows < Mpad;
  if (p.dw_acc) {
    p.off_dw = b;
    b += align_up(size_t(V) * size_t(H) * sizeof(float));
  }
  p.off_q = b;
  p.total = Mpad > 0 ? b + flce::kQueueBytes : 0;  // no rows: no launch
  return p;
}

// Widest chunk (a multiple of 256, at most min(Vpad, kMaxChunk)) for waves of `rows`
// rows whose plan fits in `bytes`; 0 if none.
int64_t widest_chunk(int64_t M, int64_t H, int64_t V, int64_t rows, bool dx_bf16, bool pipe,
                     size_t bytes) {
  const int64_t Vpad = cdiv(V, kTile) * kTile;
  const int64_t Mpad = cdiv(M, kTile) * kTile;
  const int64_t R = rows < Mpad ? rows : Mpad;
  if (!grids_ok(H, R, kTile, pipe)) return 0;
  if (Vpad <= kMaxChunk && grids_ok(H, R, Vpad, pipe) &&
      bwd_plan(M, H, V, rows, Vpad, dx_bf16, pipe).total <= bytes)
    return Vpad;
  // narrower chunks: the size grows with the chunk from here on
  const BwdPlan p0 = bwd_plan(M, H, V, rows, kTile, dx_bf16, pipe);
  if (p0.total > bytes) return 0;
  const size_t fixed = p0.total - size_t(p0.nbuf) * p0.dz_bytes;
  int64_t c = int64_t((bytes - fixed) / (size_t(p0.nbuf) * size_t(p0.rows) * 2)) / kTile * kTile;
  const int64_t cap = (Vpad <= kMaxChunk ? Vpad - kTile : kMaxChunk);
  if (c > cap) c = cap;
  // the chunk's tile columns within the dispatch limits (for the d-logit and dW grids)
  const int64_t n_mt = cdiv(R, kTile), n_ht = cdiv(H, kTile);
  const int64_t by_grid = (pipe ? (kMaxWorkgroups - 24 - n_mt * n_ht) / (n_mt + n_ht)
                                : kMaxWorkgroups / (n_mt > n_ht ? n_mt : n_ht)) * kTile;
  if (c > by_grid) c = by_grid / kTile * kTile;
  while (c > kTile && bwd_plan(M, H, V, rows, c, dx_bf16, pipe).total > bytes) c -= kTile;
  return c >= kTile ? c : 0;
}

// Pipelined launches only for steps of at most this much work (6 x rows x H x chunk
// FLOP).  Measured on MI355X: at M = H = 4096, V = 32768 (3.3e12 FLOP in one step) two
// launches instead of three take the backward from 2.60 to 2.42 ms; at M = H = 8192,
// V = 131072 (5.3e13) the grouped dW + dX launch costs 3% (36.4 -> 37.6 ms: the XCDs
// leave the dW phase at different times, and the W columns the dX tiles of all XCDs
// read in step stop being shared through the memory-side cache), and at M = 32767,
// H = 2048, V = 151936 the best pipelined schedule is 1% behind the sequential one.
constexpr double kPipeMaxStepFlop = 8e12;

// HBM bytes a plan moves beyond the d-logits themselves, plus its launches (10 us each,
// at 8 TB/s): the fp32 dX accumulator is read and written once per extra chunk, the
// fp32 dW accumulator once per extra wave; a pipelined plan makes one launch per step
// (plus one) instead of three.  Used only to rank plans that fit.
double plan_cost(int64_t M, int64_t H, int64_t V, const BwdPlan& p) {
  const int64_t Vpad = cdiv(V, kTile) * kTile;
  const double n_chunks = double(cdiv(Vpad, p.chunk)), n_waves = double(cdiv(M, p.rows));
  const double steps = n_chunks * n_waves;
  double c = 80e6 * (p.pipe ? steps + 1.0 : 3.0 * steps);
  if (p.chunk < Vpad) c += (n_chunks - 1.0) * 8.0 * double(M) * double(H);
  if (p.dw_acc) c += (n_waves - 1.0) * 8.0 * double(V) * double(H);
  return c;
}

// The schedule flce_backward (dx_bf16) or flce_backward_shard runs with `bytes` of
// workspace: among one wave of every row and waves of 16384 down to 256 rows, each
// pipelined (two d-logit buffers) or not, with the widest chunk that fits, the one that
// moves the fewest extra bytes; chunk 0 if nothing fits.
BwdPlan plan_for_workspace(int64_t M, int64_t H, int64_t V, bool dx_bf16, size_t bytes) {
  const int64_t Mpad = cdiv(M, kTile) * kTile;
  BwdPlan best;
  if (Mpad == 0) {  // no token: nothing is staged
    const int64_t Vpad = cdiv(V, kTile) * kTile;
    best.chunk = Vpad < kMaxChunk ? Vpad : kMaxChunk;
    return best;
  }
  double best_cost = 0.0;
  auto consider = [&](int64_t rows) {
    for (int pipe = 1; pipe >= 0; --pipe) {
      const int64_t c = widest_chunk(M, H, V, rows, dx_bf16, pipe == 1, bytes);
      if (c == 0) continue;
      if (pipe == 1 && 6.0 * double(rows) * double(H) * double(c) > kPipeMaxStepFlop) continue;
      const BwdPlan p = bwd_plan(M, H, V, rows, c, dx_bf16, pipe == 1);
      const double cost = plan_cost(M, H, V, p);
      if (best.chunk == 0 || cost < best_cost) {
        best = p;
        best_cost = cost;
      }
    }
  };
  consider(Mpad);  // one wave of every row
  for (int64_t rows = 16384; rows >= kTile; rows /= 2)
    if (rows < Mpad) consider(rows);
  return best;
}

// Preferred chunk: the d-logits of one wave of every row within kDzBudget.
int64_t preferred_chunk(int64_t M, int64_t V) {
  const int64_t Mpad = cdiv(M, kTile) * kTile;
  const int64_t Vpad = cdiv(V, kTile) * kTile;
  if (Mpad == 0) return Vpad < kMaxChunk ? Vpad : kMaxChunk;
  int64_t c = int64_t(kDzBudget / (size_t(Mpad) * 2)) / kTile * kTile;
  if (c < kTile) c = kTile;
  if (c > kMaxChunk) c = kMaxChunk;
  return c < Vpad ? c : Vpad;
}

// Smallest workspace any schedule fits in (independent of M once waves are possible).
size_t bwd_min_bytes(int64_t M, int64_t H, int64_t V, bool dx_bf16) {
  const int64_t Mpad = cdiv(M, kTile) * kTile;
  const int64_t Vpad = cdiv(V, kTile) * kTile;
  size_t m = SIZE_MAX;
  auto take = [&](int64_t rows, int64_t chunk) {
    const int64_t R = rows < Mpad ? rows : Mpad;
    if (Mpad == 0 || grids_ok(H, R, chunk, false))
      m = std::min(m, bwd_plan(M, H, V, rows, chunk, dx_bf16, false).total);
  };
  take(Mpad, kTile);
  if (Vpad <= kMaxChunk) take(Mpad, Vpad);
  if (Mpad > kTile) {
    take(kTile, kTile);
    if (Vpad <= kMaxChunk) take(kTile, Vpad);
  }
  return m;
}

flce_status_t hip_fail(hipError_t e, const char* what) {
  return fail(FLCE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// A forward over no tokens: only the scalar arguments are checked; nothing is read or
// written, so every pointer may be NULL.
flce_status_t check_empty(int64_t H, int64_t V, int compute_entropy) {
  flce_status_t st = check_shape(0, H, V);
  if (st != FLCE_OK) return st;
  if (compute_entropy != 0 && compute_entropy != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "compute_entropy must be 0 or 1");
  return ok();
}

// The backward over no tokens: dW = 0 (dX has no elements; nothing else is touched).
flce_status_t zero_dw_of_empty_batch(int64_t H, int64_t V, void* dW, hipStream_t stream) {
  flce_status_t st = check_shape(0, H, V);
  if (st != FLCE_OK) return st;
  if (!dW) return fail(FLCE_ERR_INVALID_VALUE, "dW is NULL");
  if (!aligned(dW, 16)) return fail(FLCE_ERR_UNSUPPORTED, "dW must be 16-byte aligned");
  const hipError_t e = flce::launch_fill_zero_u16(static_cast<uint16_t*>(dW), long(V * H), stream);
  if (e != hipSuccess) return hip_fail(e, "zero-fill kernel launch");
  return ok();
}

}  // namespace

extern "C" {

const char* flce_version(void) { return "0.1.0"; }

const char* flce_status_string(flce_status_t s) {
  switch (s) {
    case FLCE_OK: return "FLCE_OK";
    case FLCE_ERR_INVALID_VALUE: return "FLCE_ERR_INVALID_VALUE";
    case FLCE_ERR_UNSUPPORTED: return "FLCE_ERR_UNSUPPORTED";
    case FLCE_ERR_WORKSPACE_TOO_SMALL: return "FLCE_ERR_WORKSPACE_TOO_SMALL";
    case FLCE_ERR_HIP: return "FLCE_ERR_HIP";
  }
  return "FLCE_ERR_UNKNOWN";
}

const char* flce_last_error_message(void) { return g_last_error; }

flce_status_t flce_workspace_query(int64_t M, int64_t H, int64_t V, int compute_entropy,
                                   size_t* fwd_bytes, size_t* bwd_bytes) {
  if (compute_entropy != 0 && compute_entropy != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "compute_entropy must be 0 or 1");
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (fwd_bytes) {
    const int64_t cap = max_wave_rows(V);
    *fwd_bytes = fwd_layout(M < cap ? M : cap, V, compute_entropy == 1).total;
  }
  if (bwd_bytes)
    *bwd_bytes =
        bwd_plan(M, H, V, cdiv(M, kTile) * kTile, preferred_chunk(M, V), true, false).total;
  return ok();
}

flce_status_t flce_forward_workspace_min(int64_t M, int64_t H, int64_t V, int compute_entropy,
                                         size_t* bytes) {
  if (compute_entropy != 0 && compute_entropy != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "compute_entropy must be 0 or 1");
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (!bytes) return fail(FLCE_ERR_INVALID_VALUE, "bytes is NULL");
  *bytes = M == 0 ? 0 : fwd_layout(kTile, V, compute_entropy == 1).total;
  return ok();
}

flce_status_t flce_forward_wave_rows(int64_t M, int64_t H, int64_t V, int compute_entropy,
                                     size_t workspace_bytes, int64_t* rows) {
  if (compute_entropy != 0 && compute_entropy != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "compute_entropy must be 0 or 1");
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (!rows) return fail(FLCE_ERR_INVALID_VALUE, "rows is NULL");
  if (M == 0) {
    *rows = 0;
    return ok();
  }
  const int64_t r = wave_rows_for_workspace(M, V, compute_entropy == 1, workspace_bytes);
  if (r == 0)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the minimum %zu",
                workspace_bytes, fwd_layout(kTile, V, compute_entropy == 1).total);
  *rows = r;
  return ok();
}

flce_status_t flce_backward_workspace_min(int64_t M, int64_t H, int64_t V, size_t* bytes) {
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (!bytes) return fail(FLCE_ERR_INVALID_VALUE, "bytes is NULL");
  *bytes = bwd_min_bytes(M, H, V, true);
  return ok();
}

flce_status_t flce_backward_chunk_cols(int64_t M, int64_t H, int64_t V, size_t workspace_bytes,
                                       int64_t* chunk_cols) {
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (!chunk_cols) return fail(FLCE_ERR_INVALID_VALUE, "chunk_cols is NULL");
  const BwdPlan p = plan_for_workspace(M, H, V, true, workspace_bytes);
  if (p.chunk == 0)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the minimum %zu",
                workspace_bytes, bwd_min_bytes(M, H, V, true));
  *chunk_cols = p.chunk;
  return ok();
}

flce_status_t flce_backward_schedule(int64_t M, int64_t H, int64_t V, size_t workspace_bytes,
                                     int64_t* rows, int64_t* chunk_cols, int* pipelined) {
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  const BwdPlan p = plan_for_workspace(M, H, V, true, workspace_bytes);
  if (p.chunk == 0)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the minimum %zu",
                workspace_bytes, bwd_min_bytes(M, H, V, true));
  if (rows) *rows = p.rows;
  if (chunk_cols) *chunk_cols = p.chunk;
  if (pipelined) *pipelined = p.pipe ? 1 : 0;
  return ok();
}

flce_status_t flce_backward_wave_rows(int64_t M, int64_t H, int64_t V, size_t workspace_bytes,
                                      int64_t* rows) {
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (!rows) return fail(FLCE_ERR_INVALID_VALUE, "rows is NULL");
  const BwdPlan p = plan_for_workspace(M, H, V, true, workspace_bytes);
  if (p.chunk == 0)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the minimum %zu",
                workspace_bytes, bwd_min_bytes(M, H, V, true));
  *rows = p.rows;
  return ok();
}

namespace {

flce_status_t check_forward_common(const int64_t* targets, int64_t M, int64_t H, int64_t V,
                                   int compute_entropy, const void* workspace,
                                   size_t workspace_bytes, FwdLayout* L) {
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (compute_entropy != 0 && compute_entropy != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "compute_entropy must be 0 or 1");
  if (!aligned(targets, 8)) return fail(FLCE_ERR_UNSUPPORTED, "targets must be 8-byte aligned");
  if (!aligned(workspace, kAlign))
    return fail(FLCE_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  if (M > max_wave_rows(V))
    return fail(FLCE_ERR_UNSUPPORTED,
                "%lld rows over V=%lld exceed one launch (at most %lld rows); flce_forward "
                "runs such batches in token waves", (long long)M, (long long)V,
                (long long)max_wave_rows(V));
  *L = fwd_layout(M, V, compute_entropy == 1);
  if (workspace_bytes < L->total)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL, "forward needs %zu workspace bytes, got %zu",
                L->total, workspace_bytes);
  return FLCE_OK;
}

flce_status_t check_forward_inputs(const void* X, const void* W, float scale) {
  if (!std::isfinite(scale)) return fail(FLCE_ERR_INVALID_VALUE, "scale is not finite");
  if (!aligned(X, 16) || !aligned(W, 16))
    return fail(FLCE_ERR_UNSUPPORTED, "X and W must be 16-byte aligned");
  return FLCE_OK;
}

flce_status_t check_forward_outputs(int compute_entropy, const float* logprob, const float* lse,
                                    const float* entropy) {
  if (compute_entropy == 1 && !entropy)
    return fail(FLCE_ERR_INVALID_VALUE, "entropy is NULL while compute_entropy == 1");
  if (!aligned(logprob, 4) || !aligned(lse, 4) || (entropy && !aligned(entropy, 4)))
    return fail(FLCE_ERR_UNSUPPORTED, "outputs must be 4-byte aligned");
  return FLCE_OK;
}

flce::FwdTileArgs tile_args(const void* X, const void* W, const int64_t* targets, int64_t M,
                            int64_t H, int64_t V, int64_t v_off, int64_t ignore_index,
                            float scale, bool ent, const FwdLayout& L, char* ws) {
  flce::FwdTileArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.W = static_cast<const uint16_t*>(W);
  a.targets = targets;
  a.M = int(M);
  a.H = int(H);
  a.V = int(V);
  a.v_off = v_off;
  a.ignore_index = ignore_index;
  a.scale = scale;
  a.n_mt = int(L.n_mt);
  a.n_vt = int(L.n_vt);
  a.Mpad = int(L.Mpad);
  a.part_m = reinterpret_cast<float*>(ws + L.off_m);
  a.part_s = reinterpret_cast<float*>(ws + L.off_s);
  a.part_u = ent ? reinterpret_cast<float*>(ws + L.off_u) : nullptr;
  a.zt = reinterpret_cast<float*>(ws + L.off_zt);
  a.tq.ctr = reinterpret_cast<unsigned long long*>(ws + L.off_q);
  return a;
}

// Entry r of a shard table: the partials of vocabulary ids [v_lo, v_hi), laid out as
// fwd_layout(rows, v_hi - v_lo) at byte offset `at` from the merge's base.
void set_shard(flce::ShardTable& t, int r, int64_t v_lo, int64_t v_hi, const FwdLayout& L,
               size_t at) {
  t.v_lo[r] = v_lo;
  t.v_lo[r + 1] = v_hi;
  t.n_vt[r] = int(L.n_vt);
  t.part_m[r] = long((at + L.off_m) / sizeof(float));
  t.part_s[r] = long((at + L.off_s) / sizeof(float));
  t.part_u[r] = long((at + L.off_u) / sizeof(float));
  t.zt[r] = long((at + L.off_zt) / sizeof(float));
}

flce::FwdMergeArgs merge_args(const int64_t* targets, int64_t M, int64_t ignore_index, bool ent,
                              float* logprob, float* lse, float* entropy, int64_t Mpad,
                              const void* base) {
  flce::FwdMergeArgs b{};
  b.targets = targets;
  b.M = int(M);
  b.ignore_index = ignore_index;
  b.Mpad = int(Mpad);
  b.base = static_cast<const float*>(base);
  b.logprob = logprob;
  b.lse = lse;
  b.entropy = ent ? entropy : nullptr;
  return b;
}

// Merge of one unsharded layout at ws.
flce::FwdMergeArgs merge_args_single(const int64_t* targets, int64_t M, int64_t V,
                                     int64_t ignore_index, bool ent, float* logprob, float* lse,
                                     float* entropy, const FwdLayout& L, const char* ws) {
  flce::FwdMergeArgs b = merge_args(targets, M, ignore_index, ent, logprob, lse, entropy, L.Mpad, ws);
  b.sh.n = 1;
  set_shard(b.sh, 0, 0, V, L, 0);
  return b;
}

}  // namespace

flce_status_t flce_forward_partials_shard(const void* X, const void* W_shard,
                                          const int64_t* targets, int64_t M, int64_t H,
                                          int64_t V_shard, int64_t v_offset,
                                          int64_t ignore_index, float scale, int compute_entropy,
                                          void* workspace, size_t workspace_bytes,
                                          hipStream_t stream) {
  if (M == 0) return check_empty(H, V_shard, compute_entropy);
  if (!X || !W_shard || !targets || !workspace)
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among X, W, targets, workspace");
  if (v_offset < 0 || v_offset > kMaxV - V_shard)
    return fail(FLCE_ERR_INVALID_VALUE, "v_offset %lld out of range for a shard of %lld rows",
                (long long)v_offset, (long long)V_shard);
  FwdLayout L;
  flce_status_t st = check_forward_common(targets, M, H, V_shard, compute_entropy, workspace,
                                          workspace_bytes, &L);
  if (st != FLCE_OK) return st;
  st = check_forward_inputs(X, W_shard, scale);
  if (st != FLCE_OK) return st;
  const bool ent = compute_entropy == 1;
  const flce::FwdTileArgs a = tile_args(X, W_shard, targets, M, H, V_shard, v_offset,
                                        ignore_index, scale, ent, L,
                                        static_cast<char*>(workspace));
  // the target-logit kernel first: it zeroes the tile kernel's queue counters
  hipError_t e = flce::launch_target_logit(a, stream);
  if (e != hipSuccess) return hip_fail(e, "target logit kernel launch");
  e = flce::launch_fwd_tile(a, ent, stream);
  if (e != hipSuccess) return hip_fail(e, "forward tile kernel launch");
  return ok();
}

flce_status_t flce_forward_partials(const void* X, const void* W, const int64_t* targets,
                                    int64_t M, int64_t H, int64_t V, int64_t ignore_index,
                                    float scale, int compute_entropy, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  return flce_forward_partials_shard(X, W, targets, M, H, V, 0, ignore_index, scale,
                                     compute_entropy, workspace, workspace_bytes, stream);
}

flce_status_t flce_forward_merge_shards(const int64_t* targets, int64_t M, int64_t n_shards,
                                        const int64_t* shard_offsets, int64_t ignore_index,
                                        int compute_entropy, float* logprob, float* lse,
                                        float* entropy, const void* gathered,
                                        size_t shard_stride_bytes, hipStream_t stream) {
  if (M < 0) return fail(FLCE_ERR_INVALID_VALUE, "M must be >= 0 (got %lld)", (long long)M);
  if (M == 0) return ok();
  if (!targets || !shard_offsets || !logprob || !lse || !gathered)
    return fail(FLCE_ERR_INVALID_VALUE,
                "NULL pointer among targets, shard_offsets, logprob, lse, gathered");
  if (n_shards < 1 || n_shards > flce::kMaxShards)
    return fail(FLCE_ERR_UNSUPPORTED, "n_shards must be in [1, %d] (got %lld)", flce::kMaxShards,
                (long long)n_shards);
  if (compute_entropy != 0 && compute_entropy != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "compute_entropy must be 0 or 1");
  if (M > kMaxWaveRows)
    return fail(FLCE_ERR_UNSUPPORTED, "M=%lld exceeds one merge launch (at most %lld rows)",
                (long long)M, (long long)kMaxWaveRows);
  if (shard_offsets[0] != 0)
    return fail(FLCE_ERR_INVALID_VALUE, "shard_offsets[0] must be 0 (got %lld)",
                (long long)shard_offsets[0]);
  if (!aligned(targets, 8)) return fail(FLCE_ERR_UNSUPPORTED, "targets must be 8-byte aligned");
  if (!aligned(gathered, kAlign) || shard_stride_bytes % kAlign != 0)
    return fail(FLCE_ERR_UNSUPPORTED, "gathered and shard_stride_bytes must be 256-byte aligned");
  flce_status_t st = check_forward_outputs(compute_entropy, logprob, lse, entropy);
  if (st != FLCE_OK) return st;
  const bool ent = compute_entropy == 1;
  flce::FwdMergeArgs b = merge_args(targets, M, ignore_index, ent, logprob, lse, entropy,
                                    cdiv(M, kTile) * kTile, gathered);
  b.sh.n = int(n_shards);
  for (int64_t r = 0; r < n_shards; ++r) {
    const int64_t lo = shard_offsets[r], hi = shard_offsets[r + 1];
    if (hi <= lo)
      return fail(FLCE_ERR_INVALID_VALUE, "shard %lld is empty or reversed ([%lld, %lld))",
                  (long long)r, (long long)lo, (long long)hi);
    st = check_shape(M, 8, hi - lo);
    if (st != FLCE_OK) return st;
    if (hi > kMaxV) return fail(FLCE_ERR_UNSUPPORTED, "vocabulary larger than 2^30");
    const FwdLayout L = fwd_layout(M, hi - lo, ent);
    if (L.total > shard_stride_bytes)
      return fail(FLCE_ERR_WORKSPACE_TOO_SMALL,
                  "shard %lld needs %zu bytes of partials, stride is %zu", (long long)r, L.total,
                  shard_stride_bytes);
    set_shard(b.sh, int(r), lo, hi, L, size_t(r) * shard_stride_bytes);
  }
  const hipError_t e = flce::launch_fwd_merge(b, ent, stream);
  if (e != hipSuccess) return hip_fail(e, "forward merge kernel launch");
  return ok();
}

flce_status_t flce_forward_merge(const int64_t* targets, int64_t M, int64_t H, int64_t V,
                                 int64_t ignore_index, int compute_entropy, float* logprob,
                                 float* lse, float* entropy, const void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (M == 0) return check_empty(H, V, compute_entropy);
  if (!targets || !logprob || !lse || !workspace)
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among targets, logprob, lse, workspace");
  FwdLayout L;
  flce_status_t st =
      check_forward_common(targets, M, H, V, compute_entropy, workspace, workspace_bytes, &L);
  if (st != FLCE_OK) return st;
  st = check_forward_outputs(compute_entropy, logprob, lse, entropy);
  if (st != FLCE_OK) return st;
  const bool ent = compute_entropy == 1;
  const flce::FwdMergeArgs b = merge_args_single(targets, M, V, ignore_index, ent, logprob, lse,
                                                 entropy, L, static_cast<const char*>(workspace));
  const hipError_t e = flce::launch_fwd_merge(b, ent, stream);
  if (e != hipSuccess) return hip_fail(e, "forward merge kernel launch");
  return ok();
}

}  // extern "C"

namespace {

// Checks shared by flce_forward and flce_forward_noalloc (everything but the workspace).
flce_status_t check_forward_call(const void* X, const void* W, const int64_t* targets,
                                 int64_t M, int64_t H, int64_t V, float scale,
                                 int compute_entropy, const float* logprob, const float* lse,
                                 const float* entropy) {
  if (!X || !W || !targets || !logprob || !lse)
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among X, W, targets, logprob, lse");
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (compute_entropy != 0 && compute_entropy != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "compute_entropy must be 0 or 1");
  if (!aligned(targets, 8)) return fail(FLCE_ERR_UNSUPPORTED, "targets must be 8-byte aligned");
  st = check_forward_inputs(X, W, scale);
  if (st != FLCE_OK) return st;
  return check_forward_outputs(compute_entropy, logprob, lse, entropy);
}

// The forward in token waves of `rows` rows (a multiple of 256) through the workspace ws:
// per wave, the tile kernel, the target logits and the merge.
flce_status_t forward_waves(const void* X, const void* W, const int64_t* targets, int64_t M,
                            int64_t H, int64_t V, int64_t ignore_index, float scale, bool ent,
                            float* logprob, float* lse, float* entropy, char* ws, int64_t rows,
                            hipStream_t stream) {
  for (int64_t r0 = 0; r0 < M; r0 += rows) {
    const int64_t mw = M - r0 < rows ? M - r0 : rows;
    const FwdLayout L = fwd_layout(mw, V, ent);
    const flce::FwdTileArgs a =
        tile_args(static_cast<const uint16_t*>(X) + r0 * H, W, targets + r0, mw, H, V, 0,
                  ignore_index, scale, ent, L, ws);
    hipError_t e = flce::launch_target_logit(a, stream);  // zeroes the queue counters
    if (e != hipSuccess) return hip_fail(e, "target logit kernel launch");
    e = flce::launch_fwd_tile(a, ent, stream);
    if (e != hipSuccess) return hip_fail(e, "forward tile kernel launch");
    const flce::FwdMergeArgs b =
        merge_args_single(targets + r0, mw, V, ignore_index, ent, logprob + r0, lse + r0,
                          ent ? entropy + r0 : nullptr, L, ws);
    e = flce::launch_fwd_merge(b, ent, stream);
    if (e != hipSuccess) return hip_fail(e, "forward merge kernel launch");
  }
  return ok();
}

}  // namespace

extern "C" {

flce_status_t flce_forward(const void* X, const void* W, const int64_t* targets, int64_t M,
                           int64_t H, int64_t V, int64_t ignore_index, float scale,
                           int compute_entropy, float* logprob, float* lse, float* entropy,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (M == 0) return check_empty(H, V, compute_entropy);
  flce_status_t st = check_forward_call(X, W, targets, M, H, V, scale, compute_entropy, logprob,
                                        lse, entropy);
  if (st != FLCE_OK) return st;
  if (!workspace) return fail(FLCE_ERR_INVALID_VALUE, "workspace is NULL");
  if (!aligned(workspace, kAlign))
    return fail(FLCE_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  const bool ent = compute_entropy == 1;
  // token waves: as many 256-row tiles per wave as the workspace holds partials for
  const int64_t rows = wave_rows_for_workspace(M, V, ent, workspace_bytes);
  if (rows == 0)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL, "forward needs at least %zu workspace bytes, got %zu",
                fwd_layout(kTile, V, ent).total, workspace_bytes);
  return forward_waves(X, W, targets, M, H, V, ignore_index, scale, ent, logprob, lse, entropy,
                       static_cast<char*>(workspace), rows, stream);
}

static_assert(flce::kScratchBytes == FLCE_NOALLOC_SCRATCH_BYTES, "scratch size in the header");

flce_status_t flce_forward_noalloc(const void* X, const void* W, const int64_t* targets,
                                   int64_t M, int64_t H, int64_t V, int64_t ignore_index,
                                   float scale, int compute_entropy, float* logprob, float* lse,
                                   float* entropy, hipStream_t stream) {
  if (M == 0) return check_empty(H, V, compute_entropy);
  flce_status_t st = check_forward_call(X, W, targets, M, H, V, scale, compute_entropy, logprob,
                                        lse, entropy);
  if (st != FLCE_OK) return st;
  const bool ent = compute_entropy == 1;
  const int64_t rows = wave_rows_for_workspace(M, V, ent, flce::kScratchBytes);
  if (rows == 0)
    return fail(FLCE_ERR_UNSUPPORTED,
                "V=%lld needs %zu bytes of partials per 256-row wave; the static scratch of "
                "flce_forward_noalloc holds %zu (use flce_forward with a workspace)",
                (long long)V, fwd_layout(kTile, V, ent).total, flce::kScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = flce::scratch_device_address(&scratch);
  if (e != hipSuccess) return hip_fail(e, "device scratch address");
  return forward_waves(X, W, targets, M, H, V, ignore_index, scale, ent, logprob, lse, entropy,
                       static_cast<char*>(scratch), rows, stream);
}

}  // extern "C"

namespace {

flce_status_t check_backward_inputs(const void* X, const void* W, const int64_t* targets,
                                    float scale, const float* lse, const float* entropy,
                                    const float* grad_logprob, const float* grad_entropy,
                                    const void* dX, const void* dW, const void* workspace) {
  if (grad_entropy && !entropy)
    return fail(FLCE_ERR_INVALID_VALUE, "grad_entropy given but entropy is NULL");
  if (!std::isfinite(scale)) return fail(FLCE_ERR_INVALID_VALUE, "scale is not finite");
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(dX, 16) || !aligned(dW, 16))
    return fail(FLCE_ERR_UNSUPPORTED, "X, W, dX and dW must be 16-byte aligned");
  if (!aligned(targets, 8) || !aligned(lse, 4) || (entropy && !aligned(entropy, 4)) ||
      (grad_logprob && !aligned(grad_logprob, 4)) || (grad_entropy && !aligned(grad_entropy, 4)))
    return fail(FLCE_ERR_UNSUPPORTED, "targets and fp32 vectors must be naturally aligned");
  if (!aligned(workspace, kAlign))
    return fail(FLCE_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  return FLCE_OK;
}

// The backward under plan P: W holds rows v_off .. v_off + V - 1 of a vocabulary of
// V_total ids.  For each token wave and each vocabulary chunk: the d-logits of the
// wave's rows over the chunk, the chunk's rows of dW (K = the wave's rows) and the
// wave's rows of dX (K = the chunk's columns).  dX goes either to dX_bf16 (through the
// wave's fp32 accumulator in the workspace when a wave takes more than one chunk) or,
// when dX_bf16 is NULL, to the caller's fp32 dX_f32, which it overwrites (acc_in false)
// or adds to (acc_in true).  With more than one wave dW accumulates in fp32 in the
// workspace across waves in wave order (deterministic), and the last wave writes bf16.
flce_status_t backward_run(const void* X, const void* W, const int64_t* targets, int64_t M,
                           int64_t H, int64_t V, int64_t v_off, int64_t V_total,
                           int64_t ignore_index, float scale, const float* lse,
                           const float* entropy, const float* grad_logprob,
                           const float* grad_entropy, uint16_t* dX_bf16, float* dX_f32,
                           bool acc_in, void* dW, char* ws, const BwdPlan& P,
                           hipStream_t stream) {
  const int64_t Vpad = cdiv(V, kTile) * kTile;
  const int64_t n_chunks = cdiv(Vpad, P.chunk);
  const int64_t n_waves = cdiv(M, P.rows);
  const int64_t steps = n_chunks * n_waves;
  const bool entgrad = grad_entropy != nullptr;
  float* dx_acc = P.dx_acc ? reinterpret_cast<float*>(ws + P.off_dx) : nullptr;
  float* dw_acc = P.dw_acc ? reinterpret_cast<float*>(ws + P.off_dw) : nullptr;
  const uint16_t* Xb = static_cast<const uint16_t*>(X);

  // the three kernels' arguments for step k = (wave k / n_chunks, chunk k % n_chunks)
  struct Step {
    flce::DlogitsArgs d;
    flce::GemmDwArgs g;
    flce::GemmDxArgs x;
  };
  auto step_args = [&](int64_t k) {
    const int64_t w = k / n_chunks, c = k % n_chunks;
    const int64_t r0 = w * P.rows;
    const int64_t mw = (M - r0) < P.rows ? (M - r0) : P.rows;
    const int64_t n_mt = cdiv(mw, kTile);
    const int64_t vbase = c * P.chunk;
    const int64_t kc = (Vpad - vbase) < P.chunk ? (Vpad - vbase) : P.chunk;
    uint16_t* dz = reinterpret_cast<uint16_t*>(ws + size_t(k % P.nbuf) * P.dz_bytes);
    Step s{};
    flce::DlogitsArgs& d = s.d;
    d.X = Xb + r0 * H;
    d.W = static_cast<const uint16_t*>(W);
    d.targets = targets + r0;
    d.M = int(mw);
    d.H = int(H);
    d.V = int(V);
    d.v_off = v_off;
    d.V_total = V_total;
    d.ignore_index = ignore_index;
    d.scale = scale;
    d.lse = lse + r0;
    d.entropy = entropy ? entropy + r0 : nullptr;
    d.grad_logprob = grad_logprob ? grad_logprob + r0 : nullptr;
    d.grad_entropy = grad_entropy ? grad_entropy + r0 : nullptr;
    d.vbase = int(vbase);
    d.n_mt = int(n_mt);
    d.n_vt = int(kc / kTile);
    d.dz = dz;
    d.ldz = long(P.chunk);

    flce::GemmDwArgs& g = s.g;
    g.dz = dz;
    g.ldz = long(P.chunk);
    g.X = Xb + r0 * H;
    g.dW = static_cast<uint16_t*>(dW);
    g.acc = dw_acc;
    g.M = int(mw);
    g.Mpad = int(n_mt * kTile);
    g.H = int(H);
    g.V = int(V);
    g.vbase = int(vbase);
    g.chunk_cols = int(kc);
    g.n_i = int(kc / kTile);
    g.n_h = int(cdiv(H, kTile));
    g.mode = n_waves == 1 ? 0 : (w == 0 ? 1 : (w == n_waves - 1 ? 3 : 2));

    flce::GemmDxArgs& x = s.x;
    x.dz = dz;
    x.ldz = long(P.chunk);
    x.W = static_cast<const uint16_t*>(W);
    x.dX = dX_bf16 ? dX_bf16 + r0 * H : nullptr;
    x.M = int(mw);
    x.H = int(H);
    x.V = int(V);
    x.vbase = int(vbase);
    x.kcols = int(kc);
    x.n_m = int(n_mt);
    x.n_h = int(cdiv(H, kTile));
    if (dX_bf16) {
      x.acc = dx_acc;
      x.mode = n_chunks == 1 ? 0 : (c == 0 ? 1 : (c == n_chunks - 1 ? 3 : 2));
    } else {
      x.acc = dX_f32 + r0 * H;
      x.mode = (c == 0 && !acc_in) ? 1 : 2;
    }
    return s;
  };

  if (!P.pipe) {
    // queue counters: the d-logit launches use q0 and zero q1, the dW launches use q1 and
    // zero q0, so each starts from zero; q0 is zeroed here for the first step, unless no
    // launch of the call queues tiles.  Grids differ only between the first and last
    // wave and the first and last chunk, so the four corner steps cover every launch.
    unsigned long long* q0 = reinterpret_cast<unsigned long long*>(ws + P.off_q);
    unsigned long long* q1 = q0 + 8;
    auto queues = [&](int64_t k) {
      const Step s = step_args(k);
      return flce::queue_shape(int64_t(s.d.n_mt) * s.d.n_vt).queue > 0 ||
             flce::queue_shape(int64_t(s.g.n_i) * s.g.n_h).queue > 0;
    };
    hipError_t e = hipSuccess;
    if (queues(0) || queues(n_chunks - 1) || queues((n_waves - 1) * n_chunks) ||
        queues(steps - 1)) {
      e = flce::launch_fill_zero_u16(reinterpret_cast<uint16_t*>(q0), long(8 * sizeof(*q0) / 2),
                                     stream);
      if (e != hipSuccess) return hip_fail(e, "zero-fill kernel launch");
    }
    for (int64_t k = 0; k < steps; ++k) {
      Step s = step_args(k);
      s.d.tq.ctr = q0;
      s.d.tq.clear = q1;
      s.g.tq.ctr = q1;
      s.g.tq.clear = q0;
      e = flce::launch_dlogits(s.d, entgrad, stream);
      if (e != hipSuccess) return hip_fail(e, "d-logits kernel launch");
      e = flce::launch_gemm_dw(s.g, stream);
      if (e != hipSuccess) return hip_fail(e, "dW GEMM launch");
      e = flce::launch_gemm_dx(s.x, stream);
      if (e != hipSuccess) return hip_fail(e, "dX GEMM launch");
    }
    return ok();
  }
  // pipelined: launch k runs the GEMMs of step k - 1 and the d-logits of step k, which
  // write the other d-logit buffer
  for (int64_t k = 0; k <= steps; ++k) {
    flce::PipeArgs a{};
    if (k < steps) {
      a.dl = step_args(k).d;
      a.n_dl = a.dl.n_mt * a.dl.n_vt;
    }
    if (k > 0) {
      const Step s = step_args(k - 1);
      a.dw = s.g;
      a.dx = s.x;
      a.n_dw = s.g.n_i * s.g.n_h;
      a.n_dx = s.x.n_m * s.x.n_h;
    }
    const hipError_t e = flce::launch_bwd_pipe(a, entgrad, stream);
    if (e != hipSuccess) return hip_fail(e, "pipelined backward launch");
  }
  return ok();
}

}  // namespace

extern "C" {

flce_status_t flce_backward(const void* X, const void* W, const int64_t* targets, int64_t M,
                            int64_t H, int64_t V, int64_t ignore_index, float scale,
                            const float* lse, const float* entropy, const float* grad_logprob,
                            const float* grad_entropy, void* dX, void* dW, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (M == 0) return zero_dw_of_empty_batch(H, V, dW, stream);
  if (!X || !W || !targets || !lse || !dX || !dW || !workspace)
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among X, W, targets, lse, dX, dW, workspace");
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  st = check_backward_inputs(X, W, targets, scale, lse, entropy, grad_logprob, grad_entropy, dX,
                             dW, workspace);
  if (st != FLCE_OK) return st;
  const BwdPlan P = plan_for_workspace(M, H, V, true, workspace_bytes);
  if (P.chunk == 0)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL, "backward needs at least %zu workspace bytes, got %zu",
                bwd_min_bytes(M, H, V, true), workspace_bytes);

  if (!grad_logprob && !grad_entropy) {
    hipError_t e = flce::launch_fill_zero_u16(static_cast<uint16_t*>(dX), long(M * H), stream);
    if (e == hipSuccess)
      e = flce::launch_fill_zero_u16(static_cast<uint16_t*>(dW), long(V * H), stream);
    if (e != hipSuccess) return hip_fail(e, "zero-fill kernel launch");
    return ok();
  }
  return backward_run(X, W, targets, M, H, V, 0, V, ignore_index, scale, lse, entropy,
                      grad_logprob, grad_entropy, static_cast<uint16_t*>(dX), nullptr, false, dW,
                      static_cast<char*>(workspace), P, stream);
}

flce_status_t flce_backward_shard_workspace_query(int64_t M, int64_t H, int64_t V_shard,
                                                  size_t* min_bytes, size_t* preferred_bytes) {
  flce_status_t st = check_shape(M, H, V_shard);
  if (st != FLCE_OK) return st;
  const int64_t Mpad = cdiv(M, kTile) * kTile;
  if (min_bytes) *min_bytes = bwd_min_bytes(M, H, V_shard, false);
  if (preferred_bytes)
    *preferred_bytes =
        bwd_plan(M, H, V_shard, Mpad, preferred_chunk(M, V_shard), false, false).total;
  return ok();
}

flce_status_t flce_backward_shard(const void* X, const void* W_shard, const int64_t* targets,
                                  int64_t M, int64_t H, int64_t V_shard, int64_t v_offset,
                                  int64_t V_total, int64_t ignore_index, float scale,
                                  const float* lse, const float* entropy,
                                  const float* grad_logprob, const float* grad_entropy,
                                  float* dX_partial, int accumulate, void* dW_shard,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (M == 0) {
    if (V_total > kMaxV) return fail(FLCE_ERR_UNSUPPORTED, "V_total larger than 2^30");
    if (v_offset < 0 || V_shard > V_total - v_offset)
      return fail(FLCE_ERR_INVALID_VALUE, "shard [%lld, %lld) does not lie in [0, V_total=%lld)",
                  (long long)v_offset, (long long)(v_offset + V_shard), (long long)V_total);
    return zero_dw_of_empty_batch(H, V_shard, dW_shard, stream);
  }
  if (!X || !W_shard || !targets || !lse || !dX_partial || !dW_shard || !workspace)
    return fail(FLCE_ERR_INVALID_VALUE,
                "NULL pointer among X, W_shard, targets, lse, dX_partial, dW_shard, workspace");
  flce_status_t st = check_shape(M, H, V_shard);
  if (st != FLCE_OK) return st;
  if (V_total > kMaxV) return fail(FLCE_ERR_UNSUPPORTED, "V_total larger than 2^30");
  if (v_offset < 0 || V_shard > V_total - v_offset)
    return fail(FLCE_ERR_INVALID_VALUE, "shard [%lld, %lld) does not lie in [0, V_total=%lld)",
                (long long)v_offset, (long long)(v_offset + V_shard), (long long)V_total);
  if (accumulate != 0 && accumulate != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "accumulate must be 0 or 1");
  st = check_backward_inputs(X, W_shard, targets, scale, lse, entropy, grad_logprob,
                             grad_entropy, dX_partial, dW_shard, workspace);
  if (st != FLCE_OK) return st;
  const BwdPlan P = plan_for_workspace(M, H, V_shard, false, workspace_bytes);
  if (P.chunk == 0)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL,
                "shard backward needs at least %zu workspace bytes, got %zu",
                bwd_min_bytes(M, H, V_shard, false), workspace_bytes);

  if (!grad_logprob && !grad_entropy) {
    hipError_t e = flce::launch_fill_zero_u16(static_cast<uint16_t*>(dW_shard),
                                              long(V_shard * H), stream);
    if (e == hipSuccess && !accumulate)
      e = flce::launch_fill_zero_u16(reinterpret_cast<uint16_t*>(dX_partial), long(2 * M * H),
                                     stream);
    if (e != hipSuccess) return hip_fail(e, "zero-fill kernel launch");
    return ok();
  }
  return backward_run(X, W_shard, targets, M, H, V_shard, v_offset, V_total, ignore_index,
                      scale, lse, entropy, grad_logprob, grad_entropy, nullptr, dX_partial,
                      accumulate == 1, dW_shard, static_cast<char*>(workspace), P, stream);
}

flce_status_t flce_nll_reduce(const float* logprob, const int64_t* targets, int64_t M,
                              int64_t V, int64_t ignore_index, double* out, hipStream_t stream) {
  if (!out || (M > 0 && (!logprob || !targets)))
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among logprob, targets, out");
  if (M < 0 || V <= 0)
    return fail(FLCE_ERR_INVALID_VALUE, "M must be >= 0 and V positive (got M=%lld V=%lld)",
                (long long)M, (long long)V);
  if (M > kMaxM || V > kMaxV)
    return fail(FLCE_ERR_UNSUPPORTED, "shape too large (limits M, V <= 2^30)");
  if (!aligned(logprob, 4) || !aligned(targets, 8) || !aligned(out, 8))
    return fail(FLCE_ERR_UNSUPPORTED, "logprob, targets and out must be naturally aligned");
  const hipError_t e = flce::launch_nll_reduce(logprob, targets, long(M), V, ignore_index, out,
                                               stream);
  if (e != hipSuccess) return hip_fail(e, "NLL reduction kernel launch");
  return ok();
}

flce_status_t flce_nll_mean_grad(const int64_t* targets, int64_t M, int64_t V,
                                 int64_t ignore_index, const double* reduced,
                                 float* grad_logprob, hipStream_t stream) {
  if (M < 0 || V <= 0)
    return fail(FLCE_ERR_INVALID_VALUE, "M must be >= 0 and V positive (got M=%lld V=%lld)",
                (long long)M, (long long)V);
  if (M == 0) return ok();
  if (!targets || !reduced || !grad_logprob)
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among targets, reduced, grad_logprob");
  if (M > kMaxM || V > kMaxV)
    return fail(FLCE_ERR_UNSUPPORTED, "shape too large (limits M, V <= 2^30)");
  if (!aligned(targets, 8) || !aligned(reduced, 8) || !aligned(grad_logprob, 4))
    return fail(FLCE_ERR_UNSUPPORTED, "targets, reduced and grad_logprob must be naturally aligned");
  const hipError_t e = flce::launch_nll_mean_grad(targets, long(M), V, ignore_index, reduced,
                                                  grad_logprob, stream);
  if (e != hipSuccess) return hip_fail(e, "NLL gradient kernel launch");
  return ok();
}

}  // extern "C"

namespace {
flce_status_t policy_args(const float* logprob, const float* old_logprob,
                          const float* advantages, const int64_t* targets, int64_t M, int64_t V,
                          int64_t ignore_index, double eps_low, double eps_high,
                          double denominator, flce::PolicyLossArgs* a) {
  if (M < 0 || V <= 0)
    return fail(FLCE_ERR_INVALID_VALUE, "M must be >= 0 and V positive (got M=%lld V=%lld)",
                (long long)M, (long long)V);
  if (M > kMaxM || V > kMaxV)
    return fail(FLCE_ERR_UNSUPPORTED, "shape too large (limits M, V <= 2^30)");
  if (M > 0 && (!logprob || !advantages || !targets))
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among logprob, advantages, targets");
  if (!std::isfinite(eps_low) || !std::isfinite(eps_high) || eps_low < 0.0 || eps_high < 0.0)
    return fail(FLCE_ERR_INVALID_VALUE, "eps_low and eps_high must be finite and >= 0");
  if (!std::isfinite(denominator))
    return fail(FLCE_ERR_INVALID_VALUE, "denominator is not finite");
  if (!aligned(logprob, 4) || !aligned(old_logprob, 4) || !aligned(advantages, 4) ||
      !aligned(targets, 8))
    return fail(FLCE_ERR_UNSUPPORTED, "logprob, old_logprob, advantages and targets must be "
                "naturally aligned");
  *a = flce::PolicyLossArgs{logprob, old_logprob, advantages, targets, long(M), V,
                            ignore_index, eps_low, eps_high, denominator};
  return FLCE_OK;
}
}  // namespace

extern "C" {

flce_status_t flce_policy_loss_reduce(const float* logprob, const float* old_logprob,
                                      const float* advantages, const int64_t* targets,
                                      int64_t M, int64_t V, int64_t ignore_index,
                                      double eps_low, double eps_high, double denominator,
                                      float* per_token_loss, uint8_t* is_clipped, double* out,
                                      hipStream_t stream) {
  flce::PolicyLossArgs a;
  flce_status_t st = policy_args(logprob, old_logprob, advantages, targets, M, V, ignore_index,
                                 eps_low, eps_high, denominator, &a);
  if (st != FLCE_OK) return st;
  if (!out || (M > 0 && !per_token_loss))
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among per_token_loss, out");
  if (!aligned(out, 8) || !aligned(per_token_loss, 4))
    return fail(FLCE_ERR_UNSUPPORTED, "per_token_loss and out must be naturally aligned");
  const hipError_t e = flce::launch_policy_loss_reduce(a, per_token_loss, is_clipped, out, stream);
  if (e != hipSuccess) return hip_fail(e, "policy loss reduction kernel launch");
  return ok();
}

flce_status_t flce_policy_loss_grad(const float* logprob, const float* old_logprob,
                                    const float* advantages, const int64_t* targets, int64_t M,
                                    int64_t V, int64_t ignore_index, double eps_low,
                                    double eps_high, double denominator, const double* reduced,
                                    float* grad_logprob, hipStream_t stream) {
  flce::PolicyLossArgs a;
  flce_status_t st = policy_args(logprob, old_logprob, advantages, targets, M, V, ignore_index,
                                 eps_low, eps_high, denominator, &a);
  if (st != FLCE_OK) return st;
  if (M == 0) return ok();
  if (!grad_logprob || (denominator <= 0.0 && !reduced))
    return fail(FLCE_ERR_INVALID_VALUE,
                "NULL pointer among grad_logprob, reduced (needed when denominator <= 0)");
  if (!aligned(grad_logprob, 4) || !aligned(reduced, 8))
    return fail(FLCE_ERR_UNSUPPORTED, "grad_logprob and reduced must be naturally aligned");
  const hipError_t e = flce::launch_policy_loss_grad(a, reduced, grad_logprob, stream);
  if (e != hipSuccess) return hip_fail(e, "policy loss gradient kernel launch");
  return ok();
}

}  // extern "C"
