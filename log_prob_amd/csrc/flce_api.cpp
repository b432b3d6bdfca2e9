// libflce C ABI: argument validation, workspace carve-up and the launch sequence.
// Every check runs on the host before the first HIP call, so a rejected call
// enqueues nothing and needs no device.
#include <hip/hip_runtime.h>

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
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;
constexpr size_t kAlign = 256;
// Preferred size of one d-logit chunk buffer: 2 GiB.
constexpr size_t kDzBudget = size_t(2) << 30;
// Widest d-logit chunk: keeps every byte offset the kernels form inside one
// 256-row tile of the chunk buffer below 2^30.
constexpr int64_t kMaxChunk = int64_t(1) << 21;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

flce_status_t check_shape(int64_t M, int64_t H, int64_t V) {
  if (M <= 0 || H <= 0 || V <= 0)
    return fail(FLCE_ERR_INVALID_VALUE, "M, H and V must be positive (got M=%lld H=%lld V=%lld)",
                (long long)M, (long long)H, (long long)V);
  if (M > kMaxM || V > kMaxV || H > kMaxH)
    return fail(FLCE_ERR_UNSUPPORTED, "shape too large (limits M, V <= 2^30, H <= 2^20)");
  if (H % 8 != 0)
    return fail(FLCE_ERR_UNSUPPORTED, "H must be a multiple of 8 (got %lld)", (long long)H);
  const int64_t n_mt = cdiv(M, kTile), n_vt = cdiv(V, kTile), n_ht = cdiv(H, kTile);
  if (cdiv(M, flce::kFwdTileM) * cdiv(V, flce::kFwdTileN) > kMaxGrid || n_mt * n_vt > kMaxGrid ||
      n_vt * n_ht > kMaxGrid)
    return fail(FLCE_ERR_UNSUPPORTED, "shape needs more than 2^31 - 1 workgroups");
  return FLCE_OK;
}

struct FwdLayout {
  int64_t n_mt, n_vt, Mpad;
  size_t off_m, off_s, off_u, off_zt, total;
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
  L.total = L.off_zt + align_up(size_t(L.Mpad) * sizeof(float));
  return L;
}

// Tallest wave (a multiple of 256 rows, at most Mpad) whose forward partials fit in
// `bytes`; 0 if not even one 256-row wave fits.
int64_t wave_rows_for_workspace(int64_t M, int64_t V, bool ent, size_t bytes) {
  const int64_t Mpad = cdiv(M, kTile) * kTile;
  if (fwd_layout(Mpad, V, ent).total <= bytes) return Mpad;
  int64_t lo = 0, hi = Mpad / kTile;  // in tiles: lo fits (or 0), hi does not
  while (hi - lo > 1) {
    const int64_t mid = (lo + hi) / 2;
    if (fwd_layout(mid * kTile, V, ent).total <= bytes) lo = mid; else hi = mid;
  }
  return lo * kTile;
}

size_t bwd_bytes_for_chunk(int64_t M, int64_t H, int64_t V, int64_t chunk) {
  const int64_t Mpad = cdiv(M, kTile) * kTile;
  const int64_t Vpad = cdiv(V, kTile) * kTile;
  size_t b = align_up(size_t(Mpad) * size_t(chunk) * 2);
  if (chunk < Vpad) b += align_up(size_t(M) * size_t(H) * sizeof(float));
  return b;
}

int64_t preferred_chunk(int64_t M, int64_t V) {
  const int64_t Mpad = cdiv(M, kTile) * kTile;
  const int64_t Vpad = cdiv(V, kTile) * kTile;
  int64_t c = int64_t(kDzBudget / (size_t(Mpad) * 2)) / kTile * kTile;
  if (c < kTile) c = kTile;
  if (c > kMaxChunk) c = kMaxChunk;
  return c < Vpad ? c : Vpad;
}

// Widest chunk (multiple of 256, at most Vpad) whose buffers fit in `bytes`; 0 if none.
int64_t chunk_for_workspace(int64_t M, int64_t H, int64_t V, size_t bytes) {
  const int64_t Mpad = cdiv(M, kTile) * kTile;
  const int64_t Vpad = cdiv(V, kTile) * kTile;
  if (Vpad <= kMaxChunk && bwd_bytes_for_chunk(M, H, V, Vpad) <= bytes) return Vpad;
  const size_t acc = align_up(size_t(M) * size_t(H) * sizeof(float));
  if (bytes <= acc) return 0;
  int64_t c = int64_t((bytes - acc) / (size_t(Mpad) * 2)) / kTile * kTile;
  if (c > kMaxChunk) c = kMaxChunk;
  while (c >= kTile && bwd_bytes_for_chunk(M, H, V, c) > bytes) c -= kTile;
  if (c >= Vpad) c = Vpad - kTile;
  return c >= kTile ? c : 0;
}

flce_status_t hip_fail(hipError_t e, const char* what) {
  return fail(FLCE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
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
  if (fwd_bytes) *fwd_bytes = fwd_layout(M, V, compute_entropy == 1).total;
  if (bwd_bytes) *bwd_bytes = bwd_bytes_for_chunk(M, H, V, preferred_chunk(M, V));
  return ok();
}

flce_status_t flce_forward_workspace_min(int64_t M, int64_t H, int64_t V, int compute_entropy,
                                         size_t* bytes) {
  if (compute_entropy != 0 && compute_entropy != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "compute_entropy must be 0 or 1");
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (!bytes) return fail(FLCE_ERR_INVALID_VALUE, "bytes is NULL");
  *bytes = fwd_layout(kTile, V, compute_entropy == 1).total;
  return ok();
}

flce_status_t flce_forward_wave_rows(int64_t M, int64_t H, int64_t V, int compute_entropy,
                                     size_t workspace_bytes, int64_t* rows) {
  if (compute_entropy != 0 && compute_entropy != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "compute_entropy must be 0 or 1");
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (!rows) return fail(FLCE_ERR_INVALID_VALUE, "rows is NULL");
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
  *bytes = bwd_bytes_for_chunk(M, H, V, kTile);
  return ok();
}

flce_status_t flce_backward_chunk_cols(int64_t M, int64_t H, int64_t V, size_t workspace_bytes,
                                       int64_t* chunk_cols) {
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (!chunk_cols) return fail(FLCE_ERR_INVALID_VALUE, "chunk_cols is NULL");
  const int64_t c = chunk_for_workspace(M, H, V, workspace_bytes);
  if (c == 0)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes is below the minimum %zu",
                workspace_bytes, bwd_bytes_for_chunk(M, H, V, kTile));
  *chunk_cols = c;
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
                            int64_t H, int64_t V, int64_t ignore_index, float scale, bool ent,
                            const FwdLayout& L, char* ws) {
  flce::FwdTileArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.W = static_cast<const uint16_t*>(W);
  a.targets = targets;
  a.M = int(M);
  a.H = int(H);
  a.V = int(V);
  a.ignore_index = ignore_index;
  a.scale = scale;
  a.n_mt = int(L.n_mt);
  a.n_vt = int(L.n_vt);
  a.Mpad = int(L.Mpad);
  a.part_m = reinterpret_cast<float*>(ws + L.off_m);
  a.part_s = reinterpret_cast<float*>(ws + L.off_s);
  a.part_u = ent ? reinterpret_cast<float*>(ws + L.off_u) : nullptr;
  a.zt = reinterpret_cast<float*>(ws + L.off_zt);
  return a;
}

flce::FwdMergeArgs merge_args(const int64_t* targets, int64_t M, int64_t V, int64_t ignore_index,
                              bool ent, float* logprob, float* lse, float* entropy,
                              const FwdLayout& L, const char* ws) {
  flce::FwdMergeArgs b{};
  b.targets = targets;
  b.M = int(M);
  b.V = int(V);
  b.ignore_index = ignore_index;
  b.n_vt = int(L.n_vt);
  b.Mpad = int(L.Mpad);
  b.part_m = reinterpret_cast<const float*>(ws + L.off_m);
  b.part_s = reinterpret_cast<const float*>(ws + L.off_s);
  b.part_u = ent ? reinterpret_cast<const float*>(ws + L.off_u) : nullptr;
  b.zt = reinterpret_cast<const float*>(ws + L.off_zt);
  b.logprob = logprob;
  b.lse = lse;
  b.entropy = ent ? entropy : nullptr;
  return b;
}

}  // namespace

flce_status_t flce_forward_partials(const void* X, const void* W, const int64_t* targets,
                                    int64_t M, int64_t H, int64_t V, int64_t ignore_index,
                                    float scale, int compute_entropy, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  if (!X || !W || !targets || !workspace)
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among X, W, targets, workspace");
  FwdLayout L;
  flce_status_t st =
      check_forward_common(targets, M, H, V, compute_entropy, workspace, workspace_bytes, &L);
  if (st != FLCE_OK) return st;
  st = check_forward_inputs(X, W, scale);
  if (st != FLCE_OK) return st;
  const bool ent = compute_entropy == 1;
  const flce::FwdTileArgs a = tile_args(X, W, targets, M, H, V, ignore_index, scale, ent, L,
                                        static_cast<char*>(workspace));
  const hipError_t e = flce::launch_fwd_tile(a, ent, stream);
  if (e != hipSuccess) return hip_fail(e, "forward tile kernel launch");
  return ok();
}

flce_status_t flce_forward_merge(const int64_t* targets, int64_t M, int64_t H, int64_t V,
                                 int64_t ignore_index, int compute_entropy, float* logprob,
                                 float* lse, float* entropy, const void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (!targets || !logprob || !lse || !workspace)
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among targets, logprob, lse, workspace");
  FwdLayout L;
  flce_status_t st =
      check_forward_common(targets, M, H, V, compute_entropy, workspace, workspace_bytes, &L);
  if (st != FLCE_OK) return st;
  st = check_forward_outputs(compute_entropy, logprob, lse, entropy);
  if (st != FLCE_OK) return st;
  const bool ent = compute_entropy == 1;
  const flce::FwdMergeArgs b = merge_args(targets, M, V, ignore_index, ent, logprob, lse, entropy,
                                          L, static_cast<const char*>(workspace));
  const hipError_t e = flce::launch_fwd_merge(b, ent, stream);
  if (e != hipSuccess) return hip_fail(e, "forward merge kernel launch");
  return ok();
}

flce_status_t flce_forward(const void* X, const void* W, const int64_t* targets, int64_t M,
                           int64_t H, int64_t V, int64_t ignore_index, float scale,
                           int compute_entropy, float* logprob, float* lse, float* entropy,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!X || !W || !targets || !logprob || !lse || !workspace)
    return fail(FLCE_ERR_INVALID_VALUE,
                "NULL pointer among X, W, targets, logprob, lse, workspace");
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
  if (compute_entropy != 0 && compute_entropy != 1)
    return fail(FLCE_ERR_INVALID_VALUE, "compute_entropy must be 0 or 1");
  if (!aligned(targets, 8)) return fail(FLCE_ERR_UNSUPPORTED, "targets must be 8-byte aligned");
  if (!aligned(workspace, kAlign))
    return fail(FLCE_ERR_UNSUPPORTED, "workspace must be 256-byte aligned");
  st = check_forward_inputs(X, W, scale);
  if (st != FLCE_OK) return st;
  st = check_forward_outputs(compute_entropy, logprob, lse, entropy);
  if (st != FLCE_OK) return st;
  const bool ent = compute_entropy == 1;
  // token waves: as many 256-row tiles per wave as the workspace holds partials for
  const int64_t rows = wave_rows_for_workspace(M, V, ent, workspace_bytes);
  if (rows == 0)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL, "forward needs at least %zu workspace bytes, got %zu",
                fwd_layout(kTile, V, ent).total, workspace_bytes);
  char* ws = static_cast<char*>(workspace);
  for (int64_t r0 = 0; r0 < M; r0 += rows) {
    const int64_t mw = M - r0 < rows ? M - r0 : rows;
    const FwdLayout L = fwd_layout(mw, V, ent);
    const flce::FwdTileArgs a =
        tile_args(static_cast<const uint16_t*>(X) + r0 * H, W, targets + r0, mw, H, V,
                  ignore_index, scale, ent, L, ws);
    hipError_t e = flce::launch_fwd_tile(a, ent, stream);
    if (e != hipSuccess) return hip_fail(e, "forward tile kernel launch");
    const flce::FwdMergeArgs b = merge_args(targets + r0, mw, V, ignore_index, ent, logprob + r0,
                                            lse + r0, ent ? entropy + r0 : nullptr, L, ws);
    e = flce::launch_fwd_merge(b, ent, stream);
    if (e != hipSuccess) return hip_fail(e, "forward merge kernel launch");
  }
  return ok();
}

flce_status_t flce_backward(const void* X, const void* W, const int64_t* targets, int64_t M,
                            int64_t H, int64_t V, int64_t ignore_index, float scale,
                            const float* lse, const float* entropy, const float* grad_logprob,
                            const float* grad_entropy, void* dX, void* dW, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!X || !W || !targets || !lse || !dX || !dW || !workspace)
    return fail(FLCE_ERR_INVALID_VALUE, "NULL pointer among X, W, targets, lse, dX, dW, workspace");
  flce_status_t st = check_shape(M, H, V);
  if (st != FLCE_OK) return st;
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
  const int64_t chunk = chunk_for_workspace(M, H, V, workspace_bytes);
  if (chunk == 0)
    return fail(FLCE_ERR_WORKSPACE_TOO_SMALL, "backward needs at least %zu workspace bytes, got %zu",
                bwd_bytes_for_chunk(M, H, V, kTile), workspace_bytes);

  if (!grad_logprob && !grad_entropy) {
    hipError_t e = flce::launch_fill_zero_u16(static_cast<uint16_t*>(dX), long(M * H), stream);
    if (e == hipSuccess)
      e = flce::launch_fill_zero_u16(static_cast<uint16_t*>(dW), long(V * H), stream);
    if (e != hipSuccess) return hip_fail(e, "zero-fill kernel launch");
    return ok();
  }

  const int64_t n_mt = cdiv(M, kTile), Mpad = n_mt * kTile;
  const int64_t Vpad = cdiv(V, kTile) * kTile;
  const int64_t n_chunks = cdiv(Vpad, chunk);
  char* ws = static_cast<char*>(workspace);
  uint16_t* dz = reinterpret_cast<uint16_t*>(ws);
  float* acc = n_chunks > 1
                   ? reinterpret_cast<float*>(ws + align_up(size_t(Mpad) * size_t(chunk) * 2))
                   : nullptr;
  const bool entgrad = grad_entropy != nullptr;
  for (int64_t c = 0; c < n_chunks; ++c) {
    const int64_t vbase = c * chunk;
    const int64_t kc = (Vpad - vbase) < chunk ? (Vpad - vbase) : chunk;

    flce::DlogitsArgs d{};
    d.X = static_cast<const uint16_t*>(X);
    d.W = static_cast<const uint16_t*>(W);
    d.targets = targets;
    d.M = int(M);
    d.H = int(H);
    d.V = int(V);
    d.ignore_index = ignore_index;
    d.scale = scale;
    d.lse = lse;
    d.entropy = entropy;
    d.grad_logprob = grad_logprob;
    d.grad_entropy = grad_entropy;
    d.vbase = int(vbase);
    d.n_mt = int(n_mt);
    d.n_vt = int(kc / kTile);
    d.dz = dz;
    d.ldz = long(chunk);
    hipError_t e = flce::launch_dlogits(d, entgrad, stream);
    if (e != hipSuccess) return hip_fail(e, "d-logits kernel launch");

    flce::GemmDwArgs w{};
    w.dz = dz;
    w.ldz = long(chunk);
    w.X = static_cast<const uint16_t*>(X);
    w.dW = static_cast<uint16_t*>(dW);
    w.M = int(M);
    w.Mpad = int(Mpad);
    w.H = int(H);
    w.V = int(V);
    w.vbase = int(vbase);
    w.chunk_cols = int(kc);
    w.n_i = int(kc / kTile);
    w.n_h = int(cdiv(H, kTile));
    e = flce::launch_gemm_dw(w, stream);
    if (e != hipSuccess) return hip_fail(e, "dW GEMM launch");

    flce::GemmDxArgs x{};
    x.dz = dz;
    x.ldz = long(chunk);
    x.W = static_cast<const uint16_t*>(W);
    x.acc = acc;
    x.dX = static_cast<uint16_t*>(dX);
    x.M = int(M);
    x.H = int(H);
    x.V = int(V);
    x.vbase = int(vbase);
    x.kcols = int(kc);
    x.n_m = int(n_mt);
    x.n_h = int(cdiv(H, kTile));
    x.mode = n_chunks == 1 ? 0 : (c == 0 ? 1 : (c == n_chunks - 1 ? 3 : 2));
    e = flce::launch_gemm_dx(x, stream);
    if (e != hipSuccess) return hip_fail(e, "dX GEMM launch");
  }
  return ok();
}

}  // extern "C"
