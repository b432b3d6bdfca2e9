// Internal interface between the libflce host code (flce_api.cpp) and its HIP
// kernels (flce_kernels.hip).  Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

constexpr int kTile = 256;  // backward workgroup tile edge; row padding of every buffer
// Forward workgroup tile (rows of X x columns of W); kTile is a multiple of both.
constexpr int kFwdTileM = 256;
constexpr int kFwdTileN = 256;
static_assert(kTile % kFwdTileM == 0 && kTile % kFwdTileN == 0, "forward tiles pad to kTile");

// Launches above this many 256-thread workgroups exceed the dispatch packet's 32-bit
// grid size (in work-items).
constexpr int64_t kMaxWorkgroups = 0xFFFFFFFFLL / 256;

// Tail queues of a tile launch.  Workgroup b runs on XCD b % 8, and each XCD works
// through its own contiguous stream of tiles (the tile-coordinate comment in the
// kernel source).  The XCDs of one chip do not all run at the same speed, so the last
// `queue` tiles of every stream are handed out at run time: the stream's own
// workgroups take them in order from the front through that XCD's counter, and spare
// workgroups past the tiles let an XCD that has finished its stream take tiles from
// the back of another XCD's queue.  Counter x: low 32 bits count front claims, high 32
// bits back claims; a claim gets a tile iff front + back < queue before it, so each
// queued tile is taken exactly once.  The counters must be zero when the launch
// starts: a launch zeroes the counters (`clear`) of the launch after it on the stream.
struct TileQueue {
  unsigned long long* ctr;    // this launch's 8 counters (unused when queue == 0)
  unsigned long long* clear;  // 8 counters this launch sets to zero, or nullptr
  int queue;                  // queued tiles per XCD stream (set by the launcher)
};
constexpr size_t kQueueBytes = 256;  // workspace for two sets of 8 counters

// Queue tiles per XCD stream and spare workgroups of a launch of n tiles: about 4% of
// each stream queued and 2% more workgroups, each a whole number per compute unit
// (32 per XCD); none below 8 tiles per compute unit or past the dispatch limit.
struct QueueShape {
  int queue;
  int64_t spare;
};
inline QueueShape queue_shape(int64_t n) {
  const int64_t per = n >> 3;
  if (per < 256) return {0, 0};
  int64_t q = (per / 25 + 31) / 32 * 32;
  if (q > per) q = per;
  const int64_t spare = 8 * ((per / 50 + 31) / 32 * 32);
  if (n + spare > kMaxWorkgroups) return {0, 0};
  return {int(q), spare};
}

struct FwdTileArgs {
  const uint16_t* X;        // bf16 [M, H]
  const uint16_t* W;        // bf16 [V, H]: vocabulary rows v_off .. v_off + V - 1
  const int64_t* targets;   // [M], global vocabulary ids
  int M, H, V;
  int64_t v_off;            // global id of W's first row (0 when W is the whole vocabulary)
  int64_t ignore_index;
  float scale;
  int n_mt, n_vt;           // forward tiles along M and V
  int Mpad;                 // M rounded up to kTile: row stride of the partial arrays
  float* part_m;            // [n_vt, Mpad] tile row max of z
  float* part_s;            // [n_vt, Mpad] sum exp(z - m)
  float* part_u;            // [n_vt, Mpad] sum exp(z - m) (z - m)   (entropy only)
  float* zt;                // [Mpad] target logit (target_logit_kernel, rows W holds)
  TileQueue tq;             // the tile kernel's counters; target_logit_kernel zeroes them
};

// Vocabulary shards whose partials one merge combines (a single shard for an
// unsharded call).  Shard r covers global ids v_lo[r] .. v_lo[r + 1] - 1; its partial
// arrays (n_vt[r] tiles of Mpad floats each) start at float offsets part_m[r],
// part_s[r], part_u[r] (entropy only) and its target logits at zt[r], all relative
// to FwdMergeArgs::base.
constexpr int kMaxShards = 64;
struct ShardTable {
  int n;
  int64_t v_lo[kMaxShards + 1];
  int n_vt[kMaxShards];
  long part_m[kMaxShards], part_s[kMaxShards], part_u[kMaxShards], zt[kMaxShards];
};

struct FwdMergeArgs {
  const int64_t* targets;
  int M;
  int64_t ignore_index;
  int Mpad;
  const float* base;
  ShardTable sh;
  float* logprob;
  float* lse;
  float* entropy;
};
static_assert(sizeof(FwdMergeArgs) <= 4096, "merge arguments travel as kernel arguments");

struct DlogitsArgs {
  const uint16_t* X;
  const uint16_t* W;          // bf16 [V, H]: vocabulary rows v_off .. v_off + V - 1
  const int64_t* targets;     // global vocabulary ids
  int M, H, V;
  int64_t v_off;              // global id of W's first row
  int64_t V_total;            // a row is valid iff its target lies in [0, V_total)
  int64_t ignore_index;
  float scale;
  const float* lse;
  const float* entropy;       // needed iff grad_entropy != NULL
  const float* grad_logprob;  // NULL = 0
  const float* grad_entropy;  // NULL = 0
  int vbase;                  // first vocabulary column of the chunk
  int n_mt, n_vt;             // tiles along M and along the chunk
  uint16_t* dz;               // bf16 Mpad x ldz, tile-blocked: scale * dz of the chunk
  long ldz;
  TileQueue tq;
};

struct GemmDwArgs {
  const uint16_t* dz;   // bf16 Mpad x ldz, tile-blocked (256-row bands of 256 x 64 blocks)
  long ldz;
  const uint16_t* X;    // bf16 [M, H]: the token rows of dz
  uint16_t* dW;         // bf16 [V, H]
  float* acc;           // fp32 [V, H] accumulator across token waves (modes 1-3)
  int M, Mpad, H, V;
  int vbase;
  int chunk_cols;       // padded width of the chunk (multiple of 256)
  int n_i, n_h;         // tiles along the chunk and along H
  int mode;             // 0 write bf16, 1 write acc, 2 add to acc, 3 add and write bf16
  TileQueue tq;
};

struct GemmDxArgs {
  const uint16_t* dz;   // bf16 Mpad x ldz, tile-blocked (256-row bands of 256 x 64 blocks)
  long ldz;
  const uint16_t* W;    // bf16 [V, H]
  float* acc;           // fp32 [M, H] accumulator across chunks (modes 1-3)
  uint16_t* dX;         // bf16 [M, H]
  int M, H, V;
  int vbase;
  int kcols;            // padded width of the chunk (multiple of 256)
  int n_m, n_h;
  int mode;             // 0 write bf16, 1 write acc, 2 add to acc, 3 add and write bf16
};

// One launch of the pipelined backward: the dW and dX tiles of one step and the d-logit
// tiles of the next (a kind with no tiles has count 0).
struct PipeArgs {
  DlogitsArgs dl;
  GemmDwArgs dw;
  GemmDxArgs dx;
  int n_dl, n_dw, n_dx;   // tiles: dl.n_mt * dl.n_vt, dw.n_i * dw.n_h, dx.n_m * dx.n_h
};

// Clipped policy loss over per-token log-probs (see flce_policy_loss_reduce).
struct PolicyLossArgs {
  const float* logprob;      // [M]
  const float* old_logprob;  // [M] or nullptr (ratio 1)
  const float* advantages;   // [M]
  const int64_t* targets;    // [M]
  long M;
  int64_t V, ignore_index;
  double eps_low, eps_high;
  double denominator;        // > 0: the normaliser N; else the number of valid rows
};

// Device scratch of flce_forward_noalloc: a file-scope __device__ array in
// flce_kernels.hip, one copy per GPU, held until the process ends.
constexpr size_t kScratchBytes = size_t(32) << 20;
// Address of the current device's copy of that array (hipGetSymbolAddress).
hipError_t scratch_device_address(void** ptr);

hipError_t launch_fwd_tile(const FwdTileArgs& a, bool entropy, hipStream_t s);
hipError_t launch_target_logit(const FwdTileArgs& a, hipStream_t s);
hipError_t launch_fwd_merge(const FwdMergeArgs& a, bool entropy, hipStream_t s);
hipError_t launch_dlogits(const DlogitsArgs& a, bool entropy_grad, hipStream_t s);
hipError_t launch_gemm_dw(const GemmDwArgs& a, hipStream_t s);
hipError_t launch_bwd_pipe(const PipeArgs& a, bool entropy_grad, hipStream_t s);
hipError_t launch_gemm_dx(const GemmDxArgs& a, hipStream_t s);
hipError_t launch_fill_zero_u16(uint16_t* p, long n, hipStream_t s);
hipError_t launch_policy_loss_reduce(const PolicyLossArgs& a, float* per_token_loss,
                                     uint8_t* is_clipped, double* out, hipStream_t s);
hipError_t launch_policy_loss_grad(const PolicyLossArgs& a, const double* reduced, float* grad,
                                   hipStream_t s);
hipError_t launch_nll_reduce(const float* logprob, const int64_t* targets, long M, int64_t V,
                             int64_t ignore_index, double* out, hipStream_t s);
hipError_t launch_nll_mean_grad(const int64_t* targets, long M, int64_t V, int64_t ignore_index,
                                const double* reduced, float* grad, hipStream_t s);

}  // namespace flce
