// HIP kernels of libflce for gfx950 (CDNA4): fused LM-head linear + cross-entropy.
//
// Forward (Liger-Kernel FSLCE commit, "Summary" and "Implementation / Forward";
// SkyRL PR 2141, "Overview"):
//   fwd_tile     one workgroup per (256-row M tile, 256-column V tile): bf16 MFMA
//                mainloop over H computing the tile transposed (vocabulary rows,
//                token columns), then an epilogue that reduces it to per-row partial
//                statistics (max m, sum of exp(z - m), and sum of exp(z - m) (z - m)
//                for entropy) down each lane's registers.
//   target_logit z[m, t[m]] as one dot product per row.
//   fwd_merge    combines the per-tile partials of each row (max first, then the
//                rescaled sums) into lse, logprob and entropy.
// Scalar reductions: nll_reduce (sum, count and mean of -logprob over valid rows) and
// nll_mean_grad (the mean NLL's gradient with respect to logprob); policy_loss_reduce
// and policy_loss_grad (a clipped policy-gradient loss on the log-probs, token-mean
// aggregated, and its gradient with respect to logprob).
// Backward (Liger-Kernel PR 1294, "Kernel design notes": recompute the logits
// tiles, emit d-logits in the input dtype into a reusable buffer, then two grad
// GEMMs; SkyRL PR 2141, "Overview": split backward over the vocabulary):
//   bwd_dlogits  the same mainloop on the same transposed tile, epilogue forms
//                scale * dz in bf16 for one vocabulary chunk, stored tile-blocked
//                (256 x 64 blocks).
//   gemm_dw      dW[chunk] = dz_chunk^T X          (K = tokens)
//   gemm_dx      dX (+)= dz_chunk W[chunk]          (K = chunk columns)
//
// Every kernel computes 256 x 256 output tiles with 4 waves of 128 x 128 and
// v_mfma_f32_32x32x16_bf16.  K is staged 64 at a time through double-buffered LDS
// (2 x 64 KiB) by direct-to-LDS buffer loads: no staging registers, and lanes whose
// 16 bytes lie outside the operand get an out-of-range offset, which the buffer
// unit turns into zeros.  An operand whose K dimension is contiguous in memory is
// kept in LDS as 128-byte K rows and read with ds_read_b128; an operand whose M/N
// dimension is contiguous is kept as 512-byte K rows and read with the gfx950
// transposing read ds_read_b64_tr_b16, which hands each lane 4 consecutive K values
// of one column.  Both layouts XOR-swizzle 16- or 32-byte blocks by row so the
// fragment reads are free of bank conflicts.  Kernels and the host code take a
// vocabulary offset, so the same kernels serve one shard of a split vocabulary.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <utility>

#include "flce_internal.h"

#define LDS_AS __attribute__((address_space(3)))

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int NTHREADS = 256;    // 4 waves of 64 in a 2 x 2 grid over the workgroup tile
// Pin the instruction order of a sub-step: the fragment reads of sub-step kk + 1
// alternate with the first MFMAs of sub-step kk, so each read is issued a whole
// sub-step before its first use.  Left to itself the scheduler reuses fragment
// registers right after their last MFMA and issues each read only one MFMA group
// ahead, exposing the LDS latency.
constexpr bool SCHED_PIPE = true;
// A stage's loads are issued in LOAD_GROUPS groups per MFMA sub-step (at most one
// group per MFMA), placed between the sub-step's MFMA groups: half of them under the
// last sub-step of the step before (right after the barrier that frees their stage),
// the others under sub-step 0.  Measured best: 16 groups and half early (8 groups
// tie; 4 or 12 early loads cost 1.5-3%).
constexpr int LOAD_GROUPS = 16;
constexpr uint32_t OOB_OFFSET = 0x80000000u;  // beyond every descriptor's num_records
constexpr uint32_t RSRC_WORD3 = 0x00020000u;  // raw buffer, 32-bit data format

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Shape of a workgroup's mainloop: a TM x TN output tile computed by 4 waves of
// (TM / 2) x (TN / 2), K staged BK at a time through NST LDS stages.  WAVES_PER_EU
// is the occupancy the register budget is sized for: 2 lets two workgroups share a
// CU, so one workgroup's barrier and load-issue stalls hide under the other's
// matrix work (their LDS footprints must then fit 160 KiB together).
template <int TM_, int TN_, int BK_, int NST_, int WAVES_PER_EU_, int WAVES_M_ = 2,
          int WAVES_N_ = 2>
struct Shape {
  static constexpr int TM = TM_, TN = TN_, BK = BK_, NST = NST_;
  static constexpr int WAVES_PER_EU = WAVES_PER_EU_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;  // wave grid over the tile
  static constexpr int NWAVES = WAVES_M * WAVES_N, NTHREADS = 64 * NWAVES;
  static constexpr int WM = TM / WAVES_M, WN = TN / WAVES_N;    // wave tile
  static constexpr int MB = WM / 32, NB = WN / 32;    // 32 x 32 MFMA blocks per wave
  static constexpr int KK = BK / 16;                  // MFMA sub-steps per stage
  static constexpr int A_BYTES = TM * BK * 2, B_BYTES = TN * BK * 2;
  static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  static constexpr int PIPE_BYTES = NST * STAGE_BYTES;
  static constexpr int DMA_A = A_BYTES / (1024 * NWAVES), DMA_B = B_BYTES / (1024 * NWAVES);  // 1 KiB loads per wave
  static constexpr int DMA_STAGE = DMA_A + DMA_B;
  static_assert(MB >= 2 && MB % 2 == 0 && NB >= 1, "wave tile");
  static_assert(BK == 32 || BK == 64, "K per stage");
  static_assert(A_BYTES % (1024 * NWAVES) == 0 && B_BYTES % (1024 * NWAVES) == 0,
                "whole loads per wave");
  static_assert(NST >= 2 && NST <= 4, "stages");
};
// One workgroup per CU: 256 x 256 tiles, waves of 128 x 128, 128 KiB of LDS stages.
using BigShape = Shape<256, 256, 64, 2, 1>;
// The forward runs BigShape.  Eight waves of 128 x 64 (two per SIMD, Shape<256, 256,
// 64, 2, 2, 2, 4>) hide more stalls but read 1.5x the LDS; with the lean K loop they
// measured 5% slower.
using FwdShape = BigShape;
static_assert(FwdShape::TM == kFwdTileM && FwdShape::TN == kFwdTileN, "host and kernel tile");
constexpr int FWD_GROUP_M = 2048 / kFwdTileM;  // forward tile rows per L2 group

// The backward kernels run BigShape; their epilogues stage a 256 x 256 bf16 output
// tile (128 KiB) in the LDS the pipeline used.
constexpr int TILE = BigShape::TM;
constexpr int LDS_OUT = 2 * TILE * TILE;
constexpr int LDS_BIG = BigShape::PIPE_BYTES > LDS_OUT ? BigShape::PIPE_BYTES : LDS_OUT;
static_assert(BigShape::TN == TILE, "backward tile");

// ---------------------------------------------------------------------------
// Tile coordinates.  Workgroups are handed to the 8 XCDs round robin, so id b runs
// on XCD b % 8.  Ids are renumbered so each XCD receives a contiguous range of
// logical ids, walked in groups of `group_m` tile rows (tile row fastest): the
// workgroups resident on one XCD then share a few operand tiles in its L2.
// Logical id L of a grid of n_m x n_n tiles -> tile (tm, tn): groups of `group_m` tile
// rows, tile row fastest within a group.
__device__ __forceinline__ void group_coords(int L, int n_m, int n_n, int group_m, int& tm,
                                             int& tn) {
  const int width = group_m * n_n;
  const int g = L / width;
  const int first = g * group_m;
  const int gm = min(n_m - first, group_m);
  const int inner = L - g * width;
  tm = first + inner % gm;
  tn = inner / gm;
}

__device__ __forceinline__ void tile_coords(int bid, int nblocks, int n_m, int n_n, int group_m,
                                            int& tm, int& tn) {
  const int per = nblocks >> 3;
  int L = bid;
  if (bid < (per << 3)) L = (bid & 7) * per + (bid >> 3);
  group_coords(L, n_m, n_n, group_m, tm, tn);
}

// Queued tiles left in a counter (negative once exhausted).
__device__ __forceinline__ long long queue_left(unsigned long long c, int q) {
  return (long long)q - (long long)(c & 0xffffffffull) - (long long)(c >> 32);
}

// Logical id of this workgroup's tile for a launch of n tiles plus spare workgroups,
// with the last tq.queue ids of each XCD's stream (the logical ids x * per ... of
// tile_coords) taken through the counters of TileQueue; -1 when the workgroup finds
// no tile.  Lane 0 of wave 0 claims: a workgroup of the stream first from the front of
// its own XCD's queue, then (a spare at once) from the back of the queue with the most
// tiles left, until every queue is empty (each pass either takes a tile or sees a
// counter that only grows, so the loop ends).
// The bounds on both counts keep every id in range whatever the counters hold.
// Workgroup 0 also zeroes tq.clear for a later launch.
__device__ __forceinline__ int tile_claim(int n, const TileQueue& tq) {
  const int bid = blockIdx.x;
  if (bid == 0 && threadIdx.x < 8 && tq.clear)
    __hip_atomic_store(&tq.clear[threadIdx.x], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int per = n >> 3, q = tq.queue, x = bid & 7;
  if (bid < (per << 3)) {
    if ((bid >> 3) < per - q) return x * per + (bid >> 3);
  } else if (bid < n) {
    return bid;
  }
  if (q == 0) return -1;
  __shared__ int claimed;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const unsigned long long uq = (unsigned long long)q;
    int L = -1;
    if (lane == 0 && bid < n) {
      const unsigned long long old = atomicAdd(&tq.ctr[x], 1ull);
      const unsigned long long f = old & 0xffffffffull, b = old >> 32;
      if (f < uq && b < uq - f) L = x * per + per - q + (int)f;
    }
    L = __shfl(L, 0);
    while (L < 0) {
      const long long left =
          lane < 8 ? queue_left(__hip_atomic_load(&tq.ctr[lane & 7], __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT), q)
                   : 0;
      int y = -1;
      long long most = 0;
      for (int j = 0; j < 8; ++j) {
        const long long r = __shfl(left, j);
        if (r > most) {
          most = r;
          y = j;
        }
      }
      if (y < 0) break;
      if (lane == 0) {
        const unsigned long long old = atomicAdd(&tq.ctr[y], 1ull << 32);
        const unsigned long long f = old & 0xffffffffull, b = old >> 32;
        if (b < uq && f < uq - b) L = y * per + per - 1 - (int)b;
      }
      L = __shfl(L, 0);
    }
    if (lane == 0) claimed = L;
  }
  __syncthreads();
  return claimed;
}

// ---------------------------------------------------------------------------
// One operand of the mainloop, as seen by a workgroup.
//  K-contiguous (KC): `base` is element (row 0 of the tile, k = 0) of a [rows][K]
//     matrix with leading dimension ld; `valid` rows of the tile exist.
//  M/N-contiguous (MN): `base` is element (k = 0, column 0 of the tile) of a
//     [K][cols] matrix with leading dimension ld; `valid` columns of the tile exist.
// `kvalid` is the K extent that exists.  `band` = 0 for a row-major matrix; otherwise
// the matrix is tile-blocked (the d-logit buffer): 256-row bands of `band` elements,
// each a row of 256 x 64 blocks (16384 elements, row r of a block at 64 r).  A KC
// operand then reads the rows of its band (base = the band's start, ld = 64) and moves
// one block per 64 K; an MN operand reads 64-column blocks of consecutive K rows
// (base = block 0 of band 0 of its columns).
constexpr int BLK_ROWS = 256, BLK_COLS = 64, BLK_ELEMS = BLK_ROWS * BLK_COLS;
static_assert(BigShape::BK == BLK_COLS && BigShape::TM == BLK_ROWS, "one block per K step");
struct TileSrc {
  const uint16_t* base;
  long ld;
  int valid;
  int kvalid;
  long band;
};

// LDS layout of a KC tile: rows of BK bf16 (BK / 8 chunks of 16 bytes); chunk c of
// row r sits at chunk position c ^ kc_swz(r).  The 16 rows one ds_read_b128 cycle
// serves land on 16 distinct 16-byte bank groups.
template <int CHUNKS>
__device__ __forceinline__ int kc_swz(int r) {
  return CHUNKS == 8 ? ((r ^ (r >> 3)) & 7) : ((r >> 2) & 3);
}

// LDS layout of an MN tile of `cols` columns: BK K rows of 2 cols bytes (cols / 16
// blocks of 32 bytes); block b of K row k sits at block position b ^ mn_swz(k).  Each
// half-wave of a transposing fragment read takes two adjacent blocks (2j, 2j + 1) of
// 4 consecutive K rows; mn_swz maps those 4 rows to {0, 2, 5, 7}, so the 8 (row,
// block) pairs fall on the 8 distinct 32-byte bank groups of the 256-byte bank row
// (with k & 7 as the swizzle they took only 4, a 2-way conflict on every read).
__device__ __forceinline__ int mn_swz(int k) { return ((k & 3) << 1) ^ ((k >> 1) & 1); }

// One 64-lane direct-to-LDS load: lane i's 16 bytes from byte offset voff of the
// buffer go to LDS address lds_addr + 16 i.  Issued as inline assembly so that the
// compiler does not treat the fragment reads of the other stages as dependent on
// it; the mainloop waits for these loads itself (s_waitcnt vmcnt) before the
// barrier that publishes a stage.
typedef int i32x4 __attribute__((ext_vector_type(4)));
template <int IMM>
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds_addr) {
  static_assert(IMM >= 0 && IMM < 4096, "buffer instruction offset range");
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen offset:%4 lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr), "i"(IMM)
               : "memory");
}

// The same without rewriting m0: the LDS destination is the m0 of the previous
// dma16 plus IMM (the immediate offset applies to the LDS address as well as to the
// global one, which the lane offsets pre-subtract).
template <int IMM>
__device__ __forceinline__ void dma16_same_m0(i32x4 rsrc, uint32_t voff, uint32_t soff) {
  static_assert(IMM >= 0 && IMM < 4096, "buffer instruction offset range");
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "i"(IMM)
               : "memory");
}

// Buffer descriptor with a fixed record count: every lane that must not load
// already carries an offset >= OOB_OFFSET, which the buffer unit turns into zeros.
__device__ __forceinline__ i32x4 make_rsrc_fixed(const void* base) {
  const unsigned long a = (unsigned long)base;
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(a & 0xffffffffu));
  r.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
  r.z = 0x7fffffff;
  r.w = (int)RSRC_WORD3;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr_of(const char* p) {
  return (uint32_t)(uintptr_t)(LDS_AS const char*)p;
}

// Direct-to-LDS loads of one ROWS x BK operand tile (ROWS rows of a KC operand, or
// ROWS columns of an MN operand).  The tile is filled by 4 waves x N loads; load j
// of wave w fills LDS bytes [(w N + j) KiB, + 1 KiB) of the tile, lane i the 16
// bytes at i * 16.  Each lane's byte offsets relative to the K step's base address
// do not change from step to step, so they are computed once, together with the K
// position of the lane's 16 bytes within the step (in 8-element chunks for KC, in
// K rows for MN, one byte per load).  A step keeps the loads whose K position lies
// below a uniform limit and turns the others into zero fills, without branches.
template <bool KC, int ROWS, int BK, int NWAVES = 4>
struct DmaPlan {
  static constexpr int N = ROWS * BK * 2 / (1024 * NWAVES);  // loads per wave
  static constexpr int CHUNKS = BK / 8;           // KC: 16-byte chunks per tile row
  static constexpr int GPR = ROWS / 8;            // MN: 16-byte granules per K row
  static constexpr int KPOS_MAX = KC ? CHUNKS : BK;
  uint32_t voff[N];
  int wave;
  i32x4 rsrc0;         // buffer descriptor of the tile's base (k = 0), wave-uniform
  uint32_t kc_bytes;   // KC: bytes per K element (2, or 512 in a blocked matrix)
  uint32_t row_bytes;  // MN: bytes per K row within a 256-row band
  uint32_t band_bytes; // MN: bytes per 256-row band

  __device__ __forceinline__ void init(const TileSrc& s, int wave_id) {
    wave = wave_id;
    rsrc0 = make_rsrc_fixed(s.base);
    const bool blk = s.band != 0;
    kc_bytes = blk ? 2u * BLK_ROWS : 2u;
    row_bytes = (uint32_t)__builtin_amdgcn_readfirstlane((int)(blk ? 2 * BLK_COLS : s.ld * 2));
    band_bytes = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(blk ? s.band * 2 : (long)BLK_ROWS * s.ld * 2));
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int G = (wave * N + j) * 64 + lane;  // 16-byte granule of the tile
      int a, b;
      if constexpr (KC) {
        a = G / CHUNKS;                          // tile row
        b = (G % CHUNKS) ^ kc_swz<CHUNKS>(a);    // 16-byte chunk of K in the row
      } else {
        a = G / GPR;                             // K row
        b = (G % GPR) ^ (mn_swz(a) << 1);        // 16-byte chunk of columns
      }
      const bool ok = KC ? a < s.valid : 8 * b < s.valid;
      // element offset in the step: a blocked MN row's 16-byte chunk b lies in block b / 8
      const long e = (!KC && blk) ? (long)(b >> 3) * BLK_ELEMS + (long)a * BLK_COLS + 8 * (b & 7)
                                  : (long)a * s.ld + 8 * b;
      // the load's immediate offset (1 KiB x (j % 4)) is added back by the hardware
      voff[j] = (ok ? (uint32_t)(e * 2) : OOB_OFFSET) - 1024u * (j & 3);
    }
  }

  // K position of load j's 16 bytes within a step (a 16-byte chunk of K for KC, a K row
  // for MN), recomputed rather than kept: it is needed only in the few steps that
  // reach past K, and registers live across the K loop are the scarcest
  __device__ __forceinline__ int kpos(int j) const {
    const int G = (wave * N + j) * 64 + (int)(threadIdx.x & 63);
    if constexpr (KC) {
      const int a = G / CHUNKS;
      return (G % CHUNKS) ^ kc_swz<CHUNKS>(a);
    } else {
      return G / GPR;
    }
  }

  // offset of load j in a step of which `lim` K positions exist
  __device__ __forceinline__ uint32_t off(int j, int lim) const {
    return kpos(j) < lim ? voff[j] : OOB_OFFSET - 1024u * (j & 3);
  }
};

// Per-step state of one operand's loads.  A K-contiguous tile keeps one buffer base
// for the whole K loop and moves with the scalar offset (k0 times 2 bytes, or 512 in a
// blocked matrix, stays below 2^31); an M/N-contiguous tile moves its base by k0 rows
// (k0 / 256 bands and k0 % 256 rows of a band).  `lim` (uniform) is the
// number of the step's K positions that exist: 0 for a step past the end of K, whose
// loads then only zero-fill a free stage.
struct TileDma {
  i32x4 rsrc;
  uint32_t soff;
  uint32_t lds0;  // LDS byte address of this wave's first 1 KiB block of the tile
  int lim;
};

// FAST: the step lies entirely inside K (no per-lane K check, `lim` unused).  The
// descriptor and offsets are derived from the plan with scalar arithmetic only.
template <bool FAST, bool KC, int ROWS, int BK, int NW>
__device__ __forceinline__ TileDma tile_dma(const TileSrc& s, const DmaPlan<KC, ROWS, BK, NW>& plan,
                                            int k0, bool active, const char* lds_tile) {
  TileDma d;
  d.rsrc = plan.rsrc0;
  if constexpr (KC) {
    d.soff = (uint32_t)k0 * plan.kc_bytes;
  } else {
    const uint64_t base = ((uint64_t)(uint32_t)plan.rsrc0.y << 32 | (uint32_t)plan.rsrc0.x) +
                          (uint64_t)(uint32_t)(k0 >> 8) * plan.band_bytes +
                          (uint64_t)(uint32_t)(k0 & 255) * plan.row_bytes;
    d.rsrc.x = (int)(uint32_t)base;
    d.rsrc.y = (int)((base >> 32) & 0xffffu);
    d.soff = 0u;
  }
  d.lds0 = lds_addr_of(lds_tile) + (uint32_t)(plan.wave * plan.N * 1024);
  if constexpr (FAST) {
    d.lim = KC ? plan.CHUNKS : BK;
  } else {
    const int rem = s.kvalid - k0;  // K extent left from k0 (a multiple of 8 for KC)
    d.lim = !active ? 0 : KC ? min(max((rem + 7) >> 3, 0), plan.CHUNKS) : min(max(rem, 0), BK);
  }
  return d;
}

// Load j of a tile.  m0 holds the LDS base of a group of 4 loads; `set_m0` rewrites
// it (required for the first load issued after any other code that may touch m0 is
// scheduled in between), the other loads of the group ride on the immediate offset.
template <bool FAST, bool KC, int ROWS, int BK, int NW>
__device__ __forceinline__ void tile_load(const TileDma& d, const DmaPlan<KC, ROWS, BK, NW>& plan, int j,
                                          bool set_m0) {
  const uint32_t v = FAST ? plan.voff[j] : plan.off(j, d.lim);
  const uint32_t m0 = d.lds0 + (uint32_t)(j & ~3) * 1024u;
  switch (j & 3) {
    case 0: dma16<0>(d.rsrc, v, d.soff, m0); break;
    case 1: if (set_m0) dma16<1024>(d.rsrc, v, d.soff, m0); else dma16_same_m0<1024>(d.rsrc, v, d.soff); break;
    case 2: if (set_m0) dma16<2048>(d.rsrc, v, d.soff, m0); else dma16_same_m0<2048>(d.rsrc, v, d.soff); break;
    default: if (set_m0) dma16<3072>(d.rsrc, v, d.soff, m0); else dma16_same_m0<3072>(d.rsrc, v, d.soff); break;
  }
}

// The loads of one whole stage: stage load j < DMA_A is load j of the A tile, the
// rest are the B tile's (B_FIRST: the other way round).  The first half of a stage's
// loads goes out early (right after a barrier), so the order decides which operand
// waits longer: issuing the L2-resident operand first measured faster (forward with W
// first: +3%; dW with X^T first: -0.4%; dX with W first: +0.3%).
template <class S, bool A_KC, bool B_KC, bool FAST = false, bool B_FIRST = false>
struct StageDma {
  using PA = DmaPlan<A_KC, S::TM, S::BK, S::NWAVES>;
  using PB = DmaPlan<B_KC, S::TN, S::BK, S::NWAVES>;
  TileDma a, b;
  const PA* pa;
  const PB* pb;
  // issue stage loads [j0, j1) back to back (B_FIRST: the B tile's loads come first)
  __device__ __forceinline__ void issue(int j0, int j1) const {
    constexpr int DF = B_FIRST ? S::DMA_B : S::DMA_A;  // loads of the first tile
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      if (j < DF) {
        if constexpr (B_FIRST) tile_load<FAST>(b, *pb, j, j == j0);
        else tile_load<FAST>(a, *pa, j, j == j0);
      } else {
        if constexpr (B_FIRST) tile_load<FAST>(a, *pa, j - DF, j == j0 || j == DF);
        else tile_load<FAST>(b, *pb, j - DF, j == j0 || j == DF);
      }
    }
  }
};

// Per-lane LDS byte offsets of the MFMA fragments a wave reads from one operand
// tile, for sub-step kk = 0; sub-step kk adds a constant (folded into the LDS
// instruction's immediate offset where the layout allows).
//  KC tile: fragment of rows idx0 + lane % 32, K chunk 2 kk + lane / 32 (ds_read_b128).
//  MN tile: the same fragment with two transposing reads; in each 16-lane group,
//  lane i reads 4 columns (4 (i % 4) .. + 3 of the group's 16) of K row i / 4 and
//  the read hands lane j of the group column j of those 4 K rows.
template <bool KC, int NBLK, int ROWS, int BK>
struct FragPlan {
  static constexpr int ROW_BYTES = KC ? BK * 2 : ROWS * 2;  // bytes per LDS row
  uint32_t off[NBLK][KC ? BK / 16 : 2];  // [block][kk] for KC, [block][half] for MN

  // region: LDS byte offset of the operand's stage-0 tile, folded into the offsets so
  // that a stage is selected by an instruction's immediate offset
  __device__ __forceinline__ void init(int idx_base, int lane, uint32_t region) {
#pragma unroll
    for (int blk = 0; blk < NBLK; ++blk) {
      const int idx0 = idx_base + 32 * blk;
      if constexpr (KC) {
        const int r = idx0 + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
          const int c = 2 * kk + (lane >> 5);
          off[blk][kk] = region + r * ROW_BYTES + ((c ^ kc_swz<BK / 8>(r)) << 4);
        }
      } else {
        const int g = lane >> 4, i = lane & 15;
        const int c0 = idx0 + 16 * (g & 1) + 4 * (i & 3);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int k = 8 * (g >> 1) + 4 * hh + (i >> 2);  // kk adds 16 rows: mn_swz unchanged
          off[blk][hh] = region + k * ROW_BYTES + (((c0 >> 4) ^ mn_swz(k)) << 5) + ((c0 & 15) << 1);
        }
      }
    }
  }

  __device__ __forceinline__ bf16x8 read(const char* tile, int blk, int kk) const {
    if constexpr (KC) {
      return *reinterpret_cast<const bf16x8*>(tile + off[blk][kk]);
    } else {
      const i16x4 h0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4*)(tile + off[blk][0] + kk * 16 * ROW_BYTES));
      const i16x4 h1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (LDS_AS i16x4*)(tile + off[blk][1] + kk * 16 * ROW_BYTES));
      const i16x8 v = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
      return __builtin_bit_cast(bf16x8, v);
    }
  }
};

template <class S, bool A_KC, bool B_KC>
struct Frags {
  FragPlan<A_KC, S::MB, S::TM, S::BK> a;
  FragPlan<B_KC, S::NB, S::TN, S::BK> b;
};

// The LDS tiles of one K step: A and B operand tiles.
struct StagePtr {
  const char* a;
  const char* b;
};

template <class S, bool A_KC, bool B_KC>
__device__ __forceinline__ void read_frags(bf16x8 (&af)[S::MB], bf16x8 (&bfr)[S::NB],
                                           StagePtr stage, const Frags<S, A_KC, B_KC>& f, int kk) {
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb) af[mb] = f.a.read(stage.a, mb, kk);
#pragma unroll
  for (int nb = 0; nb < S::NB; ++nb) bfr[nb] = f.b.read(stage.b, nb, kk);
}

template <int MB, int NB>
__device__ __forceinline__ void mfma_block(f32x16 (&acc)[MB][NB], const bf16x8 (&af)[MB],
                                           const bf16x8 (&bfr)[NB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
}

// s_waitcnt until at most n of this wave's vector-memory operations are outstanding
// (expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

// Fragment i of sub-step kk: i < MB is A block i, the others B block i - MB.
template <class S, bool A_KC, bool B_KC>
__device__ __forceinline__ void read_frag(bf16x8 (&af)[S::MB], bf16x8 (&bfr)[S::NB],
                                          StagePtr stage, const Frags<S, A_KC, B_KC>& f, int kk,
                                          int i) {
  if (i < S::MB)
    af[i] = f.a.read(stage.a, i, kk);
  else
    bfr[i - S::MB] = f.b.read(stage.b, i - S::MB, kk);
}

// LDS read instructions of fragments [i0, i1) (a transposing fragment takes two).
template <class S, bool A_KC, bool B_KC>
constexpr int frag_read_instrs(int i0, int i1) {
  int n = 0;
  for (int i = i0; i < i1; ++i) n += (i < S::MB ? A_KC : B_KC) ? 1 : 2;
  return n;
}

// Group g (of GROUPS) of one MFMA sub-step: a share of the fragment reads of
// sub-step RKK of the stage at `rstage` (the next sub-step), each paired with one
// of the group's MFMAs, the group's other MFMAs, then a share of the stage loads
// [JB, JE) of `dma`.  Scheduling fences keep the loads between the MFMA groups, so
// the matrix pipe never waits behind a long burst of load issue.
template <int RKK, int g, int GROUPS, int JB, int JE, class S, bool A_KC, bool B_KC, class Ops>
__device__ __forceinline__ void substep_group(f32x16 (&acc)[S::MB][S::NB],
                                              const bf16x8 (&af)[S::MB], const bf16x8 (&bfr)[S::NB],
                                              bf16x8 (&af_n)[S::MB], bf16x8 (&bfr_n)[S::NB],
                                              StagePtr rstage, const Frags<S, A_KC, B_KC>& f,
                                              Ops& dma) {
  constexpr int NF = S::MB + S::NB, F = S::MB * S::NB, D = JE - JB;
  constexpr int i0 = g * NF / GROUPS, i1 = (g + 1) * NF / GROUPS;
  constexpr int m0 = g * F / GROUPS, m1 = (g + 1) * F / GROUPS;
  constexpr int R = frag_read_instrs<S, A_KC, B_KC>(i0, i1);
  constexpr int P = R < m1 - m0 ? R : m1 - m0;
#pragma unroll
  for (int i = i0; i < i1; ++i) read_frag<S>(af_n, bfr_n, rstage, f, RKK, i);
#pragma unroll
  for (int m = m0; m < m1; ++m) {
    const int mb = m / S::NB, nb = m % S::NB;
    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
  }
  if constexpr (SCHED_PIPE) {
#pragma unroll
    for (int i = 0; i < P; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    if constexpr (m1 - m0 > P) __builtin_amdgcn_sched_group_barrier(0x008, m1 - m0 - P, 0);
    if constexpr (R > P) __builtin_amdgcn_sched_group_barrier(0x100, R - P, 0);
  }
  if constexpr (D > 0) {
    __builtin_amdgcn_sched_barrier(0);
    dma.issue(JB + g * D / GROUPS, JB + (g + 1) * D / GROUPS);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Sub-step kk (MFMAs on register set kk % 2) with the reads of sub-step RKK of
// `rstage` into the other set and stage loads [JB, JE) spread over GROUPS groups.
template <int kk, int RKK, int GROUPS, int JB, int JE, class S, bool A_KC, bool B_KC, class Ops,
          int... G>
__device__ __forceinline__ void substep_with_loads(f32x16 (&acc)[S::MB][S::NB],
                                                   bf16x8 (&af)[2][S::MB], bf16x8 (&bfr)[2][S::NB],
                                                   StagePtr rstage, const Frags<S, A_KC, B_KC>& f,
                                                   Ops& dma,
                                                   std::integer_sequence<int, G...>) {
  (substep_group<RKK, G, GROUPS, JB, JE, S>(acc, af[kk & 1], bfr[kk & 1], af[(kk + 1) & 1],
                                            bfr[(kk + 1) & 1], rstage, f, dma), ...);
}

// Pin the instruction order of one MFMA sub-step whose successor's fragments are
// read during it: (ds_read, MFMA) x P, then the remaining MFMAs or reads.  A
// transposing fragment takes two read instructions, so an M/N-contiguous operand
// doubles its share of the reads; left unpinned, the scheduler put the extra reads
// right before the MFMAs that use them, which then waited for all LDS reads.
template <class S, bool A_KC, bool B_KC, bool READS>
__device__ __forceinline__ void sched_substep() {
  constexpr int F = S::MB * S::NB;                                    // MFMAs per sub-step
  constexpr int R = frag_read_instrs<S, A_KC, B_KC>(0, S::MB + S::NB);  // read instructions
  constexpr int P = R < F ? R : F;                                    // reads paired with MFMAs
  if constexpr (SCHED_PIPE) {
    if constexpr (READS) {
#pragma unroll
      for (int i = 0; i < P; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      if constexpr (F > P) __builtin_amdgcn_sched_group_barrier(0x008, F - P, 0);
      if constexpr (R > P) __builtin_amdgcn_sched_group_barrier(0x100, R - P, 0);
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, F, 0);
    }
  }
}

// The MFMA mainloop shared by every kernel: D = A B^T over K for the workgroup's
// TM x TN tile, as 4 waves of WM x WN (wave w at rows WM (w / 2), columns
// WN (w % 2)).  acc[mb][nb] is the 32 x 32 block at (32 mb, 32 nb) of the wave
// tile in the v_mfma_f32_32x32x16 layout: lane l, element e holds row
// 8 (e / 4) + 4 (l / 32) + e % 4 and column l % 32.
//
// Pipeline: two LDS stages, laid out as A0, A1, B0, B1 (the B region's base is folded
// into the B fragment offsets, so every fragment read selects its stage with the
// instruction's immediate offset and the K loop, unrolled by two, issues no address
// arithmetic).  The KK MFMA sub-steps of stage kt run with the fragments of sub-step
// kk + 1 read (into the other register set) while the MFMAs of sub-step kk are
// issued.  Before the last sub-step the wave waits for its own loads of step kt + 1
// and the barrier publishes that stage and releases stage kt (all of whose reads
// have returned); the first fragments of step kt + 1 are then read under the last
// sub-step's MFMAs, so no step starts with an LDS-latency bubble.  The loads of step
// kt + 2 go out in groups between MFMA groups: the first EARLY of them under the last
// sub-step of step kt, right after the barrier freed their stage, the rest under
// sub-step 0 of step kt + 1.  Steps that lie entirely inside K take precomputed load
// offsets; the last steps check each lane's K position, and steps past K only
// zero-fill their stage, so every step issues the same number of loads and the wait
// before each barrier is a fixed count.  Steps run in pairs (stage 0, stage 1); an
// odd step count gets one step over a zero-filled stage.
template <class S, bool A_KC, bool B_KC, bool B_FIRST = false>
__device__ __forceinline__ void mainloop(f32x16 (&acc)[S::MB][S::NB], char* smem,
                                         const TileSrc& A, const TileSrc& B, int K) {
  static_assert(S::NST == 2, "two LDS stages");
  constexpr int KK = S::KK, D = S::DMA_STAGE;
  constexpr int EARLY = D / 2;
  constexpr int F = S::MB * S::NB, GR = LOAD_GROUPS < F ? LOAD_GROUPS : F;
  static_assert(EARLY > 0 && EARLY < 64, "early loads");
  static_assert(KK % 2 == 0, "sub-step 0 of every stage uses register set 0");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr0 = (wave / S::WAVES_N) * S::WM, wc0 = (wave % S::WAVES_N) * S::WN;
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < S::NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[mb][nb][e] = 0.f;

  const int nk = (K + S::BK - 1) / S::BK;
  // steps whose K range exists in both operands (an operand may hold fewer K rows than
  // the loop runs over, e.g. X's M rows against a K of M rounded up to 256)
  const int nfull = min(K, min(A.kvalid, B.kvalid)) / S::BK;
  typename StageDma<S, A_KC, B_KC>::PA plan_a;
  typename StageDma<S, A_KC, B_KC>::PB plan_b;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  plan_a.init(A, wave_u);
  plan_b.init(B, wave_u);
  Frags<S, A_KC, B_KC> frags;
  frags.a.init(wr0, lane, 0u);
  frags.b.init(wc0, lane, 2u * S::A_BYTES);
  // loads of step st into stage s; a step past K only zero-fills it
  auto stage_dma = [&](auto fast, int st, int s) {
    constexpr bool FAST = decltype(fast)::value;
    StageDma<S, A_KC, B_KC, FAST, B_FIRST> d;
    d.pa = &plan_a;
    d.pb = &plan_b;
    const bool active = st < nk;
    const int k0 = (active ? st : 0) * S::BK;
    d.a = tile_dma<FAST>(A, plan_a, k0, active, smem + s * S::A_BYTES);
    d.b = tile_dma<FAST>(B, plan_b, k0, active, smem + 2 * S::A_BYTES + s * S::B_BYTES);
    return d;
  };
  using Slow = std::integral_constant<bool, false>;
  using Fast = std::integral_constant<bool, true>;
  using Stage0 = std::integral_constant<int, 0>;
  using Stage1 = std::integral_constant<int, 1>;
  // prologue: step 0, and the early loads of step 1
  stage_dma(Slow(), 0, 0).issue(0, D);
  stage_dma(Slow(), 1, 1).issue(0, EARLY);
  wait_vmcnt<EARLY>();  // step 0 has landed
  __syncthreads();
  bf16x8 af[2][S::MB], bfr[2][S::NB];
  read_frags<S>(af[0], bfr[0], StagePtr{smem, smem}, frags, 0);
  constexpr auto groups = std::make_integer_sequence<int, GR>();
  // one K step computed from stage STG (kt % 2 == STG)
  auto step = [&](auto stg, auto fast, int kt) {
    constexpr int STG = decltype(stg)::value;
    const StagePtr cur{smem + STG * S::A_BYTES, smem + STG * S::B_BYTES};
    const StagePtr nxt{smem + (1 - STG) * S::A_BYTES, smem + (1 - STG) * S::B_BYTES};
    {
      auto dma = stage_dma(fast, kt + 1, 1 - STG);
      substep_with_loads<0, 1, GR, EARLY, D, S>(acc, af, bfr, cur, frags, dma, groups);
    }
#pragma unroll
    for (int kk = 1; kk < KK - 1; ++kk) {
      read_frags<S>(af[(kk + 1) & 1], bfr[(kk + 1) & 1], cur, frags, kk + 1);
      mfma_block<S::MB, S::NB>(acc, af[kk & 1], bfr[kk & 1]);
      sched_substep<S, A_KC, B_KC, true>();
    }
    // keep the barrier after every MFMA issued so far (the compiler would hoist it)
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();
    __syncthreads();
    // stage kt is free now: it receives step kt + 2 (after the last step this reads
    // a stale stage; the values are never used)
    {
      auto dma = stage_dma(fast, kt + 2, STG);
      substep_with_loads<KK - 1, 0, GR, 0, EARLY, S>(acc, af, bfr, nxt, frags, dma, groups);
    }
  };
  int kt = 0;
  // iteration kt loads steps kt + 1 and kt + 2: both inside K while kt + 2 < nfull
  for (; kt + 3 < nfull; kt += 2) {
    step(Stage0(), Fast(), kt);
    step(Stage1(), Fast(), kt + 1);
  }
  // the rest, also in pairs: with an odd step count the last step computes on a
  // zero-filled stage and adds exact zeros
  for (; kt < nk; kt += 2) {
    step(Stage0(), Slow(), kt);
    step(Stage1(), Slow(), kt + 1);
  }
  // the zero fills issued under the last steps must land before the caller reuses LDS
  wait_vmcnt<0>();
  __syncthreads();
}


// Row of the wave tile held by lane `lane` in element e of a 32 x 32 block.
__device__ __forceinline__ int acc_row(int lane, int e) {
  return ((e >> 2) << 3) + ((lane >> 5) << 2) + (e & 3);
}

// ---------------------------------------------------------------------------
// An accumulator value read from its accumulation register where it is used (for
// values used once: left to itself, the register allocator moves the tile between
// register files and reads some values several times).
__device__ __forceinline__ float acc_read(float a) {
  float r;
  asm("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(a));
  return r;
}

// v_max_f32 without the quieting of its inputs that fmaxf adds (the inputs are MFMA
// results or maxima of them, never signaling NaNs).
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// ---------------------------------------------------------------------------
// bf16 output tiles of the backward kernels are staged in LDS before 16-byte
// coalesced stores.  Staging layout of a 256 x 256 tile: row r at byte 512 r, its
// 16-byte chunk c (columns 8 c .. 8 c + 7) at chunk position c ^ out_swz(r).  The
// swizzle sends the four rows one pair write touches (r0, r0 + 1, r0 + 4, r0 + 5,
// r0 even within its group of 8) to four different 64-byte bank groups.  Each wave
// stages its own 128 x 128 block and stores it 32 rows (one block row mb) at a time,
// right after staging them: no other wave touches those bytes, so no workgroup
// barrier, and the stores overlap the staging of the next block row.  The stores carry
// the non-temporal hint: no tile re-reads what it writes, and the lines would
// otherwise displace operand tiles in L2 (backward -0.7% at H = 2048, neutral at 8192).
__device__ __forceinline__ int out_swz(int r) { return ((r & 1) | ((r >> 1) & 2)) << 2; }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Staging of values in the accumulator layout (element e of block (mb, nb) is row
// wr0 + 32 mb + acc_row(lane, e), column wc0 + 32 nb + lane % 32) as bf16 pairs.
// Lanes 2i and 2i + 1 hold adjacent columns of the same rows; a lane's rows r, r + 1
// (slots e = 4 q + jp, jp + 1 with jp in {0, 2}) are packed as one bf16x2 (row r
// low), exchanged with the partner lane by a DPP swap, and one byte permute keeps the
// even lane's row r (columns c, c + 1) and the odd lane's row r + 1 (c - 1, c); the
// conversion rounds to nearest even.  The rows a lane writes are r = wr0 + 32 mb +
// 8 q + 4 (lane / 32) + jp + (lane & 1), so out_swz(r) = 4 ((lane & 1) | 2 (lane /
// 32)) for all of them: one address per column block nb, and the row offsets
// 512 (32 mb + 8 q + jp) are immediates.
struct WaveStager {
  LDS_AS char* t3;
  uint32_t addr[4];
  uint32_t sel;  // v_perm_b32 byte selector: bytes 0-3 this lane's pair, 4-7 the partner's
  int wr0, wc0, lane;

  __device__ __forceinline__ void init(char* tile, int wr0_, int wc0_, int lane_) {
    wr0 = wr0_;
    wc0 = wc0_;
    lane = lane_;
    const int lc = lane & 31, hi = lane >> 5, odd = lane & 1;
    const int sw = odd | (hi << 1);
    t3 = (LDS_AS char*)tile;
    const uint32_t base =
        (uint32_t)((wr0 + 4 * hi + odd) * 512 + (wc0 >> 3) * 16 + (lc & 6) * 2);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) addr[nb] = base + (uint32_t)((((nb ^ sw) << 2) + (lc >> 3)) << 4);
    sel = odd ? 0x03020706u : 0x05040100u;
  }

  // v0, v1: this lane's values in slots e = 4 q + jp and 4 q + jp + 1 of block (mb, nb)
  __device__ __forceinline__ void put(int mb, int q, int jp, int nb, float v0, float v1) const {
    const f32x2 pr = {v0, v1};
    const uint32_t own = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
    const uint32_t partner = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)own, 0xB1, 0xf, 0xf, true);
    *(LDS_AS uint32_t*)(t3 + addr[nb] + (32 * mb + 8 * q + jp) * 512) =
        __builtin_amdgcn_perm(partner, own, sel);
  }

  // The 16 bytes of tile row r, chunk c (columns 8 c .. 8 c + 7).
  __device__ __forceinline__ u32x4 get(int r, int c) const {
    return *(LDS_AS const u32x4*)(t3 + r * 512 + ((c ^ out_swz(r)) << 4));
  }

  // Wait until this wave's staging writes are in LDS (its own reads follow).
  __device__ __forceinline__ void fence() const { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

  // Store the wave's staged rows of block row mb to rows [0, nrows) and columns
  // [0, ncols) of a row-major matrix (dst = the tile's element (0, 0), leading
  // dimension ld; ncols a multiple of 8): 4 rows of 256 bytes per instruction.
  __device__ __forceinline__ void store_rows(int mb, uint16_t* dst, long ld, int nrows,
                                             int ncols) const {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = wr0 + 32 * mb + 4 * it + (lane >> 4), c = (wc0 >> 3) + (lane & 15);
      const u32x4 v = get(r, c);
      if (r < nrows && 8 * c < ncols)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + (long)r * ld + 8 * c));
    }
  }
};

// A wave's 128 x 128 accumulator block rounded to bf16 and stored to rows [0, nrows)
// and columns [0, ncols) of a row-major matrix (dst = the tile's element (0, 0)).
__device__ __forceinline__ void store_acc_bf16(char* tile, const f32x16 (&acc)[4][4], int wr0,
                                               int wc0, int lane, uint16_t* dst, long ld,
                                               int nrows, int ncols) {
  WaveStager st;
  st.init(tile, wr0, wc0, lane);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int jp = 0; jp < 4; jp += 2)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          st.put(mb, q, jp, nb, acc_read(acc[mb][nb][4 * q + jp]),
                 acc_read(acc[mb][nb][4 * q + jp + 1]));
    st.fence();
    st.store_rows(mb, dst, ld, nrows, ncols);
  }
}

// ---------------------------------------------------------------------------
// Forward tile kernel.

// v_permlane32_swap_b32: the upper half-wave of a (lanes 32-63) trades places with the
// lower half-wave of b, so that afterwards a holds (own a | b of lane - 32) and b holds
// (a of lane + 32 | own b).  Issued as inline assembly because the compiler builtin
// hands back only the first register; the s_nop pads cover the VALU hazards around it.
__device__ __forceinline__ void swap32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}

// x and y each combined over lanes l and l ^ 32 in one swap: the result is that of x
// in the lower half-wave and that of y in the upper one.
template <class Op>
__device__ __forceinline__ float halves_reduce(float x, float y, Op op) {
  swap32(x, y);
  return op(x, y);
}

// max(m, sgn a, sgn b) with sgn = -1 under NEG, as one v_max3_f32 issued directly:
// fmaxf on values the compiler cannot prove to be quiet NaNs (here, MFMA results)
// costs one quieting v_max per input.  m is already a running maximum of sgn-scaled
// values, so only a and b take the negation modifier.
template <bool NEG>
__device__ __forceinline__ float max3_run(float m, float a, float b) {
  float r;
  if constexpr (NEG)
    asm("v_max3_f32 %0, %1, -%2, -%3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  else
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

// Per token column of the lane, the maximum of sgn * acc over the lane's 16 MB
// vocabulary rows (sgn = -1 if NEG; the maximum of z = scale * acc is |scale| times
// that of sgn(scale) * acc); rows at or past `vrows` of the wave tile are skipped when
// RAGGED.
template <bool NEG, bool RAGGED, class S>
__device__ __forceinline__ void lane_col_max(const f32x16 (&acc)[S::MB][S::NB], int lane,
                                             int vrows, float (&mx)[S::NB]) {
  constexpr float SKIP = NEG ? INFINITY : -INFINITY;  // what the maximum ignores
#pragma unroll
  for (int nb = 0; nb < S::NB; ++nb) mx[nb] = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const bool v0 = !RAGGED || 32 * mb + acc_row(lane, e) < vrows;
      const bool v1 = !RAGGED || 32 * mb + acc_row(lane, e + 1) < vrows;
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb)
        mx[nb] = max3_run<NEG>(mx[nb], v0 ? acc[mb][nb][e] : SKIP, v1 ? acc[mb][nb][e + 1] : SKIP);
    }
}

// Per token column of the lane, the shifted sums over its 16 MB vocabulary rows in
// log2 units: s = sum 2^d and u = sum 2^d d with d = c1 z - m2 (nm2 = -m2 per column).
template <bool ENT, bool RAGGED, class S>
__device__ __forceinline__ void lane_col_sums(const f32x16 (&acc)[S::MB][S::NB], int lane,
                                              int vrows, float c1, const float (&nm2)[S::NB],
                                              float (&sv)[S::NB], float (&uv)[S::NB]) {
#pragma unroll
  for (int nb = 0; nb < S::NB; ++nb) sv[nb] = uv[nb] = 0.f;
#pragma unroll
  for (int mb = 0; mb < S::MB; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bool valid = !RAGGED || 32 * mb + acc_row(lane, e) < vrows;
#pragma unroll
      for (int nb = 0; nb < S::NB; ++nb) {
        float d = fmaf(acc[mb][nb][e], c1, nm2[nb]);
        if constexpr (RAGGED) d = valid ? d : -INFINITY;
        const float pe = __builtin_amdgcn_exp2f(d);
        sv[nb] += pe;
        if constexpr (ENT) uv[nb] = fmaf(pe, RAGGED ? fmaxf(d, -3.0e38f) : d, uv[nb]);
      }
    }
}

// One workgroup per tile of TN tokens x TM vocabulary entries of the logits, computed
// transposed: z^T = W X^T, the MFMA rows being vocabulary entries and its columns
// tokens.  Per wave, lane l then holds, for each of its NB token columns 32 nb + l % 32,
// 16 MB vocabulary rows of the wave tile, so the maxima and sums over the vocabulary
// run down the lane's own registers, meet the other half-wave in one swap, and meet the
// other wave of the same tokens through LDS.  The maximum over the tile's TM entries is
// formed first, so both row halves sum against the same shift and their partials simply
// add; thread t < TN writes the partials of token t of the tile.
template <class S, bool ENT>
__global__ __launch_bounds__(S::NTHREADS, S::WAVES_PER_EU) void fwd_tile_kernel(FwdTileArgs p) {
  constexpr int TV = S::TM, TT = S::TN, NB = S::NB, WM = S::WM, WN = S::WN;
  constexpr int RP = S::WAVES_M;  // row parts: waves sharing the same tokens
  static_assert(NB % 2 == 0, "token columns pair up across the half-waves");
  __shared__ __attribute__((aligned(1024))) char smem[S::PIPE_BYTES];
  static_assert(3 * RP * TT * 4 <= S::PIPE_BYTES, "epilogue buffers");
  int mt, vt;
  {
    const int L = tile_claim(p.n_mt * p.n_vt, p.tq);
    if (L < 0) return;
    group_coords(L, p.n_mt, p.n_vt, FWD_GROUP_M, mt, vt);
  }
  const int row0 = mt * TT, col0 = vt * TV;  // first token, first vocabulary entry
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform

  f32x16 acc[S::MB][NB];
  const TileSrc A{p.W + (long)col0 * p.H, p.H, p.V - col0, p.H, 0};
  const TileSrc B{p.X + (long)row0 * p.H, p.H, p.M - row0, p.H, 0};
  mainloop<S, true, true, true>(acc, smem, A, B, p.H);  // X (L2-resident) loads first
  // (the mainloop ends with a barrier: the LDS is free)

  const int wm = wave / S::WAVES_N;
  const int wv0 = wm * WM, wt0 = (wave % S::WAVES_N) * WN;
  const int lc = lane & 31, hi = lane >> 5;
  const float c1 = p.scale * LOG2E;  // logits in log2 units: z2 = c1 acc
  const float ac1 = fabsf(c1);
  const bool ragged = col0 + TV > p.V;
  const int vrows = p.V - col0 - wv0;  // vocabulary rows of the wave tile that exist

  // epilogue LDS: token maxima per row part [RP][TT], sums [RP][2][TT]
  float* red = reinterpret_cast<float*>(smem);
  float* comb = red + RP * TT;

  // maxima of sgn(c1) z over the wave's vocabulary rows: lane, then half-wave (token
  // columns 2 j + hi of the lane come out in half hi), then the row parts via LDS
  {
    float mx[NB];
    if (!ragged) {
      if (c1 >= 0.f) lane_col_max<false, false, S>(acc, lane, vrows, mx);
      else lane_col_max<true, false, S>(acc, lane, vrows, mx);
    } else {
      if (c1 >= 0.f) lane_col_max<false, true, S>(acc, lane, vrows, mx);
      else lane_col_max<true, true, S>(acc, lane, vrows, mx);
    }
#pragma unroll
    for (int j = 0; j < NB / 2; ++j)
      red[wm * TT + wt0 + 32 * (2 * j + hi) + lc] =
          halves_reduce(mx[2 * j], mx[2 * j + 1], [](float a, float b) { return max_raw(a, b); });
  }
  __syncthreads();

  // shifted sums against the tile maximum of each token column
  {
    float nm2[NB], sv[NB], uv[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float m = red[wt0 + 32 * nb + lc];
#pragma unroll
      for (int rp = 1; rp < RP; ++rp) m = fmaxf(m, red[rp * TT + wt0 + 32 * nb + lc]);
      nm2[nb] = -ac1 * m;
    }
    if (!ragged)
      lane_col_sums<ENT, false, S>(acc, lane, vrows, c1, nm2, sv, uv);
    else
      lane_col_sums<ENT, true, S>(acc, lane, vrows, c1, nm2, sv, uv);
#pragma unroll
    for (int j = 0; j < NB / 2; ++j) {
      const int t = wt0 + 32 * (2 * j + hi) + lc;
      comb[(2 * wm) * TT + t] =
          halves_reduce(sv[2 * j], sv[2 * j + 1], [](float a, float b) { return a + b; });
      if constexpr (ENT)
        comb[(2 * wm + 1) * TT + t] =
            halves_reduce(uv[2 * j], uv[2 * j + 1], [](float a, float b) { return a + b; });
    }
  }
  __syncthreads();
  if (tid < TT) {
    float mx = red[tid], sm = comb[tid], um = comb[TT + tid];
#pragma unroll
    for (int rp = 1; rp < RP; ++rp) {
      mx = fmaxf(mx, red[rp * TT + tid]);
      sm += comb[(2 * rp) * TT + tid];
      if constexpr (ENT) um += comb[(2 * rp + 1) * TT + tid];
    }
    const long off = (long)vt * p.Mpad + row0 + tid;
    p.part_m[off] = ac1 * mx * LN2;
    p.part_s[off] = sm;
    if constexpr (ENT) p.part_u[off] = um * LN2;
  }
}

// Target logit of every row whose target W holds: z[m, t[m]] = scale * X[m] . W[t[m] -
// v_off], bf16 products accumulated in fp32 in a fixed order (each lane over a strided
// set of 8-element groups, then a fixed butterfly over the wave).  A separate pass
// rather than a pick in the tile epilogue: the pick would have to run in every wave
// of every tile (a tile that picks only where a target lies costs more than the others
// and breaks the lockstep of an XCD's tiles), which took a quarter of the epilogue.
// One wave per row.
constexpr int TL_ROWS = 4;
__global__ __launch_bounds__(64 * TL_ROWS) void target_logit_kernel(FwdTileArgs p) {
  // zero the tile kernel's queue counters: that kernel is launched after this one
  if (blockIdx.x == 0 && threadIdx.x < 8 && p.tq.ctr)
    __hip_atomic_store(&p.tq.ctr[threadIdx.x], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * TL_ROWS + (threadIdx.x >> 6);
  if (row >= p.M) return;
  const int64_t t = p.targets[row];
  const int64_t tw = t - p.v_off;
  if (t == p.ignore_index || tw < 0 || tw >= p.V) return;
  const uint16_t* x = p.X + row * p.H;
  const uint16_t* w = p.W + tw * p.H;
  float s = 0.f;
#pragma unroll 4
  for (int k = 8 * lane; k < p.H; k += 8 * 64) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(x + k);
    const u32x4 wv = *reinterpret_cast<const u32x4*>(w + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = fmaf(__uint_as_float(xv[i] << 16), __uint_as_float(wv[i] << 16), s);
      s = fmaf(__uint_as_float(xv[i] & 0xffff0000u), __uint_as_float(wv[i] & 0xffff0000u), s);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (lane == 0) p.zt[row] = s * p.scale;
}

// Merge of the per-tile partials of each row: m* = max m_j, S = sum s_j e^(m_j - m*),
// U = sum e^(m_j - m*) (u_j + (m_j - m*) s_j); lse = m* + log S,
// logprob = min(z_t - lse, 0), entropy = max(log S - U / S, 0).
// The tiles j run over every shard of the table in order (one shard when the
// vocabulary is not split); the target logit comes from the shard that owns the target.
// A workgroup takes MERGE_ROWS rows; its MERGE_SLICES slices split each row's tiles
// (32 lanes read consecutive rows of one tile, so every load is a 128-byte line) and
// combine their maxima, then their sums, through LDS.  32 rows x 16 slices measured
// faster than 64 x 8 (fewer tiles per thread, twice the workgroups: 35 -> 22 us at
// M = H = 8192, V = 131072) and than 16 x 32 (64-byte pieces).
constexpr int MERGE_ROWS = 32, MERGE_SLICES = 16;
template <bool ENT>
__global__ __launch_bounds__(MERGE_ROWS * MERGE_SLICES) void fwd_merge_kernel(FwdMergeArgs p) {
  __shared__ float sm[3][MERGE_SLICES][MERGE_ROWS];
  const int lr = threadIdx.x % MERGE_ROWS, sl = threadIdx.x / MERGE_ROWS;
  const int row = blockIdx.x * MERGE_ROWS + lr;
  const bool live = row < p.M;
  float m = -INFINITY;
  if (live)
    for (int r = 0; r < p.sh.n; ++r) {
      const float* pm = p.base + p.sh.part_m[r] + row;
      for (int j = sl; j < p.sh.n_vt[r]; j += MERGE_SLICES) m = fmaxf(m, pm[(long)j * p.Mpad]);
    }
  sm[0][sl][lr] = m;
  __syncthreads();
  float ms = -INFINITY;
#pragma unroll
  for (int k = 0; k < MERGE_SLICES; ++k) ms = fmaxf(ms, sm[0][k][lr]);
  float S = 0.f, U = 0.f;
  if (live)
    for (int r = 0; r < p.sh.n; ++r) {
      const float* pm = p.base + p.sh.part_m[r] + row;
      const float* ps = p.base + p.sh.part_s[r] + row;
      const float* pu = p.base + p.sh.part_u[r] + row;
      for (int j = sl; j < p.sh.n_vt[r]; j += MERGE_SLICES) {
        const long off = (long)j * p.Mpad;
        const float dm = pm[off] - ms;
        const float a = __expf(dm);
        const float s = ps[off];
        S += s * a;
        if constexpr (ENT) U += a * (pu[off] + dm * s);
      }
    }
  sm[1][sl][lr] = S;
  sm[2][sl][lr] = U;
  __syncthreads();
  if (sl != 0 || !live) return;
  S = 0.f;
  U = 0.f;
#pragma unroll
  for (int k = 0; k < MERGE_SLICES; ++k) {
    S += sm[1][k][lr];
    if constexpr (ENT) U += sm[2][k][lr];
  }
  const float logS = logf(S);
  const int64_t t = p.targets[row];
  const bool valid = t != p.ignore_index && t >= 0 && t < p.sh.v_lo[p.sh.n];
  float zt = 0.f;
  if (valid) {
    int r = 0;
    while (r + 1 < p.sh.n && t >= p.sh.v_lo[r + 1]) ++r;
    zt = p.base[p.sh.zt[r] + row];
  }
  p.lse[row] = ms + logS;
  // A log-probability is at most 0 and an entropy at least 0.  When one logit holds
  // nearly all of a row's probability both values sit next to that bound, and fp32
  // rounding can put them a few ulps past it: the target logit (its own dot product)
  // and lse (from the MFMA accumulators) round differently, and the shifted sum of the
  // row's maximum element can come out a hair above 0.  The bounds are applied
  // exactly, which only moves a value towards the true one.
  p.logprob[row] = valid ? fminf(zt - (ms + logS), 0.f) : 0.f;
  if constexpr (ENT) p.entropy[row] = valid ? fmaxf(logS - U / S, 0.f) : 0.f;
}

// ---------------------------------------------------------------------------
// Staging of a d-logit tile computed transposed (vocabulary rows, token columns in the
// accumulators) for the tile-blocked buffer: token row r of the 256 x 256 bf16 tile at
// byte 512 r, its 16-byte chunk c (vocabulary columns 8 c .. 8 c + 7) at chunk
// position c ^ tswz(r).  A staging write puts 4 consecutive vocabulary entries of 32
// consecutive token rows, all in one chunk, and tswz is a bijection of r % 32, so the
// 64 lanes' 8-byte pieces fill 32 distinct chunk positions; a store read takes 8
// consecutive chunks of 4 consecutive rows per 32 lanes, which tswz (r % 4 in its top
// bits) sends to 4 distinct groups of 8 positions.  Both are free of bank conflicts
// (128 banks), and each wave's bytes are its own.
__device__ __forceinline__ int tswz(int r) { return ((r & 3) << 3) | ((r >> 2) & 7); }

struct DzStager {
  LDS_AS char* t3;
  uint32_t row[4];  // byte offset of token row wt0 + 32 nb + lane % 32
  int sw[4];
  int wt0, wv0, lane;

  __device__ __forceinline__ void init(char* tile, int wt0_, int wv0_, int lane_) {
    wt0 = wt0_;
    wv0 = wv0_;
    lane = lane_;
    t3 = (LDS_AS char*)tile;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int r = wt0 + 32 * nb + (lane & 31);
      row[nb] = (uint32_t)r * 512u + (uint32_t)(lane >> 5) * 8u;
      sw[nb] = tswz(r);
    }
  }

  // vocabulary rows wv0 + 32 mb + 8 q + 4 (lane / 32) + 0..3 of token column nb
  __device__ __forceinline__ void put(int nb, int mb, int q, const float (&d)[4]) const {
    const int c = (wv0 >> 3) + 4 * mb + q;
    const f32x2 p0 = {d[0], d[1]}, p1 = {d[2], d[3]};
    const u32x2 v = {__builtin_bit_cast(uint32_t, __builtin_convertvector(p0, bf16x2)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(p1, bf16x2))};
    *(LDS_AS u32x2*)(t3 + row[nb] + ((c ^ sw[nb]) << 4)) = v;
  }

  // Wait until this wave's staging writes are in LDS (its own reads follow).
  __device__ __forceinline__ void fence() const { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

  // Store the wave's staged token rows of block nb (32 rows, its 128 vocabulary
  // columns) to the tile-blocked buffer (dst = the tile's 256 x 64 block 0, block q at
  // dst + q BLK_ELEMS, row r at 64 r): two pieces of 32 consecutive rows, 1 KiB per
  // instruction.
  __device__ __forceinline__ void store_blocked(int nb, uint16_t* dst) const {
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int qb = it >> 2, r = wt0 + 32 * nb + 8 * (it & 3) + (lane >> 3), c8 = lane & 7;
      const int c = (wv0 >> 3) + 8 * qb + c8;
      const u32x4 v = *(LDS_AS const u32x4*)(t3 + r * 512 + ((c ^ tswz(r)) << 4));
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4*>(dst + (long)((wv0 >> 6) + qb) * BLK_ELEMS + r * BLK_COLS + 8 * c8));
    }
  }
};

// A wave's d-logits, d = 2^(c1 acc - lse2) (c0 + cb acc) + [row = target] sa with the
// per-token parameters of its 4 token columns (from LDS, see bwd_dlogits_kernel),
// rounded to bf16, staged in the wave's own part of the LDS tile and stored to the
// tile-blocked buffer at dst (the tile's 256 x 64 block 0) 32 token rows at a time.
// RAGGED: vocabulary rows at or past `vrows` of the wave tile become 0.  Every wave
// runs the same instruction stream whether or not it holds a target (the correction is
// a branch per four vocabulary rows that almost never has active lanes), which keeps
// the tiles of an XCD in step.
template <bool ENTGRAD, bool RAGGED>
__device__ __forceinline__ void stage_dlogits(char* tile, const f32x16 (&acc)[4][4],
                                              const float* r_lse2, const float* r_c0,
                                              const float* r_cb, const float* r_sa,
                                              const int* t_local, int wv0, int wt0, int lane,
                                              float c1, int vrows, uint16_t* dst) {
  const int lc = lane & 31, hi = lane >> 5;
  float L[4], C0[4], CB[4], SA[4];
  int T[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int t = wt0 + 32 * nb + lc;
    L[nb] = r_lse2[t];
    C0[nb] = r_c0[t];
    CB[nb] = ENTGRAD ? r_cb[t] : 0.f;
    SA[nb] = r_sa[t];
    T[nb] = t_local[t] - wv0 - 4 * hi;  // the target's row among the lane's, if any
  }
  DzStager st;
  st.init(tile, wt0, wv0, lane);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float av = acc_read(acc[mb][nb][4 * q + j]);
          const float pr = __builtin_amdgcn_exp2f(fmaf(av, c1, -L[nb]));
          float v = pr * (ENTGRAD ? fmaf(CB[nb], av, C0[nb]) : C0[nb]);
          if constexpr (RAGGED) v = 32 * mb + 8 * q + 4 * hi + j < vrows ? v : 0.f;
          d[j] = v;
        }
        const int dd = T[nb] - 32 * mb - 8 * q;
        if ((unsigned)dd < 4u) {
#pragma unroll
          for (int j = 0; j < 4; ++j) d[j] += dd == j ? SA[nb] : 0.f;
        }
        st.put(nb, mb, q, d);
      }
    st.fence();
    st.store_blocked(nb, dst);
  }
}

// Backward d-logits for one vocabulary chunk: dzs = scale * dz in bf16, written to
// an Mpad x ldz tile-blocked buffer (chunk column j = vocabulary column vbase + j;
// 256-row bands of 256 x 64 blocks, so that the GEMMs that read it take contiguous
// 32 KiB blocks instead of 128-byte pieces of 256 KiB-apart rows).  Columns past
// V and rows past M are written as zero.  With p = 2^(c1 acc - lse2) (c1 = scale log2 e)
// and per-row a = grad_logprob, b = grad_entropy, E = lse - entropy (all 0 on ignored
// rows):  scale dz = scale (a ([v = t] - p) + b p (E - scale acc))
//                  = p (c0 + cb acc) + [v = t] sa,
// c0 = scale (b E - a), cb = -scale^2 b, sa = scale a.
// LDS of the d-logit tile: the pipeline, then the bf16 output tile and the per-row arrays
constexpr int LDS_DLOGITS = BigShape::PIPE_BYTES > LDS_OUT + 5 * TILE * 4
                                ? BigShape::PIPE_BYTES
                                : LDS_OUT + 5 * TILE * 4;

template <bool ENTGRAD>
__device__ __forceinline__ void dlogits_tile(const DlogitsArgs& p, int mt, int vt, char* smem) {
  const int row0 = mt * TILE, ccol0 = vt * TILE, col0 = p.vbase + ccol0;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  // row tid's parameters, kept in registers over the mainloop (which may need all of
  // the LDS) and published through LDS after it
  float lse2 = 0.f, c0 = 0.f, cb = 0.f, sa = 0.f;
  int tl = -1;
  {
    const int r = row0 + tid;
    if (r < p.M) {
      // all of the row's loads go out together (validity selects afterwards, so no
      // load waits for the target's): one round trip, under the mainloop's first loads
      const int64_t t = p.targets[r];
      const float lse = p.lse[r];
      const float a = p.grad_logprob ? p.grad_logprob[r] : 0.f;
      float b = 0.f, ent = 0.f;
      if constexpr (ENTGRAD) {
        b = p.grad_entropy[r];
        ent = p.entropy[r];
      }
      const bool valid = t != p.ignore_index && t >= 0 && t < p.V_total;
      const int64_t tw = t - p.v_off;  // target as a row of W (owned iff 0 <= tw < V)
      lse2 = lse * LOG2E;
      const float sa_r = p.scale * a;
      const float c0_r = ENTGRAD ? p.scale * (b * (lse - ent) - a) : -sa_r;
      const float cb_r = ENTGRAD ? -p.scale * p.scale * b : 0.f;
      sa = valid ? sa_r : 0.f;
      c0 = valid ? c0_r : 0.f;
      cb = valid ? cb_r : 0.f;
      tl = (valid && tw >= col0 && tw < col0 + TILE && tw < p.V) ? (int)(tw - col0) : -1;
    }
  }

  // the tile computed transposed: vocabulary rows (A = W), token columns (B = X, whose
  // loads go first in each stage)
  f32x16 acc[4][4];
  const TileSrc A{p.W + (long)col0 * p.H, p.H, p.V - col0, p.H, 0};
  const TileSrc B{p.X + (long)row0 * p.H, p.H, p.M - row0, p.H, 0};
  mainloop<BigShape, true, true, true>(acc, smem, A, B, p.H);

  float* r_lse2 = reinterpret_cast<float*>(smem + LDS_OUT);
  float* r_c0 = r_lse2 + TILE;
  float* r_cb = r_c0 + TILE;
  float* r_sa = r_cb + TILE;
  int* t_local = reinterpret_cast<int*>(r_sa + TILE);
  r_lse2[tid] = lse2;
  r_c0[tid] = c0;
  if constexpr (ENTGRAD) r_cb[tid] = cb;
  r_sa[tid] = sa;
  t_local[tid] = tl;
  __syncthreads();

  const int wv0 = (wave >> 1) * 128, wt0 = (wave & 1) * 128;
  const float c1 = p.scale * LOG2E;
  const bool ragged = col0 + TILE > p.V;
  const int vrows = p.V - col0 - wv0;  // vocabulary rows of the wave tile that exist
  uint16_t* const dst = p.dz + (long)mt * BLK_ROWS * p.ldz + (long)(ccol0 / BLK_COLS) * BLK_ELEMS;
  if (!ragged)
    stage_dlogits<ENTGRAD, false>(smem, acc, r_lse2, r_c0, r_cb, r_sa, t_local, wv0, wt0, lane, c1,
                                  vrows, dst);
  else
    stage_dlogits<ENTGRAD, true>(smem, acc, r_lse2, r_c0, r_cb, r_sa, t_local, wv0, wt0, lane, c1,
                                 vrows, dst);
}

template <bool ENTGRAD>
__global__ __launch_bounds__(NTHREADS) void bwd_dlogits_kernel(DlogitsArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_DLOGITS];
  const int L = tile_claim(p.n_mt * p.n_vt, p.tq);
  if (L < 0) return;
  int mt, vt;
  group_coords(L, p.n_mt, p.n_vt, 8, mt, vt);
  dlogits_tile<ENTGRAD>(p, mt, vt, smem);
}

// ---------------------------------------------------------------------------
// The fp32 side of an output tile (modes 1-3), for dX across vocabulary chunks and dW
// across token waves.  t.acc and t.out point at the tile's element (0, 0) of an fp32
// accumulator and of the bf16 result, both with leading dimension t.ld; rows
// [0, t.nrows) and columns [0, t.ncols) of the tile exist.  Each wave moves its
// 128 x 128 block through a private 32 KiB LDS slice, 64 rows at a time, so the fp32
// accumulator is read and written in 16-byte pieces (a half-wave covers 512 contiguous
// bytes of a row) and all of a lane's loads of a slice are in flight together;
// per-element accesses in the accumulator layout would wait on one read-modify-write
// after another.  Slice layout: row r (0..63) at 512 r bytes, column c at float
// (c ^ 32 ((r >> 2) & 1)), so the two half-waves of a staging write (rows r and r + 4)
// fall on different banks.
// mode 1: acc = v; mode 2: acc += v; mode 3: out = bf16(acc + v).
struct F32Tile {
  float* acc;
  uint16_t* out;
  long ld;
  int nrows, ncols;
  int mode;
};

__device__ __forceinline__ void tile_f32(const f32x16 (&acc)[4][4], char* smem, const F32Tile& t,
                                         int wave, int lane) {
  const int wr0 = (wave >> 1) * 128, wc0 = (wave & 1) * 128;
  float* sl = reinterpret_cast<float*>(smem + wave * 32768);
  const int lc = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = 32 * mi + acc_row(lane, e);  // (r >> 2) & 1 == hi
          sl[r * 128 + ((32 * nb + lc) ^ (hi << 5))] = acc_read(acc[2 * s + mi][nb][e]);
        }
    __syncthreads();
    const int rb = wr0 + 64 * s, cb = wc0;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // granule g = 64 it + lane: row g / 32, columns 4 (g % 32) .. + 3
      float4 old[16];
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int g = 64 * (16 * half + it) + lane, r = g >> 5, c = 4 * (g & 31);
        const int m = rb + r, h = cb + c;
        old[it] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t.mode != 1 && m < t.nrows && h < t.ncols)
          old[it] = *reinterpret_cast<const float4*>(t.acc + (long)m * t.ld + h);
      }
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int g = 64 * (16 * half + it) + lane, r = g >> 5, c = 4 * (g & 31);
        const int m = rb + r, h = cb + c;
        const float4 v = *reinterpret_cast<const float4*>(sl + r * 128 + (c ^ (((r >> 2) & 1) << 5)));
        const float4 u = t.mode == 1 ? v
                                     : make_float4(old[it].x + v.x, old[it].y + v.y,
                                                   old[it].z + v.z, old[it].w + v.w);
        if (m < t.nrows && h < t.ncols) {
          if (t.mode == 3) {
            const f32x2 lo = {u.x, u.y}, hi2 = {u.z, u.w};
            const uint32_t a = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
            const uint32_t b = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi2, bf16x2));
            *reinterpret_cast<uint2*>(t.out + (long)m * t.ld + h) = make_uint2(a, b);
          } else {
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, u),
                                        reinterpret_cast<u32x4*>(t.acc + (long)m * t.ld + h));
          }
        }
      }
    }
    __syncthreads();
  }
}

// dW[vbase + i, h] = sum_m dzs[m, i] X[m, h]: A = dzs^T (MN), B = X^T (MN), K = Mpad.
// mode 0: write bf16; 1-3: the fp32 accumulator across token waves (see tile_f32).
__device__ __forceinline__ void dw_tile(const GemmDwArgs& p, int ti, int th, char* smem) {
  const int i0 = ti * TILE, h0 = th * TILE;
  f32x16 acc[4][4];
  // dzs has Mpad rows (rows past M hold zeros); X has only M rows.
  const TileSrc A{p.dz + (long)(i0 / BLK_COLS) * BLK_ELEMS, BLK_COLS, p.chunk_cols - i0, p.Mpad,
                  (long)BLK_ROWS * p.ldz};
  const TileSrc B{p.X + h0, p.H, p.H - h0, p.M, 0};
  // the X^T loads (L2-resident) go out before the streamed d-logit loads of each step
  mainloop<BigShape, false, false, true>(acc, smem, A, B, p.Mpad);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr0 = (wave >> 1) * 128, wc0 = (wave & 1) * 128;
  const int rows = min(min(TILE, p.chunk_cols - i0), p.V - (p.vbase + i0));
  const long o = (long)(p.vbase + i0) * p.H + h0;
  if (p.mode == 0)
    store_acc_bf16(smem, acc, wr0, wc0, lane, p.dW + o, p.H, rows, p.H - h0);
  else
    tile_f32(acc, smem, F32Tile{p.acc + o, p.dW + o, p.H, rows, p.H - h0, p.mode}, wave, lane);
}

__global__ __launch_bounds__(NTHREADS) void gemm_dw_kernel(GemmDwArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BIG];
  const int L = tile_claim(p.n_h * p.n_i, p.tq);
  if (L < 0) return;
  int ti, th;
  // groups run along H: the few X^T tiles stay in L2 while each dzs tile is read by
  // one group of an XCD at a time, so dzs streams from HBM about once per H group
  group_coords(L, p.n_h, p.n_i, 8, th, ti);
  dw_tile(p, ti, th, smem);
}

// dX[m, h] (+)= sum_i dzs[m, i] W[vbase + i, h]: A = dzs (KC), B = W^T (MN), K = kcols.
// mode 0: write bf16; 1: write fp32 accumulator; 2: accumulate fp32; 3: accumulate and write bf16.
__device__ __forceinline__ void dx_tile(const GemmDxArgs& p, int tm, int th, char* smem) {
  const int m0 = tm * TILE, h0 = th * TILE;
  f32x16 acc[4][4];
  // the chunk's kcols (padded) columns of dzs (band tm of the blocked buffer); W has
  // V - vbase rows left
  const long band = (long)BLK_ROWS * p.ldz;
  const TileSrc A{p.dz + (long)tm * band, BLK_COLS, p.M - m0, p.kcols, band};
  const TileSrc B{p.W + (long)p.vbase * p.H + h0, p.H, p.H - h0, p.V - p.vbase, 0};
  mainloop<BigShape, true, false>(acc, smem, A, B, p.kcols);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr0 = (wave >> 1) * 128, wc0 = (wave & 1) * 128;
  if (p.mode == 0) {
    store_acc_bf16(smem, acc, wr0, wc0, lane, p.dX + (long)m0 * p.H + h0, p.H, p.M - m0,
                   p.H - h0);
  } else {
    const long o = (long)m0 * p.H + h0;
    tile_f32(acc, smem, F32Tile{p.acc + o, p.dX + o, p.H, p.M - m0, p.H - h0, p.mode}, wave,
             lane);
  }
}

__global__ __launch_bounds__(NTHREADS) void gemm_dx_kernel(GemmDxArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BIG];
  int tm, th;
  // groups run along H: in step, the XCDs read the same W columns (shared through the
  // memory-side cache) while each streams d-logit bands of its own
  tile_coords(blockIdx.x, gridDim.x, p.n_h, p.n_m, 8, th, tm);
  dx_tile(p, tm, th, smem);
}

// ---------------------------------------------------------------------------
// Pipelined backward: one launch runs the dW and dX tiles of one step (a token wave x
// vocabulary chunk, reading that step's d-logit buffer) together with the d-logit
// tiles of the next step (writing the other buffer), so no tile of a launch depends on
// another one, and the backward takes n + 1 launches for n steps instead of 3 n.  Each
// XCD (workgroup id modulo 8) takes an eighth of each kind of tile, contiguous in that
// kind's L2-grouped order, and works through its dW tiles first, then its dX tiles,
// then its d-logit tiles; ids past an XCD's share exit at once.
static_assert(LDS_DLOGITS >= LDS_BIG, "one LDS size serves every tile kind");

__device__ __forceinline__ void xcd_share(int n, int x, int& lo, int& cnt) {
  lo = (int)((long)n * x / 8);
  cnt = (int)((long)n * (x + 1) / 8) - lo;
}

template <bool ENTGRAD>
__global__ __launch_bounds__(NTHREADS) void bwd_pipe_kernel(PipeArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS_DLOGITS];
  const int x = blockIdx.x & 7;
  int pos = blockIdx.x >> 3, lo, cnt;
  xcd_share(p.n_dw, x, lo, cnt);
  if (pos < cnt) {
    int ti, th;
    group_coords(lo + pos, p.dw.n_h, p.dw.n_i, 8, th, ti);
    dw_tile(p.dw, ti, th, smem);
    return;
  }
  pos -= cnt;
  xcd_share(p.n_dx, x, lo, cnt);
  if (pos < cnt) {
    int tm, th;
    group_coords(lo + pos, p.dx.n_h, p.dx.n_m, 8, th, tm);
    dx_tile(p.dx, tm, th, smem);
    return;
  }
  pos -= cnt;
  xcd_share(p.n_dl, x, lo, cnt);
  if (pos < cnt) {
    int mt, vt;
    group_coords(lo + pos, p.dl.n_mt, p.dl.n_vt, 8, mt, vt);
    dlogits_tile<ENTGRAD>(p.dl, mt, vt, smem);
  }
}

// Scalar cross-entropy reductions over the valid rows, in one workgroup so the order
// of every addition is fixed (bitwise repeatable): thread t takes rows t, t + 1024, ...
// in fp64, then a fixed tree over the threads.  out = {sum of -logprob, valid rows,
// mean (NaN without a valid row)}.
constexpr int NLL_THREADS = 1024;
__global__ __launch_bounds__(NLL_THREADS) void nll_reduce_kernel(const float* __restrict__ logprob,
                                                                 const int64_t* __restrict__ targets,
                                                                 long M, int64_t V,
                                                                 int64_t ignore_index,
                                                                 double* __restrict__ out) {
  __shared__ double ss[NLL_THREADS];
  __shared__ long sc[NLL_THREADS];
  const int t = threadIdx.x;
  double s = 0.0;
  long c = 0;
  for (long i = t; i < M; i += NLL_THREADS) {
    const int64_t tg = targets[i];
    if (tg != ignore_index && tg >= 0 && tg < V) {
      s -= (double)logprob[i];
      ++c;
    }
  }
  ss[t] = s;
  sc[t] = c;
  __syncthreads();
  for (int w = NLL_THREADS / 2; w > 0; w >>= 1) {
    if (t < w) {
      ss[t] += ss[t + w];
      sc[t] += sc[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    out[0] = ss[0];
    out[1] = (double)sc[0];
    out[2] = sc[0] > 0 ? ss[0] / (double)sc[0] : __builtin_nan("");
  }
}

// grad[i] = -1 / n on valid rows (n = the valid-row count in reduced[1]), else 0.
__global__ void nll_mean_grad_kernel(const int64_t* __restrict__ targets, long M, int64_t V,
                                     int64_t ignore_index, const double* __restrict__ reduced,
                                     float* __restrict__ grad) {
  const double n = reduced[1];
  const float g = n > 0.0 ? (float)(-1.0 / n) : 0.f;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < M; i += stride) {
    const int64_t tg = targets[i];
    grad[i] = (tg != ignore_index && tg >= 0 && tg < V) ? g : 0.f;
  }
}

// Clipped policy loss on the per-token log-probs (Liger-Kernel PR 1294, "Chunked Triton
// GRPO loss": the loss on top of the fused linear log-probs, with clip range and
// token-level normalisation; the page gives no formulas, the plain reading is the
// clipped surrogate).  Per valid token, in fp64: r = exp(logprob - old_logprob),
// c = min(max(r, 1 - eps_low), 1 + eps_high), loss = -min(r A, c A), clipped iff
// c A < r A.  Both kernels evaluate the same expression, so the gradient kernel takes
// the same clip decision as the reduction.
struct PolicyTerm {
  double u, cl;  // r A and c A
  bool valid;
};
__device__ __forceinline__ PolicyTerm policy_term(const PolicyLossArgs& p, long i) {
  PolicyTerm o;
  const int64_t tg = p.targets[i];
  o.valid = tg != p.ignore_index && tg >= 0 && tg < p.V;
  const double lp = (double)p.logprob[i];
  const double old = p.old_logprob ? (double)p.old_logprob[i] : lp;
  const double a = (double)p.advantages[i];
  const double r = exp(lp - old);
  const double c = fmin(fmax(r, 1.0 - p.eps_low), 1.0 + p.eps_high);
  o.u = r * a;
  o.cl = c * a;
  return o;
}

// One workgroup, fixed summation order (bitwise repeatable): thread t takes tokens
// t, t + 1024, ..., then a fixed tree.  Writes the per-token loss (0 on invalid rows)
// and clip flags, and out = {sum of the loss, valid rows, clipped rows, sum / N} with
// N = denominator if > 0, else the valid rows (NaN when N is 0).
constexpr int PL_THREADS = 1024;
__global__ __launch_bounds__(PL_THREADS) void policy_loss_reduce_kernel(
    PolicyLossArgs p, float* __restrict__ per_token_loss, uint8_t* __restrict__ is_clipped,
    double* __restrict__ out) {
  __shared__ double ss[PL_THREADS];
  __shared__ long sn[PL_THREADS], sk[PL_THREADS];
  const int t = threadIdx.x;
  double s = 0.0;
  long n = 0, k = 0;
  for (long i = t; i < p.M; i += PL_THREADS) {
    const PolicyTerm o = policy_term(p, i);
    const bool clipped = o.valid && o.cl < o.u;
    const double loss = o.valid ? -fmin(o.u, o.cl) : 0.0;
    per_token_loss[i] = (float)loss;
    if (is_clipped) is_clipped[i] = clipped ? 1 : 0;
    s += loss;
    n += o.valid ? 1 : 0;
    k += clipped ? 1 : 0;
  }
  ss[t] = s;
  sn[t] = n;
  sk[t] = k;
  __syncthreads();
  for (int w = PL_THREADS / 2; w > 0; w >>= 1) {
    if (t < w) {
      ss[t] += ss[t + w];
      sn[t] += sn[t + w];
      sk[t] += sk[t + w];
    }
    __syncthreads();
  }
  if (t == 0) {
    const double N = p.denominator > 0.0 ? p.denominator : (double)sn[0];
    out[0] = ss[0];
    out[1] = (double)sn[0];
    out[2] = (double)sk[0];
    out[3] = N > 0.0 ? ss[0] / N : __builtin_nan("");
  }
}

// grad[i] = -r A / N on valid tokens whose minimum takes the unclipped term, else 0;
// N as in the reduction (the valid-row count read from reduced[1] when the
// denominator is not positive).
__global__ void policy_loss_grad_kernel(PolicyLossArgs p, const double* __restrict__ reduced,
                                        float* __restrict__ grad) {
  const double N = p.denominator > 0.0 ? p.denominator : reduced[1];
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < p.M; i += stride) {
    const PolicyTerm o = policy_term(p, i);
    grad[i] = (o.valid && !(o.cl < o.u) && N > 0.0) ? (float)(-o.u / N) : 0.f;
  }
}

__global__ void fill_u16_kernel(uint16_t* __restrict__ p, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long j = i; j < n; j += stride) p[j] = 0;
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free forward: the partials of its token waves.  A
// __device__ array is module memory: each GPU the library runs on holds its own copy,
// at its own address, from the module's load until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: kernels get the
// address from scratch_device_address() instead.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of each GPU's copy, looked up once per device (on the first call that
// needs it, with that device current) and kept.
constexpr int kScratchDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_addr[kScratchDevices];

hipError_t scratch_device_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Launchers (host side).  Each returns the hipGetLastError() of its launch.
// Grid of a launch of n tiles with tail queues (sets tq.queue): the tiles plus the
// spare workgroups.
static unsigned queued_grid(int64_t n, TileQueue& tq) {
  const QueueShape qs = tq.ctr ? queue_shape(n) : QueueShape{0, 0};
  tq.queue = qs.queue;
  return (unsigned)(n + qs.spare);
}

hipError_t launch_fwd_tile(const FwdTileArgs& a, bool ent, hipStream_t s) {
  FwdTileArgs b = a;
  b.tq.clear = nullptr;
  const unsigned g = queued_grid((int64_t)a.n_mt * a.n_vt, b.tq);
  if (ent)
    fwd_tile_kernel<FwdShape, true><<<g, FwdShape::NTHREADS, 0, s>>>(b);
  else
    fwd_tile_kernel<FwdShape, false><<<g, FwdShape::NTHREADS, 0, s>>>(b);
  return hipGetLastError();
}

hipError_t launch_target_logit(const FwdTileArgs& a, hipStream_t s) {
  const unsigned g = (unsigned)(((long)a.M + TL_ROWS - 1) / TL_ROWS);
  target_logit_kernel<<<g, 64 * TL_ROWS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd_merge(const FwdMergeArgs& a, bool ent, hipStream_t s) {
  const unsigned g = (unsigned)((a.M + MERGE_ROWS - 1) / MERGE_ROWS);
  if (ent)
    fwd_merge_kernel<true><<<g, MERGE_ROWS * MERGE_SLICES, 0, s>>>(a);
  else
    fwd_merge_kernel<false><<<g, MERGE_ROWS * MERGE_SLICES, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_dlogits(const DlogitsArgs& a, bool entgrad, hipStream_t s) {
  DlogitsArgs b = a;
  const unsigned g = queued_grid((int64_t)a.n_mt * a.n_vt, b.tq);
  if (entgrad)
    bwd_dlogits_kernel<true><<<g, NTHREADS, 0, s>>>(b);
  else
    bwd_dlogits_kernel<false><<<g, NTHREADS, 0, s>>>(b);
  return hipGetLastError();
}

hipError_t launch_bwd_pipe(const PipeArgs& a, bool entgrad, hipStream_t s) {
  const long per = (a.n_dw + 7) / 8 + (a.n_dx + 7) / 8 + (a.n_dl + 7) / 8;
  if (per == 0) return hipSuccess;
  if (entgrad)
    bwd_pipe_kernel<true><<<(unsigned)(8 * per), NTHREADS, 0, s>>>(a);
  else
    bwd_pipe_kernel<false><<<(unsigned)(8 * per), NTHREADS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_dw(const GemmDwArgs& a, hipStream_t s) {
  GemmDwArgs b = a;
  const unsigned g = queued_grid((int64_t)a.n_i * a.n_h, b.tq);
  gemm_dw_kernel<<<g, NTHREADS, 0, s>>>(b);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const GemmDxArgs& a, hipStream_t s) {
  gemm_dx_kernel<<<(unsigned)((long)a.n_m * a.n_h), NTHREADS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_nll_reduce(const float* logprob, const int64_t* targets, long M, int64_t V,
                             int64_t ignore_index, double* out, hipStream_t s) {
  nll_reduce_kernel<<<1, NLL_THREADS, 0, s>>>(logprob, targets, M, V, ignore_index, out);
  return hipGetLastError();
}

hipError_t launch_nll_mean_grad(const int64_t* targets, long M, int64_t V, int64_t ignore_index,
                                const double* reduced, float* grad, hipStream_t s) {
  long blocks = (M + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  nll_mean_grad_kernel<<<(unsigned)blocks, 256, 0, s>>>(targets, M, V, ignore_index, reduced, grad);
  return hipGetLastError();
}

hipError_t launch_policy_loss_reduce(const PolicyLossArgs& a, float* per_token_loss,
                                     uint8_t* is_clipped, double* out, hipStream_t s) {
  policy_loss_reduce_kernel<<<1, PL_THREADS, 0, s>>>(a, per_token_loss, is_clipped, out);
  return hipGetLastError();
}

hipError_t launch_policy_loss_grad(const PolicyLossArgs& a, const double* reduced, float* grad,
                                   hipStream_t s) {
  long blocks = (a.M + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  policy_loss_grad_kernel<<<(unsigned)blocks, 256, 0, s>>>(a, reduced, grad);
  return hipGetLastError();
}

hipError_t launch_fill_zero_u16(uint16_t* p, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  long blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  fill_u16_kernel<<<(unsigned)blocks, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

}  // namespace flce
