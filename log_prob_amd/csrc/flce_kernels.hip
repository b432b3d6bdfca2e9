// HIP kernels of libflce for gfx950 (CDNA4): fused LM-head linear + cross-entropy.
//
// Forward (Liger-Kernel FSLCE commit, "Summary" and "Implementation / Forward";
// SkyRL PR 2141, "Overview"):
//   fwd_tile     one workgroup per (256-row M tile, 256-column V tile): bf16 MFMA
//                mainloop over H, then an epilogue that reduces the logit tile to
//                per-row partial statistics (max m, sum of exp(z - m), and
//                sum of exp(z - m) (z - m) for entropy) and picks the target logit.
//   fwd_merge    combines the per-tile partials of each row (max first, then the
//                rescaled sums) into lse, logprob and entropy.
// Backward (Liger-Kernel PR 1294, "Kernel design notes": recompute the logits
// tiles, emit d-logits in the input dtype into a reusable buffer, then two grad
// GEMMs; SkyRL PR 2141, "Overview": split backward over the vocabulary):
//   bwd_dlogits  the same mainloop, epilogue forms scale * dz in bf16 for one
//                vocabulary chunk.
//   gemm_dw      dW[chunk] = dz_chunk^T X          (K = tokens)
//   gemm_dx      dX (+)= dz_chunk W[chunk]          (K = chunk columns)
//
// All tiles are 256 x 256 with K staged 64 at a time through double-buffered
// LDS (2 x 64 KiB) and v_mfma_f32_32x32x16_bf16.  Operands whose K dimension is
// contiguous in memory are copied to LDS as 16-byte chunks; operands whose M/N
// dimension is contiguous are loaded as 8x8 blocks and transposed in registers,
// so the LDS layout (K contiguous, 128 bytes per row, XOR-swizzled 16-byte
// chunks) and the MFMA fragment reads are the same for every operand.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce_internal.h"

namespace flce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int TILE = 256;               // rows and columns of a workgroup tile
constexpr int BK = 64;                  // K per LDS stage
constexpr int NTHREADS = 256;           // 4 waves of 64
constexpr int TILE_BYTES = TILE * BK * 2;          // one operand tile in LDS: 32 KiB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;        // A and B
constexpr int LDS_MAIN = 2 * STAGE_BYTES;          // double buffered: 128 KiB

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// LDS tile addressing: row r holds 64 bf16 of K (8 chunks of 16 bytes).  Chunk c
// of row r lives at chunk position c ^ swz(r).  swz mixes the low and the next
// three row bits so that both 8 consecutive rows (MFMA fragment reads) and rows
// 8 apart (transposed staging writes) fall on distinct chunk positions.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return (r << 7) + ((c ^ swz(r)) << 4); }

// Workgroup id -> tile coordinates.  Workgroups are handed to the 8 XCDs round
// robin, so id b runs on XCD b % 8.  The first step renumbers ids so that each
// XCD receives a contiguous range of logical ids; the second walks logical ids
// in groups of `group_m` tile rows, tile row fastest, so the ~32 workgroups
// resident on one XCD share a few operand tiles in that XCD's L2.
__device__ __forceinline__ void tile_coords(int bid, int nblocks, int n_m, int n_n, int group_m,
                                            int& tm, int& tn) {
  const int per = nblocks >> 3;
  int L = bid;
  if (bid < (per << 3)) L = (bid & 7) * per + (bid >> 3);
  const int width = group_m * n_n;
  const int g = L / width;
  const int first = g * group_m;
  const int gm = min(n_m - first, group_m);
  const int inner = L - g * width;
  tm = first + inner % gm;
  tn = inner / gm;
}

// ---------------------------------------------------------------------------
// Global -> register staging of one 256 x 64 operand tile (8 x 16 bytes per thread).
//
// KC (K contiguous): the operand is [rows][K] with leading dimension ld; the tile
// is rows [0, 256) relative to `base`, K range [k0, k0 + 64).  Thread t loads
// chunk ids t + 256 i: row id / 8, chunk id % 8 (8 threads read one 128-byte row
// segment).  Rows >= nrows and chunks at or past K read as zero.
//
// MN (M/N contiguous): the operand is [K][cols] with leading dimension ld; the
// tile is columns [0, 256) relative to `base`.  Thread t loads the 8 x 8 block of
// K rows 8 (t / 32) + i and columns 8 (t % 32) + j; 32 threads read one 512-byte
// row segment.  Columns >= ncols and K rows >= K read as zero.
struct Stage {
  u32x4 v[8];
};

template <bool KC>
__device__ __forceinline__ void stage_load(Stage& s, const uint16_t* __restrict__ base, long ld,
                                           int nrows_or_cols, int K, int k0) {
  const int t = threadIdx.x;
  if constexpr (KC) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = t + NTHREADS * i;
      const int r = id >> 3, c = id & 7;
      const int k = k0 + (c << 3);
      u32x4 val = {0u, 0u, 0u, 0u};
      if (r < nrows_or_cols && k < K)
        val = *reinterpret_cast<const u32x4*>(base + (long)r * ld + k);
      s.v[i] = val;
    }
  } else {
    const int cb = t & 31, kb = t >> 5;
    const int col = cb << 3;
    const bool col_ok = col < nrows_or_cols;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + (kb << 3) + i;
      u32x4 val = {0u, 0u, 0u, 0u};
      if (col_ok && k < K) val = *reinterpret_cast<const u32x4*>(base + (long)k * ld + col);
      s.v[i] = val;
    }
  }
}

__device__ __forceinline__ unsigned pack_lo(unsigned a, unsigned b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ unsigned pack_hi(unsigned a, unsigned b) {
  return (a >> 16) | (b & 0xffff0000u);
}

template <bool KC>
__device__ __forceinline__ void stage_store(const Stage& s, char* __restrict__ tile) {
  const int t = threadIdx.x;
  if constexpr (KC) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int id = t + NTHREADS * i;
      *reinterpret_cast<u32x4*>(tile + lds_off(id >> 3, id & 7)) = s.v[i];
    }
  } else {
    // s.v[i] holds K row i of the block (8 columns); write column j of the block
    // as one 16-byte K chunk: element i of output j = element j of input i.
    const int cb = t & 31, kb = t >> 5;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int w = j >> 1;
      u32x4 o;
      if ((j & 1) == 0) {
        o.x = pack_lo(s.v[0][w], s.v[1][w]);
        o.y = pack_lo(s.v[2][w], s.v[3][w]);
        o.z = pack_lo(s.v[4][w], s.v[5][w]);
        o.w = pack_lo(s.v[6][w], s.v[7][w]);
      } else {
        o.x = pack_hi(s.v[0][w], s.v[1][w]);
        o.y = pack_hi(s.v[2][w], s.v[3][w]);
        o.z = pack_hi(s.v[4][w], s.v[5][w]);
        o.w = pack_hi(s.v[6][w], s.v[7][w]);
      }
      *reinterpret_cast<u32x4*>(tile + lds_off((cb << 3) + j, kb)) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// The MFMA mainloop shared by every kernel.  The workgroup computes the 256 x 256
// tile D = A B^T (A: 256 x K, B: 256 x K, both logically K-contiguous) as 4 waves
// of WM x WN (wave w at rows (w / (256/WN)) * WM, columns (w % (256/WN)) * WN).
// acc[mb][nb] is the 32 x 32 block at (32 mb, 32 nb) of the wave tile, in the
// v_mfma_f32_32x32x16 layout: lane l, element e holds row 8 (e / 4) + 4 (l / 32)
// + e % 4 and column l % 32.
template <int WM, int WN>
struct WaveTile {
  static constexpr int MB = WM / 32;
  static constexpr int NB = WN / 32;
  static constexpr int WAVES_N = TILE / WN;
  f32x16 acc[MB][NB];
};

template <bool A_KC, bool B_KC, int WM, int WN>
__device__ __forceinline__ void mainloop(WaveTile<WM, WN>& wt, char* __restrict__ smem,
                                         const uint16_t* __restrict__ A, long lda, int a_valid,
                                         int a_kvalid,
                                         const uint16_t* __restrict__ B, long ldb, int b_valid,
                                         int b_kvalid, int K) {
  using WT = WaveTile<WM, WN>;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wr0 = (wave / WT::WAVES_N) * WM;
  const int wc0 = (wave % WT::WAVES_N) * WN;
#pragma unroll
  for (int mb = 0; mb < WT::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < WT::NB; ++nb)
#pragma unroll
      for (int e = 0; e < 16; ++e) wt.acc[mb][nb][e] = 0.f;

  const int nk = (K + BK - 1) / BK;
  Stage sa, sb;
  stage_load<A_KC>(sa, A, lda, a_valid, a_kvalid, 0);
  stage_load<B_KC>(sb, B, ldb, b_valid, b_kvalid, 0);
  stage_store<A_KC>(sa, smem);
  stage_store<B_KC>(sb, smem + TILE_BYTES);
  __syncthreads();

  const int frag_row = lane & 31;
  const int frag_half = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE_BYTES;
    const bool more = kt + 1 < nk;
    if (more) {
      stage_load<A_KC>(sa, A, lda, a_valid, a_kvalid, (kt + 1) * BK);
      stage_load<B_KC>(sb, B, ldb, b_valid, b_kvalid, (kt + 1) * BK);
    }
    const char* As = cur;
    const char* Bs = cur + TILE_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int chunk = 2 * kk + frag_half;
      bf16x8 af[WT::MB], bfr[WT::NB];
#pragma unroll
      for (int mb = 0; mb < WT::MB; ++mb)
        af[mb] = *reinterpret_cast<const bf16x8*>(As + lds_off(wr0 + 32 * mb + frag_row, chunk));
#pragma unroll
      for (int nb = 0; nb < WT::NB; ++nb)
        bfr[nb] = *reinterpret_cast<const bf16x8*>(Bs + lds_off(wc0 + 32 * nb + frag_row, chunk));
#pragma unroll
      for (int mb = 0; mb < WT::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < WT::NB; ++nb)
          wt.acc[mb][nb] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], wt.acc[mb][nb], 0, 0, 0);
    }
    if (more) {
      char* nxt = smem + ((kt + 1) & 1) * STAGE_BYTES;
      stage_store<A_KC>(sa, nxt);
      stage_store<B_KC>(sb, nxt + TILE_BYTES);
    }
    __syncthreads();
  }
}

// Row of the wave tile held by lane `lane` in element e of a 32 x 32 block.
__device__ __forceinline__ int acc_row(int lane, int e) {
  return ((e >> 2) << 3) + ((lane >> 5) << 2) + (e & 3);
}

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Reduce-scatter over the 32 lanes that share a half-wave: on entry every lane
// holds 32 values v[q]; on exit lane l holds in v[0] the reduction over those
// lanes of v[l % 32].
template <class Op>
__device__ __forceinline__ void reduce_scatter32(float (&v)[32], int lane, Op op) {
#pragma unroll
  for (int s = 16; s >= 1; s >>= 1) {
    const bool upper = (lane & s) != 0;
#pragma unroll
    for (int i = 0; i < s; ++i) {
      const float send = upper ? v[i] : v[i + s];
      const float keep = upper ? v[i + s] : v[i];
      v[i] = op(keep, shfl_xor(send, s));
    }
  }
}

// Inverse of reduce_scatter32's distribution: lane l holds v[0] for slot l % 32;
// on exit every lane holds all 32 slots of its half-wave.
__device__ __forceinline__ void all_gather32(float (&v)[32], int lane) {
#pragma unroll
  for (int s = 1; s <= 16; s <<= 1) {
    const bool upper = (lane & s) != 0;
#pragma unroll
    for (int i = 0; i < s; ++i) {
      const float other = shfl_xor(v[i], s);
      const float lo = upper ? other : v[i];
      const float hi = upper ? v[i] : other;
      v[i] = lo;
      v[i + s] = hi;
    }
  }
}

// ---------------------------------------------------------------------------
// Forward tile kernel.  Wave tile 64 x 256 (4 waves stacked along M), so each wave
// owns complete rows of the workgroup's V tile and reduces them on its own.
// Lane l holds, for row slot q = 16 mb + e (mb < 2, e < 16), the 8 columns
// 32 nb + l % 32 of wave row 32 mb + acc_row(l, e).
template <bool ENT>
__global__ __launch_bounds__(NTHREADS) void fwd_tile_kernel(FwdTileArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_MAIN];
  __shared__ int t_local[TILE];
  int mt, vt;
  tile_coords(blockIdx.x, gridDim.x, p.n_mt, p.n_vt, 8, mt, vt);
  const int row0 = mt * TILE, col0 = vt * TILE;
  const int tid = threadIdx.x;
  {
    // target column relative to this tile, or -1 if not a valid target in it
    const int r = row0 + tid;
    int tl = -1;
    if (r < p.M) {
      const int64_t t = p.targets[r];
      if (t != p.ignore_index && t >= col0 && t < min<int64_t>(col0 + TILE, p.V))
        tl = (int)(t - col0);
    }
    t_local[tid] = tl;
  }

  WaveTile<64, 256> wt;
  mainloop<true, true, 64, 256>(wt, smem, p.X + (long)row0 * p.H, p.H, p.M - row0, p.H,
                                p.W + (long)col0 * p.H, p.H, p.V - col0, p.H, p.H);

  const int lane = tid & 63, wave = tid >> 6;
  const int wr0 = wave * 64;
  const int lc = lane & 31;
  const float c1 = p.scale * LOG2E;  // logits in log2 units: z2 = acc * c1

  // scale into log2 units; mask columns past V (only the last V tile has any)
  const bool ragged = col0 + TILE > p.V;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const bool colok = !ragged || (col0 + 32 * nb + lc < p.V);
#pragma unroll
      for (int e = 0; e < 16; ++e)
        wt.acc[mb][nb][e] = colok ? wt.acc[mb][nb][e] * c1 : -INFINITY;
    }

  // target logit: the unique lane holding column t[row] writes z[row, t] = z2 / log2(e)
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rl = wr0 + 32 * mb + acc_row(lane, e);
      const int d = t_local[rl] - lc;
      if (d >= 0 && (d & 31) == 0) {
        float z = 0.f;
#pragma unroll
        for (int nb = 0; nb < 8; ++nb)
          if ((d >> 5) == nb) z = wt.acc[mb][nb][e];
        p.zt[row0 + rl] = z * LN2;
      }
    }

  // tile row maxima
  float mx[32];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float m = wt.acc[mb][0][e];
#pragma unroll
      for (int nb = 1; nb < 8; ++nb) m = fmaxf(m, wt.acc[mb][nb][e]);
      mx[16 * mb + e] = m;
    }
  reduce_scatter32(mx, lane, [](float a, float b) { return fmaxf(a, b); });
  const float my_max = mx[0];
  all_gather32(mx, lane);

  // shifted sums: s = sum exp2(z2 - m2), u = sum exp2(z2 - m2) (z2 - m2)
  float sv[32], uv[32];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float m = mx[16 * mb + e];
      float s = 0.f, u = 0.f;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const float d = wt.acc[mb][nb][e] - m;
        const float pe = __builtin_amdgcn_exp2f(d);
        s += pe;
        if constexpr (ENT) u += pe * fmaxf(d, -3.0e38f);
      }
      sv[16 * mb + e] = s;
      if constexpr (ENT) uv[16 * mb + e] = u;
    }
  reduce_scatter32(sv, lane, [](float a, float b) { return a + b; });
  if constexpr (ENT) reduce_scatter32(uv, lane, [](float a, float b) { return a + b; });

  // lane l now owns row slot q = l % 32
  const int q = lc;
  const int row = row0 + wr0 + 32 * (q >> 4) + acc_row(lane, q & 15);
  const long off = (long)vt * p.Mpad + row;
  p.part_m[off] = my_max * LN2;
  p.part_s[off] = sv[0];
  if constexpr (ENT) p.part_u[off] = uv[0] * LN2;
}

// Merge of the per-tile partials of each row: m* = max m_j, S = sum s_j e^(m_j - m*),
// U = sum e^(m_j - m*) (u_j + (m_j - m*) s_j); lse = m* + log S, entropy = log S - U / S.
template <bool ENT>
__global__ __launch_bounds__(256) void fwd_merge_kernel(FwdMergeArgs p) {
  const int row = blockIdx.x * 256 + threadIdx.x;
  if (row >= p.M) return;
  float m = -INFINITY;
  for (int j = 0; j < p.n_vt; ++j) m = fmaxf(m, p.part_m[(long)j * p.Mpad + row]);
  float S = 0.f, U = 0.f;
  for (int j = 0; j < p.n_vt; ++j) {
    const long off = (long)j * p.Mpad + row;
    const float dm = p.part_m[off] - m;
    const float a = __expf(dm);
    const float s = p.part_s[off];
    S += s * a;
    if constexpr (ENT) U += a * (p.part_u[off] + dm * s);
  }
  const float logS = logf(S);
  const float lse = m + logS;
  const int64_t t = p.targets[row];
  const bool valid = t != p.ignore_index && t >= 0 && t < p.V;
  p.lse[row] = lse;
  p.logprob[row] = valid ? p.zt[row] - lse : 0.f;
  if constexpr (ENT) p.entropy[row] = valid ? logS - U / S : 0.f;
}

// ---------------------------------------------------------------------------
// Backward d-logits for one vocabulary chunk: dzs = scale * dz in bf16, written
// to a [Mpad, ldz] buffer (chunk column j = vocabulary column vbase + j).  Columns
// past V and rows past M are written as zero.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <bool ENTGRAD>
__global__ __launch_bounds__(NTHREADS) void bwd_dlogits_kernel(DlogitsArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_MAIN];
  __shared__ float r_lse2[TILE], r_a[TILE], r_b[TILE], r_E[TILE];
  __shared__ int t_local[TILE];
  int mt, vt;
  tile_coords(blockIdx.x, gridDim.x, p.n_mt, p.n_vt, 8, mt, vt);
  const int row0 = mt * TILE, ccol0 = vt * TILE, col0 = p.vbase + ccol0;
  const int tid = threadIdx.x;
  {
    const int r = row0 + tid;
    float lse = 0.f, a = 0.f, b = 0.f, E = 0.f;
    int tl = -1;
    if (r < p.M) {
      const int64_t t = p.targets[r];
      const bool valid = t != p.ignore_index && t >= 0 && t < p.V;
      lse = p.lse[r];
      if (valid) {
        a = p.grad_logprob ? p.grad_logprob[r] : 0.f;
        if constexpr (ENTGRAD) {
          b = p.grad_entropy[r];
          E = lse - p.entropy[r];
        }
        if (t >= col0 && t < col0 + TILE) tl = (int)(t - col0);
      }
    }
    r_lse2[tid] = lse * LOG2E;
    r_a[tid] = a;
    r_b[tid] = b;
    r_E[tid] = E;
    t_local[tid] = tl;
  }

  WaveTile<64, 256> wt;
  mainloop<true, true, 64, 256>(wt, smem, p.X + (long)row0 * p.H, p.H, p.M - row0, p.H,
                                p.W + (long)col0 * p.H, p.H, p.V - col0, p.H, p.H);

  const int lane = tid & 63, wave = tid >> 6;
  const int wr0 = wave * 64;
  const int lc = lane & 31;
  const float c1 = p.scale * LOG2E;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rl = wr0 + 32 * mb + acc_row(lane, e);
      const float lse2 = r_lse2[rl], a = r_a[rl], b = r_b[rl], E = r_E[rl];
      const int tl = t_local[rl];
      uint16_t* out = p.dz + (long)(row0 + rl) * p.ldz + ccol0 + lc;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        const int cl = 32 * nb + lc;
        const float acc = wt.acc[mb][nb][e];
        const float pr = __builtin_amdgcn_exp2f(acc * c1 - lse2);
        float d = (cl == tl ? a : 0.f) - a * pr;
        if constexpr (ENTGRAD) d += b * pr * (E - acc * p.scale);
        d *= p.scale;
        if (col0 + cl >= p.V) d = 0.f;
        out[32 * nb] = f32_to_bf16_rne(d);
      }
    }
}

// ---------------------------------------------------------------------------
// Plain GEMMs of the backward, 4 waves of 128 x 128.
// dW[vbase + i, h] = sum_m dzs[m, i] X[m, h]    (A = dzs^T: MN-contiguous; B = X^T: MN-contiguous)
__global__ __launch_bounds__(NTHREADS) void gemm_dw_kernel(GemmDwArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_MAIN];
  int ti, th;
  tile_coords(blockIdx.x, gridDim.x, p.n_i, p.n_h, 8, ti, th);
  const int i0 = ti * TILE, h0 = th * TILE;
  WaveTile<128, 128> wt;
  // K runs over the Mpad rows of dzs (rows past M hold zeros); X has only M rows.
  mainloop<false, false, 128, 128>(wt, smem, p.dz + i0, p.ldz, p.chunk_cols - i0, p.Mpad,
                                   p.X + h0, p.H, p.H - h0, p.M, p.Mpad);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr0 = (wave >> 1) * 128, wc0 = (wave & 1) * 128;
  const int lc = lane & 31;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int i = i0 + wr0 + 32 * mb + acc_row(lane, e);
      const int v = p.vbase + i;
      if (i >= p.chunk_cols || v >= p.V) continue;
      uint16_t* out = p.dW + (long)v * p.H;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int h = h0 + wc0 + 32 * nb + lc;
        if (h < p.H) out[h] = f32_to_bf16_rne(wt.acc[mb][nb][e]);
      }
    }
}

// dX[m, h] (+)= sum_i dzs[m, i] W[vbase + i, h]  (A = dzs: K-contiguous; B = W^T: MN-contiguous)
// mode 0: write bf16; 1: write fp32 accumulator; 2: accumulate fp32; 3: accumulate and write bf16.
__global__ __launch_bounds__(NTHREADS) void gemm_dx_kernel(GemmDxArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_MAIN];
  int tm, th;
  tile_coords(blockIdx.x, gridDim.x, p.n_m, p.n_h, 8, tm, th);
  const int m0 = tm * TILE, h0 = th * TILE;
  WaveTile<128, 128> wt;
  // K runs over the kcols (padded) columns of the chunk; W has V - vbase rows left.
  mainloop<true, false, 128, 128>(wt, smem, p.dz + (long)m0 * p.ldz, p.ldz, p.M - m0, p.kcols,
                                  p.W + (long)p.vbase * p.H + h0, p.H, p.H - h0, p.V - p.vbase,
                                  p.kcols);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wr0 = (wave >> 1) * 128, wc0 = (wave & 1) * 128;
  const int lc = lane & 31;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + wr0 + 32 * mb + acc_row(lane, e);
      if (m >= p.M) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int h = h0 + wc0 + 32 * nb + lc;
        if (h >= p.H) continue;
        const long o = (long)m * p.H + h;
        float v = wt.acc[mb][nb][e];
        if (p.mode >= 2) v += p.acc[o];
        if (p.mode == 1 || p.mode == 2)
          p.acc[o] = v;
        else
          p.dX[o] = f32_to_bf16_rne(v);
      }
    }
}

__global__ void fill_u16_kernel(uint16_t* __restrict__ p, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long stride = (long)gridDim.x * blockDim.x;
  for (long j = i; j < n; j += stride) p[j] = 0;
}

// ---------------------------------------------------------------------------
// Launchers (host side).  Each returns the hipGetLastError() of its launch.
static unsigned nblocks_of(long n) { return (unsigned)n; }

hipError_t launch_fwd_tile(const FwdTileArgs& a, bool ent, hipStream_t s) {
  const unsigned g = nblocks_of((long)a.n_mt * a.n_vt);
  if (ent)
    fwd_tile_kernel<true><<<g, NTHREADS, 0, s>>>(a);
  else
    fwd_tile_kernel<false><<<g, NTHREADS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd_merge(const FwdMergeArgs& a, bool ent, hipStream_t s) {
  const unsigned g = (unsigned)((a.M + 255) / 256);
  if (ent)
    fwd_merge_kernel<true><<<g, 256, 0, s>>>(a);
  else
    fwd_merge_kernel<false><<<g, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_dlogits(const DlogitsArgs& a, bool entgrad, hipStream_t s) {
  const unsigned g = nblocks_of((long)a.n_mt * a.n_vt);
  if (entgrad)
    bwd_dlogits_kernel<true><<<g, NTHREADS, 0, s>>>(a);
  else
    bwd_dlogits_kernel<false><<<g, NTHREADS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_dw(const GemmDwArgs& a, hipStream_t s) {
  gemm_dw_kernel<<<nblocks_of((long)a.n_i * a.n_h), NTHREADS, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const GemmDxArgs& a, hipStream_t s) {
  gemm_dx_kernel<<<nblocks_of((long)a.n_m * a.n_h), NTHREADS, 0, s>>>(a);
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
