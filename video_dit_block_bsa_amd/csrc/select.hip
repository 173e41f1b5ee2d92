// Pooled block scores and key-block selection in one kernel ("Block selection
// via pooled attention scores" and the Top-r / CDF-p modes of "Implementation
// details and design trade-offs", LongCat-Video deep dive, section "Block
// Sparse Attention"; combined top-k/CDF clamps from the zhaifeiyue notes,
// section 3). The pages score blocks from pooled vectors "without computing
// the full QK^T"; here the pooled score matrix does not leave the chip either.
//
// One workgroup of 8 waves owns a tile of query-block rows of one (batch,
// head):
//   scores  S[r][j] = (Q_pool[r] . K_pool[j]) * scale for every key block j,
//           with fp32 MFMA 16x16x4 (exact fp32 products, fp32 sums in a fixed
//           order), written into LDS. Each wave streams its own 16-column
//           slices of K_pool straight from global memory (L2-resident: 512
//           bytes per key block per head), so K_pool is read once per
//           workgroup and never staged.
//   select  one wave per row. Scores are mapped to order-preserving 32-bit
//           keys; the k-th largest key is found by a 32-step bitwise search
//           whose counts are wave ballots, and ties at the threshold go to
//           the lower key-block id. CDF mode first finds the smallest top set
//           whose softmax mass reaches p with the same bitwise search on
//           mass, then clamps the count and selects that many blocks. The
//           row's scores sit in registers (lane l holds key blocks l, l+64,
//           ...) when there are at most 4096 key blocks, and are re-read from
//           LDS at every step of the search beyond that.
// Everything is wave-uniform and summed in fixed orders, so results are
// deterministic, and a row's result does not depend on the rows it shares a
// workgroup with.
#include "launch.h"

namespace bsa {

// Order-preserving map from fp32 to uint32 (larger float -> larger key);
// -0 and +0 map to the same key. Key 0 marks "not a candidate".
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = (f == 0.f) ? 0u : __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Scores of rows i0 .. i0+rows-1 (rows <= 16) against every key block into
// LDS rows of `lds` floats (MFMA rows past `rows` are computed on row i0 and
// not kept).
// Step s = 4i + j of a 16x16x4 MFMA contracts channels 16i + 4kk + j
// (kk = 0..3): lane group kk = lane/16 supplies channel 16i + 4kk + j of its
// row (A) or column (B). Load i then brings each lane the 16 bytes at offset
// 64i + 16kk of its row, so the four lanes of a row read 64 contiguous bytes
// and one load touches 16 cache lines, not 64.
__device__ __forceinline__ void score_rows(const Geom& g, const float* __restrict__ qrow0,
                                           const float* __restrict__ kb, int rows, int lds,
                                           float* srows, int wave, int nwaves) {
  const int lane = threadIdx.x & 63;
  const int m = lane & 15;
  const int kk = lane >> 4;
  float qa[32];
  {
    const float* src = qrow0 + (size_t)(m < rows ? m : 0) * kHeadDim + 4 * kk;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float4 x = *reinterpret_cast<const float4*>(src + 16 * s);
      qa[4 * s] = x.x;
      qa[4 * s + 1] = x.y;
      qa[4 * s + 2] = x.z;
      qa[4 * s + 3] = x.w;
    }
  }
  const int ntiles = (g.nbk + 15) >> 4;
  // The next column tile's K_pool slices are loaded while the current one is
  // contracted, so the loads' latency hides behind the MFMA chain.
  auto load_cols = [&](int ct, float (&kf)[32]) {
    const int col = min(ct * 16 + m, g.nbk - 1);
    const float* src = kb + (size_t)col * kHeadDim + 4 * kk;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float4 x = *reinterpret_cast<const float4*>(src + 16 * s);
      kf[4 * s] = x.x;
      kf[4 * s + 1] = x.y;
      kf[4 * s + 2] = x.z;
      kf[4 * s + 3] = x.w;
    }
  };
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  float kf[2][32];
  if (wave < ntiles) load_cols(wave, kf[0]);
  auto tile = [&](int ct, float (&cur)[32], float (&nxt)[32]) {
    if (ct + nwaves < ntiles) load_cols(ct + nwaves, nxt);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 32; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[s], cur[s], acc, 0, 0, 0);
    // Accumulator value v is row 4*kk + v, column m of the tile.
    const int col = ct * 16 + m;
    if (col < g.nbk) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = 4 * kk + v;
        if (r < rows) srows[r * lds + col] = acc[v] * g.scale;
      }
    }
  };
  for (int ct = wave; ct < ntiles; ct += 2 * nwaves) {
    tile(ct, kf[0], kf[1]);
    if (ct + nwaves < ntiles) tile(ct + nwaves, kf[1], kf[0]);
  }
}

// Selection of one row whose n_allowed scores are row[0 .. na-1] (LDS).
// kR > 0: the row is copied into registers (kR chunks of 64 per lane,
// na <= 64 kR); kR == 0: every step re-reads it from LDS.
template <int kR>
__device__ __forceinline__ void select_row(const float* row, int na, int mode, int k, float p,
                                           int k_min, int k_max, int stride,
                                           int32_t* __restrict__ out, int32_t* __restrict__ cnt_out) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int nch = kR > 0 ? kR : (na + 63) >> 6;
  constexpr int kRegs = kR > 0 ? kR : 1;  // also the unroll count of the chunk loops
  uint32_t key_r[kRegs];
  float val_r[kRegs];
  if constexpr (kR > 0) {
#pragma unroll kRegs
    for (int c = 0; c < kR; ++c) {
      const int j = c * 64 + lane;
      const bool ok = j < na;
      val_r[c] = ok ? row[j] : -INFINITY;
      key_r[c] = ok ? order_key(val_r[c]) : 0u;
    }
  }
  // Score and key of chunk c for this lane.
  auto score = [&](int c) -> float {
    if constexpr (kR > 0) return val_r[c];
    const int j = c * 64 + lane;
    return j < na ? row[j] : -INFINITY;
  };
  auto key_of = [&](int c) -> uint32_t {
    if constexpr (kR > 0) return key_r[c];
    const int j = c * 64 + lane;
    return j < na ? order_key(row[j]) : 0u;
  };

  int keep;
  if (mode == 0) {
    keep = min(k, na);
  } else {
    // Softmax over the allowed blocks (fp32, max-subtracted).
    float m = -INFINITY;
#pragma unroll kRegs
    for (int c = 0; c < nch; ++c) m = fmaxf(m, score(c));
    m = wave_max(m);
    float z = 0.f;
#pragma unroll kRegs
    for (int c = 0; c < nch; ++c) {
      const float e = (key_of(c) != 0u) ? expf(score(c) - m) : 0.f;
      if constexpr (kR > 0) val_r[c] = e;
      z += e;
    }
    z = wave_sum(z);
    const float inv_z = 1.0f / z;
    // Probability of chunk c for this lane (the same expression, evaluated
    // the same way, whether kept in registers or recomputed).
    auto prob = [&](int c) -> float {
      if constexpr (kR > 0) return val_r[c];
      return (key_of(c) != 0u) ? expf(score(c) - m) * inv_z : 0.f;
    };
    if constexpr (kR > 0) {
#pragma unroll kRegs
      for (int c = 0; c < kR; ++c) val_r[c] *= inv_z;
    }
    // Largest key threshold whose top set still holds mass >= p.
    uint32_t tau = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      float part = 0.f;
#pragma unroll kRegs
      for (int c = 0; c < nch; ++c) part += (key_of(c) >= cand) ? prob(c) : 0.f;
      if (wave_sum(part) >= p) tau = cand;
    }
    int raw;
    if (tau == 0u) {
      raw = na;  // no prefix reaches p (p = 1 with rounding): all allowed blocks
    } else {
      int gt = 0;
      float part = 0.f;
#pragma unroll kRegs
      for (int c = 0; c < nch; ++c) {
        const uint32_t kc = key_of(c);
        gt += __popcll(__ballot(kc > tau));
        part += (kc > tau) ? prob(c) : 0.f;
      }
      float run = wave_sum(part);
      int add = 0;
      // Blocks tied at the threshold join in ascending id order until the
      // mass reaches p.
#pragma unroll kRegs
      for (int c = 0; c < nch; ++c) {
        uint64_t eq = __ballot(key_of(c) == tau);
        const float pc = prob(c);
        while (eq != 0ull && run < p) {
          const int src = __ffsll((long long)eq) - 1;
          run += __shfl(pc, src);
          ++add;
          eq &= eq - 1ull;
        }
      }
      raw = gt + add;
    }
    const int hi = min(k_max, na);
    keep = min(max(raw, k_min), hi);
  }

  // k-th largest key by a bitwise search; counts are wave ballots.
  uint32_t tau = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = tau | (1u << bit);
    int c_ge = 0;
#pragma unroll kRegs
    for (int c = 0; c < nch; ++c) c_ge += __popcll(__ballot(key_of(c) >= cand));
    if (c_ge >= keep) tau = cand;
  }
  int gt = 0;
#pragma unroll kRegs
  for (int c = 0; c < nch; ++c) gt += __popcll(__ballot(key_of(c) > tau));
  const int need_eq = keep - gt;

  int pos = 0;
  int eq_seen = 0;
#pragma unroll kRegs
  for (int c = 0; c < nch; ++c) {
    const uint32_t kc = key_of(c);
    const bool is_gt = kc > tau;
    const bool is_eq = kc == tau;
    const uint64_t eqb = __ballot(is_eq);
    const int eq_rank = eq_seen + __popcll(eqb & below);
    const bool sel = is_gt || (is_eq && eq_rank < need_eq);
    const uint64_t selb = __ballot(sel);
    if (sel) out[pos + __popcll(selb & below)] = c * 64 + lane;
    pos += __popcll(selb);
    eq_seen += __popcll(eqb);
  }
  for (int q = keep + lane; q < stride; q += 64) out[q] = -1;
  if (lane == 0) *cnt_out = keep;
}

struct SelectArgs {
  Geom g;
  int row0;       // first query block of every (batch, head) to select for
  int tiles;      // row tiles per (batch, head)
  int rows;       // rows per tile
  int lds;        // LDS row stride (floats)
  int mode, k, k_min, k_max, stride;
  float p;
};

// kR: register chunks per lane (1..64) or 0 (rows re-read from LDS);
// kWaves: waves per workgroup; kLdsFloats: LDS for the tile's score rows.
template <int kR, int kWaves, int kLdsFloats>
__global__ __launch_bounds__(64 * kWaves) void fused_select_kernel(SelectArgs a, const float* __restrict__ qp,
                                                                  const float* __restrict__ kp,
                                                                  int32_t* __restrict__ idx,
                                                                  int32_t* __restrict__ cnt) {
  __shared__ __attribute__((aligned(16))) float srows[kLdsFloats];
  const Geom& g = a.g;
  const int bh = blockIdx.x / a.tiles;
  const int tile = blockIdx.x - bh * a.tiles;
  const int i0 = a.row0 + tile * a.rows;
  const int rows = min(a.rows, g.nb - i0);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  score_rows(g, qp + ((size_t)bh * g.nb + i0) * kHeadDim, kp + (size_t)bh * g.nbk * kHeadDim, rows,
             a.lds, srows, wave, kWaves);
  __syncthreads();
  for (int r = wave; r < rows; r += kWaves) {
    const int i = i0 + r;
    const size_t row = (size_t)bh * g.nb + i;
    select_row<kR>(srows + r * a.lds, allowed_key_blocks(g, i), a.mode, a.k, a.p, a.k_min, a.k_max,
                   a.stride, idx + row * a.stride, cnt + row);
  }
}

constexpr int kSelectLds = 32768;  // floats (128 KB) of score rows per workgroup

hipError_t launch_select(const Geom& g, const float* qp, const float* kp, int mode, int k, float p,
                         int k_min, int k_max, int stride, int32_t* idx, int32_t* cnt, int row0,
                         hipStream_t stream) {
  if (row0 >= g.nb) return hipSuccess;
  SelectArgs a;
  a.g = g;
  a.row0 = row0;
  a.mode = mode;
  a.k = k;
  a.p = p;
  a.k_min = k_min;
  a.k_max = k_max;
  a.stride = stride;
  a.lds = (g.nbk + 3) & ~3;
  const int chunks = (g.nbk + 63) / 64;
  // Rows per tile: 8, one wave each (every workgroup reads all of K_pool, so
  // more rows per tile means fewer reads). Up to 2048 key blocks their scores
  // take at most 64 KB of LDS and two workgroups share a CU, one's scoring
  // overlapping the other's searches; up to 4096, 128 KB; beyond, as many
  // rows as 128 KB of LDS holds.
  int rows;
  if (chunks <= 64) rows = 8;
  else rows = a.lds <= kSelectLds / 4 ? 4 : a.lds <= kSelectLds / 2 ? 2 : 1;
  a.rows = rows;
  a.tiles = (g.nb - row0 + rows - 1) / rows;
  const dim3 grid((unsigned)((size_t)a.tiles * g.bh));
#define BSA_FUSED(R, WAVES, LDS)                                                             \
  hipLaunchKernelGGL((fused_select_kernel<R, WAVES, LDS>), grid, dim3(64 * (WAVES)), 0, stream, a, \
                     qp, kp, idx, cnt)
  // Register chunks are rounded up to a multiple of 4 (8 past 32): every
  // chunk is visited at each of the 32 search steps, so padding costs time.
  if (chunks <= 1) BSA_FUSED(1, 8, 8 * 64);
  else if (chunks <= 2) BSA_FUSED(2, 8, 8 * 128);
  else if (chunks <= 4) BSA_FUSED(4, 8, 8 * 256);
  else if (chunks <= 8) BSA_FUSED(8, 8, 8 * 512);
  else if (chunks <= 12) BSA_FUSED(12, 8, 8 * 768);
  else if (chunks <= 16) BSA_FUSED(16, 8, 8 * 1024);
  else if (chunks <= 20) BSA_FUSED(20, 8, 8 * 1280);
  else if (chunks <= 24) BSA_FUSED(24, 8, 8 * 1536);
  else if (chunks <= 28) BSA_FUSED(28, 8, 8 * 1792);
  else if (chunks <= 32) BSA_FUSED(32, 8, 8 * 2048);
  else if (chunks <= 40) BSA_FUSED(40, 8, 8 * 2560);
  else if (chunks <= 48) BSA_FUSED(48, 8, 8 * 3072);
  else if (chunks <= 56) BSA_FUSED(56, 8, 8 * 3584);
  else if (chunks <= 64) BSA_FUSED(64, 8, 8 * 4096);
  else BSA_FUSED(0, 8, kSelectLds);
#undef BSA_FUSED
  return hipGetLastError();
}

}  // namespace bsa
