// Pooled block scores and key-block selection ("Block selection via pooled
// attention scores" and the Top-r / CDF-p modes of "Implementation details
// and design trade-offs", LongCat-Video deep dive, section "Block Sparse
// Attention"; combined top-k/CDF clamps from the zhaifeiyue notes, section 3).
//
// scores_kernel: S = (Q_pool K_pool^T) * scale per (batch, head), fp32. A
//   64 x 64 output tile per workgroup, both operand tiles staged in LDS with
//   the channel index outermost so that each thread reads 4 consecutive rows
//   with one 16-byte LDS load; 16 FMAs per pair of loads; fixed summation
//   order over the 128 channels.
// select_kernel: one wave64 per query-block row. The row's scores live in
//   registers (lane l holds key blocks l, l+64, ...). Scores are mapped to
//   order-preserving 32-bit keys; the k-th largest key is found by a 32-step
//   bitwise search whose counts are wave ballots. Ties at the threshold go to
//   the lower key-block id. CDF mode first finds the smallest top set whose
//   softmax mass reaches p with the same bitwise search on mass, then clamps
//   the count and selects that many blocks. Everything is wave-uniform and
//   summed in fixed orders, so results are deterministic.
#include "common.h"

namespace bsa {

constexpr int kScoreTile = 64;

__global__ __launch_bounds__(kThreads) void scores_kernel(Geom g, const float* __restrict__ qp,
                                                          const float* __restrict__ kp,
                                                          float* __restrict__ s) {
  __shared__ float qs[kHeadDim][kScoreTile + 4];
  __shared__ float ks[kHeadDim][kScoreTile + 4];
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * kScoreTile;
  const int j0 = blockIdx.x * kScoreTile;
  const int t = threadIdx.x;
  const float* qb = qp + (size_t)bh * g.nb * kHeadDim;
  const float* kb = kp + (size_t)bh * g.nb * kHeadDim;

  // Rows run fastest across lanes so that the transposed LDS stores are
  // conflict-free; every loaded 16-byte piece is used.
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int c = t + kThreads * r;
    const int row = c & 63;
    const int d4 = c >> 6;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i0 + row < g.nb) a = *reinterpret_cast<const float4*>(qb + (size_t)(i0 + row) * kHeadDim + d4 * 4);
    if (j0 + row < g.nb) b = *reinterpret_cast<const float4*>(kb + (size_t)(j0 + row) * kHeadDim + d4 * 4);
    qs[d4 * 4 + 0][row] = a.x;
    qs[d4 * 4 + 1][row] = a.y;
    qs[d4 * 4 + 2][row] = a.z;
    qs[d4 * 4 + 3][row] = a.w;
    ks[d4 * 4 + 0][row] = b.x;
    ks[d4 * 4 + 1][row] = b.y;
    ks[d4 * 4 + 2][row] = b.z;
    ks[d4 * 4 + 3][row] = b.w;
  }
  __syncthreads();

  const int tx = t & 15;
  const int ty = t >> 4;
  float acc[4][4];
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) acc[x][y] = 0.f;
#pragma unroll 8
  for (int d = 0; d < kHeadDim; ++d) {
    const float4 a = *reinterpret_cast<const float4*>(&qs[d][ty * 4]);
    const float4 b = *reinterpret_cast<const float4*>(&ks[d][tx * 4]);
    const float av[4] = {a.x, a.y, a.z, a.w};
    const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_fmaf(av[x], bv[y], acc[x][y]);
  }
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const int i = i0 + ty * 4 + x;
    if (i >= g.nb) continue;
    float* dst = s + ((size_t)bh * g.nb + i) * g.nb;
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int j = j0 + tx * 4 + y;
      if (j < g.nb) dst[j] = acc[x][y] * g.scale;
    }
  }
}

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

template <int R>
__global__ __launch_bounds__(kThreads) void select_kernel(Geom g, const float* __restrict__ s,
                                                          int mode, int k, float p, int k_min,
                                                          int k_max, int stride,
                                                          int32_t* __restrict__ idx,
                                                          int32_t* __restrict__ cnt) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= g.bh * g.nb) return;  // whole wave leaves together
  const int i = row % g.nb;
  const int na = allowed_blocks(g, i);
  const float* srow = s + (size_t)row * g.nb;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  uint32_t key[R];
  float val[R];
#pragma unroll
  for (int c = 0; c < R; ++c) {
    const int j = c * 64 + lane;
    const bool ok = j < na;
    val[c] = ok ? srow[j] : -INFINITY;
    key[c] = ok ? order_key(val[c]) : 0u;
  }

  int keep;
  if (mode == 0) {
    keep = min(k, na);
  } else {
    // Softmax over the allowed blocks (fp32, max-subtracted).
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < R; ++c) m = fmaxf(m, val[c]);
    m = wave_max(m);
    float z = 0.f;
#pragma unroll
    for (int c = 0; c < R; ++c) {
      val[c] = (key[c] != 0u) ? expf(val[c] - m) : 0.f;
      z += val[c];
    }
    z = wave_sum(z);
    const float inv_z = 1.0f / z;
#pragma unroll
    for (int c = 0; c < R; ++c) val[c] *= inv_z;
    // Largest key threshold whose top set still holds mass >= p.
    uint32_t tau = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < R; ++c) part += (key[c] >= cand) ? val[c] : 0.f;
      if (wave_sum(part) >= p) tau = cand;
    }
    int raw;
    if (tau == 0u) {
      raw = na;  // no prefix reaches p (p = 1 with rounding): all allowed blocks
    } else {
      int gt = 0;
      float part = 0.f;
#pragma unroll
      for (int c = 0; c < R; ++c) {
        gt += __popcll(__ballot(key[c] > tau));
        part += (key[c] > tau) ? val[c] : 0.f;
      }
      float run = wave_sum(part);
      int add = 0;
      // Blocks tied at the threshold join in ascending id order until the
      // mass reaches p.
#pragma unroll
      for (int c = 0; c < R; ++c) {
        uint64_t eq = __ballot(key[c] == tau);
        while (eq != 0ull && run < p) {
          const int src = __ffsll((long long)eq) - 1;
          run += __shfl(val[c], src);
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
#pragma unroll
    for (int c = 0; c < R; ++c) c_ge += __popcll(__ballot(key[c] >= cand));
    if (c_ge >= keep) tau = cand;
  }
  int gt = 0;
#pragma unroll
  for (int c = 0; c < R; ++c) gt += __popcll(__ballot(key[c] > tau));
  const int need_eq = keep - gt;

  int32_t* out = idx + (size_t)row * stride;
  int pos = 0;
  int eq_seen = 0;
#pragma unroll
  for (int c = 0; c < R; ++c) {
    const bool is_gt = key[c] > tau;
    const bool is_eq = key[c] == tau;
    const uint64_t eqb = __ballot(is_eq);
    const int eq_rank = eq_seen + __popcll(eqb & below);
    const bool sel = is_gt || (is_eq && eq_rank < need_eq);
    const uint64_t selb = __ballot(sel);
    if (sel) out[pos + __popcll(selb & below)] = c * 64 + lane;
    pos += __popcll(selb);
    eq_seen += __popcll(eqb);
  }
  for (int q = keep + lane; q < stride; q += 64) out[q] = -1;
  if (lane == 0) cnt[row] = keep;
}

hipError_t launch_scores(const Geom& g, const float* qp, const float* kp, float* s,
                         hipStream_t stream) {
  const int tiles = (g.nb + kScoreTile - 1) / kScoreTile;
  dim3 grid(tiles, tiles, g.bh);
  hipLaunchKernelGGL(scores_kernel, grid, dim3(kThreads), 0, stream, g, qp, kp, s);
  return hipGetLastError();
}

template <int R>
static hipError_t launch_select_r(const Geom& g, const float* s, int mode, int k, float p,
                                  int k_min, int k_max, int stride, int32_t* idx, int32_t* cnt,
                                  hipStream_t stream) {
  const long rows = (long)g.bh * g.nb;
  const int rows_per_wg = kThreads / 64;
  dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
  hipLaunchKernelGGL(select_kernel<R>, grid, dim3(kThreads), 0, stream, g, s, mode, k, p, k_min,
                     k_max, stride, idx, cnt);
  return hipGetLastError();
}

hipError_t launch_select(const Geom& g, const float* s, int mode, int k, float p, int k_min,
                         int k_max, int stride, int32_t* idx, int32_t* cnt,
                         hipStream_t stream) {
  const int chunks = (g.nb + 63) / 64;
  if (chunks <= 1) return launch_select_r<1>(g, s, mode, k, p, k_min, k_max, stride, idx, cnt, stream);
  if (chunks <= 2) return launch_select_r<2>(g, s, mode, k, p, k_min, k_max, stride, idx, cnt, stream);
  if (chunks <= 4) return launch_select_r<4>(g, s, mode, k, p, k_min, k_max, stride, idx, cnt, stream);
  if (chunks <= 8) return launch_select_r<8>(g, s, mode, k, p, k_min, k_max, stride, idx, cnt, stream);
  if (chunks <= 16) return launch_select_r<16>(g, s, mode, k, p, k_min, k_max, stride, idx, cnt, stream);
  if (chunks <= 32) return launch_select_r<32>(g, s, mode, k, p, k_min, k_max, stride, idx, cnt, stream);
  return launch_select_r<64>(g, s, mode, k, p, k_min, k_max, stride, idx, cnt, stream);
}

}  // namespace bsa
