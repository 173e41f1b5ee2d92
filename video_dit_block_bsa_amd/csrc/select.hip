// Pooled block scores and key-block selection ("Block selection via pooled
// attention scores" and the Top-r / CDF-p modes of "Implementation details
// and design trade-offs", LongCat-Video deep dive, section "Block Sparse
// Attention"; combined top-k/CDF clamps from the zhaifeiyue notes, section 3).
//
// scores_kernel: S = (Q_pool K_pool^T) * scale per (batch, head), fp32,
//   Nb query blocks x Nk key blocks. A
//   64 x 64 output tile per workgroup, both operand tiles staged in LDS, fp32
//   MFMA 32x32x2 with a fixed summation order over the 128 channels.
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
constexpr int kScoreRow = kHeadDim + 4;  // padded LDS row (floats)

// One 64 x 64 tile of S per workgroup; wave w computes the 32 x 32 sub-tile
// (w / 2, w % 2) with fp32 MFMA 32x32x2 (exact fp32 products, fp32 sums).
// Step kk of the 64 MFMAs contracts channels kk (lanes 0..31) and 64 + kk
// (lanes 32..63): any pairing of channels works as long as both operands use
// the same one, and this one lets a lane read four steps of its row with one
// 16-byte LDS load. Row stride 132 floats keeps those loads conflict-free.
__global__ __launch_bounds__(kThreads) void scores_kernel(Geom g, int row0, const float* __restrict__ qp,
                                                          const float* __restrict__ kp,
                                                          float* __restrict__ s) {
  __shared__ __attribute__((aligned(16))) float qs[kScoreTile][kScoreRow];
  __shared__ __attribute__((aligned(16))) float ks[kScoreTile][kScoreRow];
  const int bh = blockIdx.z;
  const int i0 = row0 + blockIdx.y * kScoreTile;
  const int j0 = blockIdx.x * kScoreTile;
  const int t = threadIdx.x;
  const float* qb = qp + (size_t)bh * g.nb * kHeadDim;
  const float* kb = kp + (size_t)bh * g.nbk * kHeadDim;

  // Stage both 64 x 128 operand tiles row-major; rows past nb are zero.
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int c = t + kThreads * r;
    const int row = c >> 5;
    const int d4 = c & 31;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float4 b = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i0 + row < g.nb) a = *reinterpret_cast<const float4*>(qb + (size_t)(i0 + row) * kHeadDim + d4 * 4);
    if (j0 + row < g.nbk) b = *reinterpret_cast<const float4*>(kb + (size_t)(j0 + row) * kHeadDim + d4 * 4);
    *reinterpret_cast<float4*>(&qs[row][d4 * 4]) = a;
    *reinterpret_cast<float4*>(&ks[row][d4 * 4]) = b;
  }
  __syncthreads();

  const int lane = t & 63;
  const int w = t >> 6;
  const int wr = w >> 1, wc = w & 1;
  const int m = lane & 31;
  const int h = lane >> 5;
  const float* arow = &qs[32 * wr + m][64 * h];
  const float* brow = &ks[32 * wc + m][64 * h];
  f32x16 acc = {};
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const float4 a = *reinterpret_cast<const float4*>(arow + 4 * c);
    const float4 b = *reinterpret_cast<const float4*>(brow + 4 * c);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.x, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.y, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.z, b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.w, b.w, acc, 0, 0, 0);
  }
  // Accumulator value v holds row 8(v/4) + 4h + v%4, column m of the sub-tile.
  const int j = j0 + 32 * wc + m;
  if (j < g.nbk) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int i = i0 + 32 * wr + 8 * (v >> 2) + 4 * h + (v & 3);
      if (i < g.nb) s[((size_t)bh * g.nb + i) * g.nbk + j] = acc[v] * g.scale;
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

// Rows row0 .. nb-1 of every (batch, head).
template <int R>
__global__ __launch_bounds__(kThreads) void select_kernel(Geom g, int row0, const float* __restrict__ s,
                                                          int mode, int k, float p, int k_min,
                                                          int k_max, int stride,
                                                          int32_t* __restrict__ idx,
                                                          int32_t* __restrict__ cnt) {
  const int lane = threadIdx.x & 63;
  const int rows_per_head = g.nb - row0;
  const int local = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (local >= g.bh * rows_per_head) return;  // whole wave leaves together
  const int i = row0 + local % rows_per_head;
  const int row = (local / rows_per_head) * g.nb + i;
  const int na = allowed_key_blocks(g, i);
  const float* srow = s + (size_t)row * g.nbk;
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

hipError_t launch_scores(const Geom& g, const float* qp, const float* kp, float* s, int row0,
                         hipStream_t stream) {
  if (row0 >= g.nb) return hipSuccess;
  dim3 grid((g.nbk + kScoreTile - 1) / kScoreTile, (g.nb - row0 + kScoreTile - 1) / kScoreTile,
            g.bh);
  hipLaunchKernelGGL(scores_kernel, grid, dim3(kThreads), 0, stream, g, row0, qp, kp, s);
  return hipGetLastError();
}

template <int R>
static hipError_t launch_select_r(const Geom& g, const float* s, int mode, int k, float p,
                                  int k_min, int k_max, int stride, int32_t* idx, int32_t* cnt,
                                  int row0, hipStream_t stream) {
  const long rows = (long)g.bh * (g.nb - row0);
  if (rows <= 0) return hipSuccess;
  const int rows_per_wg = kThreads / 64;
  dim3 grid((unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
  hipLaunchKernelGGL(select_kernel<R>, grid, dim3(kThreads), 0, stream, g, row0, s, mode, k, p,
                     k_min, k_max, stride, idx, cnt);
  return hipGetLastError();
}

hipError_t launch_select(const Geom& g, const float* s, int mode, int k, float p, int k_min,
                         int k_max, int stride, int32_t* idx, int32_t* cnt, int row0,
                         hipStream_t stream) {
  const int chunks = (g.nbk + 63) / 64;
#define BSA_SELECT_R(R) \
  return launch_select_r<R>(g, s, mode, k, p, k_min, k_max, stride, idx, cnt, row0, stream)
  if (chunks <= 1) BSA_SELECT_R(1);
  if (chunks <= 2) BSA_SELECT_R(2);
  if (chunks <= 4) BSA_SELECT_R(4);
  if (chunks <= 8) BSA_SELECT_R(8);
  if (chunks <= 16) BSA_SELECT_R(16);
  if (chunks <= 32) BSA_SELECT_R(32);
  BSA_SELECT_R(64);
#undef BSA_SELECT_R
}

}  // namespace bsa
