// Block mean-pooling of Q and K ("Pooled block similarity computation" of the
// LongCat-Video deep dive, section "Block Sparse Attention"): the pooled
// vector of block b is the mean of the tokens of b, each block being a
// ct x ch x cw box of the latent grid (keys use the key chunk when it
// differs: "Implementation details and design trade-offs").
//
// One workgroup per (batch*head, block). Thread t reads channel chunk
// t % 16 (8 bf16 = 16 bytes) of tokens 8*(t/16) .. 8*(t/16)+7 of the block,
// from Q and from K; a wave's 64 lanes read 4 tokens x 256 contiguous bytes
// per load, so every load is a full-row, coalesced access. Partial sums go
// through LDS and are added in a fixed order, so the result is deterministic
// (and the same as summing the 8 tokens, then the 16 groups, in order).
// HBM-bound: 2 x 32 KB read and 2 x 512 B written per workgroup.
#include "launch.h"

namespace bsa {

__global__ __launch_bounds__(kThreads) void pool_kernel(Geom g, int blk0, const bf16_bits* __restrict__ q,
                                                        const bf16_bits* __restrict__ k,
                                                        float* __restrict__ qp,
                                                        float* __restrict__ kp) {
  __shared__ float part[2][16][kHeadDim + 4];
  const int blk = blk0 + blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int chunk = t & 15;
  const int grp = t >> 4;
  const size_t head_off = (size_t)bh * g.S * kHeadDim;

  // All 16 loads of this thread (8 tokens of Q, the same 8 of K) are issued
  // before any is summed, so each thread keeps 256 bytes in flight.
  u32x4 raw[2][8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const size_t off = head_off + (size_t)block_token(g, blk, grp * 8 + r) * kHeadDim + chunk * 8;
    raw[0][r] = *reinterpret_cast<const u32x4*>(q + off);
    raw[1][r] = *reinterpret_cast<const u32x4*>(k + off);
  }
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_to_f32(raw[which][r][e] & 0xffffu);
        acc[2 * e + 1] += bf16_to_f32(raw[which][r][e] >> 16);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[which][grp][chunk * 8 + e] = acc[e];
  }
  __syncthreads();
  // Threads 0..127 finish Q, 128..255 finish K: channel t % 128, the 16
  // partial sums added in a fixed order.
  const int which = t >> 7;
  const int c = t & (kHeadDim - 1);
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += part[which][r][c];
  float* dst = (which == 0 ? qp : kp);
  dst[((size_t)bh * g.nb + blk) * kHeadDim + c] = s * (1.0f / kBlockTokens);
}

// Pooling of one tensor when the key chunk differs from the query chunk, or
// when the grid has partial blocks:
// blocks of n = 64 .. 1024 tokens (query blocks, or key blocks with kKeys).
// Thread t adds channel chunk t % 16 of the n/16 consecutive slots
// (t/16)*n/16 ..; the 16 partial sums meet in LDS in a fixed order, as above.
// Blocks blk0, blk0+1, ... of each (batch, head); pooled row blk goes to row
// blk of an array of out_rows rows per (batch, head). A partial block at the
// grid's edge ("3D block partitioning" counts blocks with ceilings) is the
// mean of its slots inside the grid; the others are not read.
template <bool kKeys>
__global__ __launch_bounds__(kThreads) void pool_one_kernel(Geom g, int blk0, int out_rows,
                                                            const bf16_bits* __restrict__ x,
                                                            float* __restrict__ xp) {
  __shared__ float part[16][kHeadDim + 4];
  const int blk = blk0 + blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int chunk = t & 15;
  const int grp = t >> 4;
  const int n = kKeys ? g.nk : g.nq;
  const int per = n >> 4;  // a multiple of 4
  const size_t head_off = (size_t)bh * g.S * kHeadDim;
  int count = n;
  if (g.partial) {
    const int nw = kKeys ? g.nWk : g.nW, nh = kKeys ? g.nHk : g.nH;
    const int ct = kKeys ? g.ctk : g.ct, ch = kKeys ? g.chk : g.ch, cw = kKeys ? g.cwk : g.cw;
    const int bw = blk % nw, bhh = (blk / nw) % nh, bt = blk / (nw * nh);
    count = min(ct, g.T - bt * ct) * min(ch, g.H - bhh * ch) * min(cw, g.W - bw * cw);
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int r0 = 0; r0 < per; r0 += 4) {
    u32x4 raw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = grp * per + r0 + r;
      const int tok = kKeys ? key_block_token(g, blk, j) : block_token(g, blk, j);
      if (g.partial && !(kKeys ? key_slot_valid(g, blk, j) : block_slot_valid(g, blk, j)))
        raw[r] = u32x4{0u, 0u, 0u, 0u};
      else
        raw[r] = *reinterpret_cast<const u32x4*>(x + head_off + (size_t)tok * kHeadDim + chunk * 8);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_to_f32(raw[r][e] & 0xffffu);
        acc[2 * e + 1] += bf16_to_f32(raw[r][e] >> 16);
      }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[grp][chunk * 8 + e] = acc[e];
  __syncthreads();
  if (t < kHeadDim) {
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += part[r][t];
    xp[((size_t)bh * out_rows + blk) * kHeadDim + t] = sum * (1.0f / (float)count);
  }
}

hipError_t launch_pool_queries(const Geom& g, const bf16_bits* q, float* qp, int blk0,
                               hipStream_t stream) {
  if (blk0 >= g.nb) return hipSuccess;
  hipLaunchKernelGGL(pool_one_kernel<false>, dim3(g.nb - blk0, g.bh), dim3(kThreads), 0, stream, g,
                     blk0, g.nb, q, qp);
  return hipGetLastError();
}

hipError_t launch_pool_keys(const Geom& g, const bf16_bits* k, float* kp, int blk0, int blk_end,
                            int out_rows, hipStream_t stream) {
  if (blk0 >= blk_end) return hipSuccess;
  hipLaunchKernelGGL(pool_one_kernel<true>, dim3(blk_end - blk0, g.bh), dim3(kThreads), 0, stream, g,
                     blk0, out_rows, k, kp);
  return hipGetLastError();
}

hipError_t launch_pool(const Geom& g, const bf16_bits* q, const bf16_bits* k, float* qp,
                       float* kp, int blk0, hipStream_t stream) {
  if (blk0 >= g.nb) return hipSuccess;
  dim3 grid(g.nb - blk0, g.bh);
  hipLaunchKernelGGL(pool_kernel, grid, dim3(kThreads), 0, stream, g, blk0, q, k, qp, kp);
  return hipGetLastError();
}

}  // namespace bsa
