// Block-restricted flash attention ("Sparse attention computation" of the
// LongCat-Video deep dive, section "Block Sparse Attention": softmax over the
// keys of the selected blocks only) and its dense baseline, for gfx950.
//
// Work decomposition
//   One workgroup (4 x wave64) per (batch*head, query block of 128 tokens);
//   wave w owns queries 32w .. 32w+31 of the block. The workgroup walks the
//   query block's key-block list; for each key block the 128 x 128 K tile and
//   the 128 x 128 V^T tile are staged in LDS (rows padded to 272 bytes so the
//   16-byte fragment reads of 32 consecutive rows hit distinct banks).
//
// Math per key block and wave (bf16 MFMA 32x32x16, fp32 accumulate)
//   S^T = K Q^T     4 key sub-tiles x 8 channel steps = 32 MFMA. Q^T stays in
//                   registers for the whole loop (B operand); K rows come from
//                   LDS (A operand).
//   online softmax  each lane owns one query (C column) and holds 64 of its
//                   128 scores; the row max needs one exchange with lane^32.
//                   exp2 with scale*log2(e) folded in.
//   O^T += V^T P^T  4 channel sub-tiles x 8 key steps = 32 MFMA; P^T is taken
//                   straight from the S^T accumulators (converted to bf16),
//                   V^T rows come from LDS.
//   For the P^T registers to line up with natural key order, the K rows are
//   read with bits 2 and 3 of the row index swapped: the accumulator of row m
//   then holds key swap23(m), and the 8 values a lane contributes to one
//   16-key MFMA step are consecutive keys.
//
// V^T comes from pack_v_kernel, which rewrites V per block as [channel][key]
// (an 8 x 8 register transpose per thread). The attention epilogue divides
// by the softmax sum and writes O in latent order.
//
// Workgroup order is XCD-aware: MI355X dispatches consecutive workgroups
// round-robin over its 8 XCDs, so the id is remapped to give each XCD a
// contiguous run of query blocks of the same head (spatial neighbours select
// overlapping key blocks, which then hit that XCD's L2), while all XCDs work
// on the same head at a time (its K/V stay resident in the shared cache).
#include "common.h"

namespace bsa {

constexpr int kPitch = kHeadDim + 8;  // LDS row pitch in bf16 elements

__device__ __forceinline__ bf16x8 lds_frag(const bf16_bits* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// V [S][d] in latent order -> V^T per block: vt[block][d][slot].
__global__ __launch_bounds__(kThreads) void pack_v_kernel(Geom g, const bf16_bits* __restrict__ v,
                                                          bf16_bits* __restrict__ vt) {
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int dg = t & 15;  // channels 8*dg .. 8*dg+7
  const int kg = t >> 4;  // slots 8*kg .. 8*kg+7
  const bf16_bits* src = v + (size_t)bh * g.S * kHeadDim;
  u32x4 in[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int tok = block_token(g, blk, kg * 8 + e);
    in[e] = *reinterpret_cast<const u32x4*>(src + (size_t)tok * kHeadDim + dg * 8);
  }
  bf16_bits* dst = vt + ((size_t)bh * g.nb + blk) * kBlockTokens * kHeadDim;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    u32x4 out;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint32_t lo = in[2 * a][r >> 1];
      const uint32_t hi = in[2 * a + 1][r >> 1];
      out[a] = (r & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    *reinterpret_cast<u32x4*>(dst + (size_t)(dg * 8 + r) * kBlockTokens + kg * 8) = out;
  }
}

__device__ __forceinline__ int swap23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <bool kDense>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(
    Geom g, const bf16_bits* __restrict__ q, const bf16_bits* __restrict__ k,
    const bf16_bits* __restrict__ vt, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cnt, int stride, bf16_bits* __restrict__ o, int nq8,
    float c_log2) {
  __shared__ __attribute__((aligned(16))) bf16_bits ks[kBlockTokens * kPitch];
  __shared__ __attribute__((aligned(16))) bf16_bits vs[kHeadDim * kPitch];

  // XCD-aware remap: hardware id x runs on XCD x % 8; give XCD c the query
  // blocks [c*chunk, (c+1)*chunk) of the current head.
  const int x = blockIdx.x;
  const int pair = x / nq8;
  const int r = x - pair * nq8;
  const int chunk = nq8 >> 3;
  const int qb = (r & 7) * chunk + (r >> 3);
  if (qb >= g.nb) return;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int n = lane & 31;
  const int gs = lane >> 5;
  const size_t hoff = (size_t)pair * g.S * kHeadDim;
  const bf16_bits* qh = q + hoff;
  const bf16_bits* kh = k + hoff;
  const bf16_bits* vth = vt + hoff;
  bf16_bits* oh = o + hoff;

  const int qtok = block_token(g, qb, 32 * w + n);
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const u32x4*>(qh + (size_t)qtok * kHeadDim + 16 * s + 8 * gs));

  int count;
  const int32_t* list = nullptr;
  if (kDense) {
    count = allowed_blocks(g, qb);
  } else {
    list = idx + ((size_t)pair * g.nb + qb) * stride;
    count = min(max(cnt[(size_t)pair * g.nb + qb], 0), stride);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) oacc[u] = f32x16{};
  float m_run = -INFINITY;
  float l_part = 0.f;
  const int krow = swap23(n);

  for (int it = 0; it < count; ++it) {
    const int kb = kDense ? it : list[it];
    if (!kDense && (kb < 0 || kb >= g.nb)) continue;  // same value in every lane

    __syncthreads();  // the previous tiles are no longer being read
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int c = t + kThreads * rr;
      const int row = c >> 4;
      const int col = c & 15;
      const int ktok = block_token(g, kb, row);
      const u32x4 kv = *reinterpret_cast<const u32x4*>(kh + (size_t)ktok * kHeadDim + col * 8);
      const u32x4 vv = *reinterpret_cast<const u32x4*>(
          vth + ((size_t)kb * kHeadDim + row) * kBlockTokens + col * 8);
      *reinterpret_cast<u32x4*>(&ks[row * kPitch + col * 8]) = kv;
      *reinterpret_cast<u32x4*>(&vs[row * kPitch + col * 8]) = vv;
    }
    __syncthreads();

    // S^T = K Q^T for this wave's 32 queries and all 128 keys.
    f32x16 sacc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      sacc[tt] = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 a = lds_frag(&ks[(32 * tt + krow) * kPitch + 16 * s + 8 * gs]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[tt], 0, 0, 0);
      }
    }

    // Online softmax for this lane's query.
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[tt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c_log2);
    m_run = m_new;
    const float mc = m_new * c_log2;
    float rs = 0.f;
    bf16x8 pf[8];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x2 pr[4];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[tt][8 * h + j], c_log2, -mc));
          rs += pv;
          pr[j >> 1][j & 1] = pv;
        }
        bf16x2 b0 = __builtin_convertvector(pr[0], bf16x2);
        bf16x2 b1 = __builtin_convertvector(pr[1], bf16x2);
        bf16x2 b2 = __builtin_convertvector(pr[2], bf16x2);
        bf16x2 b3 = __builtin_convertvector(pr[3], bf16x2);
        u32x4 packed = {__builtin_bit_cast(uint32_t, b0), __builtin_bit_cast(uint32_t, b1),
                        __builtin_bit_cast(uint32_t, b2), __builtin_bit_cast(uint32_t, b3)};
        pf[2 * tt + h] = __builtin_bit_cast(bf16x8, packed);
      }
    }
    l_part = l_part * alpha + rs;
#pragma unroll
    for (int u = 0; u < 4; ++u) oacc[u] *= alpha;

    // O^T += V^T P^T.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 a = lds_frag(&vs[(32 * u + n) * kPitch + 16 * s + 8 * gs]);
        oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s], oacc[u], 0, 0, 0);
      }
    }
  }

  const float l = l_part + __shfl_xor(l_part, 32);
  const float inv = (l > 0.f) ? 1.0f / l : 0.f;
  bf16_bits* orow = oh + (size_t)qtok * kHeadDim;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const f32x2 lo = {oacc[u][4 * a4 + 0] * inv, oacc[u][4 * a4 + 1] * inv};
      const f32x2 hi = {oacc[u][4 * a4 + 2] * inv, oacc[u][4 * a4 + 3] * inv};
      const u32x2 packed = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                            __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2))};
      *reinterpret_cast<u32x2*>(orow + 32 * u + 8 * a4 + 4 * gs) = packed;
    }
  }
}

hipError_t launch_pack_v(const Geom& g, const bf16_bits* v, bf16_bits* vt, hipStream_t stream) {
  dim3 grid(g.nb, g.bh);
  hipLaunchKernelGGL(pack_v_kernel, grid, dim3(kThreads), 0, stream, g, v, vt);
  return hipGetLastError();
}

hipError_t launch_attention(const Geom& g, const bf16_bits* q, const bf16_bits* k,
                            const bf16_bits* vt, const int32_t* idx, const int32_t* cnt,
                            int stride, bool dense, bf16_bits* o, hipStream_t stream) {
  const int nq8 = (g.nb + 7) / 8 * 8;
  const float c_log2 = g.scale * 1.4426950408889634f;
  dim3 grid((unsigned)((size_t)g.bh * nq8));
  if (dense)
    hipLaunchKernelGGL(attn_kernel<true>, grid, dim3(kThreads), 0, stream, g, q, k, vt, idx, cnt,
                       stride, o, nq8, c_log2);
  else
    hipLaunchKernelGGL(attn_kernel<false>, grid, dim3(kThreads), 0, stream, g, q, k, vt, idx,
                       cnt, stride, o, nq8, c_log2);
  return hipGetLastError();
}

}  // namespace bsa
