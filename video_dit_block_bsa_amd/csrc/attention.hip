// Block-restricted flash attention ("Sparse attention computation" of the
// LongCat-Video deep dive, section "Block Sparse Attention": softmax over the
// keys of the selected blocks only) and its dense baseline, for gfx950.
//
// Work decomposition
//   One workgroup (4 x wave64) per (batch*head, query block of 128 tokens),
//   two workgroups per CU; wave w owns queries 32w .. 32w+31 of the block.
//   The workgroup walks the query block's key-block list; for each key block
//   the 128 x 128 K and V tiles are staged in LDS as [token][channel] rows.
//
// Math per key block and wave (bf16 MFMA 32x32x16, fp32 accumulate)
//   S^T = K Q^T     4 key sub-tiles x 8 channel steps = 32 MFMA. Q^T stays in
//                   registers for the whole loop (B operand); K rows come from
//                   LDS (A operand).
//   online softmax  each lane owns one query (C column) and holds 64 of its
//                   128 scores; the row max needs one exchange with lane^32.
//                   exp2 with scale*log2(e) folded in.
//   O^T += V^T P^T  4 channel sub-tiles x 8 key steps = 32 MFMA; P^T is taken
//                   straight from the S^T accumulators (converted to bf16).
//                   The V^T operand is read from the [key][channel] V tile
//                   with gfx950's transposing LDS read (ds_read_b64_tr_b16),
//                   two 4-key reads per fragment, so V needs no repacked copy.
//   For the P^T registers to line up with natural key order, the K rows are
//   read with bits 2 and 3 of the row index swapped: the accumulator of row m
//   then holds key swap23(m), and the 8 values a lane contributes to one
//   16-key MFMA step are consecutive keys.
//
// Tiles reach LDS with direct-to-LDS loads (global_load_lds_dwordx4), no
// VGPR staging: V of the current key block is fetched while S and the
// softmax run, K of the next key block while P V runs. LDS rows are unpadded;
// XOR swizzles on 16-byte chunks keep the operand reads free of bank
// conflicts. The epilogue divides by the softmax sum and writes O in latent
// order.
//
// Workgroup order is XCD-aware: MI355X dispatches consecutive workgroups
// round-robin over its 8 XCDs, so the id is remapped to give each XCD a
// contiguous run of query blocks of the same head (spatial neighbours select
// overlapping key blocks, which then hit that XCD's L2), while all XCDs work
// on the same head at a time (its K/V stay resident in the shared cache).
#include "common.h"

namespace bsa {

__device__ __forceinline__ bf16x8 lds_frag(const bf16_bits* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ int swap23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// Kernel arguments. Block ids are split into (bt, bh, bw) with multiply-high
// division by magic numbers (exact for the ranges the host checks), so the
// per-key-block address math stays on the scalar unit.
struct AttnArgs {
  Geom g;
  const bf16_bits* q;
  const bf16_bits* k;
  const bf16_bits* v;
  const int32_t* idx;
  const int32_t* cnt;
  bf16_bits* o;
  int stride;
  int nq8;           // query blocks per head rounded up to a multiple of 8
  uint32_t mag_nw;   // floor(2^32 / nW) + 1
  uint32_t mag_nhw;  // floor(2^32 / (nH*nW)) + 1
  float c_log2;      // scale * log2(e)
};

// Latent-order token of the first slot of block i.
__device__ __forceinline__ int block_origin(const AttnArgs& a, int i) {
  const Geom& g = a.g;
  const int bt = (int)__umulhi((uint32_t)i, a.mag_nhw);
  const int rem = i - bt * g.nH * g.nW;
  const int bh = (int)__umulhi((uint32_t)rem, a.mag_nw);
  const int bw = rem - bh * g.nW;
  return ((bt * g.ct) * g.H + bh * g.ch) * g.W + bw * g.cw;
}

// Offset (in tokens) of slot j inside its block.
__device__ __forceinline__ int slot_offset(const Geom& g, int j) {
  const int iw = j % g.cw;
  const int r2 = j / g.cw;
  return ((r2 / g.ch) * g.H + r2 % g.ch) * g.W + iw;
}

// Softmax rescaling is lazy: the running max m (log2 units) is only moved
// when a tile's max exceeds it by more than this, so most tiles skip the
// O *= alpha pass. Probabilities stay <= 2^8, well inside fp32 and bf16.
constexpr float kRescaleSlack = 8.0f;

typedef __attribute__((address_space(3))) void lds_void;

// Tiles live in LDS as 128 rows of 256 bytes (16 chunks of 16 bytes) with
// no padding. Chunk c of row r is stored at chunk c ^ swz(r), where swz(r) is
// swap23 of the row's low four bits. The MFMA operand reads of a wave touch
// rows swap23(n) + const with the same logical chunk, which this spreads over
// all 16 chunk positions: conflict-free. Each direct-to-LDS load writes 64
// lanes x 16 bytes = 4 whole rows, so lane L of a load writes physical chunk
// L % 16 of row base + L / 16 and fetches the logical chunk that lands there.
__device__ __forceinline__ int swz(int row) { return swap23(row & 15); }

// V tiles are read four rows at a time (transposing reads); spreading rows
// r..r+3 over the four 64-byte slots of a 256-byte row keeps them apart.
__device__ __forceinline__ int swzv(int row) { return 4 * (row & 3); }
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

template <bool kDense>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) bf16_bits ks[kBlockTokens * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits vs[kHeadDim * kBlockTokens];
  const Geom& g = a.g;

  // XCD-aware remap: hardware id x runs on XCD x % 8; give XCD c the query
  // blocks [c*chunk, (c+1)*chunk) of the current head.
  const int x = blockIdx.x;
  const int pair = x / a.nq8;
  const int r = x - pair * a.nq8;
  const int chunk = a.nq8 >> 3;
  const int qb = (r & 7) * chunk + (r >> 3);
  if (qb >= g.nb) return;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int n = lane & 31;
  const int gs = lane >> 5;
  const size_t hoff = (size_t)pair * g.S * kHeadDim;
  const char* kh = reinterpret_cast<const char*>(a.k + hoff);
  const char* vh = reinterpret_cast<const char*>(a.v + hoff);

  const int qtok = block_origin(a, qb) + slot_offset(g, 32 * w + n);
  bf16x8 qf[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    qf[s] = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const u32x4*>(a.q + hoff + (size_t)qtok * kHeadDim + 16 * s + 8 * gs));

  // This wave stages rows 32w .. 32w+31 of each tile: 8 loads of 4 rows.
  uint32_t koff[8], voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 32 * w + 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ swz(row);
    koff[i] = (uint32_t)slot_offset(g, row) * (kHeadDim * 2) + c * 16;
    const int cv = (lane & 15) ^ swzv(row);
    voff[i] = (uint32_t)slot_offset(g, row) * (kHeadDim * 2) + cv * 16;
  }
  char* ks_w = reinterpret_cast<char*>(ks) + 32 * w * 256;
  char* vs_w = reinterpret_cast<char*>(vs) + 32 * w * 256;

  int count;
  const int32_t* list = nullptr;
  if (kDense) {
    count = allowed_blocks(g, qb);
  } else {
    list = a.idx + ((size_t)pair * g.nb + qb) * a.stride;
    count = min(max(a.cnt[(size_t)pair * g.nb + qb], 0), a.stride);
  }
  // Next usable list position at or after `from` (ids outside [0, nb) are skipped).
  auto next_valid = [&](int from) {
    if (kDense) return from;
    while (from < count) {
      const int kb = list[from];
      if (kb >= 0 && kb < g.nb) break;
      ++from;
    }
    return from;
  };
  auto kb_at = [&](int pos) { return kDense ? pos : list[pos]; };
  auto load_k = [&](int kb) {
    const char* base = kh + (size_t)block_origin(a, kb) * (kHeadDim * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(base + koff[i], (lds_void*)(ks_w + i * 1024), 16, 0, 0);
  };
  auto load_v = [&](int kb) {
    const char* base = vh + (size_t)block_origin(a, kb) * (kHeadDim * 2);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_global_load_lds(base + voff[i], (lds_void*)(vs_w + i * 1024), 16, 0, 0);
  };

  f32x16 oacc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) oacc[u] = f32x16{};
  float m2 = -INFINITY;  // running max of score * c_log2
  float l_part = 0.f;    // this lane's share of the softmax denominator
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  const int rowA = swap23(n);  // operand row of this lane inside a 32-row sub-tile
  const int cx = n & 15;       // chunk swizzle of that row
  // Transposing V reads: in each group of 16 lanes, lane j points at key
  // 16s + 8gs + (j%16)/4 (+4 for the second read) and channels
  // 32u + 16*((lane/16)%2) + 4*(j%4) .. +3; lane i then receives channel
  // 32u + (lane%32) of those four keys. Chunk c of V row r sits at c ^ swzv(r).
  int vtr_base[4];
  {
    const int jj = lane & 15;
    const int q = jj >> 2;
    const int c0 = 2 * ((lane >> 4) & 1) + ((jj & 3) >> 1);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      vtr_base[u] = (8 * gs + q) * 256 + ((4 * u + c0) ^ (4 * q)) * 16 + 8 * (jj & 1);
  }

  int pos = next_valid(0);
  if (pos < count) load_k(kb_at(pos));
  while (pos < count) {
    const int kb = kb_at(pos);
    const int nxt = next_valid(pos + 1);

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's K rows are in LDS
    __builtin_amdgcn_s_barrier();        // all K rows in; every wave is done with vs
    load_v(kb);

    // S^T = K Q^T for this wave's 32 queries and all 128 keys.
    // Channel steps outermost: four independent accumulators between
    // dependent MFMAs.
    f32x16 sacc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) sacc[tt] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const bf16x8 af = lds_frag(&ks[(32 * tt + rowA) * kHeadDim + (((2 * s + gs) ^ cx) << 3)]);
        sacc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[s], sacc[tt], 0, 0, 0);
      }
    }

    // Online softmax for this lane's query (both lane halves agree on m2).
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[tt][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * a.c_log2;
    const bool grow = mx > m2 + kRescaleSlack;
    if (__ballot(grow) != 0ull) {
      const float m_new = grow ? mx : m2;
      const float alpha = __builtin_amdgcn_exp2f(m2 - m_new);
      m2 = m_new;
      l_part *= alpha;
#pragma unroll
      for (int u = 0; u < 4; ++u) oacc[u] *= alpha;
    }
    bf16x8 pf[8];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 packed;
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
          const f32x2 pr = {
              __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[tt][8 * h + 2 * j2], a.c_log2, -m2)),
              __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[tt][8 * h + 2 * j2 + 1], a.c_log2, -m2))};
          const bf16x2 pb = __builtin_convertvector(pr, bf16x2);
          l_part = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l_part, false);
          packed[j2] = __builtin_bit_cast(uint32_t, pb);
        }
        pf[2 * tt + h] = __builtin_bit_cast(bf16x8, packed);
      }
    }

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's V rows are in LDS
    __builtin_amdgcn_s_barrier();        // all V rows in; every wave is done with ks
    if (nxt < count) load_k(kb_at(nxt));

    // O^T += V^T P^T. The V tile is [key][channel] in LDS; each V^T operand
    // fragment (channel 32u + lane%32, keys 16s + 8gs .. +7) is two
    // transposing reads of four keys each.
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const char* p0 = reinterpret_cast<const char*>(vs) + vtr_base[u] + s * 16 * 256;
        const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0));
        const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0 + 4 * 256));
        const bf16x8 af = __builtin_bit_cast(
            bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
        oacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, pf[s], oacc[u], 0, 0, 0);
      }
    }
    pos = nxt;
  }

  const float l = l_part + __shfl_xor(l_part, 32);
  const float inv = (l > 0.f) ? 1.0f / l : 0.f;
  bf16_bits* orow = a.o + hoff + (size_t)qtok * kHeadDim;
  // Accumulator value i of sub-tile u is channel 32u + 8(i/4) + 4gs + i%4.
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

hipError_t launch_attention(const Geom& g, const bf16_bits* q, const bf16_bits* k,
                            const bf16_bits* v, const int32_t* idx, const int32_t* cnt,
                            int stride, bool dense, bf16_bits* o, hipStream_t stream) {
  AttnArgs a;
  a.g = g;
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.cnt = cnt;
  a.o = o;
  a.stride = stride;
  a.nq8 = (g.nb + 7) / 8 * 8;
  a.mag_nw = (uint32_t)(0x100000000ull / (uint64_t)g.nW + 1);
  a.mag_nhw = (uint32_t)(0x100000000ull / (uint64_t)(g.nH * g.nW) + 1);
  a.c_log2 = g.scale * 1.4426950408889634f;
  dim3 grid((unsigned)((size_t)g.bh * a.nq8));
  if (dense)
    hipLaunchKernelGGL(attn_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bsa
