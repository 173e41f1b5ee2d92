// Backward pass of the block-restricted attention for gfx950: gradients of
// L = sum(dO * O) with respect to Q, K and V, with the key-block selection of
// the forward held fixed (a discrete choice, which carries no gradient). The
// LongCat-Video deep dive, section "Block Sparse Attention", gives the
// operator a backward pass ("Implementation details and design trade-offs")
// and uses the selection while training ("Block selection via pooled
// attention scores": r = N_k/8 in distillation, N_k/16 for the refinement
// expert).
//
// For query block i with gathered keys K_J, values V_J, scale s and the
// log-normaliser lse the forward wrote:
//   P   = exp(s Q_i K_J^T - lse)            recomputed, never stored
//   D   = rowsum(dO_i * O_i)                 one float per query
//   dP  = dO_i V_J^T,  dS = P * (dP - D)     softmax Jacobian
//   dQ_i += s dS K_J,  dK_J += s dS^T Q_i,  dV_J += P^T dO_i
//
// Four launches, all stream-ordered:
//   bwd_prep_kernel   D and lse*log2(e) per query, stored per block in slot
//                     order; clears the key-block -> query-block bit mask.
//   bwd_mask_kernel   sets bit (kb, qb) of the mask for every kept pair: the
//                     transposed selection, in a form whose bits come out in
//                     ascending query-block order whatever order the atomics
//                     land in, so dK and dV are deterministic.
//   bwd_dq_kernel     one workgroup per (batch*head, query block), walking the
//                     query block's key-block list: dQ = s sum dS K.
//   bwd_dkdv_kernel   one workgroup per (batch*head, key block), walking the
//                     set bits of its mask row: dK = s sum dS^T Q, dV = sum P^T dO.
// dQ and dK/dV each compute S and dP (P recomputed from lse), so no partial
// sums are exchanged between workgroups (no floating-point atomics) and
// every output is written once, by one workgroup.
//
// MFMA layout (bf16 32x32x16, fp32 accumulate). A 128-row tile lives in LDS
// as 128 rows of 256 bytes; chunk c (16 bytes) of row r is stored at chunk
// c ^ f(r) with f(r) = 4 (r mod 4) + (r / 4 mod 4). The tiles of this pass
// are read two ways: as row operands (lane n reads row swap23(n) at one
// chunk; 16 lanes meet 16 distinct rows of a 16-row group, which f sends to
// 16 distinct chunks) and through the transposing read ds_read_b64_tr_b16
// (32 lanes read four consecutive rows at one 64-byte column group; f puts
// the four rows in four different 64-byte groups). Both are free of bank
// conflicts with this one swizzle.
#include <type_traits>

#include "launch.h"
#include "tile.h"

namespace bsa {

constexpr float kLog2e = 1.4426950408889634f;


// ---------------------------------------------------------------- prep ---
// One workgroup per (block, batch*head). Thread t reads 16-byte chunk t % 16
// (channels 8(t%16) .. +7) of slots 16i + t/16, i = 0..7, from O and dO, so
// each load of a wave covers four whole 256-byte rows; the 16 lanes of a
// slot then add their partial dot products with four lane exchanges. stats
// holds, per (batch*head, block), 128 values lse*log2(e) followed by 128
// values D, in slot order (64-token blocks fill the first 64 of each). A
// query with lse = -inf (no key block) gets +inf, so that its recomputed
// probabilities are exp2(x - inf) = 0.
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(Geom g, int nbw,
                                                            const bf16_bits* __restrict__ o,
                                                            const bf16_bits* __restrict__ dout,
                                                            const float* __restrict__ lse,
                                                            float* __restrict__ stats,
                                                            uint32_t* __restrict__ mask) {
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int t = threadIdx.x;
  const int chunk = t & 15;
  const int r = t >> 4;
  // A slot of a partial block outside the grid has no token: D = 0 and
  // lse*log2(e) = +inf, so every probability recomputed for it is 0.
  auto slot_tok = [&](int j, bool& inside) __attribute__((always_inline)) {
    inside = j < g.nq && (!g.partial || block_slot_valid(g, blk, j));
    return inside ? block_token(g, blk, j) : 0;
  };
  u32x4 ov[8], dv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bool inside;
    const int tok = slot_tok(16 * i + r, inside);
    const size_t off = ((size_t)bh * g.S + tok) * kHeadDim + 8 * chunk;
    ov[i] = inside ? *reinterpret_cast<const u32x4*>(o + off) : u32x4{0u, 0u, 0u, 0u};
    dv[i] = inside ? *reinterpret_cast<const u32x4*>(dout + off) : u32x4{0u, 0u, 0u, 0u};
  }
  float* st = stats + ((size_t)bh * g.nb + blk) * (2 * kBlockTokens);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = __builtin_fmaf(bf16_to_f32(ov[i][e] & 0xffffu), bf16_to_f32(dv[i][e] & 0xffffu), acc);
      acc = __builtin_fmaf(bf16_to_f32(ov[i][e] >> 16), bf16_to_f32(dv[i][e] >> 16), acc);
    }
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) acc += __shfl_xor(acc, x);
    const int j = 16 * i + r;
    if (chunk == 0 && j < g.nq) st[kBlockTokens + j] = acc;
  }
  if (t < g.nq) {
    bool inside;
    const int tok = slot_tok(t, inside);
    const float l = inside ? lse[(size_t)bh * g.S + tok] : -INFINITY;
    st[t] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
  // Mask rows are per key block (nbk of them); query block blk clears rows
  // blk, blk + nb, ...
  for (int kb = blk; kb < g.nbk; kb += g.nb)
    if (t < nbw) mask[((size_t)bh * g.nbk + kb) * nbw + t] = 0u;
}

// ---------------------------------------------------------------- mask ---
// Wave w of workgroup x handles query block 4x + w: every valid id kb of its
// list sets bit qb of mask row kb. Ids outside [0, nbk) are skipped and the
// count is clamped to [0, stride], as in the forward.
__global__ __launch_bounds__(kThreads) void bwd_mask_kernel(Geom g, int nbw, int stride,
                                                            const int32_t* __restrict__ idx,
                                                            const int32_t* __restrict__ cnt,
                                                            uint32_t* __restrict__ mask) {
  const int qb = 4 * blockIdx.x + (threadIdx.x >> 6);
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (qb >= g.nb) return;
  const size_t row = (size_t)bh * g.nb + qb;
  const int count = min(max(cnt[row], 0), stride);
  const uint32_t bit = 1u << (qb & 31);
  for (int p = lane; p < count; p += 64) {
    const int kb = idx[row * stride + p];
    if (kb >= 0 && kb < g.nbk)
      atomicOr(&mask[((size_t)bh * g.nbk + kb) * nbw + (qb >> 5)], bit);
  }
}

// ------------------------------------------------------- tile addressing ---
// The dQ and dK/dV kernels run 8 waves (two per SIMD) per workgroup; each
// wave stages 16 rows of every 128-row tile.
constexpr int kBwdWaves = 8;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kRowsPerWave = kBlockTokens / kBwdWaves;
constexpr int kHalfTile = kBlockTokens / 2;

// Keeps the scheduler from hoisting the next phase's LDS operand reads above
// the current phase, which would raise register pressure for no gain (the
// second wave on the SIMD hides the latency); measured 3% faster than
// without.
__device__ __forceinline__ void phase_fence() { __builtin_amdgcn_sched_barrier(0); }

// Per-lane byte offsets into a swizzled 128-row tile.
struct TileLanes {
  // Row operand: lane (n, gs) reads row 32t + swap23(n), logical chunk
  // 2s + gs (channels 16s + 8gs .. +7) at  t * 8192 + (ra ^ 32s).
  int ra;
  // Transposing read for channel group u and 16-row step k: the lane's two
  // reads (rows +0..3 and +4..7 of its 8-row half) are at
  //   (16k)*256 + (ta ^ 64u)  and  (16k + 4)*256 + (ta ^ 64u ^ 16).
  int ta;
  // Direct-to-LDS tile load i (i = 0..3) of wave w covers rows 16w + 4i .. +3;
  // lane L writes physical chunk L % 16 of row 16w + 4i + L / 16 and fetches
  // global byte (row token)*256 + (ld ^ 16i), see load_tile; ldk is the same
  // for key tiles (slot offsets of the key chunk).
  uint32_t ld, ldk;
};

__device__ __forceinline__ TileLanes tile_lanes(const Geom& g, int w, int lane) {
  TileLanes t;
  const int n = lane & 31;
  const int gs = lane >> 5;
  // f(swap23(n)) for the row-operand lanes: bits 0-1 of the row are n's,
  // bits 2-3 are n's bits 3 and 2.
  const int f_row = ((n & 3) << 2) | ((n >> 3) & 1) | (((n >> 2) & 1) << 1);
  t.ra = swap23(n) * 256 + 16 * (gs ^ f_row);
  // Transposing read: in each 16-lane group, lane j reads row 8gs + j/4 (+4)
  // at channels 16*((lane/16)%2) + 4*(j%4) .. +3 of the channel group.
  const int jj = lane & 15;
  const int q4 = jj >> 2;
  const int hb = (lane >> 4) & 1;
  const int c1 = (jj & 3) >> 1;
  t.ta = (8 * gs + q4) * 256 + 64 * q4 + 16 * ((2 * hb + c1) ^ (2 * gs)) + 8 * (jj & 1);
  // Tile loads: row 16w + 4i + r (r = L/16) has f = 4r + i, so the lane
  // fetches logical chunk (L%16) ^ 4r ^ i. The slot offset is linear in the
  // bits of the slot index (power-of-two chunk sides), so the row's token is
  // that of slot 16w + r plus that of slot 4i.
  // With 64-token blocks, rows 64..127 of a tile hold a second block, so the
  // slot of row x is x mod 64.
  const int r = lane >> 4;
  const int row = kRowsPerWave * w + r;
  t.ld = (uint32_t)slot_offset(g, row & (g.nq - 1)) * (kHeadDim * 2) +
         (uint32_t)(((lane & 15) ^ (r << 2)) << 4);
  t.ldk = (uint32_t)key_slot_offset(g, g.nk == 64 ? (row & 63) : row) * (kHeadDim * 2) +
          (uint32_t)(((lane & 15) ^ (r << 2)) << 4);
  return t;
}

// Issues the four direct-to-LDS loads of this wave's 16 rows (16w .. +15)
// of a 128-row tile: row x holds slot jbase + (x & smask) of block `blk`
// (a query block, or a key block with kKeys), whose slot 0 is token
// `origin`; `lane0` is the lane's byte offset for the first load (ld or
// ldk). A row of a partial block that lies outside the grid fetches row 0
// of the block instead: every address stays inside the tensor, and the
// values it brings are multiplied by probability 0 (their scores are masked
// or their stats give P = 0).
template <bool kKeys, bool kPartial>
__device__ __forceinline__ void load_rows16(const AttnArgs& a, __amdgpu_buffer_rsrc_t rs,
                                            uint32_t lane0, int w, int blk, int origin, int jbase,
                                            int smask, bf16_bits* tile) {
  const Geom& g = a.g;
  const uint32_t base = (uint32_t)origin * (kHeadDim * 2);
  char* dst = reinterpret_cast<char*>(tile) + kRowsPerWave * w * 256;
  bool cut = false;
  Extent ex = {0, 0, 0};
  if (kPartial) {
    ex = kKeys ? key_block_extent<kPartial>(a, blk) : block_extent<kPartial>(a, blk);
    cut = kKeys ? (ex.t != g.ctk || ex.h != g.chk || ex.w != g.cwk)
                : (ex.t != g.ct || ex.h != g.ch || ex.w != g.cw);
  }
  // Bit x of `inside`: row 16w + x of the tile lies inside the grid (worked
  // out on the scalar unit; only for a cut block).
  uint32_t inside = 0xffffu;
  if (cut) {
    inside = 0u;
    for (int x = 0; x < kRowsPerWave; ++x) {
      const int j = jbase + ((kRowsPerWave * w + x) & smask);
      if (kKeys ? key_slot_inside(a, ex, j) : slot_inside(a, ex, j)) inside |= 1u << x;
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsPerWave / 4; ++i) {
    const uint32_t row_s =
        (uint32_t)(kKeys ? key_slot_offset(g, 4 * i) : slot_offset(g, 4 * i)) * (kHeadDim * 2);
    uint32_t voff = lane0 ^ (uint32_t)(16 * i);
    uint32_t soff = base + row_s;
    if (cut) {
      const int lane = threadIdx.x & 63;
      const bool in = ((inside >> (4 * i + (lane >> 4))) & 1u) != 0u;
      voff = in ? voff + row_s : (uint32_t)(lane & 15) * 16u;
      soff = base;
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + i * 1024), 16, voff, soff, 0, 0);
  }
}

__device__ __forceinline__ bf16x8 row_operand(const char* tile, int sub, int s, const TileLanes& tl) {
  return *reinterpret_cast<const bf16x8*>(tile + sub * 8192 + (tl.ra ^ (32 * s)));
}

// A operand X^T (channel group u, rows 16k .. 16k+15 of the tile) through two
// transposing reads: lane l gets channel 32u + l%32 of rows 16k + 8gs + 0..7.
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, int k, int u, const TileLanes& tl) {
  const char* p0 = tile + 16 * k * 256 + (tl.ta ^ (64 * u));
  const char* p1 = tile + (16 * k + 4) * 256 + (tl.ta ^ (64 * u) ^ 16);
  const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p0));
  const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p1));
  return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  const f32x2 v = {x, y};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Writes a 128-channel accumulator set (4 groups of 32 channels x 32 tokens,
// lane column = token) times `mul` as bf16 to row `row` (lane's token).
__device__ __forceinline__ void store_rows(bf16_bits* row, const f32x16 (&acc)[4], float mul, int gs) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const u32x2 packed = {pack_bf16(acc[u][4 * a4 + 0] * mul, acc[u][4 * a4 + 1] * mul),
                            pack_bf16(acc[u][4 * a4 + 2] * mul, acc[u][4 * a4 + 3] * mul)};
      *reinterpret_cast<u32x2*>(row + 32 * u + 8 * a4 + 4 * gs) = packed;
    }
}

// XCD-aware workgroup order, as in the forward: hardware id x runs on XCD
// x % 8; XCD c gets the blocks [c*chunk, (c+1)*chunk) of the current head.
// With `chunked` false the order is the plain one (block x of the head), which
// deals neighbouring blocks to different XCDs.
__device__ __forceinline__ void xcd_block(const AttnArgs& a, int& pair, int& blk, bool chunked = true) {
  const int x = blockIdx.x;
  pair = x / a.nq8;
  const int r = x - pair * a.nq8;
  const int chunk = a.nq8 >> 3;
  blk = chunked ? (r & 7) * chunk + (r >> 3) : r;
}

// ------------------------------------------------------------------ dQ ---
// Query blocks of 128 tokens: wave w owns queries 32(w%4) .. +31 and
// sub-tiles 2(w/4), 2(w/4)+1 (keys 64(w/4) .. +63) of every 128-key unit.
// Query blocks of 64 tokens (kSplit): wave w owns queries 32(w%2) .. +31 and
// sub-tile w/2 (keys 32(w/2) .. +31) of every unit. Either way no product is
// computed twice, and the waves of a query slice add their partial dQ once at
// the end, in a fixed order. Q^T and dO^T of the wave's queries stay in
// registers as B operands. Per 32-key sub-tile:
//   S^T = K Q^T, dP^T = V dO^T    (8 channel steps each)
//   dS^T = P^T * (dP^T - D)       lane's query: one lse and one D per lane
//   dQ^T += K^T dS^T              (4 channel groups x 2 key steps; K^T by
//                                  transposing reads of the same K tile)
// Units are walked as in the forward (kKeyMode 0: a 128-token key block;
// 1: unit `b` of a key block of 256+ tokens; 2: two 64-token key blocks,
// the lower one's keys in rows 0..63, the upper one's in rows 64..127). K and
// V tiles are double-buffered in LDS (two separate objects each, the loop
// unrolled by two so every read names its buffer at compile time and never
// waits for the loads into the other one).
//
// kUnion (64-token query blocks, 128-token key blocks, grids the chunks
// divide), as in the forward: one workgroup takes the blocks at t-rows 2m and
// 2m+1 of a column as the 128 query slots of one box (after an odd number of
// rows the last one alone) and walks the union of their key lists, each key
// tile gathered once. Waves 0..3 serve the first block and 4..7 the second
// (wave w: query slice w%2 of its block, key part (w/2)%2), so each SIMD,
// holding waves w and w+4, keeps one wave busy when only one block selected
// a unit; the other block's waves skip its products.
template <int kKeyMode, bool kSplit, bool kPartial, bool kUnion = false>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dq_kernel(
    AttnArgs a, const bf16_bits* __restrict__ qp, const bf16_bits* __restrict__ kp,
    const bf16_bits* __restrict__ vp, const bf16_bits* __restrict__ dop,
    const float* __restrict__ stats, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ cntp, bf16_bits* __restrict__ dqp) {
  __shared__ __attribute__((aligned(1024))) bf16_bits k0s[kBlockTokens * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits v0s[kBlockTokens * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits k1s[kBlockTokens * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits v1s[kBlockTokens * kHeadDim];
  const Geom& g = a.g;
  int pair, qi;
  xcd_block(a, pair, qi);
  const int nhw = g.nH * g.nW;  // query blocks per t-row
  // kUnion: qi indexes pairs; pair p holds block p + (p / nhw) * nhw and, if
  // it exists, the block one t-row after it.
  const int qb = kUnion ? qi + div_magic<false>(qi, a.mag_nhw) * nhw : qi;
  if (qb >= g.nb) return;
  const bool has_b = kUnion && qb + nhw < g.nb;  // the pair's second block exists

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  // Query slice (32 queries of the block, or of the pair's box) and key part.
  const int qs = kUnion ? 2 * (w >> 2) + (w & 1) : kSplit ? (w & 1) : (w & 3);
  const int kpart = kUnion ? ((w >> 1) & 1) : kSplit ? (w >> 1) : (w >> 2);
  const int n = lane & 31;
  const int gs = lane >> 5;
  const size_t hoff = (size_t)pair * g.S * kHeadDim;
  const uint32_t head_bytes = (uint32_t)g.S * (kHeadDim * 2);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(kp + hoff), (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(vp + hoff), (short)0, head_bytes, kBufferWord3);
  const TileLanes tl = tile_lanes(g, w, lane);

  // A query slot of a partial block outside the grid computes on slot 0 (its
  // stats make every probability 0) and is not written.
  // kUnion: the slices of a missing second block compute on slot 0 of the
  // first (they own no unit) and are not written.
  const bool q_inside =
      kUnion ? (qs < 2 || has_b) : !kPartial || block_slot_valid(g, qb, 32 * qs + n);
  const int qtok = block_origin<kPartial>(a, qb) + (q_inside ? slot_offset(g, 32 * qs + n) : 0);
  bf16x8 qf[8], df[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const size_t off = hoff + (size_t)qtok * kHeadDim + 16 * s + 8 * gs;
    qf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + off));
    df[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(dop + off));
  }
  // Stats of the wave's queries (kUnion: of its own block of the pair).
  const int sblk = (kUnion && qs >= 2 && has_b) ? qb + nhw : qb;
  const int sslot = 32 * (kUnion ? (qs & 1) : qs) + n;
  const float* st = stats + ((size_t)pair * g.nb + sblk) * (2 * kBlockTokens);
  const float lse2 = st[sslot];
  const float dd = st[kBlockTokens + sslot];

  const int32_t* list = idx + ((size_t)pair * g.nb + qb) * a.stride;
  const int count = min(max(cntp[(size_t)pair * g.nb + qb], 0), a.stride);
  const int32_t* list_b = has_b ? list + (size_t)nhw * a.stride : nullptr;  // the second block's list
  const int count_b = has_b ? min(max(cntp[(size_t)pair * g.nb + qb + nhw], 0), a.stride) : 0;
  auto next_valid_in = [&](const int32_t* l, int c, int from) __attribute__((always_inline)) {
    while (from < c) {
      const int kb = l[from];
      if (kb >= 0 && kb < g.nbk) break;
      ++from;
    }
    return from;
  };
  auto next_valid = [&](int from) __attribute__((always_inline)) {
    return next_valid_in(list, count, from);
  };
  // Unit cursor, as in the forward: (position, unit within the key block)
  // for kKeyMode 0 and 1, (position of the lower block, position of the upper
  // block) for kKeyMode 2; the unit exists while .a < count. kUnion:
  // (positions in the two lists, the unit's key block = the smaller entry,
  // bit 0 / 1 set when it is the first / second list's); the unit exists
  // while either position is inside its list.
  struct Cursor {
    int a, b, kb, m;
  };
  auto union_unit = [&](int pa, int pb) __attribute__((always_inline)) -> Cursor {
    const int ka = pa < count ? list[pa] : 0x7fffffff;
    const int kb = pb < count_b ? list_b[pb] : 0x7fffffff;
    const int k = min(ka, kb);
    return {pa, pb, k, (ka == k ? 1 : 0) | (kb == k ? 2 : 0)};
  };
  auto live = [&](const Cursor& c) __attribute__((always_inline)) {
    return kUnion ? (c.a < count || c.b < count_b) : c.a < count;
  };
  auto first_unit = [&]() __attribute__((always_inline)) -> Cursor {
    if constexpr (kUnion) return union_unit(next_valid(0), next_valid_in(list_b, count_b, 0));
    const int p = next_valid(0);
    return {p, kKeyMode == 2 ? next_valid(p + 1) : 0, 0, 0};
  };
  auto next_unit = [&](Cursor c) __attribute__((always_inline)) -> Cursor {
    if constexpr (kUnion) {
      return union_unit((c.m & 1) ? next_valid(c.a + 1) : c.a,
                        (c.m & 2) ? next_valid_in(list_b, count_b, c.b + 1) : c.b);
    } else if constexpr (kKeyMode == 1) {
      if (c.b + 1 < (1 << a.unit_shift)) return {c.a, c.b + 1, 0, 0};
      return {next_valid(c.a + 1), 0, 0, 0};
    } else if constexpr (kKeyMode == 2) {
      const int p = next_valid(c.b + 1);
      return {p, next_valid(p + 1), 0, 0};
    } else {
      return {next_valid(c.a + 1), 0, 0, 0};
    }
  };
  // This wave's rows of a unit's K or V tile: waves 4..7 stage rows 64..127,
  // which in kKeyMode 2 are the upper block's (the lower one again when it is
  // missing: those rows are never used).
  auto load_unit = [&](Cursor c, __amdgpu_buffer_rsrc_t rs, bf16_bits* tile)
                       __attribute__((always_inline)) {
    if constexpr (kKeyMode == 2) {
      const int kb = list[(w >= 4 && c.b < count) ? c.b : c.a];
      load_rows16<true, kPartial>(a, rs, tl.ldk, w, kb, key_block_origin<kPartial>(a, kb), 0,
                                  kHalfTile - 1, tile);
    } else if constexpr (kKeyMode == 1) {
      const int kb = list[c.a];
      load_rows16<true, kPartial>(a, rs, tl.ldk, w, kb,
                                  key_block_origin<kPartial>(a, kb) +
                                      key_slot_offset(g, c.b * kBlockTokens),
                                  c.b * kBlockTokens, kBlockTokens - 1, tile);
    } else {
      const int kb = kUnion ? c.kb : list[c.a];
      load_rows16<true, kPartial>(a, rs, tl.ldk, w, kb, key_block_origin<kPartial>(a, kb), 0,
                                  kBlockTokens - 1, tile);
    }
  };

  f32x16 dq[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) dq[u] = f32x16{};

  // The wave's key part is a template constant inside the loop, so every LDS
  // address is one of a few per-lane offsets plus an immediate.
  auto compute = [&](auto kpc, const char* kt, const char* vt, Cursor un) __attribute__((always_inline)) {
    constexpr int NS = kSplit ? 1 : 2;                          // sub-tiles per wave
    constexpr int TT0 = kSplit ? decltype(kpc)::value : 2 * decltype(kpc)::value;
    constexpr bool kUpper = kKeyMode == 2 && TT0 >= 2;          // rows of the upper block
    if constexpr (kUpper) {
      if (un.b >= count) return;  // a lone last 64-token block: no upper half
    }
    if constexpr (kUnion) {
      if (((un.m >> (w >> 2)) & 1) == 0) return;  // not selected by this wave's block
    }
    f32x16 sacc[NS], pacc[NS];
#pragma unroll
    for (int t2 = 0; t2 < NS; ++t2) sacc[t2] = pacc[t2] = f32x16{};
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int t2 = 0; t2 < NS; ++t2) {
        sacc[t2] = mfma(row_operand(kt, TT0 + t2, s, tl), qf[s], sacc[t2]);
        pacc[t2] = mfma(row_operand(vt, TT0 + t2, s, tl), df[s], pacc[t2]);
      }
    if constexpr (kPartial) {
      // Keys of a partial key block outside the grid: S = -inf, so P = 0.
      // Value i of sub-tile tt is key 32 tt + 16 (i/8) + 8 gs + i%8 of the
      // unit; the lane part goes through an empty asm so that nothing
      // derived from it is hoisted out of the loop.
      const Extent e = key_block_extent<kPartial>(a, list[kUpper ? un.b : un.a]);
      if (e.t != g.ctk || e.h != g.chk || e.w != g.cwk) {
        int lb = (kKeyMode == 1 ? un.b * kBlockTokens : 0) - (kUpper ? kHalfTile : 0) + 8 * gs;
        asm volatile("" : "+v"(lb));
#pragma unroll
        for (int t2 = 0; t2 < NS; ++t2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = lb + 32 * (TT0 + t2) + 16 * (i >> 3) + (i & 7);
            if (!key_slot_inside(a, e, j)) sacc[t2][i] = -INFINITY;
          }
      }
    }
    phase_fence();
    // Accumulator value i of sub-tile tt is key 32tt + swap23(row): values
    // 0..7 are keys +8gs .. +8gs+7, values 8..15 keys +16+8gs ..; as a B
    // operand they are key steps 2tt and 2tt+1.
    bf16x8 dsf[2 * NS];
#pragma unroll
    for (int t2 = 0; t2 < NS; ++t2)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 packed;
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
          const int i0 = 8 * hh + 2 * j2;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t2][i0], a.c_log2, -lse2));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t2][i0 + 1], a.c_log2, -lse2));
          packed[j2] = pack_bf16(p0 * (pacc[t2][i0] - dd), p1 * (pacc[t2][i0 + 1] - dd));
        }
        dsf[2 * t2 + hh] = __builtin_bit_cast(bf16x8, packed);
      }
    phase_fence();
#pragma unroll
    for (int ks = 0; ks < 2 * NS; ++ks)
#pragma unroll
      for (int u = 0; u < 4; ++u) dq[u] = mfma(tr_operand(kt, 2 * TT0 + ks, u, tl), dsf[ks], dq[u]);
    phase_fence();
  };

  auto run = [&](auto kpc) __attribute__((always_inline)) {
    Cursor cur = first_unit();
    if (!live(cur)) return;
    load_unit(cur, krs, k0s);
    load_unit(cur, vrs, v0s);
    Cursor nxt = next_unit(cur);
    auto step = [&](auto bc) __attribute__((always_inline)) -> bool {
      constexpr int b = decltype(bc)::value;
      bf16_bits* kt = b == 0 ? k0s : k1s;
      bf16_bits* vt = b == 0 ? v0s : v1s;
      bf16_bits* kn = b == 0 ? k1s : k0s;
      bf16_bits* vn = b == 0 ? v1s : v0s;
      // This wave's loads of the current tiles are done; after the barrier
      // everyone's are, and everyone has finished reading the other buffer.
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      workgroup_barrier();
      if (live(nxt)) {
        load_unit(nxt, krs, kn);
        load_unit(nxt, vrs, vn);
      }
      compute(kpc, reinterpret_cast<const char*>(kt), reinterpret_cast<const char*>(vt), cur);
      if (!live(nxt)) return false;
      cur = nxt;
      nxt = next_unit(cur);
      return true;
    };
    while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
    }
  };
  // Every copy of the loop runs the same barriers, so the waves stay in step.
  if constexpr (kSplit) {
    if (kpart == 0) run(std::integral_constant<int, 0>{});
    else if (kpart == 1) run(std::integral_constant<int, 1>{});
    else if (kpart == 2) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 3>{});
  } else {
    if (kpart == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
  }
  // The key parts of each query slice meet: every wave but the first of its
  // slice leaves its partial dQ in LDS (16 KB per wave, lane-contiguous
  // words; the tile buffers are idle now), the first adds them in order and
  // stores.
  __syncthreads();
  auto part = [&](int slot) __attribute__((always_inline)) -> float* {
    bf16_bits* buf = slot < 2 ? k0s : slot < 4 ? v0s : k1s;
    return reinterpret_cast<float*>(buf) + (slot & 1) * (64 * 64);
  };
  constexpr int kParts = kSplit ? 4 : 2;
  if (kpart != 0) {
    float* p = part(qs * (kParts - 1) + kpart - 1);
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) p[(u * 16 + i) * 64 + lane] = dq[u][i];
  }
  __syncthreads();
  if (kpart == 0) {
#pragma unroll
    for (int r = 1; r < kParts; ++r) {
      const float* p = part(qs * (kParts - 1) + r - 1);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[u][i] += p[(u * 16 + i) * 64 + lane];
    }
    if (q_inside) store_rows(dqp + hoff + (size_t)qtok * kHeadDim, dq, g.scale, gs);
  }
}

// ---------------------------------------------------------------- dK dV ---
// One workgroup of 8 waves per (batch*head, 128-key unit of a key block of
// 128+ tokens); wave w owns keys 32(w%4) .. +31 of the unit, in one of two
// roles:
//   w < 4  (P role):  S = Q K^T, P, dV^T += dO^T P
//   w >= 4 (dS role): dP = dO V^T, dS = P * (dP - D), dK^T += Q^T dS
// One wave cannot hold K, V, dK and dV (192 registers) and its working set
// in 256 VGPRs; split this way each role keeps one operand (K or V of its
// keys, as the B operand of S or dP) and one accumulator, no product is
// computed twice, and both roles issue the same number of MFMAs. P goes from
// the P-role wave to the dS-role wave of the same keys as bf16 through a
// two-slot LDS buffer per key slice, with one barrier per 32-query sub-tile
// (it waits for LDS traffic only, never for the tile loads in flight). Q, dO
// and the stats of the query rows are double-buffered in LDS; query blocks
// come from the set bits of the key block's mask row, in ascending order.
//
// kHalfKeys (64-token key blocks): one workgroup per key block; wave w of a
// role owns key slice w%2 (32 keys) and query half (w/2)%2 (sub-tiles 0, 1 or
// 2, 3 of each step), and the two query halves' partial dK and dV are added
// once, in a fixed order, through LDS at the end.
// kSplit (64-token query blocks): two query blocks go through the 128 query
// rows of a step, rows 0..63 of the first set bit and 64..127 of the next one
// (after an odd count the second half hands over P = 0, so it adds nothing).
template <bool kHalfKeys, bool kSplit, bool kPartial>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_dkdv_kernel(
    AttnArgs a, int nbw, const bf16_bits* __restrict__ qp, const bf16_bits* __restrict__ kp,
    const bf16_bits* __restrict__ vp, const bf16_bits* __restrict__ dop,
    const float* __restrict__ stats, const uint32_t* __restrict__ mask,
    bf16_bits* __restrict__ dkp, bf16_bits* __restrict__ dvp) {
  __shared__ __attribute__((aligned(1024))) bf16_bits q0s[kBlockTokens * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits d0s[kBlockTokens * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits q1s[kBlockTokens * kHeadDim];
  __shared__ __attribute__((aligned(1024))) bf16_bits d1s[kBlockTokens * kHeadDim];
  __shared__ __attribute__((aligned(1024))) float st0s[2 * kBlockTokens];
  __shared__ __attribute__((aligned(1024))) float st1s[2 * kBlockTokens];
  __shared__ __attribute__((aligned(1024))) char xch[4 * 2 * 2048];  // [key slice][slot][2 KB]
  __shared__ uint32_t mrow[kBlockTokens];
  const Geom& g = a.g;
  // With condition frames the leading (condition) key blocks carry the
  // longest query lists; the contiguous per-XCD order would put them all on
  // the first XCDs (measured: 40.5 ms against 29.5 ms for the backward of the
  // 61,440-token video-continuation shape), so they are dealt round-robin.
  int pair, unit;
  xcd_block(a, pair, unit, g.cond_kblocks == 0);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool ds_role = (w >> 2) != 0;
  const int ks = kHalfKeys ? (w & 1) : (w & 3);  // key slice
  const int qh = kHalfKeys ? ((w >> 1) & 1) : 0; // query half
  const int xs_id = kHalfKeys ? (2 * ks + qh) : ks; // the P hand-off buffer of the wave pair
  const int n = lane & 31;
  const int gs = lane >> 5;
  const int kb = unit >> a.unit_shift;
  const int slot = (unit & ((1 << a.unit_shift) - 1)) * kBlockTokens + 32 * ks + n;
  if (kb >= g.nbk) return;

  const size_t hoff = (size_t)pair * g.S * kHeadDim;
  const uint32_t head_bytes = (uint32_t)g.S * (kHeadDim * 2);
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(qp + hoff), (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t drs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(dop + hoff), (short)0, head_bytes, kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(stats + (size_t)pair * g.nb * (2 * kBlockTokens)), (short)0,
      (uint32_t)g.nb * (2 * kBlockTokens * 4), kBufferWord3);
  const TileLanes tl = tile_lanes(g, w, lane);

  // P role keeps K of its keys (B operand of S), dS role keeps V (of dP). A
  // key slot of a partial block outside the grid computes on the block's
  // slot 0 and is not written; query slots outside the grid have zero
  // probabilities (their stats), so they add nothing to dK or dV.
  const bool k_inside = !kPartial || key_slot_valid(g, kb, slot);
  const int ktok = key_block_origin<kPartial>(a, kb) + (k_inside ? key_slot_offset(g, slot) : 0);
  bf16x8 xf[8];
  {
    const bf16_bits* src = ds_role ? vp : kp;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      xf[s] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4*>(src + hoff + (size_t)ktok * kHeadDim + 16 * s + 8 * gs));
  }
  if (t < nbw) mrow[t] = mask[((size_t)pair * g.nbk + kb) * nbw + t];
  __syncthreads();
  auto next_set = [&](int from) __attribute__((always_inline)) -> int {
    int wd = from >> 5;
    if (wd >= nbw) return g.nb;
    uint32_t bits = __builtin_amdgcn_readfirstlane(mrow[wd]) & (0xffffffffu << (from & 31));
    while (bits == 0u) {
      if (++wd >= nbw) return g.nb;
      bits = __builtin_amdgcn_readfirstlane(mrow[wd]);
    }
    return wd * 32 + __builtin_ctz(bits);
  };
  // A step's query rows: block qa in rows 0..127 (128-token blocks), or qa in
  // rows 0..63 and qb2 (nb: none) in rows 64..127 (64-token blocks).
  struct Rows {
    int qa, qb2;
  };
  auto first_rows = [&]() __attribute__((always_inline)) -> Rows {
    const int x = next_set(0);
    return {x, kSplit && x < g.nb ? next_set(x + 1) : g.nb};
  };
  auto next_rows = [&](Rows r) __attribute__((always_inline)) -> Rows {
    const int x = next_set((kSplit && r.qb2 < g.nb ? r.qb2 : r.qa) + 1);
    return {x, kSplit && x < g.nb ? next_set(x + 1) : g.nb};
  };
  auto load_rows = [&](Rows r, bf16_bits* qdst, bf16_bits* ddst, float* sdst)
                       __attribute__((always_inline)) {
    const int blk = (kSplit && w >= 4 && r.qb2 < g.nb) ? r.qb2 : r.qa;
    const int origin = block_origin<kPartial>(a, blk);
    load_rows16<false, kPartial>(a, qrs, tl.ld, w, blk, origin, 0, g.nq - 1, qdst);
    load_rows16<false, kPartial>(a, drs, tl.ld, w, blk, origin, 0, g.nq - 1, ddst);
    if (w == 0) {
      // stats of a block: lse*log2(e) at floats 0.., D at floats 128... For
      // two 64-token blocks, lanes 0..15 / 16..31 fetch the lse of the first
      // / second block, lanes 32..47 / 48..63 their D.
      uint32_t off;
      if constexpr (kSplit) {
        const int sb = ((lane & 16) && r.qb2 < g.nb) ? r.qb2 : r.qa;
        off = (uint32_t)sb * (2 * kBlockTokens * 4) + ((lane & 32) ? kBlockTokens * 4 : 0) +
              16 * (lane & 15);
      } else {
        off = (uint32_t)r.qa * (2 * kBlockTokens * 4) + 16 * lane;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, (lds_void*)sdst, 16, off, 0, 0, 0);
    }
  };

  f32x16 acc[4];  // dV (P role) or dK (dS role)
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x16{};

  // Sub-tiles TT0 .. TT0 + NT - 1 of a step (the query half is a template
  // constant, so every LDS address is a per-lane offset plus an immediate).
  // keep_hi: whether query rows 64..127 hold a query block (64-token blocks).
  auto compute = [&](auto rolec, auto qhc, const char* qt, const char* dt, const float* sts,
                     bool keep_hi) __attribute__((always_inline)) {
    constexpr bool dsr = decltype(rolec)::value != 0;
    constexpr int NT = kHalfKeys ? 2 : 4;
    constexpr int TT0 = kHalfKeys ? 2 * decltype(qhc)::value : 0;
    char* xbase = xch + xs_id * 4096;
#pragma unroll
    for (int tl2 = 0; tl2 < NT; ++tl2) {
      const int tt = TT0 + tl2;
      char* xs = xbase + (tl2 & 1) * 2048;
      bf16x8 bop[2];
      if constexpr (!dsr) {
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) sacc = mfma(row_operand(qt, tt, s, tl), xf[s], sacc);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int q0 = 32 * tt + 16 * hh + 8 * gs;
          u32x4 packed;
#pragma unroll
          for (int j2 = 0; j2 < 4; ++j2) {
            const int i0 = 8 * hh + 2 * j2;
            const f32x2 l2 = *reinterpret_cast<const f32x2*>(sts + q0 + 2 * j2);
            const uint32_t pw =
                pack_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i0], a.c_log2, -l2[0])),
                          __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i0 + 1], a.c_log2, -l2[1])));
            packed[j2] = (kSplit && tt >= 2 && !keep_hi) ? 0u : pw;
          }
          bop[hh] = __builtin_bit_cast(bf16x8, packed);
          *reinterpret_cast<u32x4*>(xs + hh * 1024 + lane * 16) = packed;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the hand-off is written
        workgroup_barrier();
      } else {
        f32x16 pacc = f32x16{};
#pragma unroll
        for (int s = 0; s < 8; ++s) pacc = mfma(row_operand(dt, tt, s, tl), xf[s], pacc);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): done with the slot's previous use
        workgroup_barrier();
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int q0 = 32 * tt + 16 * hh + 8 * gs;
          const u32x4 pb = *reinterpret_cast<const u32x4*>(xs + hh * 1024 + lane * 16);
          u32x4 packed;
#pragma unroll
          for (int j2 = 0; j2 < 4; ++j2) {
            const int i0 = 8 * hh + 2 * j2;
            const f32x2 d2 = *reinterpret_cast<const f32x2*>(sts + kBlockTokens + q0 + 2 * j2);
            packed[j2] = pack_bf16(bf16_to_f32(pb[j2] & 0xffffu) * (pacc[i0] - d2[0]),
                                   bf16_to_f32(pb[j2] >> 16) * (pacc[i0 + 1] - d2[1]));
          }
          bop[hh] = __builtin_bit_cast(bf16x8, packed);
        }
      }
      const char* xt = dsr ? qt : dt;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = mfma(tr_operand(xt, 2 * tt + k2, u, tl), bop[k2], acc[u]);
    }
  };

  // The same sub-tiles with the MFMA operands read from LDS ahead of their
  // use (grids the chunks divide; the general kernels, which need the
  // registers, keep `compute`): right after a sub-tile's chain is issued, the
  // wave reads all eight operands of that sub-tile's accumulation and the
  // first four of the next sub-tile's chain, so the reads complete under the
  // chain's MFMAs (dS role) or the exponentials (P role) and the barrier's
  // wait for the hand-off finds them done. Measured at 215K tokens: backward
  // 163.7 against 168.1 ms on one box (all eight chain operands ahead, or only
  // four accumulation operands, gained less; all of both spilled); the
  // outputs are bit-identical, since every product and sum is the same.
  auto compute_pf = [&](auto rolec, auto qhc, const char* qt, const char* dt, const float* sts,
                        bool keep_hi) __attribute__((always_inline)) {
    constexpr bool dsr = decltype(rolec)::value != 0;
    constexpr int NT = kHalfKeys ? 2 : 4;
    constexpr int TT0 = kHalfKeys ? 2 * decltype(qhc)::value : 0;
    char* xbase = xch + xs_id * 4096;
    const char* rt = dsr ? dt : qt;  // row operands of the chain (dO for dP, Q for S)
    const char* xt = dsr ? qt : dt;  // transposed operands of the accumulation
    constexpr int kRop = 4;  // chain operands read ahead
    constexpr int kTop = 8;  // accumulation operands read ahead
    bf16x8 rop[kRop];
#pragma unroll
    for (int s = 0; s < kRop; ++s) rop[s] = row_operand(rt, TT0, s, tl);
#pragma unroll
    for (int tl2 = 0; tl2 < NT; ++tl2) {
      const int tt = TT0 + tl2;
      char* xs = xbase + (tl2 & 1) * 2048;
      f32x16 cacc = f32x16{};
#pragma unroll
      for (int s = 0; s < 8; ++s) cacc = mfma(s < kRop ? rop[s] : row_operand(rt, tt, s, tl), xf[s], cacc);
      bf16x8 top[kTop];
#pragma unroll
      for (int i = 0; i < kTop; ++i) top[i] = tr_operand(xt, 2 * tt + (i >> 2), i & 3, tl);
      if (tl2 + 1 < NT) {
#pragma unroll
        for (int s = 0; s < kRop; ++s) rop[s] = row_operand(rt, tt + 1, s, tl);
      }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 bop[2];
      if constexpr (!dsr) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int q0 = 32 * tt + 16 * hh + 8 * gs;
          u32x4 packed;
#pragma unroll
          for (int j2 = 0; j2 < 4; ++j2) {
            const int i0 = 8 * hh + 2 * j2;
            const f32x2 l2 = *reinterpret_cast<const f32x2*>(sts + q0 + 2 * j2);
            const uint32_t pw =
                pack_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(cacc[i0], a.c_log2, -l2[0])),
                          __builtin_amdgcn_exp2f(__builtin_fmaf(cacc[i0 + 1], a.c_log2, -l2[1])));
            packed[j2] = (kSplit && tt >= 2 && !keep_hi) ? 0u : pw;
          }
          bop[hh] = __builtin_bit_cast(bf16x8, packed);
          *reinterpret_cast<u32x4*>(xs + hh * 1024 + lane * 16) = packed;
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the hand-off is written
        workgroup_barrier();
      } else {
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): done with the slot's previous use
        workgroup_barrier();
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int q0 = 32 * tt + 16 * hh + 8 * gs;
          const u32x4 pb = *reinterpret_cast<const u32x4*>(xs + hh * 1024 + lane * 16);
          u32x4 packed;
#pragma unroll
          for (int j2 = 0; j2 < 4; ++j2) {
            const int i0 = 8 * hh + 2 * j2;
            const f32x2 d2 = *reinterpret_cast<const f32x2*>(sts + kBlockTokens + q0 + 2 * j2);
            packed[j2] = pack_bf16(bf16_to_f32(pb[j2] & 0xffffu) * (cacc[i0] - d2[0]),
                                   bf16_to_f32(pb[j2] >> 16) * (cacc[i0 + 1] - d2[1]));
          }
          bop[hh] = __builtin_bit_cast(bf16x8, packed);
        }
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[u] = mfma(4 * k2 + u < kTop ? top[4 * k2 + u] : tr_operand(xt, 2 * tt + k2, u, tl), bop[k2], acc[u]);
    }
  };

  auto run = [&](auto rolec, auto qhc) __attribute__((always_inline)) {
    Rows cur = first_rows();
    if (cur.qa >= g.nb) return;
    load_rows(cur, q0s, d0s, st0s);
    Rows nxt = next_rows(cur);
    auto step = [&](auto bc) __attribute__((always_inline)) -> bool {
      constexpr int b = decltype(bc)::value;
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
      workgroup_barrier();
      if (nxt.qa < g.nb) load_rows(nxt, b == 0 ? q1s : q0s, b == 0 ? d1s : d0s, b == 0 ? st1s : st0s);
      if constexpr (!kPartial)
        compute_pf(rolec, qhc, reinterpret_cast<const char*>(b == 0 ? q0s : q1s),
                   reinterpret_cast<const char*>(b == 0 ? d0s : d1s), b == 0 ? st0s : st1s,
                   !kSplit || cur.qb2 < g.nb);
      else
        compute(rolec, qhc, reinterpret_cast<const char*>(b == 0 ? q0s : q1s),
                reinterpret_cast<const char*>(b == 0 ? d0s : d1s), b == 0 ? st0s : st1s,
                !kSplit || cur.qb2 < g.nb);
      if (nxt.qa >= g.nb) return false;
      cur = nxt;
      nxt = next_rows(cur);
      return true;
    };
    while (step(std::integral_constant<int, 0>{}) && step(std::integral_constant<int, 1>{})) {
    }
  };
  // Every copy of the loop runs the same barriers, so the waves stay in step.
  using std::integral_constant;
  if (ds_role) {
    if (qh == 0) run(integral_constant<int, 1>{}, integral_constant<int, 0>{});
    else run(integral_constant<int, 1>{}, integral_constant<int, 1>{});
  } else {
    if (qh == 0) run(integral_constant<int, 0>{}, integral_constant<int, 0>{});
    else run(integral_constant<int, 0>{}, integral_constant<int, 1>{});
  }
  if constexpr (kHalfKeys) {
    // The two query halves of each (role, key slice) meet: the second half's
    // wave leaves its partial sums in LDS (16 KB per wave, lane-contiguous
    // words; the tile buffers are idle now), the first adds them and stores.
    __syncthreads();
    const int pslot = 2 * (ds_role ? 1 : 0) + ks;  // 0..3
    float* part = reinterpret_cast<float*>(pslot < 2 ? q0s : d0s) + (pslot & 1) * (64 * 64);
    if (qh == 1) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 16; ++i) part[(u * 16 + i) * 64 + lane] = acc[u][i];
    }
    __syncthreads();
    if (qh == 1) return;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[u][i] += part[(u * 16 + i) * 64 + lane];
  }
  if (!k_inside) return;
  if (ds_role)
    store_rows(dkp + hoff + (size_t)ktok * kHeadDim, acc, g.scale, gs);
  else
    store_rows(dvp + hoff + (size_t)ktok * kHeadDim, acc, 1.0f, gs);
}

hipError_t launch_attention_bwd(const Geom& g, const bf16_bits* q, const bf16_bits* k,
                                const bf16_bits* v, const bf16_bits* o, const bf16_bits* dout,
                                const float* lse, const int32_t* idx, const int32_t* cnt,
                                int stride, float* stats, uint32_t* mask, bf16_bits* dq,
                                bf16_bits* dk, bf16_bits* dv, hipStream_t stream) {
  const AttnArgs a = make_attn_args(g, stride);
  const int nbw = (g.nb + 31) / 32;
  hipLaunchKernelGGL(bwd_prep_kernel, dim3(g.nb, g.bh), dim3(kThreads), 0, stream, g, nbw, o, dout,
                     lse, stats, mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_mask_kernel, dim3((g.nb + 3) / 4, g.bh), dim3(kThreads), 0, stream, g, nbw,
                     stride, idx, cnt, mask);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool split = g.nq != kBlockTokens;
  const int mode = g.nk == 64 ? 2 : g.nk > kBlockTokens ? 1 : 0;
  const bool part = needs_general(g);
  const dim3 grid((unsigned)((size_t)g.bh * a.nq8));
  const int nhw = g.nH * g.nW;
  // Grids the chunks divide (with more than one block along w and within a
  // frame) run kernels compiled without the general code (the default
  // kernels sit at the 256-VGPR limit). 64-token query blocks with 128-token
  // key blocks go in t-adjacent pairs.
  if (split && mode == 0 && !part) {
    AttnArgs au = a;
    au.nq8 = ((g.nb / nhw + 1) / 2 * nhw + 7) / 8 * 8;
    hipLaunchKernelGGL((bwd_dq_kernel<0, false, false, true>), dim3((unsigned)((size_t)g.bh * au.nq8)),
                       dim3(kBwdThreads), 0, stream, au, q, k, v, dout, stats, idx, cnt, dq);
  } else {
#define BSA_LAUNCH_DQ(MODE, SPLIT, PART)                                                      \
  hipLaunchKernelGGL((bwd_dq_kernel<MODE, SPLIT, PART>), grid, dim3(kBwdThreads), 0, stream, a, \
                     q, k, v, dout, stats, idx, cnt, dq)
#define BSA_LAUNCH_DQ_P(MODE, SPLIT) \
  if (part) BSA_LAUNCH_DQ(MODE, SPLIT, true); else BSA_LAUNCH_DQ(MODE, SPLIT, false)
  if (split) {
    if (mode == 0) { BSA_LAUNCH_DQ_P(0, true); }
    else if (mode == 1) { BSA_LAUNCH_DQ_P(1, true); }
    else { BSA_LAUNCH_DQ_P(2, true); }
  } else {
    if (mode == 0) { BSA_LAUNCH_DQ_P(0, false); }
    else if (mode == 1) { BSA_LAUNCH_DQ_P(1, false); }
    else { BSA_LAUNCH_DQ_P(2, false); }
  }
#undef BSA_LAUNCH_DQ_P
#undef BSA_LAUNCH_DQ
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dK/dV: one workgroup per 128-key unit of a key block of 128+ tokens, or
  // per 64-token key block.
  AttnArgs au = a;
  const int units = mode == 2 ? g.nbk : (g.nbk << a.unit_shift);
  au.nq8 = (units + 7) / 8 * 8;
  const dim3 grid_u((unsigned)((size_t)g.bh * au.nq8));
#define BSA_LAUNCH_DKDV(HALF, SPLIT, PART)                                                          \
  hipLaunchKernelGGL((bwd_dkdv_kernel<HALF, SPLIT, PART>), grid_u, dim3(kBwdThreads), 0, stream, au, \
                     nbw, q, k, v, dout, stats, mask, dk, dv)
#define BSA_LAUNCH_DKDV_P(HALF, SPLIT) \
  if (part) BSA_LAUNCH_DKDV(HALF, SPLIT, true); else BSA_LAUNCH_DKDV(HALF, SPLIT, false)
  if (mode == 2) {
    if (split) { BSA_LAUNCH_DKDV_P(true, true); }
    else { BSA_LAUNCH_DKDV_P(true, false); }
  } else {
    if (split) { BSA_LAUNCH_DKDV_P(false, true); }
    else { BSA_LAUNCH_DKDV_P(false, false); }
  }
#undef BSA_LAUNCH_DKDV_P
#undef BSA_LAUNCH_DKDV
  return hipGetLastError();
}

}  // namespace bsa
